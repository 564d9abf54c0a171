/*
 * mhc_oracle.c -- CPU oracle for the mHC layer boundary.  TEST INFRASTRUCTURE:
 * only the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load it.  It shares no code, header, table or constant with the GPU library.
 *
 * Plain, slow, obviously correct.  Every output is a closed-form function of the
 * inputs.  The steps whose rounding the pages fix are done in FP32 exactly as
 * printed there (the residual update and the lagged collapse: FP32 FMA chains
 * rounded to BF16); everything else is FP64.
 *
 * Sources (vLLM "DeepSeek-V4.1 shifted mHC boundary" page = page B;
 * "Hyper Connection Preprocessing GPU Kernel Study" blog = page P):
 *   weight rounding/split  page B, prepare_boundary_weight (TF32 nearest ties away,
 *                          BF16 high part, BF16 low part of the remainder)
 *   residual update        page B, residual_update (post[s]*x then FMA over j of
 *                          comb[j][s]*X[j], FP32, rounded to BF16)
 *   lagged collapse        page B, lagged_collapse (FMA chain from 0 over j of
 *                          pre[j]*X'[j], FP32, rounded to BF16; sums of squares of
 *                          the BF16 values)
 *   mixes / rstd / pre / post   page B, coefficients; page P, "computing A_l",
 *                          "computing C_l", "square sum and RMSNorm"
 *   comb (Sinkhorn)        page B, coefficients + sinkhorn + col_normalize;
 *                          page P, "computing B_l"
 *   layer input RMSNorm    page B, kernel "totals in rank order" + layer_input_words
 *   non-shifted pre        page P, write_layer_input and "why this kernel is called pre"
 *   precomputed mixes      page P, "square sum and RMSNorm" (path 1) and "explaining
 *                          split-K": dot_mix and sqrsum summed over the splits
 *
 * Readings where the pages leave a step open are listed in the design notes;
 * the ones that matter here:
 *   - softmax and normalisations are e/sum + eps and c/(sum + eps), in FP64;
 *   - the row sum is ((c0+c1)+c2)+c3 then + eps; the column sum is
 *     (r0+r1)+(r2+r3) then + eps;
 *   - layer_input = bf16(li * rstd_li * norm_w) with one rounding from FP64;
 *   - no flush to zero (inputs never hold subnormals).
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fPIC -shared [-fopenmp]
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define NHC 4
#define NMIX 24

static float bits_to_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f32_to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bf16_to_f32(uint16_t b) { return bits_to_f32((uint32_t)b << 16); }

/* ---- rounding helpers -------------------------------------------------- */

/* TF32 (10 explicit mantissa bits), nearest with ties away from zero: add half
 * of the dropped 13-bit field to the magnitude, then clear the field. */
uint32_t oracle_tf32_bits(uint32_t b) { return (b + 0x1000u) & 0xFFFFE000u; }

/* FP32 -> BF16, round to nearest even (finite inputs). */
uint16_t oracle_bf16_from_f32(float f) {
    uint32_t u = f32_to_bits(f);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

/* FP64 -> BF16 with a single rounding, nearest even, for values in BF16's
 * normal range (or zero). */
uint16_t oracle_bf16_from_f64(double v) {
    if (v == 0.0) return signbit(v) ? 0x8000u : 0x0000u;
    int e;
    double m = frexp(fabs(v), &e);          /* |v| = m * 2^e, m in [0.5, 1) */
    double s = ldexp(m, 8);                 /* 8 significant bits above the point */
    double whole = floor(s);
    double frac = s - whole;                /* exact */
    if (frac > 0.5 || (frac == 0.5 && fmod(whole, 2.0) == 1.0)) whole += 1.0;
    float r = (float)ldexp(whole, e - 8);   /* exact: at most 9 bits */
    uint32_t u = f32_to_bits(r) | (v < 0 ? 0x80000000u : 0u);
    return (uint16_t)(u >> 16);
}

/* ---- weight preparation -------------------------------------------------- */

/* hi = bf16(t), lo = bf16(t - hi) with t = tf32(w): their sum is t exactly. */
void oracle_split_weight(const float* w, size_t n, float* tf32_out,
                         uint16_t* hi_out, uint16_t* lo_out) {
    for (size_t i = 0; i < n; ++i) {
        float t = bits_to_f32(oracle_tf32_bits(f32_to_bits(w[i])));
        uint16_t hi = oracle_bf16_from_f32(t);
        uint16_t lo = oracle_bf16_from_f32(t - bf16_to_f32(hi));
        if (tf32_out) tf32_out[i] = t;
        if (hi_out) hi_out[i] = hi;
        if (lo_out) lo_out[i] = lo;
    }
}

/* Prepared-weight bytes, rebuilt from the layout that the library's header
 * documents, element by element:
 *   index(step, s, m, l, e) = ((((step*4 + s)*3 + m)*64 + l)*8 + e)  (uint16 units)
 *   column k = s*d + 32*step + 8*(l/16) + e
 *   r = l%16: part = (r%4 < 2) ? high : low,  mix = 8*m + 2*(r/4) + (r%2)
 * out holds 192*d uint16. */
int oracle_prepare_weight(const float* w, int d, uint16_t* out) {
    if (d <= 0 || d % 32) return 1;
    const size_t K = (size_t)NHC * d;
    for (int step = 0; step < d / 32; ++step)
        for (int s = 0; s < NHC; ++s)
            for (int m = 0; m < 3; ++m)
                for (int l = 0; l < 64; ++l)
                    for (int e = 0; e < 8; ++e) {
                        int r = l % 16;
                        int mix = 8 * m + 2 * (r / 4) + (r % 2);
                        int high = (r % 4) < 2;
                        size_t k = (size_t)s * d + 32 * step + 8 * (l / 16) + e;
                        uint16_t hi, lo;
                        oracle_split_weight(&w[(size_t)mix * K + k], 1, NULL, &hi, &lo);
                        size_t idx = ((((size_t)step * 4 + s) * 3 + m) * 64 + l) * 8 + e;
                        out[idx] = high ? hi : lo;
                    }
    return 0;
}

/* ---- per-token pieces ------------------------------------------------------ */

static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

/* Row softmax of the 4x4 logits plus eps, one column normalisation, then
 * (iters - 1) x (row normalisation, column normalisation).  c is row-major:
 * c[4*i + k] = row i, column k. */
void oracle_sinkhorn(const double logits[16], double eps, int iters, double c[16]) {
    for (int i = 0; i < 4; ++i) {
        const double* v = &logits[4 * i];
        double mx = fmax(fmax(v[0], v[1]), fmax(v[2], v[3]));
        double e[4], sum = 0.0;
        for (int k = 0; k < 4; ++k) { e[k] = exp(v[k] - mx); }
        sum = ((e[0] + e[1]) + e[2]) + e[3];
        for (int k = 0; k < 4; ++k) c[4 * i + k] = e[k] / sum + eps;
    }
    for (int it = 0; it < iters; ++it) {
        if (it > 0) {
            for (int i = 0; i < 4; ++i) {
                double rs = ((c[4 * i] + c[4 * i + 1]) + c[4 * i + 2]) + c[4 * i + 3] + eps;
                for (int k = 0; k < 4; ++k) c[4 * i + k] = c[4 * i + k] / rs;
            }
        }
        for (int k = 0; k < 4; ++k) {
            double cs = (c[k] + c[4 + k]) + (c[8 + k] + c[12 + k]) + eps;
            for (int i = 0; i < 4; ++i) c[4 * i + k] = c[4 * i + k] / cs;
        }
    }
}

typedef struct {
    float rms_eps, pre_eps, post_mult, sinkhorn_eps;
    int sinkhorn_iters;
    float norm_eps;
} oracle_params;

/* pre / post / comb of one token from its 24 mixes and sum of squares. */
static void coefficients(const double mix[NMIX], double ssq, int d, const float* scale,
                         const float* base, const oracle_params* p, double* rstd_out,
                         double pre[4], double post[4], double comb[16]) {
    double rstd = 1.0 / sqrt(ssq / (4.0 * d) + (double)p->rms_eps);
    double logits[16];
    for (int j = 0; j < 4; ++j) {
        double vp = mix[j] * rstd * (double)scale[0] + (double)base[j];
        double vq = mix[4 + j] * rstd * (double)scale[1] + (double)base[4 + j];
        pre[j] = sigmoid(vp) + (double)p->pre_eps;
        post[j] = (double)p->post_mult * sigmoid(vq);
    }
    for (int n = 0; n < 16; ++n)
        logits[n] = mix[8 + n] * rstd * (double)scale[2] + (double)base[8 + n];
    oracle_sinkhorn(logits, (double)p->sinkhorn_eps, p->sinkhorn_iters, comb);
    *rstd_out = rstd;
}

/* li = bf16(FMA chain over j of pc[j]*xn[j], from 0) in FP32; ssq_li = sum of
 * li^2; rstd_li = 1/sqrt(ssq_li/d + norm_eps); layer_input = bf16(li*rstd_li*
 * norm_w) with one rounding from FP64, or li without norm_w.  xn holds the four
 * streams' values (as FP32) stream-major; li is scratch of d floats. */
static void collapse(const float* xn, const float pc[4], int d, const uint16_t* norm_w,
                     const oracle_params* p, float* li, double* ssq_li_out,
                     double* rstd_li_out, uint16_t* li_out, uint16_t* layer_input) {
    double ssq_li = 0.0;
    for (int h = 0; h < d; ++h) {
        float acc = 0.0f;
        for (int j = 0; j < 4; ++j) acc = fmaf(pc[j], xn[(size_t)j * d + h], acc);
        li[h] = bf16_to_f32(oracle_bf16_from_f32(acc));
        ssq_li += (double)li[h] * (double)li[h];
    }
    double rstd_li = 1.0 / sqrt(ssq_li / (double)d + (double)p->norm_eps);
    for (int h = 0; h < d; ++h) {
        uint16_t lb = oracle_bf16_from_f32(li[h]);
        if (li_out) li_out[h] = lb;
        if (layer_input)
            layer_input[h] = norm_w ? oracle_bf16_from_f64((double)li[h] * rstd_li *
                                                           (double)bf16_to_f32(norm_w[h]))
                                    : lb;
    }
    *ssq_li_out = ssq_li;
    *rstd_li_out = rstd_li;
}

/*
 * The shifted boundary (shifted=1) or the non-shifted pre (shifted=0) for the
 * tokens listed in tok[0..n_tok).  Inputs are the full [T,...] arrays; outputs
 * are indexed by position in tok.  tf32w is tf32(W) as produced by
 * oracle_split_weight ([24, 4d] floats).
 *
 *   shifted=1: X' = update(X, x, post_prev, comb_prev); li from pre_lag.
 *   shifted=0: X' = X; li from the fresh pre (cast to FP32, as the collapse
 *              runs in FP32).  x, post_prev, comb_prev, pre_lag are unused.
 *
 * Outputs (any may be NULL except where noted):
 *   xn[n_tok,4,d] bf16, li[n_tok,d] bf16, layer_input[n_tok,d] bf16,
 *   mixes[n_tok,24], ssq[n_tok], rstd[n_tok], ssq_li[n_tok], rstd_li[n_tok],
 *   pre[n_tok,4], post[n_tok,4], comb[n_tok,16]   (FP64)
 * norm_w may be NULL (no RMSNorm: layer_input = li).
 */
int oracle_run(int shifted, int T, int d, const int* tok, int n_tok,
               const uint16_t* X, const uint16_t* x, const float* post_prev,
               const float* comb_prev, const float* pre_lag, const float* tf32w,
               const float* scale, const float* base, const uint16_t* norm_w,
               const oracle_params* p,
               uint16_t* xn_out, uint16_t* li_out, uint16_t* layer_input,
               double* mixes_out, double* ssq_out, double* rstd_out, double* ssq_li_out,
               double* rstd_li_out, double* pre_out, double* post_out, double* comb_out) {
    if (T <= 0 || d <= 0 || n_tok < 0 || p->sinkhorn_iters < 1) return 1;
    for (int i = 0; i < n_tok; ++i)
        if (tok[i] < 0 || tok[i] >= T) return 2;
    const size_t K = (size_t)NHC * d;
    int status = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (int ti = 0; ti < n_tok; ++ti) {
        const size_t t = (size_t)tok[ti];
        float* xn = (float*)malloc(sizeof(float) * K);      /* X' as FP32 (BF16 values) */
        float* li = (float*)malloc(sizeof(float) * d);
        if (!xn || !li) { free(xn); free(li); status = 3; continue; }

        /* residual update (or identity for the non-shifted pre) */
        for (int h = 0; h < d; ++h) {
            float Xj[4];
            for (int j = 0; j < 4; ++j) Xj[j] = bf16_to_f32(X[(t * 4 + j) * d + h]);
            for (int s = 0; s < 4; ++s) {
                float v;
                if (shifted) {
                    float nu = post_prev[t * 4 + s] * bf16_to_f32(x[t * d + h]);
                    for (int j = 0; j < 4; ++j)
                        nu = fmaf(comb_prev[t * 16 + j * 4 + s], Xj[j], nu);
                    v = bf16_to_f32(oracle_bf16_from_f32(nu));
                } else {
                    v = Xj[s];
                }
                xn[(size_t)s * d + h] = v;
            }
        }

        /* sum of squares of X' and the 24 mixes tf32(W) . flat(X') */
        double ssq = 0.0;
        for (size_t k = 0; k < K; ++k) ssq += (double)xn[k] * (double)xn[k];
        double mix[NMIX];
        for (int n = 0; n < NMIX; ++n) {
            double acc = 0.0;
            for (size_t k = 0; k < K; ++k) acc += (double)tf32w[n * K + k] * (double)xn[k];
            mix[n] = acc;
        }
        double rstd, pre[4], post[4], comb[16];
        coefficients(mix, ssq, d, scale, base, p, &rstd, pre, post, comb);

        /* collapse: lagged pre for the boundary, fresh pre for the non-shifted pre */
        float pc[4];
        for (int j = 0; j < 4; ++j) pc[j] = shifted ? pre_lag[t * 4 + j] : (float)pre[j];
        double ssq_li, rstd_li;
        collapse(xn, pc, d, norm_w, p, li, &ssq_li, &rstd_li,
                 li_out ? &li_out[(size_t)ti * d] : NULL,
                 layer_input ? &layer_input[(size_t)ti * d] : NULL);

        /* outputs */
        if (xn_out)
            for (size_t k = 0; k < K; ++k) xn_out[ti * K + k] = oracle_bf16_from_f32(xn[k]);
        if (mixes_out) memcpy(&mixes_out[(size_t)ti * NMIX], mix, sizeof mix);
        if (ssq_out) ssq_out[ti] = ssq;
        if (rstd_out) rstd_out[ti] = rstd;
        if (ssq_li_out) ssq_li_out[ti] = ssq_li;
        if (rstd_li_out) rstd_li_out[ti] = rstd_li;
        if (pre_out) memcpy(&pre_out[(size_t)ti * 4], pre, sizeof pre);
        if (post_out) memcpy(&post_out[(size_t)ti * 4], post, sizeof post);
        if (comb_out) memcpy(&comb_out[(size_t)ti * 16], comb, sizeof comb);
        free(xn);
        free(li);
    }
    return status;
}

/*
 * The non-shifted pre from a projection computed elsewhere ("pure" path):
 * mixes = sum over splits q (in order) of dot_mix[q][t][:], ssq likewise from
 * sqrsum[q][t] (FP64), then the coefficients and the collapse of X with the fresh
 * pre exactly as in oracle_run(shifted=0).  Outputs as in oracle_run (mixes_out
 * and ssq_out receive the summed values).
 */
int oracle_pre_from_mixes(int T, int d, int splits, const int* tok, int n_tok,
                          const uint16_t* X, const float* dot_mix, const float* sqrsum,
                          const float* scale, const float* base, const uint16_t* norm_w,
                          const oracle_params* p, uint16_t* layer_input, uint16_t* li_out,
                          double* mixes_out, double* ssq_out, double* rstd_out,
                          double* rstd_li_out, double* pre_out, double* post_out,
                          double* comb_out) {
    if (T <= 0 || d <= 0 || splits < 1 || n_tok < 0 || p->sinkhorn_iters < 1) return 1;
    for (int i = 0; i < n_tok; ++i)
        if (tok[i] < 0 || tok[i] >= T) return 2;
    const size_t K = (size_t)NHC * d;
    int status = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int ti = 0; ti < n_tok; ++ti) {
        const size_t t = (size_t)tok[ti];
        float* xn = (float*)malloc(sizeof(float) * K);
        float* li = (float*)malloc(sizeof(float) * d);
        if (!xn || !li) { free(xn); free(li); status = 3; continue; }
        for (size_t k = 0; k < K; ++k) xn[k] = bf16_to_f32(X[t * K + k]);
        double mix[NMIX], ssq = 0.0;
        for (int n = 0; n < NMIX; ++n) mix[n] = 0.0;
        for (int q = 0; q < splits; ++q) {
            for (int n = 0; n < NMIX; ++n) mix[n] += (double)dot_mix[((size_t)q * T + t) * NMIX + n];
            ssq += (double)sqrsum[(size_t)q * T + t];
        }
        double rstd, pre[4], post[4], comb[16];
        coefficients(mix, ssq, d, scale, base, p, &rstd, pre, post, comb);
        float pc[4];
        for (int j = 0; j < 4; ++j) pc[j] = (float)pre[j];
        double ssq_li, rstd_li;
        collapse(xn, pc, d, norm_w, p, li, &ssq_li, &rstd_li,
                 li_out ? &li_out[(size_t)ti * d] : NULL,
                 layer_input ? &layer_input[(size_t)ti * d] : NULL);
        if (mixes_out) memcpy(&mixes_out[(size_t)ti * NMIX], mix, sizeof mix);
        if (ssq_out) ssq_out[ti] = ssq;
        if (rstd_out) rstd_out[ti] = rstd;
        if (rstd_li_out) rstd_li_out[ti] = rstd_li;
        if (pre_out) memcpy(&pre_out[(size_t)ti * 4], pre, sizeof pre);
        if (post_out) memcpy(&post_out[(size_t)ti * 4], post, sizeof post);
        if (comb_out) memcpy(&comb_out[(size_t)ti * 16], comb, sizeof comb);
        free(xn);
        free(li);
    }
    return status;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
