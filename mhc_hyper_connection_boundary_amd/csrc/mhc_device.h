// Device-side building blocks of the mHC boundary for gfx950 (wave64, MFMA).
//
// Lane map used by every token-tile kernel.  A wave owns a tile of 16 tokens;
// lane l works on token n = l % 16 and on the 8 hidden elements
// h = 32*step + 8*g + [0, 8) with g = l / 16, for all four streams.  That is
// exactly the B operand of one v_mfma_f32_16x16x32_bf16 per stream (column =
// token, k group = g), so the updated residual feeds the matrix cores from
// registers.  The prepared weight supplies the matching A operands.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mhc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kTile = 16;          // tokens per wave tile (MFMA N)
constexpr int kStep = 32;          // hidden elements per wave step (MFMA K per stream)
constexpr int kPart = 32;          // floats per partial record: 24 mixes, ssq, ssq_li, pad
constexpr int kFragsPerStep = 12;  // 4 streams x 3 A tiles of 64 lanes x 16 bytes

struct Scalars {
    float rms_eps, pre_eps, post_mult, sinkhorn_eps;
    int sinkhorn_iters;
    float norm_eps;
};

// ---- LDS-poison debug build ------------------------------------------------
//
// Built with -DMHC_LDS_POISON (libmhc_lds_poison.so), every kernel starts by
// filling its workgroup's whole LDS allocation (the static arrays, plus
// dyn_bytes of dynamic LDS) with all-ones words, a NaN as FP32, so a read of
// LDS that the kernel never wrote turns its outputs into NaN instead of
// reusing whatever an earlier workgroup left there.  In the product build the
// macro is empty.
#ifdef MHC_LDS_POISON
__device__ __forceinline__ void poison_lds(unsigned dyn_bytes) {
    const unsigned words = (__builtin_amdgcn_groupstaticsize() + dyn_bytes) / 4;
    // (LDS address 0 from a run-time value: a literal 0 would be the null pointer)
    __attribute__((address_space(3))) unsigned* lds =
        (__attribute__((address_space(3))) unsigned*)(uintptr_t)__builtin_amdgcn_readfirstlane(0u);
    for (unsigned i = threadIdx.x; i < words; i += blockDim.x) lds[i] = 0xffffffffu;
    __syncthreads();
}
#define MHC_POISON_LDS(dyn_bytes) ::mhc::poison_lds(dyn_bytes)
#else
#define MHC_POISON_LDS(dyn_bytes) ((void)0)
#endif

// ---- BF16 <-> FP32 --------------------------------------------------------

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two FP32 values -> packed BF16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint32_t word(const uint4& v, int p) {
    return p == 0 ? v.x : p == 1 ? v.y : p == 2 ? v.z : v.w;
}
__device__ __forceinline__ void set_word(uint4& v, int p, uint32_t w) {
    if (p == 0) v.x = w; else if (p == 1) v.y = w; else if (p == 2) v.z = w; else v.w = w;
}

// ---- 16-byte global accesses ----------------------------------------------------
//
// kNt sets the nontemporal (streaming) hint.  Large batches stream the residual
// X, the block output x and the updated residual X' with it, which keeps them
// from displacing the layer input in the last-level cache between the kernel
// that writes it and the one that reads it back (and measured faster on its
// own: a tile-major mover of the boundary's bytes went from 5.43 to 5.71 TB/s).
template <bool kNt>
__device__ __forceinline__ uint4 ld16(const void* p) {
    if constexpr (kNt) {
        const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
        return make_uint4(v[0], v[1], v[2], v[3]);
    } else {
        return *reinterpret_cast<const uint4*>(p);
    }
}

template <bool kNt>
__device__ __forceinline__ void st16(void* p, const uint4& v) {
    if constexpr (kNt) {
        const u32x4_t w = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
    } else {
        *reinterpret_cast<uint4*>(p) = v;
    }
}

// ---- per-token coefficients of the previous layer ---------------------------

struct PrevCoef {
    float post[4];
    float comb[16];  // comb[4*j + s]: source stream j -> destination stream s
    float pre[4];    // lagged pre
};

__device__ __forceinline__ void load_prev(PrevCoef& c, const float* __restrict__ post_prev,
                                          const float* __restrict__ comb_prev,
                                          const float* __restrict__ pre_lag, size_t t) {
    const float4 p = *reinterpret_cast<const float4*>(post_prev + t * 4);
    const float4 q = *reinterpret_cast<const float4*>(pre_lag + t * 4);
    c.post[0] = p.x; c.post[1] = p.y; c.post[2] = p.z; c.post[3] = p.w;
    c.pre[0] = q.x; c.pre[1] = q.y; c.pre[2] = q.z; c.pre[3] = q.w;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float4 r = *reinterpret_cast<const float4*>(comb_prev + t * 16 + 4 * j);
        c.comb[4 * j + 0] = r.x; c.comb[4 * j + 1] = r.y;
        c.comb[4 * j + 2] = r.z; c.comb[4 * j + 3] = r.w;
    }
}

// ---- residual update + lagged collapse for 8 hidden elements ------------------
//
// X'[s] = bf16(FMA chain over j of comb[j][s]*X[j], from post[s]*x)   (FP32)
// li    = bf16(FMA chain over j of pre[j]*X'[j], from 0)              (FP32)
// ssq += X'^2 (BF16 values), ssq_li += li^2 (BF16 values).
__device__ __forceinline__ void update_collapse(const uint4 (&X)[4], const uint4& xw,
                                                const PrevCoef& c, uint4 (&Xn)[4], uint4& li,
                                                float& ssq, float& ssq_li) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t xp = word(xw, p);
        const float xv[2] = {bf_lo(xp), bf_hi(xp)};
        float Xv[4][2];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t w = word(X[j], p);
            Xv[j][0] = bf_lo(w);
            Xv[j][1] = bf_hi(w);
        }
        float r[4][2];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            float nu[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                nu[e] = c.post[s] * xv[e];
#pragma unroll
                for (int j = 0; j < 4; ++j) nu[e] = __builtin_fmaf(c.comb[4 * j + s], Xv[j][e], nu[e]);
            }
            const uint32_t packed = pack_bf16(nu[0], nu[1]);
            set_word(Xn[s], p, packed);
            r[s][0] = bf_lo(packed);
            r[s][1] = bf_hi(packed);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            ssq = __builtin_fmaf(r[s][0], r[s][0], ssq);
            ssq = __builtin_fmaf(r[s][1], r[s][1], ssq);
        }
        float acc[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            acc[e] = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[e] = __builtin_fmaf(c.pre[j], r[j][e], acc[e]);
        }
        const uint32_t lw = pack_bf16(acc[0], acc[1]);
        set_word(li, p, lw);
        const float l0 = bf_lo(lw), l1 = bf_hi(lw);
        ssq_li = __builtin_fmaf(l0, l0, ssq_li);
        ssq_li = __builtin_fmaf(l1, l1, ssq_li);
    }
}

// Sum of squares of 4 streams x 8 BF16 values (non-shifted pre: X' = X).
__device__ __forceinline__ void square_sum(const uint4 (&X)[4], float& ssq) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t w = word(X[s], p);
            const float a = bf_lo(w), b = bf_hi(w);
            ssq = __builtin_fmaf(a, a, ssq);
            ssq = __builtin_fmaf(b, b, ssq);
        }
}

// ---- projection on the matrix cores -------------------------------------------

// One step: for each stream s, acc[m] += A(step, s, m) x X'[s] for the 3 A tiles.
__device__ __forceinline__ void mfma_step(const uint4 (&A)[kFragsPerStep], const uint4 (&Xn)[4],
                                          f32x4_t (&acc)[3]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const bf16x8_t b = __builtin_bit_cast(bf16x8_t, Xn[s]);
#pragma unroll
        for (int m = 0; m < 3; ++m) {
            const bf16x8_t a = __builtin_bit_cast(bf16x8_t, A[s * 3 + m]);
            acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[m], 0, 0, 0);
        }
    }
}

// Lane (n, g) holds, after the projection, result rows 4g..4g+3 of each A tile
// for token n: rows 4g / 4g+2 are the high / low products of mix 8m+2g, rows
// 4g+1 / 4g+3 those of mix 8m+2g+1.  mix_of(acc, m, j) is mix 8m + 2g + j.
__device__ __forceinline__ float mix_of(const f32x4_t (&acc)[3], int m, int j) {
    return acc[m][j] + acc[m][j + 2];
}

// ---- quad exchange (lanes 4q..4q+3) ----------------------------------------------

// Value of the lane whose index differs in bit 0 / bit 1 (DPP quad_perm).
__device__ __forceinline__ float quad_xor1(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_xor2(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 0x4E, 0xF, 0xF, false));
}

__device__ __forceinline__ float sigmoid(float v) { return 1.0f / (1.0f + expf(-v)); }

// 1/x for a positive normal x: the hardware estimate (v_rcp_f32, within 1 ulp)
// refined by one Newton-Raphson step r + r(1 - x r).  Used for the softmax sum
// of the comb logits, which lies in [1, 4].
__device__ __forceinline__ float recip(float x) {
    const float r = __builtin_amdgcn_rcpf(x);
    return __builtin_fmaf(r, __builtin_fmaf(-x, r, 1.0f), r);
}

// Coefficients of one token, computed by the 4 lanes of a quad: lane i of the
// quad owns row i of comb and pre[i], post[i].  tot points at the token's
// reduced record (24 mixes, then the sum of squares).  Column sums use the
// (r0 + r1) + (r2 + r3) order, row sums ((c0 + c1) + c2) + c3; each
// normalisation multiplies by the reciprocal of (sum + eps) (see recip).
struct TokenCoef {
    float rstd, pre, post;
    float row[4];
};

// 1/sqrt(x): the hardware estimate (v_rsq_f32, about 1 ulp) refined by one
// Newton-Raphson step y(1.5 - 0.5 x y^2); x below the smallest normal takes the
// IEEE path.  Used for rstd and rstd_li, whose arguments are sums of squares
// plus eps.
__device__ __forceinline__ float rsqrt_nr(float x) {
    if (!(x >= 1.17549435e-38f)) return 1.0f / sqrtf(x);
    const float y = __builtin_amdgcn_rsqf(x);
    return y * __builtin_fmaf(-0.5f * x * y, y, 1.5f);
}

// scale[0..2] and the bases of coefficient row i (pre[i], post[i], comb row
// i), loaded by the lane that will compute that row, ahead of the reductions.
struct CoefParams {
    float s0, s1, s2, bpre, bpost;
    float bcomb[4];
};

__device__ __forceinline__ CoefParams load_coef_params(const float* __restrict__ scale,
                                                       const float* __restrict__ base, int i) {
    CoefParams c;
    c.s0 = scale[0];
    c.s1 = scale[1];
    c.s2 = scale[2];
    c.bpre = base[i];
    c.bpost = base[4 + i];
    const float4 b = *reinterpret_cast<const float4*>(base + 8 + 4 * i);
    c.bcomb[0] = b.x; c.bcomb[1] = b.y; c.bcomb[2] = b.z; c.bcomb[3] = b.w;
    return c;
}

// rstd, pre[i] and post[i] of a token: the cheap part of the coefficients,
// which the collapse of the non-shifted pre waits for.
__device__ __forceinline__ void pre_post(TokenCoef& o, const float* tot, int i, int hidden,
                                         const CoefParams& cp, const Scalars& p) {
    o.rstd = rsqrt_nr(tot[24] * (0.25f / (float)hidden) + p.rms_eps);
    o.pre = sigmoid(__builtin_fmaf(tot[i] * o.rstd, cp.s0, cp.bpre)) + p.pre_eps;
    o.post = sigmoid(__builtin_fmaf(tot[4 + i] * o.rstd, cp.s1, cp.bpost)) * p.post_mult;
}

// Row i of the Sinkhorn comb (needs o.rstd from pre_post; all 4 lanes of the
// quad must call it together).
__device__ __forceinline__ void comb_row(TokenCoef& o, const float* tot, int i,
                                         const CoefParams& cp, const Scalars& p) {
    float v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = __builtin_fmaf(tot[8 + 4 * i + k] * o.rstd, cp.s2, cp.bcomb[k]);
    const float mx = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
    float e[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) e[k] = expf(v[k] - mx);
    const float inv = recip(((e[0] + e[1]) + e[2]) + e[3]);
    float c[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) c[k] = __builtin_fmaf(e[k], inv, p.sinkhorn_eps);
    for (int it = 0; it < p.sinkhorn_iters; ++it) {
        // The iterations use the bare hardware reciprocal (within 1 ulp): the
        // normalisations are a contraction, so each step's rounding is damped
        // by the ones after it, and the dependent chain is 2 FMAs shorter per
        // normalisation than with a Newton step (measured: the same largest
        // comb error against the oracle, 2e-7 on the peaked stress logits).
        if (it > 0) {
            const float rinv = __builtin_amdgcn_rcpf((((c[0] + c[1]) + c[2]) + c[3]) + p.sinkhorn_eps);
#pragma unroll
            for (int k = 0; k < 4; ++k) c[k] *= rinv;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float s = c[k] + quad_xor1(c[k]);      // rows (0+1) and (2+3)
            s = s + quad_xor2(s);                   // (0+1) + (2+3)
            c[k] *= __builtin_amdgcn_rcpf(s + p.sinkhorn_eps);
        }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) o.row[k] = c[k];
}

// Rotations within a DPP row of 16 lanes.
__device__ __forceinline__ float row_ror8(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 0x128, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_ror4(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 0x124, 0xF, 0xF, false));
}

// The Sinkhorn comb of one token on the 16 lanes of one DPP row (all 16 must
// call it together): lane 4i + k owns element (i, k) and returns it.  Row
// sums run (c0 + c1) + (c2 + c3) over the quad, column sums (r0 + r2) +
// (r1 + r3) through rotations by 8 and 4 lanes; additions commute, so every
// lane of a row or column gets the same bits.  The softmax's row maximum and
// sum follow the same pattern.  Each iteration is a chain of about 10
// instructions against about 30 when one lane owns a row.
__device__ __forceinline__ float comb16(const float* tot, int lane16, float rstd, float s2,
                                        float bcomb, const Scalars& p) {
    const float v = __builtin_fmaf(tot[8 + lane16] * rstd, s2, bcomb);
    float mx = fmaxf(v, quad_xor1(v));
    mx = fmaxf(mx, quad_xor2(mx));
    const float e = expf(v - mx);
    float se = e + quad_xor1(e);
    se = se + quad_xor2(se);
    float c = __builtin_fmaf(e, recip(se), p.sinkhorn_eps);
    for (int it = 0; it < p.sinkhorn_iters; ++it) {
        // (the bare hardware reciprocal, as in comb_row)
        if (it > 0) {
            float r = c + quad_xor1(c);
            r = r + quad_xor2(r);
            c *= __builtin_amdgcn_rcpf(r + p.sinkhorn_eps);
        }
        float q = c + row_ror8(c);
        q = q + row_ror4(q);
        c *= __builtin_amdgcn_rcpf(q + p.sinkhorn_eps);
    }
    return c;
}

__device__ __forceinline__ TokenCoef coefficients(const float* tot, int i, int hidden,
                                                  const CoefParams& cp, const Scalars& p) {
    TokenCoef o;
    pre_post(o, tot, i, hidden, cp, p);
    comb_row(o, tot, i, cp, p);
    return o;
}

}  // namespace mhc
