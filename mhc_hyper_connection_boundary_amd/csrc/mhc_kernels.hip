// gfx950 kernels of the mHC boundary and their host-side launchers.
//
// Split schedule (any token count):
//   k_partial   one workgroup = 4 waves on a tile of one, two or four 16-token
//               groups and a slice of hidden, in steps of 128 elements of every
//               row: the rows are split over the waves for the 16-byte loads
//               of X and x, the residual update, the lagged collapse and the
//               stores of X' and li (4 rows x 256 bytes per instruction); X'
//               reaches the matrix cores through LDS, where each wave projects
//               one 32-element k-block of the step for every group from one
//               set of weight fragments.  The waves' partials are combined in
//               a fixed order and written as one record per (token, slice).
//   k_partial_pre_wide  the non-shifted pre's four-group form with 64-element
//               wave steps (both 64-byte halves of each 128-byte line per
//               lane), for plans with an even number of 32-element steps.
//   k_finish    one workgroup per (tile, hidden slice): sums the records of
//               its tokens over the slices in slice order, forms rstd_li and
//               rescales li into the layer input; it also computes pre /
//               post / Sinkhorn comb of one or more of the tile's tokens.
//   k_pre_finish (non-shifted pre) one workgroup per token: coefficients
//               first, then the collapse with the fresh pre and the RMSNorm.
// Weight preparation: k_prepare_weight.
#include <atomic>

#include "mhc_device.h"
#include "mhc_launch.h"

namespace mhc {
namespace {

// ---------------------------------------------------------------------------
// Weight preparation: one thread per 16-byte A-operand word (8 BF16).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float tf32_ties_away(float w) {
    return __uint_as_float((__float_as_uint(w) + 0x1000u) & 0xFFFFE000u);
}

__global__ __launch_bounds__(256) void k_prepare_weight(const float* __restrict__ w, int hidden,
                                                        uint4* __restrict__ out, int n_words) {
    const int o = blockIdx.x * blockDim.x + threadIdx.x;
    if (o >= n_words) return;
    const int l = o % 64;
    const int m = (o / 64) % 3;
    const int s = (o / 192) % 4;
    const int step = o / 768;
    const int r = l % 16;
    const int mix = 8 * m + 2 * (r / 4) + (r % 2);
    const bool high = (r % 4) < 2;
    const size_t k = (size_t)s * hidden + 32 * step + 8 * (l / 16);
    const float* src = w + (size_t)mix * 4 * hidden + k;
    uint32_t words[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        float part[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const float t = tf32_ties_away(src[2 * p + e]);
            const float hi = bf_lo((uint32_t)(pack_bf16(t, 0.0f) & 0xFFFFu));
            part[e] = high ? hi : t - hi;
        }
        words[p] = pack_bf16(part[0], part[1]);
    }
    out[o] = make_uint4(words[0], words[1], words[2], words[3]);
}

// ---------------------------------------------------------------------------
// Split schedule, kernel 1: partial sums of a tile of 16G tokens over a slice
// of hidden (SHIFTED: the boundary; otherwise the non-shifted pre, which only
// reads X), one record per (token, slice).  A workgroup step covers 4
// k-blocks (128 hidden elements) of every row of the tile; the slice holds
// steps_per_wave of them (ONE: exactly one, so no next-step buffers: the
// plans of decode sizes and of INVARIANT, at 136 registers with one group and
// 216 with two instead of 196 and 306).  Wave w loads, updates, stores and
// collapses tokens 16r + 4w .. 16r + 4w + 3 of the tile (r < G), lane L on
// token 16r + 4w + L/16 and 16-byte chunk L%16 of the step's 256-byte run, so
// each load and store instruction covers 4 rows x 256 bytes (a plain mover:
// 5.37 TB/s, against 4.60 for the 16 rows x 64 bytes of the matrix-core
// layout).  X' goes to a double-buffered LDS stage ([group][token][stream]
// [chunk], chunks XOR-swizzled by the token: no bank conflicts either way),
// from which wave w reads k-block w of the step for the projection after one
// barrier; the buffer a step writes was last read before the previous step's
// barrier.  Wave w projects k-blocks first + w, first + 4 + w, ... of its
// slice for all G groups from one set of weight fragments per k-block.  A
// token's sums of squares belong to one wave (a butterfly over its 16 lanes),
// the same order for every G and every position in the tile, so INVARIANT's
// bits do not depend on the batch.  Against the earlier form of this kernel,
// which loaded in the matrix-core layout (16 rows x 64 bytes per instruction),
// cold, d=7168, us: boundary T=32 10.95 -> 10.51, T=128 15.2 -> 14.3, T=512
// 31.7 -> 28.5, T=1024 51.7 -> 44.7, T=2048 88.8 -> 79.3; INVARIANT T=1024
// 61.1 -> 51.1, T=8192 419 -> 353; pre T=32 9.87 -> 9.62, T=2048 60.1 -> 56.7.
// ---------------------------------------------------------------------------
template <bool SHIFTED, int G, bool NT, bool ONE>
__global__ __launch_bounds__(256) void k_partial(
    int T, int hidden, int steps_per_wave, int slices, const uint16_t* __restrict__ x,
    const uint16_t* __restrict__ X, const float* __restrict__ post_prev,
    const float* __restrict__ comb_prev, const float* __restrict__ pre_lag,
    const uint4* __restrict__ wprep, uint16_t* __restrict__ xn_out,
    uint16_t* __restrict__ li_out, float* __restrict__ part) {
    MHC_POISON_LDS(0);
    constexpr int kTok = kTile * G;  // tokens of the workgroup
    constexpr int kGroupStage = kTile * 4 * 16;  // one group's X' of a step: [token][stream][chunk]
    __shared__ uint4 stage[2][G][kGroupStage];
    __shared__ float red[4][kTok][24];
    __shared__ float sqo[kTok][2];

    const int tile = blockIdx.x / slices;  // (tile-major grid)
    const int slice = blockIdx.x - tile * slices;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int n = lane & 15;
    const int g = lane >> 4;
    const int ch = lane & 15;                 // the lane's chunk of the step's run
    const int t4 = 4 * wave + (lane >> 4);   // the lane's token within each group
    // A lane past the last token works on token T-1 and stores nothing.
    bool own[G];
    size_t tok[G];
    PrevCoef c[G];
#pragma unroll
    for (int r = 0; r < G; ++r) {
        const int t = tile * kTok + 16 * r + t4;
        own[r] = t < T;
        tok[r] = own[r] ? (size_t)t : (size_t)(T - 1);
        if (SHIFTED) load_prev(c[r], post_prev, comb_prev, pre_lag, tok[r]);
    }

    // The slice covers k-blocks [first, last), a whole number of workgroup
    // steps (hidden is a multiple of 256).
    const int nsteps = hidden / kStep;
    const int first = slice * 4 * steps_per_wave;
    const int last = min(first + 4 * steps_per_wave, nsteps);
    const int wsteps = ONE ? 1 : (last - first) / 4;

    f32x4_t acc[G][3];
    float ssq[G], ssq_li[G];
#pragma unroll
    for (int q = 0; q < G; ++q) {
#pragma unroll
        for (int m = 0; m < 3; ++m) acc[q][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        ssq[q] = 0.0f;
        ssq_li[q] = 0.0f;
    }

    // Step j's weight fragments are requested first, then step j+1's
    // activations: loads complete in issue order, so the projection never
    // waits on HBM.
    auto load_step = [&](uint4 (&Xv)[G][4], uint4 (&xv)[G], int j) {
        const int h = (first + 4 * j) * kStep + 8 * ch;
#pragma unroll
        for (int r = 0; r < G; ++r) {
#pragma unroll
            for (int s = 0; s < 4; ++s) Xv[r][s] = ld16<NT>(X + (tok[r] * 4 + s) * hidden + h);
            xv[r] = make_uint4(0, 0, 0, 0);
            if (SHIFTED) xv[r] = ld16<NT>(x + tok[r] * hidden + h);
        }
    };
    uint4 Xv[G][4], xv[G];
    load_step(Xv, xv, 0);
    for (int j = 0; j < wsteps; ++j) {
        uint4 A[kFragsPerStep];
        const uint4* wp = wprep + (size_t)(first + 4 * j + wave) * kFragsPerStep * 64 + lane;
#pragma unroll
        for (int i = 0; i < kFragsPerStep; ++i) A[i] = wp[i * 64];
        __builtin_amdgcn_sched_barrier(0);
        uint4 Xnx[G][4], xnx[G];
        if (!ONE && j + 1 < wsteps) load_step(Xnx, xnx, j + 1);
        __builtin_amdgcn_sched_barrier(0);

        const int h = (first + 4 * j) * kStep + 8 * ch;
        uint4* st = &stage[j & 1][0][0];
#pragma unroll
        for (int r = 0; r < G; ++r) {
            uint4 Xn[4];
            if (SHIFTED) {
                uint4 li;
                update_collapse(Xv[r], xv[r], c[r], Xn, li, ssq[r], ssq_li[r]);
                if (own[r]) {
#pragma unroll
                    for (int s = 0; s < 4; ++s) st16<NT>(xn_out + (tok[r] * 4 + s) * hidden + h, Xn[s]);
                    *reinterpret_cast<uint4*>(li_out + tok[r] * hidden + h) = li;
                }
            } else {
#pragma unroll
                for (int s = 0; s < 4; ++s) Xn[s] = Xv[r][s];
                square_sum(Xv[r], ssq[r]);
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) st[r * kGroupStage + (t4 * 4 + s) * 16 + (ch ^ t4)] = Xn[s];
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < G; ++q) {
            uint4 B[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) B[s] = st[q * kGroupStage + (n * 4 + s) * 16 + ((4 * wave + g) ^ n)];
            mfma_step(A, B, acc[q]);
        }
#pragma unroll
        for (int r = 0; r < G; ++r) {
#pragma unroll
            for (int s = 0; s < 4; ++s) Xv[r][s] = Xnx[r][s];
            xv[r] = xnx[r];
        }
    }

    // Mixes: the 4 waves in a fixed order.  Sums of squares: the owning
    // wave's 16 lanes of each token (every lane ends with the same bits).
#pragma unroll
    for (int q = 0; q < G; ++q)
#pragma unroll
        for (int m = 0; m < 3; ++m)
#pragma unroll
            for (int j = 0; j < 2; ++j) red[wave][16 * q + n][8 * m + 2 * g + j] = mix_of(acc[q], m, j);
#pragma unroll
    for (int r = 0; r < G; ++r) {
        float a = ssq[r], b = ssq_li[r];
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) {
            a += __shfl_xor(a, o);
            b += __shfl_xor(b, o);
        }
        if (ch == 0) {
            sqo[16 * r + t4][0] = a;
            sqo[16 * r + t4][1] = b;
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kTok * 26; i += blockDim.x) {
        const int tn = i / 26, v = i % 26;
        const float sum = v < 24 ? ((red[0][tn][v] + red[1][tn][v]) + red[2][tn][v]) + red[3][tn][v]
                                 : sqo[tn][v - 24];
        const int tt = tile * kTok + tn;
        if (tt < T) part[((size_t)tt * slices + slice) * kPart + v] = sum;
    }
}

// Non-shifted partial kernel with 64-element wave steps: two 32-element
// k-blocks per step, every lane reading both 64-byte halves of each 128-byte
// line it touches, as in the fused kernels.  Launched for four token groups
// and an even number of 32-element steps per wave (the slice then holds
// whole 64-element steps); its records hold the sums of k_partial's, in
// another order within the slice.  (With two groups it would need 306
// registers, one workgroup per CU instead of two, and measured slower.)
template <int G, bool NT>
__global__ __launch_bounds__(256) void k_partial_pre_wide(
    int T, int hidden, int steps_per_wave, int slices, const uint16_t* __restrict__ X,
    const uint4* __restrict__ wprep, float* __restrict__ part) {
    MHC_POISON_LDS(0);
    constexpr int kTok = kTile * G;
    __shared__ float red[4][kTok][24];
    __shared__ float sq[4][4][kTok];

    const int tile = blockIdx.x / slices;  // (tile-major grid)
    const int slice = blockIdx.x - tile * slices;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int n = lane & 15;
    const int g = lane >> 4;
    const uint16_t* Xrow[G];
#pragma unroll
    for (int q = 0; q < G; ++q) {
        const int t = tile * kTok + 16 * q + n;
        Xrow[q] = X + (size_t)(t < T ? t : T - 1) * 4 * hidden;
    }

    // The slice covers 32-element steps [first, last), both even: 64-element
    // steps [first / 2, last / 2), wave w taking first / 2 + w, + 4, ...
    const int nsteps = hidden / kStep;
    const int first = slice * 4 * steps_per_wave;
    const int last = min(first + 4 * steps_per_wave, nsteps);
    const int wlast = last / 2;

    f32x4_t acc[G][3];
    float ssq[G];
#pragma unroll
    for (int q = 0; q < G; ++q) {
#pragma unroll
        for (int m = 0; m < 3; ++m) acc[q][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        ssq[q] = 0.0f;
    }

    auto load_w = [&](uint4 (&a)[2][4], int q, int ws) {
        const int h = ws * 2 * kStep + g * 8;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            a[0][j] = ld16<NT>(Xrow[q] + (size_t)j * hidden + h);
            a[1][j] = ld16<NT>(Xrow[q] + (size_t)j * hidden + h + kStep);
        }
    };
    uint4 cur[G][2][4];
    if (first / 2 + wave < wlast) {
#pragma unroll
        for (int q = 0; q < G; ++q) load_w(cur[q], q, first / 2 + wave);
    }
    for (int ws = first / 2 + wave; ws < wlast; ws += 4) {
        uint4 A0[kFragsPerStep], A1[kFragsPerStep];
        const uint4* wp = wprep + (size_t)(2 * ws) * kFragsPerStep * 64 + lane;
#pragma unroll
        for (int i = 0; i < kFragsPerStep; ++i) {
            A0[i] = wp[i * 64];
            A1[i] = wp[(kFragsPerStep + i) * 64];
        }
        __builtin_amdgcn_sched_barrier(0);
        uint4 nxt[G][2][4];
        if (ws + 4 < wlast) {
#pragma unroll
            for (int q = 0; q < G; ++q) load_w(nxt[q], q, ws + 4);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < G; ++q) {
            square_sum(cur[q][0], ssq[q]);
            square_sum(cur[q][1], ssq[q]);
            mfma_step(A0, cur[q][0], acc[q]);
            mfma_step(A1, cur[q][1], acc[q]);
        }
#pragma unroll
        for (int q = 0; q < G; ++q)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int j = 0; j < 4; ++j) cur[q][b][j] = nxt[q][b][j];
    }

    // Combine the 4 waves in a fixed order: waves ascending, lane groups ascending.
#pragma unroll
    for (int q = 0; q < G; ++q) {
#pragma unroll
        for (int m = 0; m < 3; ++m)
#pragma unroll
            for (int j = 0; j < 2; ++j) red[wave][16 * q + n][8 * m + 2 * g + j] = mix_of(acc[q], m, j);
        sq[wave][g][16 * q + n] = ssq[q];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kTok * 26; i += blockDim.x) {
        const int tn = i / 26, v = i % 26;
        float sum;
        if (v < 24) {
            sum = ((red[0][tn][v] + red[1][tn][v]) + red[2][tn][v]) + red[3][tn][v];
        } else if (v == 24) {
            sum = 0.0f;
            for (int w = 0; w < 4; ++w)
                for (int q = 0; q < 4; ++q) sum += sq[w][q][tn];
        } else {
            sum = 0.0f;
        }
        const int tt = tile * kTok + tn;
        if (tt < T) part[((size_t)tt * slices + slice) * kPart + v] = sum;
    }
}

// ---------------------------------------------------------------------------
// Split schedule, kernel 2: totals, coefficients, layer input.
//
// Sum over slices q = first, first + stride, ... < count of part[t][q][v], q
// ascending.  The loads are issued in batches of 8 so they overlap; the
// additions keep the slice order.  slice_first requests the first batch (the
// only one unless count > 8 * stride) at addresses clamped to the last slice,
// so that a caller can request several sums before waiting and no load sits
// under a branch (after a conditional block that loads, the compiler waits
// for every outstanding load); slice_rest adds it and any further batches.
// count >= 1.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void slice_first(float (&v)[8], const float* __restrict__ src,
                                            int first, int stride, int count,
                                            size_t elem_stride = kPart) {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = src[(size_t)min(first + k * stride, count - 1) * elem_stride];
}

__device__ __forceinline__ float slice_rest(const float (&v)[8], const float* __restrict__ src,
                                            int first, int stride, int count,
                                            size_t elem_stride = kPart) {
    float sum = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) sum = first + k * stride < count ? sum + v[k] : sum;
    for (int q0 = first + 8 * stride; q0 < count; q0 += 8 * stride) {
        float w[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) w[k] = src[(size_t)min(q0 + k * stride, count - 1) * elem_stride];
#pragma unroll
        for (int k = 0; k < 8; ++k) sum = q0 + k * stride < count ? sum + w[k] : sum;
    }
    return sum;
}

__device__ __forceinline__ float slice_sum(const float* __restrict__ src, int first, int stride,
                                           int count, size_t elem_stride = kPart) {
    float v[8];
    slice_first(v, src, first, stride, count, elem_stride);
    return slice_rest(v, src, first, stride, count, elem_stride);
}

// Remaining coefficient tokens of a workgroup (tokens hs + k*finish_slices,
// k >= 1), when there are fewer than 16 rescale workgroups per tile: all at
// once, 16 lanes per token, with the same two-level slice order and the same
// comb arithmetic as the first token.
__device__ __forceinline__ void finish_more_coefficients(
    int T, int hidden, int slices, int finish_slices, int tile, int hs, int tid,
    const float* __restrict__ part, const float* __restrict__ scale,
    const float* __restrict__ base, const Scalars& p, float (*mred)[8][26],
    float (*mtot)[26], float* __restrict__ pre_out, float* __restrict__ post_out,
    float* __restrict__ comb_out, float* __restrict__ mixes_out, float* __restrict__ rstd_out) {
    const int nk = (kTile - 1 - hs) / finish_slices;  // tokens hs + (k + 1) * finish_slices
    if (nk <= 0) return;
    const int first = tile * kTile + hs + finish_slices;
    for (int item = tid; item < nk * 200; item += blockDim.x) {
        const int k = item / 200, r = item % 200, grp = r / 25, v = r % 25;
        const int t = first + k * finish_slices;
        mred[k][grp][v] =
            t < T ? slice_sum(part + (size_t)t * slices * kPart + v, grp, 8, slices) : 0.0f;
    }
    __syncthreads();
    for (int item = tid; item < nk * 25; item += blockDim.x) {
        const int k = item / 25, v = item % 25;
        float sum = 0.0f;
        for (int q = 0; q < 8; ++q) sum += mred[k][q][v];
        mtot[k][v] = sum;
    }
    __syncthreads();
    if (tid < 16 * nk) {  // 16 lanes per token, as for the first token
        const int k = tid >> 4, l16 = tid & 15, i = tid & 3;
        const int t = first + k * finish_slices;
        const CoefParams cp = load_coef_params(scale, base, i);
        TokenCoef o;
        pre_post(o, mtot[k], i, hidden, cp, p);
        const float c = comb16(mtot[k], l16, o.rstd, cp.s2, base[8 + l16], p);
        if (t < T) {
            comb_out[(size_t)t * 16 + l16] = c;
            if (l16 < 4) {
                pre_out[(size_t)t * 4 + i] = o.pre;
                post_out[(size_t)t * 4 + i] = o.post;
                if (mixes_out)
                    for (int kk = 0; kk < 6; ++kk) mixes_out[(size_t)t * 24 + 6 * i + kk] = mtot[k][6 * i + kk];
                if (rstd_out && i == 0) rstd_out[t] = o.rstd;
            }
        }
    }
}

// Workgroup (tile, hs): rstd_li of the tile's 16 tokens; the coefficients of
// tokens hs, hs + finish_slices, ... of the tile; li -> layer input over hidden
// [hs*width, (hs+1)*width).  Every reduction over slices is a fixed two-level
// order: interleaved groups summed in slice order, then the groups in order.
// The partial records, li and norm_w of the first coefficient token and of the
// first two rescale chunks of every thread are all requested before the first
// wait, so the kernel pays about one memory round trip.
__global__ __launch_bounds__(256) void k_finish(
    int T, int hidden, int slices, int finish_slices, int slice_width,
    const float* __restrict__ part, const float* __restrict__ scale,
    const float* __restrict__ base, const uint16_t* __restrict__ norm_w, Scalars p,
    uint16_t* __restrict__ layer_input, float* __restrict__ pre_out,
    float* __restrict__ post_out, float* __restrict__ comb_out, float* __restrict__ mixes_out,
    float* __restrict__ rstd_out) {
    MHC_POISON_LDS(0);
    __shared__ float lsum[kTile][16];
    __shared__ float rli[kTile];
    __shared__ float cred[8][26];
    __shared__ float ctot[26];
    __shared__ float mred[kTile - 1][8][26];
    __shared__ float mtot[kTile - 1][26];

    const int tile = blockIdx.x / finish_slices;  // (tile-major grid)
    const int hs = blockIdx.x - tile * finish_slices;
    const int tid = threadIdx.x;
    const int h0 = hs * slice_width;
    const int width = max(0, min(slice_width, hidden - h0));
    const int chunks = width / 8;

    // All loads go first, none under a branch: the coefficient parameters, the
    // rescale chunks u = tid and tid + 256 (the common case), then the first
    // batches of the slice sums.  Lanes without work read one shared address
    // (so their requests coalesce) and their results are dropped.
    const CoefParams cp = load_coef_params(scale, base, tid & 3);
    const float bcomb = base[8 + (tid & 15)];
    const uint16_t* nw_src = norm_w ? norm_w : layer_input;
    uint4 li_v[2], nw_v[2];
    bool have[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int u = tid + k * (int)blockDim.x;
        const int tn = chunks ? u / chunks : kTile, cidx = chunks ? u % chunks : 0;
        have[k] = norm_w && u < kTile * chunks && tile * kTile + tn < T;
        const size_t t = have[k] ? (size_t)(tile * kTile + tn) : 0;
        const int h = have[k] ? h0 + cidx * 8 : 0;
        li_v[k] = *reinterpret_cast<const uint4*>(layer_input + t * hidden + h);
        nw_v[k] = *reinterpret_cast<const uint4*>(nw_src + h);
    }

    // Phase 1: partial sums of li squares (thread (tn, group) adds slices
    // group, group + 16, ...) and of the first coefficient token's 25 values
    // (thread (v, group) adds slices group, group + 8, ...).
    const int ltn = tid >> 4, lgrp = tid & 15;
    const int lt = tile * kTile + ltn;
    const float* lsrc = part + (size_t)min(lt, T - 1) * slices * kPart + 25;
    float lv[8];
    slice_first(lv, lsrc, lgrp, 16, slices);
    const int t_first = tile * kTile + hs;
    const bool coef_first = hs < kTile && t_first < T;
    // (first = slices: every request clamps to the last slice of token 0)
    const float* csrc = coef_first ? part + (size_t)t_first * slices * kPart + min(tid & 31, 24) : part;
    const int cfirst = coef_first ? tid >> 5 : slices;
    float cv[8];
    slice_first(cv, csrc, cfirst, 8, slices);
    const float ls = slice_rest(lv, lsrc, lgrp, 16, slices);
    const float cs = slice_rest(cv, csrc, cfirst, 8, slices);
    lsum[ltn][lgrp] = lt < T ? ls : 0.0f;
    if (coef_first && (tid & 31) < 25) cred[tid >> 5][tid & 31] = cs;
    __syncthreads();
    // Phase 2: totals.
    if (tid < kTile) {
        float sum = 0.0f;
        for (int grp = 0; grp < 16; ++grp) sum += lsum[tid][grp];
        rli[tid] = rsqrt_nr(sum * (1.0f / (float)hidden) + p.norm_eps);
    } else if (tid >= 32 && tid < 32 + 25 && coef_first) {
        float sum = 0.0f;
        for (int q = 0; q < 8; ++q) sum += cred[q][tid - 32];
        ctot[tid - 32] = sum;
    }
    __syncthreads();
    // Phase 3: 16 lanes of wave 0 run the coefficients of the first token (the
    // Sinkhorn comb on all of them, pre / post on the first 4) while the other
    // waves rescale li.
    auto emit_coef = [&](int t) {
        TokenCoef o;
        pre_post(o, ctot, tid & 3, hidden, cp, p);
        comb_out[(size_t)t * 16 + tid] = comb16(ctot, tid, o.rstd, cp.s2, bcomb, p);
        if (tid < 4) {
            pre_out[(size_t)t * 4 + tid] = o.pre;
            post_out[(size_t)t * 4 + tid] = o.post;
            if (mixes_out)
                for (int k = 0; k < 6; ++k) mixes_out[(size_t)t * 24 + 6 * tid + k] = ctot[6 * tid + k];
            if (rstd_out && tid == 0) rstd_out[t] = o.rstd;
        }
    };
    if (coef_first && tid < 16) emit_coef(t_first);

    auto rescale = [&](int u, const uint4& li, const uint4& nw) {
        const int tn = u / chunks, cidx = u % chunks;
        const float r = rli[tn];
        uint4 out;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t a = word(li, q), b = word(nw, q);
            set_word(out, q, pack_bf16((bf_lo(a) * r) * bf_lo(b), (bf_hi(a) * r) * bf_hi(b)));
        }
        *reinterpret_cast<uint4*>(layer_input + (size_t)(tile * kTile + tn) * hidden + h0 + cidx * 8) = out;
    };
    if (norm_w) {  // (without norm_w, layer_input already holds li)
#pragma unroll
        for (int k = 0; k < 2; ++k)
            if (have[k]) rescale(tid + k * (int)blockDim.x, li_v[k], nw_v[k]);
        for (int u = tid + 2 * (int)blockDim.x; u < kTile * chunks; u += (int)blockDim.x) {
            if (tile * kTile + u / chunks >= T) break;
            const int h = h0 + (u % chunks) * 8;
            const uint4 li = *reinterpret_cast<const uint4*>(layer_input + (size_t)(tile * kTile + u / chunks) * hidden + h);
            rescale(u, li, *reinterpret_cast<const uint4*>(norm_w + h));
        }
    }
    if (finish_slices < kTile)
        finish_more_coefficients(T, hidden, slices, finish_slices, tile, hs, tid, part, scale,
                                 base, p, mred, mtot, pre_out, post_out, comb_out, mixes_out,
                                 rstd_out);
}


// ---------------------------------------------------------------------------
// Non-shifted pre, kernel 2: one workgroup (256 or 512 threads) per token.
// It is the last reader of X and the only writer of the layer input.  When X
// is at least 128 MiB (half the last-level cache) both streams carry the
// nontemporal hint (NT), measured with norm: d=7168 T=8192 219 -> 188 us,
// T=4096 114 -> 103, T=3072 89 -> 85, T=2341 (just over the threshold)
// 68.0 -> 69.5; d=16384 T=1024 73 -> 69.  Below it the hint costs: T=2048
// d=7168 57 -> 63 us, T=32 9.8 -> 10.3.
// ---------------------------------------------------------------------------
// Where the partial sums of the projection live: value v (24 mixes, then the
// sum of squares) of token t in split q is
//   mix:  mix[q*mix_split + t*mix_tok + v]      ssq: ssq[q*ssq_split + t*ssq_tok]
struct PartialLayout {
    const float* mix;
    const float* ssq;
    size_t mix_split, mix_tok, ssq_split, ssq_tok;
    int splits;
};

template <bool NT>
__global__ __launch_bounds__(512) void k_pre_finish(
    int hidden, PartialLayout pl, const uint16_t* __restrict__ X,
    const float* __restrict__ scale, const float* __restrict__ base,
    const uint16_t* __restrict__ norm_w, Scalars p, uint16_t* __restrict__ layer_input,
    float* __restrict__ pre_out, float* __restrict__ post_out, float* __restrict__ comb_out,
    float* __restrict__ mixes_out, float* __restrict__ rstd_out) {
    MHC_POISON_LDS(norm_w ? (unsigned)hidden * 2 + (unsigned)hidden / 8 * 4 : 0u);
    // With norm_w: li of the row, [hidden / 8] chunks, then the sum of squares
    // of each chunk, [hidden / 8] floats.
    extern __shared__ uint4 li_s[];
    __shared__ float tot[26];
    __shared__ float pre_s[4];
    __shared__ float cred[8][26];
    __shared__ float rli;

    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const int nch = hidden / 8;             // 16-byte chunks of a row
    const int nc = (int)blockDim.x - 64;    // collapse threads: waves 1.. (192 or 448)
    const int u0 = tid - 64;                // collapse thread index
    float* const chunk_ssq = reinterpret_cast<float*>(li_s + nch);
    const uint16_t* Xrow = X + (size_t)t * 4 * hidden;

    // Waves 1-3 request their first two chunks of X before anything waits;
    // wave 0 gathers the token's projection record.
    CoefParams cp;
    if (tid < 4) cp = load_coef_params(scale, base, tid);
    const float comb_s2 = scale[2], comb_b = base[8 + (tid & 15)];  // (the comb's 16 lanes)
    uint4 bufA[4], bufB[4];
    auto load_chunk = [&](uint4 (&b)[4], int cidx) {
        if (cidx < nch) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                b[j] = ld16<NT>(Xrow + (size_t)j * hidden + cidx * 8);
        }
    };
    // Thread (group, v) of the first 200 sums splits group, group + 8, ... of
    // value v (24 mixes, then the sum of squares); the 8 group sums are then
    // added in group order.  At most 8 loads per thread, issued together.  With
    // 8 splits or fewer every group holds at most one split, so the plain sum in
    // split order is the same number and the LDS stage is skipped.
    const bool two_level = pl.splits > 8;
    if (!two_level) {
        if (tid < 25)
            tot[tid] = tid < 24 ? slice_sum(pl.mix + (size_t)t * pl.mix_tok + tid, 0, 1, pl.splits,
                                            pl.mix_split)
                                : slice_sum(pl.ssq + (size_t)t * pl.ssq_tok, 0, 1, pl.splits,
                                            pl.ssq_split);
    } else if (tid < 200) {
        const int grp = tid / 25, v = tid % 25;
        cred[grp][v] = v < 24 ? slice_sum(pl.mix + (size_t)t * pl.mix_tok + v, grp, 8, pl.splits,
                                          pl.mix_split)
                              : slice_sum(pl.ssq + (size_t)t * pl.ssq_tok, grp, 8, pl.splits,
                                          pl.ssq_split);
    }
    if (tid >= 64) {
        load_chunk(bufA, u0);
        load_chunk(bufB, u0 + nc);
    }
    __syncthreads();
    if (two_level) {
        if (tid < 25) {
            float sum = 0.0f;
#pragma unroll
            for (int grp = 0; grp < 8; ++grp) sum += cred[grp][tid];
            tot[tid] = sum;
        }
        __syncthreads();
    }
    // pre is published as soon as it exists: the collapse does not wait for
    // the Sinkhorn iterations, which wave 0 runs at the end.
    TokenCoef o;
    if (tid < 4) {
        pre_post(o, tot, tid, hidden, cp, p);
        pre_s[tid] = o.pre;
    }
    __syncthreads();

    if (tid >= 64) {
        const float pr[4] = {pre_s[0], pre_s[1], pre_s[2], pre_s[3]};
        auto collapse = [&](uint4 (&b)[4], int cidx) {
            uint4 Xv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) Xv[j] = b[j];
            load_chunk(b, cidx + 2 * nc);       // two chunks ahead
            uint4 li;
            float ssq_li = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float acc[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    acc[e] = 0.0f;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t w = word(Xv[j], q);
                        acc[e] = __builtin_fmaf(pr[j], e ? bf_hi(w) : bf_lo(w), acc[e]);
                    }
                }
                const uint32_t lw = pack_bf16(acc[0], acc[1]);
                set_word(li, q, lw);
                ssq_li = __builtin_fmaf(bf_lo(lw), bf_lo(lw), ssq_li);
                ssq_li = __builtin_fmaf(bf_hi(lw), bf_hi(lw), ssq_li);
            }
            if (norm_w) {
                li_s[cidx] = li;
                chunk_ssq[cidx] = ssq_li;
            } else st16<NT>(layer_input + (size_t)t * hidden + cidx * 8, li);
        };
        for (int cidx = u0; cidx < nch; cidx += 2 * nc) {
            collapse(bufA, cidx);
            if (cidx + nc < nch) collapse(bufB, cidx + nc);
        }
    }
    if (norm_w) {
        __syncthreads();
        // Chunk sums in an order fixed by hidden alone (the number of collapse
        // threads varies with the batch): lane l adds chunks l, l + 64, ... in
        // order, then the 64 lanes are combined by the butterfly.
        if (tid >= 64 && tid < 128) {
            float v = 0.0f;
#pragma unroll 4
            for (int k = u0; k < nch; k += 64) v += chunk_ssq[k];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
            if (u0 == 0) rli = rsqrt_nr(v * (1.0f / (float)hidden) + p.norm_eps);
        }
        __syncthreads();
        if (tid >= 64) {
            const float r = rli;
            for (int cidx = u0; cidx < nch; cidx += nc) {
                const int h = cidx * 8;
                const uint4 li = li_s[cidx];
                const uint4 nw = *reinterpret_cast<const uint4*>(norm_w + h);
                uint4 out;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t a = word(li, q), b = word(nw, q);
                    set_word(out, q, pack_bf16((bf_lo(a) * r) * bf_lo(b), (bf_hi(a) * r) * bf_hi(b)));
                }
                st16<NT>(layer_input + (size_t)t * hidden + h, out);
            }
        }
    }
    // Wave 0: the Sinkhorn comb on 16 lanes (rstd as pre_post forms it),
    // overlapping the layer-input work above.
    if (tid < 16) {
        const float rstd = rsqrt_nr(tot[24] * (0.25f / (float)hidden) + p.rms_eps);
        comb_out[(size_t)t * 16 + tid] = comb16(tot, tid, rstd, comb_s2, comb_b, p);
        if (tid < 4) {
            pre_out[(size_t)t * 4 + tid] = o.pre;
            post_out[(size_t)t * 4 + tid] = o.post;
            if (mixes_out)
                for (int k = 0; k < 6; ++k) mixes_out[(size_t)t * 24 + 6 * tid + k] = tot[6 * tid + k];
            if (rstd_out && tid == 0) rstd_out[t] = o.rstd;
        }
    }
}

// ---------------------------------------------------------------------------
// Residual update alone.  Workgroup (token, chunk group), token-major in a
// 1-D grid: 256 threads, thread i covers hidden [8*(chunk*256 + i), +8) of all
// four streams, so every wave instruction reads or writes 1 KB of one row and
// neighbouring workgroups cover the rest of the token's rows.  The token's
// coefficients are workgroup-uniform (scalar loads).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_post(int hidden, int chunks, const uint16_t* __restrict__ x,
                                              const uint16_t* __restrict__ X,
                                              const float* __restrict__ post_prev,
                                              const float* __restrict__ comb_prev,
                                              uint16_t* __restrict__ xn_out) {
    const size_t t = blockIdx.x / chunks;
    const int h = ((blockIdx.x - (int)t * chunks) * blockDim.x + threadIdx.x) * 8;
    if (h >= hidden) return;
    PrevCoef c;
    load_prev(c, post_prev, comb_prev, post_prev, t);  // (pre unused)
    uint4 Xv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) Xv[j] = *reinterpret_cast<const uint4*>(X + (t * 4 + j) * hidden + h);
    const uint4 xv = *reinterpret_cast<const uint4*>(x + t * hidden + h);
    uint4 Xn[4], li;
    float ssq = 0.0f, ssq_li = 0.0f;
    update_collapse(Xv, xv, c, Xn, li, ssq, ssq_li);  // li and the sums are unused
#pragma unroll
    for (int s = 0; s < 4; ++s) *reinterpret_cast<uint4*>(xn_out + (t * 4 + s) * hidden + h) = Xn[s];
}

// Residual update alone, in the movers' fastest patterns: item = (tile of
// tokens, slice of RUN hidden elements), tile-major, 16 tokens per item for
// RUN = 512 and 32 for RUN = 256.  Wave w takes 4 tokens
// (RUN = 512: tokens 4w..4w+3, each instruction 1 row x 1024 contiguous
// bytes) or 8 (RUN = 256: tokens 8w..8w+7, instruction p covering tokens
// 8w + 2p and 8w + 2p + 1, 2 rows x 512 bytes); stream j = 4 is the block
// output.  All 20 loads of a lane are issued before any arithmetic.  Tokens
// past T read the last token's rows and store nothing.  Taken from 128 MiB of
// X, with the nontemporal hint on every load and store (cold, us, the kernel
// above -> RUN = 256: d=7168 T=8192 198 -> 192, d=4096 T=16384 212 -> 197;
// plain loads and stores 202 at T=8192; at T=1000 it was slower, 25 -> 30).
// RUN = 512 where hidden is a multiple of 512 but not of 2048 (d=7168 T=8192
// 192.4 -> 182.1, T=4096 99.1 -> 95.6); where the token stride is a multiple
// of 16 KiB it measured slower (d=4096 T=16384 197 -> 204).
template <bool NT, int RUN>
__global__ __launch_bounds__(256) void k_post_rows(int T, int hidden, const uint16_t* __restrict__ x,
                                                   const uint16_t* __restrict__ X,
                                                   const float* __restrict__ post_prev,
                                                   const float* __restrict__ comb_prev,
                                                   uint16_t* __restrict__ xn_out) {
    static_assert(RUN == 256 || RUN == 512, "runs of 256 or 512 elements");
    constexpr int kTok = RUN == 512 ? 16 : 32;  // tokens of an item
    const int slices = hidden / RUN;
    const int tile = blockIdx.x / slices, slice = blockIdx.x - tile * slices;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int col = slice * RUN + (RUN == 512 ? l : (l & 31)) * 8;
    int tk[4];
    bool ok[4];
    uint4 v[4][5];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int t = RUN == 512 ? tile * kTok + 4 * w + p : tile * kTok + 8 * w + 2 * p + (l >> 5);
        ok[p] = t < T;
        tk[p] = ok[p] ? t : T - 1;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[p][j] = ld16<NT>(X + ((size_t)tk[p] * 4 + j) * hidden + col);
        v[p][4] = ld16<NT>(x + (size_t)tk[p] * hidden + col);
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        PrevCoef c;
        load_prev(c, post_prev, comb_prev, post_prev, (size_t)tk[p]);  // (pre unused)
        const uint4 Xv[4] = {v[p][0], v[p][1], v[p][2], v[p][3]};
        uint4 Xn[4], li;
        float ssq = 0.0f, ssq_li = 0.0f;
        update_collapse(Xv, v[p][4], c, Xn, li, ssq, ssq_li);  // li and the sums are unused
        if (ok[p]) {
#pragma unroll
            for (int s = 0; s < 4; ++s) st16<NT>(xn_out + ((size_t)tk[p] * 4 + s) * hidden + col, Xn[s]);
        }
    }
}


// ---------------------------------------------------------------------------
// Weight prefetch: every thread reads four 16-byte words of the prepared weight
// so that its lines are resident in the last-level cache (and the reading
// XCD's L2) when the boundary runs.  The empty asm consumes each value, so the
// loads are kept; nothing is written.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_prefetch(const uint4* __restrict__ w, int n_words) {
    const int base = blockIdx.x * 1024 + threadIdx.x;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int i = base + k * 256;
        if (i < n_words) {
            const uint4 v = w[i];
            asm volatile("" ::"v"(v.x), "v"(v.y), "v"(v.z), "v"(v.w));
        }
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// Launchers (host).  Shapes were validated by the caller.
// ---------------------------------------------------------------------------
hipError_t launch_prepare_weight(const float* w, int hidden, void* out, hipStream_t stream) {
    const int n_words = (hidden / kStep) * kFragsPerStep * 64;
    hipLaunchKernelGGL(k_prepare_weight, dim3((n_words + 255) / 256), dim3(256), 0, stream, w,
                       hidden, reinterpret_cast<uint4*>(out), n_words);
    return hipGetLastError();
}

hipError_t launch_prefetch_weight(const void* wprep, int hidden, hipStream_t stream) {
    const int n_words = (hidden / kStep) * kFragsPerStep * 64;
    hipLaunchKernelGGL(k_prefetch, dim3((n_words + 1023) / 1024), dim3(256), 0, stream,
                       reinterpret_cast<const uint4*>(wprep), n_words);
    return hipGetLastError();
}

hipError_t launch_post(int T, int hidden, const uint16_t* x, const uint16_t* X,
                       const float* post_prev, const float* comb_prev, uint16_t* xn_out,
                       hipStream_t stream) {
    if ((size_t)T * 4 * (size_t)hidden * 2 >= ((size_t)128 << 20)) {
        if (hidden % 512 == 0 && hidden % 2048 != 0)
            hipLaunchKernelGGL((k_post_rows<true, 512>), dim3((unsigned)((T + 15) / 16) * (unsigned)(hidden / 512)),
                               dim3(256), 0, stream, T, hidden, x, X, post_prev, comb_prev, xn_out);
        else
            hipLaunchKernelGGL((k_post_rows<true, 256>), dim3((unsigned)((T + 31) / 32) * (unsigned)(hidden / 256)),
                               dim3(256), 0, stream, T, hidden, x, X, post_prev, comb_prev, xn_out);
        return hipGetLastError();
    }
    const int chunks = (hidden / 8 + 255) / 256;
    hipLaunchKernelGGL(k_post, dim3((unsigned)T * (unsigned)chunks), dim3(256), 0, stream, hidden,
                       chunks, x, X, post_prev, comb_prev, xn_out);
    return hipGetLastError();
}

template <int G, bool NT>
static void launch_partial_g(bool shifted, const SplitPlan& plan, int T, int hidden,
                             const uint16_t* x, const uint16_t* X, const float* post_prev,
                             const float* comb_prev, const float* pre_lag, const uint4* w,
                             uint16_t* xn_out, uint16_t* li_out, float* part, hipStream_t stream) {
    const dim3 grid((unsigned)((T + kTile * G - 1) / (kTile * G)) * (unsigned)plan.slices);
    const bool one = plan.steps_per_wave == 1;
    if (shifted) {
        if constexpr (G <= 2) {  // (four groups would spill in the shifted kernel)
            if (one)
                hipLaunchKernelGGL((k_partial<true, G, NT, true>), grid, dim3(256), 0, stream, T,
                                   hidden, plan.steps_per_wave, plan.slices, x, X, post_prev,
                                   comb_prev, pre_lag, w, xn_out, li_out, part);
            else
                hipLaunchKernelGGL((k_partial<true, G, NT, false>), grid, dim3(256), 0, stream, T,
                                   hidden, plan.steps_per_wave, plan.slices, x, X, post_prev,
                                   comb_prev, pre_lag, w, xn_out, li_out, part);
        }
        return;
    }
    if (one) {
        hipLaunchKernelGGL((k_partial<false, G, NT, true>), grid, dim3(256), 0, stream, T, hidden,
                           plan.steps_per_wave, plan.slices, nullptr, X, nullptr, nullptr, nullptr,
                           w, nullptr, nullptr, part);
        return;
    }
    // Four groups over several steps keep the 64-element-step kernel (T=8192:
    // 185.7 us against 188.4 with k_partial; T=4096 104.3 against 101.5).
    if constexpr (G == 4) {  // (the plan gives four groups an even number of steps)
        if (plan.steps_per_wave % 2 == 0) {
            hipLaunchKernelGGL((k_partial_pre_wide<G, NT>), grid, dim3(256), 0, stream, T, hidden,
                               plan.steps_per_wave, plan.slices, X, w, part);
            return;
        }
    }
    hipLaunchKernelGGL((k_partial<false, G, NT, false>), grid, dim3(256), 0, stream, T, hidden,
                       plan.steps_per_wave, plan.slices, nullptr, X, nullptr, nullptr, nullptr, w,
                       nullptr, nullptr, part);
}

template <int G>
static void launch_partial_nt(bool shifted, const SplitPlan& plan, int T, int hidden,
                              const uint16_t* x, const uint16_t* X, const float* post_prev,
                              const float* comb_prev, const float* pre_lag, const uint4* w,
                              uint16_t* xn_out, uint16_t* li_out, float* part, hipStream_t stream) {
    if (plan.stream)
        launch_partial_g<G, true>(shifted, plan, T, hidden, x, X, post_prev, comb_prev, pre_lag,
                                  w, xn_out, li_out, part, stream);
    else
        launch_partial_g<G, false>(shifted, plan, T, hidden, x, X, post_prev, comb_prev, pre_lag,
                                   w, xn_out, li_out, part, stream);
}

hipError_t launch_partial(bool shifted, const SplitPlan& plan, int T, int hidden,
                          const uint16_t* x, const uint16_t* X, const float* post_prev,
                          const float* comb_prev, const float* pre_lag, const void* wprep,
                          uint16_t* xn_out, uint16_t* li_out, float* part, hipStream_t stream) {
    const uint4* w = reinterpret_cast<const uint4*>(wprep);
    if (plan.groups == 4 && !shifted)
        launch_partial_nt<4>(shifted, plan, T, hidden, x, X, post_prev, comb_prev, pre_lag, w,
                             xn_out, li_out, part, stream);
    else if (plan.groups == 2)
        launch_partial_nt<2>(shifted, plan, T, hidden, x, X, post_prev, comb_prev, pre_lag, w,
                             xn_out, li_out, part, stream);
    else
        launch_partial_nt<1>(shifted, plan, T, hidden, x, X, post_prev, comb_prev, pre_lag, w,
                             xn_out, li_out, part, stream);
    return hipGetLastError();
}

namespace {
constexpr int kMaxDevices = 64;

int current_device() {
    int dev = 0;
    return hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices ? dev : -1;
}

int query_compute_units(int dev) {
    int units = 0;
    return hipDeviceGetAttribute(&units, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess
               ? units
               : 0;
}
}  // namespace

int device_compute_units() {
    static std::atomic<int> cache[kMaxDevices];  // 0: not asked yet; -1: unknown
    const int dev = current_device();
    if (dev < 0) return 0;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        const int units = query_compute_units(dev);
        v = units > 0 ? units : -1;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v > 0 ? v : 0;
}

int partial_resident_workgroups(int groups) {
    static std::atomic<int> cache[kMaxDevices][2];  // 0: not asked yet; -1: unknown
    const int dev = current_device();
    if (dev < 0) return 0;
    std::atomic<int>& slot = cache[dev][groups == 2 ? 1 : 0];
    int v = slot.load(std::memory_order_relaxed);
    if (v == 0) {
        const int units = query_compute_units(dev);
        int per_unit = 0;
        hipError_t e;
        e = groups == 2 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_unit, k_partial<true, 2, false, false>, 256, 0)
                        : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_unit, k_partial<true, 1, false, false>, 256, 0);
        v = (e == hipSuccess && units > 0 && per_unit > 0) ? units * per_unit : -1;
        slot.store(v, std::memory_order_relaxed);
    }
    return v > 0 ? v : 0;
}

hipError_t launch_finish(const SplitPlan& plan, int T, int hidden, const float* part,
                         const float* scale, const float* base, const uint16_t* norm_w,
                         const Scalars& p, uint16_t* layer_input, float* pre_out,
                         float* post_out, float* comb_out, float* mixes, float* rstd,
                         hipStream_t stream) {
    const dim3 grid((unsigned)((T + kTile - 1) / kTile) * (unsigned)plan.finish_slices);
    hipLaunchKernelGGL(k_finish, grid, dim3(256), 0, stream, T, hidden, plan.slices,
                       plan.finish_slices, plan.finish_width, part, scale, base, norm_w, p,
                       layer_input, pre_out, post_out, comb_out, mixes, rstd);
    return hipGetLastError();
}

static hipError_t launch_pre_finish_layout(int T, int hidden, const PartialLayout& pl,
                                           const uint16_t* X, const float* scale,
                                           const float* base, const uint16_t* norm_w,
                                           const Scalars& p, uint16_t* layer_input,
                                           float* pre_out, float* post_out, float* comb_out,
                                           float* mixes, float* rstd, hipStream_t stream) {
    // Small batches: 448 collapse threads, so a row of 7168 is requested in
    // one round trip; large batches: 192, more workgroups per CU.
    const size_t lds = norm_w ? (size_t)hidden * 2 + (size_t)hidden / 8 * sizeof(float) : 0;
    const int threads = T <= 512 ? 512 : 256;
    const bool nt = (size_t)T * 4 * (size_t)hidden * 2 >= ((size_t)128 << 20);
    if (nt)
        hipLaunchKernelGGL(k_pre_finish<true>, dim3(T), dim3(threads), lds, stream, hidden, pl, X,
                           scale, base, norm_w, p, layer_input, pre_out, post_out, comb_out, mixes,
                           rstd);
    else
        hipLaunchKernelGGL(k_pre_finish<false>, dim3(T), dim3(threads), lds, stream, hidden, pl, X,
                           scale, base, norm_w, p, layer_input, pre_out, post_out, comb_out, mixes,
                           rstd);
    return hipGetLastError();
}

hipError_t launch_pre_finish(const SplitPlan& plan, int T, int hidden, const uint16_t* X,
                             const float* part, const float* scale, const float* base,
                             const uint16_t* norm_w, const Scalars& p, uint16_t* layer_input,
                             float* pre_out, float* post_out, float* comb_out, float* mixes,
                             float* rstd, hipStream_t stream) {
    const size_t rec = (size_t)plan.slices * kPart;
    const PartialLayout pl{part, part + 24, kPart, rec, kPart, rec, plan.slices};
    return launch_pre_finish_layout(T, hidden, pl, X, scale, base, norm_w, p, layer_input,
                                    pre_out, post_out, comb_out, mixes, rstd, stream);
}

hipError_t launch_pre_mixes(int T, int hidden, int splits, const uint16_t* X,
                            const float* dot_mix, const float* sqrsum, const float* scale,
                            const float* base, const uint16_t* norm_w, const Scalars& p,
                            uint16_t* layer_input, float* pre_out, float* post_out,
                            float* comb_out, hipStream_t stream) {
    const PartialLayout pl{dot_mix, sqrsum, (size_t)T * 24, 24, (size_t)T, 1, splits};
    return launch_pre_finish_layout(T, hidden, pl, X, scale, base, norm_w, p, layer_input,
                                    pre_out, post_out, comb_out, nullptr, nullptr, stream);
}

}  // namespace mhc
