// Single-pass non-shifted pre for decode-size batches ([P] "computing pre_mix
// early", "computing layer_input A_l X_l"; [B] module description: one launch
// for the whole boundary): one launch reads X once.
//
// Workgroup q owns hidden elements [128 q, 128 q + 128) of every token of the
// batch (T <= 64: wave w holds tokens 16 w .. 16 w + 15, lane (n, g) token
// 16 w + n and elements 8 g .. 8 g + 7 of each 32-element k-block).  It keeps
// its X in registers for the whole call:
//   1  projection partials and sum of squares of the slice (matrix cores), one
//      record per (token, slice);
//   2  device-wide barrier; then every workgroup sums the pre mixes and the
//      sum of squares of every token over the slices (a fixed order, the same
//      in every workgroup, so all of them hold the same pre bits) and forms
//      pre;
//   3  the collapse li = bf16(sum_j pre_j X_j) from the registers;
//   4  with norm_w: the li sum of squares of the slice, a second barrier,
//      rstd_li of every token, the normalised layer input;
// and the workgroup with q = t mod slices also forms post, the Sinkhorn comb
// and the debug outputs of token t, while the other workgroups reach the
// second barrier.
//
// Every workgroup waits on all the others, so all of them must be resident at
// once: the host launches at most one workgroup per compute unit (hidden / 128
// <= 128 workgroups, one per CU at 512 registers a wave) and takes the split
// schedule where the device has fewer compute units.  A wait that runs out
// counts in the workspace's error slot instead of hanging.
#include "mhc_coherent.h"
#include "mhc_device.h"
#include "mhc_launch.h"

namespace mhc {
namespace {

constexpr int kOneWidth = 128;               // hidden elements per workgroup
constexpr int kOneKb = kOneWidth / kStep;    // k-blocks per workgroup
constexpr int kOneMaxTokens = 64;            // one 16-token group per wave
constexpr int kGroups = 4;                   // slice groups of every record sum
constexpr int kRec1 = 8;                     // floats: pre mixes 0-3, ssq, ssq_li, pad
constexpr int kRec2 = 20;                    // floats: mixes 4-23

struct PreOneArgs {
    int T, hidden, slices;
    const uint16_t* X;
    const uint4* wprep;
    const float* scale;
    const float* base;
    const uint16_t* norm_w;
    uint16_t* layer_input;
    float* pre_out;
    float* post_out;
    float* comb_out;
    float* mixes_out;
    float* rstd_out;
    float* rec1;     // [T][slices][kRec1]
    float* rec2;     // [T][slices][kRec2]
    unsigned* sync;  // [0] first barrier, [1] second barrier, [2] errors, [3] exits
    Scalars p;
};

// Slices of group grp: [grp * per, min((grp + 1) * per, S)), per = ceil(S / kGroups).
__device__ __forceinline__ int group_begin(int grp, int S) { return grp * ((S + kGroups - 1) / kGroups); }
__device__ __forceinline__ int group_end(int grp, int S) {
    return min(S, (grp + 1) * ((S + kGroups - 1) / kGroups));
}

// Sum over the slices of group grp (in slice order) of the 16-byte value at
// byte offset off0 + sl * stride of a record buffer (device-coherent loads,
// eight in flight at a time).
__device__ __forceinline__ float4 sum_group4(__amdgpu_buffer_rsrc_t rs, unsigned off0, unsigned stride, int grp,
                                             int S) {
    const int b = group_begin(grp, S), e = group_end(grp, S);
    float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = b; s0 < e; s0 += 8) {
        u32x4_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, off0 + (unsigned)min(s0 + u, e - 1) * stride, 0,
                                                         kCoherent);
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (s0 + u < e) {
                sum.x += __uint_as_float(v[u].x);
                sum.y += __uint_as_float(v[u].y);
                sum.z += __uint_as_float(v[u].z);
                sum.w += __uint_as_float(v[u].w);
            }
    }
    return sum;
}

__device__ __forceinline__ float sum_group1(__amdgpu_buffer_rsrc_t rs, unsigned off0, unsigned stride, int grp,
                                            int S) {
    const int b = group_begin(grp, S), e = group_end(grp, S);
    float sum = 0.0f;
    for (int s0 = b; s0 < e; s0 += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = ld_coh(rs, off0 + (unsigned)min(s0 + u, e - 1) * stride);
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (s0 + u < e) sum += v[u];
    }
    return sum;
}

template <bool NORM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_pre_one(PreOneArgs a) {
    MHC_POISON_LDS(0);
    __shared__ float4 gsum[kOneMaxTokens][2][kGroups];   // group sums of the 8-float records
    __shared__ float tot8[kOneMaxTokens][kRec1];           // pre mixes 0-3, ssq, ssq_li
    __shared__ float pre_s[kOneMaxTokens][4];
    __shared__ float4 gsum2[kOneMaxTokens][5][kGroups];   // designated tokens: mixes 4-23
    __shared__ float ctot[kOneMaxTokens][26];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
    const int T = a.T, hidden = a.hidden, S = a.slices, slice = blockIdx.x;
    const int t = 16 * wave + n;  // this lane's token
    const unsigned row_bytes = (unsigned)hidden * 2;
    unsigned* const bar1 = a.sync;
    unsigned* const bar2 = a.sync + 1;
    unsigned* const errors = a.sync + 2;
    unsigned* const exits = a.sync + 3;
    const auto r1 = rsrc(a.rec1, (unsigned)(T * S * kRec1 * 4));
    const auto r2 = rsrc(a.rec2, (unsigned)(T * S * kRec2 * 4));

    // ---- 1: X of the slice (rows past the batch read 0) and the weight fragments
    const auto x_rs = rsrc(a.X, (unsigned)T * 4 * row_bytes);
    uint4 Xv[kOneKb][4];
#pragma unroll
    for (int kb = 0; kb < kOneKb; ++kb)
#pragma unroll
        for (int s = 0; s < 4; ++s)
            Xv[kb][s] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(
                           x_rs, ((unsigned)t * 4 + s) * row_bytes + (slice * kOneWidth + kb * kStep + g * 8) * 2,
                           0, 0));
    uint4 A[kOneKb][kFragsPerStep];
#pragma unroll
    for (int kb = 0; kb < kOneKb; ++kb)
#pragma unroll
        for (int i = 0; i < kFragsPerStep; ++i)
            A[kb][i] = a.wprep[((size_t)(slice * kOneKb + kb) * kFragsPerStep + i) * 64 + lane];
    f32x4_t acc[3] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    float ssq = 0.0f;
#pragma unroll
    for (int kb = 0; kb < kOneKb; ++kb) {
        square_sum(Xv[kb], ssq);
        mfma_step(A[kb], Xv[kb], acc);
    }
    // records: lane (n, g) holds mixes 8m + 2g + jj of token n; ssq added over g in order
    {
        const float a1 = __shfl(ssq, n + 16), a2 = __shfl(ssq, n + 32), a3 = __shfl(ssq, n + 48);
        if (t < T) {
            float* q1 = a.rec1 + ((size_t)t * S + slice) * kRec1;
            float* q2 = a.rec2 + ((size_t)t * S + slice) * kRec2;
#pragma unroll
            for (int m = 0; m < 3; ++m)
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    const int mix = 8 * m + 2 * g + jj;
                    if (mix < 4)
                        st_dev(q1 + mix, mix_of(acc, m, jj));
                    else
                        st_dev(q2 + mix - 4, mix_of(acc, m, jj));
                }
            if (g == 0) st_dev(q1 + 4, ((ssq + a1) + a2) + a3);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        add_dev(bar1, 1u);
        if (!wait_count(bar1, (unsigned)S)) add_dev(errors, 1u);
    }
    __syncthreads();

    // ---- 2: pre of every token from the records.  Thread (token tt, half h,
    // group grp) sums 16 bytes of the 8-float records over the group's slices;
    // the four groups are then added in group order.
    for (int p = tid; p < T * 2 * kGroups; p += 256) {
        const int tt = p / (2 * kGroups), h = (p / kGroups) & 1, grp = p % kGroups;
        gsum[tt][h][grp] = sum_group4(r1, ((unsigned)tt * S * kRec1 + 4 * h) * 4, kRec1 * 4, grp, S);
    }
    __syncthreads();
    if (tid < T * 2) {
        const int tt = tid >> 1, h = tid & 1;
        float4 s = gsum[tt][h][0];
#pragma unroll
        for (int grp = 1; grp < kGroups; ++grp) {
            const float4 v = gsum[tt][h][grp];
            s.x += v.x;
            s.y += v.y;
            s.z += v.z;
            s.w += v.w;
        }
        tot8[tt][4 * h + 0] = s.x;
        tot8[tt][4 * h + 1] = s.y;
        tot8[tt][4 * h + 2] = s.z;
        tot8[tt][4 * h + 3] = s.w;
    }
    __syncthreads();
    if (tid < T * 4) {
        // (the arithmetic of pre_post)
        const int tt = tid >> 2, i = tid & 3;
        const float rstd = rsqrt_nr(tot8[tt][4] * (0.25f / (float)hidden) + a.p.rms_eps);
        pre_s[tt][i] = sigmoid(__builtin_fmaf(tot8[tt][i] * rstd, a.scale[0], a.base[i])) + a.p.pre_eps;
    }
    __syncthreads();

    // ---- 3: the collapse with the fresh pre, from registers
    uint4 li[kOneKb];
    float ssq_li = 0.0f;
    {
        const int tc = min(t, T - 1);
        const float pr[4] = {pre_s[tc][0], pre_s[tc][1], pre_s[tc][2], pre_s[tc][3]};
#pragma unroll
        for (int kb = 0; kb < kOneKb; ++kb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float c[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    c[e] = 0.0f;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t w = word(Xv[kb][j], q);
                        c[e] = __builtin_fmaf(pr[j], e ? bf_hi(w) : bf_lo(w), c[e]);
                    }
                }
                const uint32_t lw = pack_bf16(c[0], c[1]);
                set_word(li[kb], q, lw);
                ssq_li = __builtin_fmaf(bf_lo(lw), bf_lo(lw), ssq_li);
                ssq_li = __builtin_fmaf(bf_hi(lw), bf_hi(lw), ssq_li);
            }
    }
    uint16_t* const li_row = a.layer_input + (size_t)t * hidden + slice * kOneWidth + g * 8;
    if (NORM) {
        const float b1 = __shfl(ssq_li, n + 16), b2 = __shfl(ssq_li, n + 32), b3 = __shfl(ssq_li, n + 48);
        if (t < T && g == 0) st_dev(a.rec1 + ((size_t)t * S + slice) * kRec1 + 5, ((ssq_li + b1) + b2) + b3);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) add_dev(bar2, 1u);
    } else if (t < T) {
#pragma unroll
        for (int kb = 0; kb < kOneKb; ++kb) *reinterpret_cast<uint4*>(li_row + kb * kStep) = li[kb];
    }

    // ---- the coefficients of this workgroup's tokens t = slice, slice + S, ...
    // (post, comb, debug outputs; pre as every workgroup formed it)
    const int ntok = slice < T ? (T - 1 - slice) / S + 1 : 0;
    if (ntok > 0) {
        for (int p = tid; p < ntok * 5 * kGroups; p += 256) {
            const int k = p / (5 * kGroups), qd = (p / kGroups) % 5, grp = p % kGroups;
            const int tt = slice + k * S;
            gsum2[k][qd][grp] = sum_group4(r2, ((unsigned)tt * S * kRec2 + 4 * qd) * 4, kRec2 * 4, grp, S);
        }
        __syncthreads();
        for (int p = tid; p < ntok * 26; p += 256) {
            const int k = p / 26, v = p % 26, tt = slice + k * S;
            float val;
            if (v < 4) {
                val = tot8[tt][v];
            } else if (v < 24) {
                const int qd = (v - 4) >> 2, c = (v - 4) & 3;
                val = 0.0f;
#pragma unroll
                for (int grp = 0; grp < kGroups; ++grp) {
                    const float4 s4 = gsum2[k][qd][grp];
                    val += c == 0 ? s4.x : c == 1 ? s4.y : c == 2 ? s4.z : s4.w;
                }
            } else {
                val = v == 24 ? tot8[tt][4] : 0.0f;
            }
            ctot[k][v] = val;
        }
        __syncthreads();
        for (int p = tid; p < ntok * 16; p += 256) {
            const int k = p >> 4, l16 = p & 15, i = l16 & 3, tt = slice + k * S;
            const CoefParams cp = load_coef_params(a.scale, a.base, i);
            TokenCoef o;
            pre_post(o, ctot[k], i, hidden, cp, a.p);
            const float cv = comb16(ctot[k], l16, o.rstd, cp.s2, a.base[8 + l16], a.p);
            a.comb_out[(size_t)tt * 16 + l16] = cv;
            if (l16 < 4) {
                a.pre_out[(size_t)tt * 4 + i] = pre_s[tt][i];
                a.post_out[(size_t)tt * 4 + i] = o.post;
                if (a.mixes_out)
                    for (int kq = 0; kq < 6; ++kq) a.mixes_out[(size_t)tt * 24 + 6 * i + kq] = ctot[k][6 * i + kq];
                if (a.rstd_out && i == 0) a.rstd_out[tt] = o.rstd;
            }
        }
    }

    // ---- 4: rstd_li of every token, the normalised layer input
    if (NORM) {
        __shared__ float gli[kOneMaxTokens][kGroups];
        __shared__ float rli_s[kOneMaxTokens];
        if (tid == 0) {
            if (!wait_count(bar2, (unsigned)S)) add_dev(errors, 1u);
        }
        __syncthreads();
        for (int p = tid; p < T * kGroups; p += 256) {
            const int tt = p / kGroups, grp = p % kGroups;
            gli[tt][grp] = sum_group1(r1, ((unsigned)tt * S * kRec1 + 5) * 4, kRec1 * 4, grp, S);
        }
        __syncthreads();
        if (tid < T) {
            float s = gli[tid][0];
#pragma unroll
            for (int grp = 1; grp < kGroups; ++grp) s += gli[tid][grp];
            rli_s[tid] = rsqrt_nr(s * (1.0f / (float)hidden) + a.p.norm_eps);
        }
        __syncthreads();
        if (t < T) {
            const float r = rli_s[t];
#pragma unroll
            for (int kb = 0; kb < kOneKb; ++kb) {
                const uint4 nw = *reinterpret_cast<const uint4*>(a.norm_w + slice * kOneWidth + kb * kStep + g * 8);
                uint4 out;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t av = word(li[kb], q), bv = word(nw, q);
                    set_word(out, q, pack_bf16((bf_lo(av) * r) * bf_lo(bv), (bf_hi(av) * r) * bf_hi(bv)));
                }
                *reinterpret_cast<uint4*>(li_row + kb * kStep) = out;
            }
        }
    }

    // Every workgroup has passed both waits once it counts itself out; the last
    // one returns the counters to zero.
    if (tid == 0) {
        if (add_dev(exits, 1u) == gridDim.x - 1u) {
            st_dev(bar1, 0u);
            st_dev(bar2, 0u);
            st_dev(exits, 0u);
        }
    }
}

}  // namespace

bool pre_one_supported(int T, int hidden, int compute_units) {
    return T >= 1 && T <= kOneMaxTokens && hidden % kOneWidth == 0 && compute_units >= hidden / kOneWidth;
}

size_t pre_one_data_bytes(int T, int hidden) {
    return (size_t)T * (hidden / kOneWidth) * (kRec1 + kRec2) * sizeof(float);
}

hipError_t launch_pre_one(int T, int hidden, const uint16_t* X, const void* wprep, const float* scale,
                          const float* base, const uint16_t* norm_w, const Scalars& p, uint16_t* layer_input,
                          float* pre, float* post, float* comb, float* mixes, float* rstd, void* workspace,
                          hipStream_t stream) {
    char* ws = static_cast<char*>(workspace);
    PreOneArgs a;
    a.T = T;
    a.hidden = hidden;
    a.slices = hidden / kOneWidth;
    a.X = X;
    a.wprep = reinterpret_cast<const uint4*>(wprep);
    a.scale = scale;
    a.base = base;
    a.norm_w = norm_w;
    a.layer_input = layer_input;
    a.pre_out = pre;
    a.post_out = post;
    a.comb_out = comb;
    a.mixes_out = mixes;
    a.rstd_out = rstd;
    a.sync = reinterpret_cast<unsigned*>(ws);
    a.rec1 = reinterpret_cast<float*>(ws + kCounterBytes);
    a.rec2 = a.rec1 + (size_t)T * a.slices * kRec1;
    a.p = p;
    if (norm_w)
        hipLaunchKernelGGL(k_pre_one<true>, dim3(a.slices), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(k_pre_one<false>, dim3(a.slices), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace mhc
