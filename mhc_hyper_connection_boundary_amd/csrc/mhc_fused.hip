// Fused schedules of the mHC boundary and of the non-shifted pre: one
// workgroup owns a tile of tokens and all of hidden, so the partial sums never
// leave the chip.  Two shapes:
//   k_fused / k_fused_pre        8 waves, 16-token tiles (one token group per
//                                wave; two waves per SIMD);
//   k_fused_w4 / k_fused_pre_w4  4 waves, 32-token tiles (two token groups
//                                sharing each weight fragment; one wave per
//                                SIMD, so a wave may hold 512 registers).
// The host picks the shape from the batch size, the width and the number of
// compute units.
//
// A projection step of a wave covers 64 hidden elements (two 32-element MFMA
// k-blocks); wave w takes steps w, w + waves, ..., so the waves together sweep
// contiguous kilobytes of every row.  k_fused and k_fused_pre_w4 load and
// store in row layout, each instruction covering whole 128-byte runs of 8
// rows, and ds_bpermute moves the data into the matrix-core layout for the
// arithmetic and back for the stores (k_fused_pre loads both 64-byte halves
// of each line in the matrix-core layout).  k_fused_w4 splits the rows over
// its waves instead:
// each of its instructions covers 512-byte runs of 2 rows, and X' reaches the
// matrix-core layout through LDS.  While a wave computes step i (residual
// update, X' store, lagged collapse, sums of squares) the activations of step
// i+1 are in flight; the weight fragments of step i come from L2 and feed the
// matrix cores.  Where the token stride is a multiple of 16 KiB the boundary
// tiles start their sweeps at different steps, so that the tiles, which all
// run at about the same pace, do not hit the same columns at the same time.
//
// The BF16 li of the tile must wait for rstd_li, which depends on the whole
// row: the first 5 to 9 steps of every wave park it in LDS, the last one or
// two in registers, the steps between in the layer-input buffer itself, which
// the epilogue reads back and overwrites with the normalised values.  After
// the loop the waves' partials are combined in LDS in a fixed order; one quad
// per token computes pre / post / Sinkhorn comb while the other waves already
// write the layer input.  Every CU finishes its tile at about the same time,
// so nothing overlaps the epilogue: its loads (norm_w, the first parked steps)
// are requested before the reductions, and several parked steps stay in
// flight while it writes.
#include "mhc_device.h"
#include "mhc_launch.h"

namespace mhc {
namespace {

constexpr int kWaves = 8;
constexpr int kWide = 2 * kStep;  // hidden elements per wave step: two MFMA k-blocks

template <int S, int RegMax = 3>   // S = hidden / (kWaves * kWide): steps per wave
struct FusedShape {
    static constexpr int kSteps = S;
    static constexpr int kLiLds = S < 8 ? S : 8;  // first steps: li waits in LDS (16 KB each)
    static constexpr int kLiReg = S - kLiLds < RegMax ? S - kLiLds : RegMax;  // last: registers
};                                                // (steps between: layer_input)

template <int S>                  // the 8-wave pre keeps no li in registers
struct FusedPreShape {
    static constexpr int kSteps = S;
    static constexpr int kLiLds = FusedShape<S>::kLiLds;
    static constexpr int kLiReg = 0;
};

__device__ __forceinline__ uint4 load_stream(const uint16_t* p) {
    return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ void store_stream(uint16_t* p, const uint4& v) {
    *reinterpret_cast<uint4*>(p) = v;
}

// Row-layout activations of one wave step: instruction i, stream j: lane L
// holds row 8i + L/8 of the token group, bytes 16(L%8) of the step's 128-byte
// run, so each load instruction reads 8 rows x 128 bytes; HBM serves such
// runs faster than 16 rows x 64 bytes (a plain mover: 4.91 against
// 4.60 TB/s).  X and x are read once, with the nontemporal hint: the parked
// layer input that the epilogue reads back keeps more of the last-level
// cache (d=7168, T=8192: 295 -> 289-291 us; the same hint on the X' stores,
// on the parked li or on the final layer-input stores measured slower).
struct ActRows {
    uint4 X[2][4];  // [instruction][stream]
    uint4 x[2];
};

template <int kHidden>
__device__ __forceinline__ void load_rows(ActRows& a, const uint16_t* __restrict__ X,
                                          const uint16_t* __restrict__ x, const int (&tok)[2], int hl) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint16_t* Xr = X + (size_t)tok[i] * (4 * kHidden) + hl;
#pragma unroll
        for (int j = 0; j < 4; ++j) a.X[i][j] = ld16<true>(Xr + j * kHidden);
        a.x[i] = ld16<true>(x + (size_t)tok[i] * kHidden + hl);
    }
}

// Lane (g, n) of block b takes chunk 4b + g of row n: from instruction n / 8,
// lane 8(n % 8) + 4b + g.
__device__ __forceinline__ uint4 rows_to_mfma(const uint4& r0, const uint4& r1, int idx, bool hi) {
    uint4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int v0 = __builtin_amdgcn_ds_bpermute(idx, (int)word(r0, k));
        const int v1 = __builtin_amdgcn_ds_bpermute(idx, (int)word(r1, k));
        set_word(o, k, (uint32_t)(hi ? v1 : v0));
    }
    return o;
}

// The inverse move, for stores: row-layout register i (lane L: row 8i + L/8,
// chunk c = L%8) takes lane 16(c%4) + 8i + L/8 of matrix-core block c/4.
__device__ __forceinline__ uint4 mfma_to_rows(const uint4& m0, const uint4& m1, int idx, bool hi) {
    uint4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int v0 = __builtin_amdgcn_ds_bpermute(idx, (int)word(m0, k));
        const int v1 = __builtin_amdgcn_ds_bpermute(idx, (int)word(m1, k));
        set_word(o, k, (uint32_t)(hi ? v1 : v0));
    }
    return o;
}

__device__ __forceinline__ void load_frags(uint4 (&A)[kFragsPerStep], const uint4* __restrict__ wprep,
                                           int kblock, int lane) {
    const uint4* wp = wprep + (size_t)kblock * kFragsPerStep * 64 + lane;
#pragma unroll
    for (int i = 0; i < kFragsPerStep; ++i) A[i] = wp[i * 64];
}

// Writing the layer input of a token tile once rstd_li is known.  The li of
// a wave's steps sits in LDS (first kLiLds steps), in registers (last kLiReg)
// or, for the steps between, in the layer-input buffer itself.  prefetch()
// runs right after the main loop: it requests norm_w of the on-chip steps, then
// the first kDepth parked steps (li, written earlier by this same lane, and
// norm_w); since loads complete in issue order, the on-chip steps never wait
// for parked ones, and all of it is in flight during the reductions and the
// Sinkhorn.  emit() then writes the on-chip steps and the parked ones, each
// parked step's slot refilled kDepth steps ahead.  A lane owns kGroups tokens
// (16 apart); lanes past the last token write nothing, since another lane
// working on the same token T-1 would otherwise read back a value that has
// already been normalised.  kMaxDepth bounds the parked steps in flight.
//
// kNorm: norm_w is given.  Every kernel is built both ways and the host picks
// one, so no load sits under a branch on it: after a conditional block that
// loads, the compiler waits for every outstanding load where the paths join,
// which would expose the whole prefetch at once.
template <class Shape, int kWavesN, int kGroups, int kMaxDepth, bool kNorm>
struct LayerInputEpilogue {
    static constexpr int kParkEnd = Shape::kSteps - Shape::kLiReg;  // parked: [kLiLds, kParkEnd)
    static constexpr int kParked = kParkEnd - Shape::kLiLds;
    static constexpr int kDepth =  // parked steps in flight
        kParked < kMaxDepth ? (kParked > 0 ? kParked : 1) : kMaxDepth;
    static constexpr int kLds = Shape::kLiLds > 0 ? Shape::kLiLds : 1;
    static constexpr int kReg = Shape::kLiReg > 0 ? Shape::kLiReg : 1;

    const uint16_t* norm_w;
    uint16_t* li_row[kGroups];
    bool valid[kGroups];
    int wave, g;
    uint4 ring_li[kDepth][kGroups][2], ring_nw[kDepth][2];
    uint4 lds_nw[kLds][2], keep_nw[kReg][2];

    __device__ __forceinline__ int step_h(int i) const { return (i * kWavesN + wave) * kWide + g * 8; }

    // Lanes past the last token read the row of token T-1, whatever another
    // lane has written there; put() drops their values.
    __device__ __forceinline__ void load_parked(int i) {
        const int slot = (i - Shape::kLiLds) % kDepth, h = step_h(i);
        ring_nw[slot][0] = load_stream(norm_w + h);
        ring_nw[slot][1] = load_stream(norm_w + h + kStep);
#pragma unroll
        for (int q = 0; q < kGroups; ++q) {
            ring_li[slot][q][0] = load_stream(li_row[q] + h);
            ring_li[slot][q][1] = load_stream(li_row[q] + h + kStep);
        }
    }

    __device__ __forceinline__ void prefetch() {
        if constexpr (kNorm) {
#pragma unroll
            for (int i = 0; i < Shape::kLiLds; ++i) {
                lds_nw[i][0] = load_stream(norm_w + step_h(i));
                lds_nw[i][1] = load_stream(norm_w + step_h(i) + kStep);
            }
#pragma unroll
            for (int rr = 0; rr < Shape::kLiReg; ++rr) {
                keep_nw[rr][0] = load_stream(norm_w + step_h(kParkEnd + rr));
                keep_nw[rr][1] = load_stream(norm_w + step_h(kParkEnd + rr) + kStep);
            }
#pragma unroll
            for (int i = Shape::kLiLds; i < kParkEnd && i < Shape::kLiLds + kDepth; ++i) load_parked(i);
        }
    }


    __device__ __forceinline__ void put(int q, int h, const uint4& li, const uint4& nw, float r) {
        if (!valid[q]) return;
        uint4 out = li;
        if constexpr (kNorm) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t a = word(li, k), b = word(nw, k);
                set_word(out, k, pack_bf16((bf_lo(a) * r) * bf_lo(b), (bf_hi(a) * r) * bf_hi(b)));
            }
        }
        store_stream(li_row[q] + h, out);
    }

    // lds_li(i, q, b) and keep_li(rr, q, b): li of block b of token group q in
    // LDS step i and in register step rr.
    template <class LdsLi, class KeepLi>
    __device__ __forceinline__ void emit(const LdsLi& lds_li, const KeepLi& keep_li,
                                         const float (&r)[kGroups]) {
#pragma unroll
        for (int i = 0; i < Shape::kLiLds; ++i) {
            const int h = step_h(i);
#pragma unroll
            for (int q = 0; q < kGroups; ++q) {
                put(q, h, lds_li(i, q, 0), lds_nw[i][0], r[q]);
                put(q, h + kStep, lds_li(i, q, 1), lds_nw[i][1], r[q]);
            }
        }
#pragma unroll
        for (int rr = 0; rr < Shape::kLiReg; ++rr) {
            const int h = step_h(kParkEnd + rr);
#pragma unroll
            for (int q = 0; q < kGroups; ++q) {
                put(q, h, keep_li(rr, q, 0), keep_nw[rr][0], r[q]);
                put(q, h + kStep, keep_li(rr, q, 1), keep_nw[rr][1], r[q]);
            }
        }
        if constexpr (!kNorm) return;  // without norm_w the parked li already is the layer input
#pragma unroll
        for (int i = Shape::kLiLds; i < kParkEnd; ++i) {
            const int slot = (i - Shape::kLiLds) % kDepth, h = step_h(i);
#pragma unroll
            for (int q = 0; q < kGroups; ++q) {
                put(q, h, ring_li[slot][q][0], ring_nw[slot][0], r[q]);
                put(q, h + kStep, ring_li[slot][q][1], ring_nw[slot][1], r[q]);
            }
            if (i + kDepth < kParkEnd) load_parked(i + kDepth);
        }
    }
};

// The same for the kernels whose li is kept in row layout.  Register (q, k)
// of a lane holds one row of the tile (row[q][k]) and 8 elements at hl0 of
// each step's run, so a lane needs one norm_w register per step: in k_fused
// and k_fused_pre_w4 row 16q + 8k + L/8, chunk L%8 of the wave's 128-byte run
// (8 rows x 128 bytes per instruction); in k_fused_w4 one of the wave's 8
// tokens, chunk L%32 of the step's 512-byte run (wave index 0 here: the whole
// run is the wave's).  Lanes on rows past the last token read the row of
// token T-1 and write nothing, as above.  The wave's i-th step covers step
// (i + rot) mod kSteps of the row (the tile's rotation, see k_fused_w4);
// kNtOut puts the nontemporal hint on the final layer-input stores.
template <class Shape, int kWavesN, int kGroups, int kMaxDepth, bool kNorm, bool kNtOut>
struct LayerInputRows {
    static constexpr int kParkEnd = Shape::kSteps - Shape::kLiReg;  // parked: [kLiLds, kParkEnd)
    static constexpr int kParked = kParkEnd - Shape::kLiLds;
    static constexpr int kDepth = kParked < kMaxDepth ? (kParked > 0 ? kParked : 1) : kMaxDepth;
    static constexpr int kLds = Shape::kLiLds > 0 ? Shape::kLiLds : 1;
    static constexpr int kReg = Shape::kLiReg > 0 ? Shape::kLiReg : 1;

    const uint16_t* norm_w;
    uint16_t* row[kGroups][2];  // [group][instruction]
    bool valid[kGroups][2];
    int wave, hl0, rot;
    uint4 ring_li[kDepth][kGroups][2], ring_nw[kDepth];
    uint4 lds_nw[kLds], keep_nw[kReg];

    __device__ __forceinline__ int col(int i) const {
        const int a = i + rot >= Shape::kSteps ? i + rot - Shape::kSteps : i + rot;
        return (a * kWavesN + wave) * kWide + hl0;
    }

    __device__ __forceinline__ void load_parked(int i) {
        const int slot = (i - Shape::kLiLds) % kDepth, c = col(i);
        ring_nw[slot] = load_stream(norm_w + c);
#pragma unroll
        for (int q = 0; q < kGroups; ++q)
#pragma unroll
            for (int k = 0; k < 2; ++k) ring_li[slot][q][k] = load_stream(row[q][k] + c);
    }

    __device__ __forceinline__ void prefetch() {
        if constexpr (kNorm) {
#pragma unroll
            for (int i = 0; i < Shape::kLiLds; ++i) lds_nw[i] = load_stream(norm_w + col(i));
#pragma unroll
            for (int rr = 0; rr < Shape::kLiReg; ++rr) keep_nw[rr] = load_stream(norm_w + col(kParkEnd + rr));
#pragma unroll
            for (int i = Shape::kLiLds; i < kParkEnd && i < Shape::kLiLds + kDepth; ++i) load_parked(i);
        }
    }

    __device__ __forceinline__ void put(int q, int k, int c, const uint4& li, const uint4& nw, float r) {
        if (!valid[q][k]) return;
        uint4 out = li;
        if constexpr (kNorm) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t a = word(li, e), b = word(nw, e);
                set_word(out, e, pack_bf16((bf_lo(a) * r) * bf_lo(b), (bf_hi(a) * r) * bf_hi(b)));
            }
        }
        st16<kNtOut>(row[q][k] + c, out);
    }

    // lds_li(i, q, k) and keep_li(rr, q, k): li register (q, k) of LDS step i
    // and of register step rr; r[q][k]: rstd_li of that register's row.
    template <class LdsLi, class KeepLi>
    __device__ __forceinline__ void emit(const LdsLi& lds_li, const KeepLi& keep_li,
                                         const float (&r)[kGroups][2]) {
#pragma unroll
        for (int i = 0; i < Shape::kLiLds; ++i)
#pragma unroll
            for (int q = 0; q < kGroups; ++q)
#pragma unroll
                for (int k = 0; k < 2; ++k) put(q, k, col(i), lds_li(i, q, k), lds_nw[i], r[q][k]);
#pragma unroll
        for (int rr = 0; rr < Shape::kLiReg; ++rr)
#pragma unroll
            for (int q = 0; q < kGroups; ++q)
#pragma unroll
                for (int k = 0; k < 2; ++k)
                    put(q, k, col(kParkEnd + rr), keep_li(rr, q, k), keep_nw[rr], r[q][k]);
        if constexpr (!kNorm) return;  // without norm_w the parked li already is the layer input
#pragma unroll
        for (int i = Shape::kLiLds; i < kParkEnd; ++i) {
            const int slot = (i - Shape::kLiLds) % kDepth;
#pragma unroll
            for (int q = 0; q < kGroups; ++q)
#pragma unroll
                for (int k = 0; k < 2; ++k) put(q, k, col(i), ring_li[slot][q][k], ring_nw[slot], r[q][k]);
            if (i + kDepth < kParkEnd) load_parked(i + kDepth);
        }
    }
};

template <int S, bool kNorm>  // kNorm: norm_w is given
__global__ __launch_bounds__(512) void k_fused(
    int T, const uint16_t* __restrict__ x, const uint16_t* __restrict__ X,
    const float* __restrict__ post_prev, const float* __restrict__ comb_prev,
    const float* __restrict__ pre_lag, const uint4* __restrict__ wprep,
    const float* __restrict__ scale, const float* __restrict__ base,
    const uint16_t* __restrict__ norm_w, Scalars p, uint16_t* __restrict__ xn_out,
    uint16_t* __restrict__ layer_input, float* __restrict__ pre_out,
    float* __restrict__ post_out, float* __restrict__ comb_out, float* __restrict__ mixes_out,
    float* __restrict__ rstd_out) {
    MHC_POISON_LDS(0);
    using Shape = FusedShape<S, 1>;  // two or three li steps in registers spill (row-layout moves)
    constexpr int hidden = S * kWide * kWaves;
    __shared__ uint4 li_lds[Shape::kLiLds > 0 ? Shape::kLiLds : 1][kWaves][2][64];
    __shared__ float red[kWaves][kTile][24];
    __shared__ float sq[kWaves][4][kTile][2];
    __shared__ float tot[kTile][26];
    __shared__ float rli[kTile];

    const int tile = blockIdx.x;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int n = lane & 15;
    const int t0 = tile * kTile;
    const int t_end = min(t0 + kTile, T);
    const size_t tc = t0 + n < t_end ? (size_t)(t0 + n) : (size_t)(t_end - 1);

    PrevCoef c;
    load_prev(c, post_prev, comb_prev, pre_lag, tc);

    f32x4_t acc[3] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    float ssq = 0.0f, ssq_li = 0.0f;

    // Wave w takes steps w, w + 8, ...: at any moment the 8 waves cover 512
    // contiguous hidden elements of every row of the tile.  The activations
    // are loaded in row layout (lane L: row 8i + L/8, 8 rows x 128 bytes per
    // load), moved into the matrix-core layout with ds_bpermute, and X' and li
    // go back to row layout for their stores; where hidden is a multiple of
    // 2048 (token stride a multiple of 16 KiB) each tile starts its sweep at
    // its own step (the rotation of k_fused_w4).
    int tok[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int t = t0 + 8 * i + (lane >> 3);
        tok[i] = t < t_end ? t : t_end - 1;
    }
    const int hl0 = (lane & 7) * 8;
    const int pidx[2] = {(8 * (n & 7) + (lane >> 4)) * 4, (8 * (n & 7) + 4 + (lane >> 4)) * 4};
    const bool phi = n >= 8;
    const int ridx[2] = {(16 * (lane & 3) + (lane >> 3)) * 4, (16 * (lane & 3) + 8 + (lane >> 3)) * 4};
    const bool rhi = (lane & 7) >= 4;
    const bool row1 = t0 + 8 < t_end;  // rows 8..15 hold a token of the tile (uniform)
    constexpr bool kRotate = hidden % 2048 == 0;
    const int rot = kRotate ? (int)((((unsigned)tile * 2654435761u) >> 12) % (unsigned)S) : 0;
    auto astep = [&](int i) { return i + rot >= S ? i + rot - S : i + rot; };
    ActRows cur;
    load_rows<hidden>(cur, X, x, tok, (astep(0) * kWaves + wave) * kWide + hl0);
    // One wave step.  keep: li stays in the caller's registers (last steps);
    // otherwise it waits in LDS (first steps) or in the layer-input buffer.
    auto body = [&](int i, bool keep, uint4 (&li)[2]) {
        const int step = astep(i) * kWaves + wave;
        const int hr = step * kWide + hl0;
        ActRows nxt;
        if (i + 1 < S) load_rows<hidden>(nxt, X, x, tok, (astep(i + 1) * kWaves + wave) * kWide + hl0);
        uint4 Xn[2][4], lm[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            uint4 Xs[4], xs;
#pragma unroll
            for (int j = 0; j < 4; ++j) Xs[j] = rows_to_mfma(cur.X[0][j], cur.X[1][j], pidx[b], phi);
            xs = rows_to_mfma(cur.x[0], cur.x[1], pidx[b], phi);
            update_collapse(Xs, xs, c, Xn[b], lm[b], ssq, ssq_li);
        }
        // A lane past the last token works on the tile's last token, so it
        // stores the same bytes as that token's own lane; rows 8..15 of a tile
        // of at most 8 tokens are skipped (a uniform branch).
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const bool rows = k == 0 || row1;
            if (rows) {
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2)
                    st16<true>(xn_out + (size_t)tok[k] * (4 * hidden) + (size_t)s2 * hidden + hr,
                               mfma_to_rows(Xn[0][s2], Xn[1][s2], ridx[k], rhi));
            }
            li[k] = mfma_to_rows(lm[0], lm[1], ridx[k], rhi);
            if (!keep) {
                if (i < Shape::kLiLds)
                    li_lds[i][wave][k][lane] = li[k];
                else if (rows)
                    store_stream(layer_input + (size_t)tok[k] * hidden + hr, li[k]);
            }
        }
        // The weight fragments (L2-resident) are fetched only now, so they hold
        // no registers during the VALU work above; the other wave of the SIMD
        // runs its VALU phase while this one waits for them.
        __builtin_amdgcn_sched_barrier(0);
        uint4 A0[kFragsPerStep], A1[kFragsPerStep];
        load_frags(A0, wprep, 2 * step, lane);
        load_frags(A1, wprep, 2 * step + 1, lane);
        mfma_step(A0, Xn[0], acc);
        mfma_step(A1, Xn[1], acc);
        cur = nxt;
    };
#pragma unroll 1
    for (int i = 0; i < S - Shape::kLiReg; ++i) {
        uint4 li[2];
        body(i, false, li);
    }
    uint4 li_keep[Shape::kLiReg > 0 ? Shape::kLiReg : 1][2];
#pragma unroll
    for (int r = 0; r < Shape::kLiReg; ++r) body(S - Shape::kLiReg + r, true, li_keep[r]);
    // From here on the lane's indices come from an opaque copy of the thread
    // index (see k_fused_w4).
    int tl = (int)threadIdx.x;
    asm volatile("" : "+v"(tl));
    const int lw = tl >> 6, ll = tl & 63, ln = ll & 15, lg = ll >> 4, er = ll >> 3;
    // The coefficient parameters are requested before the epilogue's loads, so
    // that waiting for them does not wait for those.
    CoefParams cp;
    if (lw == 0) cp = load_coef_params(scale, base, ll & 3);
    auto erow = [&](int k) {
        const int t = t0 + 8 * k + er;
        return layer_input + (size_t)(t < t_end ? t : t_end - 1) * hidden;
    };
    LayerInputRows<Shape, kWaves, 1, 3, kNorm, true> out{
        norm_w, {{erow(0), erow(1)}}, {{t0 + er < t_end, t0 + 8 + er < t_end}}, lw, (ll & 7) * 8, rot};
    out.prefetch();

    // Partials of the 8 waves, combined in a fixed order.
#pragma unroll
    for (int m = 0; m < 3; ++m)
#pragma unroll
        for (int j = 0; j < 2; ++j) red[lw][ln][8 * m + 2 * lg + j] = mix_of(acc, m, j);
    sq[lw][lg][ln][0] = ssq;
    sq[lw][lg][ln][1] = ssq_li;
    __syncthreads();
    if (threadIdx.x < kTile * 26) {
        const int tn = threadIdx.x / 26, v = threadIdx.x % 26;
        float sum = 0.0f;
        if (v < 24) {
#pragma unroll
            for (int w = 0; w < kWaves; ++w) sum += red[w][tn][v];
        } else {
#pragma unroll
            for (int w = 0; w < kWaves; ++w)
#pragma unroll
                for (int q = 0; q < 4; ++q) sum += sq[w][q][tn][v - 24];
        }
        tot[tn][v] = sum;
        if (v == 25) rli[tn] = rsqrt_nr(sum * (1.0f / (float)hidden) + p.norm_eps);
    }
    __syncthreads();

    if (lw == 0) {
        const int tn = ll >> 2, i = ll & 3;
        const int tt = t0 + tn;
        const TokenCoef o = coefficients(tot[tn], i, hidden, cp, p);
        if (tt < T) {
            pre_out[(size_t)tt * 4 + i] = o.pre;
            post_out[(size_t)tt * 4 + i] = o.post;
            *reinterpret_cast<float4*>(comb_out + (size_t)tt * 16 + 4 * i) =
                make_float4(o.row[0], o.row[1], o.row[2], o.row[3]);
            if (mixes_out)
                for (int k = 0; k < 6; ++k) mixes_out[(size_t)tt * 24 + 6 * i + k] = tot[tn][6 * i + k];
            if (rstd_out && i == 0) rstd_out[tt] = o.rstd;
        }
    }

    // Layer input for this wave's steps.
    const float r[1][2] = {{rli[er], rli[8 + er]}};
    out.emit([&](int i, int, int k) { return li_lds[i][lw][k][ll]; },
             [&](int rr, int, int k) { return li_keep[rr][k]; }, r);
}

// ---------------------------------------------------------------------------
// Fused schedule on 4 waves per workgroup (one per SIMD) with 32-token tiles.
// The weight fragments are the costly loads of the 8-wave kernel: one 1 KB
// load per fragment per 16 tokens.  Here each wave feeds two 16-token groups
// (tokens n and n + 16 of the tile in lane n) from one set of fragments, which
// halves the fragment loads per token.  With one wave per SIMD a wave may hold
// 512 registers (architectural plus accumulation registers).  Each step issues
// its fragments first and the next step's activations after them, so the
// projection never waits on HBM (loads complete in issue order).
// ---------------------------------------------------------------------------
constexpr int kWaves4 = 4;
constexpr int kTileW4 = 32;

// S = hidden / (kWaves4 * kWide): steps; li of the first (at most LdsMax)
// steps waits in LDS, 16 KB each, and of the last (at most RegMax) in
// registers.
template <int S, int LdsMax = 8, int RegMax = 2>
struct FusedW4Shape {
    static constexpr int kSteps = S;
    static constexpr int kLiLds = S < LdsMax ? S : LdsMax;  // first steps: li waits in LDS
    static constexpr int kLiReg = S - kLiLds < RegMax ? S - kLiLds : RegMax;  // last: registers
};                                                // (steps between: layer_input)

// ---------------------------------------------------------------------------
// The 4-wave boundary.  The tile's rows are split over the waves for the
// memory side and its columns for the projection.  Wave w owns tokens
// 4w..4w+3 and 16+4w..16+4w+3 of the tile; at every step it loads, updates,
// stores and collapses 256 contiguous hidden elements of each of their rows:
// for p = 0..3, lane L holds token 4w + 16(p/2) + 2(p%2) + L/32 and 16-byte
// chunk L%32 of the step's 512-byte run, so every load and store instruction
// covers 2 rows x 512 bytes.  The update and the lagged collapse are
// elementwise and run in this layout as they are; only the projection needs
// the matrix-core layout.  X' therefore goes through LDS: for each half q of
// the tile (tokens 16q..16q+15, registers p = 2q, 2q+1 of every wave) a 32 KB
// stage ([token][stream][chunk], chunks XOR-swizzled by the token, so that
// both the row-order writes and the matrix-core reads are free of bank
// conflicts), from which each wave reads, after a barrier, the operands of its
// 64 columns (step 4i + w of 64 elements: MFMA k-blocks 8i + 2w, 8i + 2w + 1)
// for the 16 tokens.  The halves alternate, so the matrix-core work of one
// half overlaps the update of the other, and each stage is rewritten only
// after the barrier that follows its reads.  A wave owns the sums of squares
// of its tokens whole (a butterfly over a token's 32 lanes), so rstd_li needs
// no cross-wave step.  The stages leave room for 5 li steps in LDS; one more
// stays in registers (more measured no faster: the peeled steps' code).
// Against the previous design of this kernel (each wave on 64 columns of all
// 32 rows, 8 rows x 128 bytes per instruction, moved with ds_bpermute; li in
// LDS for 9 steps), cold, us: d=7168 T=8192 251 -> 244, T=5120 198 -> 183;
// d=8192 T=8192 287 -> 267; d=4096 T=8192 148 -> 134, T=16384 278 -> 254;
// d=1024 T=8192 49.5 -> 42.7; d=7168 T=16384 (two rounds) 499 -> 506.
// ---------------------------------------------------------------------------
constexpr int kRun = kWaves4 * kWide;  // hidden elements of a row per step (512 bytes)

// Row-run activations of one step: [p][stream] and [p] (see above).
struct ActRuns {
    uint4 X[4][4];
    uint4 x[4];
};

template <int kHidden>
__device__ __forceinline__ void load_runs(ActRuns& a, const uint16_t* __restrict__ X,
                                          const uint16_t* __restrict__ x, const int (&tok)[4], int h) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint16_t* Xr = X + (size_t)tok[q] * (4 * kHidden) + h;
#pragma unroll
        for (int j = 0; j < 4; ++j) a.X[q][j] = ld16<true>(Xr + j * kHidden);
        a.x[q] = ld16<true>(x + (size_t)tok[q] * kHidden + h);
    }
}

template <int S, bool kNorm>  // kNorm: norm_w is given
__global__ __launch_bounds__(256) void k_fused_w4(
    int T, int tile_tokens, const uint16_t* __restrict__ x, const uint16_t* __restrict__ X,
    const float* __restrict__ post_prev, const float* __restrict__ comb_prev,
    const float* __restrict__ pre_lag, const uint4* __restrict__ wprep,
    const float* __restrict__ scale, const float* __restrict__ base,
    const uint16_t* __restrict__ norm_w, Scalars p, uint16_t* __restrict__ xn_out,
    uint16_t* __restrict__ layer_input, float* __restrict__ pre_out,
    float* __restrict__ post_out, float* __restrict__ comb_out, float* __restrict__ mixes_out,
    float* __restrict__ rstd_out) {
    MHC_POISON_LDS(0);
    using Shape = FusedW4Shape<S, 5, 1>;
    constexpr int hidden = S * kRun;
    __shared__ uint4 stage[2][16 * 4 * 32];  // X' of one step: [half][token][stream][chunk ^ token]
    __shared__ uint4 li_lds[Shape::kLiLds > 0 ? Shape::kLiLds : 1][kWaves4][4][64];
    __shared__ __align__(16) PrevCoef cf[kTileW4];
    __shared__ float tot[kTileW4][25];  // 24 mixes, the sum of squares of X'

    const int tile = blockIdx.x;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int n = lane & 15;
    const int g = lane >> 4;
    const int ch = lane & 31;  // the lane's chunk of the step's 512-byte run
    const int t0 = tile * tile_tokens;
    const int t_end = min(t0 + tile_tokens, T);
    // Every CU runs its tile at about the same pace, so without a rotation all
    // tiles read and write the same columns of their rows at the same time.
    // Where the token stride (8 hidden bytes) is a multiple of 16 KiB, those
    // addresses share their low bits and crowd into a few memory channels:
    // there each tile starts its sweep at its own step, drawn from a
    // multiplicative hash of the tile index (a rotation equal to the tile index
    // itself correlates with the address bits and measured slower still).  The
    // step order is fixed per tile, so each token's sums still have one order.
    // Cold calls, T=8192 (us, lockstep -> rotated, measured on the previous
    // design): d=2048 93 -> 80, d=4096 184 -> 148, d=6144 260 -> 220, d=8192
    // 390 -> 284; stress d=4096 T=16384 350 -> 284.  At d=1024, 5120 and 7168
    // the rotation measured 1-9 us slower (the tiles of an XCD then stop
    // sharing the weight fragments in its L2).
    constexpr bool kRotate = S % 8 == 0;
    const int rot = kRotate ? (int)((((unsigned)tile * 2654435761u) >> 12) % (unsigned)S) : 0;
    auto astep = [&](int i) { return i + rot >= S ? i + rot - S : i + rot; };

    // The previous layer's coefficients of the tile's tokens, into LDS (token
    // rows past the tile's last token repeat it, as below).
    if (threadIdx.x < kTileW4 * 6) {
        const int tl = threadIdx.x / 6, k = threadIdx.x - 6 * (threadIdx.x / 6);
        const size_t t = (size_t)min(t0 + tl, t_end - 1);
        const float* src = k == 0 ? post_prev + t * 4 : k == 5 ? pre_lag + t * 4 : comb_prev + t * 16 + 4 * (k - 1);
        reinterpret_cast<float4*>(&cf[tl])[k] = *reinterpret_cast<const float4*>(src);
    }

    // A lane past the tile's last token works on that token (its loads and its
    // share of the stage) but stores nothing: the token's own lane may sit in
    // another wave.
    int tl[4], tok[4];
    bool own[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        tl[q] = 4 * wave + 16 * (q >> 1) + 2 * (q & 1) + (lane >> 5);
        own[q] = t0 + tl[q] < t_end;
        tok[q] = own[q] ? t0 + tl[q] : t_end - 1;
    }

    f32x4_t acc[2][3];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int m = 0; m < 3; ++m) acc[q][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float ssq[4] = {0.0f, 0.0f, 0.0f, 0.0f}, ssq_li[4] = {0.0f, 0.0f, 0.0f, 0.0f};

    // One activation buffer: as soon as a half's update has read its rows,
    // the same registers receive that half's rows of the next step, so the
    // loads of the next step are in flight during the rest of this one with
    // no second buffer and no register copy.
    ActRuns cur;
    load_runs<hidden>(cur, X, x, tok, astep(0) * kRun + 8 * ch);
    __syncthreads();  // cf
    // One step.  keep: li stays in the caller's registers (last step);
    // otherwise it waits in LDS (first steps) or in the layer-input buffer.
    auto body = [&](int i, bool keep, uint4 (&li)[4]) {
        const int step = astep(i) * kWaves4 + wave;  // the wave's 64 columns for the projection
        const int h = astep(i) * kRun + 8 * ch;
        const int hn = astep(i + 1 < S ? i + 1 : i) * kRun + 8 * ch;  // the next step's
        uint4 A0[kFragsPerStep], A1[kFragsPerStep];
        load_frags(A0, wprep, 2 * step, lane);
        load_frags(A1, wprep, 2 * step + 1, lane);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int hq = 0; hq < 2; ++hq) {
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int q = 2 * hq + k, t16 = tl[q] - 16 * hq;
                const PrevCoef c = cf[tl[q]];
                uint4 Xn[4];
                update_collapse(cur.X[q], cur.x[q], c, Xn, li[q], ssq[q], ssq_li[q]);
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) {
                    if (own[q])  // X' is not read again here: nontemporal
                        st16<true>(xn_out + (size_t)tok[q] * (4 * hidden) + (size_t)s2 * hidden + h, Xn[s2]);
                    stage[hq][(t16 * 4 + s2) * 32 + (ch ^ t16)] = Xn[s2];
                }
                if (!keep) {
                    if (i < Shape::kLiLds)
                        li_lds[i][wave][q][lane] = li[q];
                    else if (own[q])
                        store_stream(layer_input + (size_t)tok[q] * hidden + h, li[q]);
                }
            }
            if (i + 1 < S) {
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const int q = 2 * hq + k;
                    const uint16_t* Xr = X + (size_t)tok[q] * (4 * hidden) + hn;
#pragma unroll
                    for (int j = 0; j < 4; ++j) cur.X[q][j] = ld16<true>(Xr + j * hidden);
                    cur.x[q] = ld16<true>(x + (size_t)tok[q] * hidden + hn);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            uint4 B[2][4];
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) B[b][s2] = stage[hq][(n * 4 + s2) * 32 + ((8 * wave + 4 * b + g) ^ n)];
            mfma_step(A0, B[0], acc[hq]);
            mfma_step(A1, B[1], acc[hq]);
        }
    };
#pragma unroll 1
    for (int i = 0; i < S - Shape::kLiReg; ++i) {
        uint4 li[4];
        body(i, false, li);
    }
    uint4 li_keep[Shape::kLiReg > 0 ? Shape::kLiReg : 1][4];
#pragma unroll
    for (int r = 0; r < Shape::kLiReg; ++r) body(S - Shape::kLiReg + r, true, li_keep[r]);
    // From here on the lane's indices come from an opaque copy of the thread
    // index, so the compiler cannot compute them before the loop and keep them
    // (spilled) through it: a reload from scratch would wait for every load the
    // epilogue has in flight.
    int tx = (int)threadIdx.x;
    asm volatile("" : "+v"(tx));
    const int lw = tx >> 6, ll = tx & 63, ln = ll & 15, lg = ll >> 4, lh = ll >> 5;
    CoefParams cp;
    if (lw < 2) cp = load_coef_params(scale, base, ll & 3);
    // Epilogue register (q, k) is the lane's token p = 2q + k.
    auto etok = [&](int q, int k) { return 4 * lw + 16 * q + 2 * k + lh; };
    auto erow = [&](int q, int k) {
        const int t = t0 + etok(q, k);
        return layer_input + (size_t)(t < t_end ? t : t_end - 1) * hidden;
    };
    auto evalid = [&](int q, int k) { return t0 + etok(q, k) < t_end; };
    // The wave's columns are the whole 256 of each step (wave index 0 there).
    LayerInputRows<Shape, kWaves4, 2, 5, kNorm, true> out{
        norm_w, {{erow(0, 0), erow(0, 1)}, {erow(1, 0), erow(1, 1)}},
        {{evalid(0, 0), evalid(0, 1)}, {evalid(1, 0), evalid(1, 1)}}, 0, (ll & 31) * 8, rot};
    out.prefetch();

    // The wave's own tokens: sums of squares over their 32 lanes (butterfly,
    // the same bits in every lane), rstd_li in registers, the X' sum into tot.
    float rl[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        float a = ssq[q], b = ssq_li[q];
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) {
            a += __shfl_xor(a, o);
            b += __shfl_xor(b, o);
        }
        if ((ll & 31) == 0) tot[etok(q >> 1, q & 1)][24] = a;
        rl[q] = rsqrt_nr(b * (1.0f / (float)hidden) + p.norm_eps);
    }
    // Mixes of the 4 waves, added into tot one wave at a time from 0.0f, wave
    // 0 first: each mix is ((w0 + w1) + w2) + w3.
#pragma unroll
    for (int w = 0; w < kWaves4; ++w) {
        if (lw == w) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int tn = 16 * q + ln;
#pragma unroll
                for (int m = 0; m < 3; ++m)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int v = 8 * m + 2 * lg + j;
                        tot[tn][v] = (w == 0 ? 0.0f : tot[tn][v]) + mix_of(acc[q], m, j);
                    }
            }
        }
        __syncthreads();
    }

    if (lw < 2) {  // 32 tokens x 4 lanes: waves 0 and 1
        const int tn = 16 * lw + (ll >> 2), ci = ll & 3;
        const int tt = t0 + tn;
        const TokenCoef o = coefficients(tot[tn], ci, hidden, cp, p);
        if (tt < t_end) {
            pre_out[(size_t)tt * 4 + ci] = o.pre;
            post_out[(size_t)tt * 4 + ci] = o.post;
            *reinterpret_cast<float4*>(comb_out + (size_t)tt * 16 + 4 * ci) =
                make_float4(o.row[0], o.row[1], o.row[2], o.row[3]);
            if (mixes_out)
                for (int k = 0; k < 6; ++k) mixes_out[(size_t)tt * 24 + 6 * ci + k] = tot[tn][6 * ci + k];
            if (rstd_out && ci == 0) rstd_out[tt] = o.rstd;
        }
    }

    // Layer input of the wave's tokens.
    const float r[2][2] = {{rl[0], rl[1]}, {rl[2], rl[3]}};
    out.emit([&](int i, int q, int k) { return li_lds[i][lw][2 * q + k][ll]; },
             [&](int rr, int q, int k) { return li_keep[rr][2 * q + k]; }, r);
}

template <int S>
hipError_t launch_w4_s(int T, int tile_tokens, const uint16_t* x, const uint16_t* X, const float* post_prev,
                       const float* comb_prev, const float* pre_lag, const void* wprep,
                       const float* scale, const float* base, const uint16_t* norm_w,
                       const Scalars& p, uint16_t* xn_out, uint16_t* layer_input,
                       float* pre_out, float* post_out, float* comb_out, float* mixes,
                       float* rstd, hipStream_t stream) {
    hipLaunchKernelGGL((norm_w ? k_fused_w4<S, true> : k_fused_w4<S, false>),
                       dim3((T + tile_tokens - 1) / tile_tokens), dim3(kWaves4 * 64), 0, stream,
                       T, tile_tokens, x, X, post_prev, comb_prev, pre_lag,
                       reinterpret_cast<const uint4*>(wprep), scale, base, norm_w, p, xn_out,
                       layer_input, pre_out, post_out, comb_out, mixes, rstd);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Non-shifted pre, fused: one 8-wave workgroup per 16-token tile.  Pass 1
// streams the tile's X through the sums of squares and the projection (same
// step order as k_fused, X' = X), loading it in the matrix-core layout
// itself.  After the fixed-order
// reduction wave 0 publishes pre, then runs the Sinkhorn; pass 2 reads the
// tile's X again, which was read a few tens of microseconds earlier and is
// normally still in the last-level cache, collapses it with the fresh pre,
// and parks li as k_fused does (LDS for the first steps, then the
// layer-input buffer) until rstd_li is known.
// ---------------------------------------------------------------------------
// Lane (n, g) holds, for token n, the 8 hidden elements 64*step + 32*b + 8*g
// + [0, 8) of block b = 0, 1 (both 64-byte halves of every 128-byte line, read
// back to back); block b is directly the B operand of MFMA k-block 2*step + b.
struct ActX {
    uint4 X[2][4];  // [block][stream]
};

__device__ __forceinline__ void load_x4(ActX& a, const uint16_t* __restrict__ Xrow, int hidden,
                                        int h) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        a.X[0][j] = load_stream(Xrow + (size_t)j * hidden + h);
        a.X[1][j] = load_stream(Xrow + (size_t)j * hidden + h + kStep);
    }
}

// Row-layout X of one wave step (the pre has no block output): as ActRows
// without x.  Plain loads: the second pass reads X again.
struct ActRowsX {
    uint4 X[2][4];  // [instruction][stream]
};

template <int kHidden>
__device__ __forceinline__ void load_rows_x(ActRowsX& a, const uint16_t* __restrict__ X,
                                            const int (&tok)[2], int hl) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint16_t* Xr = X + (size_t)tok[i] * (4 * kHidden) + hl;
#pragma unroll
        for (int j = 0; j < 4; ++j) a.X[i][j] = load_stream(Xr + j * kHidden);
    }
}

// The matrix-core blocks of a row-layout step.
__device__ __forceinline__ void rows_x_to_mfma(const ActRowsX& a, uint4 (&m)[2][4], const int (&pidx)[2],
                                               bool phi) {
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j) m[b][j] = rows_to_mfma(a.X[0][j], a.X[1][j], pidx[b], phi);
}

// li = bf16(FMA chain over j of pre[j] * X[j], from 0) for 8 elements; adds li^2.
__device__ __forceinline__ uint4 collapse8(const uint4 (&Xv)[4], const float (&pr)[4],
                                           float& ssq_li) {
    uint4 li;
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
    return li;
}

template <int S, bool kNorm>  // kNorm: norm_w is given
__global__ __launch_bounds__(512) void k_fused_pre(
    int T, const uint16_t* __restrict__ X, const uint4* __restrict__ wprep,
    const float* __restrict__ scale, const float* __restrict__ base,
    const uint16_t* __restrict__ norm_w, Scalars p, uint16_t* __restrict__ layer_input,
    float* __restrict__ pre_out, float* __restrict__ post_out, float* __restrict__ comb_out,
    float* __restrict__ mixes_out, float* __restrict__ rstd_out) {
    MHC_POISON_LDS(0);
    using Shape = FusedShape<S>;
    using PreShape = FusedPreShape<S>;
    constexpr int hidden = S * kWide * kWaves;
    __shared__ uint4 li_lds[Shape::kLiLds > 0 ? Shape::kLiLds : 1][kWaves][2][64];
    __shared__ float red[kWaves][kTile][24];
    __shared__ float sq[kWaves][4][kTile];
    __shared__ float tot[kTile][26];
    __shared__ float pre_s[kTile][4];
    __shared__ float rli[kTile];

    const int tile = blockIdx.x;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int n = lane & 15;
    const int g = lane >> 4;
    const int t = tile * kTile + n;
    const size_t tc = t < T ? (size_t)t : (size_t)(T - 1);
    const uint16_t* Xrow = X + tc * 4 * hidden;
    uint16_t* li_row = layer_input + tc * hidden;

    // Pass 1: sums of squares and the projection.
    f32x4_t acc[3] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    float ssq = 0.0f;
    ActX cur;
    load_x4(cur, Xrow, hidden, wave * kWide + g * 8);
#pragma unroll 1
    for (int i = 0; i < S; ++i) {
        const int step = i * kWaves + wave;
        const int h = step * kWide + g * 8;
        ActX nxt;
        if (i + 1 < S) load_x4(nxt, Xrow, hidden, h + kWaves * kWide);
        square_sum(cur.X[0], ssq);
        square_sum(cur.X[1], ssq);
        __builtin_amdgcn_sched_barrier(0);
        uint4 A0[kFragsPerStep], A1[kFragsPerStep];
        load_frags(A0, wprep, 2 * step, lane);
        load_frags(A1, wprep, 2 * step + 1, lane);
        mfma_step(A0, cur.X[0], acc);
        mfma_step(A1, cur.X[1], acc);
        cur = nxt;
    }
    // Pass 2's first activations are requested before the reductions.
    load_x4(cur, Xrow, hidden, wave * kWide + g * 8);
    CoefParams cp;
    if (wave == 0) cp = load_coef_params(scale, base, lane & 3);
#pragma unroll
    for (int m = 0; m < 3; ++m)
#pragma unroll
        for (int j = 0; j < 2; ++j) red[wave][n][8 * m + 2 * g + j] = mix_of(acc, m, j);
    sq[wave][g][n] = ssq;
    __syncthreads();
    if (threadIdx.x < kTile * 25) {
        const int tn = threadIdx.x / 25, v = threadIdx.x % 25;
        float sum = 0.0f;
        if (v < 24) {
#pragma unroll
            for (int w = 0; w < kWaves; ++w) sum += red[w][tn][v];
        } else {
#pragma unroll
            for (int w = 0; w < kWaves; ++w)
#pragma unroll
                for (int q = 0; q < 4; ++q) sum += sq[w][q][tn];
        }
        tot[tn][v] = sum;
    }
    __syncthreads();
    TokenCoef o;
    const int ctn = lane >> 2, ci = lane & 3;
    if (wave == 0) {
        pre_post(o, tot[ctn], ci, hidden, cp, p);
        pre_s[ctn][ci] = o.pre;
    }
    __syncthreads();
    if (wave == 0) {
        comb_row(o, tot[ctn], ci, cp, p);
        const int tt = tile * kTile + ctn;
        if (tt < T) {
            pre_out[(size_t)tt * 4 + ci] = o.pre;
            post_out[(size_t)tt * 4 + ci] = o.post;
            *reinterpret_cast<float4*>(comb_out + (size_t)tt * 16 + 4 * ci) =
                make_float4(o.row[0], o.row[1], o.row[2], o.row[3]);
            if (mixes_out)
                for (int k = 0; k < 6; ++k) mixes_out[(size_t)tt * 24 + 6 * ci + k] = tot[ctn][6 * ci + k];
            if (rstd_out && ci == 0) rstd_out[tt] = o.rstd;
        }
    }

    // Pass 2: the collapse with the fresh pre.
    const float pr[4] = {pre_s[n][0], pre_s[n][1], pre_s[n][2], pre_s[n][3]};
    float ssq_li = 0.0f;
#pragma unroll 1
    for (int i = 0; i < S; ++i) {
        const int step = i * kWaves + wave;
        const int h = step * kWide + g * 8;
        ActX nxt;
        if (i + 1 < S) load_x4(nxt, Xrow, hidden, h + kWaves * kWide);
        const uint4 l0 = collapse8(cur.X[0], pr, ssq_li);
        const uint4 l1 = collapse8(cur.X[1], pr, ssq_li);
        if (i < Shape::kLiLds) {
            li_lds[i][wave][0][lane] = l0;
            li_lds[i][wave][1][lane] = l1;
        } else {
            store_stream(li_row + h, l0);
            store_stream(li_row + h + kStep, l1);
        }
        cur = nxt;
    }
    LayerInputEpilogue<PreShape, kWaves, 1, 5, kNorm> out{norm_w, {li_row}, {t < T}, wave, g};
    out.prefetch();
    sq[wave][g][n] = ssq_li;
    __syncthreads();
    if (threadIdx.x < kTile) {
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
#pragma unroll
            for (int q = 0; q < 4; ++q) sum += sq[w][q][threadIdx.x];
        rli[threadIdx.x] = rsqrt_nr(sum * (1.0f / (float)hidden) + p.norm_eps);
    }
    __syncthreads();
    const float r[1] = {rli[n]};
    out.emit([&](int i, int, int b) { return li_lds[i][wave][b][lane]; },
             [&](int, int, int) { return uint4{}; }, r);
}

template <int S, bool kNorm>  // kNorm: norm_w is given
__global__ __launch_bounds__(256) void k_fused_pre_w4(
    int T, const uint16_t* __restrict__ X, const uint4* __restrict__ wprep,
    const float* __restrict__ scale, const float* __restrict__ base,
    const uint16_t* __restrict__ norm_w, Scalars p, uint16_t* __restrict__ layer_input,
    float* __restrict__ pre_out, float* __restrict__ post_out, float* __restrict__ comb_out,
    float* __restrict__ mixes_out, float* __restrict__ rstd_out) {
    MHC_POISON_LDS(0);
    using Shape = FusedW4Shape<S, 9>;
    constexpr int hidden = S * kWide * kWaves4;
    __shared__ uint4 li_lds[Shape::kLiLds > 0 ? Shape::kLiLds : 1][kWaves4][2][2][64];
    __shared__ float sq[kWaves4][4][kTileW4];
    __shared__ float tot[kTileW4][26];
    __shared__ float pre_s[kTileW4][4];
    __shared__ float rli[kTileW4];
    // Pass 1's per-wave mixes live in the li area: pass 2 writes li only after
    // they have been summed (barriers in between).
    static_assert(sizeof(float) * kWaves4 * kTileW4 * 24 <= sizeof(li_lds), "mix partials fit");
    float (*red)[kTileW4][24] = reinterpret_cast<float (*)[kTileW4][24]>(&li_lds[0][0][0][0][0]);

    const int tile = blockIdx.x;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int n = lane & 15;
    const int g = lane >> 4;
    const int t0 = tile * kTileW4;
    // Row layout as in k_fused: lane L loads row 8i + L/8 of token group q
    // (tokens past the last one clamped to it), 8 rows x 128 bytes per load;
    // ds_bpermute moves the data into the matrix-core layout, where the sums
    // and the collapse run on the same values in the same order as before, and
    // li goes back to row layout for its stores.
    int tok[2][2];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int t = t0 + 16 * q + 8 * i + (lane >> 3);
            tok[q][i] = t < T ? t : T - 1;
        }
    const int hl0 = (lane & 7) * 8;
    const int pidx[2] = {(8 * (n & 7) + g) * 4, (8 * (n & 7) + 4 + g) * 4};
    const bool phi = n >= 8;
    const int ridx[2] = {(16 * (lane & 3) + (lane >> 3)) * 4, (16 * (lane & 3) + 8 + (lane >> 3)) * 4};
    const bool rhi = (lane & 7) >= 4;
    // Rotated sweeps as in k_fused_w4 (cold, T=8192: d=4096 137 -> 132 us,
    // d=8192 321 -> 283 us; both passes take the same step order).
    constexpr bool kRotate = hidden % 2048 == 0;
    const int rot = kRotate ? (int)((((unsigned)tile * 2654435761u) >> 12) % (unsigned)S) : 0;
    auto astep = [&](int i) { return i + rot >= S ? i + rot - S : i + rot; };

    // Pass 1: sums of squares and the projection.
    f32x4_t acc[2][3];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int m = 0; m < 3; ++m) acc[q][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float ssq[2] = {0.0f, 0.0f};
    ActRowsX cur[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) load_rows_x<hidden>(cur[q], X, tok[q], (astep(0) * kWaves4 + wave) * kWide + hl0);
#pragma unroll 1
    for (int i = 0; i < S; ++i) {
        const int step = astep(i) * kWaves4 + wave;
        uint4 A0[kFragsPerStep], A1[kFragsPerStep];
        load_frags(A0, wprep, 2 * step, lane);
        load_frags(A1, wprep, 2 * step + 1, lane);
        __builtin_amdgcn_sched_barrier(0);
        ActRowsX nxt[2];
        if (i + 1 < S) {
#pragma unroll
            for (int q = 0; q < 2; ++q)
                load_rows_x<hidden>(nxt[q], X, tok[q], (astep(i + 1) * kWaves4 + wave) * kWide + hl0);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            uint4 Xm[2][4];
            rows_x_to_mfma(cur[q], Xm, pidx, phi);
            square_sum(Xm[0], ssq[q]);
            square_sum(Xm[1], ssq[q]);
            mfma_step(A0, Xm[0], acc[q]);
            mfma_step(A1, Xm[1], acc[q]);
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) cur[q] = nxt[q];
    }
    // Pass 2's first activations are requested before the reductions.
#pragma unroll
    for (int q = 0; q < 2; ++q) load_rows_x<hidden>(cur[q], X, tok[q], (astep(0) * kWaves4 + wave) * kWide + hl0);
    CoefParams cp;
    if (wave < 2) cp = load_coef_params(scale, base, lane & 3);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
        for (int m = 0; m < 3; ++m)
#pragma unroll
            for (int j = 0; j < 2; ++j) red[wave][16 * q + n][8 * m + 2 * g + j] = mix_of(acc[q], m, j);
        sq[wave][g][16 * q + n] = ssq[q];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < kTileW4 * 25; idx += kWaves4 * 64) {
        const int tn = idx / 25, v = idx % 25;
        float sum = 0.0f;
        if (v < 24) {
#pragma unroll
            for (int w = 0; w < kWaves4; ++w) sum += red[w][tn][v];
        } else {
#pragma unroll
            for (int w = 0; w < kWaves4; ++w)
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) sum += sq[w][qq][tn];
        }
        tot[tn][v] = sum;
    }
    __syncthreads();
    TokenCoef o;
    const int ctn = 16 * (wave & 1) + (lane >> 2), ci = lane & 3;
    if (wave < 2) {
        pre_post(o, tot[ctn], ci, hidden, cp, p);
        pre_s[ctn][ci] = o.pre;
    }
    __syncthreads();
    if (wave < 2) {  // the Sinkhorn of the 32 tokens, ahead of these waves' collapse
        comb_row(o, tot[ctn], ci, cp, p);
        const int tt = t0 + ctn;
        if (tt < T) {
            pre_out[(size_t)tt * 4 + ci] = o.pre;
            post_out[(size_t)tt * 4 + ci] = o.post;
            *reinterpret_cast<float4*>(comb_out + (size_t)tt * 16 + 4 * ci) =
                make_float4(o.row[0], o.row[1], o.row[2], o.row[3]);
            if (mixes_out)
                for (int k = 0; k < 6; ++k) mixes_out[(size_t)tt * 24 + 6 * ci + k] = tot[ctn][6 * ci + k];
            if (rstd_out && ci == 0) rstd_out[tt] = o.rstd;
        }
    }

    // Pass 2: the collapse with the fresh pre.
    float pr[2][4];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j) pr[q][j] = pre_s[16 * q + n][j];
    float ssq_li[2] = {0.0f, 0.0f};
    auto body = [&](int i, bool keep, uint4 (&li)[2][2]) {
        const int step = astep(i) * kWaves4 + wave;
        const int hr = step * kWide + hl0;
        ActRowsX nxt[2];
        if (i + 1 < S) {
#pragma unroll
            for (int q = 0; q < 2; ++q)
                load_rows_x<hidden>(nxt[q], X, tok[q], (astep(i + 1) * kWaves4 + wave) * kWide + hl0);
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            uint4 Xm[2][4], lm[2];
            rows_x_to_mfma(cur[q], Xm, pidx, phi);
            lm[0] = collapse8(Xm[0], pr[q], ssq_li[q]);
            lm[1] = collapse8(Xm[1], pr[q], ssq_li[q]);
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                li[q][k] = mfma_to_rows(lm[0], lm[1], ridx[k], rhi);
                if (!keep) {
                    if (i < Shape::kLiLds)
                        li_lds[i][wave][q][k][lane] = li[q][k];
                    else
                        store_stream(layer_input + (size_t)tok[q][k] * hidden + hr, li[q][k]);
                }
            }
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) cur[q] = nxt[q];
    };
#pragma unroll 1
    for (int i = 0; i < S - Shape::kLiReg; ++i) {
        uint4 li[2][2];
        body(i, false, li);
    }
    uint4 li_keep[Shape::kLiReg > 0 ? Shape::kLiReg : 1][2][2];
#pragma unroll
    for (int r = 0; r < Shape::kLiReg; ++r) body(S - Shape::kLiReg + r, true, li_keep[r]);
    // The epilogue's rows come from an opaque copy of the thread index (see k_fused_w4).
    int tl = (int)threadIdx.x;
    asm volatile("" : "+v"(tl));
    const int er = (tl & 63) >> 3;
    auto erow = [&](int q, int k) {
        const int t = t0 + 16 * q + 8 * k + er;
        return layer_input + (size_t)(t < T ? t : T - 1) * hidden;
    };
    LayerInputRows<Shape, kWaves4, 2, 5, kNorm, false> out{
        norm_w, {{erow(0, 0), erow(0, 1)}, {erow(1, 0), erow(1, 1)}},
        {{t0 + er < T, t0 + 8 + er < T}, {t0 + 16 + er < T, t0 + 24 + er < T}}, tl >> 6, (tl & 7) * 8, rot};
    out.prefetch();

#pragma unroll
    for (int q = 0; q < 2; ++q) sq[wave][g][16 * q + n] = ssq_li[q];
    __syncthreads();
    if (threadIdx.x < kTileW4) {
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves4; ++w)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) sum += sq[w][qq][threadIdx.x];
        rli[threadIdx.x] = rsqrt_nr(sum * (1.0f / (float)hidden) + p.norm_eps);
    }
    __syncthreads();
    const float r[2][2] = {{rli[er], rli[8 + er]}, {rli[16 + er], rli[24 + er]}};
    out.emit([&](int i, int q, int k) { return li_lds[i][wave][q][k][lane]; },
             [&](int rr, int q, int k) { return li_keep[rr][q][k]; }, r);
}

template <int S>
hipError_t launch_pre_w4_s(int T, const uint16_t* X, const void* wprep, const float* scale,
                           const float* base, const uint16_t* norm_w, const Scalars& p,
                           uint16_t* layer_input, float* pre_out, float* post_out,
                           float* comb_out, float* mixes, float* rstd, hipStream_t stream) {
    hipLaunchKernelGGL((norm_w ? k_fused_pre_w4<S, true> : k_fused_pre_w4<S, false>),
                       dim3((T + kTileW4 - 1) / kTileW4), dim3(kWaves4 * 64), 0, stream, T, X,
                       reinterpret_cast<const uint4*>(wprep), scale, base, norm_w, p,
                       layer_input, pre_out, post_out, comb_out, mixes, rstd);
    return hipGetLastError();
}

template <int S>
hipError_t launch_pre_s(int T, const uint16_t* X, const void* wprep, const float* scale,
                        const float* base, const uint16_t* norm_w, const Scalars& p,
                        uint16_t* layer_input, float* pre_out, float* post_out, float* comb_out,
                        float* mixes, float* rstd, hipStream_t stream) {
    hipLaunchKernelGGL((norm_w ? k_fused_pre<S, true> : k_fused_pre<S, false>),
                       dim3((T + kTile - 1) / kTile), dim3(kWaves * 64), 0, stream, T, X,
                       reinterpret_cast<const uint4*>(wprep), scale, base, norm_w, p,
                       layer_input, pre_out, post_out, comb_out, mixes, rstd);
    return hipGetLastError();
}

template <int S>
hipError_t launch_s(int T, const uint16_t* x, const uint16_t* X, const float* post_prev,
                    const float* comb_prev, const float* pre_lag, const void* wprep,
                    const float* scale, const float* base, const uint16_t* norm_w,
                    const Scalars& p, uint16_t* xn_out, uint16_t* layer_input, float* pre_out,
                    float* post_out, float* comb_out, float* mixes, float* rstd,
                    hipStream_t stream) {
    hipLaunchKernelGGL((norm_w ? k_fused<S, true> : k_fused<S, false>),
                       dim3((T + kTile - 1) / kTile), dim3(kWaves * 64), 0, stream,
                       T, x, X, post_prev, comb_prev, pre_lag,
                       reinterpret_cast<const uint4*>(wprep), scale, base, norm_w, p, xn_out,
                       layer_input, pre_out, post_out, comb_out, mixes, rstd);
    return hipGetLastError();
}

}  // namespace

// The boundary kernels at hidden 7168 come from further compilations of this
// file, each under another of LLVM's machine schedulers: the 16-token kernel
// under max-ilp (MHC_FUSED_MAXILP), the 4-wave kernel under max-memory-clause
// (MHC_FUSED_MAXCLAUSE).  The same arithmetic in the same order, so the same
// bits.  Cold, d=7168, us, default scheduler -> the unit's: 16-token tiles
// (two runs) T=2560 115 -> 111.6 / 113.0, T=4096 135 -> 130.8 / 134.8, T=9216
// 358 -> 340.5 / 338.8, T=12288 392 -> 378 / 378.7; 4-wave tiles T=4608 173.2
// -> 167.5, T=5120 183.6 -> 177.5, T=8192 244.5 -> 243.3, T=6144 and 16384
// level.  The 4-wave kernel measured level under max-ilp; the 16-token kernel
// measured 1-8% slower under max-ilp at hidden 4096, 5120, 6144 and 8192, so
// the other widths keep the default scheduler.
hipError_t launch_fused_7168(int T, const uint16_t* x, const uint16_t* X, const float* post_prev,
                             const float* comb_prev, const float* pre_lag, const void* wprep,
                             const float* scale, const float* base, const uint16_t* norm_w,
                             const Scalars& p, uint16_t* xn_out, uint16_t* layer_input,
                             float* pre_out, float* post_out, float* comb_out, float* mixes,
                             float* rstd, hipStream_t stream);
hipError_t launch_fused_w4_7168(int T, int tile_tokens, const uint16_t* x, const uint16_t* X,
                                const float* post_prev, const float* comb_prev,
                                const float* pre_lag, const void* wprep, const float* scale,
                                const float* base, const uint16_t* norm_w, const Scalars& p,
                                uint16_t* xn_out, uint16_t* layer_input, float* pre_out,
                                float* post_out, float* comb_out, float* mixes, float* rstd,
                                hipStream_t stream);

#if defined(MHC_FUSED_MAXCLAUSE)

hipError_t launch_fused_w4_7168(int T, int tile_tokens, const uint16_t* x, const uint16_t* X,
                                const float* post_prev, const float* comb_prev,
                                const float* pre_lag, const void* wprep, const float* scale,
                                const float* base, const uint16_t* norm_w, const Scalars& p,
                                uint16_t* xn_out, uint16_t* layer_input, float* pre_out,
                                float* post_out, float* comb_out, float* mixes, float* rstd,
                                hipStream_t stream) {
    return launch_w4_s<7168 / 256>(T, tile_tokens, x, X, post_prev, comb_prev, pre_lag, wprep,
                                   scale, base, norm_w, p, xn_out, layer_input, pre_out, post_out,
                                   comb_out, mixes, rstd, stream);
}

#elif defined(MHC_FUSED_MAXILP)

hipError_t launch_fused_7168(int T, const uint16_t* x, const uint16_t* X, const float* post_prev,
                             const float* comb_prev, const float* pre_lag, const void* wprep,
                             const float* scale, const float* base, const uint16_t* norm_w,
                             const Scalars& p, uint16_t* xn_out, uint16_t* layer_input,
                             float* pre_out, float* post_out, float* comb_out, float* mixes,
                             float* rstd, hipStream_t stream) {
    return launch_s<7168 / 512>(T, x, X, post_prev, comb_prev, pre_lag, wprep, scale, base, norm_w,
                                p, xn_out, layer_input, pre_out, post_out, comb_out, mixes, rstd,
                                stream);
}

#else  // the default scheduler: every other kernel and width, and the dispatch

bool fused_supported(int hidden) {
    switch (hidden) {
        case 1024: case 2048: case 4096: case 5120: case 6144: case 7168: case 8192:
            return true;
        default:
            return false;
    }
}

hipError_t launch_fused(int T, int hidden, const uint16_t* x, const uint16_t* X,
                        const float* post_prev, const float* comb_prev, const float* pre_lag,
                        const void* wprep, const float* scale, const float* base,
                        const uint16_t* norm_w, const Scalars& p, uint16_t* xn_out,
                        uint16_t* layer_input, float* pre_out, float* post_out, float* comb_out,
                        float* mixes, float* rstd, hipStream_t stream) {
#define MHC_FUSED_CASE(D)                                                                     \
    case D:                                                                                   \
        return launch_s<D / 512>(T, x, X, post_prev, comb_prev, pre_lag, wprep, scale, base,  \
                                 norm_w, p, xn_out, layer_input, pre_out, post_out, comb_out, \
                                 mixes, rstd, stream);
    switch (hidden) {
        MHC_FUSED_CASE(1024)
        MHC_FUSED_CASE(2048)
        MHC_FUSED_CASE(4096)
        MHC_FUSED_CASE(5120)
        MHC_FUSED_CASE(6144)
        case 7168:
            return launch_fused_7168(T, x, X, post_prev, comb_prev, pre_lag, wprep, scale, base,
                                     norm_w, p, xn_out, layer_input, pre_out, post_out, comb_out,
                                     mixes, rstd, stream);
        MHC_FUSED_CASE(8192)
        default:
            return hipErrorInvalidValue;
    }
#undef MHC_FUSED_CASE
}

hipError_t launch_fused_w4(int T, int tile_tokens, int hidden, const uint16_t* x,
                           const uint16_t* X, const float* post_prev, const float* comb_prev,
                           const float* pre_lag, const void* wprep, const float* scale,
                           const float* base, const uint16_t* norm_w, const Scalars& p,
                           uint16_t* xn_out, uint16_t* layer_input, float* pre_out,
                           float* post_out, float* comb_out, float* mixes, float* rstd,
                           hipStream_t stream) {
    if (tile_tokens < 1 || tile_tokens > kTileW4) return hipErrorInvalidValue;
#define MHC_W4_CASE(D)                                                                        \
    case D:                                                                                   \
        return launch_w4_s<D / 256>(T, tile_tokens, x, X, post_prev, comb_prev, pre_lag, wprep, scale, \
                                    base, norm_w, p, xn_out, layer_input, pre_out, post_out,  \
                                    comb_out, mixes, rstd, stream);
    switch (hidden) {
        MHC_W4_CASE(1024)
        MHC_W4_CASE(2048)
        MHC_W4_CASE(4096)
        MHC_W4_CASE(5120)
        MHC_W4_CASE(6144)
        case 7168:
            return launch_fused_w4_7168(T, tile_tokens, x, X, post_prev, comb_prev, pre_lag, wprep,
                                        scale, base, norm_w, p, xn_out, layer_input, pre_out,
                                        post_out, comb_out, mixes, rstd, stream);
        MHC_W4_CASE(8192)
        default:
            return hipErrorInvalidValue;
    }
#undef MHC_W4_CASE
}

hipError_t launch_fused_pre(int T, int hidden, const uint16_t* X, const void* wprep,
                            const float* scale, const float* base, const uint16_t* norm_w,
                            const Scalars& p, uint16_t* layer_input, float* pre_out,
                            float* post_out, float* comb_out, float* mixes, float* rstd,
                            bool tiles32, hipStream_t stream) {
#define MHC_FUSED_PRE_CASE(D)                                                                  \
    case D:                                                                                    \
        return tiles32 ? launch_pre_w4_s<D / 256>(T, X, wprep, scale, base, norm_w, p,         \
                                                  layer_input, pre_out, post_out, comb_out,    \
                                                  mixes, rstd, stream)                         \
                       : launch_pre_s<D / 512>(T, X, wprep, scale, base, norm_w, p,            \
                                               layer_input, pre_out, post_out, comb_out, mixes, \
                                               rstd, stream);
    switch (hidden) {
        MHC_FUSED_PRE_CASE(1024)
        MHC_FUSED_PRE_CASE(2048)
        MHC_FUSED_PRE_CASE(4096)
        MHC_FUSED_PRE_CASE(5120)
        MHC_FUSED_PRE_CASE(6144)
        MHC_FUSED_PRE_CASE(7168)
        MHC_FUSED_PRE_CASE(8192)
        default:
            return hipErrorInvalidValue;
    }
#undef MHC_FUSED_PRE_CASE
}

#endif  // the scheduler units

}  // namespace mhc
