// Streaming schedule of the shifted boundary: one persistent launch that runs
// the whole boundary for any token count.
//
// Work items are (tile of 64 tokens, slice of 32*KB hidden elements), taken in
// tile-major order from a queue (an atomic counter), so the items in flight at
// any moment cover whole rows of a few consecutive tiles: HBM serves that far
// better than the same bytes spread over every tile of the batch (a mover of
// the boundary's bytes: 5.3 TB/s persistent tile-major against 4.7 TB/s with
// one workgroup per tile over all of hidden).
//
// An item runs two phases:
//   A  the partial work of tile b, slice j: residual update, X' (stored),
//      lagged collapse li (stored into the layer-input buffer), sums of
//      squares and the projection on the matrix cores.  Wave w owns tokens
//      16w..16w+15 of the tile for every k-block of the slice; the four waves
//      share each k-block's weight fragments through LDS.  One partial record
//      per token and slice (24 mixes, ssq, ssq_li).  The last item of the tile
//      to finish computes the tile's rstd_li and raises the tile's flag.
//   B  the finishing work of tile r = b - lag, slice j: the coefficients
//      (pre, post, Sinkhorn comb) of tokens j, j + slices, ... of the tile from
//      the records summed in a fixed order, and the RMSNorm of li over the
//      slice.  Tiles past the last one run phase B only.
// Phase B waits for tile r's flag.  Every item of tile r has a smaller queue
// position than the item waiting for it, and phase A never waits, so every
// wait ends (whatever the number of resident workgroups); a spin bound guards
// it anyway.  With the lag, tile r has normally finished long before.
//
// Cross-workgroup data (records, li, rstd_li, flags) is written with
// device-coherent stores (sc1) and read with device-coherent loads, and a
// writer waits for its stores before it counts itself in; no cache-wide
// writeback or invalidate is needed (both cost tens to hundreds of
// microseconds on this part).  The counters return to zero at the end of
// every launch, so the workspace must hold zeros before the first call only.
#include <atomic>

#include "mhc_coherent.h"
#include "mhc_device.h"
#include "mhc_launch.h"

namespace mhc {
namespace {

constexpr int kWavesS = 4;
constexpr int kTileS = kTile * kWavesS;  // 64 tokens per tile: one 16-token group per wave

struct StreamArgs {
    int T, hidden, tiles, slices, lag, items;
    const uint16_t* x;
    const uint16_t* X;
    const float* post_prev;
    const float* comb_prev;
    const float* pre_lag;
    const uint4* wprep;
    const float* scale;
    const float* base;
    const uint16_t* norm_w;
    uint16_t* xn_out;
    uint16_t* layer_input;
    float* pre_out;
    float* post_out;
    float* comb_out;
    float* mixes_out;
    float* rstd_out;
    float* part;    // [T][slices][kPart] partial records
    float* rli;     // [T] rstd_li
    unsigned* sync; // queue head, exits, error count, then per tile: arrivals, flags, done
    Scalars p;
};

// Activations of one step (two k-blocks, h = 0, 1) for one lane: 8 hidden
// elements of the 4 streams of X and of x in each k-block.
struct Act2 {
    uint4 X[2][4];
    uint4 x[2];
};

// The six weight fragments a thread stages for one step (named members: an
// array here ends up in scratch memory).
struct Frag6 {
    uint4 f0, f1, f2, f3, f4, f5;
};

// The rows of one tile: X (4 per token), x, X' and the layer input, each a
// buffer resource that ends at the tile's last token, so accesses of lanes
// past the last token read 0 and write nothing.
struct TileRows {
    __amdgpu_buffer_rsrc_t X, x, Xo, li;
};

__device__ __forceinline__ TileRows tile_rows(const StreamArgs& s, int b) {
    const int rows = min(kTileS, s.T - b * kTileS);
    const size_t first = (size_t)b * kTileS * s.hidden;
    const unsigned row_bytes = (unsigned)s.hidden * 2;
    TileRows r;
    r.X = rsrc(s.X + 4 * first, 4 * rows * row_bytes);
    r.x = rsrc(s.x + first, rows * row_bytes);
    r.Xo = rsrc(s.xn_out + 4 * first, 4 * rows * row_bytes);
    r.li = rsrc(s.layer_input + first, rows * row_bytes);
    return r;
}

// Lane (n, g) of wave w: row 16w + n of the tile, 8 elements at column col
// and at col + 32 (the other half of the same 128-byte line, loaded right
// after it).  X stream j sits j rows further (soffset j * row_bytes).
__device__ __forceinline__ void load_act2(Act2& a, const TileRows& r, unsigned row, unsigned row_bytes,
                                          unsigned col) {
    const unsigned vX = row * 4 * row_bytes + col * 2, vx = row * row_bytes + col * 2;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            a.X[h][j] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(r.X, vX + h * kStep * 2, j * row_bytes, 0));
#pragma unroll
    for (int h = 0; h < 2; ++h)
        a.x[h] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r.x, vx + h * kStep * 2, 0, 0));
}


template <int KB, bool NORM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_stream(StreamArgs a) {
    MHC_POISON_LDS(0);
    static_assert(KB % 2 == 0 && KB >= 6 && KB <= 16, "k-blocks per item");
    constexpr int KS = KB / 2;                      // steps (pairs of k-blocks) per item
    constexpr int TT = kTileS;
    constexpr int kCoefTok = 3;                     // coefficient tokens handled at once
    constexpr unsigned kRec = kPart * 4;            // bytes per partial record
    __shared__ uint4 frag[2][2 * kFragsPerStep][64];  // a step's weight fragments, double buffered
    __shared__ float cred[kCoefTok][8][26];
    __shared__ float ctot[kCoefTok][26];
    __shared__ float prev_s[2][TT][24];             // this and the next tile's post[4], comb[16], pre[4]
    __shared__ int s_next, s_last;

    const int tid = threadIdx.x;
    const int S = a.slices, T = a.T, hidden = a.hidden;
    unsigned* const head = a.sync;
    unsigned* const exits = a.sync + 1;
    unsigned* const errors = a.sync + 2;  // waits that ran out (never cleared; zero unless a bug)
    unsigned* const arrive = a.sync + 3;
    unsigned* const flag = arrive + a.tiles;
    unsigned* const done = flag + a.tiles;

    if (tid == 0) s_next = (int)add_dev(head, 1u);
    __syncthreads();
    int q = __builtin_amdgcn_readfirstlane(s_next);
    __syncthreads();
    unsigned ticket = 0;  // (thread 0) the queue position of the item after q

    // Pipeline state: activations of the next partial step.
    Act2 cur;
    int buf = 0, pb = 0;
    bool primed = false;  // cur / frag[buf] / prev_s[pb] hold (q, step 0)
    // (thread 0) the finisher counts of this item's and the previous item's
    // phase B: the tile and the value the done counter had.
    constexpr unsigned kNone = 0xffffffffu;
    unsigned this_rt = kNone, this_done = 0, pending_rt = kNone, pending_done = 0;
    auto clear_if_last = [&](unsigned rt_, unsigned old) {
        if (rt_ != kNone && old == (unsigned)S - 1u) {
            st_dev(arrive + rt_, 0u);
            st_dev(flag + rt_, 0u);
            st_dev(done + rt_, 0u);
        }
    };

    // (positions are compared as unsigned: whatever a counter holds, an item
    // outside [0, items) ends the loop and addresses nothing)
    while ((unsigned)q < (unsigned)a.items) {
        // Lane indexes and everything derived from them are computed anew for
        // each item: hoisted out of the loop they would hold registers
        // throughout (and spill).
        int tl = threadIdx.x;
        asm volatile("" : "+v"(tl));
        const int lane = tl & 63, n = lane & 15, g = lane >> 4;
        const int wave = __builtin_amdgcn_readfirstlane(tl >> 6);
        // Fragment words of step st (k-blocks 2 st, 2 st + 1: 24 fragments) that
        // this thread stages: fragments 6*wave .. 6*wave+5.
        auto load_frag = [&](int st) -> Frag6 {
            const uint4* src = a.wprep + (size_t)st * 2 * kFragsPerStep * 64 + 6 * wave * 64 + lane;
            return Frag6{src[0], src[64], src[128], src[192], src[256], src[320]};
        };
        auto store_frag = [&](const Frag6& f, int fbuf) {
            uint4* dst = &frag[fbuf][6 * wave][lane];
            dst[0] = f.f0;
            dst[64] = f.f1;
            dst[128] = f.f2;
            dst[192] = f.f3;
            dst[256] = f.f4;
            dst[320] = f.f5;
        };

        // The previous-layer coefficients of the tile from token tok0 on go to
        // prev_s: element e = tl + 256 k (k = 0, 1; e < 6 TT) is float4 e % 6 of
        // token e / 6 (post, comb rows 0-3, pre).  The loads are unconditional
        // (clamped indexes), so both are in flight together.
        auto pc_load = [&](int k, int tok0) -> float4 {
            const int e = min(tl + 256 * k, TT * 6 - 1);
            const int tok = min(tok0 + e / 6, T - 1), part4 = e % 6;
            const float* src = part4 == 0 ? a.post_prev + (size_t)tok * 4
                             : part4 < 5 ? a.comb_prev + (size_t)tok * 16 + 4 * (part4 - 1)
                                         : a.pre_lag + (size_t)tok * 4;
            return *reinterpret_cast<const float4*>(src);
        };
        auto pc_store = [&](float4 v0, float4 v1, int pbuf) {
            static_assert(256 < TT * 6 && TT * 6 <= 512, "two float4 per thread");
            *reinterpret_cast<float4*>(&prev_s[pbuf][tl / 6][4 * (tl % 6)]) = v0;
            const int e = tl + 256;
            if (e < TT * 6) *reinterpret_cast<float4*>(&prev_s[pbuf][e / 6][4 * (e % 6)]) = v1;
        };

        const int b = q / S, j = q - b * S;
        const bool has_partial = b < a.tiles;
        const int rt = b - a.lag;
        const bool has_rescale = rt >= 0 && rt < a.tiles;
        unsigned arrive_old = 0;
        int qn = a.items;  // the next item (known in the last step)
        // The next item is taken while this one runs: in its second step
        // (it is needed in the last), or at once if it has no partial phase.  Taken any earlier, in particular before workgroups
        // still starting up have taken their first items, it would hold back
        // an item that another workgroup could run.
        if (tid == 0 && !has_partial) ticket = add_dev(head, 1u);

        if (has_partial) {
            const unsigned row_bytes = (unsigned)hidden * 2, row = 16 * wave + n;
            const int t = b * TT + (int)row;
            const bool valid = t < T;
            const TileRows rows = tile_rows(a, b);
            if (!primed) {
                const Frag6 f = load_frag(j * KS);
                const float4 pc0 = pc_load(0, b * TT), pc1 = pc_load(1, b * TT);
                load_act2(cur, rows, row, row_bytes, j * KB * kStep + g * 8);
                store_frag(f, buf);
                pc_store(pc0, pc1, pb);
                __syncthreads();
            }
            f32x4_t acc[3] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
            float ssq = 0.0f, ssq_li = 0.0f;
            TileRows rows_n = rows;
            float4 pcn0, pcn1;  // the next tile's previous-layer coefficients, on their way to LDS
            bool next_partial = false;
            int jn = 0;         // the next item's slice
#pragma unroll 1
            for (int st = 0; st < KS; ++st) {
                const unsigned col = (j * KB + 2 * st) * kStep + g * 8;  // the step's first k-block
                if (st == 1 && tid == 0) ticket = add_dev(head, 1u);
                if (st + 1 == KS) {
                    // The next item: its first step follows this item's last
                    // one in the pipeline if it has a partial phase.
                    qn = __builtin_amdgcn_readfirstlane(s_next);
                    next_partial = (unsigned)qn < (unsigned)a.items && qn / S < a.tiles;
                    if (next_partial) {
                        const int bn = qn / S;
                        jn = qn - bn * S;
                        rows_n = tile_rows(a, bn);
                        pcn0 = pc_load(0, bn * TT);
                        pcn1 = pc_load(1, bn * TT);
                    }
                }
                // The next step's weight fragments and activations.
                const bool have_next = st + 1 < KS || next_partial;
                const int next_st = st + 1 < KS ? j * KS + st + 1 : jn * KS;  // (a step of the whole row)
                // (the fragment loads are unconditional, so that they stay in registers)
                const Frag6 fn = load_frag(have_next ? next_st : 0);
                Act2 nxt;
                if (have_next)
                    load_act2(nxt, st + 1 < KS ? rows : rows_n, row, row_bytes, next_st * 2 * kStep + g * 8);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    // (the scheduler keeps the two k-blocks apart: interleaved,
                    // they would need more registers than two waves per SIMD have)
                    __builtin_amdgcn_sched_barrier(0);
                    // this lane's token: post[4], comb[16], pre[4] (read for
                    // each k-block: registers are scarcer than LDS bandwidth)
                    PrevCoef c;
                    const float* v = prev_s[pb][row];
#pragma unroll
                    for (int k = 0; k < 4; ++k) c.post[k] = v[k];
#pragma unroll
                    for (int k = 0; k < 16; ++k) c.comb[k] = v[4 + k];
#pragma unroll
                    for (int k = 0; k < 4; ++k) c.pre[k] = v[20 + k];
                    uint4 Xn[4], li;
                    update_collapse(cur.X[h], cur.x[h], c, Xn, li, ssq, ssq_li);
                    const unsigned ch = col + h * kStep;
                    const unsigned vX = row * 4 * row_bytes + ch * 2, vx = row * row_bytes + ch * 2;
#pragma unroll
                    for (int s2 = 0; s2 < 4; ++s2)
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, Xn[s2]), rows.Xo, vX,
                                                               s2 * row_bytes, 0);
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, li), rows.li, vx, 0,
                                                           NORM ? kCoherent : 0);
                    // the projection, one stream's three A tiles at a time
#pragma unroll
                    for (int s2 = 0; s2 < 4; ++s2) {
                        const bf16x8_t bx = __builtin_bit_cast(bf16x8_t, Xn[s2]);
#pragma unroll
                        for (int m = 0; m < 3; ++m)
                            acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8_t, frag[buf][kFragsPerStep * h + 3 * s2 + m][lane]), bx,
                                acc[m], 0, 0, 0);
                    }
                }
                if (have_next) store_frag(fn, buf ^ 1);
                if (st + 2 == KS) {
                    if (tid == 0) s_next = (int)ticket;  // (the grab of step 1 returned long ago)
                }
                __syncthreads();
                buf ^= 1;
                if (have_next) cur = nxt;
            }
            primed = next_partial;
            // Records of this wave's 16 tokens: lane (n, g) holds mixes
            // 8m + 2g + jj; the sums of squares are added over g in order.
            {
                const float a1 = __shfl(ssq, n + 16), a2 = __shfl(ssq, n + 32), a3 = __shfl(ssq, n + 48);
                const float b1 = __shfl(ssq_li, n + 16), b2 = __shfl(ssq_li, n + 32),
                            b3 = __shfl(ssq_li, n + 48);
                if (valid) {
                    float* rec = a.part + ((size_t)t * S + j) * kPart;
#pragma unroll
                    for (int m = 0; m < 3; ++m)
#pragma unroll
                        for (int jj = 0; jj < 2; ++jj) st_dev(rec + 8 * m + 2 * g + jj, mix_of(acc, m, jj));
                    if (g == 0) {
                        st_dev(rec + 24, ((ssq + a1) + a2) + a3);
                        st_dev(rec + 25, ((ssq_li + b1) + b2) + b3);
                    }
                }
            }
            // Everything this thread wrote (records, li) has landed before the
            // tile counts this item in.  (This also waits for the next item's
            // first two k-blocks, requested one and two k-blocks ago.)
            __builtin_amdgcn_s_waitcnt(0);
            if (next_partial) {
                pb ^= 1;
                pc_store(pcn0, pcn1, pb);
            }
            __syncthreads();
            if (tid == 0) arrive_old = add_dev(arrive + b, 1u);
        } else {
            primed = false;
        }

        if (has_rescale) {
            // ---- phase B: tile rt, slice j ----
            if (tid == 0) {
                if (!wait_flag(flag + rt)) add_dev(errors, 1u);
            }
            __syncthreads();
            // The loads of the phase go out together: li of the slice with
            // its rstd_li, then the records of the first coefficient round.
            const int rows_r = min(TT, T - rt * TT);
            // li of the slice for this wave's 16 tokens: 16 rows x 32*KB
            // elements.  kLpr lanes cover a row's slice (16 bytes each), a
            // load instruction covers kRpi rows.
            constexpr int kLpr = KB * kStep / 8, kRpi = 64 / kLpr, kLoads = 16 / kRpi;
            const int lcol = j * KB * kStep + (lane % kLpr) * 8;
            uint4 lv[kLoads], nw;
            float rl[kLoads];
            if (NORM) {
                const auto li_rs = rsrc(a.layer_input + (size_t)rt * TT * hidden, (unsigned)(rows_r * hidden * 2));
                const auto rli_rs = rsrc(a.rli + (size_t)rt * TT, (unsigned)rows_r * 4);
                nw = *reinterpret_cast<const uint4*>(a.norm_w + lcol);
#pragma unroll
                for (int i = 0; i < kLoads; ++i) {
                    const int row = 16 * wave + kRpi * i + lane / kLpr;
                    const unsigned off = (unsigned)((min(row, rows_r - 1) * hidden + lcol) * 2);
                    lv[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(li_rs, off, 0, kCoherent));
                    rl[i] = ld_coh(rli_rs, (unsigned)row * 4);
                }
            }
            // Coefficient tokens of this item: j, j + S, ... of the tile, in
            // rounds of kCoefTok (j < S <= TT: at least one round).  Thread
            // p = tid + 256 it = (token kk, group grp, value v) adds slices grp,
            // grp + 8, ... in order, four slices per load batch.
            const auto rec_rs = rsrc(a.part + (size_t)rt * TT * S * kPart, (unsigned)rows_r * S * kRec);
            // coefficient constants of this thread's place in a quad / DPP row
            const CoefParams cpar = load_coef_params(a.scale, a.base, tl & 3);
            const float bcomb16 = a.base[8 + (tl & 15)];
            unsigned roff[3];
            int rgrp[3];
            float rval[3][4];
            auto rec_site = [&](int k0, int it, unsigned& off, int& grp_out) {
                const int p = tl + 256 * it, kk = p / 200, r = p - 200 * kk, grp = r / 25, v = r - 25 * grp;
                const int k = k0 + kk * S;
                grp_out = grp;
                off = p < kCoefTok * 200 && k < rows_r ? ((unsigned)(k * S + grp) * kPart + v) * 4 : kOob;
            };
#pragma unroll
            for (int it = 0; it < 3; ++it) {
                rec_site(j, it, roff[it], rgrp[it]);
#pragma unroll
                for (int u = 0; u < 4; ++u) rval[it][u] = ld_coh(rec_rs, roff[it] + (unsigned)(8 * u) * kRec);
            }
            if (NORM) {
                // the normalised layer input of the slice
#pragma unroll
                for (int i = 0; i < kLoads; ++i) {
                    const int row = 16 * wave + kRpi * i + lane / kLpr;
                    if (row < rows_r) {
                        const float r = rl[i];
                        uint4 out;
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            const uint32_t av = word(lv[i], k), bv = word(nw, k);
                            set_word(out, k, pack_bf16((bf_lo(av) * r) * bf_lo(bv), (bf_hi(av) * r) * bf_hi(bv)));
                        }
                        *reinterpret_cast<uint4*>(a.layer_input + ((size_t)rt * TT + row) * hidden + lcol) = out;
                    }
                }
            }
            for (int k0 = j; k0 < TT; k0 += kCoefTok * S) {
                if (k0 != j) {
#pragma unroll
                    for (int it = 0; it < 3; ++it) {
                        rec_site(k0, it, roff[it], rgrp[it]);
#pragma unroll
                        for (int u = 0; u < 4; ++u) rval[it][u] = ld_coh(rec_rs, roff[it] + (unsigned)(8 * u) * kRec);
                    }
                }
                float sum[3] = {0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int it = 0; it < 3; ++it)
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        if (rgrp[it] + 8 * u < S) sum[it] += rval[it][u];
                for (int s0 = 32; s0 < S; s0 += 32) {
                    float val[3][4];
#pragma unroll
                    for (int it = 0; it < 3; ++it)
#pragma unroll
                        for (int u = 0; u < 4; ++u) val[it][u] = ld_coh(rec_rs, roff[it] + (unsigned)(s0 + 8 * u) * kRec);
#pragma unroll
                    for (int it = 0; it < 3; ++it)
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            if (rgrp[it] + s0 + 8 * u < S) sum[it] += val[it][u];
                }
#pragma unroll
                for (int it = 0; it < 3; ++it) {
                    const int p = tl + 256 * it, kk = p / 200, r = p - 200 * kk, grp = r / 25, v = r - 25 * grp;
                    if (p < kCoefTok * 200) cred[kk][grp][v] = sum[it];
                }
                __syncthreads();
                if (tid < kCoefTok * 25) {
                    const int kk = tl / 25, v = tl % 25;
                    float s = 0.0f;
#pragma unroll
                    for (int grp = 0; grp < 8; ++grp) s += cred[kk][grp][v];
                    ctot[kk][v] = s;
                }
                __syncthreads();
                if (tid < kCoefTok * 16) {
                    const int kk = tl >> 4, l16 = tl & 15, i = tl & 3;
                    const int k = k0 + kk * S;
                    const int tt = rt * TT + k;
                    TokenCoef o;
                    pre_post(o, ctot[kk], i, hidden, cpar, a.p);
                    const float cv = comb16(ctot[kk], l16, o.rstd, cpar.s2, bcomb16, a.p);
                    if (k < rows_r) {
                        a.comb_out[(size_t)tt * 16 + l16] = cv;
                        if (l16 < 4) {
                            a.pre_out[(size_t)tt * 4 + i] = o.pre;
                            a.post_out[(size_t)tt * 4 + i] = o.post;
                            if (a.mixes_out)
                                for (int kq = 0; kq < 6; ++kq)
                                    a.mixes_out[(size_t)tt * 24 + 6 * i + kq] = ctot[kk][6 * i + kq];
                            if (a.rstd_out && i == 0) a.rstd_out[tt] = o.rstd;
                        }
                    }
                }
                __syncthreads();
            }
            if (tid == 0) {
                // (its result is looked at one item later, when it has long returned)
                this_done = add_dev(done + rt, 1u);
                this_rt = (unsigned)rt;
            }
        }

        if (has_partial) {
            // The last item of tile b to finish: rstd_li of its tokens, then the flag.
            if (tid == 0) s_last = arrive_old == (unsigned)S - 1u;
            __syncthreads();
            if (s_last) {
                if (NORM) {
                    // Four threads per token: thread (tok, part) adds slices
                    // part, part + 4, ... in order, then the four sums are
                    // added in order.  Rows past the batch read 0.
                    const int tok = tl >> 2, part = tl & 3;
                    const int rows_b = min(TT, T - b * TT);
                    const auto rs = rsrc(a.part + (size_t)b * TT * S * kPart, (unsigned)rows_b * S * kRec);
                    const unsigned off = ((unsigned)(tok * S + part) * kPart + 25) * 4;
                    float sum = 0.0f;
                    for (int s0 = 0; s0 < S; s0 += 32) {
                        float v[8];
#pragma unroll
                        for (int u = 0; u < 8; ++u) v[u] = ld_coh(rs, off + (unsigned)(s0 + 4 * u) * kRec);
#pragma unroll
                        for (int u = 0; u < 8; ++u)
                            if (part + s0 + 4 * u < S) sum += v[u];
                    }
                    const int q0 = lane & ~3;
                    const float tot = ((__shfl(sum, q0) + __shfl(sum, q0 + 1)) + __shfl(sum, q0 + 2)) + __shfl(sum, q0 + 3);
                    if (part == 0 && tok < rows_b)
                        st_dev(a.rli + (size_t)b * TT + tok, rsqrt_nr(tot * (1.0f / (float)hidden) + a.p.norm_eps));
                }
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
                if (tid == 0) st_dev(flag + b, 1u);
            }
        }
        // The previous item's finishing: the last of a tile's S finishers
        // clears the tile's counters (nothing reads them again in this launch).
        if (tid == 0) {
            clear_if_last(pending_rt, pending_done);
            pending_rt = this_rt;
            pending_done = this_done;
            this_rt = kNone;
        }
        if (!has_partial) {
            if (tid == 0) s_next = (int)ticket;
            __syncthreads();
            qn = __builtin_amdgcn_readfirstlane(s_next);
        }
        q = qn;
    }
    // Every workgroup ends here; the last one clears the queue.
    if (tid == 0) {
        clear_if_last(pending_rt, pending_done);
        if (add_dev(exits, 1u) == gridDim.x - 1u) {
            st_dev(head, 0u);
            st_dev(exits, 0u);
        }
    }
}

}  // namespace

}  // namespace mhc

namespace mhc {

namespace {

constexpr int kStreamKb = 8;          // k-blocks per item: 256-element slices
constexpr int kMaxDevicesS = 64;

int stream_current_device() {
    int dev = 0;
    return hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevicesS ? dev : -1;
}

// Workgroups of k_stream the current device holds at once (0 if unknown).
int stream_resident_workgroups() {
    static std::atomic<int> cache[kMaxDevicesS];  // 0: not asked yet; -1: unknown
    const int dev = stream_current_device();
    if (dev < 0) return 0;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int units = 0, per_unit = 0;
        const bool ok =
            hipDeviceGetAttribute(&units, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_unit, k_stream<kStreamKb, true>,
                                                         256, 0) == hipSuccess;
        v = ok && units > 0 && per_unit > 0 ? units * per_unit : -1;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v > 0 ? v : 0;
}

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

}  // namespace

StreamPlan stream_plan(int T, int hidden) {
    StreamPlan p;
    p.kb = kStreamKb;
    p.slices = hidden / (kStreamKb * kStep);
    p.tiles = (T + kTileS - 1) / kTileS;
    int resident = stream_resident_workgroups();
    if (resident <= 0) resident = 512;
    // Tile r is finished by the items of tile r + lag: about two rounds of
    // resident workgroups later, so that it has normally finished by then.
    const int lag = (2 * resident + p.slices - 1) / p.slices + 1;
    p.lag = lag < p.tiles ? lag : p.tiles;
    p.items = (p.tiles + p.lag) * p.slices;
    p.grid = resident < p.items ? resident : p.items;
    p.sync_words = 3 + 3 * p.tiles;
    return p;
}

size_t stream_data_bytes(int T, int hidden) {
    const StreamPlan p = stream_plan(T, hidden);
    return align256((size_t)T * 4) + (size_t)T * p.slices * kPart * sizeof(float);
}

hipError_t launch_stream(const StreamPlan& plan, int T, int hidden, const uint16_t* x,
                         const uint16_t* X, const float* post_prev, const float* comb_prev,
                         const float* pre_lag, const void* wprep, const float* scale,
                         const float* base, const uint16_t* norm_w, const Scalars& p,
                         uint16_t* xn_out, uint16_t* layer_input, float* pre_out,
                         float* post_out, float* comb_out, float* mixes, float* rstd,
                         void* workspace, hipStream_t stream) {
    char* ws = static_cast<char*>(workspace);
    StreamArgs a;
    a.T = T;
    a.hidden = hidden;
    a.tiles = plan.tiles;
    a.slices = plan.slices;
    a.lag = plan.lag;
    a.items = plan.items;
    a.x = x;
    a.X = X;
    a.post_prev = post_prev;
    a.comb_prev = comb_prev;
    a.pre_lag = pre_lag;
    a.wprep = reinterpret_cast<const uint4*>(wprep);
    a.scale = scale;
    a.base = base;
    a.norm_w = norm_w;
    a.xn_out = xn_out;
    a.layer_input = layer_input;
    a.pre_out = pre_out;
    a.post_out = post_out;
    a.comb_out = comb_out;
    a.mixes_out = mixes;
    a.rstd_out = rstd;
    a.sync = reinterpret_cast<unsigned*>(ws);
    a.rli = reinterpret_cast<float*>(ws + kCounterBytes);
    a.part = reinterpret_cast<float*>(ws + kCounterBytes + align256((size_t)T * 4));
    a.p = p;
    if (norm_w)
        hipLaunchKernelGGL((k_stream<kStreamKb, true>), dim3(plan.grid), dim3(256), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((k_stream<kStreamKb, false>), dim3(plan.grid), dim3(256), 0,
                           stream, a);
    return hipGetLastError();
}

}  // namespace mhc
