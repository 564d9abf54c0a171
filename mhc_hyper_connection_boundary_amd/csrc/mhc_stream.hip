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

#include "mhc_device.h"
#include "mhc_launch.h"

namespace mhc {
namespace {

constexpr int kWavesS = 4;
constexpr int kTileS = kTile * kWavesS;  // 64 tokens per tile: one 16-token group per wave
constexpr int kCoherent = 16;            // buffer cache-policy bit sc1: device-coherent access
constexpr int kSpinLimit = 1 << 22;      // polls (with a short sleep) before a wait gives up

// Buffer resource over `bytes` bytes from base: accesses past the end read 0
// and write nothing.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ unsigned ld_dev(const unsigned* p) {
    return __hip_atomic_load(const_cast<unsigned*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
    return __uint_as_float(ld_dev(reinterpret_cast<const unsigned*>(p)));
}
__device__ __forceinline__ void st_dev(unsigned* p, unsigned v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(float* p, float v) {
    st_dev(reinterpret_cast<unsigned*>(p), __float_as_uint(v));
}
__device__ __forceinline__ unsigned add_dev(unsigned* p, unsigned v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

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

// Activations of one k-block for one lane: 8 hidden elements of the 4 streams
// of X and of x, for token tc.
struct ActS {
    uint4 X[4];
    uint4 x;
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

// Lane (n, g) of wave w: row 16w + n of the tile, 8 elements at column col.
// X stream j sits j rows further (soffset j * row_bytes).
template <bool NT>
__device__ __forceinline__ void load_act_s(ActS& a, const TileRows& r, unsigned row, unsigned row_bytes,
                                           unsigned col) {
    const unsigned vX = row * 4 * row_bytes + col * 2, vx = row * row_bytes + col * 2;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        a.X[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r.X, vX, j * row_bytes, NT ? 2 : 0));
    a.x = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r.x, vx, 0, NT ? 2 : 0));
}

// Spin (thread 0) until *p is nonzero; false if the bound ran out.
__device__ __forceinline__ bool wait_flag(const unsigned* p) {
    for (int n = 0; n < kSpinLimit; ++n) {
        if (ld_dev(p) != 0u) return true;
        __builtin_amdgcn_s_sleep(2);
    }
    return false;
}

template <int KB, bool NORM, bool NT>
__global__ __launch_bounds__(256) void k_stream(StreamArgs a) {
    static_assert(KB >= 2 && KB <= 16, "k-blocks per item");
    constexpr int TT = kTileS;
    constexpr int kCoefTok = 3;                     // coefficient tokens handled at once
    __shared__ uint4 frag[2][kFragsPerStep][64];    // a k-block's weight fragments, double buffered
    __shared__ float cred[kCoefTok][8][26];
    __shared__ float ctot[kCoefTok][26];
    __shared__ float srli[TT];
    __shared__ float prev_s[TT][24];                // the next tile's post[4], comb[16], pre[4]
    __shared__ int s_next, s_last;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
    const int S = a.slices, T = a.T, hidden = a.hidden;
    unsigned* const head = a.sync;
    unsigned* const exits = a.sync + 1;
    unsigned* const errors = a.sync + 2;  // waits that ran out (never cleared; zero unless a bug)
    unsigned* const arrive = a.sync + 3;
    unsigned* const flag = arrive + a.tiles;
    unsigned* const done = flag + a.tiles;

    // Fragment words of k-block kb that this thread stages: fragments 3*wave .. 3*wave+2.
    auto load_frag = [&](uint4 (&f)[3], int kb) {
        const uint4* src = a.wprep + (size_t)kb * kFragsPerStep * 64 + lane;
#pragma unroll
        for (int k = 0; k < 3; ++k) f[k] = src[(3 * wave + k) * 64];
    };
    auto store_frag = [&](const uint4 (&f)[3], int buf) {
#pragma unroll
        for (int k = 0; k < 3; ++k) frag[buf][3 * wave + k][lane] = f[k];
    };

    if (tid == 0) s_next = (int)add_dev(head, 1u);
    __syncthreads();
    int q = s_next;
    __syncthreads();
    unsigned ticket = 0;  // (thread 0) the queue position of the item after q
    if (tid == 0) ticket = add_dev(head, 1u);

    // Pipeline state: activations and coefficients of the next partial k-block.
    ActS cur;
    PrevCoef c;
    int buf = 0;
    bool primed = false;  // cur / c / frag[buf] hold (q, k-block 0)
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
        const int b = q / S, j = q - b * S;
        const bool has_partial = b < a.tiles;
        const int rt = b - a.lag;
        const bool has_rescale = rt >= 0 && rt < a.tiles;
        unsigned arrive_old = 0;
        int qn = a.items;  // the next item (known from the second-to-last k-block on)

        if (has_partial) {
            const unsigned row_bytes = (unsigned)hidden * 2, row = 16 * wave + n;
            const int t = b * TT + (int)row;
            const bool valid = t < T;
            const TileRows rows = tile_rows(a, b);
            if (!primed) {
                uint4 f[3];
                load_frag(f, j * KB);
                load_act_s<NT>(cur, rows, row, row_bytes, j * KB * kStep + g * 8);
                load_prev(c, a.post_prev, a.comb_prev, a.pre_lag, valid ? (size_t)t : (size_t)(T - 1));
                store_frag(f, buf);
                __syncthreads();
            }
            f32x4_t acc[3] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
            float ssq = 0.0f, ssq_li = 0.0f;
            TileRows rows_n = rows;
            float4 pc_st[2];  // the next tile's previous-layer coefficients, on their way to LDS
            bool next_partial = false;
#pragma unroll 1
            for (int kb = 0; kb < KB; ++kb) {
                const unsigned col = (j * KB + kb) * kStep + g * 8;
                // The next k-block: (q, kb + 1), or the first one of the next
                // item if that item has a partial phase.
                bool have_next = kb + 1 < KB;
                int next_kb = j * KB + kb + 1;
                unsigned next_col = col + kStep;
                if (kb + 1 == KB) {
                    qn = s_next;
                    next_partial = (unsigned)qn < (unsigned)a.items && qn / S < a.tiles;
                    const int bn = next_partial ? qn / S : 0;
                    if (next_partial) {
                        have_next = true;
                        next_kb = (qn - bn * S) * KB;
                        next_col = next_kb * kStep + g * 8;
                        rows_n = tile_rows(a, bn);
#pragma unroll
                        for (int k = 0; k < 2; ++k) {
                            const int e = tid + 256 * k;  // (token, float4) of the next tile
                            const int tok = min(bn * TT + e / 6, T - 1), part4 = e % 6;
                            const float* src = part4 == 0 ? a.post_prev + (size_t)tok * 4
                                             : part4 < 5 ? a.comb_prev + (size_t)tok * 16 + 4 * (part4 - 1)
                                                         : a.pre_lag + (size_t)tok * 4;
                            if (e < TT * 6) pc_st[k] = *reinterpret_cast<const float4*>(src);
                        }
                    }
                }
                uint4 fn[3];
                ActS nxt;
                if (have_next) {
                    load_frag(fn, next_kb);
                    load_act_s<NT>(nxt, kb + 1 < KB ? rows : rows_n, row, row_bytes, next_col);
                }
                uint4 A[kFragsPerStep];
#pragma unroll
                for (int i = 0; i < kFragsPerStep; ++i) A[i] = frag[buf][i][lane];
                uint4 Xn[4], li;
                update_collapse(cur.X, cur.x, c, Xn, li, ssq, ssq_li);
                const unsigned vX = row * 4 * row_bytes + col * 2, vx = row * row_bytes + col * 2;
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, Xn[s2]), rows.Xo, vX,
                                                           s2 * row_bytes, NT ? 2 : 0);
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, li), rows.li, vx, 0,
                                                       NORM ? kCoherent : 0);
                mfma_step(A, Xn, acc);
                if (have_next) store_frag(fn, buf ^ 1);
                if (kb + 2 == KB) {
                    if (tid == 0) s_next = (int)ticket;  // (the lookahead grab returned long ago)
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
            // prefetch, which the next k-block needs first anyway.)
            __builtin_amdgcn_s_waitcnt(0);
            if (next_partial) {
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const int e = tid + 256 * k;
                    if (e < TT * 6) *reinterpret_cast<float4*>(&prev_s[e / 6][4 * (e % 6)]) = pc_st[k];
                }
            }
            __syncthreads();
            if (tid == 0) arrive_old = add_dev(arrive + b, 1u);
            if (next_partial) {
                // this lane's token of the next tile: post[4], comb[16], pre[4]
                const float* v = prev_s[row];
#pragma unroll
                for (int k = 0; k < 4; ++k) c.post[k] = v[k];
#pragma unroll
                for (int k = 0; k < 16; ++k) c.comb[k] = v[4 + k];
#pragma unroll
                for (int k = 0; k < 4; ++k) c.pre[k] = v[20 + k];
            }
        } else {
            if (tid == 0) s_next = (int)ticket;
            __syncthreads();
            qn = s_next;
            primed = false;
        }

        if (has_rescale) {
            // ---- phase B: tile rt, slice j ----
            if (tid == 0) {
                if (!wait_flag(flag + rt)) add_dev(errors, 1u);
            }
            __syncthreads();
            if (NORM && tid < TT) srli[tid] = rt * TT + tid < T ? ld_dev(a.rli + rt * TT + tid) : 0.0f;
            __syncthreads();
            // Coefficient tokens of this item: j, j + S, ... of the tile.
            for (int k0 = j; k0 < TT; k0 += kCoefTok * S) {
                // thread p = (token kk, group grp, value v): slices grp, grp + 8, ...
                for (int p = tid; p < kCoefTok * 200; p += 256) {
                    const int kk = p / 200, r = p % 200, grp = r / 25, v = r % 25;
                    const int k = k0 + kk * S;
                    const int tt = rt * TT + k;
                    float sum = 0.0f;
                    if (k < TT && tt < T) {
                        const float* src = a.part + (size_t)tt * S * kPart + v;
                        for (int sl = grp; sl < S; sl += 8) sum += ld_dev(src + (size_t)sl * kPart);
                    }
                    cred[kk][grp][v] = sum;
                }
                __syncthreads();
                if (tid < kCoefTok * 25) {
                    const int kk = tid / 25, v = tid % 25;
                    float sum = 0.0f;
#pragma unroll
                    for (int grp = 0; grp < 8; ++grp) sum += cred[kk][grp][v];
                    ctot[kk][v] = sum;
                }
                __syncthreads();
                if (tid < kCoefTok * 16) {
                    const int kk = tid >> 4, l16 = tid & 15, i = tid & 3;
                    const int k = k0 + kk * S;
                    const int tt = rt * TT + k;
                    const CoefParams cp = load_coef_params(a.scale, a.base, i);
                    TokenCoef o;
                    pre_post(o, ctot[kk], i, hidden, cp, a.p);
                    const float cv = comb16(ctot[kk], l16, o.rstd, cp.s2, a.base[8 + l16], a.p);
                    if (k < TT && tt < T) {
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
            if (NORM) {
                // li of the slice for this wave's 16 tokens: 16 rows x 32*KB
                // elements.  kLpr lanes cover a row's slice (16 bytes each), a
                // load instruction covers kRpi rows.
                constexpr int kLpr = KB * kStep / 8, kRpi = 64 / kLpr, kLoads = 16 / kRpi;
                const int rows_r = min(TT, T - rt * TT);
                const auto li_rs = rsrc(a.layer_input + (size_t)rt * TT * hidden, (unsigned)(rows_r * hidden * 2));
                const int col = j * KB * kStep + (lane % kLpr) * 8;
                const uint4 nw = *reinterpret_cast<const uint4*>(a.norm_w + col);
                uint4 lv[kLoads];
#pragma unroll
                for (int i = 0; i < kLoads; ++i) {
                    const int row = 16 * wave + kRpi * i + lane / kLpr;
                    const unsigned off = (unsigned)((min(row, rows_r - 1) * hidden + col) * 2);
                    lv[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(li_rs, off, 0, kCoherent));
                }
#pragma unroll
                for (int i = 0; i < kLoads; ++i) {
                    const int row = 16 * wave + kRpi * i + lane / kLpr;
                    if (row < rows_r) {
                        const float r = srli[row];
                        uint4 out;
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            const uint32_t av = word(lv[i], k), bv = word(nw, k);
                            set_word(out, k, pack_bf16((bf_lo(av) * r) * bf_lo(bv), (bf_hi(av) * r) * bf_hi(bv)));
                        }
                        *reinterpret_cast<uint4*>(a.layer_input + ((size_t)rt * TT + row) * hidden + col) = out;
                    }
                }
            }
            __syncthreads();
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
                if (NORM && tid < TT && b * TT + tid < T) {
                    const size_t tt = (size_t)b * TT + tid;
                    const float* src = a.part + tt * S * kPart + 25;
                    float sum = 0.0f;
                    for (int sl = 0; sl < S; ++sl) sum += ld_dev(src + (size_t)sl * kPart);
                    st_dev(a.rli + tt, rsqrt_nr(sum * (1.0f / (float)hidden) + a.p.norm_eps));
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
        q = qn;
        if (tid == 0 && (unsigned)q < (unsigned)a.items) ticket = add_dev(head, 1u);
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
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_unit, k_stream<kStreamKb, true, true>,
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
        hipLaunchKernelGGL((k_stream<kStreamKb, true, true>), dim3(plan.grid), dim3(256), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((k_stream<kStreamKb, false, true>), dim3(plan.grid), dim3(256), 0,
                           stream, a);
    return hipGetLastError();
}

}  // namespace mhc
