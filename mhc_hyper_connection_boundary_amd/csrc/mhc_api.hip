// C ABI of the mHC boundary library: host-side validation, scheduling and
// launches.  Validation is pure host code that makes no HIP call, so every
// refusal happens before anything is enqueued.
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <cstdlib>

#include "mhc.h"
#include "mhc_device.h"
#include "mhc_launch.h"

namespace mhc {

namespace {

constexpr long kTargetWaves = 2048;  // waves of k_partial work to aim for
constexpr int kFinishTarget = 2048;  // k_finish workgroups to aim for
constexpr int kFusedMinTokens = 3072; // automatic schedule, compute units unknown: fused from here
constexpr int kTwoGroupStepsShifted = 8;  // split boundary: two token groups per wave from here
constexpr int kTwoGroupStepsPre = 4;      // split pre: two groups from here (fewer registers)
constexpr int kFourGroupStepsPre = 16;    // split pre: four groups from here
constexpr int kRoundCost = 2;             // split grid: fixed cost of a round of workgroups, in steps
constexpr int kStreamMinTokens = 1 << 30; // split: the streaming plan from this many tokens (off:
                                          // measured slower than the round plan at every size)
constexpr int kStreamGroupsShifted = 2;   // streaming plan: 16-token groups per wave, boundary
constexpr int kStreamGroupsPre = 4;       // streaming plan: 16-token groups per wave, pre
constexpr int kStreamStepsPerWave = 2;    // streaming plan: 32-element steps per wave and slice
constexpr int kStreamFinishWidth = 1024;  // streaming plan: hidden elements per finishing workgroup
constexpr bool kStreamNontemporal = true; // streaming plan: nontemporal residual streams
constexpr int kW4MinTileTokens = 18;  // automatic schedule: balanced 4-wave tiles of at least this
constexpr int kW4MinTileTokens2 = 28; // ... and of at least this over two or more rounds
constexpr int kW4MinTokens = 8192;    // fused schedule: 32-token tiles on 4 waves from here

int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

bool shape_ok(int hidden) {
    return hidden >= MHC_MIN_HIDDEN && hidden <= MHC_MAX_HIDDEN && hidden % 256 == 0;
}

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
    const void* p;
    size_t bytes;
};

bool overlap(const Span& a, const Span& b) {
    if (!a.p || !b.p || !a.bytes || !b.bytes) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Each output must be disjoint from every other output and every input.
bool any_alias(const Span* outs, int n_out, const Span* ins, int n_in) {
    for (int i = 0; i < n_out; ++i) {
        for (int j = i + 1; j < n_out; ++j)
            if (overlap(outs[i], outs[j])) return true;
        for (int j = 0; j < n_in; ++j)
            if (overlap(outs[i], ins[j])) return true;
    }
    return false;
}

mhc_status check_params(const mhc_params* p) {
    if (!p) return MHC_ERR_INVALID_ARGUMENT;
    if (p->sinkhorn_iters < 1) return MHC_ERR_INVALID_ARGUMENT;
    if (!(p->rms_eps >= 0.f) || !(p->pre_eps >= 0.f) || !(p->sinkhorn_eps >= 0.f) ||
        !(p->norm_eps >= 0.f) || !(p->post_mult == p->post_mult))
        return MHC_ERR_INVALID_ARGUMENT;
    if (p->schedule < MHC_SCHEDULE_AUTO || p->schedule > MHC_SCHEDULE_ONEPASS)
        return MHC_ERR_INVALID_ARGUMENT;
    return MHC_OK;
}

// Which kernels run mhc_boundary.  FUSED is honoured (the caller gets
// UNSUPPORTED_SHAPE where the width has no fused kernel): 16-token tiles below
// kW4MinTokens, 32-token tiles from there.  AUTO, from the compute-unit count
// (one fused workgroup per CU):
//   the split schedule while 16-token tiles would fill less than 5/8 of one
//   round of CUs (T < 2560 on 256 CUs);
//   4-wave tiles of the balanced size ceil(T / (rounds x units)) (at most 32
//   tokens) where that is at least kW4MinTileTokens in one round, or at least
//   kW4MinTileTokens2 in more;
//   16-token tiles otherwise, over as many rounds as they take.
// Measured cold (us; split / 16-token / balanced 4-wave tiles): d=7168 T=2560
// 126 / 115 / 160, T=4096 180 / 137 / 173, T=4608 202 / 228 / 177, T=6144
// 267 / 240 / 201, T=8192 348 / 268 / 247, T=9216 410 / 361 / 342, T=12288
// 519 / 394 / 396, T=16384 694 / 524 / 513; d=4096 T=4096 125 / 77 / 102,
// T=4608 131 / 122 / 101, T=8192 224 / 148 / 134, T=9216 235 / 189 / 192,
// T=12288 346 / 216 / 215, T=16384 459 / 288 / 258; d=1024 T=4608 44 / 38 /
// 36, T=8192 64 / 48 / 42, T=9216 80 / 57 / 68, T=16384 114 / 91 / 76;
// d=2048, 5120, 6144 and 8192 alike.  Two rounds of 18- or 24-token tiles
// are level with or behind the 16-token tiles except at d >= 7168.  Where the
// compute-unit count is unknown, AUTO falls back to 16-token tiles from
// kFusedMinTokens and 32-token tiles from kW4MinTokens.
enum class BoundaryPath { Split, Fused16, Fused32, Stream };
struct BoundaryChoice {
    BoundaryPath path;
    int tile_tokens;  // Fused32: tokens per tile (at most 32)
};

BoundaryChoice boundary_path(int schedule, int tokens, int hidden) {
    if (schedule == MHC_SCHEDULE_STREAM) return {BoundaryPath::Stream, 0};
    if (schedule == MHC_SCHEDULE_FUSED)
        return tokens >= kW4MinTokens ? BoundaryChoice{BoundaryPath::Fused32, 32}
                                      : BoundaryChoice{BoundaryPath::Fused16, 16};
    if (schedule != MHC_SCHEDULE_AUTO || !fused_supported(hidden)) return {BoundaryPath::Split, 0};
    const long units = device_compute_units();
    if (units <= 0) {
        if (tokens < kFusedMinTokens) return {BoundaryPath::Split, 0};
        return tokens >= kW4MinTokens ? BoundaryChoice{BoundaryPath::Fused32, 32}
                                      : BoundaryChoice{BoundaryPath::Fused16, 16};
    }
    const long tiles16 = ceil_div(tokens, 16);
    if (8 * tiles16 < 5 * units) return {BoundaryPath::Split, 0};
    const long rounds = (ceil_div(tokens, 32) + units - 1) / units;
    const int balanced = (int)ceil_div(tokens, (int)(rounds * units));
    if (balanced >= (rounds == 1 ? kW4MinTileTokens : kW4MinTileTokens2))
        return {BoundaryPath::Fused32, balanced};
    return {BoundaryPath::Fused16, 16};
}

// The non-shifted pre reads X twice on either schedule, and its split runs
// faster at every size measured (d=7168, T=8192: 227 against 259 us with
// RMSNorm), so AUTO keeps it split.

Scalars scalars(const mhc_params* p) {
    Scalars s;
    s.rms_eps = p->rms_eps;
    s.pre_eps = p->pre_eps;
    s.post_mult = p->post_mult;
    s.sinkhorn_eps = p->sinkhorn_eps;
    s.sinkhorn_iters = p->sinkhorn_iters;
    s.norm_eps = p->norm_eps;
    return s;
}

}  // namespace

SplitPlan split_plan(int T, int hidden, bool invariant, bool shifted) {
    SplitPlan plan;
    const int nsteps = hidden / kStep;
    const int tiles = ceil_div(T, kTile);
    const int max_spw = ceil_div(nsteps, 4);
    plan.stream = false;
    if (!invariant && T >= kStreamMinTokens) {
        // Streaming plan for large batches: 32-token tiles (64 for the pre,
        // whose kernel reads only X) by 256-element slices, in tile-major
        // order, with nontemporal hints on the residual streams.  Measured as
        // a mover of the boundary's bytes: 5.6 TB/s in this shape against
        // 4.9 TB/s for one workgroup per tile over all of hidden.
        plan.groups = shifted ? kStreamGroupsShifted : kStreamGroupsPre;
        plan.steps_per_wave = std::min(kStreamStepsPerWave, max_spw);
        plan.slices = ceil_div(nsteps, 4 * plan.steps_per_wave);
        plan.finish_width = std::min(hidden, kStreamFinishWidth);
        plan.finish_slices = ceil_div(hidden, plan.finish_width);
        plan.stream = kStreamNontemporal;
        return plan;
    }
    // Batch-invariant: one step per wave whatever T is, so every sum of a token
    // has the same order for every batch.  Otherwise about kTargetWaves waves.
    int spw = invariant ? 1 : (int)std::max<long>(1, (long)tiles * nsteps / kTargetWaves);
    spw = std::min(spw, max_spw);
    plan.groups = 1;
    if (!invariant) {
        // Two token groups (four for the pre, whose kernel has the registers)
        // share each fragment load once there are enough steps per wave.  The
        // steps per wave are then chosen so the grid fills whole rounds of
        // slots: the least rounds x (steps per wave + a fixed cost of
        // kRoundCost steps per round).  While the finest split fits one round
        // this keeps one step per wave, as INVARIANT does.  The boundary's
        // slots are the workgroups the device holds at once; the pre's are the
        // compute units (one workgroup each), which measured faster there than
        // filling every resident slot.
        plan.groups = spw >= (shifted ? kTwoGroupStepsShifted : kTwoGroupStepsPre) ? 2 : 1;
        if (!shifted && spw >= kFourGroupStepsPre) plan.groups = 4;
        const long resident = shifted ? partial_resident_workgroups(plan.groups)
                                      : device_compute_units();
        if (resident > 0) {
            const long group_tiles = ceil_div(T, kTile * plan.groups);
            long best = -1;
            // (the pre's four-group kernel takes whole 64-element steps: an even
            // number of 32-element steps per wave)
            const bool even = !shifted && plan.groups == 4;
            for (int s = 1; s <= max_spw; ++s) {
                int w = ceil_div(nsteps, 4 * s);
                if (even) w += w & 1;
                const long rounds = (group_tiles * ceil_div(nsteps, 4 * w) + resident - 1) / resident;
                const long cost = rounds * (w + kRoundCost);
                if (best < 0 || cost < best) {
                    best = cost;
                    spw = w;
                }
            }
        }
    }
    // INVARIANT from 64 tiles: two token groups share each fragment load. A
    // token's sums have the same order for any number of groups, so the bits
    // still do not depend on T (d=7168, cold: pre T=2048 65.5 -> 62.6 us,
    // T=8192 281 -> 265.5 us; the boundary, once the one-step kernel let two
    // of its two-group workgroups share a CU: T=1024 55.8 -> 53.7 us, T=8192
    // 411 -> 406 us).
    if (invariant && tiles >= 64) plan.groups = 2;
    plan.steps_per_wave = spw;
    plan.slices = ceil_div(nsteps, 4L * spw);
    // Finisher workgroups per tile: each rescales at least 256 elements of
    // its 16 rows (128 for batches of at most 16 tiles, where more, lighter
    // workgroups shorten the call: d=7168, T=32 11.1 -> 10.9 us, T=256 19.4 ->
    // 19.2 us; from 32 tiles the wider slices are faster).
    const int min_width = tiles <= 16 ? 128 : 256;
    int fs = std::max(1, std::min(ceil_div(kFinishTarget, tiles), hidden / min_width));
    plan.finish_width = ceil_div(ceil_div(hidden, fs), 8) * 8;
    plan.finish_slices = ceil_div(hidden, plan.finish_width);
    return plan;
}

static_assert(kCounterBytes >= 4 * (3 + 3 * ((size_t)MHC_MAX_TOKENS + 63) / 64),
              "the counters region covers every batch size");

// The finest split (one step per wave) has the most slices: enough for every plan.
size_t split_workspace_bytes(int T, int hidden) {
    return (size_t)T * split_plan(T, hidden, true, true).slices * kPart * sizeof(float);
}

}  // namespace mhc

using namespace mhc;

// ---- mhc_boundary: validation and launches shared by both entry points --------

namespace {

// Everything but the workspace: parameters, shape, required pointers, alignment
// and aliasing among the inputs and outputs.
mhc_status check_boundary(int tokens, int hidden, const uint16_t* x, const uint16_t* residual,
                          const float* post_prev, const float* comb_prev, const float* pre_lag,
                          const void* w_prepared, const float* scale, const float* base,
                          const uint16_t* norm_w, const mhc_params* params,
                          uint16_t* residual_out, uint16_t* layer_input, float* pre_out,
                          float* post_out, float* comb_out, float* mixes, float* rstd) {
    mhc_status st = check_params(params);
    if (st != MHC_OK) return st;
    if (params->schedule == MHC_SCHEDULE_ONEPASS) return MHC_ERR_INVALID_ARGUMENT;  // (mhc_pre only)
    if (tokens < 0) return MHC_ERR_INVALID_ARGUMENT;
    if (tokens > MHC_MAX_TOKENS || !shape_ok(hidden)) return MHC_ERR_UNSUPPORTED_SHAPE;
    if (params->schedule == MHC_SCHEDULE_FUSED && !fused_supported(hidden))
        return MHC_ERR_UNSUPPORTED_SHAPE;
    if (tokens == 0) return MHC_OK;
    if (!x || !residual || !post_prev || !comb_prev || !pre_lag || !w_prepared || !scale ||
        !base || !residual_out || !layer_input || !pre_out || !post_out || !comb_out)
        return MHC_ERR_INVALID_ARGUMENT;
    const void* ptrs[] = {x, residual, post_prev, comb_prev, pre_lag, w_prepared, scale, base,
                          norm_w, residual_out, layer_input, pre_out, post_out, comb_out,
                          mixes, rstd};
    for (const void* q : ptrs)
        if (q && !aligned(q)) return MHC_ERR_MISALIGNED;
    const size_t T = tokens, d = hidden;
    const Span outs[] = {{residual_out, T * 4 * d * 2}, {layer_input, T * d * 2},
                         {pre_out, T * 16}, {post_out, T * 16}, {comb_out, T * 64},
                         {mixes, mixes ? T * 96 : 0}, {rstd, rstd ? T * 4 : 0}};
    const Span ins[] = {{x, T * d * 2}, {residual, T * 4 * d * 2}, {post_prev, T * 16},
                        {comb_prev, T * 64}, {pre_lag, T * 16}, {w_prepared, 384 * d},
                        {scale, 12}, {base, 96}, {norm_w, norm_w ? d * 2 : 0}};
    if (any_alias(outs, 7, ins, 9)) return MHC_ERR_ALIASING;
    return MHC_OK;
}

// Bytes of partial records the boundary's schedule for this batch writes: the
// split schedules' [T][slices][32] FP32 records; 0 on the fused kernels.
size_t boundary_scratch_bytes(int tokens, int hidden, int schedule) {
    const BoundaryPath path = boundary_path(schedule, tokens, hidden).path;
    if (path == BoundaryPath::Stream) return kCounterBytes + stream_data_bytes(tokens, hidden);
    if (path != BoundaryPath::Split) return 0;
    const SplitPlan plan = split_plan(tokens, hidden, schedule == MHC_SCHEDULE_INVARIANT, true);
    return kCounterBytes + (size_t)tokens * plan.slices * kPart * sizeof(float);
}

// Launches of a validated call; part receives the split schedules' records.
// MHC_SYNC_DEBUG=1 in the environment (read once per process): every entry
// point waits for the kernels it enqueued and reports a failed one as
// MHC_ERR_DEVICE, so a fault is tied to the call that caused it.  A debugging
// aid: it makes each call synchronous, and a stream under graph capture cannot
// be waited on.
bool sync_debug() {
    static const bool on = [] {
        const char* e = std::getenv("MHC_SYNC_DEBUG");
        return e != nullptr && e[0] == '1' && e[1] == '\0';
    }();
    return on;
}

mhc_status finish_call(mhc_status st, hipStream_t stream) {
    if (st != MHC_OK || !sync_debug()) return st;
    if (hipStreamSynchronize(stream) != hipSuccess) return MHC_ERR_DEVICE;
    return hipGetLastError() == hipSuccess ? MHC_OK : MHC_ERR_DEVICE;
}

mhc_status run_boundary(int tokens, int hidden, const uint16_t* x, const uint16_t* residual,
                        const float* post_prev, const float* comb_prev, const float* pre_lag,
                        const void* w_prepared, const float* scale, const float* base,
                        const uint16_t* norm_w, const mhc_params* params,
                        uint16_t* residual_out, uint16_t* layer_input, float* pre_out,
                        float* post_out, float* comb_out, float* mixes, float* rstd, void* ws,
                        hipStream_t hs) {
    const Scalars s = scalars(params);
    float* const part = reinterpret_cast<float*>(static_cast<char*>(ws) + kCounterBytes);
    const BoundaryChoice choice = boundary_path(params->schedule, tokens, hidden);
    if (choice.path == BoundaryPath::Stream) {
        const StreamPlan plan = stream_plan(tokens, hidden);
        return launch_stream(plan, tokens, hidden, x, residual, post_prev, comb_prev, pre_lag,
                             w_prepared, scale, base, norm_w, s, residual_out, layer_input,
                             pre_out, post_out, comb_out, mixes, rstd, ws, hs) == hipSuccess
                   ? MHC_OK
                   : MHC_ERR_DEVICE;
    }
    if (choice.path != BoundaryPath::Split) {
        if (!fused_supported(hidden)) return MHC_ERR_UNSUPPORTED_SHAPE;
        const hipError_t e =
            choice.path == BoundaryPath::Fused32
                ? launch_fused_w4(tokens, choice.tile_tokens, hidden, x, residual, post_prev,
                                  comb_prev, pre_lag, w_prepared, scale, base, norm_w, s,
                                  residual_out, layer_input, pre_out, post_out, comb_out, mixes,
                                  rstd, hs)
                : launch_fused(tokens, hidden, x, residual, post_prev, comb_prev, pre_lag,
                               w_prepared, scale, base, norm_w, s, residual_out, layer_input,
                               pre_out, post_out, comb_out, mixes, rstd, hs);
        return e == hipSuccess ? MHC_OK : MHC_ERR_DEVICE;
    }
    const SplitPlan plan =
        split_plan(tokens, hidden, params->schedule == MHC_SCHEDULE_INVARIANT, true);
    // layer_input first receives li; the finishing kernel rescales it in place.
    if (launch_partial(true, plan, tokens, hidden, x, residual, post_prev, comb_prev, pre_lag,
                       w_prepared, residual_out, layer_input, part, hs) != hipSuccess)
        return MHC_ERR_DEVICE;
    if (launch_finish(plan, tokens, hidden, part, scale, base, norm_w, s, layer_input, pre_out,
                      post_out, comb_out, mixes, rstd, hs) != hipSuccess)
        return MHC_ERR_DEVICE;
    return MHC_OK;
}

// ---- the no-allocation entry point's scratch ---------------------------------------
//
// For callers that cannot allocate (graph capture, serving loops, harnesses
// that forbid hipMalloc): a device array holding the split schedules' partial
// records, MHC_NOALLOC_SCRATCH_BYTES in size.  Every GPU that the library runs
// on holds its own copy until the process ends.  Host code never passes the
// array's name to a kernel: it is only a host-side stand-in.  The device
// address is looked up once per device, with that device current, and kept.
static __device__ __align__(256) unsigned char scratch[MHC_NOALLOC_SCRATCH_BYTES];

constexpr int kScratchDevices = 64;

void* scratch_address() {
    static std::atomic<void*> addr[kScratchDevices];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return nullptr;
    void* p = addr[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        addr[dev].store(p, std::memory_order_release);
    }
    return p;
}

}  // namespace

extern "C" {

int mhc_abi_version(void) { return MHC_ABI_VERSION; }

const char* mhc_status_string(mhc_status s) {
    switch (s) {
        case MHC_OK: return "ok";
        case MHC_ERR_INVALID_ARGUMENT: return "invalid argument";
        case MHC_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
        case MHC_ERR_MISALIGNED: return "pointer not 16-byte aligned";
        case MHC_ERR_ALIASING: return "output overlaps another buffer";
        case MHC_ERR_WORKSPACE: return "workspace missing or too small";
        case MHC_ERR_DEVICE: return "HIP launch failed";
        case MHC_ERR_SCRATCH_LIMIT:
            return "batch needs more than the no-allocation entry point's scratch";
    }
    return "unknown status";
}

const char* mhc_boundary_kernels(int tokens, int hidden, int schedule) {
    if (tokens <= 0 || tokens > MHC_MAX_TOKENS || !shape_ok(hidden) || schedule < MHC_SCHEDULE_AUTO ||
        schedule > MHC_SCHEDULE_STREAM)
        return "";
    if (schedule == MHC_SCHEDULE_FUSED && !fused_supported(hidden)) return "";
    switch (boundary_path(schedule, tokens, hidden).path) {
        case BoundaryPath::Fused32: return "k_fused_w4";
        case BoundaryPath::Fused16: return "k_fused";
        case BoundaryPath::Stream: return "k_stream";
        case BoundaryPath::Split: break;
    }
    return "k_partial+k_finish";
}

size_t mhc_prepared_weight_bytes(int hidden) {
    return shape_ok(hidden) ? (size_t)384 * hidden : 0;
}

size_t mhc_workspace_bytes(int tokens, int hidden) {
    if (tokens <= 0 || tokens > MHC_MAX_TOKENS || !shape_ok(hidden)) return 0;
    return kCounterBytes +
           std::max(split_workspace_bytes(tokens, hidden), stream_data_bytes(tokens, hidden));
}

mhc_status mhc_prepare_weight(const float* w, int hidden, void* w_prepared, void* stream) {
    if (!w || !w_prepared) return MHC_ERR_INVALID_ARGUMENT;
    if (!shape_ok(hidden)) return MHC_ERR_UNSUPPORTED_SHAPE;
    if (!aligned(w) || !aligned(w_prepared)) return MHC_ERR_MISALIGNED;
    const Span out{w_prepared, mhc_prepared_weight_bytes(hidden)};
    const Span in{w, (size_t)24 * 4 * hidden * sizeof(float)};
    if (overlap(out, in)) return MHC_ERR_ALIASING;
    if (launch_prepare_weight(w, hidden, w_prepared, (hipStream_t)stream) != hipSuccess)
        return MHC_ERR_DEVICE;
    return finish_call(MHC_OK, (hipStream_t)stream);
}

mhc_status mhc_pre_mixes(int tokens, int hidden, int splits, const uint16_t* residual,
                         const float* dot_mix, const float* sqrsum, const float* scale,
                         const float* base, const uint16_t* norm_w, const mhc_params* params,
                         uint16_t* layer_input, float* pre, float* post, float* comb,
                         void* stream) {
    mhc_status st = check_params(params);
    if (st != MHC_OK) return st;
    if (tokens < 0 || splits < 1 || splits > 64) return MHC_ERR_INVALID_ARGUMENT;
    if (tokens > MHC_MAX_TOKENS || !shape_ok(hidden)) return MHC_ERR_UNSUPPORTED_SHAPE;
    if (tokens == 0) return MHC_OK;
    if (!residual || !dot_mix || !sqrsum || !scale || !base || !layer_input || !pre || !post ||
        !comb)
        return MHC_ERR_INVALID_ARGUMENT;
    const void* ptrs[] = {residual, dot_mix, sqrsum, scale, base, norm_w, layer_input, pre, post,
                          comb};
    for (const void* q : ptrs)
        if (q && !aligned(q)) return MHC_ERR_MISALIGNED;
    const size_t T = tokens, d = hidden, S = splits;
    const Span outs[] = {{layer_input, T * d * 2}, {pre, T * 16}, {post, T * 16}, {comb, T * 64}};
    const Span ins[] = {{residual, T * 4 * d * 2}, {dot_mix, S * T * 96}, {sqrsum, S * T * 4},
                        {scale, 12}, {base, 96}, {norm_w, norm_w ? d * 2 : 0}};
    if (any_alias(outs, 4, ins, 6)) return MHC_ERR_ALIASING;
    if (launch_pre_mixes(tokens, hidden, splits, residual, dot_mix, sqrsum, scale, base, norm_w,
                         scalars(params), layer_input, pre, post, comb,
                         (hipStream_t)stream) != hipSuccess)
        return MHC_ERR_DEVICE;
    return finish_call(MHC_OK, (hipStream_t)stream);
}

mhc_status mhc_prefetch_weight(const void* w_prepared, int hidden, void* stream) {
    if (!w_prepared) return MHC_ERR_INVALID_ARGUMENT;
    if (!shape_ok(hidden)) return MHC_ERR_UNSUPPORTED_SHAPE;
    if (!aligned(w_prepared)) return MHC_ERR_MISALIGNED;
    if (launch_prefetch_weight(w_prepared, hidden, (hipStream_t)stream) != hipSuccess)
        return MHC_ERR_DEVICE;
    return finish_call(MHC_OK, (hipStream_t)stream);
}

mhc_status mhc_post(int tokens, int hidden, const uint16_t* x, const uint16_t* residual,
                    const float* post_prev, const float* comb_prev, uint16_t* residual_out,
                    void* stream) {
    if (tokens < 0) return MHC_ERR_INVALID_ARGUMENT;
    if (tokens > MHC_MAX_TOKENS || !shape_ok(hidden)) return MHC_ERR_UNSUPPORTED_SHAPE;
    if (tokens == 0) return MHC_OK;
    if (!x || !residual || !post_prev || !comb_prev || !residual_out)
        return MHC_ERR_INVALID_ARGUMENT;
    const void* ptrs[] = {x, residual, post_prev, comb_prev, residual_out};
    for (const void* q : ptrs)
        if (!aligned(q)) return MHC_ERR_MISALIGNED;
    const size_t T = tokens, d = hidden;
    const Span outs[] = {{residual_out, T * 4 * d * 2}};
    const Span ins[] = {{x, T * d * 2}, {residual, T * 4 * d * 2}, {post_prev, T * 16},
                        {comb_prev, T * 64}};
    if (any_alias(outs, 1, ins, 4)) return MHC_ERR_ALIASING;
    if (launch_post(tokens, hidden, x, residual, post_prev, comb_prev, residual_out,
                    (hipStream_t)stream) != hipSuccess)
        return MHC_ERR_DEVICE;
    return finish_call(MHC_OK, (hipStream_t)stream);
}

mhc_status mhc_pre(int tokens, int hidden, const uint16_t* residual, const void* w_prepared,
                   const float* scale, const float* base, const uint16_t* norm_w,
                   const mhc_params* params, uint16_t* layer_input, float* pre, float* post,
                   float* comb, float* mixes, float* rstd, void* workspace,
                   size_t workspace_bytes, void* stream) {
    mhc_status st = check_params(params);
    if (st != MHC_OK) return st;
    if (tokens < 0) return MHC_ERR_INVALID_ARGUMENT;
    if (tokens > MHC_MAX_TOKENS || !shape_ok(hidden)) return MHC_ERR_UNSUPPORTED_SHAPE;
    if (params->schedule == MHC_SCHEDULE_FUSED && !fused_supported(hidden))
        return MHC_ERR_UNSUPPORTED_SHAPE;
    if (params->schedule == MHC_SCHEDULE_ONEPASS && tokens > 0 &&
        !pre_one_supported(tokens, hidden, device_compute_units()))
        return MHC_ERR_UNSUPPORTED_SHAPE;
    if (tokens == 0) return MHC_OK;
    if (!residual || !w_prepared || !scale || !base || !layer_input || !pre || !post || !comb)
        return MHC_ERR_INVALID_ARGUMENT;
    const void* ptrs[] = {residual, w_prepared, scale, base, norm_w, layer_input, pre, post,
                          comb, mixes, rstd, workspace};
    for (const void* q : ptrs)
        if (q && !aligned(q)) return MHC_ERR_MISALIGNED;
    const size_t T = tokens, d = hidden;
    const size_t need = mhc_workspace_bytes(tokens, hidden);
    const Span outs[] = {{layer_input, T * d * 2}, {pre, T * 16}, {post, T * 16}, {comb, T * 64},
                         {mixes, mixes ? T * 96 : 0}, {rstd, rstd ? T * 4 : 0},
                         {workspace, need}};
    const Span ins[] = {{residual, T * 4 * d * 2}, {w_prepared, 384 * d}, {scale, 12},
                        {base, 96}, {norm_w, norm_w ? d * 2 : 0}};
    if (any_alias(outs, 7, ins, 5)) return MHC_ERR_ALIASING;
    if (!workspace || workspace_bytes < need) return MHC_ERR_WORKSPACE;

    const Scalars s = scalars(params);
    hipStream_t hs = (hipStream_t)stream;
    if (params->schedule == MHC_SCHEDULE_FUSED) {
        if (!fused_supported(hidden)) return MHC_ERR_UNSUPPORTED_SHAPE;
        if (launch_fused_pre(tokens, hidden, residual, w_prepared, scale, base, norm_w, s,
                             layer_input, pre, post, comb, mixes, rstd, tokens >= kW4MinTokens,
                             hs) != hipSuccess)
            return MHC_ERR_DEVICE;
        return finish_call(MHC_OK, hs);
    }
    if (params->schedule == MHC_SCHEDULE_ONEPASS) {
        if (launch_pre_one(tokens, hidden, residual, w_prepared, scale, base, norm_w, s, layer_input, pre,
                           post, comb, mixes, rstd, workspace, hs) != hipSuccess)
            return MHC_ERR_DEVICE;
        return finish_call(MHC_OK, hs);
    }
    const SplitPlan plan =
        split_plan(tokens, hidden, params->schedule == MHC_SCHEDULE_INVARIANT, false);
    // (past the streaming schedule's counters, which it must not touch)
    float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + kCounterBytes);
    if (launch_partial(false, plan, tokens, hidden, nullptr, residual, nullptr, nullptr, nullptr,
                       w_prepared, nullptr, nullptr, part, hs) != hipSuccess)
        return MHC_ERR_DEVICE;
    if (launch_pre_finish(plan, tokens, hidden, residual, part, scale, base, norm_w, s,
                          layer_input, pre, post, comb, mixes, rstd, hs) != hipSuccess)
        return MHC_ERR_DEVICE;
    return finish_call(MHC_OK, hs);
}

mhc_status mhc_boundary(int tokens, int hidden, const uint16_t* x, const uint16_t* residual,
                        const float* post_prev, const float* comb_prev, const float* pre_lag,
                        const void* w_prepared, const float* scale, const float* base,
                        const uint16_t* norm_w, const mhc_params* params,
                        uint16_t* residual_out, uint16_t* layer_input, float* pre_out,
                        float* post_out, float* comb_out, float* mixes, float* rstd,
                        void* workspace, size_t workspace_bytes, void* stream) {
    mhc_status st = check_boundary(tokens, hidden, x, residual, post_prev, comb_prev, pre_lag,
                                   w_prepared, scale, base, norm_w, params, residual_out,
                                   layer_input, pre_out, post_out, comb_out, mixes, rstd);
    if (st != MHC_OK || tokens == 0) return st;
    if (workspace && !aligned(workspace)) return MHC_ERR_MISALIGNED;
    const size_t T = tokens, d = hidden;
    const size_t need = mhc_workspace_bytes(tokens, hidden);
    const Span ws{workspace, need};
    const Span others[] = {{x, T * d * 2}, {residual, T * 4 * d * 2}, {post_prev, T * 16},
                           {comb_prev, T * 64}, {pre_lag, T * 16}, {w_prepared, 384 * d},
                           {scale, 12}, {base, 96}, {norm_w, norm_w ? d * 2 : 0},
                           {residual_out, T * 4 * d * 2}, {layer_input, T * d * 2},
                           {pre_out, T * 16}, {post_out, T * 16}, {comb_out, T * 64},
                           {mixes, mixes ? T * 96 : 0}, {rstd, rstd ? T * 4 : 0}};
    if (any_alias(&ws, 1, others, 16)) return MHC_ERR_ALIASING;
    if (!workspace || workspace_bytes < need) return MHC_ERR_WORKSPACE;
    return finish_call(run_boundary(tokens, hidden, x, residual, post_prev, comb_prev, pre_lag,
                                    w_prepared, scale, base, norm_w, params, residual_out,
                                    layer_input, pre_out, post_out, comb_out, mixes, rstd, workspace,
                                    (hipStream_t)stream),
                       (hipStream_t)stream);
}

mhc_status mhc_boundary_noalloc(int tokens, int hidden, const uint16_t* x,
                                const uint16_t* residual, const float* post_prev,
                                const float* comb_prev, const float* pre_lag,
                                const void* w_prepared, const float* scale, const float* base,
                                const uint16_t* norm_w, const mhc_params* params,
                                uint16_t* residual_out, uint16_t* layer_input, float* pre_out,
                                float* post_out, float* comb_out, float* mixes, float* rstd,
                                void* stream) {
    mhc_status st = check_boundary(tokens, hidden, x, residual, post_prev, comb_prev, pre_lag,
                                   w_prepared, scale, base, norm_w, params, residual_out,
                                   layer_input, pre_out, post_out, comb_out, mixes, rstd);
    if (st != MHC_OK || tokens == 0) return st;
    if (boundary_scratch_bytes(tokens, hidden, params->schedule) > sizeof(scratch))
        return MHC_ERR_SCRATCH_LIMIT;
    void* ws = scratch_address();
    if (!ws) return MHC_ERR_DEVICE;
    return finish_call(run_boundary(tokens, hidden, x, residual, post_prev, comb_prev, pre_lag,
                                    w_prepared, scale, base, norm_w, params, residual_out,
                                    layer_input, pre_out, post_out, comb_out, mixes, rstd, ws,
                                    (hipStream_t)stream),
                       (hipStream_t)stream);
}

}  // extern "C"
