// Host-side launch interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mhc {

struct Scalars;

// Work split of the split schedule for (T, hidden).  Both kernels take a 1-D
// grid in tile-major order: workgroup id = tile * slices + slice, so the
// workgroups in flight at any moment cover whole rows of a few consecutive
// token tiles (HBM serves that far better than the same bytes spread over
// every tile of the batch: 5.6 against 4.9 TB/s for a mover of the boundary's
// bytes).
//   k_partial: slice q of a tile covers hidden steps
//              [4q * steps_per_wave, 4(q + 1) * steps_per_wave) of 32 elements,
//              4 at a time; wave w projects steps 4q * steps_per_wave + w,
//              + 4, ...
//   k_finish:  workgroup q of a 16-token tile rescales hidden
//              [q * finish_width, (q + 1) * finish_width).
struct SplitPlan {
    int groups;          // 16-token groups per wave in the partial kernel (1, 2 or 4)
    int steps_per_wave;
    int slices;
    int finish_slices;
    int finish_width;
    bool stream;         // nontemporal hints on the residual streams (large batches)
};

SplitPlan split_plan(int T, int hidden, bool invariant, bool shifted);

// Workgroups of the boundary's multi-step partial kernel (1 or 2 token groups)
// the current device holds at once: compute units times resident workgroups
// per unit.  0 if the runtime cannot say.
int partial_resident_workgroups(int groups);

// Compute units of the current device; 0 if the runtime cannot say.
int device_compute_units();
size_t split_workspace_bytes(int T, int hidden);

hipError_t launch_prepare_weight(const float* w, int hidden, void* out, hipStream_t stream);

hipError_t launch_prefetch_weight(const void* wprep, int hidden, hipStream_t stream);

hipError_t launch_post(int T, int hidden, const uint16_t* x, const uint16_t* X,
                       const float* post_prev, const float* comb_prev, uint16_t* xn_out,
                       hipStream_t stream);

hipError_t launch_partial(bool shifted, const SplitPlan& plan, int T, int hidden,
                          const uint16_t* x, const uint16_t* X, const float* post_prev,
                          const float* comb_prev, const float* pre_lag, const void* wprep,
                          uint16_t* xn_out, uint16_t* li_out, float* part, hipStream_t stream);

hipError_t launch_finish(const SplitPlan& plan, int T, int hidden, const float* part,
                         const float* scale, const float* base, const uint16_t* norm_w,
                         const Scalars& p, uint16_t* layer_input, float* pre_out,
                         float* post_out, float* comb_out, float* mixes, float* rstd,
                         hipStream_t stream);

hipError_t launch_pre_finish(const SplitPlan& plan, int T, int hidden, const uint16_t* X,
                             const float* part, const float* scale, const float* base,
                             const uint16_t* norm_w, const Scalars& p, uint16_t* layer_input,
                             float* pre_out, float* post_out, float* comb_out, float* mixes,
                             float* rstd, hipStream_t stream);

// Non-shifted pre from precomputed projection partials (dot_mix [splits, T, 24],
// sqrsum [splits, T]).
hipError_t launch_pre_mixes(int T, int hidden, int splits, const uint16_t* X,
                            const float* dot_mix, const float* sqrsum, const float* scale,
                            const float* base, const uint16_t* norm_w, const Scalars& p,
                            uint16_t* layer_input, float* pre_out, float* post_out,
                            float* comb_out, hipStream_t stream);

// Fused schedule: one 8-wave workgroup per 16-token tile over all of hidden.
bool fused_supported(int hidden);
hipError_t launch_fused(int T, int hidden, const uint16_t* x, const uint16_t* X,
                        const float* post_prev, const float* comb_prev, const float* pre_lag,
                        const void* wprep, const float* scale, const float* base,
                        const uint16_t* norm_w, const Scalars& p, uint16_t* xn_out,
                        uint16_t* layer_input, float* pre_out, float* post_out, float* comb_out,
                        float* mixes, float* rstd, hipStream_t stream);

// Fused schedule on 4 waves with tiles of tile_tokens <= 32 tokens (two token
// groups per wave share the weight fragments); same widths as launch_fused.
hipError_t launch_fused_w4(int T, int tile_tokens, int hidden, const uint16_t* x,
                           const uint16_t* X, const float* post_prev, const float* comb_prev,
                           const float* pre_lag, const void* wprep, const float* scale,
                           const float* base, const uint16_t* norm_w, const Scalars& p,
                           uint16_t* xn_out, uint16_t* layer_input, float* pre_out,
                           float* post_out, float* comb_out, float* mixes, float* rstd,
                           hipStream_t stream);

// Non-shifted pre, fused: one workgroup per token tile, two passes over the
// tile's X (fused_supported widths); tiles32 selects 32-token tiles on 4 waves
// instead of 16-token tiles on 8 waves.
hipError_t launch_fused_pre(int T, int hidden, const uint16_t* X, const void* wprep,
                            const float* scale, const float* base, const uint16_t* norm_w,
                            const Scalars& p, uint16_t* layer_input, float* pre_out,
                            float* post_out, float* comb_out, float* mixes, float* rstd,
                            bool tiles32, hipStream_t stream);

// Every workspace starts with the streaming schedule's queue and tile
// counters: a fixed region sized for the largest batch (2^20 tokens in 64-token
// tiles), which no other kernel writes and which the streaming kernel leaves
// zero after every call, so that one workspace can serve every schedule and
// batch size.  The split schedules' records and the streaming schedule's data
// follow it.
constexpr size_t kCounterBytes = ((size_t)4 * (3 + 3 * (((size_t)1 << 20) / 64)) + 255) / 256 * 256;

// Streaming schedule of the boundary (one persistent launch, work queue of
// (64-token tile, 32*kb-element slice) items).  After the counters the
// workspace holds rstd_li per token and the partial records.
struct StreamPlan {
    int kb;          // 32-element k-blocks per item
    int slices;      // items per tile
    int tiles;       // 64-token tiles
    int lag;         // tile r is finished by the items of tile r + lag
    int items;       // queue length: (tiles + lag) * slices
    int grid;        // persistent workgroups
    int sync_words;  // counters at the start of the workspace
};

StreamPlan stream_plan(int T, int hidden);
size_t stream_data_bytes(int T, int hidden);  // after the counters
// Single-pass non-shifted pre (T <= 64, one workgroup per 128 elements of
// hidden, all resident at once): whether it runs on a device with this many
// compute units, the bytes of its records (after the counters region), and
// the launch.
bool pre_one_supported(int T, int hidden, int compute_units);
size_t pre_one_data_bytes(int T, int hidden);
hipError_t launch_pre_one(int T, int hidden, const uint16_t* X, const void* wprep, const float* scale,
                          const float* base, const uint16_t* norm_w, const Scalars& p, uint16_t* layer_input,
                          float* pre, float* post, float* comb, float* mixes, float* rstd, void* workspace,
                          hipStream_t stream);

hipError_t launch_stream(const StreamPlan& plan, int T, int hidden, const uint16_t* x,
                         const uint16_t* X, const float* post_prev, const float* comb_prev,
                         const float* pre_lag, const void* wprep, const float* scale,
                         const float* base, const uint16_t* norm_w, const Scalars& p,
                         uint16_t* xn_out, uint16_t* layer_input, float* pre_out,
                         float* post_out, float* comb_out, float* mixes, float* rstd,
                         void* workspace, hipStream_t stream);  // workspace: counters first

}  // namespace mhc
