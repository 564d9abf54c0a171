/*
 * mhc.h -- C ABI of the MI355X (gfx950) mHC layer-boundary library.
 *
 * The manifold-constrained hyper-connection (mHC) boundary works on a residual
 * of n_hc = 4 BF16 streams per token.  Per token t (streams s, j in 0..3,
 * hidden h in 0..d-1, flat index k = s*d + h):
 *
 *   X'[s][h]  = bf16( FMA chain over j = 0..3 of comb[j][s]*X[j][h], started
 *                     from post[s]*x[h] in FP32 )
 *   mix[n]    = sum_k tf32(W)[n][k] * X'[k]                 (n = 0..23)
 *   rstd      = 1 / sqrt( sum_k X'[k]^2 / (4d) + rms_eps )
 *   pre[j]    = sigmoid( mix[j]*rstd*scale[0] + base[j] ) + pre_eps
 *   post[j]   = post_mult * sigmoid( mix[4+j]*rstd*scale[1] + base[4+j] )
 *   comb[i][k]= Sinkhorn of the logits mix[8+4i+k]*rstd*scale[2] + base[8+4i+k]:
 *               row softmax + eps, one column normalisation, then
 *               (sinkhorn_iters - 1) x (row, column) normalisations,
 *               each normalisation dividing by (sum + sinkhorn_eps)
 *   li[h]     = bf16( FMA chain over j = 0..3 of pre_lag[j]*X'[j][h], from 0 )
 *   layer_input[h] = bf16( li[h] * rstd_li * norm_w[h] ),
 *               rstd_li = 1 / sqrt( sum_h li[h]^2 / d + norm_eps );
 *               layer_input = li when norm_w is NULL.
 *
 * Sources: the vLLM page "DeepSeek-V4.1 shifted mHC boundary for decode-size
 * batches" (module description; residual_update; lagged_collapse;
 * coefficients; sinkhorn; col_normalize; layer_input_words;
 * prepare_boundary_weight; mhc_shifted_post_pre_boundary) and the blog "The
 * Hyper Connection Preprocessing GPU Kernel Study" (Table 1 variable map;
 * "square sum and RMSNorm"; "computing A_l", "computing C_l", "computing B_l";
 * "computing layer_input A_l X_l"; "memory layout assumptions").
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers on the current HIP device, contiguous,
 *     row-major, 16-byte aligned.  BF16 tensors are passed as uint16_t bit
 *     patterns.  The caller allocates and owns every buffer and keeps it alive
 *     until the work on `stream` has completed.  The library keeps no pointer
 *     after it returns and allocates no device memory.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *     asynchronously; the library never synchronises.
 *   - Arguments are validated on the host before anything is enqueued; on any
 *     error nothing is launched and no output is written.  Execution faults
 *     surface at the caller's next synchronisation.
 *   - Results are deterministic: every reduction runs in a fixed order, so
 *     equal inputs give bitwise-equal outputs from call to call.
 *   - An empty batch (tokens == 0) is a no-op: once the parameters and
 *     `hidden` pass their checks the call returns MHC_OK without reading any
 *     pointer (they may be NULL) and without enqueueing anything.
 */
#ifndef MHC_H
#define MHC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MHC_ABI_VERSION 1
#define MHC_N_HC 4          /* residual streams (the pages' hc_mult / kHc4) */
#define MHC_MIXES 24        /* 4 pre + 4 post + 16 comb (the pages' kMixHc4) */
#define MHC_MAX_TOKENS (1 << 20)
#define MHC_MIN_HIDDEN 256
#define MHC_MAX_HIDDEN 16384
/* Size of the device array that mhc_boundary_noalloc uses in place of a
 * workspace (64 MiB per GPU, held until the process ends). */
#define MHC_NOALLOC_SCRATCH_BYTES (64u << 20)

/* Status codes.  The refusals mirror the ones of mhc_shifted_post_pre_boundary
 * on the vLLM page, which returns None for a token count out of range or for a
 * tensor that is not contiguous or not 16-byte aligned; here each cause has a
 * code of its own and nothing is enqueued.  MHC_ERR_WORKSPACE has no
 * counterpart there (that kernel keeps its partial sums on chip): it sits at
 * 5, so MHC_ERR_DEVICE is 6. */
typedef enum {
    MHC_OK = 0,
    MHC_ERR_INVALID_ARGUMENT = 1, /* tokens < 0, NULL required pointer, iters < 1, eps < 0 */
    MHC_ERR_UNSUPPORTED_SHAPE = 2,/* hidden % 256 != 0, hidden outside [256, 16384], tokens > MHC_MAX_TOKENS */
    MHC_ERR_MISALIGNED = 3,       /* a pointer not 16-byte aligned */
    MHC_ERR_ALIASING = 4,         /* an output overlaps another output or an input */
    MHC_ERR_WORKSPACE = 5,        /* workspace NULL or smaller than mhc_workspace_bytes() */
    MHC_ERR_DEVICE = 6,           /* a HIP call or kernel launch failed */
    MHC_ERR_SCRATCH_LIMIT = 7     /* mhc_boundary_noalloc: the batch's schedule needs more
                                     partial-record space than MHC_NOALLOC_SCRATCH_BYTES */
} mhc_status;

/* Scheduling choice for mhc_boundary and mhc_pre (results are identical up
 * to the accumulation order of the FP32 sums; each choice is deterministic:
 * the same call on the same inputs gives the same bits on the same device).
 * AUTO and SPLIT size the split to the current device's compute units and
 * occupancy, so on a device with another compute-unit count they may sum in
 * another order; INVARIANT does not depend on the device.  FUSED exists for
 * hidden in {1024, 2048, 4096, 5120, 6144, 7168, 8192}; asked for any other
 * width it returns MHC_ERR_UNSUPPORTED_SHAPE.
 *
 * INVARIANT is the batch-invariant mode (the vLLM page, module notes on the
 * pinned reduction order of mhc_fused_hc): every FP32 sum of a token runs in
 * an order fixed by hidden alone, so a token's outputs are bit-identical for
 * any token count T and any position in the batch.  It runs the split kernels
 * with one 32-element step per wave (the finest split).  AUTO and SPLIT pick
 * that same split while its workgroups, ceil(T / 16) * hidden / 128, fit in
 * one round (mhc_boundary: the device's resident workgroups, T <= 144 at
 * hidden 7168 on 256 compute units; mhc_pre: one workgroup per compute unit,
 * T <= 64), so small decode batches give the same bits under all three. */
typedef enum {
    MHC_SCHEDULE_AUTO = 0,        /* mhc_boundary, from the device's compute-unit count:
                                     SPLIT while 16-token tiles would fill less than 5/8 of
                                     one round of compute units (T < 2560 on 256); where the
                                     fused kernels exist, 4-wave tiles of ceil(T / (rounds x
                                     units)) <= 32 tokens where that is at least 18 in one
                                     round or 28 in more, else 16-token tiles over as many
                                     rounds as they take.  mhc_pre: SPLIT */
    MHC_SCHEDULE_SPLIT = 1,       /* hidden split over many workgroups + finishing kernel */
    MHC_SCHEDULE_FUSED = 2,       /* one workgroup per token tile owns all of hidden: 16-token
                                     tiles on 8 waves, or from 8192 tokens 32-token tiles on
                                     4 waves */
    MHC_SCHEDULE_INVARIANT = 3,   /* batch-invariant: split with an order fixed by hidden */
    MHC_SCHEDULE_STREAM = 4,      /* mhc_boundary: one persistent launch over a queue of
                                     (64-token tile, 256-element slice) items in tile-major
                                     order; mhc_pre: SPLIT */
    MHC_SCHEDULE_ONEPASS = 5      /* mhc_pre only: one launch that reads X once ([P]
                                     "computing pre_mix early"), for 1 <= T <= 64 on a device
                                     with at least hidden / 128 compute units (one workgroup
                                     per 128 elements of hidden holds every token's slice of X
                                     in registers; the workgroups wait on each other, so all
                                     must be resident at once); UNSUPPORTED_SHAPE otherwise.
                                     mhc_boundary refuses it (INVALID_ARGUMENT); mhc_pre_mixes
                                     ignores the schedule. */
} mhc_schedule;

/* Runtime scalars (the pages pass them as kernel arguments). */
typedef struct {
    float rms_eps;        /* eps of the mix RMS (hc_norm_eps) */
    float pre_eps;        /* added to sigmoid for pre (hc_pre_eps) */
    float post_mult;      /* post scale (hc_post_scale), usually 2 */
    float sinkhorn_eps;   /* softmax floor and normalisation eps */
    int sinkhorn_iters;   /* >= 1: column passes; row passes = iters - 1 */
    float norm_eps;       /* eps of the layer-input RMSNorm */
    int schedule;         /* mhc_schedule (mhc_boundary and mhc_pre) */
} mhc_params;

/* Bytes of the prepared weight for `hidden`: 384 * hidden (0 if unsupported).
 * The counterpart of boundary_weight_shape on the vLLM page (the size of
 * prepare_boundary_weight's output), for the layout below.
 *
 * Layout (uint16 BF16 elements).  Element (step, s, m, l, e) with
 * step in [0, hidden/32), s in [0,4), m in [0,3), l in [0,64), e in [0,8) sits at
 *     ((((step*4 + s)*3 + m)*64 + l)*8 + e)
 * and holds part P of mix n at column k of W, where
 *     k = s*hidden + 32*step + 8*(l/16) + e,   r = l % 16,
 *     n = 8*m + 2*(r/4) + (r % 2),   P = high if (r % 4) < 2 else low,
 *     high = bf16(t), low = bf16(t - high), t = tf32(W[n][k]) (ties away).
 * The 64 x 8 block of one (step, s, m) is the A operand of one
 * 16x16x32 BF16 matrix-core product (row = l % 16, k group = l / 16): the
 * result rows 4q+0 / 4q+2 hold the high / low products of mix 8m+2q and rows
 * 4q+1 / 4q+3 those of mix 8m+2q+1.  high + low == t exactly, and every
 * BF16 x BF16 product is exact in FP32, so the projection equals the TF32 one. */
size_t mhc_prepared_weight_bytes(int hidden);

/* Device workspace bytes that mhc_pre / mhc_boundary need for `tokens`
 * tokens of `hidden` under every schedule.  The vLLM page's kernel reduces a
 * token's partial sums over its 16-CTA cluster on chip (module description:
 * fixed-order reductions; the kernel's "totals in rank order"); the split and
 * streaming schedules here pass them between workgroups through this
 * workspace instead.  Layout:
 *   bytes [0, 196864)  the streaming schedule's counters (a queue head, then
 *                      three 32-bit counters per 64-token tile, sized for
 *                      MHC_MAX_TOKENS).  They must hold zeros before the
 *                      workspace is first used with MHC_SCHEDULE_STREAM; every
 *                      streaming call returns them to zero before it ends, and
 *                      no other schedule writes them.  A workspace zero-filled
 *                      once after allocation therefore serves every schedule
 *                      and any number of calls (calls that share it must be
 *                      ordered, e.g. on one stream).
 *   the rest           partial records, rewritten by every call: the split
 *                      schedules' 128 bytes per token per 128 elements of
 *                      hidden (T * hidden bytes in all), or the streaming
 *                      schedule's rstd_li (4 bytes per token, padded to 256)
 *                      and 128 bytes per token per 256 elements of hidden. */
size_t mhc_workspace_bytes(int tokens, int hidden);  /* 0 for tokens == 0 or an invalid shape */

/* Round W to TF32, split it into BF16 high/low parts and write them in the
 * layout above.  (prepare_boundary_weight on the vLLM page.)
 *   w           [24, 4*hidden] FP32, rows = 4 pre | 4 post | 16 comb (row-major 4x4)
 *   w_prepared  mhc_prepared_weight_bytes(hidden) bytes, written
 * Errors: INVALID_ARGUMENT (NULL), UNSUPPORTED_SHAPE, MISALIGNED, ALIASING, DEVICE. */
mhc_status mhc_prepare_weight(const float* w, int hidden, void* w_prepared, void* stream);

/* Non-shifted mHC pre (the blog's mhc_pre_big_fuse, with the projection and
 * the sum of squares computed here): X' = X, pre/post/comb from the mixes of
 * X, and layer_input = bf16(FMA chain of the FRESH pre[j]*X[j]), then the
 * optional RMSNorm with norm_w.
 *   residual    [T, 4, hidden] BF16            (read)
 *   w_prepared  from mhc_prepare_weight         (read)
 *   scale [3], base [24] FP32                   (read)
 *   norm_w      [hidden] BF16 or NULL           (read)
 *   layer_input [T, hidden] BF16                (written)
 *   pre, post   [T, 4] FP32; comb [T, 4, 4] FP32 (written; comb row i = source stream)
 *   mixes       [T, 24] FP32 or NULL; rstd [T] FP32 or NULL (debug outputs)
 *   workspace   >= mhc_workspace_bytes(T, hidden) bytes, zero-filled once
 *               before its first use (layout at mhc_workspace_bytes) */
mhc_status mhc_pre(int tokens, int hidden, const uint16_t* residual, const void* w_prepared,
                   const float* scale, const float* base, const uint16_t* norm_w,
                   const mhc_params* params, uint16_t* layer_input, float* pre, float* post,
                   float* comb, float* mixes, float* rstd, void* workspace,
                   size_t workspace_bytes, void* stream);

/* Shifted mHC boundary (mhc_shifted_post_pre_boundary on the vLLM page):
 * residual update with the previous layer's post/comb, projection, new
 * pre/post/comb, and the layer input collapsed with the LAGGED pre.
 *   x           [T, hidden] BF16 block output    (read)
 *   residual    [T, 4, hidden] BF16              (read)
 *   post_prev   [T, 4] FP32; comb_prev [T, 4, 4] FP32 (row j = source stream,
 *               column s = destination stream); pre_lag [T, 4] FP32   (read)
 *   w_prepared, scale, base, norm_w              as for mhc_pre
 *   residual_out [T, 4, hidden] BF16 = X'        (written)
 *   layer_input  [T, hidden] BF16                (written)
 *   pre_out, post_out [T, 4]; comb_out [T, 4, 4] FP32 (written)
 *   mixes, rstd, workspace                       as for mhc_pre */
mhc_status mhc_boundary(int tokens, int hidden, const uint16_t* x, const uint16_t* residual,
                        const float* post_prev, const float* comb_prev, const float* pre_lag,
                        const void* w_prepared, const float* scale, const float* base,
                        const uint16_t* norm_w, const mhc_params* params,
                        uint16_t* residual_out, uint16_t* layer_input, float* pre_out,
                        float* post_out, float* comb_out, float* mixes, float* rstd,
                        void* workspace, size_t workspace_bytes, void* stream);

/* mhc_boundary for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same arguments, kernels and results as mhc_boundary (bit for bit), but
 * no workspace: what the workspace holds (the streaming schedule's counters,
 * then the split or streaming schedule's partial records, in the layout
 * described at mhc_workspace_bytes) goes to a device array of
 * MHC_NOALLOC_SCRATCH_BYTES inside the library (one per GPU, looked up on the
 * first call on each device and kept until the process ends).  The call itself
 * allocates nothing.
 *   Limit: batches whose schedule needs more space than the array holds
 *   return MHC_ERR_SCRATCH_LIMIT with nothing enqueued.  The space is the
 *   192 KiB counters region plus 128 bytes per token per hidden slice of the
 *   split schedule (INVARIANT: tokens * hidden bytes), or plus 4 + 128 *
 *   (hidden / 256) bytes per token for STREAM; the fused kernels need none.
 *   (At hidden 7168 AUTO fits every batch, since it runs the fused kernels
 *   from 2560 tokens on 256 compute units, from 3072 where the count is
 *   unknown.)
 *   Sharing: every call on one GPU uses the same array, so calls that overlap
 *   in time on one GPU (concurrent streams) race and give wrong results;
 *   calls ordered on one stream are safe.  The array starts zeroed, as the
 *   counters require, and the streaming kernel leaves its counters at zero;
 *   the records are overwritten by each call, so nothing has to be cleared
 *   between calls.
 * Errors: those of mhc_boundary, with MHC_ERR_SCRATCH_LIMIT in place of
 * MHC_ERR_WORKSPACE. */
mhc_status mhc_boundary_noalloc(int tokens, int hidden, const uint16_t* x,
                                const uint16_t* residual, const float* post_prev,
                                const float* comb_prev, const float* pre_lag,
                                const void* w_prepared, const float* scale, const float* base,
                                const uint16_t* norm_w, const mhc_params* params,
                                uint16_t* residual_out, uint16_t* layer_input, float* pre_out,
                                float* post_out, float* comb_out, float* mixes, float* rstd,
                                void* stream);

/* Non-shifted pre from a projection computed elsewhere (the blog's "pure" path:
 * mhc_pre_big_fuse with precomputed dot_mix and sqrsum, optionally split-K):
 *   dot_mix  [splits, T, 24] FP32  partial mixes, summed over splits in order
 *   sqrsum   [splits, T] FP32      partial sums of squares of the residual, likewise
 *   residual [T, 4, hidden] BF16; scale [3], base [24]; norm_w [hidden] BF16 or NULL
 * rstd = 1/sqrt(sqrsum/(4*hidden) + rms_eps); pre / post / comb as in mhc_pre;
 * layer_input = bf16(FMA chain of pre[j]*X[j]) then the optional RMSNorm.
 *   splits in [1, 64].  Outputs layer_input [T, hidden] BF16, pre, post [T, 4],
 *   comb [T, 4, 4] FP32.  ("square sum and RMSNorm", "explaining split-K" and
 *   "computing layer_input" in the blog.)
 * Errors: INVALID_ARGUMENT (incl. splits out of range), UNSUPPORTED_SHAPE,
 * MISALIGNED, ALIASING, DEVICE. */
mhc_status mhc_pre_mixes(int tokens, int hidden, int splits, const uint16_t* residual,
                         const float* dot_mix, const float* sqrsum, const float* scale,
                         const float* base, const uint16_t* norm_w, const mhc_params* params,
                         uint16_t* layer_input, float* pre, float* post, float* comb,
                         void* stream);

/* Residual update alone (the "post" half of the boundary): X'[s] =
 * bf16(FMA chain over j of comb_prev[j][s]*X[j], from post_prev[s]*x), the same
 * bits as mhc_boundary's residual_out.  (residual_update on the vLLM page; the
 * mhc_post kernel the blog mentions after "why this kernel is called pre".)
 *   x [T, hidden] BF16, residual [T, 4, hidden] BF16, post_prev [T, 4] FP32,
 *   comb_prev [T, 4, 4] FP32 (read); residual_out [T, 4, hidden] BF16 (written).
 * Errors: INVALID_ARGUMENT, UNSUPPORTED_SHAPE, MISALIGNED, ALIASING, DEVICE. */
mhc_status mhc_post(int tokens, int hidden, const uint16_t* x, const uint16_t* residual,
                    const float* post_prev, const float* comb_prev, uint16_t* residual_out,
                    void* stream);

/* Weight prefetch: reads the prepared weight (384 * hidden bytes, read only)
 * so that it is resident in the last-level cache when a following mhc_boundary
 * or mhc_pre reads it.  ROCm has no programmatic dependent launch; the stand-in
 * for the vLLM page's early weight loads (issued before the kernel waits on
 * its producer) is to enqueue this on a stream forked from the caller's before
 * the producer of x, joined back before mhc_boundary, so the weight fetch
 * overlaps the producer instead of the boundary.  It writes nothing.
 *
 * NOT RECOMMENDED as a latency optimisation.  Measured in a HIP graph beside a
 * 4 us producer, a decode call (32 tokens, hidden 7168) takes 27.7 us with the
 * fork, prefetch and join against 12.1 us without; the most the prefetch can
 * save is the cold-versus-warm weight fetch, about 1.2 us.  The join is a
 * dependency between two streams of the graph, which the runtime resolves with
 * a signal between hardware queues; that costs far more than the fetch it
 * hides.  Callers get the better latency from the plain mhc_boundary call.
 * Errors: INVALID_ARGUMENT (NULL), UNSUPPORTED_SHAPE, MISALIGNED, DEVICE. */
mhc_status mhc_prefetch_weight(const void* w_prepared, int hidden, void* stream);

/* The kernels mhc_boundary launches for this batch size, width and schedule
 * (an MHC_SCHEDULE_* value), as the library itself decides them: static text,
 * "k_fused_w4" (32-token tiles, or fewer where AUTO balances the tiles over
 * whole rounds of compute units), "k_fused" (16-token tiles),
 * "k_partial+k_finish" (the split schedule: two launches) or "k_stream" (one
 * persistent launch).  AUTO's choice depends on the current device's
 * compute-unit count.  Returns "" where mhc_boundary would refuse the shape or
 * the schedule, and for tokens <= 0 (nothing is launched).  Host only. */
const char* mhc_boundary_kernels(int tokens, int hidden, int schedule);

/* Static text for a status code (the refusal causes listed with mhc_status). */
const char* mhc_status_string(mhc_status status);

/* MHC_ABI_VERSION of the loaded library. */
int mhc_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MHC_H */
