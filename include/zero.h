/*
 * zero.h -- C ABI of the MI355X (gfx950) ZeRO sharded-optimizer step.
 *
 * One data-parallel rank owns one equal part ("shard") of the flat parameter
 * space and, in each optimizer step,
 *   1. sums the replicas' gradients over its shard (the arithmetic of the
 *      gradient reduce-scatter),
 *   2. undoes the fp16/bf16 loss scale, flags inf/nan and takes its part of
 *      the global L2 norm,
 *   3. combines the norm and flag over the world and derives the clip factor,
 *   4. applies AdamW to its fp32 master weights and Adam moments, skipping
 *      the whole step when any gradient overflowed,
 *   5. casts the new masters into its slice of the full low-precision
 *      parameter buffer (the all-gather's contribution).
 *
 * Sources, cited by page title and section:
 *   [P1] "ZeRO技术解析：大模型分布式训练的革命性突破" (intelliparadigm.com)
 *   [P2] "大模型分片训练：ZeRO-3策略在PyTorch中的实现" (dn008.com.cn); this
 *        page has no section numbers and is cited by passage topic
 *   [P3] "ZeRO 和分片优化器" (aiunderstanding.org)
 *
 * Conventions for every call.
 *   - Returns ZERO_OK (0) or a negative ZERO_E* code; zero_last_error()
 *     then describes the failure (per calling thread).  Arguments are
 *     checked before any work is queued: a call that fails has queued
 *     nothing and touched no memory.
 *   - The caller owns every buffer.  No call allocates device memory.
 *     The one device array the library holds itself is the scratch
 *     workspace of zero_shard_step_noalloc (67,375,616 bytes per GPU,
 *     created with the library's code).  "device" pointers are HIP device
 *     addresses on the current device; "host" pointers are ordinary
 *     process memory.
 *   - `stream` is a hipStream_t passed as void* (NULL: the null stream).
 *     Device work is queued on it and the call returns without waiting,
 *     unless a call says otherwise.
 *   - Device pointers must be 16-byte aligned (ZERO_EALIGN otherwise).
 *   - Element counts are 64-bit; shards beyond 2^32 elements are fine.
 *   - Calls keep no state between them, except the scratch array of
 *     zero_shard_step_noalloc; concurrent calls on different buffers are
 *     safe.  Calls that write the same buffers race.
 *   - A call's inputs and outputs must not overlap, unless the call says
 *     that it updates a buffer in place.
 */
#ifndef ZERO_H
#define ZERO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZERO_OK        0
#define ZERO_EINVAL   (-1)   /* an argument is out of range or NULL        */
#define ZERO_EALIGN   (-2)   /* a device pointer is not 16-byte aligned    */
#define ZERO_ESIZE    (-3)   /* a caller buffer or table is too small      */
#define ZERO_EDEVICE  (-4)   /* the HIP runtime reported an error          */

/* Low-precision formats of gradients and working parameters: [P1] §3.3
 * enables either fp16 or bf16 mixed precision, never both. */
#define ZERO_FP16 1
#define ZERO_BF16 2
/* fp32 replica gradients: the buffers zero_accumulate_local fills when a
 * window of micro-batches is summed on each replica before the reduce.
 * Valid as zero_step_args.grad_dtype only. */
#define ZERO_FP32 3

/* Largest number of data-parallel replicas one reduce can sum. */
#define ZERO_MAX_REPLICAS 64

/* Layouts of a rank's fp32 optimizer state (zero_step_args.state_layout).
 * SEPARATE: three arrays master[s], exp_avg[s], exp_avg_sq[s].
 * TILED: one array of ceil(s / ZERO_STATE_TILE) tiles, tile k holding
 *   master, then exp_avg, then exp_avg_sq of elements
 *   [k*ZERO_STATE_TILE, (k+1)*ZERO_STATE_TILE), ZERO_STATE_TILE values each:
 *   element i's master is at (i / T) * 3T + i % T, its exp_avg T further
 *   and its exp_avg_sq 2T further (T = ZERO_STATE_TILE).  The update pass
 *   then moves two state streams instead of six. */
#define ZERO_STATE_SEPARATE 0
#define ZERO_STATE_TILED    1
#define ZERO_STATE_TILE     256

/* Thread-local text of the last failure on this thread ("" if none). */
const char* zero_last_error(void);

/* ------------------------------------------------------------------------
 * Partition.  [P1] §2.1 splits the parameters into N parts and lets each
 * GPU update only the optimizer state of its own part; [P1] §4.1 says ZeRO
 * cuts the flat parameter space rather than whole modules; [P3] (technical
 * insight) has each GPU keep only the matching gradient slice.
 *
 * shard_numel is the smallest multiple of `alignment` with
 * world_size * shard_numel >= numel; rank r owns flat elements
 * [r*shard_numel, (r+1)*shard_numel), of which the first
 * valid_numel(r) = clamp(numel - r*shard_numel, 0, shard_numel) are real and
 * the rest is padding at the end of the flat space.
 * Errors: numel < 0, world_size < 1, alignment < 1 or not a power of two,
 * a padded count beyond INT64_MAX, out == NULL -> ZERO_EINVAL.  Host only;
 * touches no device.
 */
typedef struct {
    int64_t numel;          /* real flat parameter count                  */
    int64_t shard_numel;    /* elements per rank, padding included        */
    int64_t padded_numel;   /* world_size * shard_numel                   */
    int32_t world_size;
    int32_t alignment;
} zero_partition_t;

int zero_partition(int64_t numel, int32_t world_size, int32_t alignment,
                   zero_partition_t* out);

/* Real (unpadded) element count of `rank`; -1 if rank is out of range. */
int64_t zero_partition_valid_numel(const zero_partition_t* p, int32_t rank);

/* ------------------------------------------------------------------------
 * Bucket plan.  [P1] §2.2: gradients travel in buckets whose size
 * (reduce_bucket_size) sets the communication granularity; [P1] §5.1 and §6
 * suggest 2e8 elements; [P1] §5.2 lists contiguous_gradients for memory
 * locality.
 *
 * Tensors are laid end to end in the given order with no gaps: tensor t
 * occupies flat [slots[t].offset, slots[t].offset + tensor_numel[t]).
 * Buckets are greedy runs of whole tensors holding at most
 * reduce_bucket_size elements; a larger tensor is a bucket of its own.
 * Host arrays: tensor_numel[n_tensors] (in), slots[n_tensors] (out),
 * buckets[bucket_cap] (out).  *n_buckets receives the bucket count; when it
 * exceeds bucket_cap the call fails with ZERO_ESIZE and *n_buckets holds the
 * capacity needed.  Errors: n_tensors < 0, a negative size, sizes summing
 * past INT64_MAX, reduce_bucket_size < 1, a NULL pointer -> ZERO_EINVAL.
 * Host only.
 */
typedef struct {
    int64_t offset;         /* first flat element of the tensor           */
    int64_t numel;
    int32_t bucket;         /* index of the bucket that holds it          */
    int32_t reserved;
} zero_tensor_slot_t;

typedef struct {
    int64_t begin;          /* flat range [begin, end) of the bucket      */
    int64_t end;
    int32_t first_tensor;
    int32_t n_tensors;
} zero_bucket_t;

int zero_bucket_plan(const int64_t* tensor_numel, int32_t n_tensors,
                     int64_t reduce_bucket_size, zero_tensor_slot_t* slots,
                     zero_bucket_t* buckets, int32_t bucket_cap,
                     int32_t* n_buckets);

/* ------------------------------------------------------------------------
 * Flatten one replica's gradients into its contiguous flat buffer
 * ([P1] §5.2 contiguous_gradients; buckets per [P1] §2.2).
 *
 * For each t < n_tensors, copies tensor_numel = slots[t].numel 16-bit
 * values from src_dev[t] (device, 2-byte aligned, any offset) to flat
 * elements [slots[t].offset, +numel) of flat_dev (device, 16-byte aligned),
 * writes zeros over any gap between the end of slot t - 1 and the start of
 * slot t, then over [end of the last slot, flat_numel) -- the partition
 * padding when flat_numel is the padded size.  Elements before the first
 * slot are not touched.  So every element the step may read, from the
 * first slot on, holds a gradient or zero.  slots (host) must have
 * non-decreasing, non-overlapping ranges inside [0, flat_numel); src_dev is
 * a host array of device pointers.  A bucket at a time may be flattened by
 * passing its slots and flat_numel = bucket end (no padding is then
 * written).  The sources must not overlap flat_dev.  Bit copy:
 * dtype (ZERO_FP16 / ZERO_BF16) is checked, the values are not
 * interpreted.
 * Errors: NULL pointers, bad dtype, slots out of order or out of range ->
 * ZERO_EINVAL; flat_dev misaligned -> ZERO_EALIGN; launch -> ZERO_EDEVICE.
 */
int zero_bucket_flatten(const zero_tensor_slot_t* slots, int32_t n_tensors,
                        const void* const* src_dev, int32_t dtype,
                        void* flat_dev, int64_t flat_numel, void* stream);

/* ------------------------------------------------------------------------
 * The shard step.
 *
 * (zero_step_scalars_t, below, may hold the step's scalars in device
 * memory; declared here so the arguments can point at it.) */
struct zero_step_scalars_s;

/*
 * Arguments of one rank's step.  Hyper-parameters follow [P1] §3.1 (AdamW,
 * lr 6e-5, weight_decay 0.01), [P1] §6 (gradient_clipping 1.0) and
 * [P1] §3.3 / §5.1 (fp16 loss scale); the fp32 master weights and two Adam
 * moments are the state [P3] (FAQ) and [P2] (memory arithmetic) describe.
 */
typedef struct {
    int32_t world_size;       /* ranks in the data-parallel world          */
    int32_t rank;             /* this rank, in [0, world_size)             */
    int64_t shard_numel;      /* from zero_partition                       */
    int64_t valid_numel;      /* real elements of this rank's shard        */
    int32_t grad_dtype;       /* ZERO_FP16, ZERO_BF16, or ZERO_FP32 for
                                 replicas summed by zero_accumulate_local */
    int32_t param_dtype;      /* ZERO_FP16 or ZERO_BF16, independent of
                                 grad_dtype: the decode follows grad_dtype,
                                 the cast param_dtype                     */
    int32_t n_replicas;       /* gradients summed, 1..ZERO_MAX_REPLICAS    */
    /* 0: pass 1 sets the workspace's fp32 gradient slice to this reduce's
     * result; 1: it adds the result to the slice already there (micro-batch
     * 2..K of a gradient-accumulation window, see zero_shard_accumulate).  */
    int32_t accumulate;
    /* host array of n_replicas device pointers; entry i points at this
     * rank's slice (flat element rank*shard_numel) of replica i's flat
     * gradient buffer.  valid_numel values are read from each.            */
    const void* const* replica_grad;
    float* master;            /* device fp32[shard_numel], updated in place */
    float* exp_avg;           /* device fp32[shard_numel], Adam m           */
    float* exp_avg_sq;        /* device fp32[shard_numel], Adam v           */
    /* device buffer of world_size*shard_numel param_dtype values; this rank
     * writes elements [rank*shard_numel, rank*shard_numel + valid_numel).  */
    void* full_params;
    void* workspace;          /* device, zero_shard_workspace_bytes() long  */
    size_t workspace_bytes;
    double lr, beta1, beta2, eps, weight_decay;
    int64_t step;             /* t of this update, >= 1; advance it only
                                 after a step that was not skipped         */
    double loss_scale;        /* S > 0: gradients hold S * dL/dw           */
    double grad_predivide;    /* D > 0: the sum is divided by S*D          */
    double max_grad_norm;     /* <= 0 disables clipping                    */
    /* ZeRO-3 ([P1] §1.2.3, [P2] stage table): the rank keeps only its own
     * shard of the low-precision parameters.  When not NULL the cast goes
     * to param_shard[0, valid_numel) (device, 16-byte aligned) and
     * full_params is not used (may be NULL); zero_gather_params collects a
     * layer's parameters from all ranks' shards before its forward.       */
    void* param_shard;
    /* Optional second set of state buffers (device, fp32[shard_numel], 16-byte
     * aligned, not overlapping master / exp_avg / exp_avg_sq): when all three
     * are set, pass 2 reads the state from master, exp_avg, exp_avg_sq and
     * writes the new state here instead of in place; a caller alternating
     * two sets ("ping-pong") saves the in-place read-modify-write.  All NULL:
     * in place.  Not used by zero_offload_apply (must be NULL there).      */
    float* master_out;
    float* exp_avg_out;
    float* exp_avg_sq_out;
    /* ZERO_STATE_SEPARATE (0) or ZERO_STATE_TILED.  Tiled: `master` is the
     * rank's tiled state (fp32[3 * ZERO_STATE_TILE * ceil(shard_numel /
     * ZERO_STATE_TILE)], 16-byte aligned) and exp_avg, exp_avg_sq must be
     * NULL; the optional second set is master_out alone (tiled too), with
     * exp_avg_out and exp_avg_sq_out NULL.  zero_state_tile and
     * zero_state_untile convert between the layouts. */
    int32_t state_layout;
    int32_t reserved;         /* 0 */
    /* Optional device copy of the step's scalars (zero_step_scalars_t,
     * 16-byte aligned), for HIP graphs replayed across steps.  NULL: the
     * kernels take the scalars above as launch arguments, fixed when a
     * graph is captured.  Set: the reduce reads its unscale multiplier, the
     * AdamW pass its constants and zero_shard_step's combine its clip
     * threshold and peer values from this buffer when they run, so a
     * captured step replays with whatever the caller last wrote there
     * (zero_step_scalars fills it on the host).  The fields above are still
     * checked.  zero_offload_apply does not read it. */
    const struct zero_step_scalars_s* scalars;
} zero_step_args;

/* Result of the cross-rank combine, 32 bytes in device memory. */
typedef struct {
    double  sumsq;            /* sum of squares of the unscaled gradient    */
    double  norm;             /* sqrt(sumsq)                                */
    float   coef;             /* clip factor applied to the gradient (1: none) */
    int32_t overflow;         /* 1: some gradient was inf/nan; step skipped */
    int32_t clipped;          /* 1: coef < 1 was applied                    */
    int32_t reserved;
} zero_global_t;

typedef zero_global_t zero_step_info;

/* Bytes of workspace a rank needs: the fp32 reduced gradient of its shard
 * (shard_numel * 4, rounded up to 256), one 16-byte partial sum of squares
 * and flag per block of the reduce pass (1024 elements each; the block
 * count is rounded up to a multiple of 8, or of 2048 for large shards, so
 * that every XCD gets whole runs), one partials slot (see
 * zero_partials_bytes) and one zero_global_t.  Host only. */
size_t zero_shard_workspace_bytes(int64_t shard_numel);

/* Bytes of the partials table zero_shard_reduce / zero_shard_combine share
 * for n_slots ranks: per slot a 16-byte header and at most 256 partial sums
 * of squares (fp64) with their flags, whatever the shard size.  Host only. */
size_t zero_partials_bytes(int32_t n_slots);

/* Pass 1 of a rank's step, for worlds simulated in one process.
 * [P1] §2.1, [P3] technical insight: the reduce-scatter leaves each rank the
 * sum over replicas of its own gradient slice.  For i < valid_numel:
 *   acc  = g_0[i] + g_1[i] + ... + g_{R-1}[i]   (fp32, replica order)
 *   g[i] = acc * fp32(1 / (loss_scale * grad_predivide))
 * stored as fp32 at the start of a->workspace, with one fp64 sum of g^2 and
 * one inf/nan flag per 1024 elements after it; then folds those, in a fixed
 * order, into at most 256 partials in slot `slot` of partials_dev (device,
 * zero_partials_bytes(n_slots) long).  Every partial sum, and hence the
 * norm, depends only on the values and valid_numel: the result is the same
 * from run to run.
 * Errors: as zero_shard_step; slot < 0 -> ZERO_EINVAL. */
int zero_shard_reduce(const zero_step_args* a, int32_t slot,
                      void* partials_dev, void* stream);

/* Gradient accumulation over micro-batches: [P1] §3.1 configuration
 * (gradient_accumulation_steps), [P2] practice notes (accumulating small
 * batches stands in for a large one), [P3] technical insight (each GPU keeps
 * only the gradient slice of its own parameters).  Every micro-batch is
 * reduced over the replicas as in zero_shard_reduce, and the rank's fp32
 * slice in the workspace accumulates them: with a->accumulate = 0 the slice
 * is set, with 1 it becomes
 *   g[i] = g[i] + (g_0[i] + ... + g_{R-1}[i]) * fp32(1 / (loss_scale * grad_predivide))
 * This call runs that pass only, for the micro-batches before the last of a
 * window; the last one goes through zero_shard_step (or zero_shard_reduce,
 * combine and apply) with accumulate = 1, so that the norm, the overflow
 * flag, clipping and AdamW act on the accumulated slice.  The loss scale
 * must stay the same within a window.  Errors: as zero_shard_step. */
int zero_shard_accumulate(const zero_step_args* a, void* stream);

/* Gradient accumulation before the reduce: the other reading of
 * gradient_accumulation_steps ([P1] §3.1, §5.1), the pattern of [P1]
 * §1.2.2's no_sync snippet, where each replica keeps its micro-batch
 * gradients locally and the replicas are synchronised once per window.
 * Each replica sums its window into an fp32 buffer of its own:
 *   acc[i] = first ? x : acc[i] + x,   x = grad[i] widened to fp32 (exact)
 * for i in [0, n), in micro-batch order.  The step then reduces the
 * replicas' fp32 buffers: zero_step_args.grad_dtype = ZERO_FP32 with
 * replica_grad pointing at this rank's slice of each replica's acc.  The
 * loss scale must stay the same within a window; it is undone once, in the
 * reduce.  grad: device, n values of grad_dtype (ZERO_FP16 or ZERO_BF16);
 * acc: device fp32[n]; both 16-byte aligned and not overlapping; first is 0
 * or 1.  Asynchronous on `stream`.  Errors: n < 0, a NULL pointer when
 * n > 0, a bad dtype or first -> ZERO_EINVAL; misalignment -> ZERO_EALIGN. */
int zero_accumulate_local(const void* grad, int32_t grad_dtype, float* acc, int64_t n,
                          int32_t first, void* stream);

/* Combine slots [0, n_slots) of partials_dev in a fixed order into one
 * zero_global_t at global_dev (device): the global sum of squares and norm,
 * the overflow flag (any slot flagged, or a non-finite sum), and the clip
 * factor max_grad_norm / (norm + 1e-6), applied only when below 1 and
 * max_grad_norm > 0 ([P1] §6 gradient_clipping).  max_grad_norm is a
 * launch argument (fixed under graph capture). */
int zero_shard_combine(const void* partials_dev, int32_t n_slots,
                       double max_grad_norm, void* global_dev, void* stream);

/* Pass 2 of a rank's step.  Reads *global_dev; if its overflow flag is set
 * nothing is written (the skipped step of [P1] §3.3 / §5.1 loss scaling).
 * Otherwise for i < valid_numel, with g' = g * coef:
 *   m'  = b1 m + (1 - b1) g'
 *   v'  = b2 v + (1 - b2) g'^2
 *   p'  = p (1 - lr wd) - lr/(1 - b1^t) * m' / (sqrt(v')/sqrt(1 - b2^t) + eps)
 * (AdamW, [P1] §3.1; each GPU updates only its part, [P1] §2.1), all in
 * fp32, then full_params[rank*shard_numel + i] = round-to-nearest-even of p'
 * in param_dtype (the all-gather's contribution, [P1] §2.1). */
int zero_shard_apply(const zero_step_args* a, const void* global_dev,
                     void* stream);

/* One rank's whole step: zero_shard_reduce into the workspace, a combine
 * with the peers' contribution (peer_sumsq is the other ranks' total sum of
 * squares and peer_overflow their OR'd flag; 0 and 0 when this rank holds
 * the whole world or stands alone), then zero_shard_apply.
 * If info is not NULL the call waits for the stream and copies the
 * combine's result into *info (host); otherwise it does not wait.
 * Errors: world_size < 1, rank outside [0, world_size), valid_numel outside
 * [0, shard_numel], shard_numel not a multiple of 8, bad dtype, n_replicas
 * outside [1, ZERO_MAX_REPLICAS], accumulate not 0 or 1, step < 1, loss_scale or grad_predivide
 * <= 0, lr, betas or eps out of range, a NULL pointer -> ZERO_EINVAL; a
 * misaligned device pointer -> ZERO_EALIGN; workspace_bytes too small ->
 * ZERO_ESIZE; a HIP failure -> ZERO_EDEVICE.  When valid_numel is 0 the
 * rank touches no element and only the workspace must be given.
 * Graph capture: without info the call queues four kernels and nothing
 * else, so it can be captured in a HIP graph.  By default the step's
 * scalars (t, lr, betas, eps, weight decay, loss scale, predivide,
 * max_grad_norm, peer_sumsq, peer_overflow) travel as kernel arguments and
 * are fixed at capture: every replay uses the captured values.  With
 * a->scalars set, the kernels read them from that device buffer instead
 * (see zero_step_scalars), and one capture serves every step. */
int zero_shard_step(const zero_step_args* a, double peer_sumsq,
                    int32_t peer_overflow, zero_step_info* info, void* stream);

/* ------------------------------------------------------------------------
 * Step scalars in device memory.  Every per-step constant the kernels use,
 * computed on the host exactly as the kernels' launch arguments are (each
 * in fp64 from the step's hyper-parameters and rounded once to fp32), so a
 * step that reads them from device memory gives the same bits as one that
 * takes them as arguments.  A caller that captures the step in a HIP graph
 * points zero_step_args.scalars at a device copy, and before each replay
 * fills a host copy with zero_step_scalars (t, the learning rate and the
 * loss scale may all change) and copies it to the device.  64 bytes.
 * ([P1] §3.1 AdamW hyper-parameters, §3.3 / §5.1 loss scale, §6 clipping.)
 */
typedef struct zero_step_scalars_s {
    float   inv_scale;        /* fp32(1 / (loss_scale * grad_predivide))     */
    float   decay;            /* fp32(1 - lr * weight_decay)                 */
    float   beta1;            /* fp32(beta1)                                 */
    float   one_minus_beta1;  /* fp32(1 - beta1)                             */
    float   beta2;            /* fp32(beta2)                                 */
    float   one_minus_beta2;  /* fp32(1 - beta2)                             */
    float   step_size;        /* fp32(lr / (1 - beta1^t))                    */
    float   inv_sqrt_bc2;     /* fp32(1 / sqrt(1 - beta2^t))                 */
    float   eps;              /* fp32(eps)                                   */
    int32_t peer_overflow;    /* the peers' OR'd flag (zero_shard_step)      */
    int32_t reserved[2];      /* 0                                           */
    double  max_grad_norm;    /* <= 0 disables clipping                      */
    double  peer_sumsq;       /* the peers' sum of squares (zero_shard_step) */
} zero_step_scalars_t;

/* Fill *out from a's hyper-parameters (lr, betas, eps, weight_decay, step,
 * loss_scale, grad_predivide, max_grad_norm) and the peers' contribution.
 * Errors: any of them out of range (as zero_shard_step checks them), a
 * negative or NaN peer_sumsq, NULL arguments -> ZERO_EINVAL.  Host only. */
int zero_step_scalars(const zero_step_args* a, double peer_sumsq, int32_t peer_overflow,
                      zero_step_scalars_t* out);

/* ------------------------------------------------------------------------
 * The step without any allocation, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, and harnesses
 * that forbid hipMalloc.  It is zero_shard_step with the workspace taken
 * from a scratch array inside the library instead of from the caller: one
 * array of 67,375,616 bytes per GPU (the workspace of a
 * ZERO_NOALLOC_MAX_SHARD-element shard), created with the library's code
 * on each GPU that runs it and held until the process ends.  The call
 * itself allocates nothing (no hipMalloc, no allocating library routine).
 *
 * Arguments as zero_shard_step, except: a->workspace must be NULL and
 * a->workspace_bytes 0; a->accumulate must be 0 (the scratch keeps no
 * accumulation window between calls); shard_numel at most
 * ZERO_NOALLOC_MAX_SHARD.  Every call on one GPU uses that GPU's one array:
 * calls queued on one stream are ordered and safe, but two calls that may
 * run at the same time on one GPU (different streams, different host
 * threads) race on it and give wrong results.  The array keeps the last
 * call's contents; nothing in it has to start at zero, since every step
 * writes all it reads.  The first call on a device looks up the array's
 * address there.
 * Errors: as zero_shard_step; a non-NULL workspace or accumulate set ->
 * ZERO_EINVAL; shard_numel > ZERO_NOALLOC_MAX_SHARD -> ZERO_ESIZE; the
 * address lookup failing -> ZERO_EDEVICE. */
#define ZERO_NOALLOC_MAX_SHARD 16777216LL

int zero_shard_step_noalloc(const zero_step_args* a, double peer_sumsq, int32_t peer_overflow,
                            zero_step_info* info, void* stream);

/* ------------------------------------------------------------------------
 * Dynamic loss scaler for fp16 ([P1] §3.3: loss_scale_window 100,
 * hysteresis 2; [P1] §5.1: initial_scale_power 16, min_loss_scale 1).  The
 * pages give only these knobs; the rule is this library's reading:
 *   start:        scale = 2^initial_scale_power, good = 0, hyst = hysteresis
 *   overflow:     skip the step; good = 0; if hyst > 1 then hyst -= 1,
 *                 else scale = max(scale / 2, min_loss_scale)
 *   no overflow:  good += 1; when good == loss_scale_window:
 *                 scale *= 2, good = 0, hyst = hysteresis
 * The new scale applies to the next step's loss.  Host only.
 * Errors: NULL st, loss_scale_window < 1, hysteresis < 1,
 * min_loss_scale <= 0, initial_scale_power outside [-126, 127]
 * -> ZERO_EINVAL.
 */
typedef struct {
    double  scale;
    double  min_scale;
    int32_t good_steps;
    int32_t hysteresis_left;
    int32_t window;
    int32_t hysteresis;
} zero_loss_scaler_t;

int zero_loss_scaler_init(int32_t initial_scale_power, int32_t loss_scale_window,
                          int32_t hysteresis, double min_loss_scale,
                          zero_loss_scaler_t* st);

int zero_loss_scaler_update(zero_loss_scaler_t* st, int32_t overflow,
                            int32_t* skip_step);

/* ------------------------------------------------------------------------
 * ZeRO-3 parameter gather.  [P1] §1.2.3 (parameters themselves are
 * partitioned; sub_group_size, stage3_prefetch_bucket_size), [P2] (before a
 * layer's forward an all-gather fetches its parameters, which are freed
 * after), [P3] technical insight (the all-gather assembles the layer's full
 * parameters on every GPU, then the slices a GPU does not own are dropped).
 *
 * Copies flat parameters [lo, hi) of partition *p into dst[0, hi - lo)
 * (device, 16-byte aligned) from the ranks' shards: shards is a host array
 * of p->world_size device pointers, entry r holding rank r's shard of
 * 16-bit parameters (at least its valid elements; r * shard_numel is its
 * first flat element).  Only the shards [lo, hi) meets are read.  On one
 * GPU the shards may be slices of one buffer; across GPUs they would be
 * peer-mapped pointers.  dst must not overlap the shards.  Bit copy: dtype
 * is checked, values are not read.
 * Errors: NULL arguments, a partition that zero_partition does not
 * reproduce from its numel, world_size and alignment, lo < 0, hi < lo,
 * hi > numel, bad dtype, a NULL shard that [lo, hi) meets -> ZERO_EINVAL;
 * misaligned dst or shard -> ZERO_EALIGN; launch -> ZERO_EDEVICE. */
int zero_gather_params(const zero_partition_t* p, const void* const* shards, int32_t dtype,
                       int64_t lo, int64_t hi, void* dst, void* stream);

/* ------------------------------------------------------------------------
 * Optimizer step offloaded to the host CPU.  [P1] §1.2.3 and §3.1
 * configuration (offload_optimizer: device cpu, pin_memory true), §6
 * (ZeRO-3 with CPU offload fits 200B parameters on 8 A100s); [P3] real-world
 * implementations (ZeRO-Offload pushes optimizer state to CPU memory).
 *
 * The rank's fp32 master weights and both moments live in host memory
 * (pinned memory is strongly recommended: it makes the copies DMA).  Pass 1
 * and the combine still run on the GPU (zero_shard_reduce /
 * zero_shard_accumulate, zero_shard_combine); this call replaces
 * zero_shard_apply.  It reads the combine's result; if the step overflowed
 * it touches nothing.  Otherwise it streams the fp32 reduced gradient to
 * the host chunk by chunk, applies the same fp32 AdamW update as the GPU
 * pass (identical operations in identical order, so identical bits) on
 * the host's threads, and streams the cast parameters back into the rank's
 * slice of the device's full parameter buffer.  Device-to-host copies, host
 * arithmetic and host-to-device copies of neighbouring chunks overlap.
 * The call returns when everything is done (it waits for `stream`).
 */
typedef struct {
    void*   grad_stage[2];    /* host, chunk_elems * 4 bytes each (pinned)   */
    void*   param_stage[2];   /* host, chunk_elems * 2 bytes each (pinned)   */
    int64_t chunk_elems;      /* > 0, a multiple of 8                        */
    int32_t n_threads;        /* host threads; 0: zero_host_threads()        */
    int32_t reserved;
} zero_offload_staging_t;

/* a: as for zero_shard_apply (and checked the same way), except that
 * master, exp_avg and exp_avg_sq are HOST pointers (fp32[shard_numel],
 * updated in place; with a->state_layout ZERO_STATE_TILED, master is the
 * host tiled state and the other two are NULL); the replica pointers are
 * checked but not read.  global_dev: the combine's zero_global_t (device).  info, if
 * not NULL, receives it.  Errors: as zero_shard_apply; a NULL or short
 * staging buffer, chunk_elems not a positive multiple of 8 -> ZERO_EINVAL;
 * a HIP failure -> ZERO_EDEVICE. */
int zero_offload_apply(const zero_step_args* a, const void* global_dev,
                       const zero_offload_staging_t* staging, zero_step_info* info,
                       void* stream);

/* The host AdamW of zero_offload_apply on n elements, all pointers HOST:
 * for i < n, g' = g[i] * coef, then the update of zero_shard_apply on
 * master, exp_avg, exp_avg_sq (fp32, in place), and, if params_out is not
 * NULL, params_out[i] = round-to-nearest-even of the new master in
 * param_dtype.  Hyper-parameters as in zero_step_args; step is t >= 1.
 * n_threads 0 uses zero_host_threads().  Errors: n < 0, a NULL array
 * when n > 0, bad dtype or hyper-parameters -> ZERO_EINVAL.  Host only. */
int zero_host_adamw(int64_t n, const float* g, float coef, float* master, float* exp_avg,
                    float* exp_avg_sq, void* params_out, int32_t param_dtype, double lr,
                    double beta1, double beta2, double eps, double weight_decay,
                    int64_t step, int32_t n_threads);

/* The host thread count that n_threads = 0 selects: OMP_NUM_THREADS when it
 * is set to a positive number, else the number of CPUs the calling process
 * may run on (its affinity mask), else the hardware's thread count.  A
 * container whose CPU share is smaller than the host sets one of the first
 * two.  Never fails; at least 1. */
int32_t zero_host_threads(void);

/* ------------------------------------------------------------------------
 * Sharded checkpoint and resume.  [P2] practice notes: a sharded run must be
 * saved through the engine (engine.save_checkpoint()), because a plain
 * torch.save of the state dict loses the shard information.  Each rank
 * saves one file holding its part of the optimizer state together with the
 * partition it was cut by, so a run can resume on the same world or be
 * re-partitioned onto a different one.
 *
 * File layout (all little-endian), one file per rank:
 *   bytes [0, 128)                          zero_ckpt_header_t
 *   then valid_numel fp32 values each of    master, exp_avg, exp_avg_sq
 * Element e of the rank's slice is flat parameter rank*shard_numel + e.
 */
#define ZERO_CKPT_MAGIC   0x3143535AU   /* "ZSC1" */
#define ZERO_CKPT_VERSION 1

typedef struct {
    uint32_t magic;           /* ZERO_CKPT_MAGIC                            */
    uint32_t version;         /* ZERO_CKPT_VERSION                          */
    int64_t  numel;           /* flat parameter count of the run            */
    int64_t  shard_numel;     /* elements per rank, padding included        */
    int64_t  valid_numel;     /* real elements saved for this rank          */
    int32_t  world_size;
    int32_t  rank;
    int32_t  alignment;
    int32_t  param_dtype;     /* ZERO_FP16 or ZERO_BF16                     */
    int64_t  step;            /* optimizer steps applied; next t = step + 1 */
    int32_t  has_scaler;      /* 1: the scaler fields below are in use      */
    int32_t  reserved0;
    zero_loss_scaler_t scaler;
    uint64_t payload_bytes;   /* 3 * valid_numel * 4                        */
    uint8_t  pad[24];         /* zero; the header is 128 bytes            */
} zero_ckpt_header_t;

/* Fill *out for `rank` of partition *p.  scaler may be NULL (bf16 runs).
 * Errors: NULL p or out, rank out of range, bad dtype, step < 0 ->
 * ZERO_EINVAL.  Host only. */
int zero_ckpt_header_make(const zero_partition_t* p, int32_t rank, int32_t param_dtype,
                          int64_t step, const zero_loss_scaler_t* scaler,
                          zero_ckpt_header_t* out);

/* Check a header read from a file of file_bytes bytes: magic, version, a
 * partition that zero_partition reproduces from (numel, world_size,
 * alignment), the rank's valid count and the payload size.  On success
 * *part receives that partition (may be NULL).  Errors: anything
 * inconsistent -> ZERO_EINVAL; a short file -> ZERO_ESIZE.  Host only. */
int zero_ckpt_header_check(const zero_ckpt_header_t* h, uint64_t file_bytes,
                           zero_partition_t* part);

/* Re-partition one fp32 state array (master, exp_avg or exp_avg_sq) from
 * partition *from to partition *to of the same numel: the elastic resume
 * of a checkpoint on a different world size.  src_dev is a host array of
 * from->world_size device pointers, entry k holding old rank k's slice
 * (at least its valid elements); dst_dev is a host array of
 * to->world_size device pointers to new slices of to->shard_numel
 * elements each (16-byte aligned).  Every flat element i < numel is copied
 * from old rank i / from->shard_numel to new rank i / to->shard_numel; the
 * new slices' padding is zeroed.  Source and destination must not
 * overlap.  Device work only, queued on `stream`; the copies follow
 * zero_repartition_plan.
 * Errors: NULL arguments, different numel, a partition that zero_partition
 * does not reproduce from its numel, world_size and alignment, a NULL
 * pointer for a rank that holds elements -> ZERO_EINVAL; misaligned
 * pointers -> ZERO_EALIGN; launch -> ZERO_EDEVICE. */
int zero_repartition(const zero_partition_t* from, const float* const* src_dev,
                     const zero_partition_t* to, float* const* dst_dev, void* stream);

/* Layout conversion of a rank's optimizer state (ZERO_STATE_SEPARATE <->
 * ZERO_STATE_TILED; the layouts are described at ZERO_STATE_TILE).
 * zero_state_tile: for i in [0, n), element first + i of the tiled array
 * `tiled` receives master[i], exp_avg[i] and exp_avg_sq[i];
 * zero_state_untile: the reverse, element first + i of `tiled` into
 * master[i], exp_avg[i], exp_avg_sq[i].  A rank's whole state is n =
 * shard_numel, first = 0; a chunk at a time is fine (checkpoints do that).
 * The separate arrays hold n values each; `tiled` holds at least the whole
 * tiles of elements [0, first + n), 3 * ZERO_STATE_TILE * ceil((first + n)
 * / ZERO_STATE_TILE) values.  Bit copies; device pointers (16-byte
 * aligned), asynchronous on `stream`; the two sides must not overlap.
 * Tile slots of elements outside [first, first + n) are not touched.
 * Errors: n < 0, first < 0, a NULL pointer when n > 0 -> ZERO_EINVAL;
 * misalignment -> ZERO_EALIGN; launch -> ZERO_EDEVICE. */
int zero_state_tile(const float* master, const float* exp_avg, const float* exp_avg_sq, int64_t n,
                    float* tiled, int64_t first, void* stream);
int zero_state_untile(const float* tiled, int64_t first, int64_t n, float* master, float* exp_avg,
                      float* exp_avg_sq, void* stream);

/* zero_repartition for a ZERO_STATE_TILED state: all three fields of the
 * state move at once.  src_dev[k] is old rank k's tiled state, dst_dev[j]
 * new rank j's (to->shard_numel elements' worth of whole tiles, 16-byte
 * aligned); the new ranks' padding elements are zeroed in all three fields.
 * The copies follow zero_repartition_plan.  Errors as zero_repartition
 * ([P2] practice notes: a run resumes under another world size). */
int zero_repartition_tiled(const zero_partition_t* from, const float* const* src_dev,
                           const zero_partition_t* to, float* const* dst_dev, void* stream);

/* Where new rank `new_rank` of partition *to finds its real elements under
 * partition *from of the same numel: the read plan of an elastic resume
 * ([P2] practice notes: the saved shard information lets a run continue
 * on another world).  zero_repartition copies along these pieces on the
 * device; a checkpoint reader follows them to seek in the old ranks' files.
 *
 * Piece q moves `count` elements from element old_offset of old rank
 * old_rank's slice to element new_offset of the new rank's slice.  The
 * pieces come in ascending new_offset, old_rank and new_offset both
 * increase from piece to piece, and together they cover the new rank's
 * real elements [0, valid_numel) exactly once; each lies inside its old
 * rank's real elements.  The new rank's padding [valid_numel, shard_numel)
 * is in no piece (a reader zeroes it).  At most from->world_size pieces.
 * pieces: host array of piece_cap entries (out); *n_pieces receives the
 * count (0 for a rank with no real elements).  When it exceeds piece_cap
 * the call fails with ZERO_ESIZE and *n_pieces holds the capacity needed.
 * Errors: NULL from, to or n_pieces, pieces NULL with piece_cap > 0,
 * piece_cap < 0, a partition that zero_partition does not reproduce from
 * its numel, world_size and alignment, different numel, new_rank out of
 * range -> ZERO_EINVAL.  Host only. */
typedef struct {
    int64_t old_offset;       /* first element, inside the old rank's slice */
    int64_t new_offset;       /* first element, inside the new rank's slice */
    int64_t count;            /* elements, > 0                               */
    int32_t old_rank;         /* rank of *from whose slice holds them        */
    int32_t reserved;         /* 0                                           */
} zero_repartition_piece_t;

int zero_repartition_plan(const zero_partition_t* from, const zero_partition_t* to,
                          int32_t new_rank, zero_repartition_piece_t* pieces,
                          int32_t piece_cap, int32_t* n_pieces);

#ifdef __cplusplus
}
#endif
#endif /* ZERO_H */
