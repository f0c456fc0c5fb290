/*
 * zero_oracle.h -- CPU oracle for the per-rank ZeRO sharded-optimizer step.
 *
 * TEST INFRASTRUCTURE ONLY.  This is a plain, slow, single-threaded C
 * implementation of what the step computes, used to check the HIP library.
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load it.  It shares no code, header, table or constant with the HIP path.
 *
 * Sources (three web pages on ZeRO, cited by title and section):
 *   [P1] "ZeRO技术解析：大模型分布式训练的革命性突破" (intelliparadigm.com)
 *   [P2] "大模型分片训练：ZeRO-3策略在PyTorch中的实现" (dn008.com.cn),
 *        no section numbers: cited by passage topic
 *   [P3] "ZeRO 和分片优化器" (aiunderstanding.org)
 *
 * Precision.  Where the pages fix a precision it is kept: fp32 master
 * weights and fp32 Adam moments ([P3] FAQ on Adam state; [P2] memory
 * arithmetic for a d_model=4096 layer, which counts weights, gradients,
 * momentum and variance at 4 bytes each), fp16/bf16 gradients and working
 * parameters ([P1] §3.3).  So the reduced gradient partition and the AdamW
 * update are evaluated in fp32, one IEEE operation at a time in the order
 * written below; the reduce is the fp32 running sum in replica order, so the
 * overflow decision is taken in fp32 too.  What the pages leave open in
 * precision (the norm, the clip factor, the update's scalar constants) is
 * computed in fp64 and rounded once where it enters fp32 arithmetic.
 * Parity status of each function:
 *   oracle_partition, oracle_bucket_plan      pinned (brute force, page numbers)
 *   oracle_*_to_f32, oracle_f32_to_*          pinned (decoders exhaustive against
 *                                             numpy / torch; encoders exhaustive
 *                                             over all 2^32 fp32 patterns against
 *                                             an integer reference written from
 *                                             the IEEE-754 definition)
 *   oracle_reduce                             pinned (identity, N*g, fsum)
 *   oracle_reduce_accumulate                  pinned (numpy fp32 sum over
 *                                             micro-batches, one micro-batch,
 *                                             sign of zero)
 *   oracle_accumulate_local, oracle_reduce_f32
 *                                             pinned (numpy fp32 sums, closed
 *                                             form, a hand-rounded example
 *                                             that separates the two orders)
 *   oracle_clip                               pinned (library clip, closed form)
 *   oracle_adamw                              pinned (closed form, library AdamW)
 *   oracle_scaler_*                           parity unpinned by the pages:
 *       the pages give only the knob names and values; the update rule is a
 *       stated reading, checked against hand-traced sequences of that reading.
 */
#ifndef ZERO_ORACLE_H
#define ZERO_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_FP16 = 1, ORACLE_BF16 = 2 };

/* ---- partition ([P1] §2.1; [P3] technical-insight section) ------------ */
/* Smallest multiple of `alignment` that, times world_size, covers numel.
 * Writes shard size, padded size and each rank's count of real elements.
 * Returns 0, or -1 on invalid input. */
int oracle_partition(int64_t numel, int32_t world_size, int32_t alignment,
                     int64_t* shard_numel, int64_t* padded_numel,
                     int64_t* valid_per_rank /* world_size entries or NULL */);

/* ---- gradient buckets ([P1] §2.2, §5.1, §5.2) --------------------------- */
/* Tensors are laid end to end in the given order (contiguous gradients);
 * buckets are greedy runs of whole tensors holding at most bucket_size
 * elements; a tensor larger than bucket_size is a bucket of its own.
 * Returns the bucket count, or -1 on invalid input. */
int32_t oracle_bucket_plan(const int64_t* tensor_numel, int32_t n_tensors,
                           int64_t bucket_size, int64_t* offset,
                           int32_t* bucket_of);

/* ---- number formats ([P1] §3.3: fp16 or bf16 mixed precision) --------- */
float    oracle_f16_to_f32(uint16_t h);
float    oracle_bf16_to_f32(uint16_t b);
uint16_t oracle_f32_to_f16(float x);   /* round to nearest, ties to even */
uint16_t oracle_f32_to_bf16(float x);  /* round to nearest, ties to even */
void oracle_f32_to_f16_array(int64_t n, const float* x, uint16_t* out);
void oracle_f32_to_bf16_array(int64_t n, const float* x, uint16_t* out);
void oracle_f16_to_f32_array(int64_t n, const uint16_t* h, float* out);
void oracle_bf16_to_f32_array(int64_t n, const uint16_t* b, float* out);

/* ---- replica reduce, unscale, overflow, sum of squares ----------------- *
 * [P1] §2.1 and [P3] technical insight: gradients are reduce-scattered, so a
 * rank keeps the sum over replicas of its own slice.  [P1] §3.3, §5.1: loss
 * scaling, so the sum is divided by the scale.  For i in [0, n):
 *   acc  = replica[0][i] + replica[1][i] + ... (fp32, left to right)
 *   g[i] = acc * inv_scale                       (fp32)
 *   *overflow |= g[i] is inf or nan
 *   *sumsq    += (double)g[i] * (double)g[i]     (fp64, index order)
 * `replicas` holds n_replicas pointers to n 16-bit values each. */
void oracle_reduce(int32_t n_replicas, const uint16_t* const* replicas,
                   int32_t dtype, int64_t n, float inv_scale, float* g,
                   double* sumsq, int32_t* overflow);

/* ---- gradient accumulation over micro-batches --------------------------- *
 * [P1] §3.1 configuration (gradient_accumulation_steps), [P2] practice notes
 * (accumulation stands in for a larger batch), [P3] technical insight (each
 * GPU keeps only the gradient slice of its own parameters).  Reading: every
 * micro-batch is reduce-scattered, and the rank accumulates its own slice in
 * fp32.  For micro-batch 2..K of a window, for i in [0, n):
 *   acc  = replica[0][i] + replica[1][i] + ... (fp32, left to right)
 *   g[i] = g[i] + acc * inv_scale                (fp32, g read and written)
 *   *overflow |= g[i] is inf or nan
 *   *sumsq    += (double)g[i] * (double)g[i]     (fp64, index order)
 * Micro-batch 1 is oracle_reduce, which sets g.  The flags and sums of the
 * last micro-batch are the ones the step uses. */
void oracle_reduce_accumulate(int32_t n_replicas, const uint16_t* const* replicas,
                              int32_t dtype, int64_t n, float inv_scale, float* g,
                              double* sumsq, int32_t* overflow);

/* ---- gradient accumulation before the reduce ----------------------------- *
 * The other reading of gradient_accumulation_steps ([P1] §3.1, §5.1), the
 * pattern of [P1] §1.2.2's no_sync snippet: each replica keeps the
 * gradients of its micro-batches locally, summed in an fp32 buffer of its
 * own, and the gradients are synchronised once per window.  For i in [0, n):
 *   acc[i] = first ? x : acc[i] + x     (fp32), x = grad[i] widened to fp32
 * The reduce then sums the replicas' fp32 buffers with oracle_reduce_f32. */
void oracle_accumulate_local(int32_t dtype, int64_t n, const uint16_t* grad, float* acc,
                             int32_t first);

/* oracle_reduce over fp32 replica buffers (those oracle_accumulate_local
 * fills): the same running sum in replica order, unscale, flag and fp64 sum
 * of squares. */
void oracle_reduce_f32(int32_t n_replicas, const float* const* replicas, int64_t n,
                       float inv_scale, float* g, double* sumsq, int32_t* overflow);

/* ---- gradient clipping ([P1] §6 configuration: gradient_clipping 1.0) --- *
 * norm = sqrt(sumsq); coef = max_norm / (norm + 1e-6); the gradient is
 * scaled by coef only when max_norm > 0 and coef < 1.  Returns 1 when
 * clipping applies and writes the norm and the factor (1.0 otherwise). */
int32_t oracle_clip(double sumsq, double max_norm, double* norm, double* coef);

/* ---- AdamW ([P1] §3.1: AdamW, lr 6e-5, weight_decay 0.01) -------------- *
 * Decoupled weight decay, bias-corrected moments, t is 1-based:
 *   g'  = g * coef
 *   m'  = b1 m + (1 - b1) g'
 *   v'  = b2 v + (1 - b2) g'^2
 *   p'  = p (1 - lr wd) - lr/(1-b1^t) * m' / (sqrt(v') / sqrt(1-b2^t) + eps)
 * evaluated in fp32 in the order given in zero_oracle.c, with the scalar
 * factors computed in fp64 and rounded once to fp32.  coef is the clip
 * factor (1.0 when clipping does not apply). */
void oracle_adamw(int64_t n, const float* g, float* p, float* m, float* v,
                  double coef, double lr, double beta1, double beta2,
                  double eps, double weight_decay, int64_t t);

/* ---- dynamic loss scaler ([P1] §3.3 and §5.1 knobs) --------------------- *
 * Parity unpinned by the pages: the rule below is a reading.
 *   start: scale = 2^initial_scale_power, good = 0, hyst = hysteresis
 *   overflow: skip the step, good = 0; if hyst > 1 then hyst -= 1,
 *             else scale = max(scale / 2, min_scale)
 *   no overflow: good += 1; when good reaches window: scale *= 2, good = 0,
 *                hyst = hysteresis */
typedef struct {
    double  scale;
    int32_t good;
    int32_t hyst;
    int32_t window;
    int32_t hysteresis;
    double  min_scale;
} oracle_scaler;

void    oracle_scaler_init(oracle_scaler* s, int32_t initial_scale_power,
                           int32_t window, int32_t hysteresis,
                           double min_scale);
int32_t oracle_scaler_update(oracle_scaler* s, int32_t overflow); /* skip */

#ifdef __cplusplus
}
#endif
#endif
