/*
 * zero_oracle.c -- CPU oracle for the per-rank ZeRO sharded-optimizer step.
 *
 * TEST INFRASTRUCTURE ONLY (see zero_oracle.h).  Plain scalar loops,
 * single-threaded, built with gcc -O2 -ffp-contract=off and no fast-math so
 * that every fp32 and fp64 operation below is one IEEE-754 operation in the
 * order written.  Nothing here is shared with the HIP library.
 */
#include "zero_oracle.h"

#include <math.h>
#include <stddef.h>

/* ------------------------------------------------------------------------ */
/* Partition.  [P1] §2.1: the parameters are cut into N parts, one per GPU,
 * and each GPU updates only the optimizer state of its own part; [P1] §4.1:
 * ZeRO cuts the flat parameter space, not module by module.  Equal parts,
 * the padding at the end, the part size a multiple of `alignment`.        */
int oracle_partition(int64_t numel, int32_t world_size, int32_t alignment,
                     int64_t* shard_numel, int64_t* padded_numel,
                     int64_t* valid_per_rank)
{
    if (numel < 0 || world_size < 1 || alignment < 1) return -1;
    /* ceil(numel / N) elements per rank, then up to the next multiple of
     * the alignment: the smallest aligned s with N * s >= numel. */
    int64_t per_rank = numel / world_size + (numel % world_size != 0 ? 1 : 0);
    int64_t s = (per_rank + alignment - 1) / alignment * alignment;
    *shard_numel = s;
    *padded_numel = s * (int64_t)world_size;
    if (valid_per_rank) {
        for (int32_t r = 0; r < world_size; ++r) {
            int64_t left = numel - (int64_t)r * s;
            if (left < 0) left = 0;
            if (left > s) left = s;
            valid_per_rank[r] = left;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Buckets.  [P1] §2.2: the reduce bucket size sets how much gradient each
 * communication carries; [P1] §5.2: contiguous gradients for memory
 * locality.  Offsets are the running total of the sizes in order.        */
int32_t oracle_bucket_plan(const int64_t* tensor_numel, int32_t n_tensors,
                           int64_t bucket_size, int64_t* offset,
                           int32_t* bucket_of)
{
    if (n_tensors < 0 || bucket_size < 1) return -1;
    int64_t running = 0;
    int64_t filled = 0;          /* elements already in the open bucket */
    int32_t bucket = -1;         /* index of the open bucket, none yet  */
    for (int32_t t = 0; t < n_tensors; ++t) {
        int64_t n = tensor_numel[t];
        if (n < 0) return -1;
        offset[t] = running;
        running += n;
        int need_new = (bucket < 0) || (filled > 0 && filled + n > bucket_size);
        if (need_new) {
            bucket += 1;
            filled = 0;
        }
        bucket_of[t] = bucket;
        filled += n;
    }
    return bucket + 1;
}

/* ------------------------------------------------------------------------ */
/* Number formats, from the IEEE-754 binary16 layout (1 sign, 5 exponent,
 * 10 fraction bits, bias 15) and the bfloat16 layout (1 sign, 8 exponent,
 * 7 fraction bits, bias 127).  Values are built with ldexp in fp64, which
 * is exact for every one of them, then narrowed to fp32 (also exact).     */
float oracle_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double mag;
    if (e == 0)
        mag = ldexp((double)f, -24);               /* zero and subnormals */
    else if (e == 31)
        mag = (f != 0) ? NAN : INFINITY;
    else
        mag = ldexp((double)(1024 + f), e - 25);   /* (1 + f/2^10) 2^(e-15) */
    return (float)(sign ? -mag : mag);
}

float oracle_bf16_to_f32(uint16_t b)
{
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 0xff;
    int f = b & 0x7f;
    double mag;
    if (e == 0)
        mag = ldexp((double)f, -133);              /* f/2^7 * 2^-126 */
    else if (e == 255)
        mag = (f != 0) ? NAN : INFINITY;
    else
        mag = ldexp((double)(128 + f), e - 134);   /* (1 + f/2^7) 2^(e-127) */
    return (float)(sign ? -mag : mag);
}

/* Round |x| to the grid of a format with `frac_bits` fraction bits and
 * smallest exponent `emin` (normal numbers), ties to even.  The grid step
 * for a value in [2^k, 2^(k+1)) is 2^(k - frac_bits), never finer than the
 * subnormal step 2^(emin - frac_bits).  Returns the rounded magnitude.    */
static double round_to_format(double a, int frac_bits, int emin)
{
    int e;
    (void)frexp(a, &e);                   /* a in [2^(e-1), 2^e) */
    int q = (e - 1) - frac_bits;
    if (q < emin - frac_bits) q = emin - frac_bits;
    double units = ldexp(a, -q);          /* exact: a has 24 significant bits */
    double r = nearbyint(units);          /* default mode: nearest, ties even */
    return ldexp(r, q);
}

/* Encode a magnitude that is exactly representable in the format. */
static uint16_t encode_format(double y, int frac_bits, int emin, int bias)
{
    if (y == 0.0) return 0;
    double min_normal = ldexp(1.0, emin);
    if (y < min_normal)
        return (uint16_t)ldexp(y, -(emin - frac_bits)); /* subnormal code */
    int e;
    (void)frexp(y, &e);
    int k = e - 1;                                      /* y in [2^k, 2^(k+1)) */
    double frac = ldexp(y, -k) - 1.0;                   /* in [0, 1) */
    uint16_t fbits = (uint16_t)ldexp(frac, frac_bits);
    return (uint16_t)(((k + bias) << frac_bits) | fbits);
}

uint16_t oracle_f32_to_f16(float x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x)) return (uint16_t)(sign | 0x7e00);
    if (isinf(x)) return (uint16_t)(sign | 0x7c00);
    double a = fabs((double)x);
    if (a == 0.0) return sign;
    double y = round_to_format(a, 10, -14);
    if (y > 65504.0) return (uint16_t)(sign | 0x7c00);  /* largest finite */
    return (uint16_t)(sign | encode_format(y, 10, -14, 15));
}

uint16_t oracle_f32_to_bf16(float x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x)) return (uint16_t)(sign | 0x7fc0);
    if (isinf(x)) return (uint16_t)(sign | 0x7f80);
    double a = fabs((double)x);
    if (a == 0.0) return sign;
    double y = round_to_format(a, 7, -126);
    double max_finite = ldexp(255.0, 120);              /* (2 - 2^-7) 2^127 */
    if (y > max_finite) return (uint16_t)(sign | 0x7f80);
    return (uint16_t)(sign | encode_format(y, 7, -126, 127));
}

/* Every 16-bit code decoded once, by the functions above, when the library
 * loads; the reduce looks values up here.  The tables hold exactly what the
 * decoders return, so they change nothing but the speed. */
static float f16_value[65536];
static float bf16_value[65536];

__attribute__((constructor)) static void build_decode_tables(void)
{
    for (uint32_t c = 0; c < 65536u; ++c) {
        f16_value[c] = oracle_f16_to_f32((uint16_t)c);
        bf16_value[c] = oracle_bf16_to_f32((uint16_t)c);
    }
}

void oracle_f32_to_f16_array(int64_t n, const float* x, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_f16(x[i]);
}

void oracle_f32_to_bf16_array(int64_t n, const float* x, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_bf16(x[i]);
}

void oracle_f16_to_f32_array(int64_t n, const uint16_t* h, float* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = f16_value[h[i]];
}

void oracle_bf16_to_f32_array(int64_t n, const uint16_t* b, float* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_value[b[i]];
}

/* ------------------------------------------------------------------------ */
/* Replica reduce.  [P1] §2.1: gradients are reduce-scattered in backward;
 * [P3] technical insight: each GPU keeps only the gradient slice that
 * matches the parameters it owns.  The sum over replicas is the fp32
 * running sum in replica order; [P1] §3.3 / §5.1 loss scaling is undone by
 * one fp32 multiply; the overflow test and the fp64 sum of squares follow. */
void oracle_reduce(int32_t n_replicas, const uint16_t* const* replicas,
                   int32_t dtype, int64_t n, float inv_scale, float* g,
                   double* sumsq, int32_t* overflow)
{
    const float* value = (dtype == ORACLE_FP16) ? f16_value : bf16_value;
    double ss = *sumsq;
    int32_t bad = *overflow;
    for (int64_t i = 0; i < n; ++i) {
        float acc = 0.0f;
        for (int32_t r = 0; r < n_replicas; ++r) {
            float x = value[replicas[r][i]];
            acc = (r == 0) ? x : acc + x;
        }
        float gi = acc * inv_scale;
        g[i] = gi;
        if (!isfinite(gi)) bad = 1;
        ss += (double)gi * (double)gi;
    }
    *sumsq = ss;
    *overflow = bad;
}

/* ------------------------------------------------------------------------ */
/* Gradient accumulation.  [P1] §3.1 lists gradient_accumulation_steps; [P2]
 * practice notes: accumulation simulates a large batch with small ones;
 * [P3] technical insight: each GPU keeps only the gradient slice of its own
 * parameters, so the accumulated gradient is the rank's slice.  Each later
 * micro-batch's reduced, unscaled slice is added to the running fp32 slice;
 * the flag and the sum of squares are those of the updated slice.        */
void oracle_reduce_accumulate(int32_t n_replicas, const uint16_t* const* replicas,
                              int32_t dtype, int64_t n, float inv_scale, float* g,
                              double* sumsq, int32_t* overflow)
{
    const float* value = (dtype == ORACLE_FP16) ? f16_value : bf16_value;
    double ss = *sumsq;
    int32_t bad = *overflow;
    for (int64_t i = 0; i < n; ++i) {
        float acc = 0.0f;
        for (int32_t r = 0; r < n_replicas; ++r) {
            float x = value[replicas[r][i]];
            acc = (r == 0) ? x : acc + x;
        }
        float gi = g[i] + acc * inv_scale;
        g[i] = gi;
        if (!isfinite(gi)) bad = 1;
        ss += (double)gi * (double)gi;
    }
    *sumsq = ss;
    *overflow = bad;
}

/* ------------------------------------------------------------------------ */
/* Accumulation before the reduce ([P1] §1.2.2 no_sync pattern, §3.1
 * gradient_accumulation_steps): a replica's micro-batch gradients are
 * widened and summed into its own fp32 buffer in micro-batch order; the
 * first micro-batch of a window sets the buffer.                         */
void oracle_accumulate_local(int32_t dtype, int64_t n, const uint16_t* grad, float* acc,
                             int32_t first)
{
    const float* value = (dtype == ORACLE_FP16) ? f16_value : bf16_value;
    for (int64_t i = 0; i < n; ++i) {
        float x = value[grad[i]];
        acc[i] = first ? x : acc[i] + x;
    }
}

/* The replica reduce of oracle_reduce, on fp32 replica buffers.           */
void oracle_reduce_f32(int32_t n_replicas, const float* const* replicas, int64_t n,
                       float inv_scale, float* g, double* sumsq, int32_t* overflow)
{
    double ss = *sumsq;
    int32_t bad = *overflow;
    for (int64_t i = 0; i < n; ++i) {
        float acc = 0.0f;
        for (int32_t r = 0; r < n_replicas; ++r) {
            float x = replicas[r][i];
            acc = (r == 0) ? x : acc + x;
        }
        float gi = acc * inv_scale;
        g[i] = gi;
        if (!isfinite(gi)) bad = 1;
        ss += (double)gi * (double)gi;
    }
    *sumsq = ss;
    *overflow = bad;
}

/* ------------------------------------------------------------------------ */
/* Global-norm clipping.  [P1] §6 configuration: gradient_clipping 1.0.
 * The factor max_norm / (norm + 1e-6) applies only when it is below one.  */
int32_t oracle_clip(double sumsq, double max_norm, double* norm, double* coef)
{
    *norm = sqrt(sumsq);
    double c = max_norm / (*norm + 1e-6);
    if (max_norm > 0.0 && c < 1.0) {
        *coef = c;
        return 1;
    }
    *coef = 1.0;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* AdamW on the owned shard.  [P1] §3.1: optimizer AdamW with lr 6e-5 and
 * weight_decay 0.01; [P1] §2.1: each GPU updates only its own partition;
 * [P3] FAQ and the [P2] memory arithmetic: fp32 master weights and fp32
 * first and second moments.  Textbook AdamW (decoupled decay, bias
 * correction from t = 1) evaluated in fp32, the precision of the state:
 * the scalars are computed in fp64 and rounded once to fp32, then each
 * element takes these fp32 operations, one rounding each, in this order:
 *   g' = g * coef
 *   m' = b1 * m + c1 * g'                      b1 = beta1, c1 = 1 - beta1
 *   v' = b2 * v + c2 * (g' * g')               b2 = beta2, c2 = 1 - beta2
 *   d  = sqrt(v') * inv_sqrt_bc2 + eps         inv_sqrt_bc2 = 1/sqrt(1 - beta2^t)
 *   p' = p * decay - step_size * (m' / d)      decay = 1 - lr wd,
 *                                              step_size = lr / (1 - beta1^t)
 * which is lr * m_hat / (sqrt(v_hat) + eps) with m_hat = m'/(1 - beta1^t)
 * and v_hat = v'/(1 - beta2^t) written out.                               */
void oracle_adamw(int64_t n, const float* g, float* p, float* m, float* v,
                  double coef, double lr, double beta1, double beta2,
                  double eps, double weight_decay, int64_t t)
{
    const float cf = (float)coef;
    const float b1 = (float)beta1;
    const float c1 = (float)(1.0 - beta1);
    const float b2 = (float)beta2;
    const float c2 = (float)(1.0 - beta2);
    const float decay = (float)(1.0 - lr * weight_decay);
    const float step_size = (float)(lr / (1.0 - pow(beta1, (double)t)));
    const float inv_sqrt_bc2 = (float)(1.0 / sqrt(1.0 - pow(beta2, (double)t)));
    const float epsf = (float)eps;
    for (int64_t i = 0; i < n; ++i) {
        float gi = g[i] * cf;
        float m1 = b1 * m[i] + c1 * gi;
        float v1 = b2 * v[i] + c2 * (gi * gi);
        float d = sqrtf(v1) * inv_sqrt_bc2 + epsf;
        float p1 = p[i] * decay - step_size * (m1 / d);
        m[i] = m1;
        v[i] = v1;
        p[i] = p1;
    }
}

/* ------------------------------------------------------------------------ */
/* Dynamic loss scaler.  [P1] §3.3 and §5.1 give fp16 with loss_scale_window
 * 100, hysteresis 2, initial_scale_power 16, min_loss_scale 1.  The rule is
 * a reading (parity unpinned by the pages), stated in the header.         */
void oracle_scaler_init(oracle_scaler* s, int32_t initial_scale_power,
                        int32_t window, int32_t hysteresis, double min_scale)
{
    s->scale = ldexp(1.0, initial_scale_power);
    s->good = 0;
    s->hyst = hysteresis;
    s->window = window;
    s->hysteresis = hysteresis;
    s->min_scale = min_scale;
}

int32_t oracle_scaler_update(oracle_scaler* s, int32_t overflow)
{
    if (overflow) {
        s->good = 0;
        if (s->hyst > 1) {
            s->hyst -= 1;
        } else {
            double halved = s->scale / 2.0;
            s->scale = halved > s->min_scale ? halved : s->min_scale;
        }
        return 1;
    }
    s->good += 1;
    if (s->good == s->window) {
        s->scale *= 2.0;
        s->good = 0;
        s->hyst = s->hysteresis;
    }
    return 0;
}
