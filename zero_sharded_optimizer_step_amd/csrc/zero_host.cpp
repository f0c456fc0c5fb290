// zero_host.cpp -- host-only parts of the library: errors, partition, bucket
// plan, loss scaler and argument checks.  No HIP calls in this file, so these
// entry points work on a machine without a GPU.
#include <cmath>
#include <cstdio>
#include <cstring>

#include "zero_internal.h"

namespace zero {

static thread_local char g_error[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_error, sizeof g_error, fmt, ap);
    va_end(ap);
    return code;
}

void clear_error() { g_error[0] = '\0'; }

static bool finite_positive(double x) { return std::isfinite(x) && x > 0.0; }

AdamConsts adam_consts(double lr, double beta1, double beta2, double eps, double weight_decay,
                       int64_t step) {
    AdamConsts k;
    const double t = static_cast<double>(step);
    k.decay = static_cast<float>(1.0 - lr * weight_decay);
    k.b1 = static_cast<float>(beta1);
    k.c1 = static_cast<float>(1.0 - beta1);
    k.b2 = static_cast<float>(beta2);
    k.c2 = static_cast<float>(1.0 - beta2);
    k.step_size = static_cast<float>(lr / (1.0 - std::pow(beta1, t)));
    k.inv_sqrt_bc2 = static_cast<float>(1.0 / std::sqrt(1.0 - std::pow(beta2, t)));
    k.eps = static_cast<float>(eps);
    return k;
}

int validate_step_args(const zero_step_args* a, bool check_workspace) {
    if (!a) return fail(ZERO_EINVAL, "args is NULL");
    if (a->world_size < 1) return fail(ZERO_EINVAL, "world_size %d < 1", a->world_size);
    if (a->rank < 0 || a->rank >= a->world_size)
        return fail(ZERO_EINVAL, "rank %d outside [0, %d)", a->rank, a->world_size);
    if (a->shard_numel < 0 || a->shard_numel % kShardMultiple != 0)
        return fail(ZERO_EINVAL, "shard_numel %lld must be a non-negative multiple of 8",
                    (long long)a->shard_numel);
    if (a->valid_numel < 0 || a->valid_numel > a->shard_numel)
        return fail(ZERO_EINVAL, "valid_numel %lld outside [0, shard_numel=%lld]",
                    (long long)a->valid_numel, (long long)a->shard_numel);
    if (a->grad_dtype != ZERO_FP16 && a->grad_dtype != ZERO_BF16 && a->grad_dtype != ZERO_FP32)
        return fail(ZERO_EINVAL, "grad_dtype %d is not ZERO_FP16, ZERO_BF16 or ZERO_FP32",
                    a->grad_dtype);
    if (a->param_dtype != ZERO_FP16 && a->param_dtype != ZERO_BF16)
        return fail(ZERO_EINVAL, "param_dtype %d is not ZERO_FP16 or ZERO_BF16", a->param_dtype);
    if (a->n_replicas < 1 || a->n_replicas > ZERO_MAX_REPLICAS)
        return fail(ZERO_EINVAL, "n_replicas %d outside [1, %d]", a->n_replicas,
                    ZERO_MAX_REPLICAS);
    if (a->accumulate != 0 && a->accumulate != 1)
        return fail(ZERO_EINVAL, "accumulate %d is not 0 or 1", a->accumulate);
    if (a->step < 1) return fail(ZERO_EINVAL, "step %lld < 1", (long long)a->step);
    if (!finite_positive(a->loss_scale))
        return fail(ZERO_EINVAL, "loss_scale must be finite and > 0");
    if (!finite_positive(a->grad_predivide))
        return fail(ZERO_EINVAL, "grad_predivide must be finite and > 0");
    if (!std::isfinite(a->lr) || a->lr < 0.0) return fail(ZERO_EINVAL, "lr must be finite and >= 0");
    if (!(a->beta1 >= 0.0 && a->beta1 < 1.0)) return fail(ZERO_EINVAL, "beta1 outside [0, 1)");
    if (!(a->beta2 >= 0.0 && a->beta2 < 1.0)) return fail(ZERO_EINVAL, "beta2 outside [0, 1)");
    if (!finite_positive(a->eps)) return fail(ZERO_EINVAL, "eps must be finite and > 0");
    if (!std::isfinite(a->weight_decay)) return fail(ZERO_EINVAL, "weight_decay must be finite");
    if (std::isnan(a->max_grad_norm)) return fail(ZERO_EINVAL, "max_grad_norm is NaN");
    if (check_workspace && !a->workspace) return fail(ZERO_EINVAL, "workspace is NULL");
    if (check_workspace && !aligned16(a->workspace))
        return fail(ZERO_EALIGN, "workspace is not 16-byte aligned");
    if (a->state_layout != ZERO_STATE_SEPARATE && a->state_layout != ZERO_STATE_TILED)
        return fail(ZERO_EINVAL, "state_layout %d is not ZERO_STATE_SEPARATE or ZERO_STATE_TILED",
                    a->state_layout);
    if (a->reserved != 0) return fail(ZERO_EINVAL, "reserved must be 0");
    const bool tiled = a->state_layout == ZERO_STATE_TILED;
    if (tiled && (a->exp_avg || a->exp_avg_sq || a->exp_avg_out || a->exp_avg_sq_out))
        return fail(ZERO_EINVAL, "a tiled state is `master` (and `master_out`) alone: exp_avg, "
                                 "exp_avg_sq and their outputs must be NULL");
    // A rank with no real elements reads and writes no element, so its data
    // pointers may be NULL (empty tensors).
    if (a->valid_numel > 0) {
        if (!a->replica_grad || !a->master || (!tiled && (!a->exp_avg || !a->exp_avg_sq)) ||
            (!a->full_params && !a->param_shard))
            return fail(ZERO_EINVAL, "a required pointer is NULL");
        for (int i = 0; i < a->n_replicas; ++i) {
            if (!a->replica_grad[i]) return fail(ZERO_EINVAL, "replica_grad[%d] is NULL", i);
            if (!aligned16(a->replica_grad[i]))
                return fail(ZERO_EALIGN, "replica_grad[%d] is not 16-byte aligned", i);
        }
        if (!aligned16(a->master) || !aligned16(a->exp_avg) || !aligned16(a->exp_avg_sq) ||
            !aligned16(a->full_params) || !aligned16(a->param_shard))
            return fail(ZERO_EALIGN, "a state or parameter pointer is not 16-byte aligned");
    }
    const int n_out = (a->master_out != nullptr) + (a->exp_avg_out != nullptr) +
                      (a->exp_avg_sq_out != nullptr);
    if (tiled) {
        if (a->master_out && !aligned16(a->master_out))
            return fail(ZERO_EALIGN, "master_out is not 16-byte aligned");
        if (a->master_out && a->master_out == a->master)
            return fail(ZERO_EINVAL, "output state must not be the input state (leave it NULL "
                                     "to update in place)");
    } else if (n_out != 0 && n_out != 3) {
        return fail(ZERO_EINVAL, "master_out, exp_avg_out and exp_avg_sq_out are set together");
    }
    if (!tiled && n_out == 3) {
        if (!aligned16(a->master_out) || !aligned16(a->exp_avg_out) || !aligned16(a->exp_avg_sq_out))
            return fail(ZERO_EALIGN, "an output state pointer is not 16-byte aligned");
        if (a->master_out == a->master || a->exp_avg_out == a->exp_avg ||
            a->exp_avg_sq_out == a->exp_avg_sq)
            return fail(ZERO_EINVAL, "output state must not be the input state (leave it NULL "
                                     "to update in place)");
    }
    if (!aligned16(a->scalars)) return fail(ZERO_EALIGN, "scalars is not 16-byte aligned");
    // Start of this rank's slice of the full buffer: shard_numel is a
    // multiple of 8, so 2-byte elements keep 16-byte alignment.
    if (check_workspace && a->workspace_bytes < zero_shard_workspace_bytes(a->shard_numel))
        return fail(ZERO_ESIZE, "workspace_bytes %zu < %zu needed", a->workspace_bytes,
                    zero_shard_workspace_bytes(a->shard_numel));
    return ZERO_OK;
}

int check_partition(const zero_partition_t* p, const char* what) {
    if (!p) return fail(ZERO_EINVAL, "%s is NULL", what);
    zero_partition_t q;
    if (zero_partition(p->numel, p->world_size, p->alignment, &q) != ZERO_OK)
        return fail(ZERO_EINVAL, "%s (numel %lld, world_size %d, alignment %d) is not a valid "
                                 "partition", what, (long long)p->numel, p->world_size,
                    p->alignment);
    if (q.shard_numel != p->shard_numel || q.padded_numel != p->padded_numel)
        return fail(ZERO_EINVAL, "%s has shard_numel %lld / padded_numel %lld; zero_partition "
                                 "gives %lld / %lld", what, (long long)p->shard_numel,
                    (long long)p->padded_numel, (long long)q.shard_numel,
                    (long long)q.padded_numel);
    return ZERO_OK;
}

}  // namespace zero

using namespace zero;

extern "C" {

const char* zero_last_error(void) { return g_error; }

int zero_partition(int64_t numel, int32_t world_size, int32_t alignment,
                   zero_partition_t* out) {
    clear_error();
    if (!out) return fail(ZERO_EINVAL, "out is NULL");
    if (numel < 0) return fail(ZERO_EINVAL, "numel %lld < 0", (long long)numel);
    if (world_size < 1) return fail(ZERO_EINVAL, "world_size %d < 1", world_size);
    if (alignment < 1 || (alignment & (alignment - 1)) != 0)
        return fail(ZERO_EINVAL, "alignment %d is not a power of two", alignment);
    // One aligned unit is world_size * alignment elements of the flat space;
    // every rank gets the same number of units.  The padded count must stay
    // representable.
    const int64_t unit = static_cast<int64_t>(world_size) * alignment;
    const int64_t units = numel / unit + (numel % unit ? 1 : 0);
    if (units > INT64_MAX / unit)
        return fail(ZERO_EINVAL, "numel %lld padded to whole units of %lld overflows int64",
                    (long long)numel, (long long)unit);
    out->numel = numel;
    out->shard_numel = units * alignment;
    out->padded_numel = out->shard_numel * world_size;
    out->world_size = world_size;
    out->alignment = alignment;
    return ZERO_OK;
}

int64_t zero_partition_valid_numel(const zero_partition_t* p, int32_t rank) {
    if (!p || rank < 0 || rank >= p->world_size) return -1;
    const int64_t begin = static_cast<int64_t>(rank) * p->shard_numel;
    if (begin >= p->numel) return 0;
    const int64_t left = p->numel - begin;
    return left < p->shard_numel ? left : p->shard_numel;
}

int zero_bucket_plan(const int64_t* tensor_numel, int32_t n_tensors,
                     int64_t reduce_bucket_size, zero_tensor_slot_t* slots,
                     zero_bucket_t* buckets, int32_t bucket_cap, int32_t* n_buckets) {
    clear_error();
    if (n_tensors < 0) return fail(ZERO_EINVAL, "n_tensors %d < 0", n_tensors);
    if (reduce_bucket_size < 1)
        return fail(ZERO_EINVAL, "reduce_bucket_size %lld < 1", (long long)reduce_bucket_size);
    if (!n_buckets || (n_tensors > 0 && (!tensor_numel || !slots)) || bucket_cap < 0 ||
        (bucket_cap > 0 && !buckets))
        return fail(ZERO_EINVAL, "a required pointer is NULL or bucket_cap < 0");
    int64_t total = 0;
    for (int32_t t = 0; t < n_tensors; ++t) {
        if (tensor_numel[t] < 0)
            return fail(ZERO_EINVAL, "tensor_numel[%d] = %lld < 0", t, (long long)tensor_numel[t]);
        if (tensor_numel[t] > INT64_MAX - total)
            return fail(ZERO_EINVAL, "the tensor sizes sum past int64 at tensor %d", t);
        total += tensor_numel[t];
    }

    int32_t count = 0;         // buckets opened so far
    int64_t cursor = 0;        // flat offset of the next tensor
    int64_t open_begin = 0;    // flat start of the open bucket
    int32_t open_first = 0;    // first tensor of the open bucket
    auto close_bucket = [&](int32_t end_tensor) {
        if (count >= 1 && count <= bucket_cap) {
            zero_bucket_t& b = buckets[count - 1];
            b.begin = open_begin;
            b.end = cursor;
            b.first_tensor = open_first;
            b.n_tensors = end_tensor - open_first;
        }
    };
    for (int32_t t = 0; t < n_tensors; ++t) {
        const int64_t n = tensor_numel[t];
        // A new bucket starts at the first tensor, and whenever the open
        // bucket already holds elements and this tensor would push it past
        // the bucket size.  An oversize tensor therefore sits alone.
        const bool holds_elements = cursor > open_begin;
        if (count == 0 || (holds_elements && (cursor - open_begin) + n > reduce_bucket_size)) {
            close_bucket(t);
            open_begin = cursor;
            open_first = t;
            ++count;
        }
        slots[t].offset = cursor;
        slots[t].numel = n;
        slots[t].bucket = count - 1;
        slots[t].reserved = 0;
        cursor += n;
    }
    close_bucket(n_tensors);
    *n_buckets = count;
    if (count > bucket_cap)
        return fail(ZERO_ESIZE, "plan needs %d buckets, capacity is %d", count, bucket_cap);
    return ZERO_OK;
}

int zero_loss_scaler_init(int32_t initial_scale_power, int32_t loss_scale_window,
                          int32_t hysteresis, double min_loss_scale,
                          zero_loss_scaler_t* st) {
    clear_error();
    if (!st) return fail(ZERO_EINVAL, "st is NULL");
    if (loss_scale_window < 1) return fail(ZERO_EINVAL, "loss_scale_window %d < 1", loss_scale_window);
    if (hysteresis < 1) return fail(ZERO_EINVAL, "hysteresis %d < 1", hysteresis);
    if (!finite_positive(min_loss_scale)) return fail(ZERO_EINVAL, "min_loss_scale must be > 0");
    if (initial_scale_power < -126 || initial_scale_power > 127)
        return fail(ZERO_EINVAL, "initial_scale_power %d outside [-126, 127]", initial_scale_power);
    st->scale = std::ldexp(1.0, initial_scale_power);
    st->min_scale = min_loss_scale;
    st->good_steps = 0;
    st->hysteresis_left = hysteresis;
    st->window = loss_scale_window;
    st->hysteresis = hysteresis;
    return ZERO_OK;
}

int zero_loss_scaler_update(zero_loss_scaler_t* st, int32_t overflow, int32_t* skip_step) {
    clear_error();
    if (!st || !skip_step) return fail(ZERO_EINVAL, "st or skip_step is NULL");
    if (st->window < 1 || st->hysteresis < 1 || !finite_positive(st->min_scale))
        return fail(ZERO_EINVAL, "scaler state was not initialised");
    if (overflow) {
        // The step is dropped.  Hysteresis absorbs isolated overflows;
        // once spent, every overflow halves the scale down to the floor.
        *skip_step = 1;
        st->good_steps = 0;
        if (st->hysteresis_left > 1) {
            st->hysteresis_left -= 1;
        } else {
            const double half = st->scale * 0.5;
            st->scale = half < st->min_scale ? st->min_scale : half;
        }
        return ZERO_OK;
    }
    *skip_step = 0;
    if (++st->good_steps >= st->window) {
        st->scale *= 2.0;
        st->good_steps = 0;
        st->hysteresis_left = st->hysteresis;
    }
    return ZERO_OK;
}

static_assert(sizeof(zero_ckpt_header_t) == 128, "checkpoint header is 128 bytes");

int zero_ckpt_header_make(const zero_partition_t* p, int32_t rank, int32_t param_dtype,
                          int64_t step, const zero_loss_scaler_t* scaler,
                          zero_ckpt_header_t* out) {
    clear_error();
    if (!p || !out) return fail(ZERO_EINVAL, "p or out is NULL");
    if (rank < 0 || rank >= p->world_size)
        return fail(ZERO_EINVAL, "rank %d outside [0, %d)", rank, p->world_size);
    if (param_dtype != ZERO_FP16 && param_dtype != ZERO_BF16)
        return fail(ZERO_EINVAL, "param_dtype %d is not ZERO_FP16 or ZERO_BF16", param_dtype);
    if (step < 0) return fail(ZERO_EINVAL, "step %lld < 0", (long long)step);
    std::memset(out, 0, sizeof *out);
    out->magic = ZERO_CKPT_MAGIC;
    out->version = ZERO_CKPT_VERSION;
    out->numel = p->numel;
    out->shard_numel = p->shard_numel;
    out->valid_numel = zero_partition_valid_numel(p, rank);
    out->world_size = p->world_size;
    out->rank = rank;
    out->alignment = p->alignment;
    out->param_dtype = param_dtype;
    out->step = step;
    if (scaler) {
        out->has_scaler = 1;
        out->scaler = *scaler;
    }
    out->payload_bytes = 3u * static_cast<uint64_t>(out->valid_numel) * 4u;
    return ZERO_OK;
}

int zero_ckpt_header_check(const zero_ckpt_header_t* h, uint64_t file_bytes,
                           zero_partition_t* part) {
    clear_error();
    if (!h) return fail(ZERO_EINVAL, "h is NULL");
    if (h->magic != ZERO_CKPT_MAGIC) return fail(ZERO_EINVAL, "not a checkpoint shard (bad magic)");
    if (h->version != ZERO_CKPT_VERSION)
        return fail(ZERO_EINVAL, "checkpoint version %u, this library reads %d", h->version,
                    ZERO_CKPT_VERSION);
    zero_partition_t p;
    if (zero_partition(h->numel, h->world_size, h->alignment, &p) != ZERO_OK)
        return fail(ZERO_EINVAL, "checkpoint partition (%lld, %d, %d) is invalid",
                    (long long)h->numel, h->world_size, h->alignment);
    if (p.shard_numel != h->shard_numel)
        return fail(ZERO_EINVAL, "shard_numel %lld does not match the partition's %lld",
                    (long long)h->shard_numel, (long long)p.shard_numel);
    if (h->rank < 0 || h->rank >= h->world_size)
        return fail(ZERO_EINVAL, "rank %d outside [0, %d)", h->rank, h->world_size);
    if (h->valid_numel != zero_partition_valid_numel(&p, h->rank))
        return fail(ZERO_EINVAL, "valid_numel %lld does not match rank %d of the partition",
                    (long long)h->valid_numel, h->rank);
    if (h->param_dtype != ZERO_FP16 && h->param_dtype != ZERO_BF16)
        return fail(ZERO_EINVAL, "param_dtype %d is not ZERO_FP16 or ZERO_BF16", h->param_dtype);
    if (h->step < 0) return fail(ZERO_EINVAL, "step %lld < 0", (long long)h->step);
    if (h->has_scaler != 0 && h->has_scaler != 1) return fail(ZERO_EINVAL, "has_scaler is not 0 or 1");
    if (h->has_scaler &&
        (h->scaler.window < 1 || h->scaler.hysteresis < 1 || !finite_positive(h->scaler.scale) ||
         !finite_positive(h->scaler.min_scale)))
        return fail(ZERO_EINVAL, "saved loss-scaler state is invalid");
    const uint64_t payload = 3u * static_cast<uint64_t>(h->valid_numel) * 4u;
    if (h->payload_bytes != payload)
        return fail(ZERO_EINVAL, "payload_bytes %llu, expected %llu",
                    (unsigned long long)h->payload_bytes, (unsigned long long)payload);
    if (file_bytes < sizeof(zero_ckpt_header_t) + payload)
        return fail(ZERO_ESIZE, "file holds %llu bytes, header and payload need %llu",
                    (unsigned long long)file_bytes,
                    (unsigned long long)(sizeof(zero_ckpt_header_t) + payload));
    if (part) *part = p;
    return ZERO_OK;
}

static_assert(sizeof(zero_step_scalars_t) == 64, "step scalars are 64 bytes");

int zero_step_scalars(const zero_step_args* a, double peer_sumsq, int32_t peer_overflow,
                      zero_step_scalars_t* out) {
    clear_error();
    if (!out) return fail(ZERO_EINVAL, "out is NULL");
    int rc = validate_step_args(a, false);
    if (rc) return rc;
    if (!(peer_sumsq >= 0.0)) return fail(ZERO_EINVAL, "peer_sumsq must be >= 0 (got NaN or negative)");
    // the same constants, rounded the same way, as the launch arguments
    const AdamConsts k = adam_consts(a->lr, a->beta1, a->beta2, a->eps, a->weight_decay, a->step);
    std::memset(out, 0, sizeof *out);
    out->inv_scale = unscale_factor(a);
    out->decay = k.decay;
    out->beta1 = k.b1;
    out->one_minus_beta1 = k.c1;
    out->beta2 = k.b2;
    out->one_minus_beta2 = k.c2;
    out->step_size = k.step_size;
    out->inv_sqrt_bc2 = k.inv_sqrt_bc2;
    out->eps = k.eps;
    out->peer_overflow = peer_overflow ? 1 : 0;
    out->max_grad_norm = a->max_grad_norm;
    out->peer_sumsq = peer_sumsq;
    return ZERO_OK;
}

int zero_repartition_plan(const zero_partition_t* from, const zero_partition_t* to,
                          int32_t new_rank, zero_repartition_piece_t* pieces, int32_t piece_cap,
                          int32_t* n_pieces) {
    clear_error();
    if (!n_pieces || piece_cap < 0 || (piece_cap > 0 && !pieces))
        return fail(ZERO_EINVAL, "n_pieces is NULL, piece_cap < 0 or pieces is NULL");
    int rc;
    if ((rc = check_partition(from, "from"))) return rc;
    if ((rc = check_partition(to, "to"))) return rc;
    if (from->numel != to->numel)
        return fail(ZERO_EINVAL, "partitions cover %lld and %lld elements", (long long)from->numel,
                    (long long)to->numel);
    if (new_rank < 0 || new_rank >= to->world_size)
        return fail(ZERO_EINVAL, "new_rank %d outside [0, %d)", new_rank, to->world_size);
    // The new rank's real elements are flat [lo, hi).  Flat element i < numel
    // is element i - k*s_old of old rank k = i / s_old, one of that rank's
    // real elements; the old ranks that [lo, hi) meets give one contiguous
    // piece each.
    const int64_t s_old = from->shard_numel;
    const int64_t lo = static_cast<int64_t>(new_rank) * to->shard_numel;
    const int64_t hi = lo + zero_partition_valid_numel(to, new_rank);
    const int64_t k0 = hi > lo ? lo / s_old : 0;
    const int64_t count = hi > lo ? (hi - 1) / s_old - k0 + 1 : 0;
    *n_pieces = static_cast<int32_t>(count);
    if (count > piece_cap)
        return fail(ZERO_ESIZE, "the plan has %lld pieces, capacity is %d", (long long)count,
                    piece_cap);
    for (int64_t q = 0; q < count; ++q) {
        const int64_t k = k0 + q;
        const int64_t a = lo > k * s_old ? lo : k * s_old;
        const int64_t e = (k + 1) * s_old;
        const int64_t b = hi < e ? hi : e;
        zero_repartition_piece_t& pc = pieces[q];
        pc.old_offset = a - k * s_old;
        pc.new_offset = a - lo;
        pc.count = b - a;
        pc.old_rank = static_cast<int32_t>(k);
        pc.reserved = 0;
    }
    return ZERO_OK;
}

}  // extern "C"
