// zero_offload.cpp -- the optimizer step offloaded to the host CPU
// ("ZeRO技术解析：大模型分布式训练的革命性突破" §1.2.3 and §3.1:
// offload_optimizer to the CPU with pinned memory; "ZeRO 和分片优化器",
// real-world implementations: ZeRO-Offload keeps optimizer state in host
// memory).  Host C++ and the HIP runtime's copy API only; no kernels.
//
// The host update is the GPU pass's update, one fp32 IEEE operation at a
// time in the same order (no contraction: the library is built with
// -ffp-contract=off), with the same constants (adam_consts), so it gives
// the same bits.  The casts to bf16 / fp16 are round-to-nearest-even,
// written from the formats' bit layouts.
#include <hip/hip_runtime_api.h>

#include <sched.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

#include "zero_internal.h"

namespace zero {
namespace {

inline uint32_t bits_of(float x) {
    uint32_t u;
    std::memcpy(&u, &x, 4);
    return u;
}

// bfloat16 is the upper half of an fp32: add just under half an ulp of the
// kept part, plus one when the kept part is odd (ties to even), and
// truncate.  Overflow carries into the exponent and gives inf, as rounding
// should; NaN is kept quiet.
inline uint16_t to_bf16(float x) {
    const uint32_t u = bits_of(x);
    const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    const uint32_t quiet = (u >> 16) | 0x0040u;
    return static_cast<uint16_t>((u & 0x7fffffffu) > 0x7f800000u ? quiet : rounded);
}

// IEEE binary16 (5 exponent bits, bias 15, 10 fraction bits).
inline uint16_t to_f16(float x) {
    const uint32_t u = bits_of(x);
    const uint16_t sign = static_cast<uint16_t>((u >> 16) & 0x8000u);
    const uint32_t a = u & 0x7fffffffu;
    if (a >= 0x7f800000u) return sign | (a > 0x7f800000u ? 0x7e00u : 0x7c00u);   // NaN, inf
    if (a >= 0x477ff000u) return sign | 0x7c00u;   // >= 65520 rounds past 65504 to inf
    if (a < 0x38800000u) {                         // below 2^-14: fp16 subnormal or zero
        if (a < 0x33000000u) return sign;          // below 2^-25: rounds to zero
        const uint32_t e = a >> 23;                // 102 .. 112
        const uint32_t mant = (a & 0x7fffffu) | 0x800000u;   // value = mant * 2^(e - 150)
        const uint32_t sh = 126u - e;              // units of 2^-24: mant >> sh, sh in 14..24
        uint32_t q = mant >> sh;
        const uint32_t rem = mant & ((1u << sh) - 1u), half = 1u << (sh - 1u);
        if (rem > half || (rem == half && (q & 1u))) ++q;   // may carry into the first normal
        return static_cast<uint16_t>(sign | q);
    }
    uint32_t q = (((a >> 23) - 112u) << 10) | ((a & 0x7fffffu) >> 13);
    const uint32_t rem = a & 0x1fffu;
    if (rem > 0x1000u || (rem == 0x1000u && (q & 1u))) ++q;  // carry into the exponent is exact
    return static_cast<uint16_t>(sign | q);
}

struct HostUpdate {
    AdamConsts k;
    float coef;
    int dtype;
};

// One contiguous range; the loop body is the GPU pass's per-element update.
// The cast to the parameter dtype follows each block of kCastBlock
// elements while that block's masters are still in the core's L1 cache,
// rather than in a second pass that reads every master from memory again.
constexpr int64_t kCastBlock = 1024;

void adamw_range(const HostUpdate& u, int64_t lo, int64_t hi, const float* g, float* p, float* m,
                 float* v, uint16_t* out) {
    const AdamConsts& k = u.k;
    for (int64_t b = lo; b < hi; b += kCastBlock) {
        const int64_t e = std::min(hi, b + kCastBlock);
        for (int64_t i = b; i < e; ++i) {
            const float gi = g[i] * u.coef;
            const float m1 = k.b1 * m[i] + k.c1 * gi;
            const float v1 = k.b2 * v[i] + k.c2 * (gi * gi);
            const float d = std::sqrt(v1) * k.inv_sqrt_bc2 + k.eps;
            const float p1 = p[i] * k.decay - k.step_size * (m1 / d);
            m[i] = m1;
            v[i] = v1;
            p[i] = p1;
        }
        if (!out) continue;
        if (u.dtype == ZERO_BF16)
            for (int64_t i = b; i < e; ++i) out[i] = to_bf16(p[i]);
        else
            for (int64_t i = b; i < e; ++i) out[i] = to_f16(p[i]);
    }
}

// A rank's host state in either layout (ZERO_STATE_SEPARATE or _TILED).
struct HostState {
    float* p;
    float* m;
    float* v;
    bool tiled;       // p is the tiled array; m and v are unused
};

// Elements [base + lo, base + hi) of the state, with the gradient, and the
// cast's destination, indexed from base (g[i], out[i] belong to element
// base + i).  A tiled state is walked one tile at a time, each tile's three
// fields being three contiguous runs.
void adamw_span(const HostUpdate& u, int64_t lo, int64_t hi, const float* g, const HostState& s,
                int64_t base, uint16_t* out) {
    if (!s.tiled) {
        adamw_range(u, lo, hi, g, s.p + base, s.m + base, s.v + base, out);
        return;
    }
    for (int64_t i = lo; i < hi;) {
        const int64_t e = base + i, k = e / kStateTile;
        const int64_t end = std::min(hi, (k + 1) * kStateTile - base);
        // p[i] is element e's master: tile k starts at 3 * kStateTile * k
        float* p = s.p + 2 * kStateTile * k + base;
        adamw_range(u, i, end, g, p, p + kStateTile, p + 2 * kStateTile, out);
        i = end;
    }
}

// The thread count used when the caller passes 0: OMP_NUM_THREADS when it
// is set to a positive number, else the CPUs this process may run on, else
// the hardware's thread count.
int default_host_threads() {
    if (const char* env = std::getenv("OMP_NUM_THREADS")) {
        const long v = std::strtol(env, nullptr, 10);
        if (v > 0) return static_cast<int>(std::min<long>(v, 1024));
    }
    cpu_set_t set;
    if (sched_getaffinity(0, sizeof(set), &set) == 0) {
        const int c = CPU_COUNT(&set);
        if (c > 0) return c;
    }
    const unsigned h = std::thread::hardware_concurrency();
    return h > 0 ? static_cast<int>(h) : 1;
}

// Split elements [base, base + n) into contiguous ranges of whole 64-byte
// lines, one per thread, and run them; g and out are indexed from base.
void adamw_parallel(const HostUpdate& u, int64_t n, const float* g, const HostState& s, int64_t base,
                    uint16_t* out, int n_threads) {
    int t = n_threads > 0 ? n_threads : default_host_threads();
    if (t < 1) t = 1;
    const int64_t min_per = int64_t(1) << 16;
    if (static_cast<int64_t>(t) * min_per > n) t = static_cast<int>(std::max<int64_t>(1, n / min_per));
    if (t == 1) {
        adamw_span(u, 0, n, g, s, base, out);
        return;
    }
    const int64_t per = (n + t - 1) / t / 16 * 16 + 16;
    std::vector<std::thread> pool;
    pool.reserve(static_cast<size_t>(t));
    for (int i = 0; i < t; ++i) {
        const int64_t lo = std::min<int64_t>(n, i * per), hi = std::min<int64_t>(n, lo + per);
        if (lo < hi) pool.emplace_back(adamw_span, std::cref(u), lo, hi, g, std::cref(s), base, out);
    }
    for (auto& th : pool) th.join();
}

int hip_fail(hipError_t e, const char* what) {
    return fail(ZERO_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace
}  // namespace zero

using namespace zero;

extern "C" {

int32_t zero_host_threads(void) { return default_host_threads(); }

int zero_host_adamw(int64_t n, const float* g, float coef, float* master, float* exp_avg,
                    float* exp_avg_sq, void* params_out, int32_t param_dtype, double lr,
                    double beta1, double beta2, double eps, double weight_decay,
                    int64_t step, int32_t n_threads) {
    clear_error();
    if (n < 0) return fail(ZERO_EINVAL, "n %lld < 0", (long long)n);
    if (n > 0 && (!g || !master || !exp_avg || !exp_avg_sq))
        return fail(ZERO_EINVAL, "a required pointer is NULL");
    if (param_dtype != ZERO_FP16 && param_dtype != ZERO_BF16)
        return fail(ZERO_EINVAL, "param_dtype %d is not ZERO_FP16 or ZERO_BF16", param_dtype);
    if (step < 1) return fail(ZERO_EINVAL, "step %lld < 1", (long long)step);
    if (!std::isfinite(lr) || lr < 0.0 || !(beta1 >= 0.0 && beta1 < 1.0) ||
        !(beta2 >= 0.0 && beta2 < 1.0) || !(std::isfinite(eps) && eps > 0.0) ||
        !std::isfinite(weight_decay) || !std::isfinite(coef))
        return fail(ZERO_EINVAL, "a hyper-parameter is out of range");
    HostUpdate u{adam_consts(lr, beta1, beta2, eps, weight_decay, step), coef, param_dtype};
    const HostState hs{master, exp_avg, exp_avg_sq, false};
    adamw_parallel(u, n, g, hs, 0, static_cast<uint16_t*>(params_out), n_threads);
    return ZERO_OK;
}

int zero_offload_apply(const zero_step_args* a, const void* global_dev,
                       const zero_offload_staging_t* stg, zero_step_info* info, void* stream) {
    clear_error();
    int rc = validate_step_args(a);
    if (rc) return rc;
    if (!global_dev) return fail(ZERO_EINVAL, "global_dev is NULL");
    if (!aligned16(global_dev)) return fail(ZERO_EALIGN, "global_dev is not 16-byte aligned");
    if (a->master_out || a->exp_avg_out || a->exp_avg_sq_out)
        return fail(ZERO_EINVAL, "the offloaded step updates the host state in place");
    if (!stg) return fail(ZERO_EINVAL, "staging is NULL");
    if (stg->chunk_elems < 1 || stg->chunk_elems % 8 != 0)
        return fail(ZERO_EINVAL, "chunk_elems %lld is not a positive multiple of 8",
                    (long long)stg->chunk_elems);
    for (int i = 0; i < 2; ++i)
        if (!stg->grad_stage[i] || !stg->param_stage[i])
            return fail(ZERO_EINVAL, "a staging buffer is NULL");
    hipStream_t st = static_cast<hipStream_t>(stream);
    zero_global_t glob;
    hipError_t e = hipMemcpyAsync(&glob, global_dev, sizeof glob, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "reading the combine's result");
    if (info) *info = glob;
    if (glob.overflow || a->valid_numel == 0) return ZERO_OK;   // skipped step: nothing changes

    const HostUpdate u{adam_consts(a->lr, a->beta1, a->beta2, a->eps, a->weight_decay, a->step),
                       glob.coef, a->param_dtype};
    const HostState hs{a->master, a->exp_avg, a->exp_avg_sq, a->state_layout == ZERO_STATE_TILED};
    const int64_t n = a->valid_numel, C = stg->chunk_elems;
    const int64_t n_chunks = (n + C - 1) / C;
    const float* g_dev = static_cast<const float*>(a->workspace);
    uint16_t* out_dev = param_out(a);
    // Gradients come down on the caller's stream (after pass 1); parameters
    // go up on a second stream so the two directions of the link overlap.
    hipStream_t up = nullptr;
    hipEvent_t down_done[2] = {nullptr, nullptr}, up_done[2] = {nullptr, nullptr};
    auto cleanup = [&]() {
        for (int i = 0; i < 2; ++i) {
            if (down_done[i]) (void)hipEventDestroy(down_done[i]);
            if (up_done[i]) (void)hipEventDestroy(up_done[i]);
        }
        if (up) (void)hipStreamDestroy(up);
    };
    e = hipStreamCreateWithFlags(&up, hipStreamNonBlocking);
    for (int i = 0; i < 2 && e == hipSuccess; ++i) {
        e = hipEventCreateWithFlags(&down_done[i], hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&up_done[i], hipEventDisableTiming);
    }
    if (e != hipSuccess) {
        cleanup();
        return hip_fail(e, "creating the offload stream and events");
    }
    auto len_of = [&](int64_t c) { return std::min(C, n - c * C); };
    auto fetch = [&](int64_t c) -> hipError_t {
        hipError_t r = hipMemcpyAsync(stg->grad_stage[c & 1], g_dev + c * C,
                                      static_cast<size_t>(len_of(c)) * 4,
                                      hipMemcpyDeviceToHost, st);
        if (r == hipSuccess) r = hipEventRecord(down_done[c & 1], st);
        return r;
    };
    e = fetch(0);
    for (int64_t c = 0; c < n_chunks && e == hipSuccess; ++c) {
        if (c + 1 < n_chunks) e = fetch(c + 1);                 // its stage was consumed at c - 1
        if (e == hipSuccess) e = hipEventSynchronize(down_done[c & 1]);
        if (e == hipSuccess && c >= 2) e = hipEventSynchronize(up_done[c & 1]);   // stage free
        if (e != hipSuccess) break;
        const int64_t lo = c * C, len = len_of(c);
        uint16_t* pst = static_cast<uint16_t*>(stg->param_stage[c & 1]);
        // The staging buffers hold the chunk's elements from 0; the state
        // is addressed by element, from the chunk start lo.
        adamw_parallel(u, len, static_cast<const float*>(stg->grad_stage[c & 1]), hs, lo, pst,
                       stg->n_threads);
        e = hipMemcpyAsync(out_dev + lo, pst, static_cast<size_t>(len) * 2, hipMemcpyHostToDevice,
                           up);
        if (e == hipSuccess) e = hipEventRecord(up_done[c & 1], up);
    }
    // Wait for both streams whatever happened above: after an error some
    // copies into or out of the caller's staging buffers and parameter
    // slice may still be queued, and none may run after this call returns.
    const hipError_t e_up = hipStreamSynchronize(up);
    const hipError_t e_st = hipStreamSynchronize(st);
    if (e == hipSuccess) e = e_up;
    if (e == hipSuccess) e = e_st;
    cleanup();
    if (e != hipSuccess) return hip_fail(e, "offloaded step");
    return ZERO_OK;
}

}  // extern "C"
