// zero_kernels.hip -- gfx950 kernels of the ZeRO sharded-optimizer step and
// the ABI entry points that launch them.
//
// The step is HBM-bound (about 50 bytes moved and ~25 flops per shard element
// at 8 replicas), so the kernels are built around streaming.  Each thread
// owns one quad of 4 consecutive elements and the grid has one thread per
// quad: waves load, compute, store and retire, and the dispatcher refills
// the CUs in address order, so every stream is read and written through a
// compact moving window.  Blocks are spread over the 8 XCDs so that each XCD
// walks a contiguous eighth of the shard.  Reductions stay in registers
// until one wavefront-shuffle + LDS step per block; a fixed-shape fold and
// combine finish them in a fixed order.  Nothing here is a dense
// contraction, so there is no MFMA.
//
// Sources (cited by title and section):
//   [P1] "ZeRO技术解析：大模型分布式训练的革命性突破"
//   [P3] "ZeRO 和分片优化器"
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>
#include <vector>

#include "zero_internal.h"

namespace zero {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Replica slices: 16-bit codes (ZERO_FP16, ZERO_BF16) or fp32 (ZERO_FP32).
struct ReplicaPtrs {
    const void* p[ZERO_MAX_REPLICAS];
};

// This block's logical index under the XCD remap (zero_internal.h).
__device__ __forceinline__ int64_t xcd_block(uint32_t b, uint32_t group) {
    return xcd_logical_block(b, group);
}

// ---------------------------------------------------------------- formats
// bf16 is the upper half of an fp32; fp16 goes through the hardware convert,
// which is exact (every fp16 value, subnormals included, is an fp32 value).
template <int DT>
__device__ __forceinline__ float lo_to_f32(unsigned w) {
    if constexpr (DT == ZERO_BF16) return __uint_as_float(w << 16);
    else return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<unsigned short>(w & 0xffffu)));
}
template <int DT>
__device__ __forceinline__ float hi_to_f32(unsigned w) {
    if constexpr (DT == ZERO_BF16) return __uint_as_float(w & 0xffff0000u);
    else return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<unsigned short>(w >> 16)));
}
template <int DT>
__device__ __forceinline__ void decode4(const u32x2 v, float o[4]) {
    o[0] = lo_to_f32<DT>(v.x); o[1] = hi_to_f32<DT>(v.x);
    o[2] = lo_to_f32<DT>(v.y); o[3] = hi_to_f32<DT>(v.y);
}

// Round to nearest even with the gfx950 packed converts (v_cvt_pk_bf16_f32,
// v_cvt_pk_f16_f32).
template <int DT>
__device__ __forceinline__ unsigned pack2(float a, float b) {
    f32x2 v = {a, b};
    if constexpr (DT == ZERO_BF16) return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
    else return __builtin_bit_cast(unsigned, __builtin_convertvector(v, f16x2));
}
template <int DT>
__device__ __forceinline__ unsigned short pack1(float a) {
    return static_cast<unsigned short>(pack2<DT>(a, 0.0f) & 0xffffu);
}

__device__ __forceinline__ bool finite(float x) { return __builtin_isfinite(x); }

// One quad of a replica slice: 8 bytes of 16-bit codes, or 16 bytes of fp32.
template <int DT> struct QuadOf { typedef u32x2 T; };
template <> struct QuadOf<ZERO_FP32> { typedef f32x4 T; };

template <int DT>
__device__ __forceinline__ typename QuadOf<DT>::T load_quad(const void* base, int64_t q) {
    return __builtin_nontemporal_load(static_cast<const typename QuadOf<DT>::T*>(base) + q);
}
template <int DT>
__device__ __forceinline__ void widen4(const typename QuadOf<DT>::T v, float o[4]) {
    if constexpr (DT == ZERO_FP32) {
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    } else {
        decode4<DT>(v, o);
    }
}
// Element i of a replica slice, widened to fp32 (exact).
template <int DT>
__device__ __forceinline__ float elem(const void* base, int64_t i) {
    if constexpr (DT == ZERO_FP32) return static_cast<const float*>(base)[i];
    else return lo_to_f32<DT>(static_cast<const unsigned short*>(base)[i]);
}

// ------------------------------------------------------- block reduction
// Fixed shuffle pattern and fixed wave order: the block's result depends
// only on which values its threads hold, never on timing.  Thread 0 ends
// with the block's total.
template <int THREADS>
__device__ __forceinline__ void block_reduce(double& ss, int& bad) {
    #pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        ss += __shfl_xor(ss, off, 64);
        bad |= __shfl_xor(bad, off, 64);
    }
    if constexpr (THREADS > 64) {
        __shared__ double s_ss[THREADS / 64];
        __shared__ int s_bad[THREADS / 64];
        const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
        if (lane == 0) { s_ss[wave] = ss; s_bad[wave] = bad; }
        __syncthreads();
        if (threadIdx.x == 0) {
            ss = s_ss[0];
            bad = s_bad[0];
            for (int w = 1; w < THREADS / 64; ++w) { ss += s_ss[w]; bad |= s_bad[w]; }
        }
    }
}

// ============================================================ pass 1: reduce
// [P1] §2.1 / [P3] technical insight: the reduce-scatter leaves each rank the
// sum of all replicas' gradients over its own shard.  Here the replicas sit
// in one HBM and the sum is an fp32 running sum in replica order; the loss
// scale ([P1] §3.3, §5.1) is undone by one multiply; the inf/nan flag and
// the fp64 sum of squares for clipping ([P1] §6) ride along in registers.
// Each replica is read once, so its loads are nontemporal.
template <int DT, int NR>
__device__ __forceinline__ void sum_quad(const ReplicaPtrs& reps, int nrep, int64_t q, float acc[4]) {
    if constexpr (NR > 0) {
        typename QuadOf<DT>::T x[NR];
        #pragma unroll
        for (int r = 0; r < NR; ++r) x[r] = load_quad<DT>(reps.p[r], q);
        widen4<DT>(x[0], acc);
        #pragma unroll
        for (int r = 1; r < NR; ++r) {
            float y[4];
            widen4<DT>(x[r], y);
            #pragma unroll
            for (int k = 0; k < 4; ++k) acc[k] = acc[k] + y[k];
        }
    } else {
        widen4<DT>(load_quad<DT>(reps.p[0], q), acc);
        for (int r = 1; r < nrep; ++r) {
            float y[4];
            widen4<DT>(load_quad<DT>(reps.p[r], q), y);
            #pragma unroll
            for (int k = 0; k < 4; ++k) acc[k] = acc[k] + y[k];
        }
    }
}

// With ACC the result is added to the slice already in g (gradient
// accumulation over micro-batches; [P1] §3.1 gradient_accumulation_steps).
template <int DT, int NR, bool ACC>
__global__ __launch_bounds__(kReduceThreads) void reduce_kernel(
    ReplicaPtrs reps, int nrep, int64_t n_valid, float inv_scale,
    const zero_step_scalars_t* __restrict__ sc, float* __restrict__ g, Partial* __restrict__ partials,
    uint32_t group) {
    if (sc) inv_scale = sc->inv_scale;            // the step's scalars in device memory
    const int64_t blk = xcd_block(blockIdx.x, group);
    const int64_t q = blk * kReduceThreads + threadIdx.x;
    const int64_t full = n_valid / kQuad;              // complete quads
    double ss = 0.0;
    int bad = 0;
    if (q < full) {
        float acc[4];
        f32x4 prev;
        if constexpr (ACC) prev = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(g) + q);
        sum_quad<DT, NR>(reps, nrep, q, acc);
        f32x4 o;
        #pragma unroll
        for (int k = 0; k < 4; ++k) {
            float gk = acc[k] * inv_scale;
            if constexpr (ACC) gk = prev[k] + gk;
            bad |= !finite(gk);
            ss += static_cast<double>(gk) * static_cast<double>(gk);
            o[k] = gk;
        }
        // streamed out: the next read is a whole pass away
        __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(g) + q);
    } else if (q == full) {
        // Ragged tail: the 0-3 elements after the last complete quad.
        for (int64_t i = q * kQuad; i < n_valid; ++i) {
            float acc = 0.0f;
            for (int r = 0; r < nrep; ++r) {
                const float x = elem<DT>(reps.p[r], i);
                acc = (r == 0) ? x : acc + x;
            }
            float gi = acc * inv_scale;
            if constexpr (ACC) gi = g[i] + gi;
            bad |= !finite(gi);
            ss += static_cast<double>(gi) * static_cast<double>(gi);
            g[i] = gi;
        }
    }
    block_reduce<kReduceThreads>(ss, bad);
    if (threadIdx.x == 0) {
        partials[blk].sumsq = ss;
        partials[blk].flag = bad;
        partials[blk].pad = 0;
    }
}

// ============================================ accumulation before the reduce
// [P1] §1.2.2 (no_sync) and §3.1 (gradient_accumulation_steps): a replica
// sums its micro-batch gradients into an fp32 buffer of its own before the
// replicas are reduced once.  acc = grad widened (FIRST) or acc + grad
// widened; each stream is touched once, so loads and stores are
// nontemporal.
template <int DT, bool FIRST>
__global__ __launch_bounds__(kReduceThreads) void accumulate_local_kernel(
    const u32x2* __restrict__ grad, float* __restrict__ acc, int64_t n, uint32_t group) {
    const int64_t q = xcd_block(blockIdx.x, group) * kReduceThreads + threadIdx.x;
    const int64_t full = n / kQuad;
    if (q < full) {
        float x[4];
        decode4<DT>(__builtin_nontemporal_load(grad + q), x);
        f32x4 o;
        if constexpr (FIRST) {
            o = f32x4{x[0], x[1], x[2], x[3]};
        } else {
            const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(acc) + q);
            #pragma unroll
            for (int k = 0; k < 4; ++k) o[k] = a[k] + x[k];
        }
        __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(acc) + q);
    } else if (q == full) {
        const unsigned short* g16 = reinterpret_cast<const unsigned short*>(grad);
        for (int64_t i = q * kQuad; i < n; ++i) {
            const float x = lo_to_f32<DT>(g16[i]);
            acc[i] = FIRST ? x : acc[i] + x;
        }
    }
}

// ============================================================ fold (small)
// The reduce leaves one partial per block (about a million for a 1.6e9
// element shard).  Block b of the fold sums the contiguous run
// [b * per, (b + 1) * per) of them, per = ceil(n / gridDim), in a fixed
// order, and writes entry b of a slot; block 0 records the entry count.
__global__ __launch_bounds__(256) void fold_kernel(const Partial* __restrict__ parts, int64_t n,
                                                   unsigned char* __restrict__ slot) {
    const int64_t per = (n + gridDim.x - 1) / gridDim.x;
    const int64_t lo = static_cast<int64_t>(blockIdx.x) * per;
    const int64_t hi = lo + per < n ? lo + per : n;
    double ss = 0.0;
    int bad = 0;
    for (int64_t i = lo + threadIdx.x; i < hi; i += 256) {
        ss += parts[i].sumsq;
        bad |= parts[i].flag;
    }
    block_reduce<256>(ss, bad);
    if (threadIdx.x == 0) {
        SlotHeader* h = reinterpret_cast<SlotHeader*>(slot);
        Partial* out = reinterpret_cast<Partial*>(h + 1);
        out[blockIdx.x].sumsq = ss;
        out[blockIdx.x].flag = bad;
        out[blockIdx.x].pad = 0;
        if (blockIdx.x == 0) h->n_blocks = static_cast<int32_t>(gridDim.x);
    }
}

// =========================================================== combine (tiny)
// The implied all-reduce of 16 bytes per rank: global sum of squares, norm,
// clip factor ([P1] §6 gradient_clipping) and the OR of the overflow flags.
constexpr int kCombineThreads = 256;

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const unsigned char* __restrict__ partials, int n_slots, double peer_sumsq, int peer_overflow,
    double max_norm, const zero_step_scalars_t* __restrict__ sc, zero_global_t* __restrict__ out) {
    double ss = 0.0;
    int bad = 0;
    for (int s = 0; s < n_slots; ++s) {
        const SlotHeader* h = reinterpret_cast<const SlotHeader*>(partials + static_cast<size_t>(s) * kSlotBytes);
        int nb = h->n_blocks;
        nb = nb < 0 ? 0 : (nb > kFoldBlocks ? kFoldBlocks : nb);
        const Partial* p = reinterpret_cast<const Partial*>(h + 1);
        for (int b = threadIdx.x; b < nb; b += kCombineThreads) {
            ss += p[b].sumsq;
            bad |= p[b].flag;
        }
    }
    block_reduce<kCombineThreads>(ss, bad);
    if (threadIdx.x == 0) {
        if (sc) {                                 // the step's scalars in device memory
            peer_sumsq = sc->peer_sumsq;
            peer_overflow = sc->peer_overflow;
            max_norm = sc->max_grad_norm;
        }
        ss += peer_sumsq;
        bad |= peer_overflow;
        const double norm = sqrt(ss);
        const double c = max_norm / (norm + 1e-6);
        const int clipped = (max_norm > 0.0 && c < 1.0) ? 1 : 0;
        out->sumsq = ss;
        out->norm = norm;
        out->coef = clipped ? static_cast<float>(c) : 1.0f;
        out->overflow = (bad || !__builtin_isfinite(ss)) ? 1 : 0;
        out->clipped = clipped;
        out->reserved = 0;
    }
}

// ============================================================ pass 2: apply
// AdamW ([P1] §3.1) on the rank's fp32 masters and moments ([P3] FAQ), only
// when no replica overflowed, then the cast of the new masters into the
// rank's slice of the full low-precision buffer ([P1] §2.1 all-gather).
// One element, in fp32 with one rounding per operation (no contraction):
//   m' = b1 m + c1 g;  v' = b2 v + c2 g^2;  d = sqrt(v') * inv_sqrt_bc2 + eps;
//   p' = p * decay - step_size * (m' / d),
// with the per-step constants inv_sqrt_bc2 = 1 / sqrt(1 - b2^t),
// decay = 1 - lr wd and step_size = lr / (1 - b1^t), each rounded once to
// fp32 on the host.
__device__ __forceinline__ void adamw1(float g, float& p, float& m, float& v, const AdamConsts& k) {
    m = k.b1 * m + k.c1 * g;
    v = k.b2 * v + k.c2 * (g * g);
    const float d = __builtin_sqrtf(v) * k.inv_sqrt_bc2 + k.eps;
    p = p * k.decay - k.step_size * (m / d);
}

// coef is 1 when clipping does not apply; multiplying by it is then exact.
// In place (p2 == p, m2 == m, v2 == v) or, with OOP, from one set of state
// buffers into another; the loads are all issued before the stores either
// way.  Every stream is touched once per step, so loads and stores are all
// nontemporal.
//
// TILED: the state is one array of tiles of kStateTile elements, each tile
// holding master, exp_avg and exp_avg_sq of its elements one after the
// other (ZERO_STATE_TILED).  A block's 256 elements are exactly one tile,
// so each wave reads and writes three contiguous 1 KB runs of one 3 KB
// tile instead of three separate arrays: two state streams instead of six.
static_assert(kApplyThreads * kQuad == kStateTile, "one apply block is one state tile");

template <int PT, bool OOP, bool TILED>
__global__ __launch_bounds__(kApplyThreads) void apply_kernel(
    const float* g, const float* p, const float* m, const float* v, float* p2, float* m2, float* v2,
    unsigned short* __restrict__ out, int64_t n_valid, const zero_global_t* __restrict__ glob,
    AdamConsts k, const zero_step_scalars_t* __restrict__ sc, uint32_t group) {
    if (glob->overflow) return;                    // skipped step: touch nothing
    if (sc) {                                      // the step's scalars in device memory
        k.decay = sc->decay;
        k.b1 = sc->beta1;
        k.c1 = sc->one_minus_beta1;
        k.b2 = sc->beta2;
        k.c2 = sc->one_minus_beta2;
        k.step_size = sc->step_size;
        k.inv_sqrt_bc2 = sc->inv_sqrt_bc2;
        k.eps = sc->eps;
    }
    const int64_t blk = xcd_block(blockIdx.x, group);
    if constexpr (TILED) {
        // this block's tile; the quad offsets below are then tile offsets
        const int64_t tile = blk * (3 * kStateTile);
        p += tile;
        m = p + kStateTile;
        v = p + 2 * kStateTile;
        if constexpr (OOP) p2 += tile;
        else p2 = const_cast<float*>(p);
        m2 = p2 + kStateTile;
        v2 = p2 + 2 * kStateTile;
    } else if constexpr (!OOP) {
        p2 = const_cast<float*>(p);
        m2 = const_cast<float*>(m);
        v2 = const_cast<float*>(v);
    }
    const float coef = glob->coef;
    const int64_t q = blk * kApplyThreads + threadIdx.x;
    const int64_t full = n_valid / kQuad;
    // the state's quad index: within the tile, or in the whole array
    const int64_t sq = TILED ? threadIdx.x : q;
    if (q < full) {
        const f32x4 gq = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(g) + q);
        f32x4 pq = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + sq);
        f32x4 mq = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(m) + sq);
        f32x4 vq = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(v) + sq);
        #pragma unroll
        for (int e = 0; e < 4; ++e) {
            float pe = pq[e], me = mq[e], ve = vq[e];
            adamw1(gq[e] * coef, pe, me, ve, k);
            pq[e] = pe; mq[e] = me; vq[e] = ve;
        }
        __builtin_nontemporal_store(pq, reinterpret_cast<f32x4*>(p2) + sq);
        __builtin_nontemporal_store(mq, reinterpret_cast<f32x4*>(m2) + sq);
        __builtin_nontemporal_store(vq, reinterpret_cast<f32x4*>(v2) + sq);
        u32x2 o;
        o.x = pack2<PT>(pq.x, pq.y);
        o.y = pack2<PT>(pq.z, pq.w);
        __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(out) + q);
    } else if (q == full) {
        // the 1-3 elements after the last complete quad, all in this block's
        // tile when TILED (a block's quads cover its tile)
        for (int64_t j = q * kQuad; j < n_valid; ++j) {
            const int64_t sj = TILED ? j - blk * kStateTile : j;
            float pj = p[sj], mj = m[sj], vj = v[sj];
            adamw1(g[j] * coef, pj, mj, vj, k);
            p2[sj] = pj; m2[sj] = mj; v2[sj] = vj;
            out[j] = pack1<PT>(pj);
        }
    }
}

// ================================================================ flatten
// contiguous_gradients ([P1] §5.2): one replica's tensors are copied end to
// end into its flat buffer, then any gap between them and the padding are
// zeroed (as table entries without a source).  Each thread writes
// one aligned 16-byte vector of 8 destination elements.  The source side is
// read as aligned 16-byte vectors and shifted into place, so a tensor's
// arbitrary offset costs no unaligned accesses (the second vector of a
// shifted pair is the next thread's first, served from cache).  The few
// elements before the first and after the last aligned destination vector
// of a tensor are copied one by one by its first block.  The blocks of one
// launch are split over the XCDs in eighths (one contiguous share of the
// grid each), so each XCD copies a contiguous run of the batch's tensors.  The body is stored
// nontemporally: nothing reads it again before the next pass.
constexpr int kFlatBatch = 192;            // tensors per launch (kernel arguments)
constexpr int kFlatThreads = 256;
constexpr int64_t kFlatMaxPiece = int64_t(1) << 30;   // elements per table entry

// Each block finds its table entry before it can issue a load, and blocks
// live about a microsecond, so the lookup must stay short: a binary search
// over at most kFlatDirect entries, or over the entries of one slot of a
// coarse index (slot i = blocks [i << shift, (i + 1) << shift)) for larger
// tables.  All of it is read with scalar loads from the kernel arguments.
constexpr int kFlatSlots = 32;
constexpr int kFlatDirect = 16;

struct FlatBatch {
    const unsigned short* src[kFlatBatch];   // nullptr: write zeros
    // first flat element, counted from dst_base: a launch's pieces span
    // less than 2^32 elements (the launcher starts a new batch otherwise)
    uint32_t dst[kFlatBatch];
    uint32_t n[kFlatBatch];                  // elements (a piece is at most 2^30)
    int64_t dst_base;
    int32_t first_block[kFlatBatch + 1];     // prefix of blocks per entry
    int32_t count;
    int32_t n_blocks;                        // = first_block[count]
    int32_t slot_shift;
    int32_t slot_entry[kFlatSlots + 1];      // entry owning block i << shift; then count - 1
};
static_assert(sizeof(FlatBatch) <= 4000, "the table travels as kernel arguments");

// Elements k..k+7 of the 16 packed in (lo, hi), k uniform in 1..7.
__device__ __forceinline__ u32x4 shift_pick(const u32x4 lo, const u32x4 hi, int k) {
    const unsigned w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    u32x4 o;
#define ZERO_PICK_EVEN(K) o.x = w[K / 2]; o.y = w[K / 2 + 1]; o.z = w[K / 2 + 2]; o.w = w[K / 2 + 3];
#define ZERO_PICK_ODD(K)                                              \
    o.x = __builtin_amdgcn_alignbyte(w[(K + 1) / 2], w[(K - 1) / 2], 2);     \
    o.y = __builtin_amdgcn_alignbyte(w[(K + 1) / 2 + 1], w[(K - 1) / 2 + 1], 2); \
    o.z = __builtin_amdgcn_alignbyte(w[(K + 1) / 2 + 2], w[(K - 1) / 2 + 2], 2); \
    o.w = __builtin_amdgcn_alignbyte(w[(K + 1) / 2 + 3], w[(K - 1) / 2 + 3], 2);
    switch (k) {
        case 1: ZERO_PICK_ODD(1) break;
        case 2: ZERO_PICK_EVEN(2) break;
        case 3: ZERO_PICK_ODD(3) break;
        case 4: ZERO_PICK_EVEN(4) break;
        case 5: ZERO_PICK_ODD(5) break;
        case 6: ZERO_PICK_EVEN(6) break;
        default: ZERO_PICK_ODD(7) break;
    }
#undef ZERO_PICK_EVEN
#undef ZERO_PICK_ODD
    return o;
}

__global__ __launch_bounds__(kFlatThreads) void flatten_kernel(FlatBatch b, unsigned short* __restrict__ flat) {
    const int64_t blk = xcd_block(blockIdx.x, gridDim.x / kXcds);
    if (blk >= b.n_blocks) return;                    // grid rounded up to the XCD count
    // Which table entry owns this block: a binary search over the prefix,
    // narrowed by the coarse index when the table is large.
    int lo = 0, hi = b.count - 1;
    if (hi >= kFlatDirect) {
        const int slot = static_cast<int>(blk >> b.slot_shift);
        lo = b.slot_entry[slot];
        hi = b.slot_entry[slot + 1];
    }
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (b.first_block[mid] <= blk) lo = mid; else hi = mid - 1;
    }
    const int t = lo;
    const int64_t jb = blk - b.first_block[t];
    const unsigned short* src = b.src[t];
    const int64_t d0 = b.dst_base + b.dst[t], n = b.n[t], d1 = d0 + n;
    // Aligned body [a0, a1) of the destination, head [d0, a0), tail [a1, d1).
    int64_t a0 = (d0 + 7) & ~int64_t(7);
    if (a0 > d1) a0 = d1;
    int64_t a1 = d1 & ~int64_t(7);
    if (a1 < a0) a1 = a0;
    u32x4* dvec = reinterpret_cast<u32x4*>(flat);
    const int64_t nv = (a1 - a0) / 8;
    const int64_t q = jb * kFlatThreads + threadIdx.x;   // body vector of this thread
    if (src == nullptr) {
        if (q < nv) __builtin_nontemporal_store(u32x4{0u, 0u, 0u, 0u}, dvec + a0 / 8 + q);
        if (jb == 0) {
            if (threadIdx.x < a0 - d0) flat[d0 + threadIdx.x] = 0;
            if (threadIdx.x >= 8 && threadIdx.x - 8 < d1 - a1) flat[a1 + threadIdx.x - 8] = 0;
        }
        return;
    }
    // Source element e of the entry sits at aligned-vector element e + ms
    // of `sbase`; the body's first source element is a0 - d0.
    const int ms = static_cast<int>((reinterpret_cast<uintptr_t>(src) & 15u) >> 1);
    const u32x4* sbase = reinterpret_cast<const u32x4*>(src - ms);
    const int64_t s0 = a0 - d0 + ms;        // aligned-space index of the body start
    const int k = static_cast<int>(s0 & 7);
    const int64_t sv0 = s0 >> 3;            // aligned vector holding it
    if (q < nv) {
        u32x4 o;
        if (k == 0) o = sbase[sv0 + q];
        else o = shift_pick(sbase[sv0 + q], sbase[sv0 + q + 1], k);
        __builtin_nontemporal_store(o, dvec + a0 / 8 + q);
    }
    if (jb == 0) {
        if (threadIdx.x < a0 - d0) flat[d0 + threadIdx.x] = src[threadIdx.x];
        if (threadIdx.x >= 8 && threadIdx.x - 8 < d1 - a1) {
            const int64_t e = a1 + threadIdx.x - 8;
            flat[e] = src[e - d0];
        }
    }
}

// ========================================================= state layouts
// Moves n elements of a rank's fp32 optimizer state, all three fields,
// from element src_first of one state to element dst_first of another;
// either side separate (three arrays) or tiled (ZERO_STATE_TILED), and a
// NULL source writes zeros.  One thread per element and field: consecutive
// threads touch consecutive addresses on both sides.  Used for layout
// conversion and for re-partitioning a tiled state; neither is on the
// step's path.
struct StateRef {
    float* f[3];          // separate: the three arrays; tiled: f[0] is the tiled array
};

template <bool TILED>
__device__ __forceinline__ int64_t state_index(int64_t i, int field) {
    if constexpr (TILED)
        return (i / kStateTile) * (3 * kStateTile) + field * kStateTile + (i % kStateTile);
    else
        return i;
}

template <bool SRC_TILED, bool DST_TILED>
__global__ __launch_bounds__(256) void state_move_kernel(StateRef src, int64_t src_first, StateRef dst,
                                                         int64_t dst_first, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int field = blockIdx.y;
    if (i >= n) return;
    const float* sb = SRC_TILED ? src.f[0] : src.f[field];
    float* db = DST_TILED ? dst.f[0] : dst.f[field];
    const float x = sb ? sb[state_index<SRC_TILED>(src_first + i, field)] : 0.0f;
    db[state_index<DST_TILED>(dst_first + i, field)] = x;
}

// ================================================================ launches
int launch_error(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(ZERO_EDEVICE, "%s: %s", what, hipGetErrorString(e));
    return ZERO_OK;
}

template <int DT, bool ACC>
void launch_reduce_dt(const ReplicaPtrs& reps, int nrep, int64_t n_valid, float inv,
                      const zero_step_scalars_t* sc, float* g, Partial* parts, hipStream_t st) {
    const Grid gr = grid_for(n_valid, kReduceThreads);
    const dim3 grid(static_cast<unsigned>(gr.blocks));
    const uint32_t group = static_cast<uint32_t>(gr.group);
#define ZERO_REDUCE_CASE(NR)                                                                   \
    case NR:                                                                                   \
        hipLaunchKernelGGL((reduce_kernel<DT, NR, ACC>), grid, dim3(kReduceThreads), 0, st, reps, \
                           nrep, n_valid, inv, sc, g, parts, group);                           \
        break;
    switch (nrep) {
        ZERO_REDUCE_CASE(1) ZERO_REDUCE_CASE(2) ZERO_REDUCE_CASE(3) ZERO_REDUCE_CASE(4)
        ZERO_REDUCE_CASE(5) ZERO_REDUCE_CASE(6) ZERO_REDUCE_CASE(7) ZERO_REDUCE_CASE(8)
        default:
            hipLaunchKernelGGL((reduce_kernel<DT, 0, ACC>), grid, dim3(kReduceThreads), 0, st, reps,
                               nrep, n_valid, inv, sc, g, parts, group);
    }
#undef ZERO_REDUCE_CASE
}

// Pass 1 into the workspace; with fold, its block partials then go to `slot`.
int launch_pass1(const zero_step_args* a, hipStream_t st) {
    // An empty rank (valid_numel 0) may pass no replica array at all; its
    // launch reads no replica element.
    ReplicaPtrs reps;
    for (int r = 0; r < ZERO_MAX_REPLICAS; ++r)
        reps.p[r] = (a->replica_grad && r < a->n_replicas) ? a->replica_grad[r] : nullptr;
    const float inv = unscale_factor(a);
    const zero_step_scalars_t* sc = a->scalars;
    unsigned char* ws = static_cast<unsigned char*>(a->workspace);
    float* g = reinterpret_cast<float*>(ws);
    Partial* parts = reinterpret_cast<Partial*>(ws + ws_blocks_offset(a->shard_numel));
#define ZERO_PASS1(DT)                                                                          \
    do {                                                                                        \
        if (a->accumulate)                                                                      \
            launch_reduce_dt<DT, true>(reps, a->n_replicas, a->valid_numel, inv, sc, g, parts, st); \
        else                                                                                    \
            launch_reduce_dt<DT, false>(reps, a->n_replicas, a->valid_numel, inv, sc, g, parts, st); \
    } while (0)
    switch (a->grad_dtype) {
        case ZERO_BF16: ZERO_PASS1(ZERO_BF16); break;
        case ZERO_FP16: ZERO_PASS1(ZERO_FP16); break;
        default: ZERO_PASS1(ZERO_FP32); break;
    }
#undef ZERO_PASS1
    return launch_error("reduce kernel launch");
}

// Pass 1 into the workspace, then the fold of its block partials into `slot`.
int launch_reduce(const zero_step_args* a, unsigned char* slot, hipStream_t st) {
    int rc = launch_pass1(a, st);
    if (rc) return rc;
    const int64_t nb = reduce_blocks_for(a->valid_numel);
    const Partial* parts = reinterpret_cast<const Partial*>(static_cast<unsigned char*>(a->workspace) +
                                                            ws_blocks_offset(a->shard_numel));
    hipLaunchKernelGGL(fold_kernel, dim3(fold_blocks_for(nb)), dim3(256), 0, st, parts, nb, slot);
    return launch_error("fold kernel launch");
}

int launch_combine(const void* partials, int n_slots, double peer_ss, int peer_of, double max_norm,
                   const zero_step_scalars_t* sc, void* global, hipStream_t st) {
    hipLaunchKernelGGL(combine_kernel, dim3(1), dim3(kCombineThreads), 0, st,
                       static_cast<const unsigned char*>(partials), n_slots, peer_ss, peer_of, max_norm,
                       sc, static_cast<zero_global_t*>(global));
    return launch_error("combine kernel launch");
}

int launch_apply(const zero_step_args* a, const void* global, hipStream_t st) {
    const AdamConsts k = adam_consts(a->lr, a->beta1, a->beta2, a->eps, a->weight_decay, a->step);
    const Grid gr = grid_for(a->valid_numel, kApplyThreads);
    const dim3 grid(static_cast<unsigned>(gr.blocks));
    const uint32_t group = static_cast<uint32_t>(gr.group);
    unsigned short* out = param_out(a);
    const zero_global_t* gl = static_cast<const zero_global_t*>(global);
    const float* g = static_cast<const float*>(a->workspace);
    const bool oop = a->master_out != nullptr;
    const bool tiled = a->state_layout == ZERO_STATE_TILED;
    float* p2 = oop ? a->master_out : a->master;
    float* m2 = oop ? a->exp_avg_out : a->exp_avg;
    float* v2 = oop ? a->exp_avg_sq_out : a->exp_avg_sq;
#define ZERO_APPLY(PT, OOP, TILED)                                                                  \
    hipLaunchKernelGGL((apply_kernel<PT, OOP, TILED>), grid, dim3(kApplyThreads), 0, st, g,          \
                       a->master, a->exp_avg, a->exp_avg_sq, p2, m2, v2, out, a->valid_numel, gl, k, \
                       a->scalars, group)
#define ZERO_APPLY_LAYOUT(PT, OOP) \
    do { if (tiled) ZERO_APPLY(PT, OOP, true); else ZERO_APPLY(PT, OOP, false); } while (0)
    if (a->param_dtype == ZERO_BF16) {
        if (oop) ZERO_APPLY_LAYOUT(ZERO_BF16, true); else ZERO_APPLY_LAYOUT(ZERO_BF16, false);
    } else {
        if (oop) ZERO_APPLY_LAYOUT(ZERO_FP16, true); else ZERO_APPLY_LAYOUT(ZERO_FP16, false);
    }
#undef ZERO_APPLY_LAYOUT
#undef ZERO_APPLY
    return launch_error("apply kernel launch");
}

// Queue one state move (see state_move_kernel); n >= 0.
int launch_state_move(const StateRef& src, bool src_tiled, int64_t src_first, const StateRef& dst,
                      bool dst_tiled, int64_t dst_first, int64_t n, hipStream_t st) {
    if (n <= 0) return ZERO_OK;
    if ((n + 255) / 256 > INT32_MAX) return fail(ZERO_EINVAL, "%lld elements in one state move", (long long)n);
    const dim3 grid(static_cast<unsigned>((n + 255) / 256), 3);
#define ZERO_MOVE(S, D) \
    hipLaunchKernelGGL((state_move_kernel<S, D>), grid, dim3(256), 0, st, src, src_first, dst, dst_first, n)
    if (src_tiled) {
        if (dst_tiled) ZERO_MOVE(true, true); else ZERO_MOVE(true, false);
    } else {
        if (dst_tiled) ZERO_MOVE(false, true); else ZERO_MOVE(false, false);
    }
#undef ZERO_MOVE
    return launch_error("state move kernel launch");
}

// Copy n ranges of 16-bit values, range t from src(t) to flat elements
// [dst(t), dst(t) + len(t)) (ascending, non-overlapping), zero any gap
// between consecutive ranges, then zero [end of the last range,
// flat_numel); batched into flatten launches.  Elements before the first
// range are not touched.
template <class Src, class Dst, class Len>
int copy_ranges(int32_t n, Src src_of, Dst dst_of, Len len_of, unsigned short* flat, int64_t flat_numel,
                hipStream_t st) {
    FlatBatch b;
    b.count = 0;
    int64_t blocks = 0;
    auto flush = [&]() -> int {
        if (b.count == 0) return ZERO_OK;
        b.first_block[b.count] = static_cast<int32_t>(blocks);
        b.n_blocks = static_cast<int32_t>(blocks);
        // The coarse index: at most kFlatSlots slots of 2^shift blocks, each
        // naming the entry that owns its first block.
        int shift = 0;
        while (((blocks - 1) >> shift) >= kFlatSlots) ++shift;
        const int slots = static_cast<int>((blocks - 1) >> shift) + 1;
        b.slot_shift = shift;
        int owner = 0;
        for (int i = 0; i < slots; ++i) {
            const int64_t first = static_cast<int64_t>(i) << shift;
            while (owner + 1 < b.count && b.first_block[owner + 1] <= first) ++owner;
            b.slot_entry[i] = owner;
        }
        b.slot_entry[slots] = b.count - 1;
        const int64_t grid = (blocks + kXcds - 1) / kXcds * kXcds;
        hipLaunchKernelGGL(flatten_kernel, dim3(static_cast<unsigned>(grid)), dim3(kFlatThreads), 0, st,
                           b, flat);
        b.count = 0;
        blocks = 0;
        return launch_error("flatten kernel launch");
    };
    // One table entry per piece of at most kFlatMaxPiece elements; a
    // piece's blocks cover its aligned body vectors, at least one block
    // (its head and tail).
    auto add_piece = [&](const unsigned short* src, int64_t dst, int64_t n) -> int {
        const int64_t a0 = (dst + 7) & ~int64_t(7);
        const int64_t body = (dst + n) / 8 * 8 > a0 ? ((dst + n) / 8 * 8 - a0) / 8 : 0;
        int64_t nb = (body + kFlatThreads - 1) / kFlatThreads;
        if (nb < 1) nb = 1;
        if (b.count == kFlatBatch || blocks + nb > (int64_t(1) << 30) ||
            (b.count > 0 && dst + n - b.dst_base > int64_t(0xffffffff))) {
            int rc = flush();
            if (rc) return rc;
        }
        if (b.count == 0) b.dst_base = dst;
        b.src[b.count] = src;
        b.dst[b.count] = static_cast<uint32_t>(dst - b.dst_base);
        b.n[b.count] = static_cast<uint32_t>(n);
        b.first_block[b.count] = static_cast<int32_t>(blocks);
        blocks += nb;
        ++b.count;
        return ZERO_OK;
    };
    auto add = [&](const void* src, int64_t dst, int64_t n) -> int {
        const unsigned short* s16 = static_cast<const unsigned short*>(src);
        for (int64_t done = 0; done < n; done += kFlatMaxPiece) {
            const int64_t len = n - done < kFlatMaxPiece ? n - done : kFlatMaxPiece;
            int rc = add_piece(s16 ? s16 + done : nullptr, dst + done, len);
            if (rc) return rc;
        }
        return ZERO_OK;
    };
    int rc;
    int64_t end = 0;
    for (int32_t t = 0; t < n; ++t) {
        const int64_t d = dst_of(t), len = len_of(t);
        if (t > 0 && d > end && (rc = add(nullptr, end, d - end))) return rc;
        if ((rc = add(src_of(t), d, len))) return rc;
        end = d + len;
    }
    if ((rc = add(nullptr, end, flat_numel - end))) return rc;
    return flush();
}

// One rank's whole step once its arguments are checked: pass 1 and the fold
// into the workspace's own slot, a combine with the peers' contribution,
// pass 2, and the optional read-back of the result.
int run_step(const zero_step_args* a, double peer_sumsq, int32_t peer_overflow, zero_step_info* info,
             hipStream_t st) {
    unsigned char* ws = static_cast<unsigned char*>(a->workspace);
    unsigned char* slot = ws + ws_slot_offset(a->shard_numel);
    void* global = ws + ws_global_offset(a->shard_numel);
    int rc;
    if ((rc = launch_reduce(a, slot, st))) return rc;
    if ((rc = launch_combine(slot, 1, peer_sumsq, peer_overflow ? 1 : 0, a->max_grad_norm, a->scalars,
                             global, st)))
        return rc;
    if ((rc = launch_apply(a, global, st))) return rc;
    if (info) {
        hipError_t e = hipMemcpyAsync(info, global, sizeof(zero_global_t), hipMemcpyDeviceToHost, st);
        if (e == hipSuccess) e = hipStreamSynchronize(st);
        if (e != hipSuccess) return fail(ZERO_EDEVICE, "reading the step result: %s", hipGetErrorString(e));
    }
    return ZERO_OK;
}

}  // namespace
}  // namespace zero

using namespace zero;

// ---------------------------------------------------- allocation-free step
// The workspace of zero_shard_step_noalloc: one array per GPU, loaded with
// the library's code object and held until the process ends, sized for the
// largest shard that call accepts.  Host code never passes its name to a
// kernel (on the host it is only a stand-in for the symbol); it takes the
// device address that hipGetSymbolAddress returns for the current device.
constexpr size_t kNoAllocBytes = ws_total_bytes(ZERO_NOALLOC_MAX_SHARD);
static_assert(kNoAllocBytes == 67375616, "scratch: 64 MiB of fp32 gradient plus partials");
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];       // device address of `scratch`, per device

// The current device's address of `scratch`, looked up on the first call on
// that device and kept.
int noalloc_scratch(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(ZERO_EDEVICE, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(ZERO_EDEVICE, "device %d is beyond the %d this library tracks", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(ZERO_EDEVICE, "hipGetSymbolAddress of the scratch array on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return ZERO_OK;
}
}  // namespace

extern "C" {

size_t zero_shard_workspace_bytes(int64_t shard_numel) {
    if (shard_numel < 0) return 0;
    return ws_global_offset(shard_numel) + 256;
}

size_t zero_partials_bytes(int32_t n_slots) {
    if (n_slots < 0) return 0;
    return static_cast<size_t>(n_slots) * kSlotBytes;
}

int zero_shard_reduce(const zero_step_args* a, int32_t slot, void* partials_dev, void* stream) {
    clear_error();
    int rc = validate_step_args(a);
    if (rc) return rc;
    if (slot < 0) return fail(ZERO_EINVAL, "slot %d < 0", slot);
    if (!partials_dev) return fail(ZERO_EINVAL, "partials_dev is NULL");
    if (!aligned16(partials_dev)) return fail(ZERO_EALIGN, "partials_dev is not 16-byte aligned");
    unsigned char* s = static_cast<unsigned char*>(partials_dev) + static_cast<size_t>(slot) * kSlotBytes;
    return launch_reduce(a, s, static_cast<hipStream_t>(stream));
}

int zero_shard_accumulate(const zero_step_args* a, void* stream) {
    clear_error();
    int rc = validate_step_args(a);
    if (rc) return rc;
    return launch_pass1(a, static_cast<hipStream_t>(stream));
}

int zero_accumulate_local(const void* grad, int32_t grad_dtype, float* acc, int64_t n,
                          int32_t first, void* stream) {
    clear_error();
    if (n < 0) return fail(ZERO_EINVAL, "n %lld < 0", (long long)n);
    if (grad_dtype != ZERO_FP16 && grad_dtype != ZERO_BF16)
        return fail(ZERO_EINVAL, "grad_dtype %d is not ZERO_FP16 or ZERO_BF16", grad_dtype);
    if (first != 0 && first != 1) return fail(ZERO_EINVAL, "first %d is not 0 or 1", first);
    if (n == 0) return ZERO_OK;
    if (!grad || !acc) return fail(ZERO_EINVAL, "grad or acc is NULL");
    if (!aligned16(grad) || !aligned16(acc))
        return fail(ZERO_EALIGN, "grad or acc is not 16-byte aligned");
    const unsigned char* g0 = static_cast<const unsigned char*>(grad);
    const unsigned char* a0 = reinterpret_cast<const unsigned char*>(acc);
    if (g0 < a0 + 4 * n && a0 < g0 + 2 * n) return fail(ZERO_EINVAL, "grad and acc overlap");
    const Grid gr = grid_for(n, kReduceThreads);
    const dim3 grid(static_cast<unsigned>(gr.blocks));
    const uint32_t group = static_cast<uint32_t>(gr.group);
    const u32x2* g = static_cast<const u32x2*>(grad);
    hipStream_t st = static_cast<hipStream_t>(stream);
#define ZERO_ACC_LOCAL(DT, FIRST) \
    hipLaunchKernelGGL((accumulate_local_kernel<DT, FIRST>), grid, dim3(kReduceThreads), 0, st, g, acc, n, group)
    if (grad_dtype == ZERO_BF16) {
        if (first) ZERO_ACC_LOCAL(ZERO_BF16, true); else ZERO_ACC_LOCAL(ZERO_BF16, false);
    } else {
        if (first) ZERO_ACC_LOCAL(ZERO_FP16, true); else ZERO_ACC_LOCAL(ZERO_FP16, false);
    }
#undef ZERO_ACC_LOCAL
    return launch_error("accumulate kernel launch");
}

int zero_shard_combine(const void* partials_dev, int32_t n_slots, double max_grad_norm,
                       void* global_dev, void* stream) {
    clear_error();
    if (!partials_dev || !global_dev) return fail(ZERO_EINVAL, "partials_dev or global_dev is NULL");
    if (n_slots < 1) return fail(ZERO_EINVAL, "n_slots %d < 1", n_slots);
    if (std::isnan(max_grad_norm)) return fail(ZERO_EINVAL, "max_grad_norm is NaN");
    if (!aligned16(partials_dev) || !aligned16(global_dev))
        return fail(ZERO_EALIGN, "partials_dev or global_dev is not 16-byte aligned");
    return launch_combine(partials_dev, n_slots, 0.0, 0, max_grad_norm, nullptr, global_dev,
                          static_cast<hipStream_t>(stream));
}

int zero_shard_apply(const zero_step_args* a, const void* global_dev, void* stream) {
    clear_error();
    int rc = validate_step_args(a);
    if (rc) return rc;
    if (!global_dev) return fail(ZERO_EINVAL, "global_dev is NULL");
    if (!aligned16(global_dev)) return fail(ZERO_EALIGN, "global_dev is not 16-byte aligned");
    return launch_apply(a, global_dev, static_cast<hipStream_t>(stream));
}

int zero_shard_step(const zero_step_args* a, double peer_sumsq, int32_t peer_overflow,
                    zero_step_info* info, void* stream) {
    clear_error();
    int rc = validate_step_args(a);
    if (rc) return rc;
    if (!(peer_sumsq >= 0.0)) return fail(ZERO_EINVAL, "peer_sumsq must be >= 0 (got NaN or negative)");
    return run_step(a, peer_sumsq, peer_overflow, info, static_cast<hipStream_t>(stream));
}

int zero_shard_step_noalloc(const zero_step_args* a, double peer_sumsq, int32_t peer_overflow,
                            zero_step_info* info, void* stream) {
    clear_error();
    int rc = validate_step_args(a, false);
    if (rc) return rc;
    if (a->workspace || a->workspace_bytes)
        return fail(ZERO_EINVAL, "workspace must be NULL and workspace_bytes 0: this call uses the "
                                 "library's own scratch memory");
    if (a->accumulate)
        return fail(ZERO_EINVAL, "accumulate must be 0: the scratch memory holds no accumulation "
                                 "window between calls");
    if (a->shard_numel > ZERO_NOALLOC_MAX_SHARD)
        return fail(ZERO_ESIZE, "shard_numel %lld exceeds ZERO_NOALLOC_MAX_SHARD (%lld)",
                    (long long)a->shard_numel, (long long)ZERO_NOALLOC_MAX_SHARD);
    if (!(peer_sumsq >= 0.0)) return fail(ZERO_EINVAL, "peer_sumsq must be >= 0 (got NaN or negative)");
    void* ws = nullptr;
    if ((rc = noalloc_scratch(&ws))) return rc;
    zero_step_args b = *a;
    b.workspace = ws;
    b.workspace_bytes = kNoAllocBytes;
    return run_step(&b, peer_sumsq, peer_overflow, info, static_cast<hipStream_t>(stream));
}

int zero_bucket_flatten(const zero_tensor_slot_t* slots, int32_t n_tensors, const void* const* src_dev,
                        int32_t dtype, void* flat_dev, int64_t flat_numel, void* stream) {
    clear_error();
    if (n_tensors < 0) return fail(ZERO_EINVAL, "n_tensors %d < 0", n_tensors);
    if (!flat_dev || (n_tensors > 0 && (!slots || !src_dev)))
        return fail(ZERO_EINVAL, "a required pointer is NULL");
    if (dtype != ZERO_FP16 && dtype != ZERO_BF16)
        return fail(ZERO_EINVAL, "dtype %d is not ZERO_FP16 or ZERO_BF16", dtype);
    if (flat_numel < 0) return fail(ZERO_EINVAL, "flat_numel %lld < 0", (long long)flat_numel);
    if (!aligned16(flat_dev)) return fail(ZERO_EALIGN, "flat_dev is not 16-byte aligned");
    int64_t prev_end = 0;
    for (int32_t t = 0; t < n_tensors; ++t) {
        const zero_tensor_slot_t& s = slots[t];
        if (s.numel < 0 || s.offset < prev_end || s.offset > flat_numel || s.numel > flat_numel - s.offset)
            return fail(ZERO_EINVAL, "slot %d [%lld, +%lld) is out of order or outside [0, %lld)", t,
                        (long long)s.offset, (long long)s.numel, (long long)flat_numel);
        if (s.numel > 0 && !src_dev[t]) return fail(ZERO_EINVAL, "src_dev[%d] is NULL", t);
        if (reinterpret_cast<uintptr_t>(src_dev[t]) & 1u)
            return fail(ZERO_EALIGN, "src_dev[%d] is not 2-byte aligned", t);
        prev_end = s.offset + s.numel;
    }
    return copy_ranges(
        n_tensors, [&](int32_t t) { return static_cast<const unsigned short*>(src_dev[t]); },
        [&](int32_t t) { return slots[t].offset; }, [&](int32_t t) { return slots[t].numel; },
        static_cast<unsigned short*>(flat_dev), flat_numel, static_cast<hipStream_t>(stream));
}

int zero_gather_params(const zero_partition_t* p, const void* const* shards, int32_t dtype,
                       int64_t lo, int64_t hi, void* dst, void* stream) {
    clear_error();
    if (!p || !shards || !dst) return fail(ZERO_EINVAL, "a required pointer is NULL");
    if (dtype != ZERO_FP16 && dtype != ZERO_BF16)
        return fail(ZERO_EINVAL, "dtype %d is not ZERO_FP16 or ZERO_BF16", dtype);
    int rc = check_partition(p, "the partition");
    if (rc) return rc;
    if (lo < 0 || hi < lo || hi > p->numel)
        return fail(ZERO_EINVAL, "range [%lld, %lld) outside [0, %lld)", (long long)lo,
                    (long long)hi, (long long)p->numel);
    if (!aligned16(dst)) return fail(ZERO_EALIGN, "dst is not 16-byte aligned");
    if (hi == lo) return ZERO_OK;
    const int64_t s = p->shard_numel, k0 = lo / s;
    const int32_t n = static_cast<int32_t>((hi - 1) / s - k0 + 1);
    for (int32_t q = 0; q < n; ++q) {
        if (!shards[k0 + q]) return fail(ZERO_EINVAL, "shards[%lld] is NULL", (long long)(k0 + q));
        if (reinterpret_cast<uintptr_t>(shards[k0 + q]) & 1u)
            return fail(ZERO_EALIGN, "shards[%lld] is not 2-byte aligned", (long long)(k0 + q));
    }
    auto a_of = [&](int32_t q) { const int64_t k = k0 + q; return lo > k * s ? lo : k * s; };
    auto b_of = [&](int32_t q) { const int64_t e = (k0 + q + 1) * s; return hi < e ? hi : e; };
    return copy_ranges(
        n,
        [&](int32_t q) {
            return static_cast<const unsigned short*>(shards[k0 + q]) + (a_of(q) - (k0 + q) * s);
        },
        [&](int32_t q) { return a_of(q) - lo; }, [&](int32_t q) { return b_of(q) - a_of(q); },
        static_cast<unsigned short*>(dst), hi - lo, static_cast<hipStream_t>(stream));
}

int zero_repartition(const zero_partition_t* from, const float* const* src_dev,
                     const zero_partition_t* to, float* const* dst_dev, void* stream) {
    clear_error();
    if (!from || !to || !src_dev || !dst_dev) return fail(ZERO_EINVAL, "a required pointer is NULL");
    int rc;
    if ((rc = check_partition(from, "from"))) return rc;
    if ((rc = check_partition(to, "to"))) return rc;
    if (from->numel != to->numel)
        return fail(ZERO_EINVAL, "partitions cover %lld and %lld elements", (long long)from->numel,
                    (long long)to->numel);
    for (int32_t k = 0; k < from->world_size; ++k) {
        if (zero_partition_valid_numel(from, k) > 0 && !src_dev[k])
            return fail(ZERO_EINVAL, "src_dev[%d] is NULL", k);
        if (reinterpret_cast<uintptr_t>(src_dev[k]) & 3u)
            return fail(ZERO_EALIGN, "src_dev[%d] is not 4-byte aligned", k);
    }
    for (int32_t j = 0; j < to->world_size; ++j) {
        if (to->shard_numel > 0 && !dst_dev[j]) return fail(ZERO_EINVAL, "dst_dev[%d] is NULL", j);
        if (!aligned16(dst_dev[j])) return fail(ZERO_EALIGN, "dst_dev[%d] is not 16-byte aligned", j);
    }
    // New rank j copies the pieces of its read plan, each one contiguous
    // run of an old rank's slice, as 16-bit halves through the flatten
    // kernel; its padding is zero-filled after them.
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t s_new = to->shard_numel;
    std::vector<zero_repartition_piece_t> plan;
    for (int32_t j = 0; j < to->world_size; ++j) {
        if (s_new == 0) break;
        int32_t n_pieces = 0;
        rc = zero_repartition_plan(from, to, j, plan.data(), static_cast<int32_t>(plan.size()),
                                   &n_pieces);
        if (rc == ZERO_ESIZE) {
            try {
                plan.resize(static_cast<size_t>(n_pieces));
            } catch (...) {
                return fail(ZERO_ESIZE, "no host memory for a plan of %d pieces", n_pieces);
            }
            rc = zero_repartition_plan(from, to, j, plan.data(), n_pieces, &n_pieces);
        }
        if (rc) return rc;
        rc = copy_ranges(
            n_pieces,
            [&](int32_t q) {
                return reinterpret_cast<const unsigned short*>(src_dev[plan[q].old_rank] +
                                                               plan[q].old_offset);
            },
            [&](int32_t q) { return 2 * plan[q].new_offset; },
            [&](int32_t q) { return 2 * plan[q].count; },
            reinterpret_cast<unsigned short*>(dst_dev[j]), 2 * s_new, st);
        if (rc) return rc;
    }
    return ZERO_OK;
}

int zero_state_tile(const float* master, const float* exp_avg, const float* exp_avg_sq, int64_t n,
                    float* tiled, int64_t first, void* stream) {
    clear_error();
    if (n < 0 || first < 0) return fail(ZERO_EINVAL, "n %lld or first %lld < 0", (long long)n,
                                        (long long)first);
    if (n == 0) return ZERO_OK;
    if (!master || !exp_avg || !exp_avg_sq || !tiled)
        return fail(ZERO_EINVAL, "a required pointer is NULL");
    if (!aligned16(master) || !aligned16(exp_avg) || !aligned16(exp_avg_sq) || !aligned16(tiled))
        return fail(ZERO_EALIGN, "a pointer is not 16-byte aligned");
    if (n > (INT64_MAX - first) / 3) return fail(ZERO_EINVAL, "first + n overflows");
    StateRef src{{const_cast<float*>(master), const_cast<float*>(exp_avg), const_cast<float*>(exp_avg_sq)}};
    StateRef dst{{tiled, nullptr, nullptr}};
    return launch_state_move(src, false, 0, dst, true, first, n, static_cast<hipStream_t>(stream));
}

int zero_state_untile(const float* tiled, int64_t first, int64_t n, float* master, float* exp_avg,
                      float* exp_avg_sq, void* stream) {
    clear_error();
    if (n < 0 || first < 0) return fail(ZERO_EINVAL, "n %lld or first %lld < 0", (long long)n,
                                        (long long)first);
    if (n == 0) return ZERO_OK;
    if (!master || !exp_avg || !exp_avg_sq || !tiled)
        return fail(ZERO_EINVAL, "a required pointer is NULL");
    if (!aligned16(master) || !aligned16(exp_avg) || !aligned16(exp_avg_sq) || !aligned16(tiled))
        return fail(ZERO_EALIGN, "a pointer is not 16-byte aligned");
    if (n > (INT64_MAX - first) / 3) return fail(ZERO_EINVAL, "first + n overflows");
    StateRef src{{const_cast<float*>(tiled), nullptr, nullptr}};
    StateRef dst{{master, exp_avg, exp_avg_sq}};
    return launch_state_move(src, true, first, dst, false, 0, n, static_cast<hipStream_t>(stream));
}

int zero_repartition_tiled(const zero_partition_t* from, const float* const* src_dev,
                           const zero_partition_t* to, float* const* dst_dev, void* stream) {
    clear_error();
    if (!from || !to || !src_dev || !dst_dev) return fail(ZERO_EINVAL, "a required pointer is NULL");
    int rc;
    if ((rc = check_partition(from, "from"))) return rc;
    if ((rc = check_partition(to, "to"))) return rc;
    if (from->numel != to->numel)
        return fail(ZERO_EINVAL, "partitions cover %lld and %lld elements", (long long)from->numel,
                    (long long)to->numel);
    for (int32_t k = 0; k < from->world_size; ++k) {
        if (zero_partition_valid_numel(from, k) > 0 && !src_dev[k])
            return fail(ZERO_EINVAL, "src_dev[%d] is NULL", k);
        if (!aligned16(src_dev[k])) return fail(ZERO_EALIGN, "src_dev[%d] is not 16-byte aligned", k);
    }
    for (int32_t j = 0; j < to->world_size; ++j) {
        if (to->shard_numel > 0 && !dst_dev[j]) return fail(ZERO_EINVAL, "dst_dev[%d] is NULL", j);
        if (!aligned16(dst_dev[j])) return fail(ZERO_EALIGN, "dst_dev[%d] is not 16-byte aligned", j);
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    std::vector<zero_repartition_piece_t> plan;
    for (int32_t j = 0; j < to->world_size; ++j) {
        if (to->shard_numel == 0) break;
        int32_t n_pieces = 0;
        rc = zero_repartition_plan(from, to, j, plan.data(), static_cast<int32_t>(plan.size()),
                                   &n_pieces);
        if (rc == ZERO_ESIZE) {
            try {
                plan.resize(static_cast<size_t>(n_pieces));
            } catch (...) {
                return fail(ZERO_ESIZE, "no host memory for a plan of %d pieces", n_pieces);
            }
            rc = zero_repartition_plan(from, to, j, plan.data(), n_pieces, &n_pieces);
        }
        if (rc) return rc;
        StateRef dst{{dst_dev[j], nullptr, nullptr}};
        for (int32_t q = 0; q < n_pieces; ++q) {
            StateRef src{{const_cast<float*>(src_dev[plan[q].old_rank]), nullptr, nullptr}};
            if ((rc = launch_state_move(src, true, plan[q].old_offset, dst, true, plan[q].new_offset,
                                        plan[q].count, st)))
                return rc;
        }
        // the new rank's padding, all three fields, is zeroed
        const int64_t valid = zero_partition_valid_numel(to, j);
        StateRef none{{nullptr, nullptr, nullptr}};
        if ((rc = launch_state_move(none, true, 0, dst, true, valid, to->shard_numel - valid, st)))
            return rc;
    }
    return ZERO_OK;
}

}  // extern "C"
