// zero_internal.h -- declarations shared by the host and device sources of
// the library.  Not part of the public ABI (include/zero.h is).
#pragma once

#include <cstdarg>
#include <cstddef>
#include <cstdint>

#include "zero.h"

namespace zero {

// Record a failure for zero_last_error() and return `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

inline bool aligned16(const void* p) {
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

constexpr size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Launch geometry.  Both streaming passes give each thread one "quad" of 4
// consecutive elements and launch one thread per quad (no grid-stride
// loop): blocks are dispatched in order, so the set of addresses in flight
// stays a compact window of every stream, which keeps HBM pages open.  The
// hardware deals dispatch-order blocks to the 8 XCDs round robin; the
// kernels remap them so that each XCD takes runs of `group` consecutive
// logical blocks (256 for large grids, measured best; the whole eighth of
// the grid for small ones), which keeps every XCD on contiguous memory
// while all of them advance through the shard together.  Everything
// depends only on valid_numel, so the per-block partial sums, and hence the
// norm, are identical from run to run.
constexpr int kQuad = 4;
// shard_numel must be a multiple of this, so that every rank's slice of the
// full 16-bit parameter buffer starts on a 16-byte boundary.
constexpr int64_t kShardMultiple = 8;
constexpr int kReduceThreads = 256;        // reduce: 1024 elements per block
constexpr int kApplyThreads = 64;          // apply: 256 elements per block
constexpr int kXcds = 8;
constexpr int kFoldBlocks = 256;           // fixed-size per-rank summary
constexpr int kStateTile = ZERO_STATE_TILE; // elements per tile of a tiled state

// fp32 values of a rank's tiled state: three per element, whole tiles.
constexpr size_t tiled_state_floats(int64_t shard_numel) {
    return 3u * static_cast<size_t>((shard_numel + kStateTile - 1) / kStateTile) * kStateTile;
}

// One partial sum of squares (fp64) and inf/nan flag.
struct Partial {
    double sumsq;
    int32_t flag;
    int32_t pad;
};

// One slot of the partials table: a 16-byte header holding how many
// entries follow, then up to kFoldBlocks partials.
struct SlotHeader {
    int32_t n_blocks;
    int32_t pad[3];
};
constexpr size_t kSlotBytes = sizeof(SlotHeader) + kFoldBlocks * sizeof(Partial);

// Quads (the last one possibly partial) of n elements.
constexpr int64_t quads_of(int64_t n) { return (n + kQuad - 1) / kQuad; }

// A launch: `blocks` (a multiple of kXcds * group) of which the first
// `needed` hold work, remapped in XCD runs of `group` logical blocks.
struct Grid {
    int64_t blocks;
    int32_t group;
};
constexpr int64_t kXcdGroup = 256;

// Blocks of `threads` threads covering quads_of(n) quads, at least one.
constexpr Grid grid_for(int64_t n, int threads) {
    int64_t b = (quads_of(n) + threads - 1) / threads;
    if (b < 1) b = 1;
    if (b >= kXcds * kXcdGroup) {
        const int64_t unit = kXcds * kXcdGroup;
        return Grid{(b + unit - 1) / unit * unit, static_cast<int32_t>(kXcdGroup)};
    }
    const int64_t nb = (b + kXcds - 1) / kXcds * kXcds;
    return Grid{nb, static_cast<int32_t>(nb / kXcds)};
}
// Logical block of dispatch-order block b (which the hardware sends to XCD
// b % kXcds) in a grid that is a multiple of kXcds * group blocks: XCD x
// takes logical blocks [k * kXcds * group + x * group, ... + group) for
// k = 0, 1, ...  With group = grid / kXcds that is one contiguous share of
// the grid per XCD.  constexpr, so the kernels and the host-side check of
// the launch grids use the same code.
constexpr int64_t xcd_logical_block(uint32_t b, uint32_t group) {
    return static_cast<int64_t>((b / kXcds) / group) * (kXcds * group) + (b % kXcds) * group +
           (b / kXcds) % group;
}
constexpr int64_t reduce_blocks_for(int64_t n) { return grid_for(n, kReduceThreads).blocks; }
constexpr int64_t apply_blocks_for(int64_t n) { return grid_for(n, kApplyThreads).blocks; }
inline int fold_blocks_for(int64_t reduce_blocks) {
    return static_cast<int>(reduce_blocks < kFoldBlocks ? reduce_blocks : kFoldBlocks);
}

// Byte offsets inside a zero_shard_step workspace: the fp32 reduced
// gradient, the reduce's per-block partials, one slot, one zero_global_t.
constexpr size_t ws_grad_bytes(int64_t shard_numel) {
    return round_up(static_cast<size_t>(shard_numel) * 4u, 256);
}
constexpr size_t ws_blocks_offset(int64_t shard_numel) { return ws_grad_bytes(shard_numel); }
constexpr size_t ws_blocks_bytes(int64_t shard_numel) {
    return round_up(static_cast<size_t>(reduce_blocks_for(shard_numel)) * sizeof(Partial), 256);
}
constexpr size_t ws_slot_offset(int64_t shard_numel) {
    return ws_blocks_offset(shard_numel) + ws_blocks_bytes(shard_numel);
}
constexpr size_t ws_global_offset(int64_t shard_numel) {
    return ws_slot_offset(shard_numel) + round_up(kSlotBytes, 256);
}

// The whole workspace of a shard (zero_shard_workspace_bytes).
constexpr size_t ws_total_bytes(int64_t shard_numel) { return ws_global_offset(shard_numel) + 256; }

// Where a rank's cast parameters go: its ZeRO-3 shard when given, else
// its slice of the full buffer.
inline unsigned short* param_out(const zero_step_args* a) {
    if (a->param_shard) return static_cast<unsigned short*>(a->param_shard);
    return static_cast<unsigned short*>(a->full_params) +
           static_cast<size_t>(a->rank) * static_cast<size_t>(a->shard_numel);
}

// Checks every field of a step's arguments (see zero_shard_step); without
// check_workspace the workspace fields are not looked at (the caller
// supplies the workspace itself).
int validate_step_args(const zero_step_args* a, bool check_workspace = true);

// ZERO_OK when *p is exactly what zero_partition makes of its numel,
// world_size and alignment; otherwise records why (naming the partition
// `what`) and returns ZERO_EINVAL.  Every entry point that takes a
// partition struct re-derives it this way, so a hand-built one with an
// inconsistent or overflowing shard size is refused.
int check_partition(const zero_partition_t* p, const char* what);

// AdamW's per-step fp32 constants, each computed in fp64 from the step's
// hyper-parameters and rounded once; the GPU pass and the host (offloaded)
// pass both use exactly these.
struct AdamConsts {
    float decay;          // 1 - lr * wd
    float b1, c1;         // beta1, 1 - beta1
    float b2, c2;         // beta2, 1 - beta2
    float step_size;      // lr / (1 - beta1^t)
    float inv_sqrt_bc2;   // 1 / sqrt(1 - beta2^t)
    float eps;
};
AdamConsts adam_consts(double lr, double beta1, double beta2, double eps, double weight_decay,
                       int64_t step);

// The unscale multiplier fp32(1 / (loss_scale * grad_predivide)) of a step.
inline float unscale_factor(const zero_step_args* a) {
    return static_cast<float>(1.0 / (a->loss_scale * a->grad_predivide));
}

}  // namespace zero
