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

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Reduce-pass geometry: each thread owns 8 consecutive elements per
// iteration; a grid of at most kMaxReduceBlocks blocks strides over the
// shard.  The block count depends only on valid_numel, so the per-block
// partial sums, and hence the norm, are identical from run to run.
constexpr int kReduceThreads = 256;
constexpr int kVec = 8;
constexpr int kMaxReduceBlocks = 2048;

// One partial per reduce block.
struct Partial {
    double sumsq;
    int32_t flag;
    int32_t pad;
};

// Layout of one slot of the partials table: a 16-byte header holding the
// number of blocks the reduce wrote, then kMaxReduceBlocks partials.
struct SlotHeader {
    int32_t n_blocks;
    int32_t pad[3];
};
constexpr size_t kSlotBytes = sizeof(SlotHeader) + kMaxReduceBlocks * sizeof(Partial);

int reduce_blocks_for(int64_t valid_numel);

// Byte offsets inside a zero_shard_step workspace.
inline size_t ws_grad_bytes(int64_t shard_numel) {
    return round_up(static_cast<size_t>(shard_numel) * 4u, 256);
}
inline size_t ws_partials_offset(int64_t shard_numel) { return ws_grad_bytes(shard_numel); }
inline size_t ws_global_offset(int64_t shard_numel) {
    return ws_partials_offset(shard_numel) + round_up(kSlotBytes, 256);
}

// Checks every field of a step's arguments (see zero_shard_step).
int validate_step_args(const zero_step_args* a);

}  // namespace zero
