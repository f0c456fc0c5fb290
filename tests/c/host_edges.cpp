// The library's host-only entry points (zero_host.cpp) at the edges of
// their argument ranges and on random inputs, built with AddressSanitizer
// and UndefinedBehaviorSanitizer by tests/test_host_sanitized.py: no call
// may read or write out of bounds, overflow a signed integer or crash, and
// every accepted result must be consistent.  Prints "all checks passed".
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "zero_internal.h"

// zero_host.cpp's argument checks refer to the workspace size, which the
// device source defines; this build has no device source, so the same
// header arithmetic stands in for it.
extern "C" size_t zero_shard_workspace_bytes(int64_t shard_numel) {
    return shard_numel < 0 ? 0 : zero::ws_total_bytes(shard_numel);
}

static int failures = 0;
#define CHECK(cond, ...)                                  \
    do {                                                  \
        if (!(cond)) {                                    \
            std::printf("FAIL line %d: ", __LINE__);      \
            std::printf(__VA_ARGS__);                     \
            std::printf(" (%s)\n", zero_last_error());    \
            ++failures;                                   \
        }                                                 \
    } while (0)

static bool partition_consistent(const zero_partition_t& p) {
    if (p.shard_numel < 0 || p.shard_numel % p.alignment != 0) return false;
    if (p.padded_numel != p.shard_numel * p.world_size || p.padded_numel < p.numel) return false;
    // minimal: one aligned unit less per rank would not cover numel
    if (p.shard_numel >= p.alignment &&
        (p.shard_numel - p.alignment) * static_cast<__int128>(p.world_size) >= p.numel)
        return false;
    int64_t sum = 0;
    for (int32_t r = 0; r < p.world_size && r < 4096; ++r) sum += zero_partition_valid_numel(&p, r);
    return p.world_size > 4096 || sum == p.numel;
}

int main() {
    std::mt19937_64 rng(12345);
    const int64_t I64 = INT64_MAX;

    // partition: edges of every argument
    const int64_t numels[] = {0, 1, 7, 8, 1 << 20, (int64_t(1) << 40) + 3, I64 / 2, I64 - 1, I64};
    const int32_t worlds[] = {1, 2, 3, 8, 1000, 65536, INT32_MAX};
    const int32_t aligns[] = {1, 2, 8, 128, 1 << 20, 1 << 30};
    int accepted = 0, refused = 0;
    for (int64_t n : numels)
        for (int32_t w : worlds)
            for (int32_t a : aligns) {
                zero_partition_t p;
                const int rc = zero_partition(n, w, a, &p);
                if (rc == ZERO_OK) {
                    ++accepted;
                    CHECK(partition_consistent(p), "partition(%lld, %d, %d)", (long long)n, w, a);
                } else {
                    ++refused;
                    CHECK(rc == ZERO_EINVAL, "partition(%lld, %d, %d) rc %d", (long long)n, w, a, rc);
                }
            }
    CHECK(accepted > 0 && refused > 0, "partition: %d accepted, %d refused", accepted, refused);
    zero_partition_t p;
    CHECK(zero_partition(-1, 1, 1, &p) == ZERO_EINVAL, "negative numel");
    CHECK(zero_partition(10, 1, 3, &p) == ZERO_EINVAL, "alignment not a power of two");
    CHECK(zero_partition(10, 0, 1, &p) == ZERO_EINVAL, "no ranks");
    CHECK(zero_partition_valid_numel(nullptr, 0) == -1, "NULL partition");

    // bucket plan: sizes at the top of int64, and random tables
    {
        int64_t sizes[3] = {I64 / 2, I64 / 2, 2};
        zero_tensor_slot_t slots[3];
        zero_bucket_t buckets[3];
        int32_t nb = 0;
        CHECK(zero_bucket_plan(sizes, 3, I64, slots, buckets, 3, &nb) == ZERO_EINVAL,
              "sizes summing past int64");
        int64_t big[2] = {I64 / 2, I64 / 2};
        CHECK(zero_bucket_plan(big, 2, 1, slots, buckets, 3, &nb) == ZERO_OK && nb == 2,
              "two huge tensors, two buckets");
        CHECK(slots[1].offset == I64 / 2 && buckets[1].end == 2 * (I64 / 2), "huge offsets");
    }
    for (int trial = 0; trial < 2000; ++trial) {
        const int n = static_cast<int>(rng() % 40);
        std::vector<int64_t> sizes(n);
        for (auto& x : sizes) x = static_cast<int64_t>(rng() % 1000);
        const int64_t bsz = 1 + static_cast<int64_t>(rng() % 2000);
        std::vector<zero_tensor_slot_t> slots(n + 1);
        const int32_t cap = static_cast<int32_t>(rng() % 50);
        std::vector<zero_bucket_t> buckets(cap + 1);
        int32_t nb = -1;
        const int rc = zero_bucket_plan(sizes.data(), n, bsz, slots.data(), buckets.data(), cap, &nb);
        CHECK(rc == ZERO_OK || (rc == ZERO_ESIZE && nb > cap), "bucket plan rc %d", rc);
        if (rc == ZERO_OK) {
            int64_t at = 0;
            for (int t = 0; t < n; ++t) {
                CHECK(slots[t].offset == at && slots[t].numel == sizes[t], "slot %d", t);
                at += sizes[t];
            }
            // a bucket holds at most bsz elements unless one tensor alone
            // is larger (with, at most, empty tensors beside it)
            for (int b = 0; b < nb; ++b) {
                int nonempty = 0;
                for (int t = buckets[b].first_tensor; t < buckets[b].first_tensor + buckets[b].n_tensors; ++t)
                    nonempty += sizes[t] > 0;
                CHECK(buckets[b].end - buckets[b].begin <= bsz || nonempty == 1, "bucket %d over size", b);
            }
        }
    }

    // re-partition plan: random valid partitions, and hand-built ones
    for (int trial = 0; trial < 3000; ++trial) {
        const int64_t n = static_cast<int64_t>(rng() % 5000);
        zero_partition_t a, b;
        const int32_t wa = 1 + static_cast<int32_t>(rng() % 17), wb = 1 + static_cast<int32_t>(rng() % 17);
        const int32_t aa = 1 << (rng() % 8), ab = 1 << (rng() % 8);
        if (zero_partition(n, wa, aa, &a) != ZERO_OK || zero_partition(n, wb, ab, &b) != ZERO_OK) {
            CHECK(false, "small partition refused");
            continue;
        }
        for (int32_t j = 0; j < wb; ++j) {
            zero_repartition_piece_t pieces[32];
            int32_t np = -1;
            const int rc = zero_repartition_plan(&a, &b, j, pieces, 32, &np);
            CHECK(rc == ZERO_OK, "plan rc %d", rc);
            int64_t covered = 0;
            for (int32_t q = 0; q < np; ++q) {
                CHECK(pieces[q].new_offset == covered && pieces[q].count > 0, "piece order");
                CHECK(pieces[q].old_offset + pieces[q].count <=
                          zero_partition_valid_numel(&a, pieces[q].old_rank), "piece inside old rank");
                CHECK(pieces[q].old_rank * a.shard_numel + pieces[q].old_offset ==
                          j * b.shard_numel + pieces[q].new_offset, "piece maps the same flat element");
                covered += pieces[q].count;
            }
            CHECK(covered == zero_partition_valid_numel(&b, j), "plan covers the real elements");
        }
        // a hand-built partition with a random shard size is refused unless consistent
        zero_partition_t h = b;
        h.shard_numel = static_cast<int64_t>(rng());
        h.padded_numel = static_cast<int64_t>(rng());
        int32_t np = 0;
        zero_repartition_piece_t pc[4];
        const int rc = zero_repartition_plan(&a, &h, 0, pc, 4, &np);
        CHECK(rc == ZERO_EINVAL || (h.shard_numel == b.shard_numel && h.padded_numel == b.padded_numel),
              "hand-built partition accepted");
    }
    {
        // the largest counts whose padded sizes still fit in int64
        zero_partition_t a, b;
        const int64_t n = I64 - (int64_t(1) << 22);
        CHECK(zero_partition(n, 3, 1 << 20, &a) == ZERO_OK, "partition near the top of int64");
        CHECK(zero_partition(n, 7, 1, &b) == ZERO_OK, "partition near the top of int64");
        CHECK(zero_partition(I64 - 1, 3, 1 << 20, &a) == ZERO_EINVAL, "padded count past int64");
        zero_partition(n, 3, 1 << 20, &a);
        zero_repartition_piece_t pieces[8];
        int32_t np = 0;
        for (int32_t j = 0; j < 7; ++j)
            CHECK(zero_repartition_plan(&a, &b, j, pieces, 8, &np) == ZERO_OK && np >= 1 && np <= 3,
                  "plan at the top of int64, rank %d", j);
    }

    // checkpoint headers: random bytes must be refused or consistent
    for (int trial = 0; trial < 20000; ++trial) {
        zero_ckpt_header_t h;
        unsigned char* raw = reinterpret_cast<unsigned char*>(&h);
        for (size_t i = 0; i < sizeof h; ++i) raw[i] = static_cast<unsigned char>(rng());
        if (trial % 2) {               // a valid start, then one field scrambled
            zero_partition_t q;
            zero_partition(static_cast<int64_t>(rng() % 100000), 1 + static_cast<int32_t>(rng() % 9),
                           8, &q);
            zero_ckpt_header_make(&q, static_cast<int32_t>(rng() % q.world_size), ZERO_BF16,
                                  static_cast<int64_t>(rng() % 100), nullptr, &h);
            raw[rng() % sizeof h] ^= static_cast<unsigned char>(1u << (rng() % 8));
        }
        zero_partition_t part;
        const int rc = zero_ckpt_header_check(&h, rng(), &part);
        CHECK(rc == ZERO_OK || rc == ZERO_EINVAL || rc == ZERO_ESIZE, "header check rc %d", rc);
        if (rc == ZERO_OK) CHECK(partition_consistent(part), "accepted header's partition");
    }

    // loss scaler: long random runs stay in range
    zero_loss_scaler_t sc;
    CHECK(zero_loss_scaler_init(127, 3, 2, 1e-30, &sc) == ZERO_OK, "scaler init at 2^127");
    for (int i = 0; i < 100000; ++i) {
        int32_t skip = 0;
        CHECK(zero_loss_scaler_update(&sc, static_cast<int32_t>(rng() % 3 == 0), &skip) == ZERO_OK,
              "scaler update");
    }
    CHECK(sc.scale >= 1e-30, "scale above its floor");

    if (failures) {
        std::printf("%d checks failed\n", failures);
        return 1;
    }
    std::printf("all checks passed\n");
    return 0;
}
