/* A plain C caller of the library's host-only entry points, built with gcc
 * against include/zero.h and libzero_mi355x.so: the ABI is usable without
 * Python.  Prints one line per check; exits non-zero on the first failure.
 * No call here reaches a GPU. */
#include <stdio.h>
#include <string.h>

#include "zero.h"

#define CHECK(cond, what)                                             \
    do {                                                              \
        if (!(cond)) {                                                \
            printf("FAIL %s (%s)\n", what, zero_last_error());        \
            return 1;                                                 \
        }                                                             \
        printf("ok   %s\n", what);                                    \
    } while (0)

int main(void) {
    zero_partition_t p;
    CHECK(zero_partition(13000000000LL, 8, 128, &p) == ZERO_OK, "partition 13B over 8");
    CHECK(p.shard_numel == 1625000064LL && p.padded_numel == 13000000512LL, "shard size");
    CHECK(zero_partition_valid_numel(&p, 7) == 1625000064LL - 512, "last rank's real count");
    CHECK(zero_partition(10, 0, 8, &p) == ZERO_EINVAL && strlen(zero_last_error()) > 0,
          "world_size 0 rejected");

    int64_t sizes[5] = {50, 90, 60, 250, 10};
    zero_tensor_slot_t slots[5];
    zero_bucket_t buckets[8];
    int32_t nb = 0;
    CHECK(zero_bucket_plan(sizes, 5, 200, slots, buckets, 8, &nb) == ZERO_OK, "bucket plan");
    CHECK(nb == 3 && buckets[0].n_tensors == 3 && buckets[1].first_tensor == 3 &&
          slots[4].offset == 450 && slots[4].bucket == 2, "greedy buckets, oversize alone");

    zero_loss_scaler_t sc;
    int32_t skip = 0;
    CHECK(zero_loss_scaler_init(16, 2, 2, 1.0, &sc) == ZERO_OK && sc.scale == 65536.0,
          "scaler init");
    CHECK(zero_loss_scaler_update(&sc, 1, &skip) == ZERO_OK && skip == 1 && sc.scale == 65536.0,
          "first overflow spends the hysteresis");
    CHECK(zero_loss_scaler_update(&sc, 1, &skip) == ZERO_OK && sc.scale == 32768.0,
          "second overflow halves the scale");
    zero_loss_scaler_update(&sc, 0, &skip);
    zero_loss_scaler_update(&sc, 0, &skip);
    CHECK(skip == 0 && sc.scale == 65536.0 && sc.hysteresis_left == 2, "window of good steps grows");

    zero_ckpt_header_t h;
    CHECK(zero_partition(1000, 4, 8, &p) == ZERO_OK, "partition 1000 over 4");
    CHECK(zero_ckpt_header_make(&p, 3, ZERO_BF16, 12, &sc, &h) == ZERO_OK, "checkpoint header");
    CHECK(sizeof h == 128 && h.valid_numel == 1000 - 3 * 256 && h.payload_bytes == 12u * 232u,
          "header layout");
    zero_partition_t q;
    CHECK(zero_ckpt_header_check(&h, 128 + h.payload_bytes, &q) == ZERO_OK && q.shard_numel == 256,
          "header check");
    CHECK(zero_ckpt_header_check(&h, 100, &q) == ZERO_ESIZE, "short file rejected");

    float g[3] = {0.5f, -0.25f, 1.0f}, m[3] = {0}, v[3] = {0}, w[3] = {0.1f, 0.2f, 0.3f};
    unsigned short out[3];
    CHECK(zero_host_adamw(3, g, 1.0f, w, m, v, out, ZERO_BF16, 6e-5, 0.9, 0.999, 1e-8, 0.01, 1, 1)
              == ZERO_OK, "host AdamW");
    CHECK(m[0] == 0.1f * 0.5f && v[2] > 0.0f && out[2] != 0, "host AdamW moved the state");

    zero_step_args a;
    memset(&a, 0, sizeof a);
    CHECK(zero_shard_step(&a, 0.0, 0, NULL, NULL) == ZERO_EINVAL, "empty step arguments rejected");
    printf("all checks passed\n");
    return 0;
}
