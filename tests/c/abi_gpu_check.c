/* A plain C caller of the library's device entry points: HIP memory from
 * hipMalloc, no Python and no torch.  It reads one world's inputs from a
 * file, runs `steps` optimizer steps of every rank (zero_shard_reduce per
 * rank, zero_shard_combine, zero_shard_apply per rank) on one stream, and
 * writes each step's combine result and the whole state to a file for the
 * test to compare with the oracle.
 *
 * Input (little-endian): int64 numel, world_size, alignment, n_replicas,
 * dtype, steps; double loss_scale, max_grad_norm; then n_replicas flat
 * gradient buffers of padded_numel 16-bit codes; then padded_numel fp32
 * masters (rank r's shard at r * shard_numel).
 * Output, per step: zero_global_t, then padded_numel fp32 master, exp_avg,
 * exp_avg_sq, then padded_numel 16-bit full parameters.
 * With a third argument `noalloc` (a world of one rank only), each step is
 * one zero_shard_step_noalloc call instead, and no workspace is allocated:
 * the library's own scratch memory serves.
 * Exit status 0 on success; a failing call prints its error. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "zero.h"

#define HIPCHECK(x)                                                                  \
    do {                                                                             \
        hipError_t e_ = (x);                                                         \
        if (e_ != hipSuccess) {                                                      \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                  \
            return 2;                                                                \
        }                                                                            \
    } while (0)
#define ZCHECK(x)                                                                    \
    do {                                                                             \
        int rc_ = (x);                                                               \
        if (rc_ != ZERO_OK) {                                                        \
            fprintf(stderr, "%s -> %d: %s\n", #x, rc_, zero_last_error());           \
            return 3;                                                                \
        }                                                                            \
    } while (0)
#define READ(ptr, bytes)                                                             \
    do {                                                                             \
        if (fread((ptr), 1, (bytes), in) != (size_t)(bytes)) {                       \
            fprintf(stderr, "short input file\n");                                   \
            return 4;                                                                \
        }                                                                            \
    } while (0)
#define WRITE(ptr, bytes)                                                            \
    do {                                                                             \
        if (fwrite((ptr), 1, (bytes), out) != (size_t)(bytes)) {                     \
            fprintf(stderr, "write failed\n");                                       \
            return 5;                                                                \
        }                                                                            \
    } while (0)

enum { MAX_RANKS = 64 };

int main(int argc, char** argv) {
    if (argc != 3 && !(argc == 4 && strcmp(argv[3], "noalloc") == 0)) {
        fprintf(stderr, "usage: %s input output [noalloc]\n", argv[0]);
        return 1;
    }
    const int noalloc = argc == 4;
    FILE* in = fopen(argv[1], "rb");
    if (!in) return 1;
    int64_t hdr[6];
    double hp[2];
    READ(hdr, sizeof hdr);
    READ(hp, sizeof hp);
    const int64_t numel = hdr[0];
    const int32_t world = (int32_t)hdr[1], align = (int32_t)hdr[2], nrep = (int32_t)hdr[3];
    const int32_t dtype = (int32_t)hdr[4], steps = (int32_t)hdr[5];
    if (world < 1 || world > MAX_RANKS || nrep < 1 || nrep > ZERO_MAX_REPLICAS) return 1;
    if (noalloc && world != 1) return 1;
    zero_partition_t part;
    ZCHECK(zero_partition(numel, world, align, &part));
    const int64_t s = part.shard_numel, padded = part.padded_numel;

    uint16_t* h_reps = (uint16_t*)malloc((size_t)nrep * padded * 2);
    float* h_f32 = (float*)malloc((size_t)padded * 4);
    uint16_t* h_full = (uint16_t*)malloc((size_t)padded * 2);
    if (!h_reps || !h_f32 || !h_full) return 6;
    READ(h_reps, (size_t)nrep * padded * 2);
    READ(h_f32, (size_t)padded * 4);
    fclose(in);

    void* d_reps[ZERO_MAX_REPLICAS];
    float *d_master, *d_m, *d_v;
    void *d_full, *d_partials, *d_global;
    void* d_ws[MAX_RANKS];
    const size_t ws_bytes = zero_shard_workspace_bytes(s);
    for (int i = 0; i < nrep; ++i) {
        HIPCHECK(hipMalloc(&d_reps[i], (size_t)padded * 2));
        HIPCHECK(hipMemcpy(d_reps[i], h_reps + (size_t)i * padded, (size_t)padded * 2,
                           hipMemcpyHostToDevice));
    }
    HIPCHECK(hipMalloc((void**)&d_master, (size_t)padded * 4));
    HIPCHECK(hipMalloc((void**)&d_m, (size_t)padded * 4));
    HIPCHECK(hipMalloc((void**)&d_v, (size_t)padded * 4));
    HIPCHECK(hipMemcpy(d_master, h_f32, (size_t)padded * 4, hipMemcpyHostToDevice));
    HIPCHECK(hipMemset(d_m, 0, (size_t)padded * 4));
    HIPCHECK(hipMemset(d_v, 0, (size_t)padded * 4));
    HIPCHECK(hipMalloc(&d_full, (size_t)padded * 2));
    HIPCHECK(hipMemset(d_full, 0, (size_t)padded * 2));
    for (int r = 0; r < world; ++r) {
        d_ws[r] = NULL;
        if (!noalloc) HIPCHECK(hipMalloc(&d_ws[r], ws_bytes));
    }
    HIPCHECK(hipMalloc(&d_partials, zero_partials_bytes(world)));
    HIPCHECK(hipMalloc(&d_global, 256));
    hipStream_t st;
    HIPCHECK(hipStreamCreate(&st));

    FILE* out = fopen(argv[2], "wb");
    if (!out) return 1;
    const void* rep_ptrs[MAX_RANKS][ZERO_MAX_REPLICAS];
    zero_step_args a[MAX_RANKS];
    for (int t = 1; t <= steps; ++t) {
        for (int r = 0; r < world; ++r) {
            for (int i = 0; i < nrep; ++i)
                rep_ptrs[r][i] = (const uint16_t*)d_reps[i] + (size_t)r * s;
            memset(&a[r], 0, sizeof a[r]);
            a[r].world_size = world;
            a[r].rank = r;
            a[r].shard_numel = s;
            a[r].valid_numel = zero_partition_valid_numel(&part, r);
            a[r].grad_dtype = dtype;
            a[r].param_dtype = dtype;
            a[r].n_replicas = nrep;
            a[r].replica_grad = rep_ptrs[r];
            a[r].master = d_master + (size_t)r * s;
            a[r].exp_avg = d_m + (size_t)r * s;
            a[r].exp_avg_sq = d_v + (size_t)r * s;
            a[r].full_params = d_full;
            a[r].workspace = d_ws[r];
            a[r].workspace_bytes = noalloc ? 0 : ws_bytes;
            a[r].lr = 6e-5;
            a[r].beta1 = 0.9;
            a[r].beta2 = 0.999;
            a[r].eps = 1e-8;
            a[r].weight_decay = 0.01;
            a[r].step = t;
            a[r].loss_scale = hp[0];
            a[r].grad_predivide = 1.0;
            a[r].max_grad_norm = hp[1];
            if (!noalloc) ZCHECK(zero_shard_reduce(&a[r], r, d_partials, st));
        }
        zero_global_t g;
        if (noalloc) {
            /* the whole step of the one rank; info waits for the stream */
            ZCHECK(zero_shard_step_noalloc(&a[0], 0.0, 0, &g, st));
        } else {
            ZCHECK(zero_shard_combine(d_partials, world, hp[1], d_global, st));
            for (int r = 0; r < world; ++r) ZCHECK(zero_shard_apply(&a[r], d_global, st));
            HIPCHECK(hipStreamSynchronize(st));
            HIPCHECK(hipMemcpy(&g, d_global, sizeof g, hipMemcpyDeviceToHost));
        }
        WRITE(&g, sizeof g);
        float* fields[3] = {d_master, d_m, d_v};
        for (int f = 0; f < 3; ++f) {
            HIPCHECK(hipMemcpy(h_f32, fields[f], (size_t)padded * 4, hipMemcpyDeviceToHost));
            WRITE(h_f32, (size_t)padded * 4);
        }
        HIPCHECK(hipMemcpy(h_full, d_full, (size_t)padded * 2, hipMemcpyDeviceToHost));
        WRITE(h_full, (size_t)padded * 2);
    }
    fclose(out);
    for (int i = 0; i < nrep; ++i) HIPCHECK(hipFree(d_reps[i]));
    for (int r = 0; r < world; ++r)
        if (d_ws[r]) HIPCHECK(hipFree(d_ws[r]));
    HIPCHECK(hipFree(d_master));
    HIPCHECK(hipFree(d_m));
    HIPCHECK(hipFree(d_v));
    HIPCHECK(hipFree(d_full));
    HIPCHECK(hipFree(d_partials));
    HIPCHECK(hipFree(d_global));
    HIPCHECK(hipStreamDestroy(st));
    free(h_reps);
    free(h_f32);
    free(h_full);
    printf("done\n");
    return 0;
}
