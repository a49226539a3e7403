/*
 * The C ABI used from C alone -- no Python, no torch: device buffers from
 * hipMalloc, three fused steps of one rank's shard through zero_shard_step
 * ("ZeRO and FSDP", A sharded Adam step), each compared bit for bit with the
 * oracle's step (test infrastructure) on host copies: master, moments and
 * the whole 16-bit weight buffer, canaries outside the slot included.
 * Prints "c-abi step ok ..." and exits 0 on success.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle_zero.h"
#include "zero_shard.h"

#define CHECK(x)                                                                    \
    do {                                                                            \
        hipError_t e_ = (x);                                                        \
        if (e_ != hipSuccess) {                                                     \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                 \
            return 2;                                                               \
        }                                                                           \
    } while (0)

/* counter-based inputs (SplitMix64 finaliser) */
static uint64_t mix(uint64_t z) {
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
/* a bf16 gradient pattern of magnitude about 2^-10: random sign and mantissa */
static uint16_t grad_bits(uint64_t i) {
    const uint64_t z = mix(i);
    return (uint16_t)(((z >> 16) & 0x8000u) | 0x3A80u | (z & 0x7Fu));
}
/* a master weight in [-0.02, 0.02) */
static float master_val(uint64_t i) {
    const uint64_t z = mix(i ^ 0x5555ull);
    return ((float)(z >> 40) / 16777216.0f - 0.5f) * 0.04f;
}

int main(void) {
    const int64_t numels[3] = {10007, 3, 5000};
    const int32_t n_dp = 4, rank = 1;
    int64_t offs[3];
    zero_layout lay;
    if (zero_flatten_layout(numels, 3, n_dp, 1, offs, &lay) != ZERO_OK) return 3;
    const int64_t S = lay.shard, n = lay.n, lo = rank * S;
    uint16_t *g = malloc((size_t)(n_dp * S) * 2);
    float *w = malloc((size_t)S * 4), *m = calloc((size_t)S, 4), *v = calloc((size_t)S, 4);
    float *got = malloc((size_t)S * 4);
    uint16_t *wout = malloc((size_t)lay.n_pad * 2), *wgot = malloc((size_t)lay.n_pad * 2);
    if (!g || !w || !m || !v || !got || !wout || !wgot) return 3;
    for (int64_t j = 0; j < S; ++j) w[j] = lo + j < n ? master_val((uint64_t)(lo + j)) : 0.0f;
    for (int64_t j = 0; j < lay.n_pad; ++j) wout[j] = 0x5A5A;

    void *dg, *dw, *dm, *dv, *dwf;
    CHECK(hipMalloc(&dg, (size_t)(n_dp * S) * 2));
    CHECK(hipMalloc(&dw, (size_t)S * 4));
    CHECK(hipMalloc(&dm, (size_t)S * 4));
    CHECK(hipMalloc(&dv, (size_t)S * 4));
    CHECK(hipMalloc(&dwf, (size_t)lay.n_pad * 2));
    CHECK(hipMemcpy(dw, w, (size_t)S * 4, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(dm, m, (size_t)S * 4, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(dv, v, (size_t)S * 4, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(dwf, wout, (size_t)lay.n_pad * 2, hipMemcpyHostToDevice));

    zero_adamw_hparams hp = {1e-4, 0.9, 0.999, 1e-8, 0.1, 1.0 / n_dp, 1};
    const double hp6[6] = {1e-4, 0.9, 0.999, 1e-8, 0.1, 1.0 / n_dp};
    for (int64_t t = 1; t <= 3; ++t) {
        for (int64_t k = 0; k < n_dp; ++k)
            for (int64_t j = 0; j < S; ++j)   /* row k: rank k's gradient for shard `rank` */
                g[k * S + j] = lo + j < n ? grad_bits((uint64_t)(t * 1000003 + k) * 65536 + j) : 0;
        CHECK(hipMemcpy(dg, g, (size_t)(n_dp * S) * 2, hipMemcpyHostToDevice));
        hp.step = t;
        const zero_status st = zero_shard_step(dg, ZERO_BF16, S, S, dw, dm, dv, dwf, ZERO_BF16,
                                               &lay, rank, 0, &hp, NULL, NULL, NULL, 0, NULL);
        if (st != ZERO_OK) {
            fprintf(stderr, "zero_shard_step: %s\n", zero_status_string(st));
            return 4;
        }
        CHECK(hipDeviceSynchronize());
        ora_step(g, ORA_BF16, n_dp, S, S, w, m, v, wout + lo, ORA_BF16, hp6, t, NULL, NULL);
        const struct { void *dev; const void *ref; size_t bytes; const char *name; } cmp[4] = {
            {dw, w, (size_t)S * 4, "master"}, {dm, m, (size_t)S * 4, "m"},
            {dv, v, (size_t)S * 4, "v"}, {dwf, wout, (size_t)lay.n_pad * 2, "weight buffer"}};
        for (int c = 0; c < 4; ++c) {
            void *host = c == 3 ? (void *)wgot : (void *)got;
            CHECK(hipMemcpy(host, cmp[c].dev, cmp[c].bytes, hipMemcpyDeviceToHost));
            if (memcmp(host, cmp[c].ref, cmp[c].bytes) != 0) {
                fprintf(stderr, "step %lld: %s differs from the oracle\n", (long long)t, cmp[c].name);
                return 1;
            }
        }
    }
    printf("c-abi step ok: 3 steps of a %lld-element shard (rank %d of %d), bitwise\n",
           (long long)S, rank, n_dp);
    return 0;
}
