/*
 * synth_core.h -- the seeded, counter-based input generator shared by the
 * host (gcc) and device (hipcc) builds of the synth module.
 *
 * It holds no arithmetic of the optimizer step.  It only turns
 * (seed, tag, element index) into a synthetic value drawn from a normal
 * distribution, so that any element of any buffer can be regenerated on its
 * own, on either side, bit for bit:
 *
 *   h   = SplitMix64 output number j+1 of a stream keyed by (seed, tag)
 *         (Steele, Lea & Flood, "Fast splittable pseudorandom number
 *         generators", OOPSLA 2014: state advanced by the golden gamma,
 *         output passed through the 64-bit finaliser)
 *   z   = quantile table lookup, linearly interpolated: the top 16 bits of h
 *         pick a cell, the next 16 bits the position inside it; the table
 *         holds the standard normal quantiles at (i + 1/2) / 65537
 *   v   = z * sigma, times `mul` when the low 20 bits of h fall below
 *         `thr` (an outlier with probability thr / 2^20)
 *   out = (float)v, and for 16-bit outputs that float truncated toward zero
 *         (bf16: keep the top half; fp16: drop mantissa bits, no rounding).
 *
 * Only IEEE double +, -, * and a double->float conversion appear, so the
 * host and device builds (both with -ffp-contract=off) agree exactly.
 */
#ifndef SYNTH_CORE_H
#define SYNTH_CORE_H

#include <stdint.h>

#ifdef __HIPCC__
#define SYN_FN __host__ __device__ static inline
#else
#define SYN_FN static inline
#endif

#define SYN_TABLE_CELLS 65536
#define SYN_TABLE_SIZE (SYN_TABLE_CELLS + 1)

enum { SYN_F32 = 0, SYN_BF16 = 1, SYN_F16 = 2 };

#define SYN_GAMMA 0x9E3779B97F4A7C15ull

SYN_FN uint64_t syn_mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* the stream's starting state for (seed, tag) */
SYN_FN uint64_t syn_key(uint64_t seed, uint64_t tag) {
    return syn_mix64(seed * SYN_GAMMA + 0x2545F4914F6CDD1Dull) ^
           syn_mix64(tag + 0x632BE59BD9B4E019ull);
}

/* output number j + 1 of the stream */
SYN_FN uint64_t syn_bits(uint64_t key, uint64_t j) {
    return syn_mix64(key + (j + 1) * SYN_GAMMA);
}

SYN_FN double syn_value(const double *table, uint64_t h, double sigma,
                        uint32_t thr, double mul) {
    uint32_t q = (uint32_t)(h >> 48);
    double f = (double)(uint32_t)((h >> 32) & 0xFFFFu) * (1.0 / 65536.0);
    double lo = table[q];
    double hi = table[q + 1];
    double z = lo + f * (hi - lo);
    double v = z * sigma;
    if ((uint32_t)(h & 0xFFFFFu) < thr) v = v * mul;
    return v;
}

SYN_FN uint32_t syn_f32_bits(float f) {
    union { float f; uint32_t u; } c;
    c.f = f;
    return c.u;
}

/* truncate a float toward zero to bf16 */
SYN_FN uint16_t syn_trunc_bf16(float f) {
    return (uint16_t)(syn_f32_bits(f) >> 16);
}

/* truncate a finite float toward zero to fp16 (saturating at 65504) */
SYN_FN uint16_t syn_trunc_f16(float f) {
    uint32_t u = syn_f32_bits(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t mag = u & 0x7FFFFFFFu;
    int32_t e = (int32_t)(mag >> 23) - 127;
    uint32_t m = mag & 0x7FFFFFu;
    if (e > 15) return (uint16_t)(sign | 0x7BFFu);
    if (e >= -14) return (uint16_t)(sign | ((uint32_t)(e + 15) << 10) | (m >> 13));
    if (e < -24) return sign;
    /* subnormal: value = (m | 2^23) * 2^(e-23) = q * 2^-24 */
    return (uint16_t)(sign | ((m | 0x800000u) >> (-e - 1)));
}

#endif
