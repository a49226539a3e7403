/*
 * oracle_zero.c -- plain CPU oracle (TEST INFRASTRUCTURE ONLY; see the
 * header).  Single-threaded, one element at a time, IEEE binary32 with
 * round-to-nearest-even for the optimizer arithmetic, built with
 * -ffp-contract=off and without any fast-math option.
 *
 * What pins each function (tests/test_oracle_*.py):
 *  - ora_flatten_layout / ora_shard_segments: the tiny workload's printed
 *    sizes (10,000 elements, 4 ranks, shard 2,500), numpy.array_split
 *    boundaries when n_dp divides N, brute-force tiling on tiny lists, the
 *    7B and GPT-2-XL totals.
 *  - converters: exhaustive against torch / numpy library conversions.
 *  - ora_reduce: exact sums (fractions) within the recursive-summation bound,
 *    numpy float64 sums, the sum-of-shards identity (reduce-scatter followed
 *    by all-gather equals all-reduce).
 *  - ora_adamw / ora_step: torch.optim.AdamW on the CPU (a library routine),
 *    the step-1 closed form (update ~ -lr*sign(g) - lr*wd*w), the constant-
 *    gradient closed form, a high-precision brute force on tiny inputs, and
 *    sharded == unsharded.
 *  - ora_model_state_bytes / ora_comm_bytes: the numbers the pages print.
 *  - ora_dim0_layout / ora_dim0_segments: torch.chunk's row boundaries per
 *    tensor, packing every rank's buffer and unpacking it again rebuilds
 *    every tensor, the 7B and GPT-2-XL totals.
 *  - fp32 gradient rows (ORA_FP32): equal to the 16-bit path bit for bit on
 *    values both formats hold, and exact sums within the summation bound.
 *  - ora_q8_*: PARITY UNPINNED against the pages (they define no quantizer);
 *    pinned to the quantizer's own properties: codes in [-127, 127], the
 *    block's largest magnitude coded +-127, the rounding bound s/2, exact
 *    invariance under power-of-two scaling and sign flips, zero and
 *    non-finite blocks, subnormal scales, hand-worked blocks and blocks
 *    found by search where rint(x / s) differs from rint(x * 127 / absmax)
 *    or from rounding the exact quotient (derived in exact rational
 *    arithmetic); ora_step_q8 equal to dequantize + the fp32-row step +
 *    quantize.
 *  - ora_reshard / ora_flat_*: slicing and concatenation of the flat vector
 *    in numpy, agreement of the two independent forms (equal shards against
 *    general pieces), round trips n_dp -> n_dp' -> n_dp, scatter after
 *    gather, and consolidation recovering every parameter tensor.
 * ora_step's sumsq output is order dependent and checked only against a
 * float64 sum within a bound (parity unpinned bitwise by design).
 */
#include "oracle_zero.h"

#include <math.h>
#include <stdint.h>
#include <string.h>

/* ceil(a / b) for a >= 0, b >= 1, without forming a + b - 1 */
static int64_t ceil_div(int64_t a, int64_t b) { return a / b + (a % b != 0); }

/* ------------------------------------------------------------------------ */
/* Layout.  "ZeRO and FSDP", "The idea, one stage at a time": one flat vector
 * of N numbers cut into n_dp equal contiguous shards; rank r owns shard r.
 * Equal shards need N_pad = n_dp * S >= N; the tail is zero padding. */

int ora_flatten_layout(const int64_t *numels, int64_t n_tensors, int32_t n_dp,
                       int64_t align, int64_t *offsets, int64_t out3[3]) {
    if (n_tensors < 0 || n_dp < 1 || align < 1 || out3 == 0) return -1;
    if (n_tensors > 0 && numels == 0) return -1;
    int64_t n = 0;
    for (int64_t i = 0; i < n_tensors; ++i) {
        if (numels[i] < 0 || numels[i] > INT64_MAX - n) return -1; /* N fits int64 */
        if (offsets) offsets[i] = n;
        n += numels[i];
    }
    if (align > INT64_MAX / n_dp) return -1;
    int64_t unit = (int64_t)n_dp * align;
    int64_t units = ceil_div(n, unit);
    if (units > INT64_MAX / unit) return -1; /* N_pad fits int64 */
    int64_t shard = units * align;
    out3[0] = n;
    out3[1] = shard * n_dp;
    out3[2] = shard;
    return 0;
}

int64_t ora_shard_segments(const int64_t *numels, int64_t n_tensors,
                           int32_t n_dp, int64_t align, int32_t rank,
                           int64_t *quads, int64_t cap) {
    int64_t lay[3];
    if (ora_flatten_layout(numels, n_tensors, n_dp, align, 0, lay) != 0)
        return -1;
    if (rank < 0 || rank >= n_dp) return -1;
    int64_t n = lay[0], shard = lay[2];
    int64_t lo = (int64_t)rank * shard, hi = lo + shard;
    int64_t count = 0, start = 0;
    for (int64_t t = 0; t < n_tensors; ++t) {
        int64_t a = start, b = start + numels[t];
        start = b;
        int64_t s = a > lo ? a : lo;
        int64_t e = b < hi ? b : hi;
        if (e > s) {
            if (count < cap) {
                quads[4 * count + 0] = t;
                quads[4 * count + 1] = s - a;
                quads[4 * count + 2] = s - lo;
                quads[4 * count + 3] = e - s;
            }
            ++count;
        }
    }
    /* the zero padding [N, N_pad) */
    int64_t s = n > lo ? n : lo;
    if (hi > s) {
        if (count < cap) {
            quads[4 * count + 0] = -1;
            quads[4 * count + 1] = s - n;
            quads[4 * count + 2] = s - lo;
            quads[4 * count + 3] = hi - s;
        }
        ++count;
    }
    return count;
}

/* Per-parameter dim-0 sharding.  "ZeRO and FSDP", FSDP section: each
 * parameter sharded along its first dimension, a unit's shards packed into
 * one buffer per collective.  The cut is torch.chunk's: ceil(rows / n_dp)
 * rows per rank, the last ranks possibly short or empty (padded). */


int ora_dim0_layout(const int64_t *rows, const int64_t *cols, int64_t n_tensors,
                    int32_t n_dp, int64_t align, int64_t *packed_off,
                    int64_t *chunk_rows, int64_t out2[2]) {
    if (n_tensors < 0 || n_dp < 1 || align < 1 || out2 == 0) return -1;
    if (n_tensors > 0 && (rows == 0 || cols == 0)) return -1;
    int64_t n = 0, p = 0;
    for (int64_t i = 0; i < n_tensors; ++i) {
        if (rows[i] < 0 || cols[i] < 0) return -1;
        int64_t c = ceil_div(rows[i], n_dp);
        /* every size fits int64: the tensor, the flat total, the packed total */
        if (cols[i] > 0 && (rows[i] > INT64_MAX / cols[i] ||
                            rows[i] * cols[i] > INT64_MAX - n ||
                            c * cols[i] > INT64_MAX - p)) return -1;
        if (packed_off) packed_off[i] = p;
        if (chunk_rows) chunk_rows[i] = c;
        p += c * cols[i];
        n += rows[i] * cols[i];
    }
    if (ceil_div(p, align) > INT64_MAX / align) return -1;
    out2[0] = n;
    out2[1] = ceil_div(p, align) * align;
    return 0;
}

int64_t ora_dim0_segments(const int64_t *rows, const int64_t *cols,
                          int64_t n_tensors, int32_t n_dp, int64_t align,
                          int32_t rank, int64_t *quads, int64_t cap) {
    int64_t lay[2];
    if (ora_dim0_layout(rows, cols, n_tensors, n_dp, align, 0, 0, lay) != 0)
        return -1;
    if (rank < 0 || rank >= n_dp) return -1;
    int64_t count = 0, p = 0;
    for (int64_t i = 0; i < n_tensors; ++i) {
        int64_t c = ceil_div(rows[i], n_dp);
        int64_t first = (int64_t)rank * c;            /* first row of the chunk */
        int64_t have = rows[i] - first;               /* rows this rank holds */
        if (have > c) have = c;
        if (have < 0) have = 0;
        if (have > 0) {
            if (count < cap) {
                quads[4 * count + 0] = i;
                quads[4 * count + 1] = first * cols[i];
                quads[4 * count + 2] = p;
                quads[4 * count + 3] = have * cols[i];
            }
            ++count;
        }
        if (have < c && cols[i] > 0) {
            if (count < cap) {
                quads[4 * count + 0] = -1;
                quads[4 * count + 1] = 0;
                quads[4 * count + 2] = p + have * cols[i];
                quads[4 * count + 3] = (c - have) * cols[i];
            }
            ++count;
        }
        p += c * cols[i];
    }
    if (lay[1] > p) {
        if (count < cap) {
            quads[4 * count + 0] = -1;
            quads[4 * count + 1] = 0;
            quads[4 * count + 2] = p;
            quads[4 * count + 3] = lay[1] - p;
        }
        ++count;
    }
    return count;
}

/* "A sharded Adam step": the shards are the pieces of numpy.array_split,
 * whose first (n mod parts) pieces are one element longer. */
int64_t ora_array_split_start(int64_t n, int64_t parts, int64_t i) {
    int64_t each = n / parts, extra = n % parts;
    return i * each + (i < extra ? i : extra);
}

/* ------------------------------------------------------------------------ */
/* 16-bit formats.  bf16 is the top half of an fp32; fp16 is IEEE binary16. */

static float bits_to_f32(uint32_t u) {
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint32_t f32_to_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

float ora_bf16_to_f32(uint16_t h) { return bits_to_f32((uint32_t)h << 16); }

float ora_f16_to_f32(uint16_t h) {
    uint32_t sign = (uint32_t)(h >> 15) << 31;
    uint32_t e = (h >> 10) & 0x1F;
    uint32_t mant = h & 0x3FF;
    if (e == 0x1F) /* Inf / NaN: keep the payload */
        return bits_to_f32(sign | 0x7F800000u | (mant << 13));
    if (e != 0) /* normal: rebias 15 -> 127 */
        return bits_to_f32(sign | ((e + 112u) << 23) | (mant << 13));
    /* zero or subnormal: value = mant * 2^-24, exact in fp32 */
    float mag = (float)mant * 0x1p-24f;
    return sign ? -mag : mag;
}

uint16_t ora_f32_to_bf16(float f) {
    uint32_t u = f32_to_bits(f);
    uint32_t sign = u & 0x80000000u;
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) /* NaN */
        return (uint16_t)((sign >> 16) | 0x7FC0u);
    /* keep the top 16 bits, rounding the dropped 16 to nearest, ties to
     * even.  A carry out of the mantissa moves to the exponent, which turns
     * the largest finite values into Inf as rounding requires. */
    uint32_t hi = u >> 16, lo = u & 0xFFFFu;
    if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u))) hi += 1;
    return (uint16_t)hi;
}

uint16_t ora_f32_to_f16(float f) {
    uint32_t u = f32_to_bits(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t mag = u & 0x7FFFFFFFu;
    if (mag > 0x7F800000u) return (uint16_t)(sign | 0x7E00u); /* NaN */
    if (mag == 0x7F800000u) return (uint16_t)(sign | 0x7C00u); /* Inf */
    int32_t e = (int32_t)(mag >> 23) - 127; /* unbiased exponent */
    uint32_t m = mag & 0x7FFFFFu;
    if (e > 15) return (uint16_t)(sign | 0x7C00u); /* overflow */
    uint32_t full;  /* significand with implicit bit, 24 bits */
    int32_t shift;  /* right shift that lands it on the fp16 grid */
    uint32_t ebits; /* fp16 biased exponent before rounding */
    if (mag >= 0x38800000u) { /* |f| >= 2^-14: fp16 normal range */
        full = m | 0x800000u;
        shift = 13;
        ebits = (uint32_t)(e + 15);
    } else {
        /* at most half of 2^-24 (a tie goes to the even 0) -> signed zero;
         * this also covers every fp32 subnormal */
        if (mag <= 0x33000000u) return sign;
        /* subnormal target: value = q * 2^-24 with
         * q = round(full * 2^(e - 23 + 24)), a right shift by -e-1 in
         * [14, 24] because -25 <= e <= -15 here */
        full = m | 0x800000u;
        shift = -e - 1;
        ebits = 0;
    }
    uint32_t q = full >> shift;
    uint32_t rem = full & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u))) q += 1;
    uint32_t out;
    if (ebits == 0) {
        out = q; /* q <= 0x400; 0x400 is the smallest normal, correctly */
    } else {
        /* q in [0x400, 0x800]; 0x800 means the mantissa overflowed */
        out = (ebits << 10) + (q - 0x400u);
        if (out >= 0x7C00u) out = 0x7C00u;
    }
    return (uint16_t)(sign | out);
}

void ora_f32_to_bf16_n(const float *x, uint16_t *y, int64_t n) {
    for (int64_t i = 0; i < n; ++i) y[i] = ora_f32_to_bf16(x[i]);
}
void ora_f32_to_f16_n(const float *x, uint16_t *y, int64_t n) {
    for (int64_t i = 0; i < n; ++i) y[i] = ora_f32_to_f16(x[i]);
}
void ora_bf16_to_f32_n(const uint16_t *x, float *y, int64_t n) {
    for (int64_t i = 0; i < n; ++i) y[i] = ora_bf16_to_f32(x[i]);
}
void ora_f16_to_f32_n(const uint16_t *x, float *y, int64_t n) {
    for (int64_t i = 0; i < n; ++i) y[i] = ora_f16_to_f32(x[i]);
}

static float widen(uint16_t h, int dt) {
    return dt == ORA_FP16 ? ora_f16_to_f32(h) : ora_bf16_to_f32(h);
}

/* element i of a gradient row buffer: fp32 as stored, 16-bit widened */
static float grad_at(const void *grads, int gdt, int64_t i) {
    if (gdt == ORA_FP32) return ((const float *)grads)[i];
    return widen(((const uint16_t *)grads)[i], gdt);
}

static uint16_t narrow(float f, int dt) {
    return dt == ORA_FP16 ? ora_f32_to_f16(f) : ora_f32_to_bf16(f);
}

static int nonfinite(float f) { return isnan(f) || isinf(f); }

/* ------------------------------------------------------------------------ */
/* AdamW.  "ZeRO and FSDP", "A sharded Adam step":
 *   m <- b1 m + (1 - b1) g,  v <- b2 v + (1 - b2) g^2,
 *   w <- w - lr * mhat / (sqrt(vhat) + eps),
 *   mhat = m / (1 - b1^t), vhat = v / (1 - b2^t), t counted from 1.
 * The configs on "DeepSpeed ZeRO" ("A worked example") and "ZeRO Optimizer,
 * in depth" ("Running it with DeepSpeed") name AdamW with a weight decay; its
 * decay is the decoupled one (Loshchilov & Hutter): the master weight is
 * first multiplied by (1 - lr * wd), then the Adam step is subtracted.
 * Every scalar below is formed in double and rounded once to fp32. */

void ora_adamw_scalars(const double hp6[6], int64_t step, float out10[10]) {
    double lr = hp6[0], beta1 = hp6[1], beta2 = hp6[2], eps = hp6[3];
    double wd = hp6[4], grad_scale = hp6[5];
    out10[0] = (float)grad_scale;                       /* s   */
    out10[1] = (float)beta1;                            /* b1  */
    out10[2] = (float)(1.0 - beta1);                    /* c1  */
    out10[3] = (float)beta2;                            /* b2  */
    out10[4] = (float)(1.0 - beta2);                    /* c2  */
    out10[5] = (float)(1.0 - pow(beta1, (double)step)); /* bc1 */
    out10[6] = (float)(1.0 - pow(beta2, (double)step)); /* bc2 */
    out10[7] = (float)lr;                               /* lr  */
    out10[8] = (float)eps;                              /* eps */
    out10[9] = (float)(1.0 - lr * wd);                  /* d   */
}

/* one element of the update; g is the averaged fp32 gradient */
static void adamw_element(float g, float *w, float *m, float *v,
                          const float c[10]) {
    float b1 = c[1], c1 = c[2], b2 = c[3], c2 = c[4];
    float bc1 = c[5], bc2 = c[6], lr = c[7], eps = c[8], d = c[9];
    float mt = b1 * *m + c1 * g;
    float vt = b2 * *v + c2 * (g * g);
    float mhat = mt / bc1;
    float vhat = vt / bc2;
    float den = sqrtf(vhat) + eps;
    float u = mhat / den;
    float wt = *w * d - lr * u;
    *m = mt;
    *v = vt;
    *w = wt;
}

/* ------------------------------------------------------------------------ */
/* The reduce.  "ZeRO and FSDP", "The idea, one stage at a time": the reduce-
 * scatter hands rank r the averaged gradient of shard r.  Here the n ranks'
 * rows for that shard (16-bit, widened; or fp32) are summed left to right (the
 * average's scale is applied with the update).
 * Overflow flag: "DeepSpeed ZeRO", "Mixed precision" says fp16 training
 * needs loss scaling; what scaling guards against is a gradient that is no
 * longer finite.  The flag is raised when a reduced (and, for the reduce,
 * accumulated) fp32 gradient element is +-Inf or NaN, which covers every
 * non-finite input row and a sum that overflows. */

static float row_sum(const void *grads, int gdt, int32_t n, int64_t ld,
                     int64_t j) {
    float a = 0.0f;
    for (int32_t k = 0; k < n; ++k) {
        float x = grad_at(grads, gdt, (int64_t)k * ld + j);
        a = (k == 0) ? x : a + x;
    }
    return a;
}

void ora_reduce(const void *grads, int gdt, int32_t n_contrib, int64_t ld,
                int64_t len, float *acc, int accumulate, uint32_t *overflow,
                double *sumsq) {
    int bad = 0;
    double ss = 0.0;
    for (int64_t j = 0; j < len; ++j) {
        float a = row_sum(grads, gdt, n_contrib, ld, j);
        float r = accumulate ? acc[j] + a : a;
        if (nonfinite(r)) bad = 1;
        acc[j] = r;
        ss += (double)r * (double)r;
    }
    if (overflow && bad) *overflow = 1u;
    if (sumsq) *sumsq += ss;
}

void ora_adamw(const float *acc, float *w, float *m, float *v, uint16_t *wout,
               int wdt, int64_t len, const double hp6[6], int64_t step,
               const uint32_t *skip) {
    if (skip && *skip) return;
    float c[10];
    ora_adamw_scalars(hp6, step, c);
    for (int64_t j = 0; j < len; ++j) {
        float g = acc[j] * c[0];
        adamw_element(g, &w[j], &m[j], &v[j], c);
        wout[j] = narrow(w[j], wdt);
    }
}

/* Clipping.  Both configs of "DeepSpeed ZeRO" ("A worked example") and "ZeRO
 * Optimizer, in depth" ("Running it with DeepSpeed") set gradient clipping
 * to 1.0: the whole gradient is scaled down to norm max_norm when its
 * global norm is larger (the usual min(1, max_norm / (norm + 1e-6))). */
float ora_clip_coef(double sumsq, float s, double max_norm) {
    double norm = sqrt(sumsq) * (double)s;
    double c = max_norm / (norm + 1e-6);
    return c < 1.0 ? (float)c : 1.0f;
}

void ora_adamw_ex(const float *acc, float *w, float *m, float *v, uint16_t *wout,
                  int wdt, int64_t len, const double hp6[6], int64_t step,
                  const uint32_t *skip, const double *sumsq, double max_norm,
                  const float *loss_scale) {
    if (skip && *skip) return;
    float c[10];
    ora_adamw_scalars(hp6, step, c);
    if (loss_scale) c[0] = (float)(hp6[5] / (double)*loss_scale);
    float clip = 1.0f;
    if (sumsq && max_norm > 0.0) clip = ora_clip_coef(*sumsq, c[0], max_norm);
    for (int64_t j = 0; j < len; ++j) {
        float g = acc[j] * c[0];
        if (clip < 1.0f) g = g * clip;
        adamw_element(g, &w[j], &m[j], &v[j], c);
        wout[j] = narrow(w[j], wdt);
    }
}

/* Dynamic loss scaling: "DeepSpeed ZeRO", "Mixed precision" -- fp16 needs a
 * loss scale; read as the usual back-off on overflow and growth after a run
 * of finite steps. */
void ora_loss_scale_update(float *scale, int32_t *good_steps, uint32_t overflow,
                           double growth, double backoff, int32_t interval) {
    if (overflow) {
        *scale = (float)((double)*scale * backoff);
        *good_steps = 0;
        return;
    }
    *good_steps += 1;
    if (*good_steps >= interval) {
        float grown = (float)((double)*scale * growth);
        if (!isinf(grown)) *scale = grown; /* never grows to infinity */
        *good_steps = 0;
    }
}

void ora_step(const void *grads, int gdt, int32_t n_dp, int64_t ld,
              int64_t len, float *w, float *m, float *v, uint16_t *wout,
              int wdt, const double hp6[6], int64_t step, uint32_t *overflow,
              double *sumsq) {
    float c[10];
    ora_adamw_scalars(hp6, step, c);
    int bad = 0;
    double ss = 0.0;
    for (int64_t j = 0; j < len; ++j) {
        float a = row_sum(grads, gdt, n_dp, ld, j);
        if (nonfinite(a)) bad = 1;
        float g = a * c[0];
        ss += (double)g * (double)g;
        adamw_element(g, &w[j], &m[j], &v[j], c);
        wout[j] = narrow(w[j], wdt);
    }
    if (overflow && bad) *overflow = 1u;
    if (sumsq) *sumsq += ss;
}

/* ------------------------------------------------------------------------ */
/* 8-bit blockwise quantization.  The pages name ZeRO++'s 8-bit weight
 * all-gather and quantized gradient reduce-scatter without a quantizer; this
 * is the plain symmetric one, block by block (parity unpinned against the
 * pages). */

static float block_absmax(const void *x, int xdt, int64_t lo, int64_t hi) {
    float m = 0.0f;
    for (int64_t j = lo; j < hi; ++j) {
        float a = fabsf(grad_at(x, xdt, j));
        if (isnan(a) || a > m) m = a;
        if (isnan(m)) break; /* NaN is sticky */
    }
    return m;
}

void ora_q8_quantize(const void *x, int xdt, int64_t len, int8_t *q, float *scales) {
    for (int64_t lo = 0, b = 0; lo < len; lo += ORA_Q8_BLOCK, ++b) {
        int64_t hi = lo + ORA_Q8_BLOCK < len ? lo + ORA_Q8_BLOCK : len;
        float amax = block_absmax(x, xdt, lo, hi);
        float s = amax / 127.0f; /* the stored scale: value = code * s */
        scales[b] = s;
        for (int64_t j = lo; j < hi; ++j) {
            if (s == 0.0f || isnan(s) || isinf(s)) {
                q[j] = 0;
                continue;
            }
            /* the code is the value measured in units of the stored scale:
             * one correctly rounded division, then ties to even */
            float r = rintf(grad_at(x, xdt, j) / s);
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            q[j] = (int8_t)r;
        }
    }
}

static float dequant(const int8_t *q, const float *scales, int64_t j) {
    return (float)q[j] * scales[j / ORA_Q8_BLOCK];
}

void ora_q8_dequantize(const int8_t *q, const float *scales, int64_t len, void *y,
                       int ydt) {
    for (int64_t j = 0; j < len; ++j) {
        float f = dequant(q, scales, j);
        if (ydt == ORA_FP32) ((float *)y)[j] = f;
        else ((uint16_t *)y)[j] = narrow(f, ydt);
    }
}

void ora_step_q8(const int8_t *gq, const float *gs, int32_t n_dp, int64_t ld,
                 int64_t sld, int64_t len, float *w, float *m, float *v,
                 int8_t *wq, float *wscales, const double hp6[6], int64_t step,
                 uint32_t *overflow, double *sumsq) {
    float c[10];
    ora_adamw_scalars(hp6, step, c);
    int bad = 0;
    double ss = 0.0;
    for (int64_t j = 0; j < len; ++j) {
        float a = 0.0f;
        for (int32_t k = 0; k < n_dp; ++k) {
            float x = dequant(gq + (int64_t)k * ld, gs + (int64_t)k * sld, j);
            a = (k == 0) ? x : a + x;
        }
        if (nonfinite(a)) bad = 1;
        float g = a * c[0];
        ss += (double)g * (double)g;
        adamw_element(g, &w[j], &m[j], &v[j], c);
    }
    ora_q8_quantize(w, ORA_FP32, len, wq, wscales);
    if (overflow && bad) *overflow = 1u;
    if (sumsq) *sumsq += ss;
}

/* ------------------------------------------------------------------------ */
/* Re-sharding: element by element, through the flat index. */

void ora_reshard(const void *const *src, int32_t n_src, int64_t src_shard,
                 void *dst, int64_t dst_shard, int32_t dst_rank, int64_t n,
                 int32_t elem_bytes) {
    (void)n_src;
    for (int64_t j = 0; j < dst_shard; ++j) {
        int64_t flat = (int64_t)dst_rank * dst_shard + j;
        unsigned char *d = (unsigned char *)dst + j * elem_bytes;
        if (flat < n) {
            int64_t r = flat / src_shard, o = flat % src_shard;
            const unsigned char *s = (const unsigned char *)src[r] + o * elem_bytes;
            memcpy(d, s, (size_t)elem_bytes);
        } else {
            memset(d, 0, (size_t)elem_bytes);
        }
    }
}

int32_t ora_flat_locate(const int64_t *flat_off, const int64_t *len,
                        int32_t n_src, int64_t n, int64_t i, int64_t *off) {
    if (i < 0 || i >= n) return -1;
    for (int32_t k = 0; k < n_src; ++k) {
        if (i >= flat_off[k] && i - flat_off[k] < len[k]) {
            *off = i - flat_off[k];
            return k;
        }
    }
    return -1;
}

void ora_flat_gather(const void *const *src, const int64_t *flat_off,
                     const int64_t *len, int32_t n_src, int64_t n,
                     int64_t begin, int64_t count, void *dst,
                     int32_t elem_bytes) {
    for (int64_t j = 0; j < count; ++j) {
        unsigned char *d = (unsigned char *)dst + j * elem_bytes;
        int64_t off = 0;
        int32_t k = ora_flat_locate(flat_off, len, n_src, n, begin + j, &off);
        if (k >= 0)
            memcpy(d, (const unsigned char *)src[k] + off * elem_bytes, (size_t)elem_bytes);
        else
            memset(d, 0, (size_t)elem_bytes);
    }
}

void ora_flat_scatter(const void *src, int64_t begin, int64_t count,
                      void *const *dst, const int64_t *flat_off,
                      const int64_t *len, int32_t n_dst, int32_t elem_bytes) {
    for (int64_t j = 0; j < count; ++j) {
        int64_t off = 0;
        int32_t k = ora_flat_locate(flat_off, len, n_dst, INT64_MAX, begin + j, &off);
        if (k >= 0)
            memcpy((unsigned char *)dst[k] + off * elem_bytes,
                   (const unsigned char *)src + j * elem_bytes, (size_t)elem_bytes);
    }
}

/* ------------------------------------------------------------------------ */
/* Accounting.  "ZeRO and FSDP", "Memory per GPU": weights 2N, gradients 2N,
 * optimizer K N; stage 1 divides the optimizer term by n_dp, stage 2 also
 * the gradients, stage 3 also the weights. */

double ora_model_state_bytes(double n, double n_dp, int stage, double k) {
    double w = 2.0 * n, g = 2.0 * n, o = k * n;
    switch (stage) {
    case 0: return w + g + o;
    case 1: return w + g + o / n_dp;
    case 2: return w + g / n_dp + o / n_dp;
    case 3: return w / n_dp + g / n_dp + o / n_dp;
    default: return -1.0;
    }
}

/* "ZeRO and FSDP", "Communication volume": a ring reduce-scatter or all-
 * gather of N elements sends (n_dp - 1) N / n_dp per GPU, an all-reduce
 * twice that.  Stage 0 all-reduces gradients; stages 1 and 2 reduce-scatter
 * gradients and all-gather weights; stage 3 all-gathers weights twice and
 * reduce-scatters gradients. */
double ora_comm_bytes(double n, double n_dp, int stage, double param_bytes,
                      double grad_bytes) {
    double f = (n_dp - 1.0) / n_dp * n;
    switch (stage) {
    case 0: return 2.0 * f * grad_bytes;
    case 1:
    case 2: return f * grad_bytes + f * param_bytes;
    case 3: return 2.0 * f * param_bytes + f * grad_bytes;
    default: return -1.0;
    }
}
