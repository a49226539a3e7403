/*
 * oracle_zero.h -- the CPU oracle for one rank's sharded mixed-precision
 * optimizer step (flatten + shard, gradient reduce, fp32 AdamW, 16-bit cast).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this code: it exists so that tests, the smoke check and the
 * benchmark's CPU-baseline leg have an independent, plainly written reference.
 * It shares no source with the HIP library (its own header, its own
 * converters, its own constant set-up).
 *
 * Everything here is single-threaded, element by element, in IEEE binary32
 * with round-to-nearest-even (fp32 is the precision the pages fix for the
 * master weights and both Adam moments), every operation written out, built
 * with -ffp-contract=off so that no multiply-add is fused.
 *
 * Sources (page title, then section):
 *  - "ZeRO and FSDP" (Zero to Frontier, section 10.3), "The idea, one stage
 *    at a time": flatten all parameters into one vector of N, cut it into
 *    n_dp equal contiguous shards, rank r owns shard r; stage 1 reduce-
 *    scatters the averaged gradient, updates the fp32 master shard, casts it
 *    to bfloat16, and all-gathers.  Same page, "A sharded Adam step": the
 *    average over ranks, Adam with bias correction from t = 1.  Same page,
 *    "Memory per GPU" and "Communication volume": the accounting formulas.
 *  - "ZeRO Optimizer, in depth ..." (aicassindra), "Where the 16 bytes per
 *    parameter go": 2 + 2 + 12 bytes per parameter.
 *  - "DeepSpeed ZeRO" (ozercemkelahmet), "Mixed precision": fp16 needs loss
 *    scaling; the configs there name AdamW.
 *
 * Parity status per function is listed in oracle_zero.c's header.
 */
#ifndef ORACLE_ZERO_H
#define ORACLE_ZERO_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage formats: 16-bit for gradients and weights; gradients may also
 * arrive in fp32 ("ZeRO and FSDP", FSDP section: the float32 reduce-scatter
 * of the mixed-precision policy; Llama 3 reduces its gradients in float32). */
enum { ORA_BF16 = 0, ORA_FP16 = 1, ORA_FP32 = 2 };

/* ---- layout: flatten + equal contiguous shards ---------------------------
 * numels[n_tensors] -> offsets[n_tensors] (prefix sums, nullable),
 * out3 = {N, N_pad, S} with S = align * ceil(N / (n_dp * align)),
 * N_pad = n_dp * S.  Returns 0, or -1 on invalid arguments. */
int ora_flatten_layout(const int64_t *numels, int64_t n_tensors, int32_t n_dp,
                       int64_t align, int64_t *offsets, int64_t out3[3]);

/* The pieces of shard `rank`: quads {tensor, tensor_off, shard_off, len},
 * tensor = -1 for padding.  Writes at most cap quads, returns the total
 * count (or -1 on invalid arguments). */
int64_t ora_shard_segments(const int64_t *numels, int64_t n_tensors,
                           int32_t n_dp, int64_t align, int32_t rank,
                           int64_t *quads, int64_t cap);

/* ---- per-parameter dim-0 sharding (FSDP2) ---------------------------------
 * "ZeRO and FSDP", FSDP section: every parameter is a distributed tensor
 * sharded along its first dimension, and a unit's shards are packed into one
 * buffer for each collective.  Tensor i has rows[i] rows of cols[i]
 * elements and is cut as torch.chunk cuts it: c_i = ceil(rows_i / n_dp) rows
 * per rank, rank r holding rows [r c_i, min((r + 1) c_i, rows_i)) (maybe
 * none).  Every rank's packed buffer holds tensor i's chunk at packed offset
 * P_i = sum over j < i of c_j cols_j, zero-padded to c_i rows, and ends with
 * zero padding up to S = align * ceil(sum c_i cols_i / align).
 * packed_off, chunk_rows (nullable): P_i and c_i.  out2 = {N, S}.
 * Returns 0, or -1 on invalid arguments (negative sizes, n_dp < 1, align < 1). */
int ora_dim0_layout(const int64_t *rows, const int64_t *cols, int64_t n_tensors,
                    int32_t n_dp, int64_t align, int64_t *packed_off,
                    int64_t *chunk_rows, int64_t out2[2]);

/* The pieces of rank `rank`'s packed buffer in buffer order: quads
 * {tensor, tensor_off, shard_off, len}, tensor = -1 for padding.  Writes at
 * most cap quads, returns the total count (or -1 on invalid arguments). */
int64_t ora_dim0_segments(const int64_t *rows, const int64_t *cols,
                          int64_t n_tensors, int32_t n_dp, int64_t align,
                          int32_t rank, int64_t *quads, int64_t cap);

/* Boundaries of numpy.array_split(range(n), parts): start of piece i. */
int64_t ora_array_split_start(int64_t n, int64_t parts, int64_t i);

/* ---- 16-bit <-> fp32 conversions ------------------------------------------ */
float ora_bf16_to_f32(uint16_t h);
float ora_f16_to_f32(uint16_t h);
uint16_t ora_f32_to_bf16(float f); /* RNE; NaN -> sign | 0x7FC0 */
uint16_t ora_f32_to_f16(float f);  /* RNE; NaN -> sign | 0x7E00 */
void ora_f32_to_bf16_n(const float *x, uint16_t *y, int64_t n);
void ora_f32_to_f16_n(const float *x, uint16_t *y, int64_t n);
void ora_bf16_to_f32_n(const uint16_t *x, float *y, int64_t n);
void ora_f16_to_f32_n(const uint16_t *x, float *y, int64_t n);

/* ---- AdamW scalars --------------------------------------------------------
 * hp6 = {lr, beta1, beta2, eps, weight_decay, grad_scale} as doubles, step
 * t >= 1.  out10 = {s, b1, c1, b2, c2, bc1, bc2, lr, eps, d} in fp32, each
 * computed in double and rounded once. */
void ora_adamw_scalars(const double hp6[6], int64_t step, float out10[10]);

/* ---- the reduce (the reduce-scatter's arithmetic for one shard) -----------
 * a_j = G_0[j] + G_1[j] + ... + G_{n-1}[j], widened to fp32 (16-bit rows)
 * or read as they are (gdt = ORA_FP32, grads then points at floats), summed
 * left to right.
 * accumulate == 0: acc[j] = a_j; else acc[j] = acc[j] + a_j.
 * overflow (nullable): set to 1 if any acc[j] after the update is +-Inf or
 * NaN (so any non-finite input, or a sum that overflowed).
 * sumsq (nullable): += sum over j of acc[j]^2 (after the update), in double. */
void ora_reduce(const void *grads, int gdt, int32_t n_contrib, int64_t ld,
                int64_t len, float *acc, int accumulate, uint32_t *overflow,
                double *sumsq);

/* ---- AdamW from an fp32 gradient buffer ------------------------------------
 * g = acc[j] * s, then the AdamW element update of w/m/v, and
 * wout[j] = 16-bit cast of the new w (wdt).  skip (nullable): if *skip != 0
 * nothing at all is written. */
void ora_adamw(const float *acc, float *w, float *m, float *v, uint16_t *wout,
               int wdt, int64_t len, const double hp6[6], int64_t step,
               const uint32_t *skip);

/* ---- clipping and dynamic loss scaling -------------------------------------
 * Global-norm clipping coefficient: with s the fp32 scale applied to the
 * accumulated gradient and sumsq the sum over the whole model of acc^2,
 * norm = sqrt(sumsq) * s and c = min(1, max_norm / (norm + 1e-6)), all in
 * double, rounded once to fp32. */
float ora_clip_coef(double sumsq, float s, double max_norm);

/* ora_adamw with the optional controls: skip (as before); loss_scale
 * (nullable): s = fl(grad_scale / *loss_scale) instead of fl(grad_scale);
 * sumsq (nullable) with max_norm > 0: every g = acc * s is then multiplied
 * by c = ora_clip_coef(*sumsq, s, max_norm) when c < 1. */
void ora_adamw_ex(const float *acc, float *w, float *m, float *v, uint16_t *wout,
                  int wdt, int64_t len, const double hp6[6], int64_t step,
                  const uint32_t *skip, const double *sumsq, double max_norm,
                  const float *loss_scale);

/* One step of the dynamic loss scale: on overflow scale *= backoff and the
 * count of good steps restarts; otherwise the count grows and, on reaching
 * interval, scale *= growth (kept unchanged if that would be infinite) and
 * the count restarts (products in double, rounded to fp32). */
void ora_loss_scale_update(float *scale, int32_t *good_steps, uint32_t overflow,
                           double growth, double backoff, int32_t interval);

/* ---- fused: reduce n_dp rows, then AdamW, then cast -----------------------
 * Equal, element by element, to ora_reduce(accumulate = 0) into a temporary
 * followed by ora_adamw.  overflow is set when a reduced a_j is non-finite
 * (the update is still applied); sumsq (nullable) += sum of g_j^2 with
 * g_j = a_j * s. */
void ora_step(const void *grads, int gdt, int32_t n_dp, int64_t ld,
              int64_t len, float *w, float *m, float *v, uint16_t *wout,
              int wdt, const double hp6[6], int64_t step, uint32_t *overflow,
              double *sumsq);

/* ---- re-sharding (checkpoint conversion) ----------------------------------
 * "ZeRO Optimizer, in depth", "Checkpoints: sharded on the way in,
 * consolidated on the way out": a sharded checkpoint is tied to its layout;
 * converting it to another GPU count (or consolidating it) moves each flat
 * element to its new place.  src[r] is old rank r's shard of src_shard
 * elements (n_src of them); dst receives new rank dst_rank's shard of
 * dst_shard elements: dst[j] = flat[dst_rank * dst_shard + j] for flat
 * indices below n, 0 beyond.  elem_bytes is 2 or 4. */
void ora_reshard(const void *const *src, int32_t n_src, int64_t src_shard,
                 void *dst, int64_t dst_shard, int32_t dst_rank, int64_t n,
                 int32_t elem_bytes);

/* The general form, for flattening, unflattening and partial checkpoints.
 * A "flat set" is n_src pieces of the flat vector, piece k holding flat
 * indices [flat_off[k], flat_off[k] + len[k]) in src[k] (pieces that do not
 * overlap).  ora_flat_locate returns the piece that holds flat index i
 * (setting *off to the index inside it), or -1 when i >= n or no piece does.
 * ora_flat_gather: dst[j] = flat[begin + j] for j < count, 0 where
 * ora_flat_locate gives -1.  ora_flat_scatter is the inverse: for every flat
 * index i in [begin, begin + count) that piece k holds, dst[k] at i's place
 * receives src[i - begin]; nothing else is written. */
int32_t ora_flat_locate(const int64_t *flat_off, const int64_t *len,
                        int32_t n_src, int64_t n, int64_t i, int64_t *off);
void ora_flat_gather(const void *const *src, const int64_t *flat_off,
                     const int64_t *len, int32_t n_src, int64_t n,
                     int64_t begin, int64_t count, void *dst,
                     int32_t elem_bytes);
void ora_flat_scatter(const void *src, int64_t begin, int64_t count,
                      void *const *dst, const int64_t *flat_off,
                      const int64_t *len, int32_t n_dst, int32_t elem_bytes);

/* ---- 8-bit blockwise quantization (ZeRO++) --------------------------------
 * "ZeRO: How DeepSpeed Made Trillion-Parameter Training Practical" and
 * "ZeRO and FSDP" (FSDP section, "Fewer bytes on the wire"): ZeRO++
 * quantizes the weight all-gather to 8 bits and the gradients of the
 * reduce-scatter.  The pages define no quantizer; the one here is the plain
 * symmetric blockwise int8 quantizer (PARITY UNPINNED against the pages: it
 * is pinned only to its own mathematical properties).
 * Blocks of ORA_Q8_BLOCK consecutive elements (the last one may be short);
 * for block i, in fp32: s_i = absmax_i / 127 (absmax over the block, NaN if
 * any element is NaN); q_j = rint(x_j / s_i), one correctly rounded
 * division, then round-to-nearest-even to an integer, clamped to
 * [-127, 127]; s_i == 0 (absmax at most 127 times half the smallest
 * subnormal) or s_i not finite gives q_j = 0 (so a block with an Inf or NaN
 * dequantizes to NaN).  Dequantized: q_j * s_i. */
#define ORA_Q8_BLOCK 256
void ora_q8_quantize(const void *x, int xdt, int64_t len, int8_t *q, float *scales);
void ora_q8_dequantize(const int8_t *q, const float *scales, int64_t len, void *y,
                       int ydt);

/* Fused step with 8-bit communication on both sides: a_j = sum over k of
 * q_k[j] * s_k[j / B] (each product rounded to fp32, summed left to right;
 * row k at gq + k * ld, its scales at gs + k * sld), g = a * s, AdamW as
 * ora_step, then the new w quantized into wq / wscales (blocks from
 * element 0 of the range).  overflow / sumsq as ora_step. */
void ora_step_q8(const int8_t *gq, const float *gs, int32_t n_dp, int64_t ld,
                 int64_t sld, int64_t len, float *w, float *m, float *v,
                 int8_t *wq, float *wscales, const double hp6[6], int64_t step,
                 uint32_t *overflow, double *sumsq);

/* ---- accounting ----------------------------------------------------------
 * Model-state bytes per GPU for stage 0..3 with 2-byte weights and grads and
 * K bytes of optimizer state per parameter; -1 for any other stage. */
double ora_model_state_bytes(double n, double n_dp, int stage, double k);
/* Bytes each GPU sends per optimizer step under ring collectives. */
double ora_comm_bytes(double n, double n_dp, int stage, double param_bytes,
                      double grad_bytes);

#ifdef __cplusplus
}
#endif
#endif
