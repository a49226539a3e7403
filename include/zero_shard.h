/*
 * zero_shard.h -- C ABI of the MI355X (gfx950) library for one data-parallel
 * rank's sharded mixed-precision optimizer step.
 *
 * The path, as the pages describe it:
 *  1. Flatten every parameter into one vector of N numbers and cut it into
 *     n_dp equal contiguous shards; rank r owns shard r ("ZeRO and FSDP",
 *     Zero to Frontier 10.3, "The idea, one stage at a time").
 *  2. Reduce-scatter the 16-bit gradients so rank r holds the average over
 *     ranks of shard r (same section; "ZeRO Optimizer, in depth", "What each
 *     stage changes inside one step").  On one GPU the n_dp ranks' rows for
 *     the owned shard sit in HBM and this library performs the collective's
 *     arithmetic: widen to fp32, sum, scale.
 *  3. With gradient accumulation at stage 2, reduce after every micro-batch
 *     into an fp32 shard buffer ("ZeRO and FSDP", the catch described under
 *     "The idea, one stage at a time").
 *  4. Run AdamW on the fp32 master weights and the two fp32 moments of the
 *     shard ("ZeRO and FSDP", "A sharded Adam step": Adam with bias
 *     correction from t = 1; the configs of "DeepSpeed ZeRO", "A worked
 *     example", name AdamW, applied with decoupled weight decay).
 *  5. Cast the updated master to 16 bits into the shard's slot of the full
 *     weight buffer, which is where the all-gather delivers it ("ZeRO and
 *     FSDP", "The idea, one stage at a time").
 * The state is the 2 + 2 + 12 bytes per parameter of "ZeRO Optimizer, in
 * depth", "Where the 16 bytes per parameter go".
 *
 * Conventions for every entry point:
 *  - Device pointers are plain HIP device addresses the caller allocated
 *    (e.g. torch.empty(..., device="cuda")).  The library allocates and
 *    frees nothing, on the device or the host, and keeps no global state;
 *    the caller owns every buffer before, during and after a call.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream)
 *    and runs asynchronously: a call returns once its kernels are launched.
 *    Buffers must stay valid until the stream has passed them.
 *  - Arguments are validated on the host before anything is launched; on any
 *    error status nothing is launched and nothing is written.  (Values held
 *    in device memory -- flags, sums, a loss scale, the step constants of
 *    the _dc variants -- are read when the kernels run and used as they
 *    are.)
 *  - Element counts and offsets are in elements, never bytes; one call
 *    processes at most 2^38 elements (EINVAL beyond), and a buffer or set of
 *    rows it addresses spans at most 2^60 elements (EINVAL beyond: a layout's
 *    N_pad, or (rows - 1) * ld + len for rows ld elements apart).
 *  - Element j of the processed range is independent of every other element:
 *    any range can be processed by one call or split over several calls
 *    (buckets) with identical results -- except the optional sum of squares,
 *    a reduction over the range, whose last bits depend on the split (for a
 *    given split they are the same on every run).
 *  - Arithmetic is IEEE binary32 with round-to-nearest-even, no fused
 *    multiply-add, correctly rounded division and square root, and no
 *    flushing of denormals; the scalars are formed on the host in double
 *    and rounded once to fp32 (see zero_adamw_hparams; the _dc variants
 *    read them from device memory, formed by zero_step_consts_make).
 */
#ifndef ZERO_SHARD_H
#define ZERO_SHARD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZERO_SHARD_ABI_VERSION 4

/* every entry point is exported from the shared library */
#if defined(__GNUC__) || defined(__clang__)
#define ZERO_API __attribute__((visibility("default")))
#else
#define ZERO_API
#endif

typedef enum zero_status {
    ZERO_OK = 0,
    ZERO_EINVAL = 1,  /* a required pointer is NULL, or a size, count, rank,
                         dtype, stage or hyperparameter is out of its domain */
    ZERO_EALIAS = 2,  /* two buffers that must be disjoint overlap */
    ZERO_ERANGE = 3,  /* the range to process does not fit in the shard or
                         in the full weight buffer */
    ZERO_EDEVICE = 4  /* the HIP runtime refused a kernel launch; faults
                         inside kernels surface at the caller's next
                         synchronisation instead */
} zero_status;

/* Storage formats.  Weights are 16-bit (BF16, FP16); gradient rows may also
 * be fp32 (ZERO_FP32: the float32 reduce-scatter of the mixed-precision
 * policy in "ZeRO and FSDP", FSDP section; 4 bytes per element). */
typedef enum zero_dtype { ZERO_BF16 = 0, ZERO_FP16 = 1, ZERO_FP32 = 2 } zero_dtype;

/* Flat layout: N parameters, n_dp shards of `shard` elements each,
 * n_pad = n_dp * shard >= n; elements [n, n_pad) are zero padding.
 * shard is the smallest multiple of `align` with n_dp * shard >= n. */
typedef struct zero_layout {
    int64_t n;
    int64_t n_pad;
    int64_t shard;
    int64_t align;
    int32_t n_dp;
    int32_t reserved; /* zero */
} zero_layout;

/* AdamW hyperparameters.  Doubles on purpose: each fp32 constant of the
 * update is formed in double and rounded once, so that (1 - beta1) is the
 * float nearest 0.1 and not 1 - (float)0.9.  The constants are
 *   s = fl(grad_scale), b1 = fl(beta1), c1 = fl(1 - beta1),
 *   b2 = fl(beta2), c2 = fl(1 - beta2),
 *   bc1 = fl(1 - pow(beta1, step)), bc2 = fl(1 - pow(beta2, step)),
 *   lr = fl(lr), eps = fl(eps), d = fl(1 - lr * weight_decay)
 * with pow from the C library and fl() the round-to-nearest conversion to
 * float.  Per element j, with a_j the fp32 sum of the contributions:
 *   g = a_j * s
 *   m = b1 * m + c1 * g
 *   v = b2 * v + c2 * (g * g)
 *   w = w * d - lr * ((m / bc1) / (sqrt(v / bc2) + eps))
 *   out = 16-bit round-to-nearest-even of w
 * (each operation rounded to fp32 in this order). */
typedef struct zero_adamw_hparams {
    double lr;
    double beta1;        /* in [0, 1) */
    double beta2;        /* in [0, 1) */
    double eps;          /* finite, > 0 */
    double weight_decay; /* finite, >= 0 */
    double grad_scale;   /* finite, > 0: 1 / (n_dp * loss_scale * micro_batches)
                            averages over ranks and micro-batches and undoes a
                            static fp16 loss scale */
    int64_t step;        /* t >= 1, counted from 1 */
} zero_adamw_hparams;

/* One contiguous piece of a shard: elements [shard_off, shard_off + len) of
 * the shard are elements [tensor_off, tensor_off + len) of parameter
 * `tensor`, or of the zero padding when tensor == -1. */
typedef struct zero_segment {
    int64_t tensor;
    int64_t tensor_off;
    int64_t shard_off;
    int64_t len;
} zero_segment;

/* ZERO_SHARD_ABI_VERSION of the loaded library. */
ZERO_API int32_t zero_abi_version(void);

/* A static, human-readable name for a status code (never NULL). */
ZERO_API const char *zero_status_string(zero_status status);

/* ---- layout (host only) ------------------------------------------------
 * Flatten n_tensors parameters of numels[i] elements, in that order, into
 * one vector and cut it into n_dp equal contiguous shards ("ZeRO and FSDP",
 * "The idea, one stage at a time").  offsets (nullable, n_tensors entries)
 * receives each parameter's first flat index.  align >= 1 rounds the shard
 * up to a multiple of align (8 makes every shard slot 16-byte aligned for
 * 16-bit data); align = 1 gives the plain ceil(N / n_dp).
 * EINVAL: out NULL, numels NULL with n_tensors > 0, n_tensors < 0, a numel
 * < 0, n_dp < 1, align < 1, or N_pad overflowing int64. */
ZERO_API zero_status zero_flatten_layout(const int64_t *numels, int64_t n_tensors,
                                int32_t n_dp, int64_t align,
                                int64_t *offsets, zero_layout *out);

/* The pieces of shard `rank` in shard order: the parameters it overlaps,
 * then the padding.  Writes min(count, cap) entries to out (nullable when
 * cap == 0) and the total number to *count.  The layout must be the one
 * zero_flatten_layout returns for the same numels.
 * EINVAL: NULL layout/count, numels NULL with n_tensors > 0, cap < 0,
 * rank outside [0, n_dp), or numels inconsistent with the layout. */
ZERO_API zero_status zero_shard_segments(const zero_layout *layout,
                                const int64_t *numels, int64_t n_tensors,
                                int32_t rank, zero_segment *out, int64_t cap,
                                int64_t *count);

/* The pieces of the functional sharded step ("ZeRO and FSDP", "A sharded
 * Adam step"): rank r of n_dp holds elements [starts[r], starts[r] +
 * lens[r]) of a vector of n, cut as numpy.array_split cuts it -- the first
 * (n mod n_dp) pieces one element longer than the others, no padding.  (When
 * n_dp divides n these are the equal shards of zero_flatten_layout.)
 * starts, lens: host arrays of n_dp elements, written.  Host only.
 * EINVAL: n < 0, n_dp < 1, NULL starts or lens (nothing written). */
ZERO_API zero_status zero_array_split_layout(int64_t n, int32_t n_dp, int64_t *starts,
                                             int64_t *lens);

/* ---- per-parameter dim-0 sharding (host only) ------------------------------
 * "ZeRO and FSDP", FSDP section: FSDP2 keeps every parameter as a tensor
 * sharded along its first dimension and packs a unit's shards into one
 * buffer for each collective.  Tensor i is rows[i] x cols[i] (cols = the
 * product of its other dimensions; 1 for a vector).  It is cut as
 * torch.chunk cuts it: c_i = ceil(rows_i / n_dp) rows per rank, rank r
 * holding rows [r c_i, min((r + 1) c_i, rows_i)) -- possibly none.  Every
 * rank's packed buffer holds tensor i's chunk at offset P_i = sum over j < i
 * of c_j cols_j, zero-padded to c_i rows, and ends with zero padding up to
 * shard = align * ceil(sum c_i cols_i / align).
 * *out is a zero_layout that the device entry points take unchanged: n =
 * sum rows_i cols_i, shard as above, n_pad = n_dp * shard; rank r's packed
 * buffer is its shard, and weight_full is the all-gather buffer holding the
 * ranks' packed buffers one after another.  packed_off and chunk_rows
 * (nullable, n_tensors entries) receive P_i and c_i.
 * EINVAL: out NULL, rows/cols NULL with n_tensors > 0, n_tensors < 0, a
 * negative size, n_dp < 1, align < 1, or a size overflowing int64. */
ZERO_API zero_status zero_dim0_layout(const int64_t *rows, const int64_t *cols,
                                      int64_t n_tensors, int32_t n_dp, int64_t align,
                                      int64_t *packed_off, int64_t *chunk_rows,
                                      zero_layout *out);

/* The pieces of rank `rank`'s packed buffer in buffer order: for each
 * tensor its rows (tensor_off = first row * cols) and then its padding rows,
 * and the end padding (tensor == -1 for padding).  Conventions as for
 * zero_shard_segments; a piece list for zero_flat_gather (pack) and
 * zero_flat_scatter (unpack) follows directly: tensor t's piece is
 * (ptr_t + tensor_off, shard_off, len).
 * EINVAL as for zero_shard_segments, or rows/cols inconsistent with the
 * layout (which must come from zero_dim0_layout). */
ZERO_API zero_status zero_dim0_segments(const zero_layout *layout, const int64_t *rows,
                                        const int64_t *cols, int64_t n_tensors,
                                        int32_t rank, zero_segment *out, int64_t cap,
                                        int64_t *count);

/* ---- the sum of squares' workspace ----------------------------------------
 * A call that sums squares (sumsq != NULL: zero_shard_reduce,
 * zero_shard_step, zero_shard_step_q8) stores one fp64 partial per
 * workgroup in a caller-provided device workspace, then adds the partials
 * into *sumsq in an order fixed by len and the buffers' alignment alone --
 * the same inputs give the same bits on every run.  The workspace holds at
 * least zero_sumsq_workspace_bytes(len) bytes (8 * (256 + ceil(len / 256) +
 * 4096): 8 bytes per 256 elements plus 34 KiB), is 8-byte aligned,
 * overlaps no other argument, and is scratch: its contents on entry are
 * ignored and on exit unspecified.  Calls that share a workspace must not
 * run concurrently.  Returns -1 for len < 0 or len > 2^38. */
ZERO_API int64_t zero_sumsq_workspace_bytes(int64_t len);

/* ---- the reduce (device) ------------------------------------------------
 * The reduce-scatter's arithmetic for one shard range, with optional
 * micro-batch accumulation (stage 2 reduces after every micro-batch).
 *   grads: device, dtype gdt (BF16, FP16 or FP32), n_contrib rows; row k
 *          starts at element
 *          k * ld and holds that rank's gradient for elements [0, len) of
 *          the range.  ld = len is a packed [n_contrib][len] slab; ld =
 *          N_pad with grads already offset to the shard start reads each
 *          rank's full flat gradient in place.  Read only.
 *   acc:   device fp32[len].  accumulate == 0: acc[j] = a_j; otherwise
 *          acc[j] = acc[j] + a_j, where a_j = G_0[j] + ... + G_{n-1}[j]
 *          summed left to right in fp32 (16-bit rows widened exactly, fp32
 *          rows as stored).  No scale is applied here.
 *   overflow: device uint32 or NULL; set to 1 (never cleared) when some
 *          acc[j] after the update is +-Inf or NaN.
 *   sumsq: device double or NULL; the sum over j of acc[j]^2 (in fp64) is
 *          ADDED to it, through workspace (see zero_sumsq_workspace_bytes;
 *          ignored when sumsq is NULL).  The caller zeroes overflow and
 *          sumsq before a pass.
 * EINVAL: n_contrib < 1, len < 0, ld < len, bad gdt, a NULL grads/acc
 * with len > 0, or sumsq given with a missing, unaligned or short
 * workspace.  EALIAS: acc, overflow, sumsq, the workspace overlap each
 * other or a row.  len == 0 is a no-op. */
ZERO_API zero_status zero_shard_reduce(const void *grads, zero_dtype gdt,
                              int32_t n_contrib, int64_t ld, int64_t len,
                              float *acc, int32_t accumulate,
                              uint32_t *overflow, double *sumsq, void *workspace,
                              int64_t workspace_bytes, void *stream);

/* ---- AdamW from an fp32 gradient buffer (device) -------------------------
 * For j in [0, len): g = acc[j] * s, the AdamW update of master[j], m[j],
 * v[j] in place (see zero_adamw_hparams), and the 16-bit cast of the new
 * master written to weight_full[rank * shard + shard_off + j].
 *   acc, master, m, v: device fp32[len], pointing at shard element
 *          shard_off.  Nothing else of weight_full is touched.
 *   skip:  device uint32 or NULL; when *skip != 0 at run time the kernel
 *          writes nothing (a step skipped after an overflow).
 * EINVAL: bad layout, rank, dtype, hyperparameters, shard_off < 0, len < 0,
 * or a NULL required pointer with len > 0.  ERANGE: shard_off + len >
 * shard.  EALIAS: any two of acc, master, m, v, the weight slot, skip
 * overlap. */
ZERO_API zero_status zero_shard_adamw(const float *acc, float *master, float *m,
                             float *v, void *weight_full, zero_dtype wdt,
                             const zero_layout *layout, int32_t rank,
                             int64_t shard_off, int64_t len,
                             const zero_adamw_hparams *hp,
                             const uint32_t *skip, void *stream);

/* ---- step controls: clipping and dynamic loss scaling (device) ------------
 * Both configs of "DeepSpeed ZeRO" ("A worked example") and "ZeRO Optimizer,
 * in depth" ("Running it with DeepSpeed") clip the gradient to global norm
 * 1.0, and fp16 training needs a loss scale ("DeepSpeed ZeRO", "Mixed
 * precision").  Both are decided on the device, so a step never waits for
 * the host:
 *   1. zero_shard_reduce per micro-batch into acc, with overflow, and on the
 *      last one sumsq (= the sum of acc^2 over this rank's shard);
 *   2. all-reduce overflow (max) and sumsq (sum) over the ranks (on one GPU
 *      the caller sums the ranks' partials);
 *   3. zero_shard_adamw_ex with skip = overflow, sumsq, max_norm, loss_scale;
 *   4. zero_loss_scale_update with the same overflow flag. */

/* Dynamic loss scale in device memory (8 bytes, caller-owned). */
typedef struct zero_loss_scale {
    float scale;         /* current loss scale, finite and > 0 */
    int32_t good_steps;  /* finite steps since the scale last changed */
} zero_loss_scale;

/* Optional controls of zero_shard_adamw_ex; every pointer is a nullable
 * device address.
 *   skip:       when *skip != 0 nothing is written.
 *   sumsq:      the sum over the whole model (all ranks) of acc^2; with
 *               max_norm > 0 the gradient is clipped: with norm =
 *               sqrt(*sumsq) * s (double) and c = min(1, max_norm /
 *               (norm + 1e-6)) rounded to fp32, every g = acc * s is
 *               multiplied by c when c < 1.
 *   loss_scale: s = fl(grad_scale / loss_scale->scale) (double division,
 *               rounded once) instead of fl(grad_scale); grad_scale then
 *               holds only 1 / (n_dp * micro_batches). */
typedef struct zero_step_control {
    const uint32_t *skip;
    const double *sumsq;
    double max_norm;
    const zero_loss_scale *loss_scale;
} zero_step_control;

/* zero_shard_adamw with controls (ctl nullable = none).  Errors as for
 * zero_shard_adamw; EINVAL also for a non-finite max_norm, EALIAS when a
 * control overlaps an output. */
ZERO_API zero_status zero_shard_adamw_ex(const float *acc, float *master, float *m,
                                         float *v, void *weight_full, zero_dtype wdt,
                                         const zero_layout *layout, int32_t rank,
                                         int64_t shard_off, int64_t len,
                                         const zero_adamw_hparams *hp,
                                         const zero_step_control *ctl, void *stream);

/* One step of the dynamic loss scale, on the device: if *overflow != 0 the
 * scale is multiplied by backoff and good_steps restarts at 0; otherwise
 * good_steps grows by one and on reaching interval the scale is multiplied
 * by growth (unless that product would be infinite) and good_steps restarts
 * (products in double, rounded to fp32).
 * EINVAL: NULL state/overflow, growth not finite or < 1, backoff outside
 * (0, 1], interval < 1.  EALIAS: state and overflow overlap. */
ZERO_API zero_status zero_loss_scale_update(zero_loss_scale *state,
                                            const uint32_t *overflow, double growth,
                                            double backoff, int32_t interval,
                                            void *stream);

/* ---- fused step (device) ---------------------------------------------------
 * One pass over the range: reduce layout->n_dp rows in fp32 (as
 * zero_shard_reduce with accumulate = 0), scale by s, AdamW, cast into the
 * slot -- bit-identical to zero_shard_reduce followed by zero_shard_adamw,
 * but each element's bytes cross HBM once: 2 * n_dp bytes of gradients (4 *
 * n_dp for fp32 rows) and 12 of state read, 12 of state and 2 of weight
 * written.
 *   grads: device, dtype gdt (BF16, FP16 or FP32), layout->n_dp rows of
 *          stride ld (elements), as for zero_shard_reduce.
 *   wdt:   BF16 or FP16 (EINVAL otherwise).
 *   master, m, v: device fp32[len] at shard element shard_off.
 *   weight_full: device 16-bit buffer of layout->n_pad elements; elements
 *          [rank * shard + shard_off, ... + len) are written, nothing else.
 *   overflow: device uint32 or NULL; set to 1 when some a_j is non-finite.
 *          The update is applied regardless (a single pass cannot wait for
 *          the whole shard's verdict); use reduce + adamw with skip to gate.
 *   sumsq: device double or NULL; the sum over j of g^2 (in fp64) is ADDED
 *          to it, through workspace as for zero_shard_reduce.  It is the
 *          shard's part of the global norm of this step's gradient, known
 *          only after the update (clipping by it needs reduce + adamw_ex).
 * Errors as for zero_shard_reduce and zero_shard_adamw. */
ZERO_API zero_status zero_shard_step(const void *grads, zero_dtype gdt, int64_t ld,
                            int64_t len, float *master, float *m, float *v,
                            void *weight_full, zero_dtype wdt,
                            const zero_layout *layout, int32_t rank,
                            int64_t shard_off, const zero_adamw_hparams *hp,
                            uint32_t *overflow, double *sumsq, void *workspace,
                            int64_t workspace_bytes, void *stream);

/* ---- the fused step without a workspace ------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).
 * zero_shard_step with its sum of squares' workspace held by the library: a
 * static device array of zero_sumsq_workspace_bytes(ZERO_NOALLOC_MAX_LEN) =
 * 16,812,032 bytes, one copy on each GPU the call runs on, kept until the
 * process ends.  The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine); its results equal zero_shard_step's with a
 * workspace bit for bit, the sum of squares included.
 *   len: at most ZERO_NOALLOC_MAX_LEN when sumsq != NULL (EINVAL beyond:
 *        issue longer ranges as several calls, shard_off advancing; each
 *        adds its part to *sumsq).  Without sumsq there is no limit.
 * The array is shared by every call on one GPU: calls that sum squares and
 * may run at the same time on one GPU (other streams, other threads) race
 * on it and give wrong sums; issue them on one stream.  The first call on a
 * GPU looks up the array's device address; EDEVICE if that fails.
 * Other arguments and errors as for zero_shard_step. */
#define ZERO_NOALLOC_MAX_LEN (1LL << 29)
ZERO_API zero_status zero_shard_step_noalloc(const void *grads, zero_dtype gdt, int64_t ld,
                                             int64_t len, float *master, float *m, float *v,
                                             void *weight_full, zero_dtype wdt,
                                             const zero_layout *layout, int32_t rank,
                                             int64_t shard_off, const zero_adamw_hparams *hp,
                                             uint32_t *overflow, double *sumsq, void *stream);

/* ---- step constants in device memory (one graph for every step) ----------
 * A captured HIP graph replays the arguments it was captured with, so a
 * graph of zero_shard_step or zero_shard_adamw_ex repeats the step number
 * and learning rate of the step it captured.  The _dc variants read the
 * update's constants from device memory when their kernels run instead:
 * capture once, and before each replay write that step's constants into the
 * device buffer (zero_step_consts_make on the host, then a copy).  The step
 * number, a learning-rate schedule and every other hyperparameter may then
 * change from replay to replay -- for instance t held back after a step
 * the overflow flag skipped.  Given the constants of the same
 * hyperparameters, results are bit-identical to the hp-taking call. */

/* The update's constants as zero_adamw_hparams defines them: the ten fp32
 * values, and grad_scale itself for a dynamic loss scale (s = fl(grad_scale
 * / loss_scale) is formed from the double).  48 bytes, 8-byte aligned. */
typedef struct zero_step_consts {
    float s, b1, c1, b2, c2, bc1, bc2, lr, eps, d;
    double grad_scale;
} zero_step_consts;

/* Forms the constants of hp (host memory in and out), by the same rule as
 * the hp-taking entry points.  EINVAL: NULL hp or out, or hyperparameters
 * those entry points reject. */
ZERO_API zero_status zero_step_consts_make(const zero_adamw_hparams *hp,
                                           zero_step_consts *out);

/* zero_shard_step with its constants read from consts (device, 8-byte
 * aligned, read when the kernels run; the values are used as they are, as
 * the library cannot inspect device memory at call time).  Errors as for
 * zero_shard_step, without the hyperparameter checks; EINVAL also for a NULL
 * or unaligned consts, EALIAS when consts overlaps an output. */
ZERO_API zero_status zero_shard_step_dc(const void *grads, zero_dtype gdt, int64_t ld,
                                        int64_t len, float *master, float *m, float *v,
                                        void *weight_full, zero_dtype wdt,
                                        const zero_layout *layout, int32_t rank,
                                        int64_t shard_off, const zero_step_consts *consts,
                                        uint32_t *overflow, double *sumsq, void *workspace,
                                        int64_t workspace_bytes, void *stream);

/* A step counter on the device, so that a replayed graph needs no host
 * write at all between steps: the host fills a device table with the
 * constants of steps 1..count (zero_step_consts_make for each), and the
 * graph begins with zero_step_consts_select (consts = the row of step *t)
 * and ends with zero_step_counter_advance (t = t + 1 unless the step was
 * skipped), the step number staying put after an overflow exactly as
 * zero_shard_adamw's skip leaves the state.
 *   select:  one thread copies table[*t - 1] to *consts when 1 <= *t <=
 *            count; any other *t writes constants that are all NaN.  Every
 *            _dc entry point holds a step whose constants have a NaN s: it
 *            writes no state, weight, code or scale (a partial sum of
 *            squares of zero), and raises *overflow when given one, so a
 *            counter run past its table neither reuses an earlier step's
 *            constants nor damages the state, and advance with that flag as
 *            skip keeps the counter where it is.  consts, table: device,
 *            8-byte aligned; t: device int64, 8-byte aligned.
 *   advance: *t = *t + 1 unless skip is given and *skip != 0 (read when
 *            the kernel runs).  t: device int64, 8-byte aligned; skip:
 *            device uint32 or NULL.
 * EINVAL: a NULL required pointer, unaligned consts, table or t, count < 1.
 * EALIAS: consts overlaps the table or t; t overlaps skip. */
ZERO_API zero_status zero_step_consts_select(zero_step_consts *consts,
                                             const zero_step_consts *table, int64_t count,
                                             const int64_t *t, void *stream);
ZERO_API zero_status zero_step_counter_advance(int64_t *t, const uint32_t *skip, void *stream);

/* zero_shard_adamw_ex with its constants read from consts (as for
 * zero_shard_step_dc; with a loss scale, s = fl(consts->grad_scale /
 * scale)).  Errors as for zero_shard_adamw_ex without the hyperparameter
 * checks; EINVAL also for a NULL or unaligned consts, EALIAS when consts
 * overlaps an output. */
ZERO_API zero_status zero_shard_adamw_dc(const float *acc, float *master, float *m,
                                         float *v, void *weight_full, zero_dtype wdt,
                                         const zero_layout *layout, int32_t rank,
                                         int64_t shard_off, int64_t len,
                                         const zero_step_consts *consts,
                                         const zero_step_control *ctl, void *stream);

/* ---- moving flat ranges: flatten, unflatten, re-shard (device) -----------
 * A sharded checkpoint is tied to the layout it was written with; resuming
 * on another number of GPUs, or consolidating the shards into one set of
 * per-parameter tensors, needs each flat element moved to its new place
 * ("ZeRO Optimizer, in depth", "Checkpoints: sharded on the way in,
 * consolidated on the way out", and its list of failure modes: resuming
 * after a change of GPU count).  The same copies flatten parameter tensors
 * into a rank's shard.  All of them move flat ranges between "pieces":
 *
 * One piece of the flat vector: flat indices [flat_off, flat_off + len)
 * held contiguously at ptr (device memory, aligned to the element size).
 * The pieces passed to one call must not overlap in flat index. */
typedef struct zero_piece {
    void *ptr;
    int64_t flat_off;
    int64_t len;
} zero_piece;

/* dst[j] = flat[begin + j] for j in [0, count): the element of the piece
 * that holds flat index begin + j, or 0 where no piece holds it or the index
 * is >= n (holes and padding read as zeros).
 *   src:  host array of n_src piece descriptors (read only; their memory
 *         is read only).  elem_bytes: 2 or 4 (16-bit or fp32 data; the copy
 *         is bitwise).  dst: device, count elements.
 * EINVAL: elem_bytes not 2 or 4; n, begin, count or a piece's flat_off or
 * len negative; count > 2^38; an index range overflowing int64; a NULL
 * pointer where len or count > 0; a pointer not aligned to elem_bytes;
 * pieces that overlap in flat index.  EALIAS: dst overlaps a piece's
 * memory.  count == 0 is a no-op. */
ZERO_API zero_status zero_flat_gather(const zero_piece *src, int32_t n_src,
                                      int64_t n, int32_t elem_bytes,
                                      int64_t begin, int64_t count, void *dst,
                                      void *stream);

/* The inverse: src[j] holds flat index begin + j for j in [0, count); every
 * piece of dst receives the elements of that range it holds, and nothing
 * else of any piece is written.
 * EINVAL as for zero_flat_gather.  EALIAS: two pieces overlap in memory, or
 * a piece overlaps src. */
ZERO_API zero_status zero_flat_scatter(const void *src, int64_t begin,
                                       int64_t count, const zero_piece *dst,
                                       int32_t n_dst, int32_t elem_bytes,
                                       void *stream);

/* Re-shard: old rank r's shard of src_shard elements is at src_shards[r]
 * (host array of n_src device pointers, flat indices [r * src_shard,
 * (r + 1) * src_shard)); dst (device, dst_shard elements) receives new rank
 * dst_rank's shard, flat indices [dst_rank * dst_shard, ... + dst_shard),
 * with zeros from flat index n on.  Consolidation is dst_rank = 0 with
 * dst_shard >= n.  Equal to zero_flat_gather over those pieces.
 * EINVAL: n_src < 1, src_shard < 0, n outside [0, n_src * src_shard],
 * dst_rank < 0, dst_shard < 0, and as for zero_flat_gather.  EALIAS: dst
 * overlaps an old shard. */
ZERO_API zero_status zero_reshard(const void *const *src_shards, int32_t n_src,
                                  int64_t src_shard, int64_t n,
                                  int32_t elem_bytes, int32_t dst_rank,
                                  int64_t dst_shard, void *dst, void *stream);

/* ---- 8-bit blockwise quantization for communication (ZeRO++) ------------
 * ZeRO++ quantizes the weight all-gather to 8 bits and the gradients of the
 * reduce-scatter ("ZeRO and FSDP", FSDP section, fewer bytes on the wire;
 * "ZeRO Optimizer, in depth", "Offload and ZeRO++").  The pages define no
 * quantizer; this library uses the plain symmetric blockwise one:
 *   a vector of len elements is cut into blocks of ZERO_Q8_BLOCK (the last
 *   one may be short); block i has one fp32 scale s_i = absmax_i / 127
 *   (absmax NaN if the block holds a NaN) and codes q_j = rint(x_j / s_i):
 *   the quotient correctly rounded to fp32, then rounded to an integer with
 *   ties to even, clamped to [-127, 127] (q_j = 0 when s_i is 0, Inf or
 *   NaN, so a non-finite block dequantizes to NaN, and one whose absmax / 127
 *   rounds to zero to zeros); the value is q_j * s_i.
 * Codes: int8[len]; scales: float[ceil(len / ZERO_Q8_BLOCK)]. */
#define ZERO_Q8_BLOCK 256

/* Quantize x (device, xdt = BF16, FP16 or FP32, len elements) into q and
 * scales (device).  Any alignment (16-byte fp32 / 8-byte 16-bit input and
 * 4-byte codes take the vector path).
 * EINVAL: bad xdt, len < 0 or > 2^38, NULL pointers with len > 0.
 * EALIAS: any two of x, q, scales overlap. */
ZERO_API zero_status zero_q8_quantize(const void *x, zero_dtype xdt, int64_t len, int8_t *q,
                                      float *scales, void *stream);

/* y[j] = q[j] * scales[j / ZERO_Q8_BLOCK] in fp32, stored as ydt (BF16 and
 * FP16 rounded to nearest even).  Any alignment (16-byte y with 4-byte
 * codes for FP32, 16-byte y with 8-byte codes for 16-bit values take the
 * vector path).  Errors as for zero_q8_quantize. */
ZERO_API zero_status zero_q8_dequantize(const int8_t *q, const float *scales, int64_t len,
                                        void *y, zero_dtype ydt, void *stream);

/* Fused step with 8-bit communication on both sides: the n_dp ranks'
 * contributions arrive as quantized rows (what each sender puts on the wire
 * for this shard range), and the updated master leaves quantized (the
 * all-gather's 8-bit payload).  Per element j of the range:
 *   a_j = sum over k of q_k[j] * s_k[j / B] (each product rounded to fp32,
 *         summed left to right), g = a_j * s, AdamW as zero_shard_step;
 * then the new master of each block of B = ZERO_Q8_BLOCK elements of the
 * range is quantized into wq_full / wscales_full.
 *   gq:  device int8, layout->n_dp rows of stride ld (elements); gscales:
 *        device fp32, the rows' block scales, row k at gscales + k * sld,
 *        entry i for the range's block i.
 *   master, m, v: device fp32[len] at shard element shard_off.
 *   wq_full: device int8[n_pad]; wscales_full: device fp32[n_pad / B];
 *        elements [rank * shard + shard_off, ... + len) and their block
 *        scales are written, nothing else.
 *   overflow, sumsq, workspace: as zero_shard_step (the update is applied
 *        regardless).
 * Requirements (EINVAL otherwise): layout->shard and shard_off multiples of
 * B; gq and wq_full 4-byte aligned, ld a multiple of 4 when n_dp > 1,
 * sld >= ceil(len / B) when n_dp > 1; master, m, v 16-byte aligned.
 * Errors otherwise as for zero_shard_step; EALIAS covers the scale rows and
 * slots too.  Bytes per element: n_dp (1 + 4/B) + 12 read, 12 + 1 + 4/B
 * written. */
ZERO_API zero_status zero_shard_step_q8(const int8_t *gq, const float *gscales, int64_t ld,
                                        int64_t sld, int64_t len, float *master, float *m,
                                        float *v, int8_t *wq_full, float *wscales_full,
                                        const zero_layout *layout, int32_t rank,
                                        int64_t shard_off, const zero_adamw_hparams *hp,
                                        uint32_t *overflow, double *sumsq, void *workspace,
                                        int64_t workspace_bytes, void *stream);

/* zero_shard_step_q8 with its constants read from consts (device, 8-byte
 * aligned; see zero_shard_step_dc).  Errors as for zero_shard_step_q8
 * without the hyperparameter checks; EINVAL also for a NULL or unaligned
 * consts, EALIAS when consts overlaps an output. */
ZERO_API zero_status zero_shard_step_q8_dc(const int8_t *gq, const float *gscales, int64_t ld,
                                           int64_t sld, int64_t len, float *master, float *m,
                                           float *v, int8_t *wq_full, float *wscales_full,
                                           const zero_layout *layout, int32_t rank,
                                           int64_t shard_off, const zero_step_consts *consts,
                                           uint32_t *overflow, double *sumsq, void *workspace,
                                           int64_t workspace_bytes, void *stream);

/* ---- accounting (host only) ----------------------------------------------
 * Model-state bytes per GPU at ZeRO stage 0..3 for n parameters on n_dp
 * ranks with 2-byte weights and gradients and k bytes of optimizer state
 * per parameter ("ZeRO and FSDP", "Memory per GPU": 16N, 4N + 12N/n_dp,
 * 2N + 14N/n_dp, 16N/n_dp for k = 12).  EINVAL: out NULL, stage outside
 * 0..3, n < 0, n_dp < 1, k < 0. */
ZERO_API zero_status zero_model_state_bytes(double n, double n_dp, int32_t stage,
                                   double k, double *out);

/* Bytes each GPU sends per optimizer step with ring collectives ("ZeRO and
 * FSDP", "Communication volume"): a reduce-scatter or all-gather of N
 * elements sends (n_dp - 1) / n_dp * N per GPU, an all-reduce twice that.
 * Stage 0 all-reduces gradients; stages 1 and 2 reduce-scatter gradients
 * and all-gather weights; stage 3 all-gathers weights twice and
 * reduce-scatters gradients.  EINVAL as above, or element sizes <= 0. */
ZERO_API zero_status zero_comm_bytes(double n, double n_dp, int32_t stage,
                            double param_bytes, double grad_bytes,
                            double *out);

#ifdef __cplusplus
}
#endif
#endif /* ZERO_SHARD_H */
