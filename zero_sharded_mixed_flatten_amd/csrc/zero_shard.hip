// zero_shard.hip -- gfx950 kernels and device entry points of libzero_shard.
//
// One data-parallel rank's sharded optimizer step, as "ZeRO and FSDP" (Zero
// to Frontier 10.3) lays it out under "The idea, one stage at a time" and "A
// sharded Adam step": the ranks' 16-bit gradient rows for the owned shard
// are averaged (the reduce-scatter's arithmetic), AdamW updates the fp32
// master and moments of the shard, and the new master is cast to 16 bits
// into the shard's slot of the full weight buffer (the all-gather's
// destination).
//
// Nothing here is a contraction: the work is a stream over HBM of
// 2 * n_dp + 26 bytes per element (fused step), so the kernels are built for
// bandwidth, shaped by measurement on MI355X:
//  - Each lane owns 4 consecutive elements (a "quad").  A wave's load of a
//    gradient row is then 8 bytes per lane and one contiguous 512-byte span,
//    its load or store of an fp32 array 16 bytes per lane and one contiguous
//    1 KiB span: every memory instruction of a wave touches whole cache
//    lines, and all of a quad's loads are issued before its first add.
//    (8 elements per lane -- 16-byte gradient loads but half-used 2 KiB
//    spans for the fp32 arrays -- measured slower.)
//  - The grid is one thread per quad, with no loop: waves that finish free
//    their slot for the next workgroup, so the set of addresses in flight
//    stays a compact, moving window (persistent grid-stride variants
//    measured 10-15% slower, and even a loop that runs once costs ~1%).
//  - Fewer waves per CU than the hardware allows: with 8 + 7 streams in
//    flight the HBM controllers do better with about 8 waves per CU than
//    with 32, so each launch requests enough (otherwise unused) LDS to cap
//    the workgroups resident on a CU (per-kernel caps below).
//  - Non-temporal loads and stores: nothing is re-read, nothing should stay
//    in L2 or the Infinity Cache.
// LDS and wave reductions appear only in the optional overflow flag and sum
// of squares.
//
// Arithmetic is IEEE binary32, round-to-nearest-even, in a fixed order: the
// build uses -ffp-contract=off (no fused multiply-add), HIP's correctly
// rounded fp32 division and square root, and keeps denormals.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "host_common.h"
#include "step_common.h"
#include "zero_shard.h"

namespace {

using namespace zero_host;
using namespace zero_step;

constexpr int kBlock = 256;     // threads per workgroup of the element kernels
constexpr int kRowBatch = 8;    // rows loaded together when n_dp is not specialised
// Residency caps in waves per CU, measured per kernel at the workloads'
// sizes with one-wave workgroups (a finished wave's slot is refilled at
// once; with four-wave workgroups a slot frees only when all four are done,
// which cost 8-10%).  The variants that also sum squares take the same
// one-wave shape and store one partial per wave (flags_epilogue).
// Fused step: 10 waves with 1 row (56 B per lane in flight), 7 with 8 rows
// (112 B), and with 64 rows the 152 VGPRs per lane already allow only 12.
// With 8 fp32 rows (176 B per lane in flight) 5 waves per CU measured best
// (79.6 % of 8 TB/s against 78.7 % at 7 and 76.9 % uncapped, random data).
// The summing variants carry a double accumulation per element and store a
// partial per wave; swept separately (7B shard; GPT-2-XL list for 1 row):
// 1 row 10 -> 79.2 %, 12 -> 82.3 %, 14 -> 80.9 %; 8 rows 7 -> 77.2 %,
// 8 -> 80.3 %, 9 -> 81.4-81.7 %, 10 -> 80.8 %; 64 rows 12 -> 72.6 %, 16 -> 72.4 %; 8 fp32
// rows 5 -> 78.6 %, 6 -> 80.9 %, 7 -> 80.9 %; the accumulating fp16 reduce
// 10 -> 82.2 %, 12 -> 83.9 %, 16 -> 80.9 %.
constexpr int step_waves_per_cu(int gdt, int ndp, bool ssq = false) {
    if (gdt == ZERO_FP32) return ndp == 1 ? 10 : ssq ? 6 : 5;
    if (ssq) return ndp == 1 || ndp == 64 ? 12 : 9;
    return ndp == 1 ? 10 : ndp == 64 ? 12 : 7;
}
constexpr int kReduceWavesPerCU = 10;
constexpr int kReduceSsqWavesPerCU = 12;
constexpr int kAdamwWavesPerCU = 10;
// Device-side step controls (zero_step_control with the static part of the
// gradient scale alongside).
struct Control {
    const double *sumsq;
    double max_norm;
    const zero_loss_scale *loss_scale;
    double grad_scale;
};

template <int GDT>
__device__ __forceinline__ void add_row(float a[kQuad], typename GradT<GDT>::quad x) {
    float t[kQuad];
    widen_quad<GDT>(t, x);
#pragma unroll
    for (int e = 0; e < kQuad; ++e) a[e] = a[e] + t[e];
}

// Rows of one quad.  For NDP > 0 (row count fixed at compile time) the
// loads and the sum are separate steps so that a kernel can issue every
// load it needs -- rows and state -- before the first add (see
// loads_issued()).  NDP == 0 reads the count at run time and fetches
// kRowBatch rows at a time.
template <int GDT, int NDP>
struct Rows {
    typename GradT<GDT>::quad x[NDP > 0 ? NDP : kRowBatch];
};

template <int GDT, int NDP>
__device__ __forceinline__ void load_rows(Rows<GDT, NDP> &r,
                                          const typename GradT<GDT>::elem *__restrict__ p,
                                          int64_t ld) {
    if constexpr (NDP > 0) {
#pragma unroll
        for (int k = 0; k < NDP; ++k) r.x[k] = load_quad<GDT>(p + static_cast<int64_t>(k) * ld);
    }
}

// a[e] = G_0[e] + G_1[e] + ..., left to right in fp32
template <int GDT, int NDP>
__device__ __forceinline__ void sum_rows(float a[kQuad], Rows<GDT, NDP> &r,
                                         const typename GradT<GDT>::elem *__restrict__ p,
                                         int64_t ld, int n) {
    if constexpr (NDP > 0) {
        widen_quad<GDT>(a, r.x[0]);
#pragma unroll
        for (int k = 1; k < NDP; ++k) add_row<GDT>(a, r.x[k]);
    } else {
        for (int k = 0; k < n; k += kRowBatch) {
#pragma unroll
            for (int b = 0; b < kRowBatch; ++b)
                if (k + b < n) r.x[b] = load_quad<GDT>(p + static_cast<int64_t>(k + b) * ld);
            if (k == 0) widen_quad<GDT>(a, r.x[0]);
#pragma unroll
            for (int b = 0; b < kRowBatch; ++b)
                if (k + b < n && k + b > 0) add_row<GDT>(a, r.x[b]);
        }
    }
}

// ---------------------------------------------------------------------------
// fused step: reduce -> scale -> AdamW -> cast, one pass

// One quad of the fused step after its loads: reduce the rows, AdamW, store.
template <int GDT, int WDT, int NDP, bool OVF, bool SSQ>
__device__ __forceinline__ void step_quad_finish(Rows<GDT, NDP> &rows, f32x4 w4, f32x4 m4,
                                                 f32x4 v4,
                                                 const typename GradT<GDT>::elem *__restrict__ g,
                                                 int64_t ld, int n_dp, int64_t e0,
                                                 float *__restrict__ W, float *__restrict__ M,
                                                 float *__restrict__ V,
                                                 uint16_t *__restrict__ out, const Consts &c,
                                                 bool &bad, double &ss) {
    float a[kQuad];
    sum_rows<GDT, NDP>(a, rows, g, ld, n_dp);
    float w[kQuad] = {w4[0], w4[1], w4[2], w4[3]};
    float m[kQuad] = {m4[0], m4[1], m4[2], m4[3]};
    float v[kQuad] = {v4[0], v4[1], v4[2], v4[3]};
#pragma unroll
    for (int e = 0; e < kQuad; ++e) {
        if constexpr (OVF) bad |= !__builtin_isfinite(a[e]);
        const float gr = a[e] * c.s;
        if constexpr (SSQ) ss += static_cast<double>(gr) * static_cast<double>(gr);
        adamw_element(gr, w[e], m[e], v[e], c);
    }
    store16(W + e0, f32x4{w[0], w[1], w[2], w[3]});
    store16(M + e0, f32x4{m[0], m[1], m[2], m[3]});
    store16(V + e0, f32x4{v[0], v[1], v[2], v[3]});
    store8(out + e0, u32x2{narrow2<WDT>(w[0], w[1]), narrow2<WDT>(w[2], w[3])});
}

// One quad per lane, one-wave workgroups (TPB == kWave): the rows and the
// state of the quad are all loaded before the first add.  With SSQ the
// wave's partial sum of squares goes to part[blockIdx.x].  With DC the
// constants come from dc (device memory) instead of c.
template <int TPB, int GDT, int WDT, int NDP, bool OVF, bool SSQ, bool DC>
__global__ void __launch_bounds__(TPB)
step_quad_kernel(const typename GradT<GDT>::elem *__restrict__ grads, int64_t ld, int n_dp,
                 int64_t nquad,
                 float *__restrict__ W, float *__restrict__ M, float *__restrict__ V,
                 uint16_t *__restrict__ out, Consts c, uint32_t *__restrict__ ovf,
                 double *__restrict__ part, const zero_step_consts *__restrict__ dc) {
    bool held = false;
    if constexpr (DC) {
        c = consts_of(*dc);
        held = step_held(c);
    }
    bool bad = held;
    double ss = 0.0;
    const int64_t q = static_cast<int64_t>(blockIdx.x) * TPB + threadIdx.x;
    if (q < nquad && !held) {
        const int64_t e0 = q * kQuad;
        Rows<GDT, NDP> rows;
        load_rows<GDT, NDP>(rows, grads + e0, ld);
        const f32x4 w4 = load16(W + e0), m4 = load16(M + e0), v4 = load16(V + e0);
        loads_issued();
        step_quad_finish<GDT, WDT, NDP, OVF, SSQ>(rows, w4, m4, v4, grads + e0, ld, n_dp, e0, W,
                                                  M, V, out, c, bad, ss);
    }
    flags_epilogue<TPB, OVF, SSQ>(bad, ss, ovf, part);
}

// element-per-thread variant for unaligned buffers and ragged tails
template <int GDT, int WDT, bool OVF, bool SSQ, bool DC>
__global__ void __launch_bounds__(kBlock)
step_scalar_kernel(const typename GradT<GDT>::elem *__restrict__ grads, int64_t ld, int n_dp,
                   int64_t len,
                   float *__restrict__ W, float *__restrict__ M, float *__restrict__ V,
                   uint16_t *__restrict__ out, Consts c, uint32_t *__restrict__ ovf,
                   double *__restrict__ part, const zero_step_consts *__restrict__ dc) {
    bool held = false;
    if constexpr (DC) {
        c = consts_of(*dc);
        held = step_held(c);
    }
    bool bad = held;
    double ss = 0.0;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    for (int64_t j = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; j < len && !held;
         j += stride) {
        float a = widen1<GDT>(grads[j]);
        for (int k = 1; k < n_dp; ++k) a = a + widen1<GDT>(grads[static_cast<int64_t>(k) * ld + j]);
        if constexpr (OVF) bad |= !__builtin_isfinite(a);
        const float g = a * c.s;
        if constexpr (SSQ) ss += static_cast<double>(g) * static_cast<double>(g);
        float w = W[j], m = M[j], v = V[j];
        adamw_element(g, w, m, v, c);
        W[j] = w;
        M[j] = m;
        V[j] = v;
        out[j] = narrow1<WDT>(w);
    }
    flags_epilogue<kBlock, OVF, SSQ>(bad, ss, ovf, part);
}

// ---------------------------------------------------------------------------
// reduce into an fp32 buffer (optionally accumulating across micro-batches)

// One quad of the reduce after its loads: sum, accumulate, flags, store.
template <int GDT, int NDP, bool ACC, bool OVF, bool SSQ>
__device__ __forceinline__ void reduce_quad_finish(Rows<GDT, NDP> &rows, f32x4 prev,
                                                   const typename GradT<GDT>::elem *__restrict__ g,
                                                   int64_t ld, int n, int64_t e0,
                                                   float *__restrict__ acc, bool &bad,
                                                   double &ss) {
    float a[kQuad];
    sum_rows<GDT, NDP>(a, rows, g, ld, n);
    if constexpr (ACC) {
#pragma unroll
        for (int e = 0; e < kQuad; ++e) a[e] = prev[e] + a[e];
    }
#pragma unroll
    for (int e = 0; e < kQuad; ++e) {
        if constexpr (OVF) bad |= !__builtin_isfinite(a[e]);
        if constexpr (SSQ) ss += static_cast<double>(a[e]) * static_cast<double>(a[e]);
    }
    store16(acc + e0, f32x4{a[0], a[1], a[2], a[3]});
}

template <int TPB, int GDT, int NDP, bool ACC, bool OVF, bool SSQ>
__global__ void __launch_bounds__(TPB)
reduce_quad_kernel(const typename GradT<GDT>::elem *__restrict__ grads, int64_t ld, int n,
                   int64_t nquad,
                   float *__restrict__ acc, uint32_t *__restrict__ ovf,
                   double *__restrict__ part) {
    bool bad = false;
    double ss = 0.0;
    const int64_t q = static_cast<int64_t>(blockIdx.x) * TPB + threadIdx.x;
    if (q < nquad) {
        const int64_t e0 = q * kQuad;
        Rows<GDT, NDP> rows;
        load_rows<GDT, NDP>(rows, grads + e0, ld);
        f32x4 prev = {};
        if constexpr (ACC) prev = load16(acc + e0);
        loads_issued();
        reduce_quad_finish<GDT, NDP, ACC, OVF, SSQ>(rows, prev, grads + e0, ld, n, e0, acc, bad,
                                                    ss);
    }
    flags_epilogue<TPB, OVF, SSQ>(bad, ss, ovf, part);
}

template <int GDT, bool ACC, bool OVF, bool SSQ>
__global__ void __launch_bounds__(kBlock)
reduce_scalar_kernel(const typename GradT<GDT>::elem *__restrict__ grads, int64_t ld, int n,
                     int64_t len,
                     float *__restrict__ acc, uint32_t *__restrict__ ovf,
                     double *__restrict__ part) {
    bool bad = false;
    double ss = 0.0;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    for (int64_t j = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; j < len;
         j += stride) {
        float a = widen1<GDT>(grads[j]);
        for (int k = 1; k < n; ++k) a = a + widen1<GDT>(grads[static_cast<int64_t>(k) * ld + j]);
        if constexpr (ACC) a = acc[j] + a;
        if constexpr (OVF) bad |= !__builtin_isfinite(a);
        if constexpr (SSQ) ss += static_cast<double>(a) * static_cast<double>(a);
        acc[j] = a;
    }
    flags_epilogue<kBlock, OVF, SSQ>(bad, ss, ovf, part);
}

// ---------------------------------------------------------------------------
// AdamW from an fp32 gradient buffer, gated by an optional device flag

// The scale s and the clipping coefficient of a controlled step, from the
// device-resident loss scale and whole-model sum of squares (every thread
// computes the same value; double arithmetic, rounded once to fp32).
__device__ __forceinline__ float resolve_controls(const Control &k, Consts &c) {
    if (k.loss_scale) c.s = static_cast<float>(k.grad_scale / static_cast<double>(k.loss_scale->scale));
    float clip = 1.0f;
    if (k.sumsq && k.max_norm > 0.0) {
        const double norm = sqrt(*k.sumsq) * static_cast<double>(c.s);
        const double cc = k.max_norm / (norm + 1e-6);
        if (cc < 1.0) clip = static_cast<float>(cc);
    }
    return clip;
}

template <int TPB, int WDT, bool SKIP, bool EXT, bool DC>
__global__ void __launch_bounds__(TPB)
adamw_quad_kernel(const float *__restrict__ acc, float *__restrict__ W, float *__restrict__ M,
                  float *__restrict__ V, uint16_t *__restrict__ out, int64_t nquad, Consts c,
                  const uint32_t *__restrict__ skip, Control ctl,
                  const zero_step_consts *__restrict__ dc) {
    if constexpr (SKIP) {
        if (*skip != 0u) return;
    }
    if constexpr (DC) {
        c = consts_of(*dc);
        if (step_held(c)) return;
        ctl.grad_scale = dc->grad_scale;
    }
    float clip = 1.0f;
    if constexpr (EXT) clip = resolve_controls(ctl, c);
    const int64_t q = static_cast<int64_t>(blockIdx.x) * TPB + threadIdx.x;
    if (q < nquad) {
        const int64_t e0 = q * kQuad;
        const f32x4 g4 = load16(acc + e0);
        const f32x4 w4 = load16(W + e0), m4 = load16(M + e0), v4 = load16(V + e0);
        loads_issued();
        float w[kQuad] = {w4[0], w4[1], w4[2], w4[3]};
        float m[kQuad] = {m4[0], m4[1], m4[2], m4[3]};
        float v[kQuad] = {v4[0], v4[1], v4[2], v4[3]};
#pragma unroll
        for (int e = 0; e < kQuad; ++e) {
            float g = g4[e] * c.s;
            if constexpr (EXT) {
                if (clip < 1.0f) g = g * clip;
            }
            adamw_element(g, w[e], m[e], v[e], c);
        }
        store16(W + e0, f32x4{w[0], w[1], w[2], w[3]});
        store16(M + e0, f32x4{m[0], m[1], m[2], m[3]});
        store16(V + e0, f32x4{v[0], v[1], v[2], v[3]});
        store8(out + e0, u32x2{narrow2<WDT>(w[0], w[1]), narrow2<WDT>(w[2], w[3])});
    }
}

template <int WDT, bool SKIP, bool EXT, bool DC>
__global__ void __launch_bounds__(kBlock)
adamw_scalar_kernel(const float *__restrict__ acc, float *__restrict__ W, float *__restrict__ M,
                    float *__restrict__ V, uint16_t *__restrict__ out, int64_t len, Consts c,
                    const uint32_t *__restrict__ skip, Control ctl,
                    const zero_step_consts *__restrict__ dc) {
    if constexpr (SKIP) {
        if (*skip != 0u) return;
    }
    if constexpr (DC) {
        c = consts_of(*dc);
        if (step_held(c)) return;
        ctl.grad_scale = dc->grad_scale;
    }
    float clip = 1.0f;
    if constexpr (EXT) clip = resolve_controls(ctl, c);
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    for (int64_t j = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; j < len;
         j += stride) {
        float w = W[j], m = M[j], v = V[j];
        float g = acc[j] * c.s;
        if constexpr (EXT) {
            if (clip < 1.0f) g = g * clip;
        }
        adamw_element(g, w, m, v, c);
        W[j] = w;
        M[j] = m;
        V[j] = v;
        out[j] = narrow1<WDT>(w);
    }
}

// The constants of step *t from a table of steps 1..count (one thread);
// NaN constants for a step outside the table, which every device-constant
// kernel holds (step_held): it writes nothing.
__global__ void step_consts_select_kernel(zero_step_consts *__restrict__ out,
                                          const zero_step_consts *__restrict__ table,
                                          int64_t count, const int64_t *__restrict__ t) {
    const int64_t k = *t;
    if (k >= 1 && k <= count) {
        *out = table[k - 1];
    } else {
        const float nan = __builtin_nanf("");
        *out = zero_step_consts{nan, nan, nan, nan, nan, nan, nan, nan, nan, nan,
                                __builtin_nan("")};
    }
}

// t = t + 1 unless the step was skipped (one thread)
__global__ void step_counter_advance_kernel(int64_t *__restrict__ t,
                                            const uint32_t *__restrict__ skip) {
    if (skip == nullptr || *skip == 0u) *t = *t + 1;
}

// One step of the dynamic loss scale (one thread).
__global__ void loss_scale_kernel(zero_loss_scale *__restrict__ st,
                                  const uint32_t *__restrict__ overflow, double growth,
                                  double backoff, int32_t interval) {
    if (blockIdx.x != 0 || threadIdx.x != 0) return;
    float scale = st->scale;
    int32_t good = st->good_steps;
    if (*overflow != 0u) {
        scale = static_cast<float>(static_cast<double>(scale) * backoff);
        good = 0;
    } else {
        good += 1;
        if (good >= interval) {
            const float grown = static_cast<float>(static_cast<double>(scale) * growth);
            if (!__builtin_isinf(grown)) scale = grown;  // never grows to infinity
            good = 0;
        }
    }
    st->scale = scale;
    st->good_steps = good;
}

// ---------------------------------------------------------------------------
// host side: validation, constants, dispatch

template <int V>
using IntC = std::integral_constant<int, V>;
template <bool V>
using BoolC = std::integral_constant<bool, V>;

template <typename F>
void with_dtype(int dt, F &&f) {
    if (dt == ZERO_BF16) f(IntC<ZERO_BF16>{});
    else f(IntC<ZERO_FP16>{});
}

// gradient row formats: the weight formats plus fp32
template <typename F>
void with_gdtype(int dt, F &&f) {
    if (dt == ZERO_FP32) f(IntC<ZERO_FP32>{});
    else with_dtype(dt, f);
}

template <typename F>
void with_bool(bool b, F &&f) {
    if (b) f(BoolC<true>{});
    else f(BoolC<false>{});
}

// row counts with a compiled specialisation (the configurations' 1, 8 and
// 64 ranks); others take the batched loop.  64 fp32 rows would hold 256
// VGPRs per lane and take the batched loop too.
template <int GDT, typename F>
void with_ndp(int n, F &&f) {
    switch (n) {
    case 1: f(IntC<1>{}); break;
    case 8: f(IntC<8>{}); break;
    case 64:
        if constexpr (GDT == ZERO_FP32) f(IntC<0>{});
        else f(IntC<64>{});
        break;
    default: f(IntC<0>{}); break;
    }
}

bool gdtype_ok(int dt) { return dtype_ok(dt) || dt == ZERO_FP32; }
int64_t gdtype_bytes(int dt) { return dt == ZERO_FP32 ? 4 : 2; }

// true when any two outputs overlap, or an output overlaps an input or a
// gradient row (rows of elem bytes per element, ld elements apart)
bool any_alias(const Span *outs, int n_out, const void *rows, int n_rows, int64_t ld,
               int64_t len, int64_t elem, const Span *ins = nullptr, int n_in = 0) {
    for (int i = 0; i < n_out; ++i) {
        for (int j = i + 1; j < n_out; ++j)
            if (overlap(outs[i], outs[j])) return true;
        for (int j = 0; j < n_in; ++j)
            if (overlap(outs[i], ins[j])) return true;
        for (int k = 0; k < n_rows; ++k) {
            const void *row = static_cast<const unsigned char *>(rows) +
                              static_cast<int64_t>(k) * ld * elem;
            if (overlap(outs[i], span_of(row, len, elem))) return true;
        }
    }
    return false;
}

// the vector path's alignment of a gradient row: one quad per lane
bool rows_vec_ok(const void *g, int gdt, int n_rows, int64_t ld) {
    const bool al = gdt == ZERO_FP32 ? aligned16(g) : aligned8(g);
    return al && (n_rows == 1 || ld % kQuad == 0);
}

// one thread per item of a one-shot launch (at most kLaunchElems items)
unsigned grid_for(int64_t items, int tpb = kBlock) {
    const int64_t b = (items + tpb - 1) / tpb;
    return static_cast<unsigned>(b < 1 ? 1 : b);
}

// grid of an element-wise (grid-stride) kernel: one thread per element up
// to kMaxStrideBlocks workgroups, or at most kSsqScalarBlocks when it ends
// in a sum's atomic
unsigned scalar_grid(int64_t items, bool ssq) {
    const int64_t b = (items + kBlock - 1) / kBlock;
    const int64_t cap = ssq ? kSsqScalarBlocks : kMaxStrideBlocks;
    return static_cast<unsigned>(b < 1 ? 1 : (b > cap ? cap : b));
}

// The one-shot quad kernels run over [0, nquad) in launches of at most
// kLaunchElems elements; f(first quad, quads) issues one.
template <typename F>
void for_launches(int64_t nquad, F &&f) {
    constexpr int64_t per = kLaunchElems / kQuad;
    for (int64_t q0 = 0; q0 < nquad; q0 += per) f(q0, nquad - q0 < per ? nquad - q0 : per);
}

// the workspace of a call that sums squares: given, 8-byte aligned, large enough
bool workspace_ok(const void *ws, int64_t bytes, int64_t len) {
    return ws && aligned8(ws) && bytes >= zero_sumsq_workspace_bytes(len);
}

// partials the quad launches and the element kernel of one call store:
// one per one-wave workgroup of quads, one per element-kernel workgroup
int64_t ssq_partial_count(int64_t nquad, int64_t rest) {
    return (nquad + kWave - 1) / kWave + (rest > 0 ? scalar_grid(rest, true) : 0);
}

// Stage two of the sum: workgroup j adds partials [j * chunk, (j + 1) * chunk)
// -- each thread a strided subset in index order, then a halving tree in
// LDS -- into st2[j].  Fixed by count alone, so a call's sum is the same
// bits every time.
__global__ void __launch_bounds__(kBlock)
ssq_stage2_kernel(const double *__restrict__ part, int64_t count, int64_t chunk,
                  double *__restrict__ st2) {
    __shared__ double s[kBlock];
    const int64_t lo = static_cast<int64_t>(blockIdx.x) * chunk;
    const int64_t hi = lo + chunk < count ? lo + chunk : count;
    double t = 0.0;
    for (int64_t i = lo + threadIdx.x; i < hi; i += kBlock) t += part[i];
    s[threadIdx.x] = t;
    __syncthreads();
#pragma unroll
    for (int w = kBlock / 2; w > 0; w >>= 1) {
        if (static_cast<int>(threadIdx.x) < w) s[threadIdx.x] += s[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) st2[blockIdx.x] = s[0];
}

// Stage three: the kSsqStage2 sums by a halving tree, added to the caller's
// scalar with one atomic (calls on other streams may add to it as well).
__global__ void __launch_bounds__(kSsqStage2)
ssq_stage3_kernel(const double *__restrict__ st2, double *__restrict__ sumsq) {
    __shared__ double s[kSsqStage2];
    s[threadIdx.x] = st2[threadIdx.x];
    __syncthreads();
#pragma unroll
    for (int w = kSsqStage2 / 2; w > 0; w >>= 1) {
        if (static_cast<int>(threadIdx.x) < w) s[threadIdx.x] += s[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) unsafeAtomicAdd(sumsq, s[0]);
}

}  // namespace

namespace zero_step {

zero_status finish_sumsq(void *workspace, int64_t count, double *sumsq, hipStream_t st) {
    static_assert(kSsqStage2 == kBlock, "stage two's sums are stage three's threads");
    double *st2 = static_cast<double *>(workspace);
    const int64_t chunk = (count + kSsqStage2 - 1) / kSsqStage2;
    ssq_stage2_kernel<<<kSsqStage2, kBlock, 0, st>>>(ssq_partials(workspace), count,
                                                     chunk > 0 ? chunk : 1, st2);
    ssq_stage3_kernel<<<1, kSsqStage2, 0, st>>>(st2, sumsq);
    return launch_status();
}

}  // namespace zero_step

extern "C" int64_t zero_sumsq_workspace_bytes(int64_t len) {
    if (len < 0 || len > kMaxLen) return -1;
    return static_cast<int64_t>(sizeof(double)) * (kSsqStage2 + ssq_partials_cap(len));
}

// ===========================================================================

extern "C" zero_status zero_shard_reduce(const void *grads, zero_dtype gdt, int32_t n_contrib,
                                         int64_t ld, int64_t len, float *acc,
                                         int32_t accumulate, uint32_t *overflow,
                                         double *sumsq, void *workspace,
                                         int64_t workspace_bytes, void *stream) {
    if (!gdtype_ok(gdt) || !rows_ok(n_contrib, ld, len) || len > kMaxLen) return ZERO_EINVAL;
    if (len == 0) return ZERO_OK;
    if (!grads || !acc) return ZERO_EINVAL;
    if (sumsq && !workspace_ok(workspace, workspace_bytes, len)) return ZERO_EINVAL;
    Span outs[4];
    int n_out = 0;
    outs[n_out++] = span_of(acc, len, 4);
    if (overflow) outs[n_out++] = span_of(overflow, 1, 4);
    if (sumsq) outs[n_out++] = span_of(sumsq, 1, 8);
    if (sumsq) outs[n_out++] = span_of(workspace, workspace_bytes, 1);
    if (any_alias(outs, n_out, grads, n_contrib, ld, len, gdtype_bytes(gdt))) return ZERO_EALIAS;

    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool vec = rows_vec_ok(grads, gdt, n_contrib, ld) && aligned16(acc);
    const int64_t nquad = vec ? len / kQuad : 0;
    const int64_t done = nquad * kQuad;
    double *part = sumsq ? ssq_partials(workspace) : nullptr;
    const int64_t n_qpart = (nquad + kWave - 1) / kWave;
    with_gdtype(gdt, [&](auto GD) {
        using E = typename GradT<GD.value>::elem;
        const E *g = static_cast<const E *>(grads);
        with_bool(accumulate != 0, [&](auto AC) {
            with_bool(overflow != nullptr, [&](auto OV) {
                with_bool(sumsq != nullptr, [&](auto SS) {
                    if (nquad > 0) {
                        const size_t lds = residency_lds_bytes(
                            SS.value ? kReduceSsqWavesPerCU : kReduceWavesPerCU, kWave);
                        with_ndp<GD.value>(n_contrib, [&](auto ND) {
                            for_launches(nquad, [&](int64_t q0, int64_t nq) {
                                const int64_t o = q0 * kQuad;
                                reduce_quad_kernel<kWave, GD.value, ND.value, AC.value, OV.value,
                                                   SS.value>
                                    <<<grid_for(nq, kWave), kWave, lds, st>>>(
                                        g + o, ld, n_contrib, nq, acc + o, overflow,
                                        SS.value ? part + q0 / kWave : nullptr);
                            });
                        });
                    }
                    if (len > done) {
                        reduce_scalar_kernel<GD.value, AC.value, OV.value, SS.value>
                            <<<scalar_grid(len - done, SS.value), kBlock, 0, st>>>(
                                g + done, ld, n_contrib, len - done, acc + done, overflow,
                                SS.value ? part + n_qpart : nullptr);
                    }
                });
            });
        });
    });
    if (sumsq) {
        const zero_status s1 = launch_status();
        if (s1 != ZERO_OK) return s1;
        return finish_sumsq(workspace, ssq_partial_count(nquad, len - done), sumsq, st);
    }
    return launch_status();
}

namespace {

// the step's constants: hyperparameters on the host (hp), or constants in
// device memory (dc, read by the kernels); exactly one of the two is given
bool consts_arg_ok(const zero_adamw_hparams *hp, const zero_step_consts *dc) {
    return dc ? aligned8(dc) : hparams_ok(hp);
}

zero_status adamw_impl(const float *acc, float *master, float *m, float *v, void *weight_full,
                       zero_dtype wdt, const zero_layout *layout, int32_t rank, int64_t shard_off,
                       int64_t len, const zero_adamw_hparams *hp, const zero_step_consts *dc,
                       const zero_step_control *ctl, void *stream) {
    if (!dtype_ok(wdt) || !layout_ok(layout) || !consts_arg_ok(hp, dc)) return ZERO_EINVAL;
    if (rank < 0 || rank >= layout->n_dp || shard_off < 0 || len < 0 || len > kMaxLen)
        return ZERO_EINVAL;
    if (ctl && !std::isfinite(ctl->max_norm)) return ZERO_EINVAL;
    if (shard_off > layout->shard || len > layout->shard - shard_off) return ZERO_ERANGE;
    if (len == 0) return ZERO_OK;
    if (!acc || !master || !m || !v || !weight_full) return ZERO_EINVAL;
    uint16_t *slot = static_cast<uint16_t *>(weight_full) +
                     static_cast<int64_t>(rank) * layout->shard + shard_off;
    const Span outs[4] = {span_of(master, len, 4), span_of(m, len, 4), span_of(v, len, 4),
                          span_of(slot, len, 2)};
    // acc and the controls are read only, but no output may overlap them
    const uint32_t *skip = ctl ? ctl->skip : nullptr;
    Span ins[5];
    int n_in = 0;
    ins[n_in++] = span_of(acc, len, 4);
    if (dc) ins[n_in++] = span_of(dc, 1, sizeof(zero_step_consts));
    if (skip) ins[n_in++] = span_of(skip, 1, 4);
    if (ctl && ctl->sumsq) ins[n_in++] = span_of(ctl->sumsq, 1, 8);
    if (ctl && ctl->loss_scale) ins[n_in++] = span_of(ctl->loss_scale, 1, sizeof(zero_loss_scale));
    if (any_alias(outs, 4, nullptr, 0, 0, 0, 4, ins, n_in)) return ZERO_EALIAS;

    hipStream_t st = static_cast<hipStream_t>(stream);
    const Consts c = dc ? Consts{} : make_consts(*hp);
    const bool ext = ctl && ((ctl->sumsq && ctl->max_norm > 0.0) || ctl->loss_scale);
    const Control k{ctl ? ctl->sumsq : nullptr, ctl ? ctl->max_norm : 0.0,
                    ctl ? ctl->loss_scale : nullptr, dc ? 0.0 : hp->grad_scale};
    const bool vec = aligned16(acc) && aligned16(master) && aligned16(m) && aligned16(v) &&
                     aligned8(slot);
    const int64_t nquad = vec ? len / kQuad : 0;
    const int64_t done = nquad * kQuad;
    const size_t lds = residency_lds_bytes(kAdamwWavesPerCU, kWave);
    with_dtype(wdt, [&](auto WD) {
        with_bool(skip != nullptr, [&](auto SK) {
            with_bool(ext, [&](auto EX) {
                with_bool(dc != nullptr, [&](auto DV) {
                    for_launches(nquad, [&](int64_t q0, int64_t nq) {
                        const int64_t o = q0 * kQuad;
                        adamw_quad_kernel<kWave, WD.value, SK.value, EX.value, DV.value>
                            <<<grid_for(nq, kWave), kWave, lds, st>>>(
                                acc + o, master + o, m + o, v + o, slot + o, nq, c, skip, k, dc);
                    });
                    if (len > done) {
                        adamw_scalar_kernel<WD.value, SK.value, EX.value, DV.value>
                            <<<scalar_grid(len - done, false), kBlock, 0, st>>>(
                                acc + done, master + done, m + done, v + done, slot + done,
                                len - done, c, skip, k, dc);
                    }
                });
            });
        });
    });
    return launch_status();
}

}  // namespace

extern "C" zero_status zero_shard_adamw(const float *acc, float *master, float *m, float *v,
                                        void *weight_full, zero_dtype wdt,
                                        const zero_layout *layout, int32_t rank,
                                        int64_t shard_off, int64_t len,
                                        const zero_adamw_hparams *hp, const uint32_t *skip,
                                        void *stream) {
    const zero_step_control ctl{skip, nullptr, 0.0, nullptr};
    return adamw_impl(acc, master, m, v, weight_full, wdt, layout, rank, shard_off, len, hp,
                      nullptr, &ctl, stream);
}

extern "C" zero_status zero_shard_adamw_ex(const float *acc, float *master, float *m, float *v,
                                           void *weight_full, zero_dtype wdt,
                                           const zero_layout *layout, int32_t rank,
                                           int64_t shard_off, int64_t len,
                                           const zero_adamw_hparams *hp,
                                           const zero_step_control *ctl, void *stream) {
    return adamw_impl(acc, master, m, v, weight_full, wdt, layout, rank, shard_off, len, hp,
                      nullptr, ctl, stream);
}

extern "C" zero_status zero_shard_adamw_dc(const float *acc, float *master, float *m, float *v,
                                           void *weight_full, zero_dtype wdt,
                                           const zero_layout *layout, int32_t rank,
                                           int64_t shard_off, int64_t len,
                                           const zero_step_consts *consts,
                                           const zero_step_control *ctl, void *stream) {
    if (!consts) return ZERO_EINVAL;
    return adamw_impl(acc, master, m, v, weight_full, wdt, layout, rank, shard_off, len, nullptr,
                      consts, ctl, stream);
}

extern "C" zero_status zero_step_consts_select(zero_step_consts *consts,
                                               const zero_step_consts *table, int64_t count,
                                               const int64_t *t, void *stream) {
    if (!consts || !table || !t || count < 1 || !aligned8(consts) || !aligned8(table) ||
        !aligned8(t))
        return ZERO_EINVAL;
    if (count > INT64_MAX / static_cast<int64_t>(sizeof(zero_step_consts))) return ZERO_EINVAL;
    const Span out = span_of(consts, 1, sizeof(zero_step_consts));
    if (overlap(out, span_of(table, count, sizeof(zero_step_consts))) ||
        overlap(out, span_of(t, 1, sizeof(int64_t))))
        return ZERO_EALIAS;
    step_consts_select_kernel<<<1, 1, 0, static_cast<hipStream_t>(stream)>>>(consts, table, count,
                                                                             t);
    return launch_status();
}

extern "C" zero_status zero_step_counter_advance(int64_t *t, const uint32_t *skip, void *stream) {
    if (!t || !aligned8(t)) return ZERO_EINVAL;
    if (skip && overlap(span_of(t, 1, sizeof(int64_t)), span_of(skip, 1, 4))) return ZERO_EALIAS;
    step_counter_advance_kernel<<<1, 1, 0, static_cast<hipStream_t>(stream)>>>(t, skip);
    return launch_status();
}

extern "C" zero_status zero_step_consts_make(const zero_adamw_hparams *hp, zero_step_consts *out) {
    if (!out || !hparams_ok(hp)) return ZERO_EINVAL;
    const Consts c = make_consts(*hp);
    *out = zero_step_consts{c.s, c.b1, c.c1, c.b2, c.c2, c.bc1, c.bc2, c.lr, c.eps, c.d,
                            hp->grad_scale};
    return ZERO_OK;
}

extern "C" zero_status zero_loss_scale_update(zero_loss_scale *state, const uint32_t *overflow,
                                              double growth, double backoff, int32_t interval,
                                              void *stream) {
    if (!state || !overflow || !std::isfinite(growth) || growth < 1.0 || !(backoff > 0.0) ||
        backoff > 1.0 || interval < 1)
        return ZERO_EINVAL;
    if (overlap(span_of(state, 1, sizeof(zero_loss_scale)), span_of(overflow, 1, 4)))
        return ZERO_EALIAS;
    loss_scale_kernel<<<1, kWave, 0, static_cast<hipStream_t>(stream)>>>(state, overflow, growth,
                                                                         backoff, interval);
    return launch_status();
}

namespace {

zero_status step_impl(const void *grads, zero_dtype gdt, int64_t ld, int64_t len, float *master,
                      float *m, float *v, void *weight_full, zero_dtype wdt,
                      const zero_layout *layout, int32_t rank, int64_t shard_off,
                      const zero_adamw_hparams *hp, const zero_step_consts *dc,
                      uint32_t *overflow, double *sumsq, void *workspace,
                      int64_t workspace_bytes, void *stream) {
    if (!gdtype_ok(gdt) || !dtype_ok(wdt) || !layout_ok(layout) || !consts_arg_ok(hp, dc))
        return ZERO_EINVAL;
    const int n_dp = layout->n_dp;
    if (rank < 0 || rank >= n_dp || shard_off < 0 || !rows_ok(n_dp, ld, len) || len > kMaxLen)
        return ZERO_EINVAL;
    if (shard_off > layout->shard || len > layout->shard - shard_off) return ZERO_ERANGE;
    if (len == 0) return ZERO_OK;
    if (!grads || !master || !m || !v || !weight_full) return ZERO_EINVAL;
    if (sumsq && !workspace_ok(workspace, workspace_bytes, len)) return ZERO_EINVAL;
    uint16_t *slot = static_cast<uint16_t *>(weight_full) +
                     static_cast<int64_t>(rank) * layout->shard + shard_off;
    Span outs[7];
    int n_out = 0;
    outs[n_out++] = span_of(master, len, 4);
    outs[n_out++] = span_of(m, len, 4);
    outs[n_out++] = span_of(v, len, 4);
    outs[n_out++] = span_of(slot, len, 2);
    if (overflow) outs[n_out++] = span_of(overflow, 1, 4);
    if (sumsq) outs[n_out++] = span_of(sumsq, 1, 8);
    if (sumsq) outs[n_out++] = span_of(workspace, workspace_bytes, 1);
    const Span dspan = span_of(dc, dc ? 1 : 0, sizeof(zero_step_consts));
    if (any_alias(outs, n_out, grads, n_dp, ld, len, gdtype_bytes(gdt), &dspan, dc ? 1 : 0))
        return ZERO_EALIAS;

    hipStream_t st = static_cast<hipStream_t>(stream);
    const Consts c = dc ? Consts{} : make_consts(*hp);
    const bool vec = rows_vec_ok(grads, gdt, n_dp, ld) && aligned16(master) && aligned16(m) &&
                     aligned16(v) && aligned8(slot);
    const int64_t nquad = vec ? len / kQuad : 0;
    const int64_t done = nquad * kQuad;
    double *part = sumsq ? ssq_partials(workspace) : nullptr;
    const int64_t n_qpart = (nquad + kWave - 1) / kWave;
    with_gdtype(gdt, [&](auto GD) {
        using E = typename GradT<GD.value>::elem;
        const E *g = static_cast<const E *>(grads);
        with_dtype(wdt, [&](auto WD) {
            with_bool(overflow != nullptr, [&](auto OV) {
                with_bool(sumsq != nullptr, [&](auto SS) {
                    with_bool(dc != nullptr, [&](auto DV) {
                        if (nquad > 0) {
                            with_ndp<GD.value>(n_dp, [&](auto ND) {
                                const size_t lds = residency_lds_bytes(
                                    step_waves_per_cu(GD.value, ND.value, SS.value), kWave);
                                for_launches(nquad, [&](int64_t q0, int64_t nq) {
                                    const int64_t o = q0 * kQuad;
                                    step_quad_kernel<kWave, GD.value, WD.value, ND.value,
                                                     OV.value, SS.value, DV.value>
                                        <<<grid_for(nq, kWave), kWave, lds, st>>>(
                                            g + o, ld, n_dp, nq, master + o, m + o, v + o,
                                            slot + o, c, overflow,
                                            SS.value ? part + q0 / kWave : nullptr, dc);
                                });
                            });
                        }
                        if (len > done) {
                            step_scalar_kernel<GD.value, WD.value, OV.value, SS.value, DV.value>
                                <<<scalar_grid(len - done, SS.value), kBlock, 0, st>>>(
                                    g + done, ld, n_dp, len - done, master + done, m + done,
                                    v + done, slot + done, c, overflow,
                                    SS.value ? part + n_qpart : nullptr, dc);
                        }
                    });
                });
            });
        });
    });
    if (sumsq) {
        const zero_status s1 = launch_status();
        if (s1 != ZERO_OK) return s1;
        return finish_sumsq(workspace, ssq_partial_count(nquad, len - done), sumsq, st);
    }
    return launch_status();
}

}  // namespace

extern "C" zero_status zero_shard_step(const void *grads, zero_dtype gdt, int64_t ld,
                                       int64_t len, float *master, float *m, float *v,
                                       void *weight_full, zero_dtype wdt,
                                       const zero_layout *layout, int32_t rank,
                                       int64_t shard_off, const zero_adamw_hparams *hp,
                                       uint32_t *overflow, double *sumsq, void *workspace,
                                       int64_t workspace_bytes, void *stream) {
    return step_impl(grads, gdt, ld, len, master, m, v, weight_full, wdt, layout, rank, shard_off,
                     hp, nullptr, overflow, sumsq, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------------------
// The step for callers that cannot allocate: the sum of squares' workspace
// is a library-held device array, one copy per GPU, kept until the process
// ends.  It holds the per-workgroup partials and the stage-two sums of one
// call of up to ZERO_NOALLOC_MAX_LEN elements; every call writes the
// partials it later reads, so nothing in it needs clearing between calls.

namespace {

constexpr int64_t kScratchDoubles = kSsqStage2 + (ZERO_NOALLOC_MAX_LEN + 255) / 256 + kSsqScalarBlocks;
static_assert(static_cast<int64_t>(sizeof(double)) * kScratchDoubles ==
                  8 * (256 + (ZERO_NOALLOC_MAX_LEN + 255) / 256 + 4096),
              "the scratch holds exactly zero_sumsq_workspace_bytes(ZERO_NOALLOC_MAX_LEN)");

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

}  // namespace

static __device__ __align__(256) double scratch[kScratchDoubles];

namespace {

// The device address of the scratch array on the stream's GPU, looked up
// once per device with that device current.  (In host code `scratch` names
// a host-side stand-in, never passed to a kernel or a copy.)  nullptr when
// the runtime cannot tell the device or the address.
void *scratch_on(hipStream_t st) {
    int dev = -1;
    if (st ? hipStreamGetDevice(st, &dev) != hipSuccess : hipGetDevice(&dev) != hipSuccess)
        return nullptr;
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p) return p;
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
    void *q = nullptr;
    const hipError_t e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return nullptr;
    if (e != hipSuccess || q == nullptr) return nullptr;
    g_scratch[dev].store(q, std::memory_order_release);
    return q;
}

}  // namespace

extern "C" zero_status zero_shard_step_noalloc(const void *grads, zero_dtype gdt, int64_t ld,
                                               int64_t len, float *master, float *m, float *v,
                                               void *weight_full, zero_dtype wdt,
                                               const zero_layout *layout, int32_t rank,
                                               int64_t shard_off, const zero_adamw_hparams *hp,
                                               uint32_t *overflow, double *sumsq,
                                               void *stream) {
    if (!sumsq)
        return step_impl(grads, gdt, ld, len, master, m, v, weight_full, wdt, layout, rank,
                         shard_off, hp, nullptr, overflow, nullptr, nullptr, 0, stream);
    if (len > ZERO_NOALLOC_MAX_LEN) return ZERO_EINVAL;
    void *ws = scratch_on(static_cast<hipStream_t>(stream));
    if (!ws) return ZERO_EDEVICE;
    return step_impl(grads, gdt, ld, len, master, m, v, weight_full, wdt, layout, rank, shard_off,
                     hp, nullptr, overflow, sumsq, ws,
                     static_cast<int64_t>(sizeof(double)) * kScratchDoubles, stream);
}

extern "C" zero_status zero_shard_step_dc(const void *grads, zero_dtype gdt, int64_t ld,
                                          int64_t len, float *master, float *m, float *v,
                                          void *weight_full, zero_dtype wdt,
                                          const zero_layout *layout, int32_t rank,
                                          int64_t shard_off, const zero_step_consts *consts,
                                          uint32_t *overflow, double *sumsq, void *workspace,
                                          int64_t workspace_bytes, void *stream) {
    if (!consts) return ZERO_EINVAL;
    return step_impl(grads, gdt, ld, len, master, m, v, weight_full, wdt, layout, rank, shard_off,
                     nullptr, consts, overflow, sumsq, workspace, workspace_bytes, stream);
}
