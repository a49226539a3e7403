// step_common.h -- pieces shared by the library's step kernels (internal:
// not installed, not part of the C ABI): vector types, the fp32 constants of
// the AdamW update and their host-side formation, argument validators, the
// 16-bit conversions, streaming loads and stores, and the arithmetic of one
// element.
#ifndef ZERO_SHARD_STEP_COMMON_H
#define ZERO_SHARD_STEP_COMMON_H

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "host_common.h"
#include "zero_shard.h"

namespace zero_step {

using zero_host::kWave;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kQuad = 4;  // elements per lane

// Ranges beyond kMaxLen elements (2^38, far beyond any HBM) are rejected.
constexpr int64_t kMaxLen = int64_t(1) << 38;

// A buffer or row slab may span at most kMaxSpan elements (2^60), so that the
// byte offset of any element of up to 8 bytes fits in int64.
constexpr int64_t kMaxSpan = INT64_MAX / 8;

// n_rows rows of len elements, ld elements apart (n_rows >= 1, 0 <= len <=
// ld), spanning (n_rows - 1) * ld + len <= kMaxSpan elements
inline bool rows_ok(int64_t n_rows, int64_t ld, int64_t len) {
    if (n_rows < 1 || len < 0 || ld < len || len > kMaxSpan) return false;
    return ld == 0 || n_rows - 1 <= (kMaxSpan - len) / ld;
}

// A dispatch counts its grid in work-items in 32 bits, so one launch of a
// one-shot kernel (a thread per quad or per block lane) covers at most
// kLaunchElems elements and longer ranges go out as consecutive launches.
// 2^31 is a multiple of every quad, block and alignment unit: each piece
// starts where the range's alignment holds.
constexpr int64_t kLaunchElems = int64_t(1) << 31;

// the grid-stride (one element per thread) kernels take at most this many
// workgroups and loop over the rest
constexpr int64_t kMaxStrideBlocks = int64_t(1) << 20;

// fp32 constants of the update, formed on the host (see zero_adamw_hparams)
struct Consts {
    float s, b1, c1, b2, c2, bc1, bc2, lr, eps, d;
};

inline bool dtype_ok(int dt) { return dt == ZERO_BF16 || dt == ZERO_FP16; }

inline bool layout_ok(const zero_layout *l) {
    if (!l || l->n_dp < 1 || l->align < 1 || l->shard < 0 || l->n < 0) return false;
    if (l->shard % l->align != 0) return false;
    if (l->shard > 0 && l->n_dp > INT64_MAX / l->shard) return false;
    return l->n_pad == l->shard * l->n_dp && l->n <= l->n_pad && l->n_pad <= kMaxSpan;
}

inline bool hparams_ok(const zero_adamw_hparams *hp) {
    if (!hp || hp->step < 1) return false;
    if (!std::isfinite(hp->lr)) return false;
    if (!(hp->beta1 >= 0.0 && hp->beta1 < 1.0)) return false;
    if (!(hp->beta2 >= 0.0 && hp->beta2 < 1.0)) return false;
    if (!(std::isfinite(hp->eps) && hp->eps > 0.0)) return false;
    if (!(std::isfinite(hp->weight_decay) && hp->weight_decay >= 0.0)) return false;
    return std::isfinite(hp->grad_scale) && hp->grad_scale > 0.0;
}

// each constant in double, rounded once to fp32
inline Consts make_consts(const zero_adamw_hparams &hp) {
    const double t = static_cast<double>(hp.step);
    Consts c;
    c.s = static_cast<float>(hp.grad_scale);
    c.b1 = static_cast<float>(hp.beta1);
    c.c1 = static_cast<float>(1.0 - hp.beta1);
    c.b2 = static_cast<float>(hp.beta2);
    c.c2 = static_cast<float>(1.0 - hp.beta2);
    c.bc1 = static_cast<float>(1.0 - std::pow(hp.beta1, t));
    c.bc2 = static_cast<float>(1.0 - std::pow(hp.beta2, t));
    c.lr = static_cast<float>(hp.lr);
    c.eps = static_cast<float>(hp.eps);
    c.d = static_cast<float>(1.0 - hp.lr * hp.weight_decay);
    return c;
}

// the fp32 constants of a zero_step_consts (a kernel reads it from device
// memory when the step's constants are not kernel arguments)
__host__ __device__ inline Consts consts_of(const zero_step_consts &d) {
    return Consts{d.s, d.b1, d.c1, d.b2, d.c2, d.bc1, d.bc2, d.lr, d.eps, d.d};
}

// Device constants whose gradient scale is not a number (what a step
// counter past its table selects) hold the step: the kernel writes no
// state, no weight and no partial sum of squares beyond a zero, and raises
// the overflow flag when it has one, so that the state survives and the
// caller can tell the step was not taken.
__host__ __device__ inline bool step_held(const Consts &c) { return c.s != c.s; }

// ---------------------------------------------------------------------------
// 16-bit <-> fp32.  Widening is exact.  Narrowing uses gfx950's packed
// converts (v_cvt_pk_bf16_f32, v_cvt_pk_f16_f32): round to nearest even.

template <int DT>
__device__ __forceinline__ f32x2 widen2(uint32_t w) {
    if constexpr (DT == ZERO_BF16) {
        return f32x2{__uint_as_float(w << 16), __uint_as_float(w & 0xFFFF0000u)};
    } else {
        return __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
    }
}

template <int DT>
__device__ __forceinline__ uint32_t narrow2(float lo, float hi) {
    const f32x2 x{lo, hi};
    if constexpr (DT == ZERO_BF16) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
    } else {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, f16x2));
    }
}

// An fp32 value as rounded: the compiler may not fold the operation that
// produced it into a later 16-bit conversion (v_fma_mix* would round the
// exact result once, to 16 bits, instead of to fp32 and then to 16 bits).
__device__ __forceinline__ float as_rounded_f32(float x) {
    asm("" : "+v"(x));
    return x;
}

template <int DT>
__device__ __forceinline__ uint16_t narrow1(float f) {
    return static_cast<uint16_t>(narrow2<DT>(f, 0.0f) & 0xFFFFu);
}

// ---------------------------------------------------------------------------
// memory helpers: loads/stores of data streamed once.  Loads are marked
// non-temporal.  Stores are non-temporal at device scope (cache policy
// nt sc1): for these read-mostly streams that keeps HBM 1.5-2 % busier than
// non-temporal stores at the default scope, at every residency and row
// count tried.  No builtin sets the scope bits of a plain store, so the
// store is written out; its operands are the lane's 64-bit global address
// and the value, and "memory" keeps it in program order with every other
// access.  A store of more than 64 bits of data reads its data registers
// after it issues, so on this chip two wait states must pass before any
// later instruction may overwrite them; the compiler inserts them after its
// own stores but cannot see into this one, so the 16-byte store carries
// them itself (s_nop 1).  An 8-byte store has no such hazard.

__device__ __forceinline__ u32x2 load8(const uint16_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
}
__device__ __forceinline__ f32x4 load16(const float *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
}
__device__ __forceinline__ void store8(uint16_t *p, u32x2 x) {
    asm volatile("global_store_dwordx2 %0, %1, off nt sc1" : : "v"(p), "v"(x) : "memory");
}
__device__ __forceinline__ void store16(void *p, u32x4 x) {
    asm volatile("global_store_dwordx4 %0, %1, off nt sc1\n\ts_nop 1" : : "v"(p), "v"(x)
                 : "memory");
}
__device__ __forceinline__ void store16(float *p, f32x4 x) {
    store16(static_cast<void *>(p), __builtin_bit_cast(u32x4, x));
}
__device__ __forceinline__ void store4(void *p, uint32_t x) {
    asm volatile("global_store_dword %0, %1, off nt sc1" : : "v"(p), "v"(x) : "memory");
}

// Gradient rows: 16-bit (4 elements of a quad = 8 bytes per lane) or fp32
// (16 bytes per lane); the element type and the per-lane quad type.
template <int GDT>
struct GradT {
    using elem = uint16_t;
    using quad = u32x2;
};
template <>
struct GradT<ZERO_FP32> {
    using elem = float;
    using quad = f32x4;
};

template <int DT>
__device__ __forceinline__ float widen1(typename GradT<DT>::elem h) {
    if constexpr (DT == ZERO_FP32) {
        return h;
    } else {
        return widen2<DT>(static_cast<uint32_t>(h))[0];
    }
}

// a row's quad, non-temporal (streamed once)
template <int GDT>
__device__ __forceinline__ typename GradT<GDT>::quad load_quad(const typename GradT<GDT>::elem *p) {
    if constexpr (GDT == ZERO_FP32) {
        return load16(p);
    } else {
        return load8(p);
    }
}
// the four fp32 values of one row's quad (16-bit widening is exact)
template <int GDT>
__device__ __forceinline__ void widen_quad(float t[kQuad], typename GradT<GDT>::quad x) {
    if constexpr (GDT == ZERO_FP32) {
#pragma unroll
        for (int e = 0; e < kQuad; ++e) t[e] = x[e];
    } else {
        const f32x2 t0 = widen2<GDT>(x[0]), t1 = widen2<GDT>(x[1]);
        t[0] = t0[0];
        t[1] = t0[1];
        t[2] = t1[0];
        t[3] = t1[1];
    }
}

// Keeps the compiler from sinking any of the loads issued so far below the
// arithmetic that follows: one round trip to HBM per quad, not two.
__device__ __forceinline__ void loads_issued() { __builtin_amdgcn_sched_barrier(0); }

// The optional shard-wide outputs: one atomic per wave for the flag (only
// when a lane saw a non-finite value); for the sum, a fixed-order wave
// (then workgroup) reduction and one plain store of the workgroup's partial
// to part[blockIdx.x] -- finish_sumsq() adds the partials into the caller's
// scalar afterwards, in a fixed order.  (One atomic add per workgroup into
// one address instead would cap the rate at about 80 M workgroups/s and
// force large workgroups, which the streaming kernels lose 10 % to.)
// Every thread of the workgroup must reach this point.
template <int TPB, bool OVF, bool SSQ>
__device__ __forceinline__ void flags_epilogue(bool bad, double ss, uint32_t *ovf, double *part) {
    if constexpr (OVF) {
        if (__ballot(bad) != 0 && (threadIdx.x & (kWave - 1)) == 0) atomicOr(ovf, 1u);
    }
    if constexpr (SSQ) {
#pragma unroll
        for (int off = kWave / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off, kWave);
        if constexpr (TPB == kWave) {
            if (threadIdx.x == 0) part[blockIdx.x] = ss;
        } else {
            __shared__ double wave_part[TPB / kWave];
            if ((threadIdx.x & (kWave - 1)) == 0) wave_part[threadIdx.x / kWave] = ss;
            __syncthreads();
            if (threadIdx.x == 0) {
                double t = wave_part[0];
#pragma unroll
                for (int wv = 1; wv < TPB / kWave; ++wv) t += wave_part[wv];
                part[blockIdx.x] = t;
            }
        }
    }
}

// Sum of squares: partials of one call's workgroups, then the fixed-order
// finish.  A workspace of zero_sumsq_workspace_bytes(len) holds
// kSsqStage2 stage-two sums followed by the partials (at most
// blocks_of(len) + kSsqScalarBlocks of them).
constexpr int kSsqStage2 = 256;           // stage-two workgroups (and sums)
constexpr int64_t kSsqScalarBlocks = 4096; // grid cap of the summing element kernels
inline int64_t ssq_partials_cap(int64_t len) { return (len + 255) / 256 + kSsqScalarBlocks; }
inline double *ssq_partials(void *workspace) {
    return static_cast<double *>(workspace) + kSsqStage2;
}
// *sumsq += the sum of part[0, count), in an order fixed by count alone
// (defined with the library's other kernels; launches two small kernels)
zero_status finish_sumsq(void *workspace, int64_t count, double *sumsq, hipStream_t st);

// ---------------------------------------------------------------------------
// the arithmetic of one element

// AdamW ("ZeRO and FSDP", "A sharded Adam step", with decoupled decay):
// m = b1 m + c1 g; v = b2 v + c2 g^2; w = w d - lr (m / bc1) / (sqrt(v / bc2) + eps)
__device__ __forceinline__ void adamw_element(float g, float &w, float &m, float &v,
                                              const Consts &c) {
    const float mt = c.b1 * m + c.c1 * g;
    const float vt = c.b2 * v + c.c2 * (g * g);
    const float mhat = mt / c.bc1;
    const float vhat = vt / c.bc2;
    const float den = sqrtf(vhat) + c.eps;
    const float upd = mhat / den;
    w = w * c.d - c.lr * upd;
    m = mt;
    v = vt;
}

}  // namespace zero_step

#endif
