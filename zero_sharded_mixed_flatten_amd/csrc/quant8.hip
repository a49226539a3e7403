// quant8.hip -- gfx950 kernels for 8-bit blockwise communication (ZeRO++).
//
// ZeRO++ quantizes the weight all-gather to 8 bits and the gradients of the
// reduce-scatter ("ZeRO and FSDP", FSDP section; "ZeRO Optimizer, in depth",
// "Offload and ZeRO++").  The pages give no quantizer; the one here is the
// plain symmetric blockwise int8 quantizer, one fp32 scale per block of 256
// elements: s = absmax / 127 stored, codes q = rint(x / s), the value in
// units of the stored scale with the quotient rounded to binary32 and then
// to an integer, ties to even.
//
// A block is exactly one wave's quad layout: 64 lanes x 4 consecutive
// elements, so a block's absmax is one wave reduction (DPP within each row
// of 16 lanes, then one lane per row) and needs no LDS.  The kernels are
// one-shot grids, loads issued before arithmetic, non-temporal streaming
// access -- the layout of the 16-bit step kernels with 4-byte code loads
// (one contiguous 256-byte span per wave and row) and one scale per row and
// block read through the scalar cache.  The fused step takes one block per
// one-wave workgroup (with a sum of squares, each wave stores its partial),
// quantize and dequantize to fp32 two consecutive blocks
// per wave, and dequantize to 16 bits a pair of blocks per wave at 8 codes
// per lane, so that both its code loads and its 16-byte stores are
// contiguous across the wave.
//
// Arithmetic gives the oracle's results bit for bit: a correctly rounded
// fp32 division for absmax / 127, codes equal to rint(fl(x / s)) (formed
// with the block's reciprocal where that provably gives the same integer,
// by the division itself elsewhere; see quantize4), v_rndne_f32 for the
// rounding, and q * s rounded once to fp32.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <type_traits>

#include "host_common.h"
#include "step_common.h"
#include "zero_shard.h"

namespace {

using namespace zero_host;
using namespace zero_step;

constexpr int kB = ZERO_Q8_BLOCK;
static_assert(kB == kWave * kQuad, "a quantization block is one wave of quads");
constexpr int kRowBatchQ8 = 8;          // rows per batch when n_dp is not specialised
// The fused 8-bit step carries ~125 VALU operations per element (AdamW's
// divisions and square root, 8 dequantizations, the quantization) against
// 33 bytes: it needs more waves than the 16-bit step to hide that work under
// memory time, but not too many.  Measured on the 7B shard (8 rows, random
// data, one process, same buffers), waves per CU: 8 -> 4.81 ms, 9 -> 4.56,
// 10 -> 4.41, 11 -> 4.45, 12 -> 4.53, 14 -> 4.56-4.57.
constexpr int kQ8StepWavesPerCU = 10;   // residency cap of the fused 8-bit step
// Quantize and dequantize to fp32: Q blocks per wave, loads first.  Sweep on
// the 7B shard (blocks per wave x waves per CU), quantize fp32 -> int8 +
// scales: 1 x 32 -> 0.79 ms, 2 x 24 -> 0.67, 2 x 32 -> 0.63, 4 x 16 -> 0.68,
// 4 x 24 -> 0.67, 8 x 16 -> 0.67; dequantize to fp32: 1 x 32 -> 0.79 ms,
// 2 x 24 -> 0.65, 2 x 32 -> 0.70, 4 x 12 -> 0.65, 4 x 24 -> 0.68.
constexpr int kQ8QuantizeBlocks = 2;
constexpr int kQ8QuantizeWavesPerCU = 32;
constexpr int kQ8DequantizeF32Blocks = 2;
constexpr int kQ8DequantizeF32WavesPerCU = 24;
// Dequantize to 16 bits: one pair of blocks per wave at 8 codes per lane,
// waves per CU (to bf16): 16 -> 0.59 ms, 24 -> 0.43, 32 -> 0.37 (85 % of
// 8 TB/s); two and four pairs per wave: 0.39 and 0.40 ms; the quad layout
// (4-byte code loads, 8-byte stores) at best 0.46 ms; 16 codes per lane
// (16-byte stores at a 32-byte stride): 0.85 ms.
constexpr int kQ8DequantizeWavesPerCU = 32;

// max with NaN winning (order independent): the scale of a block holding a
// NaN is NaN
__device__ __forceinline__ float nanmax(float a, float b) { return (a != a || a > b) ? a : b; }

// one lane's value moved by a DPP lane pattern (VALU only, no LDS)
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                         0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// The wave's NaN-winning max, in every lane: within each row of 16 lanes by
// DPP (swap neighbours, swap pairs, rotate by 4, rotate by 8), then across
// the four rows from one lane of each.  nanmax is commutative and
// associative in value, so the pattern does not change the result.
__device__ __forceinline__ float wave_nanmax(float m) {
    m = nanmax(m, dpp<0xB1>(m));   // quad_perm [1,0,3,2]
    m = nanmax(m, dpp<0x4E>(m));   // quad_perm [2,3,0,1]
    m = nanmax(m, dpp<0x124>(m));  // row_ror:4
    m = nanmax(m, dpp<0x128>(m));  // row_ror:8
    const int b = __builtin_bit_cast(int, m);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
    return nanmax(nanmax(r0, r1), nanmax(r2, r3));
}

// A block's scale s = absmax / 127 (stored; value = code * s) and the
// reciprocal r = 127 / absmax, from the four values of each lane (invalid
// ones 0).  Two divisions per lane per block.
struct BlockScale {
    float s, r;
};

__device__ __forceinline__ BlockScale block_scale(const float x[kQuad]) {
    float m = 0.0f;
#pragma unroll
    for (int e = 0; e < kQuad; ++e) m = nanmax(fabsf(x[e]), m);
    const float amax = wave_nanmax(m);
    return BlockScale{amax / 127.0f, 127.0f / amax};
}

// Codes are rint(fl(x / s)); all zero when s is zero or not finite.
//
// A correctly rounded division per element is ~11 VALU instructions; the
// product y = fl(x * r) is one, and it decides the code except within a
// hair of a half-integer.  When s is normal (s >= 2^-126), r and 1/s differ
// by at most the two roundings of s and r, so y = (x / s)(1 + t) with
// |t| < 3.0000002 * 2^-24 (or an absolute error below 2^-150 where x * r is
// subnormal), and |x / s| <= absmax / s < 127.0000076: |y - x / s| < 2.28e-5.
// The binary32 quotient fl(x / s) lies within 2^-18 (half its ulp below 128)
// of x / s.  So when y is more than 2^-14 = 6.1e-5 from every half-integer,
// x / s and fl(x / s) lie strictly inside the same interval between
// half-integers as y, and rint(y) = rint(fl(x / s)).  Only lanes whose y is
// within 2^-14 of a half-integer (about 1 element in 8,000) -- and every
// element of a block whose s is subnormal, where r no longer tracks 1/s --
// take the division.  y - rint(y) is exact (the two are within 1/2 of each
// other, below 2^23), so the test itself does not round.  The division sits
// behind one wave-uniform branch per block (about 3 % of 256-element blocks
// hold such an element), so the other blocks carry no per-element branch.
__device__ __forceinline__ uint32_t quantize4(const float x[kQuad], BlockScale bs) {
    if (!(bs.s > 0.0f) || __builtin_isinf(bs.s)) return 0u;
    float r[kQuad];
    bool near[kQuad];
    bool any = bs.s < 0x1p-126f;  // wave-uniform: a subnormal scale divides everywhere
#pragma unroll
    for (int e = 0; e < kQuad; ++e) {
        const float y = x[e] * bs.r;
        r[e] = __builtin_rintf(y);
        near[e] = any || fabsf(y - r[e]) >= 0.5f - 0x1p-14f;
    }
    if (__any(near[0] || near[1] || near[2] || near[3])) {  // wave-uniform
#pragma unroll
        for (int e = 0; e < kQuad; ++e) {
            const float d = __builtin_rintf(x[e] / bs.s);
            r[e] = near[e] ? d : r[e];
        }
    }
    uint32_t packed = 0u;
#pragma unroll
    for (int e = 0; e < kQuad; ++e) {
        const float c = fminf(fmaxf(r[e], -127.0f), 127.0f);
        packed |= (static_cast<uint32_t>(static_cast<int32_t>(c)) & 0xFFu) << (8 * e);
    }
    return packed;
}

__device__ __forceinline__ float code(uint32_t packed, int e) {
    return static_cast<float>(static_cast<int8_t>((packed >> (8 * e)) & 0xFFu));
}

__device__ __forceinline__ uint32_t load_codes(const int8_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
}
__device__ __forceinline__ void store_codes(int8_t *p, uint32_t x) { store4(p, x); }

// the block handled by this wave, made wave-uniform (scalar) for the scale
// loads; a launch covers at most 2^23 blocks (kLaunchElems / kB)
// Workgroups go round-robin over the 8 XCDs (each with its own L2), so the
// 32 blocks whose scales share a 128-byte line run on all eight and each L2
// fetches the line: the 7B step reads 1.06 x its algorithmic bytes.
// Remapping workgroups so that each XCD takes whole chunks of consecutive
// blocks removes the re-reads (1.01 x) but costs more than it saves
// (measured at 16 waves per CU: 4.43 ms in plain order; chunks of 4, 8, 16
// and 32 blocks: 4.53, 4.61, 4.70 and 4.97 ms), so the order stays plain.
template <int TPB>
__device__ __forceinline__ int64_t wave_block() {
    const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    return static_cast<int64_t>(blockIdx.x) * (TPB / kWave) + w;
}

// ---------------------------------------------------------------------------
// quantize / dequantize

// The codec kernels split on a wave-uniform test: a wave whose blocks all
// lie in the range (with aligned buffers) takes straight-line vector loads,
// all issued before any arithmetic; the rest (the range's last wave, or
// unaligned buffers) take per-lane guards.  A per-lane choice between a
// vector load and element loads in the load phase would make the compiler
// wait for each load before issuing the next (the branches write the same
// registers), one load in flight per wave.

// Q consecutive blocks per wave, every load issued before the first block's
// reduction (more bytes in flight per wave).
template <int XDT, bool VEC, int Q>
__global__ void __launch_bounds__(kWave)
q8_quantize_kernel(const typename GradT<XDT>::elem *__restrict__ x, int64_t len,
                   int8_t *__restrict__ q, float *__restrict__ scales) {
    const int64_t b0 = wave_block<kWave>() * Q;
    const int lane = threadIdx.x;
    if (VEC && (b0 + Q) * kB <= len) {  // wave-uniform: Q whole blocks
        float v[Q][kQuad];
#pragma unroll
        for (int u = 0; u < Q; ++u)
            widen_quad<XDT>(v[u], load_quad<XDT>(x + (b0 + u) * kB + lane * kQuad));
        loads_issued();
        float sc[Q];
#pragma unroll
        for (int u = 0; u < Q; ++u) {
            const BlockScale bs = block_scale(v[u]);
            sc[u] = bs.s;
            store_codes(q + (b0 + u) * kB + lane * kQuad, quantize4(v[u], bs));
        }
        if (lane == 0) {
            // the wave's scales as one store when aligned (b0 is a multiple of Q)
            const uintptr_t sa = reinterpret_cast<uintptr_t>(scales);
            bool done = false;
            if constexpr (Q == 4) {
                if ((sa & 15u) == 0) {
                    *reinterpret_cast<f32x4 *>(scales + b0) = f32x4{sc[0], sc[1], sc[2], sc[3]};
                    done = true;
                }
            } else if constexpr (Q == 2) {
                if ((sa & 7u) == 0) {
                    *reinterpret_cast<f32x2 *>(scales + b0) = f32x2{sc[0], sc[1]};
                    done = true;
                }
            }
            if (!done) {
#pragma unroll
                for (int u = 0; u < Q; ++u) scales[b0 + u] = sc[u];
            }
        }
        return;
    }
    float v[Q][kQuad];
#pragma unroll
    for (int u = 0; u < Q; ++u) {
        const int64_t e0 = (b0 + u) * kB + lane * kQuad;
#pragma unroll
        for (int e = 0; e < kQuad; ++e) v[u][e] = 0.0f;
        if (VEC && e0 + kQuad <= len) {
            widen_quad<XDT>(v[u], load_quad<XDT>(x + e0));
        } else {
#pragma unroll
            for (int e = 0; e < kQuad; ++e)
                if (e0 + e < len) v[u][e] = widen1<XDT>(x[e0 + e]);
        }
    }
    loads_issued();
#pragma unroll
    for (int u = 0; u < Q; ++u) {
        const int64_t b = b0 + u;
        if (b * kB >= len) break;  // wave-uniform
        const int64_t e0 = b * kB + lane * kQuad;
        const BlockScale bs = block_scale(v[u]);
        if (lane == 0) scales[b] = bs.s;
        const uint32_t c = quantize4(v[u], bs);
        if (VEC && e0 + kQuad <= len) {
            store_codes(q + e0, c);
        } else {
#pragma unroll
            for (int e = 0; e < kQuad; ++e)
                if (e0 + e < len) q[e0 + e] = static_cast<int8_t>((c >> (8 * e)) & 0xFFu);
        }
    }
}

template <int YDT>
__device__ __forceinline__ void store_quad_any(void *y, int64_t e0, const float v[kQuad]) {
    if constexpr (YDT == ZERO_FP32) {
        store16(static_cast<float *>(y) + e0, f32x4{v[0], v[1], v[2], v[3]});
    } else {
        store8(static_cast<uint16_t *>(y) + e0,
               u32x2{narrow2<YDT>(v[0], v[1]), narrow2<YDT>(v[2], v[3])});
    }
}

template <int YDT>
__device__ __forceinline__ void store_one(void *y, int64_t e, float v) {
    if constexpr (YDT == ZERO_FP32) static_cast<float *>(y)[e] = v;
    else static_cast<uint16_t *>(y)[e] = narrow1<YDT>(v);
}

template <int YDT, bool VEC, int Q>
__global__ void __launch_bounds__(kWave)
q8_dequantize_kernel(const int8_t *__restrict__ q, const float *__restrict__ scales, int64_t len,
                     void *__restrict__ y) {
    const int64_t b0 = wave_block<kWave>() * Q;
    const int lane = threadIdx.x;
    if (VEC && (b0 + Q) * kB <= len) {  // wave-uniform: Q whole blocks
        uint32_t c[Q];
        float s[Q];
#pragma unroll
        for (int u = 0; u < Q; ++u) {
            c[u] = load_codes(q + (b0 + u) * kB + lane * kQuad);
            s[u] = scales[b0 + u];
        }
        loads_issued();
#pragma unroll
        for (int u = 0; u < Q; ++u) {
            float v[kQuad];
#pragma unroll
            for (int e = 0; e < kQuad; ++e) v[e] = as_rounded_f32(code(c[u], e) * s[u]);
            store_quad_any<YDT>(y, (b0 + u) * kB + lane * kQuad, v);
        }
        return;
    }
    uint32_t c[Q];
    float s[Q];
#pragma unroll
    for (int u = 0; u < Q; ++u) {
        const int64_t b = b0 + u;
        const int64_t e0 = b * kB + lane * kQuad;
        c[u] = 0u;
        s[u] = 0.0f;
        if (b * kB < len) s[u] = scales[b];
        if (VEC && e0 + kQuad <= len) c[u] = load_codes(q + e0);
    }
    loads_issued();
#pragma unroll
    for (int u = 0; u < Q; ++u) {
        const int64_t b = b0 + u;
        const int64_t e0 = b * kB + lane * kQuad;
        if (VEC && e0 + kQuad <= len) {
            float v[kQuad];
#pragma unroll
            for (int e = 0; e < kQuad; ++e) v[e] = as_rounded_f32(code(c[u], e) * s[u]);
            store_quad_any<YDT>(y, e0, v);
        } else {
#pragma unroll
            for (int e = 0; e < kQuad; ++e)
                if (e0 + e < len)
                    store_one<YDT>(y, e0 + e, as_rounded_f32(static_cast<float>(q[e0 + e]) * s[u]));
        }
    }
}

// Dequantize to 16 bits: a wave takes the pair of blocks 2p, 2p + 1, lanes
// 0-31 the first and 32-63 the second, 8 codes per lane (one 8-byte load,
// one 16-byte store).  Every launched wave has its first block in range.
template <int YDT, bool VEC>
__global__ void __launch_bounds__(kWave)
q8_dequantize_pair_kernel(const int8_t *__restrict__ q, const float *__restrict__ scales,
                          int64_t len, uint16_t *__restrict__ y) {
    constexpr int kPer = 2 * kQuad;  // codes per lane
    const int64_t p = wave_block<kWave>();
    const int lane = threadIdx.x;
    const int64_t b0 = 2 * p;
    const int64_t e0 = p * (2 * kB) + lane * kPer;
    if (VEC && (b0 + 2) * kB <= len) {  // wave-uniform: both blocks whole
        const u32x2 c = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(q + e0));
        const float s0 = scales[b0], s1 = scales[b0 + 1];
        loads_issued();
        const float s = lane < kWave / 2 ? s0 : s1;
        float v[kPer];
#pragma unroll
        for (int e = 0; e < kQuad; ++e) {
            v[e] = as_rounded_f32(code(c[0], e) * s);
            v[kQuad + e] = as_rounded_f32(code(c[1], e) * s);
        }
        const u32x4 o{narrow2<YDT>(v[0], v[1]), narrow2<YDT>(v[2], v[3]),
                      narrow2<YDT>(v[4], v[5]), narrow2<YDT>(v[6], v[7])};
        store16(y + e0, o);
        return;
    }
    // the range's last wave, or unaligned buffers: element by element
    const float s0 = scales[b0];
    const float s1 = (b0 + 1) * kB < len ? scales[b0 + 1] : 0.0f;  // wave-uniform
    const float s = lane < kWave / 2 ? s0 : s1;
    for (int e = 0; e < kPer; ++e)
        if (e0 + e < len) y[e0 + e] = narrow1<YDT>(as_rounded_f32(static_cast<float>(q[e0 + e]) * s));
}

// ---------------------------------------------------------------------------
// fused step: dequantize + reduce -> scale -> AdamW -> quantize, one pass

// a[e] += q_k[e] * s_k for the rows in r (first row assigns)
template <int NR>
__device__ __forceinline__ void add_code_rows(float a[kQuad], const uint32_t *c, const float *s,
                                              int count, bool first) {
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        if (k >= count) break;
#pragma unroll
        for (int e = 0; e < kQuad; ++e) {
            const float x = code(c[k], e) * s[k];
            a[e] = (first && k == 0) ? x : a[e] + x;
        }
    }
}

// the codes of row k for this lane's quad: vector when the quad is whole,
// else the valid bytes (0 beyond len)
__device__ __forceinline__ uint32_t row_codes(const int8_t *__restrict__ p, bool full, int valid) {
    if (full) return load_codes(p);
    uint32_t c = 0u;
    for (int e = 0; e < valid; ++e) c |= (static_cast<uint32_t>(static_cast<uint8_t>(p[e]))) << (8 * e);
    return c;
}

// One lane's state for the any-row-count path (its code rows are loaded in
// batches later).  FULL (wave-uniform: every quad of the block lies in the
// range) takes straight-line vector loads; otherwise each lane loads its
// valid elements one by one.
template <bool FULL>
__device__ __forceinline__ void load_state(float w[kQuad], float m[kQuad], float v[kQuad],
                                           int64_t e0, int valid, const float *__restrict__ W,
                                           const float *__restrict__ M,
                                           const float *__restrict__ V) {
    if constexpr (FULL) {
        const f32x4 w4 = load16(W + e0), m4 = load16(M + e0), v4 = load16(V + e0);
#pragma unroll
        for (int e = 0; e < kQuad; ++e) {
            w[e] = w4[e];
            m[e] = m4[e];
            v[e] = v4[e];
        }
    } else {
        for (int e = 0; e < valid; ++e) {
            w[e] = W[e0 + e];
            m[e] = M[e0 + e];
            v[e] = V[e0 + e];
        }
    }
}

// One block of the fused 8-bit step for a row count fixed at compile time.
// FULL (the block lies wholly in the range) is a template parameter, so the
// hot path carries no per-lane validity tests; the block's bases are
// wave-uniform and each lane adds a 32-bit offset, which lets the loads and
// stores take a scalar base address instead of per-lane 64-bit sums.
template <int NDP, bool OVF, bool SSQ, bool FULL>
__device__ __forceinline__ void step_q8_block(const int8_t *__restrict__ gq,
                                              const float *__restrict__ gs, int64_t ld,
                                              int64_t sld, int64_t len, int64_t b,
                                              float *__restrict__ W, float *__restrict__ M,
                                              float *__restrict__ V, int8_t *__restrict__ wq,
                                              float *__restrict__ wsc, const Consts &c,
                                              bool &bad, double &ss) {
    const uint32_t lo = (threadIdx.x % kWave) * kQuad;  // the lane's first element in the block
    const int64_t base = b * kB;
    const int8_t *gqb = gq + base;
    const float *gsb = gs + b;
    float *Wb = W + base, *Mb = M + base, *Vb = V + base;
    int8_t *wqb = wq + base;
    int valid = kQuad;
    if constexpr (!FULL) {
        const int64_t e0 = base + lo;
        valid = e0 + kQuad <= len ? kQuad : (e0 < len ? static_cast<int>(len - e0) : 0);
    }
    uint32_t cr[NDP];
    float sr[NDP];
    float w[kQuad] = {0.0f, 0.0f, 0.0f, 0.0f};
    float m[kQuad] = {0.0f, 0.0f, 0.0f, 0.0f};
    float v[kQuad] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < NDP; ++k) {
        cr[k] = FULL ? load_codes(gqb + k * ld + lo) : row_codes(gqb + k * ld + lo, false, valid);
        sr[k] = gsb[k * sld];
    }
    if constexpr (FULL) {
        const f32x4 w4 = load16(Wb + lo), m4 = load16(Mb + lo), v4 = load16(Vb + lo);
#pragma unroll
        for (int e = 0; e < kQuad; ++e) {
            w[e] = w4[e];
            m[e] = m4[e];
            v[e] = v4[e];
        }
    } else {
        for (int e = 0; e < valid; ++e) {
            w[e] = Wb[lo + e];
            m[e] = Mb[lo + e];
            v[e] = Vb[lo + e];
        }
    }
    loads_issued();
    float a[kQuad];
    add_code_rows<NDP>(a, cr, sr, NDP, true);
#pragma unroll
    for (int e = 0; e < kQuad; ++e) {
        if (FULL || e < valid) {
            if constexpr (OVF) bad |= !__builtin_isfinite(a[e]);
            const float g = a[e] * c.s;
            if constexpr (SSQ) ss += static_cast<double>(g) * static_cast<double>(g);
            adamw_element(g, w[e], m[e], v[e], c);
        } else {
            w[e] = 0.0f;  // outside the range: no part of the block's scale
        }
    }
    const BlockScale bs = block_scale(w);
    const uint32_t codes = quantize4(w, bs);
    if (lo == 0) wsc[b] = bs.s;
    if constexpr (FULL) {
        store16(Wb + lo, f32x4{w[0], w[1], w[2], w[3]});
        store16(Mb + lo, f32x4{m[0], m[1], m[2], m[3]});
        store16(Vb + lo, f32x4{v[0], v[1], v[2], v[3]});
        store_codes(wqb + lo, codes);
    } else {
        for (int e = 0; e < valid; ++e) {
            Wb[lo + e] = w[e];
            Mb[lo + e] = m[e];
            Vb[lo + e] = v[e];
            wqb[lo + e] = static_cast<int8_t>((codes >> (8 * e)) & 0xFFu);
        }
    }
}

// With DC the constants come from dc (device memory) instead of c.
template <int TPB, int NDP, bool OVF, bool SSQ, bool DC>
__global__ void __launch_bounds__(TPB)
step_q8_kernel(const int8_t *__restrict__ gq, const float *__restrict__ gs, int64_t ld,
               int64_t sld, int n_dp, int64_t len, int64_t nblocks, float *__restrict__ W,
               float *__restrict__ M, float *__restrict__ V, int8_t *__restrict__ wq,
               float *__restrict__ wsc, Consts c, uint32_t *__restrict__ ovf,
               double *__restrict__ part, const zero_step_consts *__restrict__ dc) {
    bool held = false;
    if constexpr (DC) {
        c = consts_of(*dc);
        held = step_held(c);
    }
    bool bad = held;
    double ss = 0.0;
    const int64_t b = held ? nblocks : wave_block<TPB>();  // a held step touches no block
    if constexpr (NDP > 0) {
        if (b < nblocks) {  // wave-uniform
            if ((b + 1) * kB <= len)  // wave-uniform: the whole block in the range
                step_q8_block<NDP, OVF, SSQ, true>(gq, gs, ld, sld, len, b, W, M, V, wq, wsc, c,
                                                   bad, ss);
            else
                step_q8_block<NDP, OVF, SSQ, false>(gq, gs, ld, sld, len, b, W, M, V, wq, wsc, c,
                                                    bad, ss);
        }
    } else if (b < nblocks) {  // any row count: rows in batches, as loaded
        const int lane = static_cast<int>(threadIdx.x) % kWave;
        const int64_t e0 = b * kB + lane * kQuad;
        const bool block_full = (b + 1) * kB <= len;  // wave-uniform
        const int valid = e0 + kQuad <= len ? kQuad : (e0 < len ? static_cast<int>(len - e0) : 0);
        float a[kQuad] = {0.0f, 0.0f, 0.0f, 0.0f};
        float w[kQuad] = {0.0f, 0.0f, 0.0f, 0.0f};
        float m[kQuad] = {0.0f, 0.0f, 0.0f, 0.0f};
        float v[kQuad] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (block_full) load_state<true>(w, m, v, e0, valid, W, M, V);
        else load_state<false>(w, m, v, e0, valid, W, M, V);
        loads_issued();
        uint32_t cr[kRowBatchQ8];
        float sr[kRowBatchQ8];
        for (int k0 = 0; k0 < n_dp; k0 += kRowBatchQ8) {
            const int cnt = n_dp - k0 < kRowBatchQ8 ? n_dp - k0 : kRowBatchQ8;
#pragma unroll
            for (int k = 0; k < kRowBatchQ8; ++k) {
                if (k < cnt) {
                    cr[k] = row_codes(gq + (k0 + k) * ld + e0, valid == kQuad, valid);
                    sr[k] = gs[(k0 + k) * sld + b];
                }
            }
            add_code_rows<kRowBatchQ8>(a, cr, sr, cnt, k0 == 0);
        }
#pragma unroll
        for (int e = 0; e < kQuad; ++e) {
            if (e < valid) {
                if constexpr (OVF) bad |= !__builtin_isfinite(a[e]);
                const float g = a[e] * c.s;
                if constexpr (SSQ) ss += static_cast<double>(g) * static_cast<double>(g);
                adamw_element(g, w[e], m[e], v[e], c);
            } else {
                w[e] = 0.0f;  // outside the range: no part of the block's scale
            }
        }
        const BlockScale bs = block_scale(w);
        const uint32_t codes = quantize4(w, bs);
        if (lane == 0) wsc[b] = bs.s;
        if (block_full) {
            store16(W + e0, f32x4{w[0], w[1], w[2], w[3]});
            store16(M + e0, f32x4{m[0], m[1], m[2], m[3]});
            store16(V + e0, f32x4{v[0], v[1], v[2], v[3]});
            store_codes(wq + e0, codes);
        } else {
            for (int e = 0; e < valid; ++e) {
                W[e0 + e] = w[e];
                M[e0 + e] = m[e];
                V[e0 + e] = v[e];
                wq[e0 + e] = static_cast<int8_t>((codes >> (8 * e)) & 0xFFu);
            }
        }
    }
    flags_epilogue<TPB, OVF, SSQ>(bad, ss, ovf, part);
}

// ---------------------------------------------------------------------------
// host side

template <int V>
using IntC = std::integral_constant<int, V>;
template <bool V>
using BoolC = std::integral_constant<bool, V>;

template <typename F>
void with_xdt(int dt, F &&f) {
    if (dt == ZERO_BF16) f(IntC<ZERO_BF16>{});
    else if (dt == ZERO_FP16) f(IntC<ZERO_FP16>{});
    else f(IntC<ZERO_FP32>{});
}

template <typename F>
void with_bool(bool b, F &&f) {
    if (b) f(BoolC<true>{});
    else f(BoolC<false>{});
}

bool xdt_ok(int dt) { return dt == ZERO_BF16 || dt == ZERO_FP16 || dt == ZERO_FP32; }
int64_t xdt_bytes(int dt) { return dt == ZERO_FP32 ? 4 : 2; }
int64_t blocks_of(int64_t len) { return (len + kB - 1) / kB; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool quad_aligned(const void *p, int dt) { return dt == ZERO_FP32 ? aligned16(p) : aligned8(p); }

// any two of the spans overlap
bool spans_overlap(const Span *s, int n) {
    for (int i = 0; i < n; ++i)
        for (int j = i + 1; j < n; ++j)
            if (overlap(s[i], s[j])) return true;
    return false;
}

// the launch grid of a one-shot kernel of `blocks` waves, tpb threads each
unsigned grid_waves(int64_t blocks, int tpb) {
    const int64_t per = tpb / kWave;
    return static_cast<unsigned>((blocks + per - 1) / per);
}

// [0, len) in launches of at most kLaunchElems elements (a multiple of the
// block): f(first element, elements) issues one
template <typename F>
void for_launches(int64_t len, F &&f) {
    static_assert(kLaunchElems % kB == 0, "launch pieces hold whole blocks");
    for (int64_t o = 0; o < len; o += kLaunchElems) f(o, len - o < kLaunchElems ? len - o : kLaunchElems);
}

}  // namespace

extern "C" zero_status zero_q8_quantize(const void *x, zero_dtype xdt, int64_t len, int8_t *q,
                                        float *scales, void *stream) {
    if (!xdt_ok(xdt) || len < 0 || len > kMaxLen) return ZERO_EINVAL;
    if (len == 0) return ZERO_OK;
    if (!x || !q || !scales) return ZERO_EINVAL;
    const Span sp[3] = {span_of(x, len, xdt_bytes(xdt)), span_of(q, len, 1),
                        span_of(scales, blocks_of(len), 4)};
    if (spans_overlap(sp, 3)) return ZERO_EALIAS;
    const bool vec = quad_aligned(x, xdt) && aligned4(q);
    const size_t lds = residency_lds_bytes(kQ8QuantizeWavesPerCU, kWave);
    hipStream_t st = static_cast<hipStream_t>(stream);
    with_xdt(xdt, [&](auto XD) {
        using E = typename GradT<XD.value>::elem;
        with_bool(vec, [&](auto VC) {
            for_launches(len, [&](int64_t o, int64_t n) {
                const int64_t nb = blocks_of(n);
                q8_quantize_kernel<XD.value, VC.value, kQ8QuantizeBlocks>
                    <<<grid_waves((nb + kQ8QuantizeBlocks - 1) / kQ8QuantizeBlocks, kWave), kWave,
                       lds, st>>>(static_cast<const E *>(x) + o, n, q + o, scales + o / kB);
            });
        });
    });
    return launch_status();
}

extern "C" zero_status zero_q8_dequantize(const int8_t *q, const float *scales, int64_t len,
                                          void *y, zero_dtype ydt, void *stream) {
    if (!xdt_ok(ydt) || len < 0 || len > kMaxLen) return ZERO_EINVAL;
    if (len == 0) return ZERO_OK;
    if (!y || !q || !scales) return ZERO_EINVAL;
    const Span sp[3] = {span_of(y, len, xdt_bytes(ydt)), span_of(q, len, 1),
                        span_of(scales, blocks_of(len), 4)};
    if (spans_overlap(sp, 3)) return ZERO_EALIAS;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (ydt == ZERO_FP32) {
        const bool vec = aligned16(y) && aligned4(q);
        const size_t lds = residency_lds_bytes(kQ8DequantizeF32WavesPerCU, kWave);
        constexpr int64_t kQ = kQ8DequantizeF32Blocks;
        with_bool(vec, [&](auto VC) {
            for_launches(len, [&](int64_t o, int64_t n) {
                q8_dequantize_kernel<ZERO_FP32, VC.value, kQ>
                    <<<grid_waves((blocks_of(n) + kQ - 1) / kQ, kWave), kWave, lds, st>>>(
                        q + o, scales + o / kB, n, static_cast<float *>(y) + o);
            });
        });
        return launch_status();
    }
    const size_t lds = residency_lds_bytes(kQ8DequantizeWavesPerCU, kWave);
    // 16-bit values: 8-byte code loads and 16-byte stores
    const bool vec = aligned16(y) && aligned8(q);
    with_xdt(ydt, [&](auto YD) {
        if constexpr (YD.value != ZERO_FP32) {
            with_bool(vec, [&](auto VC) {
                for_launches(len, [&](int64_t o, int64_t n) {
                    q8_dequantize_pair_kernel<YD.value, VC.value>
                        <<<grid_waves((blocks_of(n) + 1) / 2, kWave), kWave, lds, st>>>(
                            q + o, scales + o / kB, n, static_cast<uint16_t *>(y) + o);
                });
            });
        }
    });
    return launch_status();
}

namespace {

zero_status step_q8_impl(const int8_t *gq, const float *gscales, int64_t ld, int64_t sld,
                         int64_t len, float *master, float *m, float *v, int8_t *wq_full,
                         float *wscales_full, const zero_layout *layout, int32_t rank,
                         int64_t shard_off, const zero_adamw_hparams *hp,
                         const zero_step_consts *dc, uint32_t *overflow, double *sumsq,
                         void *workspace, int64_t workspace_bytes, void *stream) {
    if (!layout_ok(layout) || !(dc ? aligned8(dc) : hparams_ok(hp))) return ZERO_EINVAL;
    const int n_dp = layout->n_dp;
    if (rank < 0 || rank >= n_dp || shard_off < 0 || len < 0 || len > kMaxLen || ld < len)
        return ZERO_EINVAL;
    if (layout->shard % kB != 0 || shard_off % kB != 0) return ZERO_EINVAL;
    const int64_t nb = blocks_of(len);
    if (n_dp > 1 && (ld % kQuad != 0 || sld < nb)) return ZERO_EINVAL;
    if (n_dp > 1 && (!rows_ok(n_dp, ld, len) || !rows_ok(n_dp, sld, nb))) return ZERO_EINVAL;
    if (shard_off > layout->shard || len > layout->shard - shard_off) return ZERO_ERANGE;
    if (len == 0) return ZERO_OK;
    if (!gq || !gscales || !master || !m || !v || !wq_full || !wscales_full) return ZERO_EINVAL;
    if (sumsq && (!workspace || !aligned8(workspace) ||
                  workspace_bytes < zero_sumsq_workspace_bytes(len)))
        return ZERO_EINVAL;
    const int64_t first = static_cast<int64_t>(rank) * layout->shard + shard_off;
    int8_t *wq = wq_full + first;
    float *wsc = wscales_full + first / kB;
    if (!aligned4(gq) || !aligned4(wq) || !aligned16(master) || !aligned16(m) || !aligned16(v))
        return ZERO_EINVAL;
    // outputs pairwise disjoint, and disjoint from every code and scale row
    Span outs[9];
    int n_out = 0;
    outs[n_out++] = span_of(master, len, 4);
    outs[n_out++] = span_of(m, len, 4);
    outs[n_out++] = span_of(v, len, 4);
    outs[n_out++] = span_of(wq, len, 1);
    outs[n_out++] = span_of(wsc, nb, 4);
    if (overflow) outs[n_out++] = span_of(overflow, 1, 4);
    if (sumsq) outs[n_out++] = span_of(sumsq, 1, 8);
    if (sumsq) outs[n_out++] = span_of(workspace, workspace_bytes, 1);
    if (spans_overlap(outs, n_out)) return ZERO_EALIAS;
    for (int i = 0; i < n_out; ++i) {
        if (dc && overlap(outs[i], span_of(dc, 1, sizeof(zero_step_consts)))) return ZERO_EALIAS;
        for (int k = 0; k < n_dp; ++k) {
            if (overlap(outs[i], span_of(gq + static_cast<int64_t>(k) * ld, len, 1)) ||
                overlap(outs[i], span_of(gscales + static_cast<int64_t>(k) * sld, nb, 4)))
                return ZERO_EALIAS;
        }
    }

    hipStream_t st = static_cast<hipStream_t>(stream);
    const Consts c = dc ? Consts{} : make_consts(*hp);
    // with a sum of squares each wave (one block) stores its partial
    double *part = sumsq ? ssq_partials(workspace) : nullptr;
    with_bool(overflow != nullptr, [&](auto OV) {
        with_bool(sumsq != nullptr, [&](auto SS) {
            with_bool(dc != nullptr, [&](auto DV) {
                const size_t lds = residency_lds_bytes(kQ8StepWavesPerCU, kWave);
                auto go = [&](auto ND) {
                    for_launches(len, [&](int64_t o, int64_t n) {
                        const int64_t ob = o / kB, nbn = blocks_of(n);
                        step_q8_kernel<kWave, ND.value, OV.value, SS.value, DV.value>
                            <<<grid_waves(nbn, kWave), kWave, lds, st>>>(
                                gq + o, gscales + ob, ld, sld, n_dp, n, nbn, master + o, m + o,
                                v + o, wq + o, wsc + ob, c, overflow,
                                SS.value ? part + ob : nullptr, dc);
                    });
                };
                if (n_dp == 1) go(IntC<1>{});
                else if (n_dp == 8) go(IntC<8>{});
                else go(IntC<0>{});
            });
        });
    });
    if (sumsq) {
        const zero_status s1 = launch_status();
        if (s1 != ZERO_OK) return s1;
        return finish_sumsq(workspace, nb, sumsq, st);
    }
    return launch_status();
}

}  // namespace

extern "C" zero_status zero_shard_step_q8(const int8_t *gq, const float *gscales, int64_t ld,
                                          int64_t sld, int64_t len, float *master, float *m,
                                          float *v, int8_t *wq_full, float *wscales_full,
                                          const zero_layout *layout, int32_t rank,
                                          int64_t shard_off, const zero_adamw_hparams *hp,
                                          uint32_t *overflow, double *sumsq, void *workspace,
                                          int64_t workspace_bytes, void *stream) {
    return step_q8_impl(gq, gscales, ld, sld, len, master, m, v, wq_full, wscales_full, layout,
                        rank, shard_off, hp, nullptr, overflow, sumsq, workspace,
                        workspace_bytes, stream);
}

extern "C" zero_status zero_shard_step_q8_dc(const int8_t *gq, const float *gscales,
                                             int64_t ld, int64_t sld, int64_t len,
                                             float *master, float *m, float *v, int8_t *wq_full,
                                             float *wscales_full, const zero_layout *layout,
                                             int32_t rank, int64_t shard_off,
                                             const zero_step_consts *consts, uint32_t *overflow,
                                             double *sumsq, void *workspace,
                                             int64_t workspace_bytes, void *stream) {
    if (!consts) return ZERO_EINVAL;
    return step_q8_impl(gq, gscales, ld, sld, len, master, m, v, wq_full, wscales_full, layout,
                        rank, shard_off, nullptr, consts, overflow, sumsq, workspace,
                        workspace_bytes, stream);
}
