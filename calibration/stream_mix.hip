// stream_mix.hip -- measuring sticks for bench.py, not part of the library.
//
// The fused step of libzero_shard streams n_dp 16-bit gradient rows and the
// fp32 master, m and v in, and the fp32 master, m and v and a 16-bit weight
// slot out: 2 n_dp + 26 bytes per element.  mix_kernel moves exactly those
// bytes with the step's launch shape -- one quad (4 elements) per lane,
// one-wave workgroups, one-shot grid, every load issued before any store,
// the same cache policies (non-temporal loads; non-temporal stores at
// device scope, with the two wait states a store of more than 64 bits of
// data needs before its registers are reused), the same residency cap --
// and does no arithmetic:
// the state is stored back as loaded and the slot gets the XOR of the
// rows' bits.  Its time is the ceiling of that access pattern on this GPU,
// against which the step's own time is reported.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kWave = 64;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void store16(float *p, f32x4 x) {
    asm volatile("global_store_dwordx4 %0, %1, off nt sc1\n\ts_nop 1" : : "v"(p), "v"(x)
                 : "memory");
}
__device__ __forceinline__ void store8(uint16_t *p, u32x2 x) {
    asm volatile("global_store_dwordx2 %0, %1, off nt sc1" : : "v"(p), "v"(x) : "memory");
}

template <int NDP>
__global__ void __launch_bounds__(kWave)
mix_kernel(const uint16_t *__restrict__ rows, int64_t ld, int64_t nquad, float *__restrict__ W,
           float *__restrict__ M, float *__restrict__ V, uint16_t *__restrict__ out) {
    const int64_t q = static_cast<int64_t>(blockIdx.x) * kWave + threadIdx.x;
    if (q >= nquad) return;
    const int64_t e0 = q * 4;
    u32x2 r[NDP];
#pragma unroll
    for (int k = 0; k < NDP; ++k)
        r[k] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x2 *>(rows + static_cast<int64_t>(k) * ld + e0));
    const f32x4 w = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(W + e0));
    const f32x4 m = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(M + e0));
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(V + e0));
    __builtin_amdgcn_sched_barrier(0);
    // opaque to the compiler, so that storing a value back where it was
    // loaded is not dropped as a no-op
    f32x4 w2 = w, m2 = m, v2 = v;
    asm volatile("" : "+v"(w2), "+v"(m2), "+v"(v2));
    u32x2 x = r[0];
#pragma unroll
    for (int k = 1; k < NDP; ++k) x ^= r[k];
    store16(W + e0, w2);
    store16(M + e0, m2);
    store16(V + e0, v2);
    store8(out + e0, x);
}

// dynamic LDS (otherwise unused) that leaves room for about waves_per_cu
// one-wave workgroups on a CU
size_t residency_lds_bytes(int waves_per_cu) {
    int dev = 0, per_cu = 0, per_block = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                              dev) != hipSuccess ||
        hipDeviceGetAttribute(&per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
            hipSuccess)
        return 0;
    int64_t b = (static_cast<int64_t>(per_cu) / (waves_per_cu < 1 ? 1 : waves_per_cu) - 1024) &
                ~int64_t(255);
    if (b > per_block) b = per_block & ~255;
    return b > 0 ? static_cast<size_t>(b) : 0;
}

template <int NDP>
int launch(const uint16_t *rows, int64_t ld, int64_t len, float *W, float *M, float *V,
           uint16_t *out, int waves_per_cu, hipStream_t st) {
    const int64_t nquad = len / 4;
    const int64_t per = (int64_t(1) << 31) / 4;  // a dispatch counts work-items in 32 bits
    const size_t lds = residency_lds_bytes(waves_per_cu);
    for (int64_t q0 = 0; q0 < nquad; q0 += per) {
        const int64_t nq = nquad - q0 < per ? nquad - q0 : per;
        const int64_t o = q0 * 4;
        mix_kernel<NDP><<<static_cast<unsigned>((nq + kWave - 1) / kWave), kWave, lds, st>>>(
            rows + o, ld, nq, W + o, M + o, V + o, out + o);
    }
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace

// rows: n_dp bf16 rows of stride ld; W, M, V: fp32[len]; out: 16-bit[len];
// len a multiple of 4, every pointer 16-byte aligned (rows 8-byte, ld % 4
// == 0).  Returns 0, or 1 for an unsupported row count or a bad argument.
extern "C" __attribute__((visibility("default"))) int stream_mix(
    const void *rows, int32_t n_dp, int64_t ld, int64_t len, float *W, float *M, float *V,
    void *out, int32_t waves_per_cu, void *stream) {
    if (!rows || !W || !M || !V || !out || len < 0 || len % 4 != 0 || ld < len || ld % 4 != 0)
        return 1;
    const uint16_t *r = static_cast<const uint16_t *>(rows);
    uint16_t *o = static_cast<uint16_t *>(out);
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (n_dp) {
    case 1: return launch<1>(r, ld, len, W, M, V, o, waves_per_cu, st);
    case 8: return launch<8>(r, ld, len, W, M, V, o, waves_per_cu, st);
    case 64: return launch<64>(r, ld, len, W, M, V, o, waves_per_cu, st);
    default: return 1;
    }
}
