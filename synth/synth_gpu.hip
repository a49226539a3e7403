// synth_gpu.hip -- device build of the seeded input generator (see
// synth_core.h): fills a device buffer with the same values the host build
// produces, so large inputs never have to cross PCIe.  It draws inputs only.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "synth_core.h"

template <int KIND>
__global__ void __launch_bounds__(256)
syn_fill_kernel(uint64_t key, int64_t start, int64_t count, double sigma, uint32_t thr,
                double mul, const double *__restrict__ table, void *__restrict__ out) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < count; o += stride) {
        double v = syn_value(table, syn_bits(key, (uint64_t)(start + o)), sigma, thr, mul);
        float f = (float)v;
        if (KIND == SYN_F32)
            static_cast<float *>(out)[o] = f;
        else if (KIND == SYN_BF16)
            static_cast<uint16_t *>(out)[o] = syn_trunc_bf16(f);
        else
            static_cast<uint16_t *>(out)[o] = syn_trunc_f16(f);
    }
}

// out[o] = value of element (start + o), o in [0, count).  `table` is the
// host table (SYN_TABLE_SIZE doubles) already copied to the device.
// Returns 0, -1 on bad arguments, or the HIP error code of the launch.
extern "C" int syn_gpu_fill(int kind, uint64_t seed, uint64_t tag, int64_t start,
                            int64_t count, double sigma, uint32_t thr, double mul,
                            const double *table, void *out, void *stream) {
    if (count < 0 || start < 0 || (count > 0 && (!table || !out))) return -1;
    if (count == 0) return 0;
    const uint64_t key = syn_key(seed, tag);
    const int64_t want = (count + 255) / 256;
    const unsigned blocks = (unsigned)(want < 65536 ? want : 65536);
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (kind) {
    case SYN_F32:
        syn_fill_kernel<SYN_F32><<<blocks, 256, 0, s>>>(key, start, count, sigma, thr, mul, table, out);
        break;
    case SYN_BF16:
        syn_fill_kernel<SYN_BF16><<<blocks, 256, 0, s>>>(key, start, count, sigma, thr, mul, table, out);
        break;
    case SYN_F16:
        syn_fill_kernel<SYN_F16><<<blocks, 256, 0, s>>>(key, start, count, sigma, thr, mul, table, out);
        break;
    default:
        return -1;
    }
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? 0 : (int)e;
}
