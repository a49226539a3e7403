// host_common.h -- host-side helpers shared by the library's HIP sources
// (internal: not installed, not part of the C ABI).
#ifndef ZERO_SHARD_HOST_COMMON_H
#define ZERO_SHARD_HOST_COMMON_H

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "zero_shard.h"

namespace zero_host {

constexpr int kWave = 64;  // wave64

// byte ranges, for the disjointness checks
struct Span {
    uintptr_t lo, hi;
};

inline Span span_of(const void *p, int64_t count, int64_t elem) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Span{lo, lo + static_cast<uintptr_t>(count) * static_cast<uintptr_t>(elem)};
}

inline bool overlap(const Span &a, const Span &b) {
    return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned8(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

// Dynamic LDS requested by a streaming kernel of tpb threads per workgroup
// so that about waves_per_cu of its waves are resident on a CU (the LDS
// itself is unused).
inline size_t residency_lds_bytes(int waves_per_cu, int tpb) {
    const int wave_per_wg = tpb / kWave;
    int wg_per_cu = (waves_per_cu + wave_per_wg / 2) / wave_per_wg;
    if (wg_per_cu < 1) wg_per_cu = 1;
    int dev = 0, per_cu = 0, per_block = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                              dev) != hipSuccess ||
        hipDeviceGetAttribute(&per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
            hipSuccess)
        return 0;
    // leave 1 KiB per workgroup for the kernels' own static LDS
    int64_t b = (static_cast<int64_t>(per_cu) / wg_per_cu - 1024) & ~int64_t(255);
    if (b > per_block) b = per_block & ~255;
    return b > 0 ? static_cast<size_t>(b) : 0;
}

inline zero_status launch_status() {
    return hipGetLastError() == hipSuccess ? ZERO_OK : ZERO_EDEVICE;
}

}  // namespace zero_host

#endif
