// flat_copy.hip -- gfx950 kernel and entry points that move ranges of the
// flat parameter vector between its pieces.
//
// "ZeRO Optimizer, in depth", "Checkpoints: sharded on the way in,
// consolidated on the way out": each rank writes its own shards, a
// checkpoint is therefore tied to its layout, and resuming on another
// number of GPUs (one of that page's failure modes) or consolidating into
// per-parameter tensors needs every flat element moved to its new place.
// Flattening parameter tensors into a rank's shard ("ZeRO and FSDP", "The
// idea, one stage at a time") is the same operation in the other direction.
// All of these are bitwise copies of flat ranges between pieces of the flat
// vector, with zeros where no piece holds an index.
//
// The host turns a request into copy segments (a source byte range, or
// zeros, and a destination byte range) and launches them in batches, the
// segment table passed by value.  Each lane owns aligned 16-byte chunks of
// the destination, so every store is a full 16-byte store and a wave's store
// instruction covers one contiguous 1 KiB span; a segment's first and last
// chunks, which the segment covers only in part, are written 2 bytes at a
// time.  The source side depends on its phase, (src - dst) mod 16, uniform
// over a segment:
//  - phase 0 (the usual case: shard boundaries of layouts whose shard is a
//    multiple of 16 bytes): one 16-byte load per chunk;
//  - any other (even) phase: the two aligned 16-byte source chunks that
//    straddle the wanted bytes are loaded and the 16 bytes are extracted
//    with byte funnel shifts (v_alignbyte_b32), each phase a compiled case;
//    a chunk whose straddling source chunks would leave the source range
//    takes the 2-byte path instead, so no access leaves a segment.
// Nothing is re-read, so loads and stores are non-temporal, except the
// shifted loads, where neighbouring lanes share a source chunk.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <vector>

#include "host_common.h"
#include "zero_shard.h"

namespace {

using namespace zero_host;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 16;          // bytes per chunk
constexpr int kCopyChunks = 4;      // chunks per lane, a wave's 1 KiB apart
constexpr int kCopyWavesPerCU = 16; // residency cap of the copy kernel (measured)
constexpr int kMaxSegs = 64;        // segments per launch (by-value table)
constexpr int64_t kMaxLen = int64_t(1) << 38;
// A dispatch counts its grid in work-items in 32 bits: one launch takes at
// most kMaxCopyBlocks one-wave workgroups (2^31 work-items), and a copy
// longer than kCopyPieceBytes goes in as several segments (a multiple of the
// chunk, so each keeps the copy's alignment phase).
constexpr int64_t kMaxCopyBlocks = (int64_t(1) << 31) / kWave;
constexpr int64_t kCopyPieceBytes = int64_t(1) << 32;

struct Seg {
    const unsigned char *src;  // nullptr: the segment is zero-filled
    unsigned char *dst;
    int64_t bytes;             // even, > 0
    int64_t first_block;       // workgroups of the earlier segments
};

struct SegTable {
    Seg s[kMaxSegs];
    int32_t n;
};

__device__ __forceinline__ u32x4 load_nt(const unsigned char *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ u32x4 load_plain(const unsigned char *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}
// non-temporal at device scope (nt sc1), as the step's streaming stores;
// written out, so it carries the two wait states a store of more than 64
// bits of data needs before its registers may be overwritten
__device__ __forceinline__ void store_nt(unsigned char *p, u32x4 x) {
    asm volatile("global_store_dwordx4 %0, %1, off nt sc1\n\ts_nop 1" : : "v"(p), "v"(x)
                 : "memory");
}

// bytes [P, P + 16) of the 32 bytes lo:hi (little-endian)
template <int P>
__device__ __forceinline__ u32x4 funnel(u32x4 lo, u32x4 hi) {
    constexpr int q = P >> 2, r = P & 3;
    const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        o[i] = r == 0 ? w[i + q] : __builtin_amdgcn_alignbyte(w[i + q + 1], w[i + q], r);
    return o;
}

// The bytes of chunk x that the segment [d0, d1) covers, 2 at a time.
__device__ __noinline__ void copy_partial(const unsigned char *src, uintptr_t d0, uintptr_t d1,
                                          uintptr_t x) {
    const uintptr_t lo = x > d0 ? x : d0;
    const uintptr_t hi = x + kChunk < d1 ? x + kChunk : d1;
    for (uintptr_t y = lo; y < hi; y += 2) {
        const uint16_t val = src ? *reinterpret_cast<const uint16_t *>(src + (y - d0)) : 0;
        *reinterpret_cast<uint16_t *>(y) = val;
    }
}

// One workgroup's chunks of one segment with source phase P (P < 0: zeros).
template <int CH, int P>
__device__ __forceinline__ void copy_chunks(const unsigned char *src, uintptr_t d0, uintptr_t d1,
                                            uintptr_t first) {
    uintptr_t x[CH];
    bool full[CH];
    u32x4 val[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        x[i] = first + static_cast<uintptr_t>(i) * kWave * kChunk;
        full[i] = x[i] >= d0 && x[i] + kChunk <= d1;
        if constexpr (P > 0) {
            // the straddling aligned source chunks must lie in the source
            const uintptr_t s0 = reinterpret_cast<uintptr_t>(src);
            const uintptr_t a = s0 + (x[i] - d0) - P;
            full[i] = full[i] && a >= s0 && a + 2 * kChunk <= s0 + (d1 - d0);
        }
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        if constexpr (P < 0) {
            val[i] = u32x4{0u, 0u, 0u, 0u};
        } else if constexpr (P == 0) {
            if (full[i]) val[i] = load_nt(src + (x[i] - d0));
        } else {
            if (full[i]) {
                const unsigned char *a = src + (x[i] - d0) - P;
                val[i] = funnel<P>(load_plain(a), load_plain(a + kChunk));
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);  // every load issued before the first store
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        if (full[i]) store_nt(reinterpret_cast<unsigned char *>(x[i]), val[i]);
        else if (x[i] < d1) copy_partial(src, d0, d1, x[i]);
    }
}

template <int CH>
__global__ __launch_bounds__(kWave) void flat_copy_kernel(const SegTable t) {
    const int64_t b = blockIdx.x;
    // the segment this workgroup belongs to: the last with first_block <= b
    int lo = 0, hi = t.n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (t.s[mid].first_block <= b) lo = mid;
        else hi = mid - 1;
    }
    const unsigned char *src = t.s[lo].src;
    const uintptr_t d0 = reinterpret_cast<uintptr_t>(t.s[lo].dst);
    const uintptr_t d1 = d0 + static_cast<uintptr_t>(t.s[lo].bytes);
    const uintptr_t first =
        (d0 & ~uintptr_t(kChunk - 1)) +
        (static_cast<uintptr_t>(b - t.s[lo].first_block) * (kWave * CH) + threadIdx.x) * kChunk;
    if (!src) {
        copy_chunks<CH, -1>(src, d0, d1, first);
        return;
    }
    switch (static_cast<int>((reinterpret_cast<uintptr_t>(src) - d0) & (kChunk - 1))) {
    case 0: copy_chunks<CH, 0>(src, d0, d1, first); break;
    case 2: copy_chunks<CH, 2>(src, d0, d1, first); break;
    case 4: copy_chunks<CH, 4>(src, d0, d1, first); break;
    case 6: copy_chunks<CH, 6>(src, d0, d1, first); break;
    case 8: copy_chunks<CH, 8>(src, d0, d1, first); break;
    case 10: copy_chunks<CH, 10>(src, d0, d1, first); break;
    case 12: copy_chunks<CH, 12>(src, d0, d1, first); break;
    default: copy_chunks<CH, 14>(src, d0, d1, first); break;  // 14 (phases are even)
    }
}

// ---------------------------------------------------------------------------
// host side

struct Copy {
    const unsigned char *src;  // nullptr: zeros
    unsigned char *dst;
    int64_t bytes;
};

int64_t chunks_of(const Copy &c) {
    const uintptr_t d0 = reinterpret_cast<uintptr_t>(c.dst);
    const uintptr_t d1 = d0 + static_cast<uintptr_t>(c.bytes);
    return static_cast<int64_t>(((d1 + kChunk - 1) / kChunk) - (d0 / kChunk));
}

template <int CH>
zero_status launch_copies(const std::vector<Copy> &cs, int waves_per_cu, hipStream_t st) {
    const size_t lds = residency_lds_bytes(waves_per_cu, kWave);
    SegTable t;
    t.n = 0;
    int64_t blocks = 0;
    auto flush = [&]() -> bool {
        if (t.n == 0) return true;
        flat_copy_kernel<CH><<<static_cast<unsigned>(blocks), kWave, lds, st>>>(t);
        t.n = 0;
        blocks = 0;
        return hipGetLastError() == hipSuccess;
    };
    for (const Copy &whole : cs) {
        for (int64_t off = 0; off < whole.bytes; off += kCopyPieceBytes) {
            const Copy c{whole.src ? whole.src + off : nullptr, whole.dst + off,
                         std::min(kCopyPieceBytes, whole.bytes - off)};
            const int64_t nb = (chunks_of(c) + kWave * CH - 1) / (kWave * CH);
            if (t.n == kMaxSegs || blocks + nb > kMaxCopyBlocks) {
                if (!flush()) return ZERO_EDEVICE;
            }
            t.s[t.n++] = Seg{c.src, c.dst, c.bytes, blocks};
            blocks += nb;
        }
    }
    return flush() ? ZERO_OK : ZERO_EDEVICE;
}

bool elem_ok(int32_t eb) { return eb == 2 || eb == 4; }

bool ptr_aligned(const void *p, int32_t eb) {
    return (reinterpret_cast<uintptr_t>(p) & static_cast<uintptr_t>(eb - 1)) == 0;
}

// a piece's fields are in range and its pointer usable
bool piece_ok(const zero_piece &p, int32_t eb) {
    if (p.flat_off < 0 || p.len < 0 || p.len > INT64_MAX / 4) return false;
    if (p.flat_off > INT64_MAX - p.len) return false;
    if (p.len > 0 && (!p.ptr || !ptr_aligned(p.ptr, eb))) return false;
    return true;
}

// the non-empty pieces sorted by flat_off; false when two overlap in index
bool sorted_disjoint(const zero_piece *ps, int32_t n, std::vector<const zero_piece *> &out) {
    out.clear();
    for (int32_t k = 0; k < n; ++k)
        if (ps[k].len > 0) out.push_back(&ps[k]);
    std::sort(out.begin(), out.end(), [](const zero_piece *a, const zero_piece *b) {
        return a->flat_off < b->flat_off;
    });
    for (size_t k = 1; k < out.size(); ++k)
        if (out[k]->flat_off < out[k - 1]->flat_off + out[k - 1]->len) return false;
    return true;
}

bool range_ok(int64_t begin, int64_t count) {
    return begin >= 0 && count >= 0 && count <= kMaxLen && begin <= INT64_MAX - count;
}

zero_status gather_impl(const zero_piece *src, int32_t n_src, int64_t n, int32_t eb,
                        int64_t begin, int64_t count, void *dst, hipStream_t st) {
    if (!elem_ok(eb) || n_src < 0 || n < 0 || !range_ok(begin, count)) return ZERO_EINVAL;
    if (n_src > 0 && !src) return ZERO_EINVAL;
    for (int32_t k = 0; k < n_src; ++k)
        if (!piece_ok(src[k], eb)) return ZERO_EINVAL;
    std::vector<const zero_piece *> sorted;
    if (!sorted_disjoint(src, n_src, sorted)) return ZERO_EINVAL;
    if (count == 0) return ZERO_OK;
    if (!dst || !ptr_aligned(dst, eb)) return ZERO_EINVAL;
    const Span out = span_of(dst, count, eb);
    for (const zero_piece *p : sorted)
        if (overlap(out, span_of(p->ptr, p->len, eb))) return ZERO_EALIAS;

    unsigned char *d = static_cast<unsigned char *>(dst);
    const int64_t end = begin + count;
    const int64_t valid_end = std::min(end, std::max(n, begin));
    std::vector<Copy> cs;
    int64_t cur = begin;  // flat index up to which dst is planned
    for (const zero_piece *p : sorted) {
        const int64_t lo = std::max(p->flat_off, begin);
        const int64_t hi = std::min(p->flat_off + p->len, valid_end);
        if (hi <= lo) continue;
        if (lo > cur) cs.push_back(Copy{nullptr, d + (cur - begin) * eb, (lo - cur) * eb});
        cs.push_back(Copy{static_cast<const unsigned char *>(p->ptr) + (lo - p->flat_off) * eb,
                          d + (lo - begin) * eb, (hi - lo) * eb});
        cur = hi;
    }
    if (cur < end) cs.push_back(Copy{nullptr, d + (cur - begin) * eb, (end - cur) * eb});
    return launch_copies<kCopyChunks>(cs, kCopyWavesPerCU, st);
}

}  // namespace

extern "C" zero_status zero_flat_gather(const zero_piece *src, int32_t n_src, int64_t n,
                                        int32_t elem_bytes, int64_t begin, int64_t count,
                                        void *dst, void *stream) {
    return gather_impl(src, n_src, n, elem_bytes, begin, count, dst,
                       static_cast<hipStream_t>(stream));
}

extern "C" zero_status zero_flat_scatter(const void *src, int64_t begin, int64_t count,
                                         const zero_piece *dst, int32_t n_dst,
                                         int32_t elem_bytes, void *stream) {
    if (!elem_ok(elem_bytes) || n_dst < 0 || !range_ok(begin, count)) return ZERO_EINVAL;
    if (n_dst > 0 && !dst) return ZERO_EINVAL;
    const int32_t eb = elem_bytes;
    for (int32_t k = 0; k < n_dst; ++k)
        if (!piece_ok(dst[k], eb)) return ZERO_EINVAL;
    std::vector<const zero_piece *> sorted;
    if (!sorted_disjoint(dst, n_dst, sorted)) return ZERO_EINVAL;
    if (count == 0) return ZERO_OK;
    if (!src || !ptr_aligned(src, eb)) return ZERO_EINVAL;
    // outputs pairwise disjoint in memory, and none overlapping the input
    std::vector<Span> spans;
    for (const zero_piece *p : sorted) spans.push_back(span_of(p->ptr, p->len, eb));
    std::sort(spans.begin(), spans.end(), [](const Span &a, const Span &b) { return a.lo < b.lo; });
    for (size_t k = 1; k < spans.size(); ++k)
        if (overlap(spans[k - 1], spans[k])) return ZERO_EALIAS;
    const Span in = span_of(src, count, eb);
    for (const Span &s : spans)
        if (overlap(in, s)) return ZERO_EALIAS;

    const unsigned char *s = static_cast<const unsigned char *>(src);
    const int64_t end = begin + count;
    std::vector<Copy> cs;
    for (const zero_piece *p : sorted) {
        const int64_t lo = std::max(p->flat_off, begin);
        const int64_t hi = std::min(p->flat_off + p->len, end);
        if (hi <= lo) continue;
        cs.push_back(Copy{s + (lo - begin) * eb,
                          static_cast<unsigned char *>(p->ptr) + (lo - p->flat_off) * eb,
                          (hi - lo) * eb});
    }
    return launch_copies<kCopyChunks>(cs, kCopyWavesPerCU, static_cast<hipStream_t>(stream));
}

extern "C" zero_status zero_reshard(const void *const *src_shards, int32_t n_src,
                                    int64_t src_shard, int64_t n, int32_t elem_bytes,
                                    int32_t dst_rank, int64_t dst_shard, void *dst,
                                    void *stream) {
    if (n_src < 1 || !src_shards || src_shard < 0 || dst_rank < 0 || dst_shard < 0)
        return ZERO_EINVAL;
    if (src_shard > 0 && n_src > INT64_MAX / src_shard) return ZERO_EINVAL;
    if (n < 0 || n > n_src * src_shard) return ZERO_EINVAL;
    if (dst_shard > 0 && dst_rank > INT64_MAX / dst_shard) return ZERO_EINVAL;
    std::vector<zero_piece> pieces(static_cast<size_t>(n_src));
    for (int32_t r = 0; r < n_src; ++r)
        pieces[r] = zero_piece{const_cast<void *>(src_shards[r]), r * src_shard, src_shard};
    return gather_impl(pieces.data(), n_src, n, elem_bytes, dst_rank * dst_shard, dst_shard, dst,
                       static_cast<hipStream_t>(stream));
}
