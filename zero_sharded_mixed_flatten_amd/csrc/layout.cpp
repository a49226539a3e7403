// layout.cpp -- host-only entry points of libzero_shard: the flat layout,
// the per-shard segment map, status strings and the memory/communication
// accounting.  Integer arithmetic only for the layout.
#include <cmath>
#include <cstdint>
#include <limits>

#include "zero_shard.h"

namespace {

constexpr int64_t kI64Max = std::numeric_limits<int64_t>::max();

bool layout_ok(const zero_layout *l) {
    if (!l || l->n_dp < 1 || l->align < 1 || l->shard < 0 || l->n < 0) return false;
    if (l->shard % l->align != 0) return false;
    if (l->shard > 0 && l->n_dp > kI64Max / l->shard) return false;
    return l->n_pad == l->shard * l->n_dp && l->n <= l->n_pad;
}

}  // namespace

extern "C" int32_t zero_abi_version(void) { return ZERO_SHARD_ABI_VERSION; }

extern "C" const char *zero_status_string(zero_status s) {
    switch (s) {
    case ZERO_OK: return "ZERO_OK";
    case ZERO_EINVAL: return "ZERO_EINVAL: invalid argument";
    case ZERO_EALIAS: return "ZERO_EALIAS: buffers that must be disjoint overlap";
    case ZERO_ERANGE: return "ZERO_ERANGE: range outside the shard or weight buffer";
    case ZERO_EDEVICE: return "ZERO_EDEVICE: kernel launch failed";
    }
    return "unknown zero_status";
}

// "ZeRO and FSDP" (Zero to Frontier 10.3), "The idea, one stage at a time":
// one vector of N numbers in n_dp equal contiguous shards, rank r owns shard
// r.  Equal shards of a vector whose length n_dp does not divide need a zero
// tail: shard = align * ceil(N / (n_dp * align)), n_pad = n_dp * shard.
extern "C" zero_status zero_flatten_layout(const int64_t *numels, int64_t n_tensors,
                                           int32_t n_dp, int64_t align, int64_t *offsets,
                                           zero_layout *out) {
    if (!out || n_tensors < 0 || n_dp < 1 || align < 1) return ZERO_EINVAL;
    if (n_tensors > 0 && !numels) return ZERO_EINVAL;
    int64_t total = 0;
    for (int64_t i = 0; i < n_tensors; ++i) {
        if (numels[i] < 0 || numels[i] > kI64Max - total) return ZERO_EINVAL;
        total += numels[i];
    }
    if (align > kI64Max / n_dp) return ZERO_EINVAL;
    const int64_t unit = align * n_dp;
    const int64_t units = total / unit + (total % unit != 0 ? 1 : 0);
    if (units > kI64Max / unit) return ZERO_EINVAL;
    if (offsets) {
        int64_t pos = 0;
        for (int64_t i = 0; i < n_tensors; ++i) {
            offsets[i] = pos;
            pos += numels[i];
        }
    }
    out->n = total;
    out->shard = units * align;
    out->n_pad = units * unit;
    out->align = align;
    out->n_dp = n_dp;
    out->reserved = 0;
    return ZERO_OK;
}

extern "C" zero_status zero_shard_segments(const zero_layout *layout, const int64_t *numels,
                                           int64_t n_tensors, int32_t rank, zero_segment *out,
                                           int64_t cap, int64_t *count) {
    if (!layout_ok(layout) || !count || n_tensors < 0 || cap < 0) return ZERO_EINVAL;
    if (n_tensors > 0 && !numels) return ZERO_EINVAL;
    if (cap > 0 && !out) return ZERO_EINVAL;
    if (rank < 0 || rank >= layout->n_dp) return ZERO_EINVAL;
    int64_t total = 0;
    for (int64_t i = 0; i < n_tensors; ++i) {
        if (numels[i] < 0 || numels[i] > kI64Max - total) return ZERO_EINVAL;
        total += numels[i];
    }
    if (total != layout->n) return ZERO_EINVAL;

    const int64_t begin = static_cast<int64_t>(rank) * layout->shard;
    const int64_t end = begin + layout->shard;
    int64_t found = 0;
    auto emit = [&](int64_t tensor, int64_t tensor_off, int64_t flat_lo, int64_t len) {
        if (found < cap) out[found] = zero_segment{tensor, tensor_off, flat_lo - begin, len};
        ++found;
    };
    int64_t flat = 0;
    for (int64_t t = 0; t < n_tensors && flat < end; ++t) {
        const int64_t lo = flat, hi = flat + numels[t];
        flat = hi;
        const int64_t a = lo > begin ? lo : begin;
        const int64_t b = hi < end ? hi : end;
        if (b > a) emit(t, a - lo, a, b - a);
    }
    const int64_t pad_lo = layout->n > begin ? layout->n : begin;
    if (end > pad_lo) emit(-1, pad_lo - layout->n, pad_lo, end - pad_lo);
    *count = found;
    return ZERO_OK;
}

// "ZeRO and FSDP", FSDP section: FSDP2 keeps each parameter as a tensor
// sharded along its first dimension and packs a unit's shards into one
// buffer per collective.  The cut is torch.chunk's: c = ceil(rows / n_dp)
// rows per rank, the last ranks short or empty, each chunk zero-padded to c
// rows in the packed buffer.
namespace {

struct Dim0 {
    int64_t n, packed;  // parameters, packed elements before the end padding
};

// sizes of a dim-0 layout, or false on invalid or overflowing arguments
bool dim0_sizes(const int64_t *rows, const int64_t *cols, int64_t n_tensors, int32_t n_dp,
                int64_t *packed_off, int64_t *chunk_rows, Dim0 *out) {
    if (n_tensors < 0 || n_dp < 1) return false;
    if (n_tensors > 0 && (!rows || !cols)) return false;
    int64_t n = 0, p = 0;
    for (int64_t i = 0; i < n_tensors; ++i) {
        const int64_t r = rows[i], c = cols[i];
        if (r < 0 || c < 0) return false;
        if (c > 0 && r > kI64Max / c) return false;
        const int64_t numel = r * c;
        const int64_t chunk = r / n_dp + (r % n_dp != 0 ? 1 : 0);
        const int64_t piece = chunk * c;  // <= numel
        if (numel > kI64Max - n || piece > kI64Max - p) return false;
        if (packed_off) packed_off[i] = p;
        if (chunk_rows) chunk_rows[i] = chunk;
        n += numel;
        p += piece;
    }
    out->n = n;
    out->packed = p;
    return true;
}

}  // namespace

// "ZeRO and FSDP", "A sharded Adam step": the exercise cuts the flat vector
// with numpy.array_split -- n / n_dp elements per rank, the first n mod n_dp
// ranks one more, contiguous and in rank order.
extern "C" zero_status zero_array_split_layout(int64_t n, int32_t n_dp, int64_t *starts,
                                               int64_t *lens) {
    if (n < 0 || n_dp < 1 || !starts || !lens) return ZERO_EINVAL;
    const int64_t each = n / n_dp, extra = n % n_dp;
    int64_t at = 0;
    for (int32_t r = 0; r < n_dp; ++r) {
        starts[r] = at;
        lens[r] = each + (r < extra ? 1 : 0);
        at += lens[r];
    }
    return ZERO_OK;
}

extern "C" zero_status zero_dim0_layout(const int64_t *rows, const int64_t *cols,
                                        int64_t n_tensors, int32_t n_dp, int64_t align,
                                        int64_t *packed_off, int64_t *chunk_rows,
                                        zero_layout *out) {
    if (!out || align < 1) return ZERO_EINVAL;
    Dim0 d;
    if (!dim0_sizes(rows, cols, n_tensors, n_dp, nullptr, nullptr, &d)) return ZERO_EINVAL;
    const int64_t units = d.packed / align + (d.packed % align != 0 ? 1 : 0);
    if (units > kI64Max / align) return ZERO_EINVAL;
    const int64_t shard = units * align;
    if (shard > 0 && n_dp > kI64Max / shard) return ZERO_EINVAL;
    dim0_sizes(rows, cols, n_tensors, n_dp, packed_off, chunk_rows, &d);
    out->n = d.n;
    out->shard = shard;
    out->n_pad = shard * n_dp;
    out->align = align;
    out->n_dp = n_dp;
    out->reserved = 0;
    return ZERO_OK;
}

extern "C" zero_status zero_dim0_segments(const zero_layout *layout, const int64_t *rows,
                                          const int64_t *cols, int64_t n_tensors, int32_t rank,
                                          zero_segment *out, int64_t cap, int64_t *count) {
    if (!layout_ok(layout) || !count || cap < 0) return ZERO_EINVAL;
    if (cap > 0 && !out) return ZERO_EINVAL;
    if (rank < 0 || rank >= layout->n_dp) return ZERO_EINVAL;
    Dim0 d;
    if (!dim0_sizes(rows, cols, n_tensors, layout->n_dp, nullptr, nullptr, &d)) return ZERO_EINVAL;
    const int64_t units = d.packed / layout->align + (d.packed % layout->align != 0 ? 1 : 0);
    if (d.n != layout->n || units * layout->align != layout->shard) return ZERO_EINVAL;

    int64_t found = 0;
    auto emit = [&](int64_t tensor, int64_t tensor_off, int64_t shard_off, int64_t len) {
        if (found < cap) out[found] = zero_segment{tensor, tensor_off, shard_off, len};
        ++found;
    };
    int64_t p = 0;
    for (int64_t i = 0; i < n_tensors; ++i) {
        const int64_t chunk = rows[i] / layout->n_dp + (rows[i] % layout->n_dp != 0 ? 1 : 0);
        const int64_t first = static_cast<int64_t>(rank) * chunk;
        int64_t have = rows[i] - first;
        have = have < 0 ? 0 : (have > chunk ? chunk : have);
        if (have > 0 && cols[i] > 0) emit(i, first * cols[i], p, have * cols[i]);
        if (have < chunk && cols[i] > 0)
            emit(-1, 0, p + have * cols[i], (chunk - have) * cols[i]);
        p += chunk * cols[i];
    }
    if (layout->shard > p) emit(-1, 0, p, layout->shard - p);
    *count = found;
    return ZERO_OK;
}

// "ZeRO and FSDP", "Memory per GPU": weights 2N, gradients 2N, optimizer
// state kN per GPU; each stage moves one more term under 1/n_dp.
extern "C" zero_status zero_model_state_bytes(double n, double n_dp, int32_t stage, double k,
                                              double *out) {
    if (!out || !(n >= 0) || !(n_dp >= 1) || !(k >= 0) || stage < 0 || stage > 3)
        return ZERO_EINVAL;
    const double weights = 2.0 * n, grads = 2.0 * n, optim = k * n;
    const double shard_w = stage >= 3 ? n_dp : 1.0;
    const double shard_g = stage >= 2 ? n_dp : 1.0;
    const double shard_o = stage >= 1 ? n_dp : 1.0;
    *out = weights / shard_w + grads / shard_g + optim / shard_o;
    return ZERO_OK;
}

// "ZeRO and FSDP", "Communication volume": per GPU, a ring reduce-scatter or
// all-gather sends (n_dp - 1) / n_dp of the vector, an all-reduce twice that.
extern "C" zero_status zero_comm_bytes(double n, double n_dp, int32_t stage, double param_bytes,
                                       double grad_bytes, double *out) {
    if (!out || !(n >= 0) || !(n_dp >= 1) || !(param_bytes > 0) || !(grad_bytes > 0) ||
        stage < 0 || stage > 3)
        return ZERO_EINVAL;
    const double part = (n_dp - 1.0) / n_dp * n;  // elements per RS or AG
    switch (stage) {
    case 0: *out = 2.0 * part * grad_bytes; break;  // all-reduce of gradients
    case 1:
    case 2: *out = part * grad_bytes + part * param_bytes; break;  // RS grads, AG weights
    default: *out = part * grad_bytes + 2.0 * part * param_bytes; break;  // + AG twice
    }
    return ZERO_OK;
}
