"""Argument validation of the device entry points under random and extreme
integers (CPU only, made-up addresses): every call returns one of the
documented statuses without crashing, and whenever validation lets a call
through (ZERO_OK, or ZERO_EDEVICE from the launch that cannot happen
without a GPU) the documented limits hold -- lengths within 2^38, row
slabs within 2^60 elements, the range inside the shard and the weight
buffer, ranks and dtypes valid."""
import ctypes

import pytest
from hypothesis import HealthCheck, event, given, settings
from hypothesis import strategies as st

import zero_sharded_mixed_flatten_amd as zs

from tests.test_lib_host import cpu_only

L = zs._lib
P = ctypes.c_void_p
STATUSES = {zs.ZERO_OK, zs.ZERO_EINVAL, zs.ZERO_EALIAS, zs.ZERO_ERANGE, zs.ZERO_EDEVICE}
I64 = st.one_of(st.integers(-(1 << 63), (1 << 63) - 1), st.integers(-4, 4096),
                st.sampled_from([0, 1, 4, (1 << 31), (1 << 38), (1 << 38) + 1, (1 << 60),
                                 (1 << 61), (1 << 62), (1 << 63) - 1, -(1 << 63)]))
SMALL = st.integers(-2, 70)


def _spread(i):
    return (1 << 40) + i * (1 << 36)   # disjoint made-up device addresses


@cpu_only
@settings(max_examples=600, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(data=st.data())
def test_fused_step_validation(data):
    # mostly arguments built to be valid for a consistent layout, with at
    # most one field pushed to an extreme, so both sides of every check run
    n = data.draw(st.one_of(st.integers(0, 1 << 20), st.sampled_from([(1 << 40), (1 << 61)])))
    n_dp = data.draw(st.integers(1, 64))
    align = data.draw(st.sampled_from([1, 1, 8, 256]))
    shard = -(-n // (n_dp * align)) * align
    lay = zs.ZeroLayout(n, shard * n_dp, shard, align, n_dp, 0)
    rank = data.draw(st.integers(0, n_dp - 1))
    shard_off = data.draw(st.integers(0, shard))
    length = data.draw(st.integers(0, shard - shard_off))
    ld = length + data.draw(st.sampled_from([0, 0, 3, 64]))
    gdt, wdt, step = data.draw(st.sampled_from([0, 1, 2])), data.draw(st.sampled_from([0, 1])), 1
    field = data.draw(st.sampled_from(["none", "none", "n_dp", "rank", "ld", "length",
                                       "shard_off", "gdt", "wdt", "step", "n_pad"]))
    extreme = data.draw(I64)
    if field == "n_dp":
        lay.n_dp = max(-(1 << 31), min((1 << 31) - 1, extreme))
    elif field == "rank":
        rank = max(-(1 << 31), min((1 << 31) - 1, extreme))
    elif field == "ld":
        ld = extreme
    elif field == "length":
        length = extreme
    elif field == "shard_off":
        shard_off = extreme
    elif field == "gdt":
        gdt = data.draw(st.integers(-1, 3))
    elif field == "wdt":
        wdt = data.draw(st.integers(-1, 2))
    elif field == "step":
        step = data.draw(st.integers(-1, 0))
    elif field == "n_pad":
        lay.n_pad = extreme
    hp = zs.AdamWHParams(step=step)._c()
    s = L.zero_shard_step(P(_spread(1)), gdt, ld, length, P(_spread(2)), P(_spread(3)),
                          P(_spread(4)), P(_spread(5)), wdt, ctypes.byref(lay), rank, shard_off,
                          ctypes.byref(hp), None, None, None, 0, None)
    assert s in STATUSES
    event(f"status {s}")
    if s in (zs.ZERO_OK, zs.ZERO_EDEVICE) and length > 0:
        nd = lay.n_dp
        assert 0 < length <= (1 << 38) and ld >= length
        assert (nd - 1) * ld + length <= (1 << 60)
        assert 0 <= rank < nd and gdt in (0, 1, 2) and wdt in (0, 1) and step >= 1
        assert 0 <= shard_off and shard_off + length <= lay.shard
        assert lay.n_pad == lay.shard * nd <= (1 << 60) and lay.n <= lay.n_pad


@cpu_only
@settings(max_examples=300, deadline=None)
@given(n_rows=SMALL, ld=I64, length=I64, gdt=st.integers(-1, 3))
def test_reduce_validation(n_rows, ld, length, gdt):
    s = L.zero_shard_reduce(P(_spread(1)), gdt, n_rows, ld, length, P(_spread(2)), 0, None,
                            None, None, 0, None)
    assert s in STATUSES
    event(f"status {s}")
    if s in (zs.ZERO_OK, zs.ZERO_EDEVICE) and length > 0:
        assert n_rows >= 1 and 0 < length <= (1 << 38) and ld >= length
        assert (n_rows - 1) * ld + length <= (1 << 60) and gdt in (0, 1, 2)


@cpu_only
@settings(max_examples=300, deadline=None)
@given(n_src=st.integers(-1, 20), src_shard=I64, n=I64, eb=st.integers(0, 5),
       dst_rank=st.integers(-1, 40), dst_shard=I64)
def test_reshard_validation(n_src, src_shard, n, eb, dst_rank, dst_shard):
    srcs = (P * max(n_src, 1))(*[_spread(2 + k).__index__() for k in range(max(n_src, 1))])
    s = L.zero_reshard(srcs, n_src, src_shard, n, eb, dst_rank, dst_shard, P(_spread(1)), None)
    assert s in STATUSES
    event(f"status {s}")
    if s in (zs.ZERO_OK, zs.ZERO_EDEVICE) and dst_shard > 0:
        assert n_src >= 1 and src_shard >= 0 and 0 <= n <= n_src * src_shard
        assert eb in (2, 4) and dst_rank >= 0 and dst_shard <= (1 << 38)


@cpu_only
@settings(max_examples=500, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(data=st.data())
def test_q8_step_validation(data):
    B = zs.ZERO_Q8_BLOCK
    n_dp = data.draw(st.integers(1, 64))
    shard = B * data.draw(st.integers(0, 4096))
    lay = zs.ZeroLayout(shard * n_dp, shard * n_dp, shard, B, n_dp, 0)
    rank = data.draw(st.integers(0, n_dp - 1))
    shard_off = B * data.draw(st.integers(0, shard // B))
    length = data.draw(st.integers(0, shard - shard_off))
    nb = -(-length // B)
    ld = length + 4 * data.draw(st.integers(0, 16)) + (4 - length % 4) % 4
    sld = nb + data.draw(st.integers(0, 4))
    field = data.draw(st.sampled_from(["none", "none", "ld", "sld", "length", "shard_off",
                                       "rank", "shard"]))
    extreme = data.draw(I64)
    if field == "ld":
        ld = extreme
    elif field == "sld":
        sld = extreme
    elif field == "length":
        length = extreme
    elif field == "shard_off":
        shard_off = extreme
    elif field == "rank":
        rank = max(-(1 << 31), min((1 << 31) - 1, extreme))
    elif field == "shard":
        lay.shard = extreme
    hp = zs.AdamWHParams()._c()
    s = L.zero_shard_step_q8(P(_spread(1)), P(_spread(2)), ld, sld, length, P(_spread(3)),
                             P(_spread(4)), P(_spread(5)), P(_spread(6)), P(_spread(7)),
                             ctypes.byref(lay), rank, shard_off, ctypes.byref(hp), None, None,
                             None, 0, None)
    assert s in STATUSES
    event(f"status {s}")
    if s in (zs.ZERO_OK, zs.ZERO_EDEVICE) and length > 0:
        nbl = -(-length // B)
        assert 0 < length <= (1 << 38) and ld >= length and 0 <= rank < n_dp
        assert lay.shard % B == 0 and shard_off % B == 0 and shard_off + length <= lay.shard
        if n_dp > 1:
            assert ld % 4 == 0 and sld >= nbl
            assert (n_dp - 1) * ld + length <= (1 << 60) and (n_dp - 1) * sld + nbl <= (1 << 60)


@cpu_only
@settings(max_examples=400, deadline=None)
@given(data=st.data())
def test_flat_gather_validation(data):
    """Pieces with random (sometimes overlapping, negative or huge) flat
    ranges: a gather that gets through has pieces disjoint in flat index,
    non-negative fields without index overflow, and a count within 2^38."""
    k = data.draw(st.integers(0, 6))
    raw = []
    for i in range(k):
        off = data.draw(st.one_of(st.integers(0, 5000), I64))
        ln = data.draw(st.one_of(st.integers(0, 3000), I64))
        raw.append((off, ln))
    pieces = (zs._Piece * max(k, 1))()
    for i, (off, ln) in enumerate(raw):
        pieces[i] = zs._Piece(_spread(2 + i), off, ln)
    n = data.draw(st.one_of(st.integers(0, 10000), I64))
    begin = data.draw(st.one_of(st.integers(0, 10000), I64))
    count = data.draw(st.one_of(st.integers(0, 10000), I64))
    eb = data.draw(st.sampled_from([2, 4, 3, 0]))
    s = L.zero_flat_gather(pieces, k, n, eb, begin, count, P(_spread(1)), None)
    assert s in STATUSES
    event(f"status {s}")
    if s in (zs.ZERO_OK, zs.ZERO_EDEVICE):
        assert eb in (2, 4) and n >= 0 and begin >= 0 and 0 <= count <= (1 << 38)
        live = sorted((off, ln) for off, ln in raw if ln > 0)
        for off, ln in live:
            assert off >= 0 and ln <= ((1 << 63) - 1) // 4 and off + ln < (1 << 63)
        for (o1, l1), (o2, _) in zip(live, live[1:]):
            assert o1 + l1 <= o2
