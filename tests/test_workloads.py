"""Structure of the seeded synthetic workloads (generator properties, CPU only)."""

from __future__ import annotations

import numpy as np
import pytest

import pins
from workloads import WORKLOADS, make_routes
from workloads.generators import BLOCK, _packed_documents, bf16_bits_to_float32, float32_to_bf16_bits


def _distinct_valid_counts(r: np.ndarray, kv: int) -> np.ndarray:
    x = np.where((r >= 0) & (r < kv), r, -1)
    x.sort(axis=-1)
    first = np.ones(x.shape, dtype=bool)
    first[..., 1:] = x[..., 1:] != x[..., :-1]
    return ((x >= 0) & first).sum(axis=-1)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e-3, 65504.0], dtype=np.float32)
    back = bf16_bits_to_float32(float32_to_bf16_bits(x))
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0); 1 + 3*2^-8 ties -> 1 + 2^-6
    assert back.tolist()[:4] == [1.0, 1.0, 1.015625, -2.5]
    assert np.all(np.abs(back - x) <= np.abs(x) * 2.0 ** -8)


def test_tiny_routes():
    w = WORKLOADS["tiny"]
    r = make_routes(w)[0]
    empty = (r == -1).all(axis=1)
    assert empty.sum() == 26
    q = np.arange(w.S_q)[:, None]
    assert ((r >= 0) & (r <= q))[~empty].all()


def test_right_padded_routes():
    w = WORKLOADS["right_padded"]
    r = make_routes(w)
    assert (r[1, 3000:] == -1).all()
    cnt = _distinct_valid_counts(r, w.S_kv)
    assert cnt.sum() == 3_180_028 and (cnt == 0).sum() == 1096
    q = np.arange(w.S_q)[None, :, None]
    assert np.all((r == -1) | ((r >= 0) & (r <= q)))
    for b, i in [(0, 0), (0, 4095), (1, 2999), (0, 700)]:
        j = i // BLOCK
        blocks = {int(x) // BLOCK for x in r[b, i] if x >= 0}
        assert j in blocks and len(blocks) == min(8, j + 1)
        assert set(range(j * BLOCK, i + 1)) <= set(r[b, i].tolist())


def test_packed_thd_routes():
    w = WORKLOADS["packed_thd"]
    r = make_routes(w)[0]
    children = np.random.SeedSequence(w.seed).spawn(4)
    starts, lengths = _packed_documents(np.random.Generator(np.random.PCG64(children[3])), w.S_q)
    end = starts[-1] + lengths[-1]
    assert all(L >= BLOCK for L in lengths) and end <= w.S_q
    assert (r[end:] == -1).all()  # tail padding rows
    for d0, L in zip(starts[:3] + starts[-2:], lengths[:3] + lengths[-2:]):
        for p in (0, L // 2, L - 1):
            row = r[d0 + p]
            assert (row == 1 << 40).sum() >= 6
            assert ((row >= w.S_kv) & (row < w.S_kv + 1000)).sum() >= 7
            valid = row[(row >= 0) & (row < w.S_kv)]
            assert valid.size > 0 and valid.min() >= d0 and valid.max() <= d0 + p
            assert valid.size > np.unique(valid).size  # duplicates are present
    n = _distinct_valid_counts(r, w.S_kv).sum()
    assert 6_000_000 < n < 13_000_000


def test_cp_slice_routes():
    w = WORKLOADS["cp_slice"]
    r = make_routes(w)[0]
    p = w.q_offset + np.arange(w.S_q)
    cnt = _distinct_valid_counts(r, w.S_kv)
    np.testing.assert_array_equal(cnt, 31 * BLOCK + p % BLOCK + 1)
    assert np.all((r == -1) | ((r >= 0) & (r <= p[:, None])))
    assert cnt.sum() == 16_519_168


def test_long_int64_routes():
    w = WORKLOADS["long_int64"]
    # the pages' int32 wrap threshold: a square 46341-token table is past 2**31
    assert 46341 * 46341 > 2 ** 31 > 46340 * 46340
    assert w.B * w.S_q * w.S_kv > 2 ** 31
    r = make_routes(w)[0]
    cnt = _distinct_valid_counts(r, w.S_kv)
    assert cnt.sum() == 130_121_728
    for i in (0, 63, 64, 2047, 65535):
        s = pins.brute_route_set(r[i].tolist(), w.S_kv)
        j = i // BLOCK
        blocks = {x // BLOCK for x in s}
        assert j in blocks and 0 in blocks and len(blocks) == min(32, j + 1)
        assert max(s) == i


def test_int32_routes_same_values():
    w = WORKLOADS["right_padded"]
    np.testing.assert_array_equal(make_routes(w, np.int32), make_routes(w))
    with pytest.raises(ValueError):
        make_routes(WORKLOADS["packed_thd"], np.int32)  # holds 2**40
