"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each pin targets a plausible mistake: a wrong validity bound, missing
deduplication, a transposed head map, a dropped scale, a wrong normaliser,
swapped tile classes.  ``test_mutants_fail_pins`` plants such mistakes in a
copy of the oracle source and checks that a pin catches every one.
"""

from __future__ import annotations

import math
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
import pins
from workloads.generators import float32_to_bf16_bits, random_small_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_route_rules():
    cases = []
    with open(os.path.join(GOLDEN, "route_rules.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            dtype, kv, slots, expect = (c.strip() for c in line.split("|"))
            exp = [] if expect == "-" else [int(x) for x in expect.split()]
            cases.append((dtype, int(kv), [int(x) for x in slots.split()], exp))
    return cases


# --------------------------------------------------------------------------
# route sets, membership, tile classes
# --------------------------------------------------------------------------

def check_golden_rules(orc):
    for dtype, kv, slots, expect in _golden_route_rules():
        r = np.array([[slots]], dtype=np.int64 if dtype == "int64" else np.int32)
        lst, cnt = orc.route_lists(r, kv)
        n = len(expect)
        assert cnt[0, 0] == n, (slots, kv)
        assert lst[0, 0, :n].tolist() == expect, (slots, kv)
        assert (lst[0, 0, n:] == -1).all()
        if kv <= 1 << 16:  # the table for kv_length near 2**31 would be 2 GiB
            mem = orc.membership(r, kv)
            assert mem.shape[-1] == oracle.ldm_of(kv)
            assert np.flatnonzero(mem[0, 0]).tolist() == expect


def test_golden_route_rules():
    check_golden_rules(oracle)


def check_lists_bruteforce(orc):
    for seed, dtype in [(1, np.int64), (2, np.int32), (3, np.int64)]:
        _, _, _, r = random_small_case(seed, B=2, S_q=37, S_kv=53, Hq=2, Hkv=1, D=8, K=19,
                                       p_invalid=0.3, p_empty=0.15, route_dtype=dtype)
        lst, cnt = orc.route_lists(r, 53)
        blst, bcnt = pins.brute_lists(r, 53)
        np.testing.assert_array_equal(cnt, bcnt)
        np.testing.assert_array_equal(lst, blst)


def test_lists_bruteforce():
    check_lists_bruteforce(oracle)


def test_int32_and_int64_agree():
    _, _, _, r = random_small_case(7, B=1, S_q=64, S_kv=100, Hq=1, Hkv=1, D=8, K=40, route_dtype=np.int32)
    a = oracle.route_lists(r, 100)
    b = oracle.route_lists(r.astype(np.int64), 100)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_membership_bruteforce_and_padding():
    for kv in (53, 128, 130):
        _, _, _, r = random_small_case(11 + kv, B=2, S_q=21, S_kv=kv, Hq=1, Hkv=1, D=8, K=33)
        mem = oracle.membership(r, kv)
        ldm = oracle.ldm_of(kv)
        assert mem.shape == (2, 21, ldm) and ldm % 128 == 0 and ldm >= kv
        np.testing.assert_array_equal(mem, pins.brute_membership(r, kv, ldm))
        assert not mem[:, :, kv:].any()
        _, cnt = oracle.route_lists(r, kv)
        np.testing.assert_array_equal(mem.sum(axis=2), cnt)


def check_tile_classes(orc):
    rng = np.random.default_rng(5)
    # random tables with ragged edges in both dimensions
    for S_q, kv, K in [(300, 260, 50), (128, 128, 200), (129, 1, 3)]:
        r = rng.integers(-3, kv + 3, size=(2, S_q, K))
        got = orc.tile_class(r, kv)
        np.testing.assert_array_equal(got, pins.block_classes(pins.brute_membership(r, kv), kv))
    # constructed: full, partial and absent tiles, including a full ragged edge tile
    S_q, kv = 200, 130
    r = np.full((1, S_q, 130), -1, dtype=np.int64)
    r[0, :128, :128] = np.arange(128)            # tile (0,0): every pair a member -> full
    r[0, 128:, 0] = 128                          # tile (1,1): column 128 only -> partial
    r[0, 128:, 1] = 129                          #             plus column 129 -> every in-range pair
    r[0, 130, 2] = 5                             # tile (1,0): one member -> partial
    got = orc.tile_class(r, kv)
    assert got.shape == (1, 2, 2)
    assert got[0].tolist() == [[2, 0], [1, 2]]


def test_tile_classes():
    check_tile_classes(oracle)


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

SMALL_SHAPES = [  # (B, S_q, S_kv, Hq, Hkv, D, K)
    (1, 9, 13, 1, 1, 8, 5),
    (2, 17, 29, 4, 2, 16, 11),
    (1, 12, 40, 8, 1, 64, 24),
    (2, 8, 33, 16, 2, 32, 17),
    (1, 5, 21, 6, 3, 8, 9),
]


def check_forward_bruteforce(orc):
    for n, (B, S_q, S_kv, Hq, Hkv, D, K) in enumerate(SMALL_SHAPES):
        q, k, v, r = random_small_case(100 + n, B, S_q, S_kv, Hq, Hkv, D, K)
        scale = 1.0 / math.sqrt(D) * (1.0 + 0.37 * n)
        got = orc.forward(q, k, v, r, scale)
        ref = pins.dense_attention(q, k, v, r, scale)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_forward_bruteforce():
    check_forward_bruteforce(oracle)


def _sdpa_masked(q, k, v, mask, scale):
    """torch CPU scaled_dot_product_attention in float64 with K/V heads repeated h -> h // G."""
    qt = torch.from_numpy(pins.bf16_to_f64(q)).permute(0, 2, 1, 3)
    G = q.shape[2] // k.shape[2]
    kt = torch.from_numpy(pins.bf16_to_f64(k)).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(pins.bf16_to_f64(v)).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    m = None if mask is None else torch.from_numpy(mask)[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, is_causal=mask is None,
                                                         scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


def test_all_causal_routes_equal_dense_causal_sdpa():
    rng = np.random.default_rng(21)
    for B, S, Hq, Hkv, D in [(1, 40, 4, 1, 32), (2, 33, 8, 2, 16), (1, 24, 2, 2, 64)]:
        q, k, v, _ = random_small_case(22 + S, B, S, S, Hq, Hkv, D, 1)
        # R(i) = {0..i}: every causal key once, then padding, duplicates and garbage, shuffled
        r = np.full((B, S, 2 * S), -1, dtype=np.int64)
        for b in range(B):
            for i in range(S):
                row = list(range(i + 1)) + [int(x) for x in rng.integers(0, i + 1, size=3)]
                row += [S, S + 7, 1 << 40][: 2 * S - len(row)]
                row += [-1] * (2 * S - len(row))
                r[b, i] = rng.permutation(row)
        scale = 1.0 / math.sqrt(D)
        got = oracle.forward(q, k, v, r, scale)
        np.testing.assert_allclose(got, _sdpa_masked(q, k, v, None, scale), rtol=0, atol=1e-12)


def test_arbitrary_routes_equal_masked_sdpa():
    for n, (B, S_q, S_kv, Hq, Hkv, D, K) in enumerate(SMALL_SHAPES):
        q, k, v, r = random_small_case(300 + n, B, S_q, S_kv, Hq, Hkv, D, K, p_empty=0.2)
        scale = 0.5 + 0.1 * n
        got = oracle.forward(q, k, v, r, scale)
        mask = pins.brute_membership(r, S_kv).astype(bool)
        nonempty = mask.any(axis=2)
        ref = _sdpa_masked(q, k, v, mask, scale)
        np.testing.assert_allclose(got[nonempty], ref[nonempty], rtol=0, atol=1e-12)
        assert (got[~nonempty] == 0).all()


def test_closed_form_two_keys():
    # q = (1, 0), k0 = (0, 0), k1 = (1, 0), v0 = (1, 0), v1 = (0, 1), scale 1: s = (0, 1),
    # so o = (1, e) / (1 + e).  With q = (2, 0) and scale 1/2 the scores are the same.
    bits = lambda a: float32_to_bf16_bits(np.array(a, dtype=np.float32))
    k = bits([[[[0, 0]], [[1, 0]]]])
    v = bits([[[[1, 0]], [[0, 1]]]])
    r = np.array([[[1, 0, -1, 1]]], dtype=np.int64)
    e = math.e
    for qv, scale in (([1, 0], 1.0), ([2, 0], 0.5)):
        q = bits([[[qv]]])
        got = oracle.forward(q, k, v, r, scale)[0, 0, 0]
        np.testing.assert_allclose(got, [1 / (1 + e), e / (1 + e)], rtol=1e-15, atol=0)


def test_single_route_returns_that_v_row_exactly():
    q, k, v, _ = random_small_case(41, 2, 16, 30, 8, 2, 64, 1)
    rng = np.random.default_rng(42)
    j = rng.integers(0, 30, size=(2, 16))
    r = np.stack([j, np.full_like(j, -1), j, np.full_like(j, 30)], axis=2)  # one valid ID, repeated
    got = oracle.forward(q, k, v, r, 0.125)
    vf = pins.bf16_to_f64(v)
    for b in range(2):
        for i in range(16):
            for h in range(8):
                assert np.array_equal(got[b, i, h], vf[b, j[b, i], h // 4])


def test_zero_query_gives_mean_of_routed_rows():
    q, k, v, r = random_small_case(51, 1, 20, 25, 4, 2, 16, 10, q_zero=True, p_empty=0.0)
    got = oracle.forward(q, k, v, r, 0.3)
    vf = pins.bf16_to_f64(v)
    for i in range(20):
        s = pins.brute_route_set(r[0, i].tolist(), 25)
        for h in range(4):
            np.testing.assert_allclose(got[0, i, h], vf[0, s, h // 2].mean(axis=0), rtol=0, atol=1e-14)


def test_all_invalid_rows_are_exactly_zero():
    q, k, v, r = random_small_case(61, 2, 10, 12, 4, 1, 16, 6, p_empty=0.0)
    r[0, 3] = -1
    r[1, 7] = [12, 13, -1, 1 << 40, -(1 << 40), np.iinfo(np.int64).min]
    got = oracle.forward(q, k, v, r, 0.25)
    assert np.all(got[0, 3] == 0) and np.all(got[1, 7] == 0)
    assert not np.signbit(got[0, 3]).any() and not np.signbit(got[1, 7]).any()


def test_permuting_and_duplicating_routes_changes_nothing():
    q, k, v, r = random_small_case(71, 2, 14, 40, 4, 2, 32, 12)
    rng = np.random.default_rng(72)
    base = oracle.forward(q, k, v, r, 0.2)
    perm = np.take_along_axis(r, rng.permuted(np.tile(np.arange(12), (2, 14, 1)), axis=2), axis=2)
    dup = np.concatenate([r, r[:, :, ::-1], r[:, :, :5]], axis=2)
    for alt in (perm, dup):
        assert np.array_equal(oracle.forward(q, k, v, alt, 0.2), base)
        (la, ca), (lb, cb) = oracle.route_lists(alt, 40), oracle.route_lists(r, 40)
        np.testing.assert_array_equal(ca, cb)
        np.testing.assert_array_equal(la[..., :12], lb)
        assert (la[..., 12:] == -1).all()


def test_row_subset_matches_full():
    q, k, v, r = random_small_case(81, 2, 30, 40, 4, 2, 16, 9)
    full = oracle.forward(q, k, v, r, 0.25)
    part = oracle.forward(q, k, v, r, 0.25, rows=(17, 30))
    assert np.array_equal(part, full[:, 17:30])


# --------------------------------------------------------------------------
# planted mistakes: every mutant of the oracle must fail at least one pin
# --------------------------------------------------------------------------

MUTANTS = {
    "validity bound off by one": ("x >= 0 && x < kv_length", "x >= 0 && x <= kv_length"),
    "negative IDs accepted": ("x >= 0 && x < kv_length", "x >= -1 && x < kv_length"),
    "no deduplication": ("if (m == 0 || out[j] != out[m - 1])", "if (1)"),
    "head map h % Hkv": ("int64_t hk = h / G;", "int64_t hk = h % Hkv;"),
    "scale dropped": ("score[j] = scale * dot;", "score[j] = dot;"),
    "normaliser is the count": ("o[d] /= denom;", "o[d] /= (double)n;"),
    "list fill 0 instead of -1": ("(int32_t)set[j] : -1", "(int32_t)set[j] : 0"),
    "full and partial swapped": ("members[tj] == pairs ? 2 : 1", "members[tj] == pairs ? 1 : 2"),
    "tile key width 64": ("members[set[j] / T] += 1", "members[(set[j] / 64) % n_tj] += 1"),
}


def _pins_fail(orc) -> bool:
    for check in (check_golden_rules, check_lists_bruteforce, check_tile_classes, check_forward_bruteforce):
        try:
            check(orc)
        except AssertionError:
            return True
    return False


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutants_fail_pins(name, tmp_path):
    src = open(oracle._SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutation site for {name!r} not found"
    mutant = tmp_path / "mutant.c"
    mutant.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", str(mutant), "-o", str(so), "-lm"])
    assert _pins_fail(oracle.Oracle(str(so))), f"no pin catches mutant: {name}"


def test_unmutated_oracle_passes_the_same_pins():
    assert not _pins_fail(oracle._load())
