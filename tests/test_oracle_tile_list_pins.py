"""Pins of the oracle's forward and reverse block lists.

The block lists compact a tile-class table (fa4_qsa page, `_compact_blocks`:
partial and full block columns of each block row, int32 counts
[batch, 1, rows]; `_preprocess`: forward and reverse block lists).  They are
pinned to a hand-worked example, to numpy's stable descending argsort of the
class indicator (the ordering FlexAttention's BlockMask uses: the listed
blocks ascending, then the others ascending), and to invariants (every index
row is a permutation, the forward and reverse lists describe the same
tiles, and the counts add up with the absent tiles to the row length).
"""

from __future__ import annotations

import subprocess

import numpy as np
import pytest

import oracle
import pins
from workloads.generators import random_small_case

# Hand-worked: block row 0 has partial columns 1 and 3 and full column 2;
# row 1 has full columns 0 and 1; row 2 has partial column 0.
EXAMPLE = np.array([[[0, 1, 2, 1], [2, 2, 0, 0], [1, 0, 0, 0]]], dtype=np.int32)
EXAMPLE_LISTS = {
    "partial_count": [[[2, 0, 1]]],
    "partial_idx": [[[[1, 3, 0, 2], [0, 1, 2, 3], [0, 1, 2, 3]]]],
    "full_count": [[[1, 2, 0]]],
    "full_idx": [[[[2, 0, 1, 3], [0, 1, 2, 3], [0, 1, 2, 3]]]],
    "rev_partial_count": [[[1, 1, 0, 1]]],
    "rev_partial_idx": [[[[2, 0, 1], [0, 1, 2], [0, 1, 2], [0, 1, 2]]]],
    "rev_full_count": [[[1, 1, 1, 0]]],
    "rev_full_idx": [[[[1, 0, 2], [1, 0, 2], [0, 1, 2], [0, 1, 2]]]],
}


def argsort_lists(kinds: np.ndarray) -> dict:
    """The same lists from numpy: stable descending argsort of (class == k)."""
    out = {}
    for name, k in (("partial", 1), ("full", 2)):
        ind = (kinds == k).astype(np.int8)
        out[f"{name}_count"] = ind.sum(axis=2, dtype=np.int32)[:, None, :]
        out[f"{name}_idx"] = np.argsort(-ind, axis=2, kind="stable").astype(np.int32)[:, None]
        ind_t = ind.transpose(0, 2, 1)
        out[f"rev_{name}_count"] = ind_t.sum(axis=2, dtype=np.int32)[:, None, :]
        out[f"rev_{name}_idx"] = np.argsort(-ind_t, axis=2, kind="stable").astype(np.int32)[:, None]
    return out


def _random_kinds(seed, B, R, C):
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.choice(np.array([0, 1, 2], dtype=np.int32), size=(B, R, C), p=[0.5, 0.3, 0.2])


def check_example(orc):
    got = orc.tile_lists(EXAMPLE)
    for key, want in EXAMPLE_LISTS.items():
        assert got[key].tolist() == want, key


def check_argsort(orc):
    for seed, shape in ((1, (1, 5, 7)), (2, (2, 16, 3)), (3, (3, 1, 40)), (4, (1, 33, 65))):
        kinds = _random_kinds(seed, *shape)
        got, want = orc.tile_lists(kinds), argsort_lists(kinds)
        for key in oracle.TILE_LIST_KEYS:
            np.testing.assert_array_equal(got[key], want[key], err_msg=key)


def check_invariants(orc):
    kinds = _random_kinds(5, 2, 24, 31)
    B, R, C = kinds.shape
    got = orc.tile_lists(kinds)
    for key, n in (("partial_idx", C), ("full_idx", C), ("rev_partial_idx", R), ("rev_full_idx", R)):
        assert (np.sort(got[key], axis=-1) == np.arange(n)).all(), f"{key} rows must be permutations"
    absent = (kinds == 0).sum(axis=2)[:, None, :]
    assert ((got["partial_count"] + got["full_count"] + absent) == C).all()
    for name in ("partial", "full"):
        fwd = {(b, r, int(c)) for b in range(B) for r in range(R)
               for c in got[f"{name}_idx"][b, 0, r, :got[f"{name}_count"][b, 0, r]]}
        rev = {(b, int(r), c) for b in range(B) for c in range(C)
               for r in got[f"rev_{name}_idx"][b, 0, c, :got[f"rev_{name}_count"][b, 0, c]]}
        assert fwd == rev, f"forward and reverse {name} lists disagree"


def check_from_routes(orc):
    """End to end: lists of the classes of a random route table, classes from a numpy block reduction."""
    q, k, v, r = random_small_case(7, 2, 300, 500, 2, 1, 64, 40)
    kinds = pins.block_classes(pins.brute_membership(r, 500), 500)
    got, want = orc.tile_lists(kinds), argsort_lists(kinds)
    for key in oracle.TILE_LIST_KEYS:
        np.testing.assert_array_equal(got[key], want[key], err_msg=key)


CHECKS = (check_example, check_argsort, check_invariants, check_from_routes)


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_tile_list_pin(check):
    check(oracle._load())


MUTANTS = {
    "tail filled with -1": ("if (kinds[x * stride] != want) idx[r++] = (int32_t)x;",
                            "if (kinds[x * stride] != want) idx[r++] = -1;"),
    "full lists take partial tiles": ("compact_line(kb + r * n_cols, n_cols, 1, 2,", "compact_line(kb + r * n_cols, n_cols, 1, 1,"),
    "reverse walks a row": ("compact_line(kb + c, n_rows, n_cols, 1,", "compact_line(kb + c * n_cols, n_rows, 1, 1,"),
    "listed blocks descending": ("for (int64_t x = 0; x < n; ++x)\n        if (kinds[x * stride] == want) {",
                                 "for (int64_t x = n - 1; x >= 0; --x)\n        if (kinds[x * stride] == want) {"),
}


def _pins_fail(orc) -> bool:
    for check in CHECKS:
        try:
            check(orc)
        except AssertionError:
            return True
    return False


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_tile_list_mutants_fail_pins(name, tmp_path):
    src = open(oracle._SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name!r} not unique"
    mutant = tmp_path / "mutant.c"
    mutant.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", str(mutant), "-o", str(so), "-lm"])
    assert _pins_fail(oracle.Oracle(str(so))), f"no pin catches mutant: {name}"
