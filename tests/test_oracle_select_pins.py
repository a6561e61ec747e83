"""Pins of the oracle's route selection (qsa page, `select_qsa_token_ids`).

What fixes the selection independently of the oracle's C code:

* a hand-worked example (``tests/golden/select_example.txt``) that exercises
  the visible-block count, the relu, the sum over heads, the tie rule, the
  ascending block order, the incomplete tail and a padding row;
* a numpy brute force: dense float64 scores from ``einsum`` and a
  lexicographic sort (score descending, block ascending);
* torch.topk (float64, CPU) on tie-free random scores: the same kept set;
* the oracle's score table (``block_scores``, the yardstick of the GPU
  selection test on continuous inputs) element by element against torch
  float64 scores, relu(q k^T) summed over heads over sqrt(D), on row ranges
  that start and end inside the query length of several batch rows;
* invariants: rows that see at most token_budget/c blocks keep all of them
  whatever the values; head permutation and positive scaling of the queries
  change nothing; a query slice with its global offset equals the same rows
  of the full call; padding rows are all -1; every ID is causal and distinct.

Eleven planted mistakes, each compiled into a copy of the oracle, must each
fail at least one of these pins.
"""

from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from workloads.generators import float32_to_bf16_bits, random_select_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "select_example.txt")


def load_golden():
    keys, rows, params = [], [], {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        tag, rest = line.split(" ", 1)
        if tag == "key":
            keys.append([float(x) for x in rest.split()])
        elif tag == "row":
            _, h0, h1, want = (part.strip() for part in rest.split("|"))
            rows.append(([float(x) for x in h0.split()], [float(x) for x in h1.split()],
                         [int(x) for x in want.split()]))
        else:
            params[tag] = int(rest)
    iq = float32_to_bf16_bits(np.array([[[h0, h1] for h0, h1, _ in rows]], dtype=np.float32))
    ck = float32_to_bf16_bits(np.array([keys], dtype=np.float32))[:, :, None, :]
    want = np.array([[w for _, _, w in rows]], dtype=np.int32)
    return iq, ck, params, want


def brute_select(iq, ck, lens, budget, c, q_offset=0):
    """numpy: dense float64 scores, lexsort by (-score, block), expansion and tail."""
    q = (iq.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    k = (ck[:, :, 0, :].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    B, S_q, H, D = q.shape
    scores = np.maximum(np.einsum("bihd,bjd->bihj", q, k), 0.0).sum(axis=2) / np.sqrt(D)
    kb, W = budget // c, budget + c - 1
    out = np.full((B, S_q, W), -1, dtype=np.int32)
    for b in range(B):
        for i in range(S_q):
            t = q_offset + i
            if t >= lens[b]:
                continue
            nv = (t + 1) // c
            order = np.lexsort((np.arange(nv), -scores[b, i, :nv]))
            kept = np.sort(order[:min(kb, nv)])
            tokens = (kept[:, None] * c + np.arange(c)[None, :]).reshape(-1)
            out[b, i, :tokens.size] = tokens
            tail = np.arange(nv * c, t + 1)
            out[b, i, budget:budget + tail.size] = tail
    return out


# ---------------------------------------------------------------- checks


def check_golden(orc):
    iq, ck, p, want = load_golden()
    got = orc.select_token_ids(iq, ck, np.array([p["length"]]), p["budget"], p["c"])
    np.testing.assert_array_equal(got, want)


def check_brute_force(orc):
    cases = [  # seed, B, S_q, H, D, c, budget, lengths, integer
        (1, 2, 40, 3, 8, 4, 12, (40, 29), False),
        (2, 1, 64, 2, 16, 2, 10, (64,), True),
        (3, 2, 33, 5, 4, 3, 7, (20, 33), True),
        (4, 1, 50, 1, 8, 1, 9, (50,), False),
        (5, 1, 48, 4, 8, 8, 16, (47,), True),
        (6, 1, 30, 2, 8, 4, 3, (30,), False),  # budget < c: tails only
    ]
    for seed, B, S_q, H, D, c, budget, lens, integer in cases:
        iq, ck = random_select_case(seed, B, S_q, H, D, S_q // c, integer=integer)
        lens = np.array(lens, dtype=np.int64)
        np.testing.assert_array_equal(orc.select_token_ids(iq, ck, lens, budget, c),
                                      brute_select(iq, ck, lens, budget, c), err_msg=f"case {seed}")


def check_torch_topk(orc):
    B, S_q, H, D, c, budget = 2, 96, 4, 32, 4, 24
    iq, ck = random_select_case(11, B, S_q, H, D, S_q // c)
    lens = np.array([S_q, S_q], dtype=np.int64)
    got = orc.select_token_ids(iq, ck, lens, budget, c)
    q = torch.from_numpy((iq.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    k = torch.from_numpy((ck[:, :, 0].astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    scores = torch.relu(torch.matmul(q, k.transpose(1, 2).unsqueeze(1).contiguous())).sum(dim=2)
    kb = budget // c
    for b in range(B):
        for i in range(S_q):
            nv = (i + 1) // c
            m = min(kb, nv)
            want = set(torch.topk(scores[b, i, :nv], m).indices.tolist()) if m else set()
            blocks = got[b, i, :m * c:c] // c
            assert set(blocks.tolist()) == want, (b, i)
            assert (got[b, i, m * c:budget] == -1).all()


def check_block_scores(orc):
    """Every (batch, row, block) score of a row range against torch float64 scores of the same bf16 values."""
    B, S_q, H, D, n_blocks = 3, 37, 5, 24, 11
    iq, ck = random_select_case(31, B, S_q, H, D, n_blocks)
    q = torch.from_numpy((iq.astype(np.uint32) << 16).view(np.float32).astype(np.float64))  # [B,S_q,H,D]
    k = torch.from_numpy((ck[:, :, 0].astype(np.uint32) << 16).view(np.float32).astype(np.float64))  # [B,n,D]
    want = torch.relu(torch.matmul(q, k.transpose(1, 2).unsqueeze(1).contiguous())).sum(dim=2) / np.sqrt(D)
    for r0, r1 in ((0, S_q), (0, 1), (5, 19), (36, 37)):
        got = orc.block_scores(iq, ck, rows=(r0, r1))
        assert got.shape == (B, r1 - r0, n_blocks), got.shape
        np.testing.assert_allclose(got, want[:, r0:r1].numpy(), rtol=1e-12, atol=1e-12, err_msg=f"rows {r0}..{r1}")


def check_invariants(orc):
    B, S_q, H, D, c, budget = 2, 80, 4, 16, 4, 20
    kb = budget // c
    iq, ck = random_select_case(21, B, S_q, H, D, S_q // c)
    lens = np.array([80, 57], dtype=np.int64)
    base = orc.select_token_ids(iq, ck, lens, budget, c)
    # rows that see at most kb blocks keep all of them, whatever the values
    iq2, ck2 = random_select_case(22, B, S_q, H, D, S_q // c)
    other = orc.select_token_ids(iq2, ck2, lens, budget, c)
    dense_rows = (np.arange(S_q) + 1) // c <= kb
    np.testing.assert_array_equal(base[:, dense_rows], other[:, dense_rows])
    for i in np.nonzero(dense_rows)[0]:
        nv = (i + 1) // c
        assert (base[0, i, :nv * c] == np.arange(nv * c)).all()
    # head permutation and positive scaling of the queries
    np.testing.assert_array_equal(orc.select_token_ids(iq[:, :, ::-1].copy(), ck, lens, budget, c), base)
    doubled = float32_to_bf16_bits((iq.astype(np.uint32) << 16).view(np.float32) * 2)
    np.testing.assert_array_equal(orc.select_token_ids(doubled, ck, lens, budget, c), base)
    # a slice of query rows with its global offset
    for r0, r1 in ((0, 17), (17, 61), (61, 80)):
        part = orc.select_token_ids(iq[:, r0:r1].copy(), ck, lens, budget, c, q_offset=r0)
        np.testing.assert_array_equal(part, base[:, r0:r1])
        np.testing.assert_array_equal(orc.select_token_ids(iq, ck, lens, budget, c, rows=(r0, r1)), base[:, r0:r1])
    # padding rows, causality, distinct IDs, tail length
    for b in range(B):
        for i in range(S_q):
            row = base[b, i]
            if i >= lens[b]:
                assert (row == -1).all()
                continue
            ids = row[row >= 0]
            assert ids.max() <= i and len(set(ids.tolist())) == ids.size
            assert (row[budget:] >= 0).sum() == (i + 1) % c


CHECKS = (check_golden, check_brute_force, check_torch_topk, check_block_scores, check_invariants)


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_select_pin(check):
    check(oracle._load())


MUTANTS = {
    "visible blocks floor(t/c)": ("const int64_t nv = (t + 1) / c;", "const int64_t nv = t / c;"),
    "no relu": ("total += dot > 0.0 ? dot : 0.0;", "total += dot;"),
    "max over heads": ("total += dot > 0.0 ? dot : 0.0;", "total = dot > total ? dot : total;"),
    "ties to the larger block": ("return (x->block > y->block) - (x->block < y->block);",
                                 "return (x->block < y->block) - (x->block > y->block);"),
    "kept blocks in score order": ("qsort(kept, (size_t)m, sizeof(int64_t), cmp_int64);", ""),
    "last logical row is padding": ("if (t >= seq_lens[b]) continue;", "if (t + 1 >= seq_lens[b]) continue;"),
    "tail stops before the query": ("for (int64_t u = 0; nv * c + u <= t; ++u)", "for (int64_t u = 0; nv * c + u < t; ++u)"),
    "worst blocks kept": ("if (x->score != y->score) return x->score > y->score ? -1 : 1;",
                          "if (x->score != y->score) return x->score < y->score ? -1 : 1;"),
    # the score table alone (not used by the selection itself)
    "score table reads rows from the range start": (
        "block_score(iq + (b * S_q + i) * H * D, ck + (b * n_blocks + j) * D, H, D);\n}",
        "block_score(iq + (b * S_q + (i - row_begin)) * H * D, ck + (b * n_blocks + j) * D, H, D);\n}"),
    "score table takes the first batch row's keys": (
        "block_score(iq + (b * S_q + i) * H * D, ck + (b * n_blocks + j) * D, H, D);\n}",
        "block_score(iq + (b * S_q + i) * H * D, ck + j * D, H, D);\n}"),
    "score table blocks transposed with rows": (
        "scores[(b * n_rows + (i - row_begin)) * n_blocks + j] =",
        "scores[(b * n_blocks + j) * n_rows + (i - row_begin)] ="),
}


def _pins_fail(orc) -> bool:
    for check in CHECKS:
        try:
            check(orc)
        except AssertionError:
            return True
    return False


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_select_mutants_fail_pins(name, tmp_path):
    src = open(oracle._SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name!r} not unique"
    mutant = tmp_path / "mutant.c"
    mutant.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", str(mutant), "-o", str(so), "-lm"])
    assert _pins_fail(oracle.Oracle(str(so))), f"no pin catches mutant: {name}"
