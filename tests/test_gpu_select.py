"""GPU parity of route selection (qsa page, `select_qsa_token_ids`) against the fp64 oracle.

* Integer-valued inputs in [-3, 3]: every bf16 product and every fp32 sum
  is exact, so the GPU's fp32 scores equal the oracle's exactly and the
  outputs must match bit for bit, ties and their rule included.
* Continuous inputs: near-equal scores may be ordered differently by fp32
  rounding, so the GPU's kept set must be valid (no kept block scores below
  an unkept one by more than the rounding bound) and equal to the oracle's
  wherever the oracle's margin exceeds that bound.  Everything else (slot
  layout, dense rows, tails, padding rows) must match exactly.
* Full-size workloads: sampled rows against the oracle, structural checks on
  every row, and bit-identical results when the rows are scored in several
  workspace-bounded passes.

Rounding bound of one score (bf16 products are exact in fp32; the matrix
core sums D products per head, then H relu terms are summed): with
u = 2^-23 (one ulp, covering a sum that truncates rather than rounds),
|s_fp32 - s_exact| <= (D + H + 8) * u * sum_h sum_d |q_hd k_d|.
"""

from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

import oracle
import route_sparse_gqa_amd as qsa
from gpu_util import bf16_to_gpu, check_forward, device
from workloads import make_select_inputs, random_select_case, SELECT_WORKLOADS
from workloads.generators import float32_to_bf16_bits

pytestmark = pytest.mark.gpu

U = 2.0 ** -23


def _f64(bits):
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def run_gpu(iq, ck, lens, budget, c, q_offset=0, S_global=None, chunk=None):
    out = qsa.qsa_select_token_ids(bf16_to_gpu(iq), bf16_to_gpu(ck), torch.from_numpy(lens).to(device()),
                                   budget, c, query_position_offset=q_offset, global_sequence_length=S_global,
                                   query_chunk_size=chunk)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def score_bounds(iq, ck, rows):
    """Rounding bound of every (row, block) score, scaled by 1/sqrt(D) like the oracle's scores."""
    q = np.abs(_f64(iq[:, rows[0]:rows[1]]))
    k = np.abs(_f64(ck[:, :, 0]))
    B, R, H, D = q.shape
    mag = np.matmul(q.sum(axis=2), k.transpose(0, 2, 1))  # sum_h sum_d |q_hd| |k_d|
    return (D + H + 8) * U * mag / np.sqrt(D)


def check_rows(got, iq, ck, lens, budget, c, q_offset, rows, what):
    """Rows [r0, r1) of every batch: exact layout, valid kept sets, oracle agreement where unique."""
    r0, r1 = rows
    want = oracle.select_token_ids(iq, ck, lens, budget, c, q_offset, rows=rows)
    g = got[:, r0:r1]
    kb = budget // c
    scores = oracle.block_scores(iq, ck, rows=rows)
    eps = score_bounds(iq, ck, rows)
    B = g.shape[0]
    n_diff = 0
    for b in range(B):
        for ii in range(r1 - r0):
            t = q_offset + r0 + ii
            row, ref = g[b, ii], want[b, ii]
            nv = (t + 1) // c
            if t >= lens[b] or nv <= kb or kb == 0:
                assert (row == ref).all(), f"{what}: row {b},{r0 + ii} (dense/padding) differs"
                continue
            np.testing.assert_array_equal(row[kb * c:], ref[kb * c:], err_msg=f"{what}: tail slots of {b},{r0 + ii}")
            toks = row[:kb * c].reshape(kb, c)
            blocks = toks[:, 0] // c
            assert (toks == blocks[:, None] * c + np.arange(c)).all(), f"{what}: blocks not expanded"
            assert (np.diff(blocks) > 0).all() and blocks[-1] < nv, f"{what}: blocks not ascending / visible"
            if (row == ref).all():
                continue
            n_diff += 1
            s, e = scores[b, ii, :nv], eps[b, ii, :nv]
            kept = np.zeros(nv, bool)
            kept[blocks] = True
            lo = (s[kept] + e[kept]).min()
            hi = (s[~kept] - e[~kept]).max()
            assert lo >= hi, f"{what}: row {b},{r0 + ii} keeps a block that scores below an unkept one"
    return n_diff


# ------------------------------------------------------------ exact cases

EXACT_CASES = [  # B, S_q, H, D, c, budget, lens, q_offset, S_global
    (1, 64, 4, 64, 4, 8, (64,), 0, 64),
    (2, 200, 16, 128, 4, 32, (200, 131), 0, 200),      # ragged tiles, padding rows
    (1, 300, 20, 64, 2, 40, (1000,), 700, 1000),       # offset slice, H > 16 (two head groups)
    (1, 150, 64, 256, 8, 64, (150,), 0, 150),          # four head groups, D = 256
    (2, 97, 1, 64, 1, 16, (97, 50), 0, 97),            # c = 1: no tail slots
    (1, 129, 16, 128, 4, 3, (129,), 0, 129),           # budget < c: tails only
    (1, 600, 16, 64, 4, 1000, (600,), 0, 600),         # budget above every row's visible blocks
    (1, 2500, 8, 64, 2, 512, (2500,), 0, 2500),        # 1250 blocks: 5 score chunks, radix over 1250
    (1, 64, 4, 64, 1, 700, (17000,), 16360, 17000),    # rows across 16384 blocks: 256 x 64 and 1024 x 64 top-k
]


@pytest.mark.parametrize("case", EXACT_CASES, ids=lambda c: "x".join(map(str, c[:6])))
def test_select_exact_integer_inputs(case):
    B, S_q, H, D, c, budget, lens, q_offset, S_global = case
    print(f"select exact case {case}", flush=True)
    iq, ck = random_select_case(31 + S_q, B, S_q, H, D, S_global // c, integer=True)
    lens = np.array(lens, dtype=np.int64)
    got = run_gpu(iq, ck, lens, budget, c, q_offset, S_global)
    want = oracle.select_token_ids(iq, ck, lens, budget, c, q_offset)
    np.testing.assert_array_equal(got, want)


def _draw_select_cases(n: int, seed: int = 7_2026):
    """Seeded random selection shapes (integer inputs, so results must be exact), resampled while the
    oracle's work would exceed 4 GFLOP."""
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    while len(cases) < n:
        B, S_q = int(rng.integers(1, 4)), int(rng.integers(1, 500))
        H, D = int(rng.integers(1, 65)), int(rng.choice([64, 128, 256]))
        c = int(rng.choice([1, 2, 4, 8]))
        q_offset = int(rng.integers(0, 400)) if rng.random() < 0.4 else 0
        S_global = q_offset + S_q + (int(rng.integers(0, 100)) if q_offset else 0)
        budget = int(rng.integers(1, 700))
        lens = tuple(int(rng.integers(0, S_global + 1)) if rng.random() < 0.5 else S_global for _ in range(B))
        if 2.0 * B * S_q * (S_global // c) * H * D > 4e9:
            continue
        cases.append((B, S_q, H, D, c, budget, lens, q_offset, S_global, int(rng.integers(1, 1 << 30))))
    return cases


@pytest.mark.parametrize("case", _draw_select_cases(12),
                         ids=lambda c: "x".join(map(str, c[:6])) + f"_off{c[7]}")
def test_select_random_integer_shapes(case):
    B, S_q, H, D, c, budget, lens, q_offset, S_global, seed = case
    print(f"select random case {case}", flush=True)
    iq, ck = random_select_case(seed, B, S_q, H, D, max(S_global // c, 1), integer=True)
    lens = np.array(lens, dtype=np.int64)
    got = run_gpu(iq, ck, lens, budget, c, q_offset, S_global)
    np.testing.assert_array_equal(got, oracle.select_token_ids(iq, ck, lens, budget, c, q_offset))


def test_select_all_ties_keep_lowest_blocks():
    B, S_q, H, D, c, budget = 1, 256, 16, 128, 4, 40
    iq = np.zeros((B, S_q, H, D), np.uint16)
    ck = np.zeros((B, S_q // c, 1, D), np.uint16)
    lens = np.array([S_q], np.int64)
    got = run_gpu(iq, ck, lens, budget, c)
    np.testing.assert_array_equal(got, oracle.select_token_ids(iq, ck, lens, budget, c))
    assert (got[0, -1, :budget] == np.arange(budget)).all()


def test_select_fewer_nonzero_scores_than_the_budget():
    """Only every seventh block has a nonzero key, so many rows have fewer positive scores than kb
    blocks: every positive block is kept and the lowest-index zero-score blocks fill the rest."""
    B, S_q, H, D, c, budget = 1, 2600, 4, 64, 2, 512
    iq, ck = random_select_case(77, B, S_q, H, D, S_q // c, integer=True)
    ck[:, np.arange(S_q // c) % 7 != 0] = 0
    lens = np.array([S_q], np.int64)
    assert (oracle.block_scores(iq, ck, rows=(S_q - 1, S_q)) > 0).sum() < budget // c  # even the last row
    got = run_gpu(iq, ck, lens, budget, c)
    np.testing.assert_array_equal(got, oracle.select_token_ids(iq, ck, lens, budget, c))


def test_select_rows_at_the_topk_register_classes():
    """c = 1: rows see t + 1 blocks, so the rows cross every register width of the top-k (256 x 4 ..
    256 x 64 slots); rows on both sides of each boundary match the oracle exactly."""
    B, S_q, H, D, c, budget = 2, 9000, 2, 64, 1, 600
    iq, ck = random_select_case(78, B, S_q, H, D, S_q, integer=True)
    lens = np.array([S_q, 8500], np.int64)
    got = run_gpu(iq, ck, lens, budget, c)
    for edge in (1024, 2048, 4096, 8192, 9000):
        rows = (edge - 3, min(edge + 3, S_q))
        want = oracle.select_token_ids(iq, ck, lens, budget, c, rows=rows)
        np.testing.assert_array_equal(got[:, rows[0]:rows[1]], want, err_msg=f"rows {rows}")


def test_select_many_batch_rows_one_topk_launch():
    """33 batch rows that each span two register widths (66 runs) take one launch at the widest."""
    B, S_q, H, D, c, budget = 33, 1100, 2, 64, 1, 256
    iq, ck = random_select_case(79, B, S_q, H, D, S_q, integer=True)
    lens = np.full(B, S_q, np.int64)
    lens[5] = 600
    got = run_gpu(iq, ck, lens, budget, c)
    rows = (1000, S_q)
    want = oracle.select_token_ids(iq, ck, lens, budget, c, rows=rows)
    np.testing.assert_array_equal(got[:, rows[0]:rows[1]], want)
    np.testing.assert_array_equal(got[:, 240:260], oracle.select_token_ids(iq, ck, lens, budget, c, rows=(240, 260)))


def test_select_radix_digits_and_boundary_bins():
    """Scores hi + lo with hi in {0, 2^10, 2^20, 2^21} and lo an integer below 256: clusters whose
    members differ only in the 2nd (2^10 + lo) or the 3rd (2^20 + lo) radix digit, and many exact
    duplicates.  The rows see 2001..2064 blocks and four budgets put the kb-th largest value between
    clusters (row 30 then needs exactly the 2^21 cluster: the first digit's bin is taken whole) and
    inside each cluster, so the search ends after the first, second or third digit, with the
    boundary bin taken whole or split between equal values by the lowest-index rule.  Must equal
    the oracle exactly."""
    B, S_q, H, D, c, q_offset = 1, 64, 1, 64, 1, 2000
    n_blocks = q_offset + S_q
    rng = np.random.Generator(np.random.PCG64(2026_12))
    hi = rng.choice(np.array([0.0, 2.0 ** 10, 2.0 ** 20, 2.0 ** 21], np.float32), size=n_blocks, p=[0.3, 0.3, 0.3, 0.1])
    lo = rng.integers(0, 256, size=n_blocks).astype(np.float32)
    ck = np.zeros((B, n_blocks, 1, D), np.uint16)
    ck[0, :, 0, 0] = float32_to_bf16_bits(hi)  # powers of two and integers below 256 are exact in bf16
    ck[0, :, 0, 1] = float32_to_bf16_bits(lo)
    iq = np.zeros((B, S_q, H, D), np.uint16)
    iq[..., 0:2] = float32_to_bf16_bits(np.float32(1.0))  # score of block j = hi_j + lo_j, exact in fp32
    lens = np.array([n_blocks], np.int64)
    top_cluster = int((hi[:q_offset + 31] == 2.0 ** 21).sum())  # blocks of the 2^21 cluster row 30 sees
    for budget in (top_cluster, 300, 1000, 1500):
        print(f"select radix case budget {budget}", flush=True)
        got = run_gpu(iq, ck, lens, budget, c, q_offset, n_blocks)
        np.testing.assert_array_equal(got, oracle.select_token_ids(iq, ck, lens, budget, c, q_offset),
                                      err_msg=f"budget {budget}")


# --------------------------------------------------------- continuous cases

CONT_CASES = [  # B, S_q, H, D, c, budget
    (2, 512, 16, 128, 4, 64),
    (1, 1024, 8, 64, 4, 128),
    (1, 700, 32, 128, 2, 100),
]


@pytest.mark.parametrize("case", CONT_CASES, ids=lambda c: "x".join(map(str, c)))
def test_select_continuous_inputs(case):
    B, S_q, H, D, c, budget = case
    print(f"select continuous case {case}", flush=True)
    iq, ck = random_select_case(77 + S_q, B, S_q, H, D, S_q // c)
    lens = np.array([S_q] + [S_q - 37] * (B - 1), dtype=np.int64)
    got = run_gpu(iq, ck, lens, budget, c)
    n_diff = check_rows(got, iq, ck, lens, budget, c, 0, (0, S_q), "continuous")
    assert n_diff <= 0.02 * B * S_q, f"{n_diff} rows differ from the oracle"


@pytest.mark.parametrize("case", _draw_select_cases(6, seed=8_2026),
                         ids=lambda c: "x".join(map(str, c[:6])) + f"_off{c[7]}")
def test_select_random_continuous_shapes(case):
    B, S_q, H, D, c, budget, lens, q_offset, S_global, seed = case
    print(f"select random continuous case {case}", flush=True)
    iq, ck = random_select_case(seed, B, S_q, H, D, max(S_global // c, 1))
    lens = np.array(lens, dtype=np.int64)
    got = run_gpu(iq, ck, lens, budget, c, q_offset, S_global)
    n_diff = check_rows(got, iq, ck, lens, budget, c, q_offset, (0, S_q), "random continuous")
    assert n_diff <= 0.02 * B * S_q + 1, f"{n_diff} rows differ from the oracle"


def test_select_chunked_equals_one_pass():
    B, S_q, H, D, c, budget = 2, 777, 16, 128, 4, 64
    iq, ck = random_select_case(5, B, S_q, H, D, S_q // c)
    lens = np.array([777, 500], dtype=np.int64)
    full = run_gpu(iq, ck, lens, budget, c)
    for chunk in (1, 16, 100, 400):
        np.testing.assert_array_equal(run_gpu(iq, ck, lens, budget, c, chunk=chunk), full, err_msg=f"chunk {chunk}")


def test_select_strided_inputs():
    B, S_q, H, D, c, budget = 1, 256, 16, 64, 4, 32
    iq, ck = random_select_case(9, B, S_q, H, D, S_q // c, integer=True)
    lens = np.array([S_q], np.int64)
    want = oracle.select_token_ids(iq, ck, lens, budget, c)
    # head-major queries and keys padded per block: non-contiguous views with unit last stride
    iq_t = bf16_to_gpu(np.ascontiguousarray(iq.transpose(0, 2, 1, 3))).transpose(1, 2)
    ck_pad = np.zeros((B, S_q // c, 1, D + 64), np.uint16)
    ck_pad[..., :D] = ck
    ck_t = bf16_to_gpu(ck_pad)[..., :D]
    out = qsa.qsa_select_token_ids(iq_t, ck_t, torch.tensor([S_q], device=device()), budget, c)
    np.testing.assert_array_equal(out.cpu().numpy(), want)


# ------------------------------------------------------------- workloads

_inputs = functools.lru_cache(maxsize=1)(make_select_inputs)

def _structure(got, lens, budget, c, q_offset):
    """Every row: kept blocks ascending, complete and visible; tail and -1 layout exact."""
    B, S_q, W = got.shape
    kb = budget // c
    t = q_offset + np.arange(S_q)
    nv = (t + 1) // c
    m = np.minimum(kb, nv)
    for b in range(B):
        g = got[b]
        pad = t >= lens[b]
        assert (g[pad] == -1).all()
        live = ~pad
        slot = np.arange(W)[None, :]
        block_slots = slot < (m * c)[:, None]
        assert ((g >= 0) == (block_slots | ((slot >= budget) & (slot - budget < ((t + 1) - nv * c)[:, None]))))[live].all()
        tail_ok = np.where(slot >= budget, g == (nv * c)[:, None] + slot - budget, True)
        assert (tail_ok | (g == -1))[live].all()
        blocks = g[:, :kb * c:c] // c if kb else np.zeros((S_q, 0), int)
        for i in np.nonzero(live)[0][::97]:
            bl = blocks[i, :m[i]]
            assert (np.diff(bl) > 0).all() and (bl < nv[i]).all() and (bl >= 0).all()
            toks = g[i, :m[i] * c].reshape(-1, c)
            assert (toks == bl[:, None] * c + np.arange(c)).all()


@pytest.mark.parametrize("name", list(SELECT_WORKLOADS))
def test_select_workload(name):
    w, iq, ck, lens = _inputs(name)
    print(f"select workload {name}", flush=True)
    got = run_gpu(iq, ck, lens, w.token_budget, w.compress_ratio, w.q_offset, w.S_global)
    _structure(got, lens, w.token_budget, w.compress_ratio, w.q_offset)
    kb = w.token_budget // w.compress_ratio
    first_sparse = max(0, (kb + 1) * w.compress_ratio - 1 - w.q_offset)
    samples = [(0, min(32, w.S_q)), (max(0, first_sparse - 8), min(w.S_q, first_sparse + 24)),
               (w.S_q // 2, w.S_q // 2 + 32), (w.S_q - 32, w.S_q)]
    n_rows = n_diff = 0
    for rows in samples:
        n_diff += check_rows(got, iq, ck, lens, w.token_budget, w.compress_ratio, w.q_offset, rows, name)
        n_rows += w.B * (rows[1] - rows[0])
    assert n_diff <= max(2, 0.05 * n_rows), f"{name}: {n_diff} of {n_rows} sampled rows differ from the oracle"
    if name != "sel_long":  # the long workload's one-pass workspace is 4 GiB; its passes are checked below
        again = run_gpu(iq, ck, lens, w.token_budget, w.compress_ratio, w.q_offset, w.S_global, chunk=1000)
        np.testing.assert_array_equal(again, got)


def test_select_long_in_passes_equals_one_pass():
    w, iq, ck, lens = _inputs("sel_long")
    full = run_gpu(iq, ck, lens, w.token_budget, w.compress_ratio, w.q_offset, w.S_global)
    parts = run_gpu(iq, ck, lens, w.token_budget, w.compress_ratio, w.q_offset, w.S_global, chunk=8192)
    np.testing.assert_array_equal(parts, full)


# ------------------------------------------------------ selection -> attention

def test_selected_routes_feed_attention():
    """The selected IDs are routes: attention over them matches the oracle on the same IDs."""
    B, S, H_i, D_i, c, budget, Hq, Hkv, D = 2, 384, 8, 64, 4, 64, 8, 2, 128
    iq, ck = random_select_case(3, B, S, H_i, D_i, S // c)
    lens = np.array([384, 300], np.int64)
    routes = qsa.qsa_select_token_ids(bf16_to_gpu(iq), bf16_to_gpu(ck), torch.from_numpy(lens).to(device()),
                                      budget, c)
    rng = np.random.Generator(np.random.PCG64(4))
    q, k, v = (float32_to_bf16_bits(rng.standard_normal(s, dtype=np.float32))
               for s in ((B, S, Hq, D), (B, S, Hkv, D), (B, S, Hkv, D)))
    out = qsa.qsa_forward(bf16_to_gpu(q), bf16_to_gpu(k), bf16_to_gpu(v), routes)
    torch.cuda.synchronize()
    r = routes.cpu().numpy()
    ref = oracle.forward(q, k, v, r, 1.0 / np.sqrt(D))
    counts = oracle.route_lists(r, S)[1]
    got = out.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    check_forward(got, ref, counts, v, "selected routes")
    assert (counts[1, 300:] == 0).all() and (counts[0] > 0).all()
