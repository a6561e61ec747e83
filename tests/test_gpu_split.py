"""GPU parity of the attention's key-range split.

When one KV head's K and V rows exceed 16 MiB (S_kv * 4 * D bytes), the
attention cuts each row's list into key ranges of W IDs, computes one
partial result per range that holds routes, and merges the partials
(include/qsa.h, qsa_attention_workspace_size).  Checked here:

* output within the BF16 tolerance and lse within 2^-8 + 2^-9 of the fp64
  oracle, on routes whose rows span one range, a few, or all of them, with
  empty rows bitwise +0.0 (lse -inf), for every head dimension;
* the rows processed in several passes (a workspace of the smallest pass
  and others) give the same bits as one pass;
* the range-start table the split writes into the workspace equals a numpy
  searchsorted of the oracle's lists at the range boundaries;
* a missing or too small workspace is refused before anything runs.
"""

from __future__ import annotations

import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
import route_sparse_gqa_amd as qsa
from gpu_util import bf16_to_gpu, check_forward, device, gpu_bf16_bits
from test_gpu_backward import check_lse
from workloads.generators import random_small_case, random_windowed_routes

pytestmark = pytest.mark.gpu

CASES = [  # (B, S_q, S_kv, Hq, Hkv, D, K): S_kv * 4 * D > 16 MiB
    (1, 40, 20000, 16, 2, 256, 600),   # W = 4096: 5 ranges, the last ragged
    (2, 33, 45000, 8, 1, 128, 900),    # W = 8192: 6 ranges
    (1, 50, 90000, 4, 2, 64, 2000),    # W = 16384: 6 ranges
    (1, 60, 16385, 16, 2, 256, 40),    # one key past four ranges
    (3, 70, 26000, 12, 3, 256, 300),   # G = 4, 7 ranges
    (1, 30, 33000, 16, 1, 256, 1500),  # G = 16, 9 ranges
]


def _ids(c):
    return "B{}_Sq{}_Skv{}_Hq{}_Hkv{}_D{}_K{}".format(*c)


def _ranges(S_kv: int, D: int):
    """W and P as include/qsa.h states them."""
    W = 1
    while 2 * W * 4 * D <= 4 << 20:
        W *= 2
    while -(-S_kv // W) > 63:
        W *= 2
    return W, -(-S_kv // W)  # the split runs when there are at least 5 ranges


def _case(seed, case):
    B, S_q, S_kv, Hq, Hkv, D, K = case
    q, k, v, _ = random_small_case(seed, B, S_q, S_kv, Hq, Hkv, D, 1)
    r = random_windowed_routes(seed + 1, B, S_q, S_kv, K)
    r[:, 1::2, 0] = S_kv - 1  # every other row also routes the last key (the last, ragged range)
    r[:, ::5] = -1  # and every fifth row is empty
    return q, k, v, r


def _attention(qg, kg, vg, lst, cnt, case, scale, ws_bytes=None, lse=True):
    B, S_q, S_kv, Hq, Hkv, D, K = case
    need = qsa.qsa_attention_workspace_size(*case)
    ws = torch.empty(need if ws_bytes is None else ws_bytes, dtype=torch.uint8, device=device())
    out, lse_t = qsa.qsa_forward_preprocessed(qg, kg, vg, lst, cnt, scale, return_lse=True, workspace=ws)
    return out, lse_t, ws


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_split_matches_oracle(case):
    B, S_q, S_kv, Hq, Hkv, D, K = case
    W, P = _ranges(S_kv, D)
    assert P >= 5 and qsa.qsa_attention_workspace_size(*case) > 0
    print(f"split forward {case}: W={W} P={P}", flush=True)
    q, k, v, r = _case(3000 + sum(case), case)
    scale = 1.0 / math.sqrt(D)
    qg, kg, vg = bf16_to_gpu(q), bf16_to_gpu(k), bf16_to_gpu(v)
    lst, cnt, _, _ = qsa.qsa_preprocess(torch.from_numpy(r).to(device()), S_kv)
    out, lse, _ = _attention(qg, kg, vg, lst, cnt, case, scale)
    fused = qsa.qsa_forward(qg, kg, vg, torch.from_numpy(r).to(device()), scale)
    torch.cuda.synchronize()
    olst, ocnt = oracle.route_lists(r, S_kv)
    spans = {}
    for b in range(B):
        for i in range(S_q):
            n = ocnt[b, i]
            key = 0 if n == 0 else int(olst[b, i, n - 1] // W - olst[b, i, 0] // W + 1)
            spans[key] = spans.get(key, 0) + 1
    print(f"  rows by number of ranges spanned: {dict(sorted(spans.items()))}", flush=True)
    assert spans.get(0, 0) > 0 and spans.get(1, 0) > 0 and max(spans) >= 2  # empty, direct and merged rows
    check_forward(gpu_bf16_bits(out), oracle.forward(q, k, v, r, scale), ocnt, v, f"split {case}")
    check_lse(lse.cpu().numpy().astype(np.float64), oracle.lse(q, k, r, scale), f"split lse {case}")
    assert torch.equal(out.view(torch.int16), fused.view(torch.int16)), "qsa_forward differs from the two calls"


def test_split_passes_are_bit_identical():
    case = (2, 700, 20000, 16, 2, 256, 300)
    B, S_q, S_kv, Hq, Hkv, D, K = case
    W, P = _ranges(S_kv, D)
    print(f"split passes {case}", flush=True)
    q, k, v, r = _case(77, case)
    qg, kg, vg = bf16_to_gpu(q), bf16_to_gpu(k), bf16_to_gpu(v)
    lst, cnt, _, _ = qsa.qsa_preprocess(torch.from_numpy(r).to(device()), S_kv)
    full = qsa.qsa_attention_workspace_size(*case)
    rows = B * S_q
    r256 = lambda x: -(-x // 256) * 256
    per_pass = lambda pr: r256(4 * rows * (P + 1)) + (2 if pr < rows else 1) * (r256(2 * pr * Hq * P * D) +
                                                                                r256(4 * pr * Hq * P))
    assert full == per_pass(rows)  # every row fits the recommended size: one pass
    one, lse1, _ = _attention(qg, kg, vg, lst, cnt, case, 0.0625)
    for pass_rows in (256, 300, 1000):  # 6, 5 and 2 passes of the 1400 rows
        got, lse2, _ = _attention(qg, kg, vg, lst, cnt, case, 0.0625, ws_bytes=per_pass(pass_rows) + 512)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), one.view(torch.int16)), f"passes of {pass_rows} rows differ"
        assert torch.equal(lse2, lse1), f"lse with passes of {pass_rows} rows differs"
    ref = oracle.forward(q, k, v, r, 0.0625)
    check_forward(gpu_bf16_bits(one), ref, oracle.route_lists(r, S_kv)[1], v, "split one pass")


@pytest.mark.parametrize("K", [500, 501], ids=["K500_rows16B", "K501_rows4B"])  # one load per 4 entries, or per 1
def test_split_range_start_table(K):
    case = (1, 90, 26000, 8, 2, 256, K)
    B, S_q, S_kv, Hq, Hkv, D, K = case
    W, P = _ranges(S_kv, D)
    q, k, v, r = _case(11, case)
    lst, cnt, _, _ = qsa.qsa_preprocess(torch.from_numpy(r).to(device()), S_kv)
    _, _, ws = _attention(bf16_to_gpu(q), bf16_to_gpu(k), bf16_to_gpu(v), lst, cnt, case, 0.0625)
    torch.cuda.synchronize()
    table = ws[:4 * B * S_q * (P + 1)].cpu().numpy().view(np.int32).reshape(B * S_q, P + 1)
    olst, ocnt = oracle.route_lists(r, S_kv)
    for row in range(B * S_q):
        b, i = divmod(row, S_q)
        ids = olst[b, i, :ocnt[b, i]]
        want = np.searchsorted(ids, np.arange(P) * W, side="left").tolist() + [int(ocnt[b, i])]
        assert table[row].tolist() == want, f"row {row}"


def test_split_workspace_refused():
    case = (1, 600, 20000, 16, 2, 256, 64)
    B, S_q, S_kv, Hq, Hkv, D, K = case
    q, k, v, r = _case(5, case)
    qg, kg, vg = bf16_to_gpu(q), bf16_to_gpu(k), bf16_to_gpu(v)
    lst, cnt, _, _ = qsa.qsa_preprocess(torch.from_numpy(r).to(device()), S_kv)
    W, P = _ranges(S_kv, D)
    r256 = lambda x: -(-x // 256) * 256
    # two partial buffers of the smallest pass (256 rows), less than one buffer of all 600 rows
    smallest = r256(4 * B * S_q * (P + 1)) + 2 * (r256(2 * 256 * Hq * P * D) + r256(4 * 256 * Hq * P)) + 512
    out = torch.empty((B, S_q, Hq, D), dtype=torch.bfloat16, device=device())
    st = lambda t: (ctypes.c_int64 * t.dim())(*t.stride())
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    ws = torch.empty(smallest, dtype=torch.uint8, device=device())

    def call(ws_ptr, nbytes):
        return qsa.lib().qsa_forward_preprocessed(p(qg), st(qg), p(kg), st(kg), p(vg), st(vg), p(lst), p(cnt), B,
                                                  S_q, S_kv, Hq, Hkv, D, K, ctypes.c_float(0.1), p(out), None,
                                                  ws_ptr, nbytes, None)

    assert call(None, 0) == -10
    assert call(p(ws), smallest - 1024) == -10
    assert call(ctypes.c_void_p(ws.data_ptr() + 16), smallest - 256) == -10  # not 256-B aligned
    assert call(p(ws), smallest) == 0
    out = ws[:2 * B * S_q * Hq * D].view(torch.bfloat16)  # the output inside the workspace: refused
    assert call(p(ws), smallest) == -9
    torch.cuda.synchronize()


BACKWARD_CASES = [  # (B, S_q, S_kv, Hq, Hkv, D, K): the backward's dq takes the same key-range split
    (1, 40, 20000, 16, 2, 256, 600),
    (2, 33, 45000, 8, 1, 128, 900),
    (1, 50, 90000, 4, 2, 64, 2000),
    (1, 8200, 16400, 2, 1, 256, 4),   # more than 8192 rows: dq in three passes of up to 4096 (the last of 8)
]


@pytest.mark.parametrize("case", BACKWARD_CASES, ids=_ids)
def test_split_backward_matches_oracle(case):
    from test_gpu_backward import check_grad
    from workloads import random_dout

    B, S_q, S_kv, Hq, Hkv, D, K = case
    W, P = _ranges(S_kv, D)
    assert P >= 5
    print(f"split backward {case}: W={W} P={P}", flush=True)
    q, k, v, r = _case(7000 + sum(case), case)
    dout = random_dout(8000 + sum(case), q.shape)
    scale = 1.0 / math.sqrt(D)
    qg, kg, vg, gg = bf16_to_gpu(q), bf16_to_gpu(k), bf16_to_gpu(v), bf16_to_gpu(dout)
    lst, cnt, _, _ = qsa.qsa_preprocess(torch.from_numpy(r).to(device()), S_kv)
    out, lse = qsa.qsa_forward_preprocessed(qg, kg, vg, lst, cnt, scale, return_lse=True)
    dq, dk, dv = qsa.qsa_backward(qg, kg, vg, out, gg, lse, lst, cnt, scale)
    dq2, dk2, dv2 = qsa.qsa_backward(qg, kg, vg, out, gg, lse, lst, cnt, scale)
    torch.cuda.synchronize()
    for a, b2, name in ((dq, dq2, "dq"), (dk, dk2, "dk"), (dv, dv2, "dv")):
        assert torch.equal(a.view(torch.int16), b2.view(torch.int16)), f"{name} differs between two calls"
    _, ocnt = oracle.route_lists(r, S_kv)
    rq, rk, rv = oracle.backward(q, k, v, dout, r, scale)
    floor = 1e-3 * float(np.abs(rv).max())
    dq_b = gpu_bf16_bits(dq)
    check_grad(dq_b, rq, f"split {case} dq", floor)
    check_grad(gpu_bf16_bits(dk), rk, f"split {case} dk", floor)
    check_grad(gpu_bf16_bits(dv), rv, f"split {case} dv")
    assert not np.any(dq_b[ocnt == 0]), "empty rows must have dq exactly +0.0"
