"""GPU parity of the backward pass (and the forward's log-sum-exp) against the fp64 oracle.

* lse: within 2^-8 + 2^-9 of the oracle's (absolute, natural log).  The
  forward sums bf16-rounded probabilities; bf16 keeps 8 significant bits, so
  each is within 2^-8 relative and the log of their sum moves by at most
  2^-8; the fp32 scores and sums get a further 2^-9.  -inf exactly for
  empty rows;
* dq, dk, dv (bf16): max |err| <= 1e-2 * Y and mean |err| <= 1e-3 * Y per
  tensor, against the unrounded fp64 gradients, with the yardstick Y =
  max|ref|; for dq and dk, whose exact value can vanish (every row with a
  single route gives p = 1 and ds = 0 while the GPU's fp32 dp - delta is
  only zero up to rounding), Y is floored at 1e-3 * max|dv_ref| (dv is a
  p-weighted sum of the upstream gradient, so it carries that gradient's
  scale);
* rows with no valid route have dq exactly +0.0, keys no row routes have dk
  and dv exactly +0.0;
* the backward is deterministic: a second call gives the same bits;
* the key segments it builds (read back from the workspace) are exactly the
  (row, 64-key tile, key mask) triples of the route lists, rows ascending
  within each tile.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import route_sparse_gqa_amd as qsa
from gpu_util import bf16_to_gpu, bits_to_f64, device, gpu_bf16_bits
from workloads import WORKLOADS, make_dout, make_inputs, random_dout
from workloads.generators import random_small_case

pytestmark = pytest.mark.gpu

LSE_ABS_ERR = 2.0 ** -8 + 2.0 ** -9
GRAD_MAX_ERR_FRACTION = 1e-2
GRAD_MEAN_ERR_FRACTION = 1e-3

CASES = [  # (B, S_q, S_kv, Hq, Hkv, D, K): every D, G in {1, 2, 3, 4, 8, 16}, ragged tiles
    (1, 37, 45, 4, 1, 64, 19),
    (2, 130, 300, 16, 2, 256, 77),
    (1, 64, 200, 8, 8, 128, 40),
    (2, 33, 129, 32, 2, 64, 33),
    (1, 50, 70, 12, 3, 128, 65),
    (1, 40, 77, 6, 2, 64, 30),
    (1, 20, 1000, 2, 1, 256, 600),
    (1, 3, 1, 2, 1, 64, 5),
    (1, 1, 9, 16, 1, 256, 1),
    (3, 257, 513, 8, 1, 256, 129),
]


def _ids(case):
    return "B{}_Sq{}_Skv{}_Hq{}_Hkv{}_D{}_K{}".format(*case)


def check_grad(got_bits: np.ndarray, ref: np.ndarray, what: str, floor: float = 0.0):
    got = bits_to_f64(got_bits)
    assert np.all(np.isfinite(got)), f"{what}: non-finite gradient"
    scale = max(float(np.abs(ref).max()) if ref.size else 0.0, floor)
    err = np.abs(got - ref)
    worst = float(err.max()) if err.size else 0.0
    mean = float(err.mean()) if err.size else 0.0
    assert worst <= GRAD_MAX_ERR_FRACTION * scale + 1e-30, f"{what}: max|err| {worst:.3e} > 1e-2 * {scale:.3e}"
    assert mean <= GRAD_MEAN_ERR_FRACTION * scale + 1e-30, f"{what}: mean|err| {mean:.3e} > 1e-3 * {scale:.3e}"
    return worst / scale if scale else 0.0


def check_lse(got: np.ndarray, ref: np.ndarray, what: str):
    empty = np.isneginf(ref)
    assert np.all(np.isneginf(got[empty])), f"{what}: empty rows must have lse = -inf"
    assert np.all(np.isfinite(got[~empty])), f"{what}: non-finite lse"
    if (~empty).any():
        worst = float(np.abs(got[~empty] - ref[~empty]).max())
        assert worst <= LSE_ABS_ERR, f"{what}: lse max|err| {worst:.3e} > {LSE_ABS_ERR}"


def run_forward_backward(q, k, v, r, dout, scale, ws=None):
    qg, kg, vg, gg = bf16_to_gpu(q), bf16_to_gpu(k), bf16_to_gpu(v), bf16_to_gpu(dout)
    lst, cnt, _, _ = qsa.qsa_preprocess(torch.from_numpy(r).to(device()), k.shape[1])
    out, lse = qsa.qsa_forward_preprocessed(qg, kg, vg, lst, cnt, scale, return_lse=True)
    dq, dk, dv = qsa.qsa_backward(qg, kg, vg, out, gg, lse, lst, cnt, scale, workspace=ws)
    return (qg, kg, vg, gg, lst, cnt, out, lse), (dq, dk, dv)


def _r256(x):
    return -(-x // 256) * 256


def read_segments(ws: torch.Tensor, B, S_q, S_kv, Hq):
    """tile_start and segments from the documented workspace layout."""
    n_kt, n_w, n_c = -(-S_kv // 64), -(-S_q // 32), -(-S_q // 256)
    # delta, bit matrix, chunk prefixes, tile totals, then tile starts and segments
    off = _r256(4 * B * S_q * Hq) + _r256(4 * B * n_w * n_kt) + _r256(4 * B * n_c * n_kt) + _r256(4 * B * n_kt)
    w = ws.cpu().numpy()
    start = w[off:off + 4 * (B * n_kt + 1)].view(np.int32)
    off += _r256(4 * (B * n_kt + 1))
    total = int(start[-1])
    rec = w[off:off + 16 * total].view(np.int32).reshape(total, 4)
    segs = [(int(e[0]), int(np.uint32(e[1])) | (int(np.uint32(e[2])) << 32)) for e in rec]
    assert not rec[:, 3].any(), "segment padding must be zero"
    return n_kt, start, segs


def expected_segments(lst: np.ndarray, cnt: np.ndarray, n_kt: int):
    """{(b, tile): [(row, mask), ...]} with rows ascending, from the oracle's lists."""
    B, S_q, _ = lst.shape
    out = {}
    for b in range(B):
        for i in range(S_q):
            for key in lst[b, i, :cnt[b, i]]:
                t = int(key) // 64
                e = out.setdefault((b, t), [])
                if e and e[-1][0] == i:
                    e[-1] = (i, e[-1][1] | (1 << (int(key) % 64)))
                else:
                    e.append((i, 1 << (int(key) % 64)))
    return out


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_backward_matches_oracle(case):
    B, S_q, S_kv, Hq, Hkv, D, K = case
    print(f"backward case {case}", flush=True)
    q, k, v, r = random_small_case(3000 + sum(case), B, S_q, S_kv, Hq, Hkv, D, K)
    dout = random_dout(4000 + sum(case), q.shape)
    scale = 1.0 / math.sqrt(D)
    ws = torch.empty(qsa.qsa_backward_workspace_size(B, S_q, S_kv, Hq, Hkv, D, K), dtype=torch.uint8,
                     device=device())
    (qg, kg, vg, gg, lst, cnt, out, lse), (dq, dk, dv) = run_forward_backward(q, k, v, r, dout, scale, ws)
    torch.cuda.synchronize()

    olst, ocnt = oracle.route_lists(r, S_kv)
    check_lse(lse.cpu().numpy().astype(np.float64), oracle.lse(q, k, r, scale), f"{case} lse")
    rq, rk, rv = oracle.backward(q, k, v, dout, r, scale)
    dq_b, dk_b, dv_b = gpu_bf16_bits(dq), gpu_bf16_bits(dk), gpu_bf16_bits(dv)
    floor = 1e-3 * float(np.abs(rv).max())
    check_grad(dq_b, rq, f"{case} dq", floor)
    check_grad(dk_b, rk, f"{case} dk", floor)
    check_grad(dv_b, rv, f"{case} dv")
    assert not np.any(dq_b[ocnt == 0]), "empty rows must have dq exactly +0.0"
    routed = np.zeros((B, S_kv), dtype=bool)
    for b in range(B):
        for i in range(S_q):
            routed[b, olst[b, i, :ocnt[b, i]]] = True
    assert not np.any(dk_b[~routed]) and not np.any(dv_b[~routed]), "unrouted keys must have dk = dv = +0.0"

    # key segments, exactly
    n_kt, start, segs = read_segments(ws, B, S_q, S_kv, Hq)
    want = expected_segments(olst, ocnt, n_kt)
    assert int(start[-1]) == sum(len(x) for x in want.values())
    for b in range(B):
        for t in range(n_kt):
            got = segs[start[b * n_kt + t]:start[b * n_kt + t + 1]]
            assert got == want.get((b, t), []), f"segments of (b={b}, tile={t}) differ"

    # determinism: a second backward gives the same bits
    dq2, dk2, dv2 = qsa.qsa_backward(qg, kg, vg, out, gg, lse, lst, cnt, scale)
    for a, b2, name in ((dq, dq2, "dq"), (dk, dk2, "dk"), (dv, dv2, "dv")):
        assert torch.equal(a.view(torch.int16), b2.view(torch.int16)), f"{name} differs between two calls"


def test_backward_single_route_closed_form():
    """One valid route per row: p = 1, so dq and dk vanish up to rounding and dv collects dout."""
    B, S_q, S_kv, Hq, Hkv, D = 1, 64, 40, 8, 2, 128
    q, k, v, _ = random_small_case(5001, B, S_q, S_kv, Hq, Hkv, D, 4)
    rng = np.random.Generator(np.random.PCG64(5002))
    ids = rng.integers(0, S_kv, size=(B, S_q))
    r = np.stack([ids, np.full_like(ids, -1), ids, np.full_like(ids, S_kv)], axis=-1)
    dout = random_dout(5003, q.shape)
    _, (dq, dk, dv) = run_forward_backward(q, k, v, r, dout, 0.1)
    rq, rk, rv = oracle.backward(q, k, v, dout, r, 0.1)
    dvb = gpu_bf16_bits(dv)
    check_grad(dvb, rv, "single-route dv")
    tol = GRAD_MAX_ERR_FRACTION * float(np.abs(rv).max())
    assert float(np.abs(bits_to_f64(gpu_bf16_bits(dq))).max()) <= tol
    assert float(np.abs(bits_to_f64(gpu_bf16_bits(dk))).max()) <= tol


def test_backward_strided_inputs():
    """Head-major Q/dO views and interleaved K/V give the same gradients as contiguous copies."""
    B, S_q, S_kv, Hq, Hkv, D, K = 1, 48, 96, 8, 2, 64, 24
    q, k, v, r = random_small_case(5101, B, S_q, S_kv, Hq, Hkv, D, K)
    dout = random_dout(5102, q.shape)
    (qg, kg, vg, gg, lst, cnt, out, lse), (dq, dk, dv) = run_forward_backward(q, k, v, r, dout, 0.125)
    q_hm = qg.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    g_hm = gg.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    kv = torch.stack([kg, vg], dim=3).reshape(B, S_kv, 2 * Hkv, D)  # K and V rows interleaved per head
    dq2, dk2, dv2 = qsa.qsa_backward(q_hm, kv[:, :, 0::2], kv[:, :, 1::2], out, g_hm, lse, lst, cnt, 0.125)
    for a, b2, name in ((dq, dq2, "dq"), (dk, dk2, "dk"), (dv, dv2, "dv")):
        assert torch.equal(a.view(torch.int16), b2.view(torch.int16)), f"strided {name} differs"


BACKWARD_SAMPLES = {  # workload: (dq row ranges, dk/dv key ranges), every batch row
    "right_padded": ([(0, 128), (2990, 3010), (3968, 4096)], [(2048, 2112), (3968, 4096)]),
    "packed_thd": ([(0, 64), (16000, 16384)], [(16256, 16384)]),
    "cp_slice": ([(0, 64), (8128, 8192)], [(32704, 32768)]),
    "long_int64": ([(65024, 65536)], [(65472, 65536)]),
}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", list(BACKWARD_SAMPLES))
def test_backward_workload_samples(name):
    w = WORKLOADS[name]
    print(f"[{name}] backward at full size", flush=True)
    _, q, k, v, r = make_inputs(name)
    dout = make_dout(w)
    (_, _, _, _, lst, cnt, out, lse), (dq, dk, dv) = run_forward_backward(q, k, v, r, dout, w.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(dq.float()).all() and torch.isfinite(dk.float()).all() and torch.isfinite(dv.float()).all()
    rows, keys = BACKWARD_SAMPLES[name]
    lse_h = lse.cpu().numpy().astype(np.float64)
    for (r0, r1) in rows:
        print(f"[{name}] dq and lse rows [{r0}, {r1}) vs oracle", flush=True)
        check_lse(lse_h[:, r0:r1], oracle.lse(q, k, r, w.scale, rows=(r0, r1)), f"{name} lse [{r0},{r1})")
        rq, _, _ = oracle.backward(q, k, v, dout, r, w.scale, rows=(r0, r1), keys=(0, 0))
        check_grad(gpu_bf16_bits(dq[:, r0:r1]), rq, f"{name} dq rows [{r0},{r1})")
    for (k0, k1) in keys:
        print(f"[{name}] dk, dv keys [{k0}, {k1}) vs oracle", flush=True)
        _, rk, rv = oracle.backward(q, k, v, dout, r, w.scale, rows=(0, 0), keys=(k0, k1))
        check_grad(gpu_bf16_bits(dk[:, k0:k1]), rk, f"{name} dk keys [{k0},{k1})")
        check_grad(gpu_bf16_bits(dv[:, k0:k1]), rv, f"{name} dv keys [{k0},{k1})")
    print(f"[{name}] ok", flush=True)
