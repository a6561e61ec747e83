"""GPU parity on a seeded sweep of random small shapes.

The hand-picked cases elsewhere cover each boundary on purpose; this sweep
draws the dimensions together (batch, rows, keys, group size, head dim, route
slots, route dtype, scale, share of invalid slots and empty rows) so that
combinations nobody picked are exercised too.  Every case checks the whole
path against the fp64 oracle: preprocessing bit for bit (lists, counts,
membership, tile classes), the forward and its log-sum-exp within their
tolerances, and the three gradients within theirs.  A second sweep draws
key ranges up to 140000 and up to 5000 route slots, across every
route-normalisation path (one wavefront per row, the two bitmap sizes, the
sort), and checks preprocessing alone, bit for bit.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import route_sparse_gqa_amd as qsa
from gpu_util import bf16_to_gpu, check_forward, device, gpu_bf16_bits
from test_gpu_backward import check_grad, check_lse
from workloads import random_dout
from workloads.generators import random_small_case

pytestmark = pytest.mark.gpu


def _draw_cases(n: int, seed: int = 20261202):
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for _ in range(n):
        G = int(rng.choice([1, 2, 4, 8, 16]))
        Hkv = int(rng.integers(1, 3 if G == 16 else 4))
        cases.append(dict(
            B=int(rng.integers(1, 4)), S_q=int(rng.integers(1, 161)), S_kv=int(rng.integers(1, 1501)),
            Hq=G * Hkv, Hkv=Hkv, D=int(rng.choice([64, 128, 256])), K=int(rng.integers(1, 601)),
            dtype=np.int32 if rng.random() < 0.5 else np.int64, scale=float(rng.uniform(0.02, 0.5)),
            p_invalid=float(rng.uniform(0.0, 0.5)), p_empty=float(rng.uniform(0.0, 0.3)),
            seed=int(rng.integers(1, 1 << 30))))
    return cases


CASES = _draw_cases(16)


def _id(c):
    return "B{B}_Sq{S_q}_Skv{S_kv}_Hq{Hq}_Hkv{Hkv}_D{D}_K{K}_{t}".format(t=np.dtype(c["dtype"]).name, **c)


@pytest.mark.parametrize("c", CASES, ids=_id)
def test_random_shape_whole_path(c):
    print(f"random shape {_id(c)} scale={c['scale']:.4f}", flush=True)
    B, S_q, S_kv, Hq, Hkv, D, K = (c[x] for x in ("B", "S_q", "S_kv", "Hq", "Hkv", "D", "K"))
    q, k, v, r = random_small_case(c["seed"], B, S_q, S_kv, Hq, Hkv, D, K, p_invalid=c["p_invalid"],
                                   p_empty=c["p_empty"], route_dtype=c["dtype"])
    dout = random_dout(c["seed"] + 1, q.shape)
    scale = c["scale"]

    lst, cnt, mem, tc = qsa.qsa_preprocess(torch.from_numpy(r).to(device()), S_kv, membership=True, tile_class=True)
    qg, kg, vg, gg = bf16_to_gpu(q), bf16_to_gpu(k), bf16_to_gpu(v), bf16_to_gpu(dout)
    out, lse = qsa.qsa_forward_preprocessed(qg, kg, vg, lst, cnt, scale, return_lse=True)
    dq, dk, dv = qsa.qsa_backward(qg, kg, vg, out, gg, lse, lst, cnt, scale)
    torch.cuda.synchronize()

    olst, ocnt = oracle.route_lists(r, S_kv)
    np.testing.assert_array_equal(lst.cpu().numpy(), olst)
    np.testing.assert_array_equal(cnt.cpu().numpy(), ocnt)
    np.testing.assert_array_equal(mem.cpu().numpy(), oracle.membership(r, S_kv))
    np.testing.assert_array_equal(tc.cpu().numpy(), oracle.tile_class(r, S_kv))
    check_forward(gpu_bf16_bits(out), oracle.forward(q, k, v, r, scale), ocnt, v, "forward")
    check_lse(lse.cpu().numpy().astype(np.float64), oracle.lse(q, k, r, scale), "lse")
    rq, rk, rv = oracle.backward(q, k, v, dout, r, scale)
    floor = 1e-3 * float(np.abs(rv).max()) if rv.size else 0.0
    check_grad(gpu_bf16_bits(dq), rq, "dq", floor)
    check_grad(gpu_bf16_bits(dk), rk, "dk", floor)
    check_grad(gpu_bf16_bits(dv), rv, "dv")


def _draw_preprocess_cases(n: int, seed: int = 20261203):
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for _ in range(n):
        kv = int(rng.choice([int(rng.integers(1, 16385)), int(rng.integers(16385, 65537)),
                             int(rng.integers(65537, 140001))]))
        K = int(rng.choice([int(rng.integers(1, 1025)), int(rng.integers(1025, 2049)), int(rng.integers(2049, 5001))]))
        cases.append(dict(B=int(rng.integers(1, 3)), S_q=int(rng.integers(1, 6)), S_kv=kv, K=K,
                          dtype=np.int32 if rng.random() < 0.5 else np.int64, seed=int(rng.integers(1, 1 << 30))))
    return cases


PRE_CASES = _draw_preprocess_cases(16)


@pytest.mark.parametrize("c", PRE_CASES, ids=lambda c: "B{B}_Sq{S_q}_Skv{S_kv}_K{K}".format(**c))
def test_random_shape_preprocess(c):
    print("random preprocess B{B} Sq{S_q} Skv{S_kv} K{K}".format(**c), flush=True)
    rng = np.random.Generator(np.random.PCG64(c["seed"]))
    B, S_q, S_kv, K = c["B"], c["S_q"], c["S_kv"], c["K"]
    r = rng.integers(-5, S_kv + 5, size=(B, S_q, K), dtype=np.int64)
    runs = rng.integers(0, S_kv, size=(B, S_q, 1)) + np.arange(K)[None, None, :] // 2  # runs of consecutive IDs
    take = rng.random((B, S_q, K)) < 0.5
    r = np.where(take, runs, r)
    if c["dtype"] == np.int32:
        r = r.astype(np.int32)
    lst, cnt, mem, tc = qsa.qsa_preprocess(torch.from_numpy(r).to(device()), S_kv, membership=True, tile_class=True)
    olst, ocnt = oracle.route_lists(r, S_kv)
    np.testing.assert_array_equal(cnt.cpu().numpy(), ocnt)
    np.testing.assert_array_equal(lst.cpu().numpy(), olst)
    np.testing.assert_array_equal(mem.cpu().numpy(), oracle.membership(r, S_kv))
    np.testing.assert_array_equal(tc.cpu().numpy(), oracle.tile_class(r, S_kv))


def _draw_split_cases(n: int, seed: int = 20261203):
    """Shapes whose K/V exceed 16 MiB per KV head (the attention and dq split their key range), with
    windowed routes so that rows span one, several or all ranges."""
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for _ in range(n):
        D = int(rng.choice([64, 128, 256]))
        W = (4 << 20) // (4 * D)  # keys per range
        G = int(rng.choice([1, 2, 4, 8, 16]))
        Hkv = int(rng.integers(1, 3 if G == 16 else 4))
        cases.append(dict(
            B=int(rng.integers(1, 3)), S_q=int(rng.integers(1, 90)), S_kv=int(rng.integers(4 * W + 1, 12 * W)),
            Hq=G * Hkv, Hkv=Hkv, D=D, K=int(rng.integers(1, 1500)), scale=float(rng.uniform(0.02, 0.3)),
            seed=int(rng.integers(1, 1 << 30))))
    return cases


SPLIT_CASES = _draw_split_cases(10)


def _sid(c):
    return "B{B}_Sq{S_q}_Skv{S_kv}_Hq{Hq}_Hkv{Hkv}_D{D}_K{K}".format(**c)


@pytest.mark.parametrize("c", SPLIT_CASES, ids=_sid)
def test_random_split_shape_forward_backward(c):
    from workloads.generators import random_windowed_routes

    B, S_q, S_kv, Hq, Hkv, D, K = (c[x] for x in ("B", "S_q", "S_kv", "Hq", "Hkv", "D", "K"))
    print(f"random split shape {_sid(c)} scale={c['scale']:.4f}", flush=True)
    assert qsa.qsa_attention_workspace_size(B, S_q, S_kv, Hq, Hkv, D, K) > 0  # the split runs
    q, k, v, _ = random_small_case(c["seed"], B, S_q, S_kv, Hq, Hkv, D, 1)
    r = random_windowed_routes(c["seed"] + 2, B, S_q, S_kv, K)
    dout = random_dout(c["seed"] + 1, q.shape)
    scale = c["scale"]
    qg, kg, vg, gg = bf16_to_gpu(q), bf16_to_gpu(k), bf16_to_gpu(v), bf16_to_gpu(dout)
    lst, cnt, _, _ = qsa.qsa_preprocess(torch.from_numpy(r).to(device()), S_kv)
    out, lse = qsa.qsa_forward_preprocessed(qg, kg, vg, lst, cnt, scale, return_lse=True)
    dq, dk, dv = qsa.qsa_backward(qg, kg, vg, out, gg, lse, lst, cnt, scale)
    torch.cuda.synchronize()
    _, ocnt = oracle.route_lists(r, S_kv)
    check_forward(gpu_bf16_bits(out), oracle.forward(q, k, v, r, scale), ocnt, v, f"split {_sid(c)}")
    check_lse(lse.cpu().numpy().astype(np.float64), oracle.lse(q, k, r, scale), f"split lse {_sid(c)}")
    rq, rk, rv = oracle.backward(q, k, v, dout, r, scale)
    floor = 1e-3 * float(np.abs(rv).max()) if rv.size else 0.0
    check_grad(gpu_bf16_bits(dq), rq, f"split dq {_sid(c)}", floor)
    check_grad(gpu_bf16_bits(dk), rk, f"split dk {_sid(c)}", floor)
    check_grad(gpu_bf16_bits(dv), rv, f"split dv {_sid(c)}")
