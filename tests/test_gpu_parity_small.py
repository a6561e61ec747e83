"""GPU parity on small seeded cases: every kernel of the path against the fp64 oracle.

Preprocessing (lists, counts, membership with its padding, tile classes) must
match bit for bit; attention must meet the BF16 tolerance; the exactness
properties of the method must hold bitwise on the GPU as well.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import route_sparse_gqa_amd as qsa
from gpu_util import bf16_to_gpu, bits_to_f64, check_forward, device, gpu_bf16_bits
from test_gpu_backward import check_lse
from workloads.generators import random_small_case

pytestmark = pytest.mark.gpu

CASES = [  # (B, S_q, S_kv, Hq, Hkv, D, K): ragged sizes, several tiles, every D and group size
    (1, 37, 45, 4, 1, 64, 19),
    (2, 130, 300, 16, 2, 256, 77),
    (1, 64, 200, 8, 8, 128, 40),
    (2, 33, 129, 32, 2, 64, 33),
    (1, 50, 70, 12, 3, 128, 65),
    (1, 20, 1000, 2, 1, 256, 600),
    (1, 8, 5000, 2, 2, 64, 3000),
    (1, 3, 1, 2, 1, 64, 5),
    (1, 1, 9, 16, 1, 256, 1),
    (3, 257, 513, 8, 1, 256, 129),
]


def _ids(case):
    return "B{}_Sq{}_Skv{}_Hq{}_Hkv{}_D{}_K{}".format(*case)


@pytest.mark.parametrize("case", CASES, ids=_ids)
@pytest.mark.parametrize("route_dtype", [np.int64, np.int32], ids=["i64", "i32"])
def test_preprocess_bit_exact(case, route_dtype):
    B, S_q, S_kv, Hq, Hkv, D, K = case
    print(f"preprocess case {case} {np.dtype(route_dtype).name}", flush=True)
    _, _, _, r = random_small_case(sum(case), B, S_q, S_kv, Hq, Hkv, D, K, route_dtype=route_dtype)
    lst, cnt, mem, tc = qsa.qsa_preprocess(torch.from_numpy(r).to(device()), S_kv, membership=True, tile_class=True)
    olst, ocnt = oracle.route_lists(r, S_kv)
    np.testing.assert_array_equal(cnt.cpu().numpy(), ocnt)
    np.testing.assert_array_equal(lst.cpu().numpy(), olst)
    np.testing.assert_array_equal(mem.cpu().numpy(), oracle.membership(r, S_kv))
    np.testing.assert_array_equal(tc.cpu().numpy(), oracle.tile_class(r, S_kv))


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_forward_matches_oracle(case):
    B, S_q, S_kv, Hq, Hkv, D, K = case
    print(f"forward case {case}", flush=True)
    q, k, v, r = random_small_case(1000 + sum(case), B, S_q, S_kv, Hq, Hkv, D, K)
    scale = 1.0 / math.sqrt(D)
    out = qsa.qsa_forward(bf16_to_gpu(q), bf16_to_gpu(k), bf16_to_gpu(v), torch.from_numpy(r).to(device()), scale)
    torch.cuda.synchronize()
    ref = oracle.forward(q, k, v, r, scale)
    _, cnt = oracle.route_lists(r, S_kv)
    check_forward(gpu_bf16_bits(out), ref, cnt, v, f"forward {case}")


def test_large_route_counts_and_segments():
    """K up to the largest sort size, and a membership row wider than one 65536-column segment."""
    for (B, S_q, S_kv, K) in [(1, 4, 20000, 9000), (1, 5, 70000, 300), (2, 3, 131073, 16384)]:
        print(f"large case B{B} Sq{S_q} Skv{S_kv} K{K}", flush=True)
        q, k, v, r = random_small_case(B * S_q + K, B, S_q, S_kv, 2, 1, 64, K, p_invalid=0.1, p_empty=0.0)
        lst, cnt, mem, tc = qsa.qsa_preprocess(torch.from_numpy(r).to(device()), S_kv, True, True)
        olst, ocnt = oracle.route_lists(r, S_kv)
        np.testing.assert_array_equal(cnt.cpu().numpy(), ocnt)
        np.testing.assert_array_equal(lst.cpu().numpy(), olst)
        np.testing.assert_array_equal(mem.cpu().numpy(), oracle.membership(r, S_kv))
        np.testing.assert_array_equal(tc.cpu().numpy(), oracle.tile_class(r, S_kv))
        out = qsa.qsa_forward_preprocessed(bf16_to_gpu(q), bf16_to_gpu(k), bf16_to_gpu(v), lst, cnt, 0.125)
        check_forward(gpu_bf16_bits(out), oracle.forward(q, k, v, r, 0.125), ocnt, v, "large K")


@pytest.mark.parametrize("S_kv,K,dtype", [(131072, 4096, np.int64), (131072, 4097, np.int64), (131073, 64, np.int32),
                                          (1 << 31, 300, np.int64), (64, 4096, np.int32), (16384, 512, np.int64),
                                          (16385, 512, np.int32), (16384, 513, np.int64), (16384, 1024, np.int32),
                                          (16384, 1025, np.int64), (33, 1, np.int64), (65536, 2048, np.int64),
                                          (65537, 2048, np.int32), (65536, 2049, np.int64), (16385, 1, np.int32)])
def test_route_lists_at_the_bitmap_limits(S_kv, K, dtype):
    """Every normalisation path at its boundaries (one wavefront per row: kv <= 16384 and K <= 1024, with
    8 or 16 slots per lane; one workgroup per row: kv <= 65536 and K <= 2048 with the half-size bitmap,
    kv <= 131072 and K <= 4096 with the full one; else sorting)."""
    print(f"route lists kv={S_kv} K={K} {np.dtype(dtype).name}", flush=True)
    rng = np.random.Generator(np.random.PCG64(S_kv + K))
    B, S_q = 2, 5
    r = rng.integers(-3, min(S_kv + 3, np.iinfo(dtype).max), size=(B, S_q, K), dtype=np.int64)
    r[:, :, K // 2:] = r[:, :, :K - K // 2]  # every value of the first half appears again
    r = r.astype(dtype)
    lst, cnt, _, _ = qsa.qsa_preprocess(torch.from_numpy(r).to(device()), S_kv)
    olst, ocnt = oracle.route_lists(r, S_kv)
    np.testing.assert_array_equal(cnt.cpu().numpy(), ocnt)
    np.testing.assert_array_equal(lst.cpu().numpy(), olst)


def test_full_tiles_and_edge_tiles():
    # every pair of tile (0,0) a member, a full ragged edge tile, a partial and an absent tile
    S_q, kv = 200, 130
    r = np.full((1, S_q, 130), -1, dtype=np.int64)
    r[0, :128, :128] = np.arange(128)
    r[0, 128:, 0] = 128
    r[0, 128:, 1] = 129
    r[0, 130, 2] = 5
    _, _, mem, tc = qsa.qsa_preprocess(torch.from_numpy(r).to(device()), kv, True, True)
    assert tc.cpu().numpy()[0].tolist() == [[2, 0], [1, 2]]
    np.testing.assert_array_equal(mem.cpu().numpy(), oracle.membership(r, kv))


def test_tile_classes_without_membership():
    _, _, _, r = random_small_case(5, 2, 300, 260, 1, 1, 64, 50)
    lst, cnt, mem, tc = qsa.qsa_preprocess(torch.from_numpy(r).to(device()), 260, membership=False, tile_class=True)
    assert mem is None
    np.testing.assert_array_equal(tc.cpu().numpy(), oracle.tile_class(r, 260))


# --------------------------------------------------------------------------
# exactness properties, bitwise on the GPU
# --------------------------------------------------------------------------

def _run(q, k, v, r, scale=0.125):
    out = qsa.qsa_forward(bf16_to_gpu(q), bf16_to_gpu(k), bf16_to_gpu(v), torch.from_numpy(r).to(device()), scale)
    return gpu_bf16_bits(out)


@pytest.mark.parametrize("K,Hq,Hkv", [(64, 16, 2), (16, 4, 1), (48, 8, 8)])
def test_route_counts_at_every_chunk_boundary(K, Hq, Hkv):
    """Rows routing 0, 1, 15, 16, 17, ..., K-1 and K distinct keys (16-key chunks), the last rows of
    the buffer full; D = 256 with K a multiple of 16 is the configuration whose chunk IDs are read as
    whole 64-byte windows of the list."""
    B, S_q, S_kv, D = 2, 21, 3000, 256
    rng = np.random.Generator(np.random.PCG64(K * 7 + Hq))
    lengths = sorted({0, 1, 15, 16, 17, 31, 32, 33, K - 17, K - 16, K - 15, K - 1, K} & set(range(K + 1)))
    routes = np.full((B, S_q, K), -1, dtype=np.int64)
    for b in range(B):
        for i in range(S_q):
            n = K if i >= S_q - 2 else lengths[(b * S_q + i) % len(lengths)]
            routes[b, i, :n] = rng.choice(S_kv, size=n, replace=False)
            routes[b, i] = routes[b, i, rng.permutation(K)]
    q, k, v, _ = random_small_case(K + Hq, B, S_q, S_kv, Hq, Hkv, D, 1)
    out, lse = qsa.qsa_forward_preprocessed(
        bf16_to_gpu(q), bf16_to_gpu(k), bf16_to_gpu(v),
        *qsa.qsa_preprocess(torch.from_numpy(routes).to(device()), S_kv)[:2], 0.0625, return_lse=True)
    _, ocnt = oracle.route_lists(routes, S_kv)
    assert int(ocnt.max()) == K and int(ocnt.min()) == 0
    check_forward(gpu_bf16_bits(out), oracle.forward(q, k, v, routes, 0.0625), ocnt, v, "chunk boundaries")
    check_lse(lse.cpu().numpy().astype(np.float64), oracle.lse(q, k, routes, 0.0625), "chunk boundaries lse")


def test_single_route_returns_v_row_bitwise():
    B, S_q, S_kv, Hq, Hkv, D = 2, 40, 90, 16, 2, 256
    q, k, v, _ = random_small_case(77, B, S_q, S_kv, Hq, Hkv, D, 1)
    rng = np.random.default_rng(78)
    j = rng.integers(0, S_kv, size=(B, S_q))
    r = np.stack([np.full_like(j, -1), j, np.full_like(j, S_kv), j, np.full_like(j, 1 << 40)], axis=2)
    got = _run(q, k, v, r)
    G = Hq // Hkv
    for b in range(B):
        for i in range(S_q):
            for h in range(Hq):
                assert np.array_equal(got[b, i, h], v[b, j[b, i], h // G]), (b, i, h)


def test_all_invalid_rows_are_zero_bitwise():
    q, k, v, r = random_small_case(81, 2, 50, 60, 8, 1, 128, 21, p_empty=0.3)
    r[1, :] = -1
    r[0, 7] = [60, 61, 1 << 40, -5, np.iinfo(np.int64).min] * 4 + [np.iinfo(np.int64).max]
    got = _run(q, k, v, r)
    _, cnt = oracle.route_lists(r, 60)
    assert (cnt == 0).sum() > 50
    assert not got[cnt == 0].any()


def test_permuting_and_duplicating_routes_is_bitwise_invariant():
    q, k, v, r = random_small_case(91, 2, 70, 300, 16, 2, 256, 64)
    rng = np.random.default_rng(92)
    base = _run(q, k, v, r)
    perm = np.take_along_axis(r, rng.permuted(np.tile(np.arange(64), (2, 70, 1)), axis=2), axis=2)
    dup = np.concatenate([r[:, :, ::-1], r, r[:, :, :17]], axis=2)
    assert np.array_equal(_run(q, k, v, perm), base)
    assert np.array_equal(_run(q, k, v, dup), base)


def test_int32_and_int64_routes_give_identical_bits():
    q, k, v, r = random_small_case(95, 1, 100, 400, 8, 1, 256, 96, route_dtype=np.int32)
    assert np.array_equal(_run(q, k, v, r), _run(q, k, v, r.astype(np.int64)))


def test_forward_equals_preprocess_then_preprocessed():
    q, k, v, r = random_small_case(97, 2, 64, 256, 16, 2, 256, 100)
    qg, kg, vg, rg = bf16_to_gpu(q), bf16_to_gpu(k), bf16_to_gpu(v), torch.from_numpy(r).to(device())
    a = qsa.qsa_forward(qg, kg, vg, rg, 0.1)
    lst, cnt, _, _ = qsa.qsa_preprocess(rg, 256)
    b = qsa.qsa_forward_preprocessed(qg, kg, vg, lst, cnt, 0.1)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_strided_inputs_match_contiguous():
    B, S_q, S_kv, Hq, Hkv, D, K = 2, 48, 120, 8, 2, 128, 40
    q, k, v, r = random_small_case(99, B, S_q, S_kv, Hq, Hkv, D, K)
    base = _run(q, k, v, r)
    qg, kg, vg = bf16_to_gpu(q), bf16_to_gpu(k), bf16_to_gpu(v)
    # head-major Q viewed back as [B,S,H,D]; K/V interleaved with unused heads; routes transposed in memory
    q_hm = qg.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    k_wide = torch.zeros((B, S_kv, 2 * Hkv, D), dtype=torch.bfloat16, device=device())
    v_wide = torch.zeros_like(k_wide)
    k_wide[:, :, ::2] = kg
    v_wide[:, :, ::2] = vg
    r_t = torch.from_numpy(r).to(device()).transpose(1, 2).contiguous().transpose(1, 2)
    got = qsa.qsa_forward(q_hm, k_wide[:, :, ::2], v_wide[:, :, ::2], r_t, 0.125)
    assert np.array_equal(gpu_bf16_bits(got), base)
    # a non-unit last stride is copied by the binding
    q_odd = torch.zeros((B, S_q, Hq, 2 * D), dtype=torch.bfloat16, device=device())
    q_odd[..., ::2] = qg
    got2 = qsa.qsa_forward(q_odd[..., ::2], kg, vg, torch.from_numpy(r).to(device()), 0.125)
    assert np.array_equal(gpu_bf16_bits(got2), base)


def test_scale_changes_result_as_defined():
    q, k, v, r = random_small_case(101, 1, 30, 50, 4, 1, 64, 16)
    for scale in (1e-3, 0.37, 4.0):
        out = _run(q, k, v, r, scale)
        _, cnt = oracle.route_lists(r, 50)
        check_forward(out, oracle.forward(q, k, v, r, scale), cnt, v, f"scale {scale}")
