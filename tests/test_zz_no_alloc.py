"""GPU check of qsa_forward_noalloc (qsa_forward with the library's fixed device scratch in place of a
workspace): two calls in a row, the second on a smaller input, each against qsa_forward's output on the
same inputs (bitwise: the same kernels run) and against the fp64 oracle (BF16 tolerance); the first call
takes the key-range split in three passes (64 MiB hold two partial buffers of about 780 of its 2000 rows),
the second in one, so the scratch holds lists, range starts and partial results."""

from __future__ import annotations

import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
import route_sparse_gqa_amd as qsa
from gpu_util import bf16_to_gpu, check_forward, device, gpu_bf16_bits
from workloads.generators import random_small_case, random_windowed_routes

pytestmark = pytest.mark.gpu


def _raw_noalloc(qg, kg, vg, rg, scale, out):
    """Through the C ABI directly (ctypes), as a caller that cannot allocate would."""
    B, S_q, Hq, D = qg.shape
    S_kv, Hkv = kg.shape[1], kg.shape[2]
    K = rg.shape[2]
    st = lambda t: (ctypes.c_int64 * t.dim())(*t.stride())
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream(device()).cuda_stream)
    return qsa.lib().qsa_forward_noalloc(p(qg), st(qg), p(kg), st(kg), p(vg), st(vg), p(rg), 1, st(rg), B, S_q,
                                         S_kv, Hq, Hkv, D, K, ctypes.c_float(scale), p(out), stream)


def test_noalloc_matches_qsa_forward_twice():
    cases = [  # (B, S_q, S_kv, Hq, Hkv, D, K), each call smaller than the one before:
        (1, 2000, 20000, 16, 2, 256, 300),  # the split (5 ranges) in passes: two partial buffers in the scratch
        (2, 500, 20000, 16, 2, 256, 400),   # the split in one pass
        (1, 70, 500, 8, 1, 128, 60),
    ]
    for n, case in enumerate(cases):
        B, S_q, S_kv, Hq, Hkv, D, K = case
        print(f"noalloc call {n}: {case}", flush=True)
        q, k, v, _ = random_small_case(40 + n, B, S_q, S_kv, Hq, Hkv, D, 1)
        r = random_windowed_routes(50 + n, B, S_q, S_kv, K)
        scale = 1.0 / math.sqrt(D)
        qg, kg, vg, rg = bf16_to_gpu(q), bf16_to_gpu(k), bf16_to_gpu(v), torch.from_numpy(r).to(device())
        want = qsa.qsa_forward(qg, kg, vg, rg, scale)
        got = torch.empty_like(want)
        assert _raw_noalloc(qg, kg, vg, rg, scale, got) == 0
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"call {n}: differs from qsa_forward"
        _, ocnt = oracle.route_lists(r, S_kv)
        check_forward(gpu_bf16_bits(got), oracle.forward(q, k, v, r, scale), ocnt, v, f"noalloc call {n}")
    # the binding's wrapper of the same entry point
    again = qsa.qsa_forward_noalloc(qg, kg, vg, rg, scale)
    torch.cuda.synchronize()
    assert torch.equal(again.view(torch.int16), want.view(torch.int16))


def test_noalloc_refuses_beyond_its_scratch():
    # 8192 rows x 2048 routes: the lists alone fill the 64 MiB (host check; nothing is enqueued)
    qg = torch.zeros((1, 8192, 2, 64), dtype=torch.bfloat16, device=device())
    kg = torch.zeros((1, 64, 1, 64), dtype=torch.bfloat16, device=device())
    rg = torch.zeros((1, 8192, 2048), dtype=torch.int64, device=device())
    out = torch.empty_like(qg)
    assert _raw_noalloc(qg, kg, kg.clone(), rg, 0.125, out) == -14
    with pytest.raises(ValueError, match="scratch"):
        qsa.qsa_forward_noalloc(qg, kg, kg.clone(), rg, 0.125)
