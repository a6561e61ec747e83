"""HIP graph capture of the library's entry points.

The library allocates nothing, synchronises nothing and clears memory with
kernels only (no memset nodes), so a caller can capture whole calls into a
HIP graph (torch.cuda.graph) and replay them: the launch-bound small shapes
gain the most.  Each captured graph is replayed several times; before every
replay new inputs are copied into the captured buffers by ordinary eager work,
and every replay must equal, bit for bit, an eager call on the same inputs
(the kernels are deterministic).
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import route_sparse_gqa_amd as qsa
from gpu_util import bf16_to_gpu, device
from workloads import random_select_case
from workloads.generators import random_small_case

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _capture(fn):
    """Warm fn up on a side stream (as torch requires before capture), then capture one call."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = fn()
    torch.cuda.synchronize()
    return graph, outs


def _attention_inputs(seed, case):
    B, S_q, S_kv, Hq, Hkv, D, K = case
    q, k, v, r = random_small_case(seed, B, S_q, S_kv, Hq, Hkv, D, K)
    return bf16_to_gpu(q), bf16_to_gpu(k), bf16_to_gpu(v), torch.from_numpy(r).to(device())


@pytest.mark.parametrize("case", [(1, 256, 256, 4, 1, 64, 32), (2, 130, 300, 16, 2, 256, 77),
                                  (1, 64, 20000, 16, 2, 256, 300)],  # the last one takes the key-range split
                         ids=lambda c: "B{}_Sq{}_Skv{}_Hq{}_Hkv{}_D{}_K{}".format(*c))
def test_forward_and_backward_graph_replays_equal_eager(case):
    print(f"graph forward/backward {case}", flush=True)
    q, k, v, r = _attention_inputs(500 + sum(case), case)
    D = case[5]
    scale = 1.0 / math.sqrt(D)
    dout = torch.randn(q.shape, device=device()).to(torch.bfloat16)

    def step():
        lst, cnt, _, _ = qsa.qsa_preprocess(r, case[2])
        out, lse = qsa.qsa_forward_preprocessed(q, k, v, lst, cnt, scale, return_lse=True)
        dq, dk, dv = qsa.qsa_backward(q, k, v, out, dout, lse, lst, cnt, scale)
        return out, dq, dk, dv, qsa.qsa_forward(q, k, v, r, scale)

    graph, captured = _capture(step)
    for trial in range(REPLAYS):
        nq, nk, nv, nr = _attention_inputs(600 + 10 * trial + sum(case), case)
        q.copy_(nq)
        k.copy_(nk)
        v.copy_(nv)
        r.copy_(nr)
        dout.copy_(torch.randn(q.shape, device=device()).to(torch.bfloat16))
        graph.replay()
        torch.cuda.synchronize()
        eager = step()
        torch.cuda.synchronize()
        for name, got, want in zip(("out", "dq", "dk", "dv", "out (qsa_forward)"), captured, eager):
            assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"replay {trial}: {name} differs"


def test_selection_graph_replays_equal_eager():
    print("graph selection", flush=True)
    B, S_q, H, D, c, budget = 2, 700, 16, 128, 4, 64
    iq_np, ck_np = random_select_case(901, B, S_q, H, D, S_q // c)
    iq, ck = bf16_to_gpu(iq_np), bf16_to_gpu(ck_np)
    lens = torch.tensor([S_q, 500], dtype=torch.int64, device=device())

    def call():
        return (qsa.qsa_select_token_ids(iq, ck, lens, budget, c),)

    graph, (captured,) = _capture(call)
    for trial in range(REPLAYS):
        niq, nck = random_select_case(910 + trial, B, S_q, H, D, S_q // c)
        iq.copy_(bf16_to_gpu(niq))
        ck.copy_(bf16_to_gpu(nck))
        lens.copy_(torch.tensor([S_q - 37 * trial, 500 + trial], dtype=torch.int64))
        graph.replay()
        torch.cuda.synchronize()
        (eager,) = call()
        torch.cuda.synchronize()
        assert torch.equal(captured, eager), f"replay {trial}: token IDs differ"
        assert np.any(eager.cpu().numpy() >= 0)
