"""GPU block lists (qsa_tile_lists) against the oracle, bit for bit.

Random class tables (several 64-position chunks per line, ragged ends, values
outside 0/1/2 that belong to neither list), subsets of the outputs, and the
tile classes of every seeded workload as qsa_preprocess produces them.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import route_sparse_gqa_amd as qsa
from gpu_util import device
from workloads import WORKLOADS, make_routes

pytestmark = pytest.mark.gpu

SHAPES = [(1, 1, 1), (1, 3, 4), (2, 16, 3), (1, 65, 130), (3, 7, 200), (1, 512, 512), (2, 129, 64)]


def _kinds(seed, shape):
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.choice(np.array([0, 1, 2, 3, -1], dtype=np.int32), size=shape, p=[0.45, 0.3, 0.2, 0.03, 0.02])


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_tile_lists_match_oracle(shape):
    print(f"tile lists {shape}", flush=True)
    kinds = _kinds(sum(shape), shape)
    got = qsa.qsa_tile_lists(torch.from_numpy(kinds).to(device()))
    want = oracle.tile_lists(kinds)
    for key in qsa.TILE_LIST_KEYS:
        np.testing.assert_array_equal(got[key].cpu().numpy(), want[key], err_msg=key)


def test_tile_lists_subset_of_outputs():
    kinds = _kinds(99, (2, 40, 90))
    want = oracle.tile_lists(kinds)
    for which in (("partial_idx",), ("full_count", "rev_full_idx"), ("rev_partial_count",)):
        got = qsa.qsa_tile_lists(torch.from_numpy(kinds).to(device()), which=which)
        assert set(got) == set(which)
        for key in which:
            np.testing.assert_array_equal(got[key].cpu().numpy(), want[key], err_msg=key)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", list(WORKLOADS))
def test_tile_lists_of_workload_classes(name):
    w = WORKLOADS[name]
    print(f"[{name}] tile lists of the workload's tile classes", flush=True)
    r = make_routes(w)
    _, _, _, tc = qsa.qsa_preprocess(torch.from_numpy(r).to(device()), w.S_kv, tile_class=True)
    got = qsa.qsa_tile_lists(tc)
    want = oracle.tile_lists(oracle.tile_class(r, w.S_kv))
    for key in qsa.TILE_LIST_KEYS:
        np.testing.assert_array_equal(got[key].cpu().numpy(), want[key], err_msg=f"{name} {key}")
