"""bench.py's contract and the counts its roofline is computed from (CPU only).

* One GPU only: ``--gpus N`` with N > 1 exits with status 2 and says why,
  before anything touches a GPU.
* The routed (row, route) pairs N of the measured workloads have a closed
  form in each route recipe (the drawn blocks are distinct, so only the
  clipping of the own block and the number of earlier blocks matter); the
  generator must produce exactly that many distinct valid routes, and the
  algorithmic flops and bytes are the stated functions of N.
"""

from __future__ import annotations

import os
import subprocess
import sys

import numpy as np

import bench
import oracle
from workloads import WORKLOADS
from workloads.generators import make_routes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def closed_form_pairs(name: str) -> int:
    """N from the route recipe of each workload."""
    if name == "right_padded":  # own block clipped to <= q, plus min(7, j) earlier blocks; rows >= length empty
        return sum(sum((i % 64) + 1 + 64 * min(7, i // 64) for i in range(L)) for L in (4096, 3000))
    if name == "cp_slice":  # global position p = 24576 + i: own block clipped, plus 31 earlier blocks
        return sum(((24576 + i) % 64) + 1 for i in range(8192)) + 8192 * 31 * 64
    if name == "long_int64":  # own block clipped, block 0 and up to 30 more: min(32, j + 1) blocks in all
        return sum((q % 64) + 1 + 64 * (min(32, q // 64 + 1) - 1) for q in range(65536))
    raise KeyError(name)


def test_bench_refuses_more_than_one_gpu():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_closed_form_pair_counts():
    assert closed_form_pairs("right_padded") == 3_180_028
    assert closed_form_pairs("cp_slice") == 16_519_168
    assert closed_form_pairs("long_int64") == 130_121_728


def test_generated_routes_have_the_closed_form_count():
    w = WORKLOADS["right_padded"]
    routes = make_routes(w)
    _, counts = oracle.route_lists(routes, w.S_kv)
    assert int(counts.sum()) == closed_form_pairs("right_padded")


def test_algorithmic_flops_and_bytes():
    for name in ("right_padded", "cp_slice", "long_int64"):
        w = WORKLOADS[name]
        N = closed_form_pairs(name)
        rows = w.B * w.S_q
        flops, alg_bytes = bench.algorithmic_counts(w, N)
        assert flops == 4 * w.D * w.Hq * N  # QK^T and PV on routed pairs
        # routed K and V rows once per (row, KV head), Q read and O written (bf16), lists and counts (int32)
        assert alg_bytes == 4 * w.D * w.Hkv * N + 4 * rows * w.Hq * w.D + 4 * N + 4 * rows
    w = WORKLOADS["right_padded"]
    flops, alg_bytes = bench.algorithmic_counts(w, closed_form_pairs("right_padded"))
    assert flops == 52_101_578_752 and alg_bytes == 6_659_667_952
    assert np.isclose(alg_bytes / 8e12 * 1e3, 0.8325, atol=1e-4)  # ms at 8 TB/s


def test_roofline_is_the_compulsory_floor_over_the_time():
    """frac = t_floor / t against real peaks: for long_int64 the flops set the floor (2131.9 GFLOP at
    2.5 PFLOP/s = 0.853 ms, against 1.73 GB of compulsory bytes at 8 TB/s = 0.22 ms)."""
    w = WORKLOADS["long_int64"]
    N = closed_form_pairs("long_int64")
    flops, gather_bytes = bench.algorithmic_counts(w, N)
    min_bytes = 1_730_000_000
    for ms in (0.853, 5.0, 24.4):
        r = bench.attention_roofline(w, N, flops, gather_bytes, min_bytes, [ms], None, "k")
        assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
        assert np.isclose(r["frac"], r["t_floor_ms"] / ms)
        assert np.isclose(r["achieved"], flops / (ms * 1e-3) / 1e12)
        assert r["frac"] <= 1.0 + 1e-3
        assert np.isclose(r["gather_rate_GBs"], gather_bytes / (ms * 1e-3) / 1e9)
    assert np.isclose(bench.attention_roofline(w, N, flops, gather_bytes, min_bytes, [24.4], None, "k")["frac"],
                      0.0349, atol=5e-4)
    # a workload whose compulsory bytes dominate is counted against HBM
    r = bench.attention_roofline(w, 1000, 4 * w.D * w.Hq * 1000, 10 ** 9, 8 * 10 ** 9, [2.0], 9 * 10 ** 9, "k")
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and np.isclose(r["frac"], 0.5)
    assert np.isclose(r["hbm_traffic_GBs"], 4500.0)


def test_cpu_info_reports_model_and_affinity():
    info = bench.cpu_info()
    assert info["affinity_cores"] == len(os.sched_getaffinity(0)) >= 1
    assert "cpu_model" in info
