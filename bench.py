"""Benchmark of the route-sparse GQA forward path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input
already resident in HBM:
  1. qsa_preprocess: route normalisation (lists + counts), membership table
     and 128x128 tile classes;
  2. qsa_forward_preprocessed: the gather-attention kernel(s).
A 1 GiB scratch write between steps evicts the L2 and the Infinity Cache
(--flush-mib); the step time excludes it (HIP events per step).

The default workload is long_int64 (B=1, S=65536, K=2048), the largest
configuration that fits one GPU and the one past the int32 flat-index limit.

Prints ONE JSON line:
  value        routed-attention TFLOP/s of the whole step, F = 4*D*Hq*N flops
               with N = total distinct valid routes (16384 flop per routed
               (row, route) pair at D = 256, Hq = 16);
  roofline     the attention against its roofline on this chip.  The
               compulsory work sets the floor t_floor = max(B_min / 8 TB/s,
               F / 2.5 PFLOP/s), B_min = Q read, O written, lists, counts and
               each distinct routed K/V row once per KV head; for the
               D = 256 workloads the flops set it, so `bound` is "mfma",
               `achieved` = F / t_attention and `frac` = achieved / 2.5 PFLOP/s
               (= t_floor / t).  Beside it: the gather rate (each routed K and
               V row once per (query row, KV head), plus Q, O, lists: bytes
               the L2, the Infinity Cache and HBM serve together, not an HBM
               figure) and, when profiles/traffic.json holds rocprofv3
               FETCH_SIZE/WRITE_SIZE for the current kernel sources, the
               physical HBM-side bytes per launch (`traffic`) and their rate;
  kernels_ms   preprocess, attention, and the fused qsa_forward (route
               normalisation + attention in one call) timed separately;
  cpu_baseline the fp64 CPU oracle on a bounded sample of the same rows:
               windows of contiguous rows spread evenly over the sequence,
               so the sample's mix of row lengths is the workload's.

With ``--pass backward`` it times the backward instead (one step = one
qsa_backward call: the dq kernel, the key-segment construction and the dk/dv
kernel, on the forward's output and log-sum-exp), reporting routed TFLOP/s
with F = 10*D*Hq*N (scores, dP, dQ, dK, dV on routed pairs) and the
algorithmic bytes of the whole call against the HBM roofline.

With ``--pass tile_lists`` it times qsa_tile_lists (forward and reverse
partial/full block lists) on the workload's tile classes.

With ``--pass select`` it times route selection (qsa_select_token_ids: MFMA
block scores, per-row top-k, expansion) on a selection workload (default
sel_long), reporting scoring TFLOP/s with F = 2*H*D*sum(nv) over the rows
that see more than token_budget/c blocks (the only rows whose blocks are
scored), against the bf16 matrix-core peak.

``--counter-reference-mib M`` only runs plain device-to-device copies of M
MiB: the FETCH_SIZE / WRITE_SIZE counters of that copy, whose bytes are
known, scale the same counters read on the attention kernels.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--pass forward|backward|tile_lists|select]
"""

from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "routed-attention TFLOP/s + achieved HBM GB/s (fwd, BF16, D=256) on 1 MI355X"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
DEFAULT_WORKLOAD = "long_int64"
DEFAULT_SELECT_WORKLOAD = "sel_long"


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--pass", dest="which", choices=["forward", "backward", "tile_lists", "select"],
                    default="forward")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU-oracle sample time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flush-mib", type=int, default=1024,
                    help="write this many MiB of scratch between timed steps (evicts L2 and the Infinity Cache); "
                         "the step time comes from per-step events, without the flush")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="JSON with rocprofv3-derived HBM bytes per attention call, per workload")
    ap.add_argument("--counter-reference-mib", type=int, default=0,
                    help="only run plain device-to-device copies of this many MiB (counter scale reference)")
    ap.add_argument("--graph", action="store_true",
                    help="also capture one step (preprocess + attention) in a HIP graph and time its replays")
    return ap.parse_args()


def counter_reference_copy(mib: int, reps: int = 5) -> None:
    """Plain copies of a known size: FETCH_SIZE / WRITE_SIZE per dispatch of this kernel
    give the scale factor between the counters and bytes actually moved."""
    import torch

    dev = torch.device("cuda", 0)
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read_per_copy": n, "bytes_written_per_copy": n,
                      "copies": reps}), flush=True)


class Plan:
    """Pre-marshalled C-ABI calls for one workload (no per-step Python allocation)."""

    def __init__(self, w, q, k, v, routes, dev):
        import torch

        import route_sparse_gqa_amd as qsa

        self.w = w
        self.L = qsa.lib()
        self.stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        i8 = lambda t: ctypes.c_void_p(t.data_ptr())
        self.q = torch.from_numpy(q.view(np.int16)).to(dev).view(torch.bfloat16)
        self.k = torch.from_numpy(k.view(np.int16)).to(dev).view(torch.bfloat16)
        self.v = torch.from_numpy(v.view(np.int16)).to(dev).view(torch.bfloat16)
        self.routes = torch.from_numpy(routes).to(dev)
        B, S_q, K = routes.shape
        n_ti, n_tj = -(-S_q // 128), -(-w.S_kv // 128)
        self.lst = torch.empty((B, S_q, K), dtype=torch.int32, device=dev)
        self.cnt = torch.empty((B, S_q), dtype=torch.int32, device=dev)
        self.mem = torch.empty((B, S_q, n_tj * 128), dtype=torch.uint8, device=dev)
        self.tc = torch.empty((B, n_ti, n_tj), dtype=torch.int32, device=dev)
        self.out = torch.empty((B, S_q, w.Hq, w.D), dtype=torch.bfloat16, device=dev)
        st = lambda t: (ctypes.c_int64 * t.dim())(*t.stride())
        self.pre_args = (i8(self.routes), 1 if routes.dtype == np.int64 else 0, B, S_q, K, st(self.routes),
                         w.S_kv, i8(self.lst), i8(self.cnt), i8(self.mem), i8(self.tc), self.stream)
        att_ws = qsa.qsa_attention_workspace_size(B, S_q, w.S_kv, w.Hq, w.Hkv, w.D, K)
        self.att_ws = torch.empty(att_ws, dtype=torch.uint8, device=dev) if att_ws else None
        self.split = att_ws > 0
        self.fwd_args = (i8(self.q), st(self.q), i8(self.k), st(self.k), i8(self.v), st(self.v), i8(self.lst),
                         i8(self.cnt), B, S_q, w.S_kv, w.Hq, w.Hkv, w.D, K, ctypes.c_float(w.scale),
                         i8(self.out), None, i8(self.att_ws) if self.split else None, ctypes.c_size_t(att_ws),
                         self.stream)
        fused_ws = qsa.qsa_forward_workspace_size(B, S_q, w.S_kv, w.Hq, w.Hkv, w.D, K)
        self.fused_ws = torch.empty(fused_ws, dtype=torch.uint8, device=dev)
        self.fused_out = torch.empty_like(self.out)
        self.fused_args = (i8(self.q), st(self.q), i8(self.k), st(self.k), i8(self.v), st(self.v), i8(self.routes),
                           1 if routes.dtype == np.int64 else 0, st(self.routes), B, S_q, w.S_kv, w.Hq, w.Hkv, w.D,
                           K, ctypes.c_float(w.scale), i8(self.fused_out), i8(self.fused_ws),
                           ctypes.c_size_t(fused_ws), self.stream)

    def set_stream(self, stream: ctypes.c_void_p) -> None:
        """Point the pre-marshalled calls at another HIP stream (the stream is their last argument)."""
        self.stream = stream
        self.pre_args = self.pre_args[:-1] + (stream,)
        self.fwd_args = self.fwd_args[:-1] + (stream,)
        self.fused_args = self.fused_args[:-1] + (stream,)

    def setup_backward(self, dev):
        """Forward with log-sum-exp once, then pre-marshal qsa_backward (dout drawn from its own stream)."""
        import torch

        import route_sparse_gqa_amd as qsa
        from workloads import make_dout

        w = self.w
        B, S_q, K = self.lst.shape
        i8 = lambda t: ctypes.c_void_p(t.data_ptr())
        st = lambda t: (ctypes.c_int64 * t.dim())(*t.stride())
        self.lse = torch.empty((B, S_q, w.Hq), dtype=torch.float32, device=dev)
        args = list(self.fwd_args)
        args[-4] = i8(self.lse)
        rc = self.L.qsa_forward_preprocessed(*args)
        if rc != 0:
            raise RuntimeError(f"qsa_forward_preprocessed failed with status {rc}")
        self.dout = torch.from_numpy(make_dout(w).view(np.int16)).to(dev).view(torch.bfloat16)
        self.dq = torch.empty_like(self.q)
        self.dk = torch.empty_like(self.k)
        self.dv = torch.empty_like(self.v)
        ws_bytes = qsa.qsa_backward_workspace_size(B, S_q, w.S_kv, w.Hq, w.Hkv, w.D, K)
        self.ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        self.bwd_args = (i8(self.q), st(self.q), i8(self.k), st(self.k), i8(self.v), st(self.v), i8(self.out),
                         i8(self.dout), st(self.dout), i8(self.lse), i8(self.lst), i8(self.cnt), B, S_q, w.S_kv,
                         w.Hq, w.Hkv, w.D, K, ctypes.c_float(w.scale), i8(self.dq), i8(self.dk), i8(self.dv),
                         i8(self.ws), ctypes.c_size_t(ws_bytes), self.stream)

    def backward(self):
        rc = self.L.qsa_backward(*self.bwd_args)
        if rc != 0:
            raise RuntimeError(f"qsa_backward failed with status {rc}")

    def segment_count(self) -> int:
        """Number of (query row, 64-key tile) segments of the last backward (from its workspace)."""
        w = self.w
        B, S_q, _ = self.lst.shape
        r = lambda x: -(-x // 256) * 256
        n_kt, n_w, n_c = -(-w.S_kv // 64), -(-S_q // 32), -(-S_q // 256)
        # workspace layout (include/qsa.h): delta, bit matrix, chunk prefixes, totals, tile starts, ...
        off = r(4 * B * S_q * w.Hq) + r(4 * B * n_w * n_kt) + r(4 * B * n_c * n_kt) + r(4 * B * n_kt) + 4 * (B * n_kt)
        return int(self.ws[off:off + 4].cpu().numpy().view(np.int32)[0])

    def preprocess(self):
        rc = self.L.qsa_preprocess(*self.pre_args)
        if rc != 0:
            raise RuntimeError(f"qsa_preprocess failed with status {rc}")

    def attention(self):
        rc = self.L.qsa_forward_preprocessed(*self.fwd_args)
        if rc != 0:
            raise RuntimeError(f"qsa_forward_preprocessed failed with status {rc}")

    def fused(self):
        rc = self.L.qsa_forward(*self.fused_args)
        if rc != 0:
            raise RuntimeError(f"qsa_forward failed with status {rc}")

    def kernel_name(self) -> str:
        if self.split:
            return ("range_offsets_kernel + gather_attention_kernel (key-range split; from the second pass on "
                    "each launch also merges the previous pass) + range_combine_kernel (the last pass)")
        return "gather_attention_kernel"


def algorithmic_counts(w, N: int):
    rows = w.B * w.S_q
    flops = 4 * w.D * w.Hq * N
    kv_bytes = 4 * w.D * w.Hkv * N               # routed K and V rows, once per (query row, KV head)
    qo_bytes = 2 * 2 * rows * w.Hq * w.D         # Q read + O written, bf16
    list_bytes = 4 * N + 4 * rows                # compacted IDs read + counts
    return flops, kv_bytes + qo_bytes + list_bytes


def time_graph_replays(plan, dev, steps: int, warmup: int, flops: int) -> dict:
    """One step (preprocess + attention) captured in a HIP graph; replays timed with HIP events."""
    import torch

    eager_stream = plan.stream
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):  # torch's capture stream is current inside
        plan.set_stream(ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
        plan.preprocess()
        plan.attention()
    plan.set_stream(eager_stream)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"ms_per_step": ms, "value": flops / (ms * 1e-3) / 1e12}


def compulsory_bytes(w, plan, N: int) -> int:
    """Bytes no schedule can avoid: Q read, O written, lists and counts, and each K/V row some route
    names read once per KV head (distinct IDs per batch row, from the membership table)."""
    rows = w.B * w.S_q
    distinct = int(plan.mem.amax(dim=1).to(dtype=plan.cnt.dtype).sum().item())
    return 2 * 2 * w.D * w.Hkv * distinct + 2 * 2 * rows * w.Hq * w.D + 4 * N + 4 * rows


def backward_counts(w, N: int, segments: int):
    """Algorithmic flops and bytes of one qsa_backward call.

    dq kernel: routed K and V rows once per (query row, KV head), Q, dO and O
    read and dq written, lse read and delta written, lists and counts.  Key
    segments: the lists walked twice, one 16-byte record written per (row,
    64-key tile).  dk/dv kernel: K and V read and dK and dV written once per
    key, and per (segment, KV head) the G query heads' Q and dO rows, lse and
    delta, and the record."""
    rows = w.B * w.S_q
    G = w.Hq // w.Hkv
    flops = 10 * w.D * w.Hq * N
    b_dq = 4 * w.D * w.Hkv * N + 4 * 2 * rows * w.Hq * w.D + 2 * 4 * rows * w.Hq + 4 * N + 4 * rows
    b_seg = 2 * (4 * N + 4 * rows) + 16 * segments
    b_kv = 8 * w.D * w.Hkv * w.B * w.S_kv + (4 * G * w.D + 8 * G + 16) * w.Hkv * segments
    return flops, b_dq + b_seg + b_kv


def cpu_info() -> dict:
    """CPU model (/proc/cpuinfo) and the number of cores this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0))}


def cpu_baseline(w, q, k, v, routes, counts, target_s: float, windows: int = 16):
    """Time the fp64 oracle on `windows` windows of contiguous query rows centred at evenly spaced
    positions of the sequence (every batch row), so that the sample mixes short and long causal rows
    as the whole workload does.  The window length grows until the sample takes about target_s."""
    import oracle

    S_q = w.S_q
    per_row = counts.sum(axis=0)  # routed pairs per query position, summed over the batch
    threads = oracle.num_threads()
    n_win = min(windows, S_q)
    max_m = S_q // n_win

    def run(m):
        m = max(1, min(m, max_m))
        starts = [min(max(0, int((j + 0.5) * S_q / n_win) - m // 2), S_q - m) for j in range(n_win)]
        t0 = time.perf_counter()
        for s0 in starts:
            oracle.forward(q, k, v, routes, w.scale, rows=(s0, s0 + m))
        dt = time.perf_counter() - t0
        return dt, sum(int(per_row[s0:s0 + m].sum()) for s0 in starts), m, starts

    dt, n_routes, m, starts = run(max(1, threads // w.B))  # at least one row per thread in each window
    for _ in range(4):  # the first runs also pay thread start-up and page faults: grow until the sample is long
        if dt >= 0.8 * target_s or m >= max_m:
            break
        dt, n_routes, m, starts = run(int(m * min(16.0, 1.1 * target_s / max(dt, 1e-3))) + 1)
    rows = w.B * m * n_win
    tflops = 4 * w.D * w.Hq * n_routes / dt / 1e12
    return {
        "value": tflops,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"fp64 oracle forward on {n_win} windows of {m} query rows (of every batch row) centred at "
                  f"evenly spaced positions, first rows {starts[0]}..{starts[-1]}: {rows} rows, {n_routes} "
                  f"routed pairs (workload average {counts.sum() / counts.size:.1f} per row, sample "
                  f"{n_routes / rows:.1f}), {dt:.2f} s on {threads} OpenMP threads",
        **cpu_info(),
    }


def main():
    args = parse_args()
    if args.counter_reference_mib:
        counter_reference_copy(args.counter_reference_mib)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.which == "select":
        run_select(args)
        return

    import torch

    from workloads import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    print(f"[bench] generating workload {w.name}: {w.description}", file=sys.stderr, flush=True)
    _, q, k, v, routes = make_inputs(w.name)
    dev = torch.device("cuda", 0)
    plan = Plan(w, q, k, v, routes, dev)

    plan.preprocess()
    torch.cuda.synchronize()
    counts = plan.cnt.cpu().numpy()
    N = int(counts.sum())
    flops, gather_bytes = algorithmic_counts(w, N)
    min_bytes = compulsory_bytes(w, plan, N)

    if args.which == "backward":
        run_backward(args, w, plan, dev, N)
        return
    if args.which == "tile_lists":
        run_tile_lists(args, w, plan, dev)
        return

    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        plan.preprocess()
        plan.attention()
        plan.fused()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev = lambda: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    pre_ev = [ev() for _ in range(args.steps)]
    att_ev = [ev() for _ in range(args.steps)]
    fused_ev = [ev() for _ in range(args.steps)]
    total0, total1 = ev()
    scratch = torch.empty(args.flush_mib << 20, dtype=torch.uint8, device=dev) if args.flush_mib > 0 else None
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    total0.record(stream)
    for s in range(args.steps):
        if scratch is not None:
            scratch.fill_(s & 0xFF)
        pre_ev[s][0].record(stream)
        plan.preprocess()
        pre_ev[s][1].record(stream)
        att_ev[s][0].record(stream)
        plan.attention()
        att_ev[s][1].record(stream)
    total1.record(stream)
    torch.cuda.synchronize()
    # the fused entry point (route normalisation + attention in one call), same protocol
    for s in range(args.steps):
        if scratch is not None:
            scratch.fill_((s + 1) & 0xFF)
        fused_ev[s][0].record(stream)
        plan.fused()
        fused_ev[s][1].record(stream)
    torch.cuda.synchronize()

    att_ms = sorted(a.elapsed_time(b) for a, b in att_ev)
    ms_att = sum(att_ms) / args.steps
    ms_pre = sum(a.elapsed_time(b) for a, b in pre_ev) / args.steps
    fused_ms = sorted(a.elapsed_time(b) for a, b in fused_ev)
    if scratch is None:
        ms_step = total0.elapsed_time(total1) / args.steps
    else:  # flushes excluded: each step from its preprocess start to its attention end
        ms_step = sum(p[0].elapsed_time(a[1]) for p, a in zip(pre_ev, att_ev)) / args.steps

    graph = None
    if args.graph:
        graph = time_graph_replays(plan, dev, args.steps, args.warmup, flops)

    traffic = read_traffic(args.traffic, w.name)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, q, k, v, routes, counts, args.cpu_seconds)

    result = {
        "metric": METRIC,
        "value": flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name, "B": w.B, "S_q": w.S_q, "S_kv": w.S_kv, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D,
            "K": w.K, "q_offset": w.q_offset, "routes_N": N, "route_dtype": str(routes.dtype),
            "cache_flush_mib": args.flush_mib,
        },
        "roofline": attention_roofline(w, N, flops, gather_bytes, min_bytes, att_ms, traffic, plan.kernel_name()),
        "kernels_ms": {"preprocess(route_normalize+membership_tiles)": ms_pre, "attention": ms_att,
                       "qsa_forward(route_normalize+attention)": sum(fused_ms) / args.steps,
                       "qsa_forward_median": fused_ms[len(fused_ms) // 2], "qsa_forward_min": fused_ms[0]},
        "graph": graph,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


def attention_roofline(w, N, flops, gather_bytes, min_bytes, att_ms, traffic, kernel):
    """The attention call against the chip's roofline (see the module docstring)."""
    ms = sum(att_ms) / len(att_ms)
    t = ms * 1e-3
    t_flops = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    t_bytes = min_bytes / (HBM_PEAK_GBS * 1e9)
    if t_flops >= t_bytes:
        bound, achieved, peak, unit = "mfma", flops / t / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
    else:
        bound, achieved, peak, unit = "hbm", min_bytes / t / 1e9, HBM_PEAK_GBS, "GB/s"
    return {
        "bound": bound,
        "achieved": achieved,
        "peak": peak,
        "unit": unit,
        "frac": achieved / peak,
        "traffic": traffic,
        "kernel": kernel,
        "ms_per_launch": ms,
        "ms_per_launch_median": att_ms[len(att_ms) // 2],
        "ms_per_launch_min": att_ms[0],
        "flops_per_launch": flops,
        "flops_per_routed_pair": 4 * w.D * w.Hq,
        "routed_pairs": N,
        "compulsory_bytes": min_bytes,
        "t_floor_ms": max(t_flops, t_bytes) * 1e3,
        "gather_bytes_per_launch": gather_bytes,
        "gather_rate_GBs": gather_bytes / t / 1e9,
        "hbm_traffic_GBs": traffic / t / 1e9 if traffic else None,
    }


def read_traffic(path: str, workload: str):
    """HBM-side bytes per attention call from rocprofv3 counters (FETCH_SIZE and WRITE_SIZE, each scaled by the
    same counter on a copy of known size), when they were taken on the current kernel sources."""
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != _kernel_sha():
        return None
    entry = t.get("workloads", {}).get(workload)
    return entry.get("bytes_per_call") if entry else None


def run_backward(args, w, plan, dev, N):
    import torch

    plan.setup_backward(dev)
    print(f"[bench] backward warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(max(args.warmup, 1)):
        plan.backward()
    torch.cuda.synchronize()
    segments = plan.segment_count()
    flops, alg_bytes = backward_counts(w, N, segments)
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        ev[s][0].record(stream)
        plan.backward()
        ev[s][1].record(stream)
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in ev) / args.steps
    tflops = flops / (ms * 1e-3) / 1e12
    result = {
        "metric": "routed-attention backward TFLOP/s (dq, dk, dv; BF16) on 1 MI355X",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name, "B": w.B, "S_q": w.S_q, "S_kv": w.S_kv, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D,
            "K": w.K, "routes_N": N, "key_segments": segments,
        },
        "roofline": {
            # the compulsory floor is set by the flops, as for the forward (B_min is a few GB at most)
            "bound": "mfma",
            "achieved": tflops,
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
            "traffic": None,
            "kernel": "qsa_backward (dq_kernel + key segments + dkdv_kernel)",
            "ms_per_launch": ms,
            "gather_bytes_per_launch": alg_bytes,
            "gather_rate_GBs": alg_bytes / (ms * 1e-3) / 1e9,
        },
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)


def run_tile_lists(args, w, plan, dev):
    import torch

    import route_sparse_gqa_amd as qsa

    B, R, C = plan.tc.shape
    outs = {"partial_count": (B, R), "partial_idx": (B, R, C), "full_count": (B, R), "full_idx": (B, R, C),
            "rev_partial_count": (B, C), "rev_partial_idx": (B, C, R), "rev_full_count": (B, C),
            "rev_full_idx": (B, C, R)}
    bufs = [torch.empty(outs[k], dtype=torch.int32, device=dev) for k in qsa.TILE_LIST_KEYS]
    ptrs = [ctypes.c_void_p(t.data_ptr()) for t in bufs]

    def call(stream):
        rc = plan.L.qsa_tile_lists(ctypes.c_void_p(plan.tc.data_ptr()), B, R, C, *ptrs, stream)
        if rc != 0:
            raise RuntimeError(f"qsa_tile_lists failed with status {rc}")

    for _ in range(max(args.warmup, 1)):
        call(plan.stream)
    torch.cuda.synchronize()
    # One call is one kernel of a few microseconds, shorter than the host takes to issue a call, so
    # the timed calls are captured in one HIP graph and replayed: the kernels then run back to back
    # and the events time them, not the host.
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        capture = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        for _ in range(args.steps):
            call(capture)
    graph.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    tiles = B * R * C
    alg_bytes = 2 * 4 * tiles + 4 * 4 * tiles + 2 * 4 * (B * R + B * C)  # table read per direction, lists written
    achieved = alg_bytes / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "block-list compaction time (forward + reverse, partial + full) on 1 MI355X",
        "value": ms * 1e3, "unit": "us", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "int32", "data": "synthetic",
        "config": {"workload": w.name, "B": B, "block_rows": R, "block_cols": C},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None, "kernel": "tile_lists_kernel",
                     "ms_per_launch": ms, "alg_bytes_per_launch": alg_bytes},
        "cpu_baseline": None,
    }), flush=True)


def select_counts(w):
    """Scoring flops and algorithmic bytes of one qsa_select_token_ids call.

    Rows that see nv > kb blocks score every visible block: 2*H*D flops per
    (row, block).  Bytes: index queries of those rows and the block keys read,
    fp32 scores written and read back once, every output slot written."""
    c, kb = w.compress_ratio, w.token_budget // w.compress_ratio
    n_sum = rows_scored = 0
    for b in range(w.B):
        t = w.q_offset + np.arange(w.S_q, dtype=np.int64)
        nv = (t + 1) // c
        live = (t < w.lengths[b]) & (nv > kb) & (kb > 0)
        n_sum += int(nv[live].sum())
        rows_scored += int(live.sum())
    flops = 2 * w.H * w.D * n_sum
    alg_bytes = (2 * w.H * w.D * rows_scored + 2 * w.D * w.B * w.n_blocks + 8 * n_sum
                 + 4 * w.B * w.S_q * w.width)
    return flops, alg_bytes, n_sum, rows_scored


def select_cpu_baseline(w, iq, ck, lens, target_s: float):
    """Time the fp64 oracle's selection on query rows from the end of the workload (the longest rows)."""
    import oracle

    def run(nrows):
        r0 = w.S_q - nrows
        t0 = time.perf_counter()
        oracle.select_token_ids(iq, ck, lens, w.token_budget, w.compress_ratio, w.q_offset, rows=(r0, w.S_q))
        dt = time.perf_counter() - t0
        t = w.q_offset + np.arange(r0, w.S_q)
        nv = (t + 1) // w.compress_ratio
        kb = w.token_budget // w.compress_ratio
        n_sum = sum(int(nv[(t < L) & (nv > kb)].sum()) for L in w.lengths)
        return dt, n_sum, nrows

    dt, n_sum, nrows = run(4)
    while dt < 0.5 and nrows < w.S_q:
        dt, n_sum, nrows = run(min(w.S_q, nrows * 4))
    if dt < target_s and nrows < w.S_q:
        dt, n_sum, nrows = run(min(w.S_q, max(nrows, int(nrows * target_s / max(dt, 1e-3)))))
    return {
        "value": 2 * w.H * w.D * n_sum / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"fp64 oracle selection on the last {nrows} query rows of every batch row "
                  f"({n_sum} scored (row, block) pairs, {dt:.2f} s)",
    }


def run_select(args):
    import torch

    import route_sparse_gqa_amd as qsa
    from workloads import SELECT_WORKLOADS, make_select_inputs

    name = DEFAULT_SELECT_WORKLOAD if args.workload == DEFAULT_WORKLOAD else args.workload
    w = SELECT_WORKLOADS[name]
    print(f"[bench] generating selection workload {w.name}: {w.description}", file=sys.stderr, flush=True)
    _, iq, ck, lens = make_select_inputs(w.name)
    dev = torch.device("cuda", 0)
    L = qsa.lib()
    tq = torch.from_numpy(iq.view(np.int16)).to(dev).view(torch.bfloat16)
    tk = torch.from_numpy(ck.view(np.int16)).to(dev).view(torch.bfloat16)
    tl = torch.from_numpy(lens).to(dev)
    out = torch.empty((w.B, w.S_q, w.width), dtype=torch.int32, device=dev)
    ws_bytes = qsa.qsa_select_workspace_size(w.B, w.S_q, w.H, w.q_offset, w.compress_ratio)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    st = lambda t: (ctypes.c_int64 * t.dim())(*t.stride())
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    call_args = (p(tq), st(tq), p(tk), st(tk), p(tl), w.B, w.S_q, w.H, w.D, w.S_global, w.q_offset, w.token_budget,
                 w.compress_ratio, p(out), p(ws), ctypes.c_size_t(ws_bytes), ctypes.c_void_p(stream.cuda_stream))

    def call():
        rc = L.qsa_select_token_ids(*call_args)
        if rc != 0:
            raise RuntimeError(f"qsa_select_token_ids failed with status {rc}")

    print(f"[bench] select warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(max(args.warmup, 1)):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for s in range(args.steps):
        ev[s][0].record(stream)
        call()
        ev[s][1].record(stream)
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in ev) / args.steps
    flops, alg_bytes, n_sum, rows_scored = select_counts(w)
    tflops = flops / (ms * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle's selection on a bounded sample", file=sys.stderr, flush=True)
        cpu = select_cpu_baseline(w, iq, ck, lens, args.cpu_seconds)
    print(json.dumps({
        "metric": "route-selection block-scoring TFLOP/s (scores + top-k + expansion, BF16 in, FP32 scores) on 1 MI355X",
        "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "S_q": w.S_q, "S_global": w.S_global, "H": w.H, "D": w.D,
                   "compress_ratio": w.compress_ratio, "token_budget": w.token_budget, "q_offset": w.q_offset,
                   "rows_scored": rows_scored, "scored_pairs": n_sum},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / MFMA_BF16_PEAK_TFLOPS, "traffic": None,
                     "kernel": "qsa_select_token_ids (select_scores_kernel + select_topk_kernel)",
                     "ms_per_launch": ms, "alg_bytes_per_launch": alg_bytes,
                     "alg_bytes_rate_GBs": alg_bytes / (ms * 1e-3) / 1e9},
        "cpu_baseline": cpu,
    }), flush=True)


ATTENTION_SOURCES = ("gather_attention.hip", "device_common.h", "qsa_internal.h", "qsa_api.cpp")  # qsa_api: passes


def _kernel_sha() -> str:
    """sha256[:16] over the sources of the attention kernels (the counters are valid for this code only)."""
    import hashlib

    h = hashlib.sha256()
    for name in ATTENTION_SOURCES:
        with open(os.path.join(ROOT, "route_sparse_gqa_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
