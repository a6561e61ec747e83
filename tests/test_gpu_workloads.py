"""Full-size parity on the five seeded workloads, in the launch configuration
bench.py times (qsa_preprocess with membership and tile classes, then
qsa_forward_preprocessed).

* route lists, counts, membership (every byte, padding included, copied back
  in row chunks) and tile classes: bit-exact against the oracle on all rows;
* attention: BF16 tolerance against the fp64 oracle on every row of the four
  smaller workloads and on sampled row ranges of long_int64, including its
  last 512 rows, whose membership offsets lie past 2^31;
* the fused qsa_forward gives the same bits as the two-call path.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import route_sparse_gqa_amd as qsa
from gpu_util import bf16_to_gpu, check_forward, device, gpu_bf16_bits
from workloads import WORKLOADS, make_inputs

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]

FORWARD_ROWS = {  # query-row ranges checked against the oracle (None = every row)
    "tiny": None,
    "right_padded": None,
    "packed_thd": None,
    "cp_slice": None,
    "long_int64": [(0, 256), (30000, 30256), (65024, 65536)],
}
MEMBERSHIP_CHUNK_ROWS = 1024


def _log(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_parity(name):
    w = WORKLOADS[name]
    _log(f"[{name}] generating {w.description}")
    _, q, k, v, r = make_inputs(name)
    qg, kg, vg, rg = bf16_to_gpu(q), bf16_to_gpu(k), bf16_to_gpu(v), torch.from_numpy(r).to(device())

    _log(f"[{name}] preprocess on the GPU")
    lst, cnt, mem, tc = qsa.qsa_preprocess(rg, w.S_kv, membership=True, tile_class=True)
    out = qsa.qsa_forward_preprocessed(qg, kg, vg, lst, cnt, w.scale)
    fused = qsa.qsa_forward(qg, kg, vg, rg, w.scale)
    torch.cuda.synchronize()

    _log(f"[{name}] lists and counts vs oracle")
    olst, ocnt = oracle.route_lists(r, w.S_kv)
    np.testing.assert_array_equal(cnt.cpu().numpy(), ocnt)
    np.testing.assert_array_equal(lst.cpu().numpy(), olst)
    del olst

    _log(f"[{name}] tile classes vs oracle")
    np.testing.assert_array_equal(tc.cpu().numpy(), oracle.tile_class(r, w.S_kv))

    _log(f"[{name}] membership vs oracle, {MEMBERSHIP_CHUNK_ROWS}-row chunks")
    for b in range(w.B):
        for r0 in range(0, w.S_q, MEMBERSHIP_CHUNK_ROWS):
            r1 = min(w.S_q, r0 + MEMBERSHIP_CHUNK_ROWS)
            got = mem[b, r0:r1].cpu().numpy()
            ref = oracle.membership(r[b:b + 1, r0:r1], w.S_kv)[0]
            if not np.array_equal(got, ref):
                bad = np.argwhere(got != ref)[0]
                pytest.fail(f"{name}: membership differs at b={b} row={r0 + bad[0]} col={bad[1]}")

    assert torch.equal(out.view(torch.int16), fused.view(torch.int16)), "fused path differs from two-call path"

    ranges = FORWARD_ROWS[name] or [(0, w.S_q)]
    got_all = gpu_bf16_bits(out)
    for (r0, r1) in ranges:
        _log(f"[{name}] forward rows [{r0}, {r1}) vs oracle")
        ref = oracle.forward(q, k, v, r, w.scale, rows=(r0, r1))
        check_forward(got_all[:, r0:r1], ref, ocnt[:, r0:r1], v, f"{name} rows [{r0},{r1})")
    _log(f"[{name}] ok: N={int(ocnt.sum())}, empty rows={int((ocnt == 0).sum())}")


def test_right_padded_int32_routes_identical():
    w = WORKLOADS["right_padded"]
    _, _, _, _, r64 = make_inputs(w.name, with_qkv=False)
    a = qsa.qsa_preprocess(torch.from_numpy(r64).to(device()), w.S_kv, True, True)
    b = qsa.qsa_preprocess(torch.from_numpy(r64.astype(np.int32)).to(device()), w.S_kv, True, True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
