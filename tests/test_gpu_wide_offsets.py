"""GPU parity of the attention kernels' 64-bit row-offset path.

The forward and the dq kernel form a gathered K/V row's address as
(route ID) x (row stride) from the (batch, head) base.  They use 32-bit
offsets only when the stride is non-negative and every row lies within
4 GiB of the base; otherwise 64-bit offsets.  A wrapped 32-bit offset would
read the wrong row, the failure class of the flex_qsa page's
`_membership_flat_offset` (offsets past 2^31 in a flat index).  Both ways to
reach the wide path are exercised through the C ABI:

* K and V passed reversed: the pointer at the last token and a negative
  token stride (the data stored last token first);
* K and V as strided views into buffers larger than 4 GiB (a token stride
  chosen so that the last rows sit past 2^32 bytes).

The result must meet the BF16 tolerance against the fp64 oracle on the
unreversed, contiguous tensors, and be bitwise equal to the result of the
same call on contiguous copies (the narrow path), since only the addressing
differs.  The backward (dq, dk, dv) is checked the same way, with K and V
stored those ways and, separately, with Q and dO stored those ways (the
dk/dv kernel forms its staged query rows' offsets by the same rule).
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
from workloads import random_dout
from workloads.generators import random_small_case

pytestmark = pytest.mark.gpu


def _wide_stride(S_kv: int, row_elems: int) -> int:
    """Token stride (elements, a multiple of 8) that puts the last row past 4 GiB from its base."""
    return max(row_elems, ((1 << 31) // (S_kv - 1) + 8) // 8 * 8)


def _p(x):
    return ctypes.c_void_p(x)


def _strides(s):
    return (ctypes.c_int64 * 4)(*s)


def _uses_wide_offsets(S_kv: int, D: int, token_stride: int) -> bool:
    """The rule the kernels follow (include/qsa.h, qsa_forward_preprocessed): 64-bit offsets when the
    token stride is negative or the last row ends past 4 GiB from the base."""
    return token_stride < 0 or (S_kv - 1) * token_stride * 2 + 2 * D > (1 << 32) - 1


class KVLayout:
    """K or V [B, S_kv, Hkv, D] (bf16 bits) stored in one of three ways; .ptr/.strides address it."""

    def __init__(self, bits: np.ndarray, how: str):
        B, S_kv, Hkv, D = bits.shape
        if how == "contiguous":
            self.buf = bf16_to_gpu(bits)
            self.ptr, self.strides = self.buf.data_ptr(), (S_kv * Hkv * D, Hkv * D, D, 1)
        elif how == "reversed":
            self.buf = bf16_to_gpu(np.ascontiguousarray(bits[:, ::-1]))  # token j stored at S_kv - 1 - j
            self.ptr = self.buf.data_ptr() + 2 * (S_kv - 1) * Hkv * D
            self.strides = (S_kv * Hkv * D, -Hkv * D, D, 1)
        elif how == "huge":
            ts = _wide_stride(S_kv, Hkv * D)
            self.buf = torch.zeros((B * S_kv - 1) * ts + Hkv * D, dtype=torch.bfloat16, device=device())
            view = torch.as_strided(self.buf, (B, S_kv, Hkv, D), (S_kv * ts, ts, D, 1))
            view.copy_(bf16_to_gpu(bits))
            self.ptr, self.strides = self.buf.data_ptr(), (S_kv * ts, ts, D, 1)
        else:
            raise ValueError(how)


CASES = [  # (B, S_q, S_kv, Hq, Hkv, D, K)
    (2, 70, 300, 16, 2, 256, 77),
    (1, 45, 130, 8, 1, 128, 40),
    (1, 33, 90, 4, 2, 64, 50),
]


def _forward(q, kl: KVLayout, vl: KVLayout, lst, cnt, shape, scale, lse=None):
    B, S_q, S_kv, Hq, Hkv, D, K = shape
    out = torch.empty((B, S_q, Hq, D), dtype=torch.bfloat16, device=device())
    st = qsa.lib().qsa_forward_preprocessed(
        _p(q.data_ptr()), _strides(q.stride()), _p(kl.ptr), _strides(kl.strides), _p(vl.ptr), _strides(vl.strides),
        _p(lst.data_ptr()), _p(cnt.data_ptr()), B, S_q, S_kv, Hq, Hkv, D, K, ctypes.c_float(scale),
        _p(out.data_ptr()), _p(lse.data_ptr()) if lse is not None else None, None, 0, None)
    assert st == 0, qsa.qsa_status_string(st)
    return out


@pytest.mark.parametrize("how", ["reversed", "huge"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_Sq{}_Skv{}_Hq{}_Hkv{}_D{}_K{}".format(*c))
def test_forward_wide_offsets(case, how):
    B, S_q, S_kv, Hq, Hkv, D, K = case
    print(f"wide-offset forward {how} {case}", flush=True)
    q, k, v, r = random_small_case(7 + sum(case), B, S_q, S_kv, Hq, Hkv, D, K)
    scale = 1.0 / math.sqrt(D)
    lst, cnt, _, _ = qsa.qsa_preprocess(torch.from_numpy(r).to(device()), S_kv)
    qg = bf16_to_gpu(q)
    kw, vw = KVLayout(k, how), KVLayout(v, how)
    assert _uses_wide_offsets(S_kv, D, kw.strides[1]) and _uses_wide_offsets(S_kv, D, vw.strides[1])
    kc, vc = KVLayout(k, "contiguous"), KVLayout(v, "contiguous")
    assert not _uses_wide_offsets(S_kv, D, kc.strides[1])
    wide = _forward(qg, kw, vw, lst, cnt, case, scale)
    narrow = _forward(qg, kc, vc, lst, cnt, case, scale)
    torch.cuda.synchronize()
    assert torch.equal(wide.view(torch.int16), narrow.view(torch.int16)), "wide and narrow offsets disagree"
    ref = oracle.forward(q, k, v, r, scale)
    _, ocnt = oracle.route_lists(r, S_kv)
    check_forward(gpu_bf16_bits(wide), ref, ocnt, v, f"wide forward {how} {case}")


def _addr(x):
    """(pointer, strides) of a tensor or of a KVLayout (any [B, S, H, D] bf16 array stored one of three ways)."""
    return (x.ptr, x.strides) if isinstance(x, KVLayout) else (x.data_ptr(), tuple(x.stride()))


def _backward(q, kl: KVLayout, vl: KVLayout, out, dout, lse, lst, cnt, shape, scale):
    B, S_q, S_kv, Hq, Hkv, D, K = shape
    dq = torch.empty((B, S_q, Hq, D), dtype=torch.bfloat16, device=device())
    dk = torch.empty((B, S_kv, Hkv, D), dtype=torch.bfloat16, device=device())
    dv = torch.empty_like(dk)
    ws_bytes = qsa.qsa_backward_workspace_size(B, S_q, S_kv, Hq, Hkv, D, K)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=device())
    (q_ptr, q_st), (g_ptr, g_st) = _addr(q), _addr(dout)
    st = qsa.lib().qsa_backward(
        _p(q_ptr), _strides(q_st), _p(kl.ptr), _strides(kl.strides), _p(vl.ptr), _strides(vl.strides),
        _p(out.data_ptr()), _p(g_ptr), _strides(g_st), _p(lse.data_ptr()), _p(lst.data_ptr()),
        _p(cnt.data_ptr()), B, S_q, S_kv, Hq, Hkv, D, K, ctypes.c_float(scale), _p(dq.data_ptr()),
        _p(dk.data_ptr()), _p(dv.data_ptr()), _p(ws.data_ptr()), ctypes.c_size_t(ws_bytes), None)
    assert st == 0, qsa.qsa_status_string(st)
    return dq, dk, dv


@pytest.mark.parametrize("how", ["reversed", "huge"])
def test_backward_wide_offsets(how):
    case = (2, 70, 300, 16, 2, 256, 77)
    B, S_q, S_kv, Hq, Hkv, D, K = case
    print(f"wide-offset backward {how} {case}", flush=True)
    q, k, v, r = random_small_case(99, B, S_q, S_kv, Hq, Hkv, D, K)
    scale = 1.0 / math.sqrt(D)
    lst, cnt, _, _ = qsa.qsa_preprocess(torch.from_numpy(r).to(device()), S_kv)
    qg = bf16_to_gpu(q)
    kc, vc = KVLayout(k, "contiguous"), KVLayout(v, "contiguous")
    kw, vw = KVLayout(k, how), KVLayout(v, how)
    assert _uses_wide_offsets(S_kv, D, kw.strides[1])
    lse = torch.empty((B, S_q, Hq), dtype=torch.float32, device=device())
    out = _forward(qg, kc, vc, lst, cnt, case, scale, lse)
    dout = bf16_to_gpu(random_dout(5, (B, S_q, Hq, D)))
    narrow = _backward(qg, kc, vc, out, dout, lse, lst, cnt, case, scale)
    wide = _backward(qg, kw, vw, out, dout, lse, lst, cnt, case, scale)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), wide, narrow):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{name}: wide and narrow offsets disagree"
    from test_gpu_backward import check_grad

    dq_ref, dk_ref, dv_ref = oracle.backward(q, k, v, gpu_bf16_bits(dout), r, scale)
    floor = 1e-3 * float(np.abs(dv_ref).max())
    check_grad(gpu_bf16_bits(wide[0]), dq_ref, f"dq {how}", floor)
    check_grad(gpu_bf16_bits(wide[1]), dk_ref, f"dk {how}", floor)
    check_grad(gpu_bf16_bits(wide[2]), dv_ref, f"dv {how}")


@pytest.mark.parametrize("how", ["reversed", "huge"])
def test_backward_wide_query_rows(how):
    """Q and dO stored reversed or past 4 GiB: the dk/dv kernel's staged rows take 64-bit offsets (and dq's
    query reads their 64-bit base); results bitwise equal to contiguous Q and dO, and within tolerance."""
    case = (1, 300, 200, 16, 2, 256, 60)
    B, S_q, S_kv, Hq, Hkv, D, K = case
    print(f"wide-offset backward query rows {how} {case}", flush=True)
    q, k, v, r = random_small_case(123, B, S_q, S_kv, Hq, Hkv, D, K)
    scale = 1.0 / math.sqrt(D)
    lst, cnt, _, _ = qsa.qsa_preprocess(torch.from_numpy(r).to(device()), S_kv)
    qg = bf16_to_gpu(q)
    kc, vc = KVLayout(k, "contiguous"), KVLayout(v, "contiguous")
    lse = torch.empty((B, S_q, Hq), dtype=torch.float32, device=device())
    out = _forward(qg, kc, vc, lst, cnt, case, scale, lse)
    dout_bits = random_dout(9, (B, S_q, Hq, D))
    dout = bf16_to_gpu(dout_bits)
    ql, gl = KVLayout(q, how), KVLayout(dout_bits, how)
    assert _uses_wide_offsets(S_q, Hq * D, ql.strides[1]) and _uses_wide_offsets(S_q, Hq * D, gl.strides[1])
    narrow = _backward(qg, kc, vc, out, dout, lse, lst, cnt, case, scale)
    wide = _backward(ql, kc, vc, out, gl, lse, lst, cnt, case, scale)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), wide, narrow):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{name}: wide and narrow query rows disagree"
    from test_gpu_backward import check_grad

    dq_ref, dk_ref, dv_ref = oracle.backward(q, k, v, dout_bits, r, scale)
    floor = 1e-3 * float(np.abs(dv_ref).max())
    check_grad(gpu_bf16_bits(wide[0]), dq_ref, f"dq {how}", floor)
    check_grad(gpu_bf16_bits(wide[1]), dk_ref, f"dk {how}", floor)
    check_grad(gpu_bf16_bits(wide[2]), dv_ref, f"dv {how}")
