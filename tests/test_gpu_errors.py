"""Argument errors of the C ABI, forced from the host with real device tensors.

Every case has exactly one invalid argument, which the library rejects on
the host before anything is enqueued.
"""

from __future__ import annotations

import ctypes

import pytest
import torch

import route_sparse_gqa_amd as qsa
from gpu_util import device

pytestmark = pytest.mark.gpu

ERR = dict(NULL=-1, EMPTY=-2, KV=-3, HEADS=-4, HEAD_DIM=-5, DTYPE=-6, SCALE=-7, LAYOUT=-8, ALIAS=-9,
           WORKSPACE=-10, LIMIT=-11)


def _inputs(B=1, S_q=8, S_kv=16, Hq=4, Hkv=2, D=64, K=4):
    d = device()
    q = torch.randn(B, S_q, Hq, D, device=d).to(torch.bfloat16)
    k = torch.randn(B, S_kv, Hkv, D, device=d).to(torch.bfloat16)
    v = torch.randn(B, S_kv, Hkv, D, device=d).to(torch.bfloat16)
    r = torch.randint(-2, S_kv + 2, (B, S_q, K), device=d)
    return q, k, v, r


def _raw_forward(q, k, v, r, *, dims=None, scale=0.125, out=None, ws=None, ws_bytes=None, dtype=None):
    L = qsa.lib()
    B, S_q, Hq, D = q.shape
    S_kv, Hkv = k.shape[1], k.shape[2]
    K = r.shape[2]
    if dims:
        B, S_q, S_kv, Hq, Hkv, D, K = dims
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    need = qsa.qsa_forward_workspace_size(q.shape[0], q.shape[1], k.shape[1], q.shape[2], k.shape[2], q.shape[3],
                                          r.shape[2])
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = lambda t: (ctypes.c_int64 * t.dim())(*t.stride())
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    return L.qsa_forward(p(q), st(q), p(k), st(k), p(v), st(v), p(r), 1 if dtype is None else dtype, st(r),
                         B, S_q, S_kv, Hq, Hkv, D, K, scale, p(out), p(ws),
                         need if ws_bytes is None else ws_bytes, None)


def test_valid_call_succeeds():
    q, k, v, r = _inputs()
    assert _raw_forward(q, k, v, r) == 0
    torch.cuda.synchronize()


@pytest.mark.parametrize("scale", [0.0, -1.0, float("nan"), float("inf")])
def test_bad_scale(scale):
    q, k, v, r = _inputs()
    assert _raw_forward(q, k, v, r, scale=scale) == ERR["SCALE"]
    with pytest.raises(ValueError):
        qsa.qsa_forward(q, k, v, r, scale)


def test_heads_not_multiple():
    q, k, v, r = _inputs(Hq=6, Hkv=4)
    assert _raw_forward(q, k, v, r) == ERR["HEADS"]


def test_head_dim_unsupported():
    q, k, v, r = _inputs(D=96)
    assert _raw_forward(q, k, v, r) == ERR["HEAD_DIM"]


def test_group_too_large():
    q, k, v, r = _inputs(Hq=32, Hkv=1)
    assert _raw_forward(q, k, v, r) == ERR["LIMIT"]


def test_route_dtype():
    q, k, v, r = _inputs()
    assert _raw_forward(q, k, v, r, dtype=7) == ERR["DTYPE"]
    with pytest.raises(ValueError):
        qsa.qsa_forward(q, k, v, r.to(torch.int16))


def test_empty_dims():
    q, k, v, r = _inputs()
    for i in range(7):
        dims = [1, 8, 16, 4, 2, 64, 4]
        dims[i] = 0
        assert _raw_forward(q, k, v, r, dims=dims) == ERR["EMPTY"], i


def test_workspace_too_small_or_missing():
    q, k, v, r = _inputs()
    need = qsa.qsa_forward_workspace_size(1, 8, 16, 4, 2, 64, 4)
    assert _raw_forward(q, k, v, r, ws_bytes=need - 1) == ERR["WORKSPACE"]


def test_output_aliasing_input():
    q, k, v, r = _inputs()
    assert _raw_forward(q, k, v, r, out=q) == ERR["ALIAS"]


def test_layout_last_stride():
    q, k, v, r = _inputs()
    wide = torch.zeros(1, 8, 4, 128, dtype=torch.bfloat16, device=device())
    assert _raw_forward(wide[..., ::2], k, v, r) == ERR["LAYOUT"]


def test_preprocess_errors():
    L = qsa.lib()
    r = torch.randint(0, 10, (1, 4, 3), device=device())
    lst = torch.empty(1, 4, 3, dtype=torch.int32, device=device())
    cnt = torch.empty(1, 4, dtype=torch.int32, device=device())
    st = (ctypes.c_int64 * 3)(*r.stride())
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    assert L.qsa_preprocess(p(r), 1, 1, 4, 3, st, 0, p(lst), p(cnt), None, None, None) == ERR["KV"]
    assert L.qsa_preprocess(p(r), 1, 1, 4, 3, st, (1 << 31) + 1, p(lst), p(cnt), None, None, None) == ERR["KV"]
    assert L.qsa_preprocess(p(r), 3, 1, 4, 3, st, 10, p(lst), p(cnt), None, None, None) == ERR["DTYPE"]
    assert L.qsa_preprocess(p(r), 1, 1, 4, 0, st, 10, p(lst), p(cnt), None, None, None) == ERR["EMPTY"]
    assert L.qsa_preprocess(None, 1, 1, 4, 3, st, 10, p(lst), p(cnt), None, None, None) == ERR["NULL"]
    assert L.qsa_preprocess(p(r), 1, 1, 4, 3, st, 10, p(lst), p(lst), None, None, None) == ERR["ALIAS"]
    assert L.qsa_preprocess(p(r), 1, 1, 4, 20000, st, 10, p(lst), p(cnt), None, None, None) == ERR["LIMIT"]
    assert L.qsa_preprocess(p(r), 1, 1, 4, 3, st, 10, p(lst), p(cnt), None, None, None) == 0
    torch.cuda.synchronize()


def test_cpu_tensors_fail_loudly():
    q, k, v, r = (t.cpu() for t in _inputs())
    with pytest.raises(ValueError, match="ROCm GPU"):
        qsa.qsa_forward(q, k, v, r)


def test_caller_buffers_on_another_device_fail_before_any_launch():
    """A workspace or output the caller passes must be on the inputs' GPU: the library writes
    through its pointer, so a host tensor is refused by the binding."""
    q, k, v, r = _inputs()
    with pytest.raises(ValueError, match="workspace must be on"):
        qsa.qsa_forward(q, k, v, r, workspace=torch.empty(1 << 16, dtype=torch.uint8))
    iq = torch.zeros(1, 64, 4, 64, dtype=torch.bfloat16, device=device())
    ck = torch.zeros(1, 16, 1, 64, dtype=torch.bfloat16, device=device())
    lens = torch.full((1,), 64, dtype=torch.int64, device=device())
    with pytest.raises(ValueError, match="out must be on"):
        qsa.qsa_select_token_ids(iq, ck, lens, 16, 4, out=torch.empty(1, 64, 19, dtype=torch.int32))
    with pytest.raises(ValueError, match="workspace must be on"):
        qsa.qsa_select_token_ids(iq, ck, lens, 16, 4, workspace=torch.empty(1 << 20, dtype=torch.uint8))
