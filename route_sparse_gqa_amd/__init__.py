"""Route-sparse GQA attention (forward and backward) on AMD Instinct MI355X.

Thin Python binding over the C ABI of ``libqsa.so`` (declared in
``include/qsa.h``).  The functions below only marshal arguments: they check
that tensors live on a ROCm GPU, copy inputs whose last stride is not 1
(the pages accept arbitrary strides and copy such inputs), allocate outputs
and workspace with ``torch.empty`` and pass raw device pointers, sizes and
torch's current HIP stream to the library.  Every step of the computation
runs in the library's HIP kernels; there is no other code path.

* ``qsa_preprocess(routes, kv_length, membership=False, tile_class=False)``
* ``qsa_tile_lists(tile_class)``
* ``qsa_forward(q, k, v, routes, scale=None)``
* ``qsa_forward_noalloc(q, k, v, routes, scale=None, out=None)`` (no workspace: the library's fixed scratch)
* ``qsa_forward_preprocessed(q, k, v, route_list, route_count, scale=None, return_lse=False)``
* ``qsa_backward(q, k, v, out, dout, lse, route_list, route_count, scale=None)``
* ``qsa_select_token_ids(index_queries, compressed_keys, sequence_lengths, token_budget, compress_ratio,
  query_position_offset=0, global_sequence_length=None, query_chunk_size=None)``
* ``qsa_forward_workspace_size(B, S_q, S_kv, Hq, Hkv, D, K)``,
  ``qsa_attention_workspace_size(B, S_q, S_kv, Hq, Hkv, D, K)``,
  ``qsa_backward_workspace_size(B, S_q, S_kv, Hq, Hkv, D, K)``,
  ``qsa_select_workspace_size(B, S_q, H, q_offset, compress_ratio)``,
  ``qsa_select_chunk_workspace_size(B, S_q, H, q_offset, compress_ratio, query_chunk_size)``
* ``qsa_status_string(status)``
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqsa.so")

QSA_INT32, QSA_INT64 = 0, 1
TILE = 128
MAX_ROUTES = 16384
MAX_GROUP = 16
NOALLOC_SCRATCH_BYTES = 64 << 20

# argument-error statuses raise ValueError; HIP errors raise RuntimeError
_HIP_ERROR = -12

_lib = None


class QSAError(ValueError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {qsa_status_string(status)} (status {status})")


class QSAHipError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {qsa_status_string(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """The loaded ``libqsa.so``; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m route_sparse_gqa_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        P64 = ctypes.POINTER(ctypes.c_int64)
        L.qsa_status_string.argtypes = [i32]
        L.qsa_status_string.restype = ctypes.c_char_p
        L.qsa_forward_workspace_size.argtypes = [i64] * 7
        L.qsa_forward_workspace_size.restype = ctypes.c_size_t
        L.qsa_attention_workspace_size.argtypes = [i64] * 7
        L.qsa_attention_workspace_size.restype = ctypes.c_size_t
        L.qsa_preprocess.argtypes = [p, i32, i64, i64, i64, P64, i64, p, p, p, p, p]
        L.qsa_preprocess.restype = i32
        L.qsa_forward.argtypes = [p, P64, p, P64, p, P64, p, i32, P64, i64, i64, i64, i64, i64, i64, i64,
                                  ctypes.c_float, p, p, ctypes.c_size_t, p]
        L.qsa_forward.restype = i32
        L.qsa_forward_noalloc.argtypes = [p, P64, p, P64, p, P64, p, i32, P64, i64, i64, i64, i64, i64, i64, i64,
                                          ctypes.c_float, p, p]
        L.qsa_forward_noalloc.restype = i32
        L.qsa_forward_preprocessed.argtypes = [p, P64, p, P64, p, P64, p, p, i64, i64, i64, i64, i64, i64, i64,
                                               ctypes.c_float, p, p, p, ctypes.c_size_t, p]
        L.qsa_forward_preprocessed.restype = i32
        L.qsa_tile_lists.argtypes = [p, i64, i64, i64, p, p, p, p, p, p, p, p, p]
        L.qsa_tile_lists.restype = i32
        L.qsa_backward_workspace_size.argtypes = [i64, i64, i64, i64, i64, i64, i64]
        L.qsa_backward_workspace_size.restype = ctypes.c_size_t
        L.qsa_backward.argtypes = [p, P64, p, P64, p, P64, p, p, P64, p, p, p, i64, i64, i64, i64, i64, i64, i64,
                                   ctypes.c_float, p, p, p, p, ctypes.c_size_t, p]
        L.qsa_backward.restype = i32
        L.qsa_select_workspace_size.argtypes = [i64, i64, i64, i64, i64]
        L.qsa_select_workspace_size.restype = ctypes.c_size_t
        L.qsa_select_chunk_workspace_size.argtypes = [i64, i64, i64, i64, i64, i64]
        L.qsa_select_chunk_workspace_size.restype = ctypes.c_size_t
        L.qsa_select_token_ids.argtypes = [p, P64, p, P64, p, i64, i64, i64, i64, i64, i64, i64, i64, p, p,
                                           ctypes.c_size_t, p]
        L.qsa_select_token_ids.restype = i32
        _lib = L
    return _lib


def qsa_status_string(status: int) -> str:
    return lib().qsa_status_string(int(status)).decode()


def qsa_forward_workspace_size(B: int, S_q: int, S_kv: int, Hq: int, Hkv: int, D: int, K: int) -> int:
    return int(lib().qsa_forward_workspace_size(int(B), int(S_q), int(S_kv), int(Hq), int(Hkv), int(D), int(K)))


def qsa_attention_workspace_size(B: int, S_q: int, S_kv: int, Hq: int, Hkv: int, D: int, K: int) -> int:
    return int(lib().qsa_attention_workspace_size(int(B), int(S_q), int(S_kv), int(Hq), int(Hkv), int(D), int(K)))


def qsa_backward_workspace_size(B: int, S_q: int, S_kv: int, Hq: int, Hkv: int, D: int, K: int) -> int:
    return int(lib().qsa_backward_workspace_size(int(B), int(S_q), int(S_kv), int(Hq), int(Hkv), int(D), int(K)))


def qsa_select_workspace_size(B: int, S_q: int, H: int, q_offset: int, compress_ratio: int) -> int:
    return int(lib().qsa_select_workspace_size(int(B), int(S_q), int(H), int(q_offset), int(compress_ratio)))


def qsa_select_chunk_workspace_size(B: int, S_q: int, H: int, q_offset: int, compress_ratio: int,
                                    query_chunk_size: int) -> int:
    return int(lib().qsa_select_chunk_workspace_size(int(B), int(S_q), int(H), int(q_offset), int(compress_ratio),
                                                     int(query_chunk_size)))


def _check(status: int, where: str) -> None:
    if status == 0:
        return
    if status == _HIP_ERROR:
        raise QSAHipError(status, where)
    raise QSAError(status, where)


def _strides(t: torch.Tensor):
    return (ctypes.c_int64 * t.dim())(*t.stride())


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require_gpu(*tensors: torch.Tensor) -> torch.device:
    dev = tensors[0].device
    for t in tensors:
        if t.device.type != "cuda":
            raise ValueError("route-sparse GQA runs on a ROCm GPU only; got a tensor on " + str(t.device))
        if t.device != dev:
            raise ValueError("all tensors must be on the same device")
    return dev


def _on_device(t: torch.Tensor, dev: torch.device, name: str) -> torch.Tensor:
    """A caller-supplied output or workspace: it must live on the inputs' GPU (the library writes
    through its raw pointer)."""
    if t.device != dev:
        raise ValueError(f"{name} must be on the inputs' device {dev}, got {t.device}")
    return t


def _route_dtype(routes: torch.Tensor) -> int:
    if routes.dtype == torch.int64:
        return QSA_INT64
    if routes.dtype == torch.int32:
        return QSA_INT32
    raise ValueError(f"routes must be int32 or int64, got {routes.dtype}")


def _bf16_operand(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be bfloat16, got {t.dtype}")
    if t.dim() != 4:
        raise ValueError(f"{name} must be 4-D, got shape {tuple(t.shape)}")
    if t.stride(-1) != 1 or any(s % 8 for s in t.stride()[:3]) or t.data_ptr() % 16:
        t = t.contiguous()  # arbitrary strides are accepted by copying
    return t


def qsa_preprocess(routes: torch.Tensor, kv_length: int, membership: bool = False, tile_class: bool = False):
    """Validate, deduplicate and compact routes on the GPU.

    Returns ``(route_list, route_count, membership_or_None, tile_class_or_None)``:
    int32 [B,S_q,K] (ascending distinct valid IDs, then -1), int32 [B,S_q],
    uint8 [B,S_q,round_up(kv_length,128)], int32 [B,ceil(S_q/128),ceil(kv_length/128)].
    """
    dev = _require_gpu(routes)
    if routes.dim() != 3:
        raise ValueError(f"routes must be [B, S_q, K], got shape {tuple(routes.shape)}")
    B, S_q, K = routes.shape
    dt = _route_dtype(routes)
    kv_length = int(kv_length)
    n_ti, n_tj = -(-S_q // TILE), -(-kv_length // TILE)
    ldm = n_tj * TILE
    lst = torch.empty((B, S_q, K), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, S_q), dtype=torch.int32, device=dev)
    mem = torch.empty((B, S_q, ldm), dtype=torch.uint8, device=dev) if membership else None
    tc = torch.empty((B, n_ti, n_tj), dtype=torch.int32, device=dev) if tile_class else None
    st = lib().qsa_preprocess(_ptr(routes), dt, B, S_q, K, _strides(routes), kv_length, _ptr(lst), _ptr(cnt),
                              _ptr(mem), _ptr(tc), _stream(dev))
    _check(st, "qsa_preprocess")
    return lst, cnt, mem, tc


TILE_LIST_KEYS = ("partial_count", "partial_idx", "full_count", "full_idx", "rev_partial_count", "rev_partial_idx",
                  "rev_full_count", "rev_full_idx")


def qsa_tile_lists(tile_class: torch.Tensor, which=TILE_LIST_KEYS) -> dict:
    """Forward and reverse partial/full block lists of a tile-class table [B, R, C] (int32 0/1/2).

    Returns a dict with the requested keys of ``TILE_LIST_KEYS``: counts [B,1,R] and
    indices [B,1,R,C] per block row, and the reverse counts [B,1,C] and indices
    [B,1,C,R] per block column (listed tiles ascending, then the other positions).
    """
    dev = _require_gpu(tile_class)
    if tile_class.dtype != torch.int32 or tile_class.dim() != 3:
        raise ValueError("tile_class must be an int32 [B, rows, cols] tensor")
    tile_class = tile_class.contiguous()
    B, R, C = tile_class.shape
    shapes = {"partial_count": (B, 1, R), "partial_idx": (B, 1, R, C), "full_count": (B, 1, R),
              "full_idx": (B, 1, R, C), "rev_partial_count": (B, 1, C), "rev_partial_idx": (B, 1, C, R),
              "rev_full_count": (B, 1, C), "rev_full_idx": (B, 1, C, R)}
    unknown = set(which) - set(TILE_LIST_KEYS)
    if unknown:
        raise ValueError(f"unknown block lists: {sorted(unknown)}")
    out = {k: torch.empty(shapes[k], dtype=torch.int32, device=dev) for k in TILE_LIST_KEYS if k in which}
    st = lib().qsa_tile_lists(_ptr(tile_class), B, R, C, *(_ptr(out.get(k)) for k in TILE_LIST_KEYS), _stream(dev))
    _check(st, "qsa_tile_lists")
    return out


def _attention_shapes(q, k, v):
    if k.shape != v.shape:
        raise ValueError(f"value must have key's shape: {tuple(k.shape)} vs {tuple(v.shape)}")
    B, S_q, Hq, D = q.shape
    Bk, S_kv, Hkv, Dk = k.shape
    if Bk != B or Dk != D:
        raise ValueError(f"query {tuple(q.shape)} and key {tuple(k.shape)} disagree on batch or head dim")
    return B, S_q, Hq, D, S_kv, Hkv


def _output(out: Optional[torch.Tensor], shape, dev) -> torch.Tensor:
    if out is None:
        return torch.empty(shape, dtype=torch.bfloat16, device=dev)
    if out.dtype != torch.bfloat16 or tuple(out.shape) != tuple(shape) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous bfloat16 tensor of shape {tuple(shape)}")
    if out.device != dev:
        raise ValueError("out must be on the inputs' device")
    return out


def _scale(scale: Optional[float], D: int) -> float:
    return 1.0 / math.sqrt(D) if scale is None else float(scale)


def qsa_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, routes: torch.Tensor,
                scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Route-sparse GQA forward: BF16 [B,S_q,Hq,D] x [B,S_kv,Hkv,D] with routes [B,S_q,K]."""
    dev = _require_gpu(q, k, v, routes)
    q, k, v = _bf16_operand(q, "query"), _bf16_operand(k, "key"), _bf16_operand(v, "value")
    B, S_q, Hq, D, S_kv, Hkv = _attention_shapes(q, k, v)
    if routes.dim() != 3 or routes.shape[0] != B or routes.shape[1] != S_q:
        raise ValueError(f"routes must be [B, S_q, K] = [{B}, {S_q}, K], got {tuple(routes.shape)}")
    K = routes.shape[2]
    dt = _route_dtype(routes)
    out = _output(out, (B, S_q, Hq, D), dev)
    ws_bytes = qsa_forward_workspace_size(B, S_q, S_kv, Hq, Hkv, D, K)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    _on_device(workspace, dev, "workspace")
    st = lib().qsa_forward(_ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v), _strides(v), _ptr(routes), dt,
                           _strides(routes), B, S_q, S_kv, Hq, Hkv, D, K, _scale(scale, D), _ptr(out),
                           _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev))
    _check(st, "qsa_forward")
    return out


def qsa_forward_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, routes: torch.Tensor,
                        scale: Optional[float] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """``qsa_forward`` without a workspace: the library's fixed device scratch (64 MiB per GPU) holds it.
    For callers that cannot allocate; calls that overlap on one GPU race.  ``out`` is allocated when not
    given (pass it to allocate nothing here either)."""
    dev = _require_gpu(q, k, v, routes)
    q, k, v = _bf16_operand(q, "query"), _bf16_operand(k, "key"), _bf16_operand(v, "value")
    B, S_q, Hq, D, S_kv, Hkv = _attention_shapes(q, k, v)
    if routes.dim() != 3 or routes.shape[0] != B or routes.shape[1] != S_q:
        raise ValueError(f"routes must be [B, S_q, K] = [{B}, {S_q}, K], got {tuple(routes.shape)}")
    K = routes.shape[2]
    dt = _route_dtype(routes)
    out = _output(out, (B, S_q, Hq, D), dev)
    st = lib().qsa_forward_noalloc(_ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v), _strides(v), _ptr(routes),
                                   dt, _strides(routes), B, S_q, S_kv, Hq, Hkv, D, K, _scale(scale, D), _ptr(out),
                                   _stream(dev))
    _check(st, "qsa_forward_noalloc")
    return out


def _lists(route_list: torch.Tensor, route_count: torch.Tensor, B: int, S_q: int):
    if route_list.dtype != torch.int32 or route_count.dtype != torch.int32:
        raise ValueError("route_list and route_count must be int32")
    if route_list.dim() != 3 or tuple(route_list.shape[:2]) != (B, S_q) or tuple(route_count.shape) != (B, S_q):
        raise ValueError("route_list must be [B, S_q, K] and route_count [B, S_q]")
    return route_list.contiguous(), route_count.contiguous()


def qsa_forward_preprocessed(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, route_list: torch.Tensor,
                             route_count: torch.Tensor, scale: Optional[float] = None,
                             out: Optional[torch.Tensor] = None, return_lse: bool = False,
                             workspace: Optional[torch.Tensor] = None):
    """Gather-attention alone, on lists produced by ``qsa_preprocess(routes, S_kv)``.

    Returns ``out``, or ``(out, lse)`` with ``lse`` float32 [B,S_q,Hq] (natural-log
    log-sum-exp of each row's scaled scores, -inf for empty rows) when ``return_lse``.
    ``workspace`` (uint8, on the inputs' device) defaults to the recommended
    ``qsa_attention_workspace_size`` bytes; shapes that need none get none.
    """
    dev = _require_gpu(q, k, v, route_list, route_count)
    q, k, v = _bf16_operand(q, "query"), _bf16_operand(k, "key"), _bf16_operand(v, "value")
    B, S_q, Hq, D, S_kv, Hkv = _attention_shapes(q, k, v)
    route_list, route_count = _lists(route_list, route_count, B, S_q)
    K = route_list.shape[2]
    out = _output(out, (B, S_q, Hq, D), dev)
    lse = torch.empty((B, S_q, Hq), dtype=torch.float32, device=dev) if return_lse else None
    if workspace is None:
        ws_bytes = qsa_attention_workspace_size(B, S_q, S_kv, Hq, Hkv, D, K)
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes > 0 else None
    if workspace is not None:
        _on_device(workspace, dev, "workspace")
    st = lib().qsa_forward_preprocessed(_ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v), _strides(v),
                                        _ptr(route_list), _ptr(route_count), B, S_q, S_kv, Hq, Hkv, D, K,
                                        _scale(scale, D), _ptr(out), _ptr(lse), _ptr(workspace),
                                        workspace.numel() * workspace.element_size() if workspace is not None else 0,
                                        _stream(dev))
    _check(st, "qsa_forward_preprocessed")
    return (out, lse) if return_lse else out


def qsa_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, dout: torch.Tensor,
                 lse: torch.Tensor, route_list: torch.Tensor, route_count: torch.Tensor,
                 scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None):
    """Gradients (dq, dk, dv), bfloat16, of ``qsa_forward_preprocessed`` for upstream gradient ``dout``.

    ``out`` and ``lse`` are that forward's output and log-sum-exp (``return_lse=True``).
    Deterministic: equal inputs give bitwise-equal gradients.
    """
    dev = _require_gpu(q, k, v, out, dout, lse, route_list, route_count)
    q, k, v = _bf16_operand(q, "query"), _bf16_operand(k, "key"), _bf16_operand(v, "value")
    dout = _bf16_operand(dout, "dout")
    B, S_q, Hq, D, S_kv, Hkv = _attention_shapes(q, k, v)
    if tuple(dout.shape) != (B, S_q, Hq, D) or tuple(out.shape) != (B, S_q, Hq, D):
        raise ValueError("out and dout must have the query's shape")
    if out.dtype != torch.bfloat16:
        raise ValueError("out must be bfloat16")
    out = out.contiguous()
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, S_q, Hq):
        raise ValueError(f"lse must be float32 [B, S_q, Hq] = [{B}, {S_q}, {Hq}]")
    lse = lse.contiguous()
    route_list, route_count = _lists(route_list, route_count, B, S_q)
    K = route_list.shape[2]
    dq = torch.empty((B, S_q, Hq, D), dtype=torch.bfloat16, device=dev)
    dk = torch.empty((B, S_kv, Hkv, D), dtype=torch.bfloat16, device=dev)
    dv = torch.empty((B, S_kv, Hkv, D), dtype=torch.bfloat16, device=dev)
    ws_bytes = qsa_backward_workspace_size(B, S_q, S_kv, Hq, Hkv, D, K)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    _on_device(workspace, dev, "workspace")
    st = lib().qsa_backward(_ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v), _strides(v), _ptr(out),
                            _ptr(dout), _strides(dout), _ptr(lse), _ptr(route_list), _ptr(route_count), B, S_q,
                            S_kv, Hq, Hkv, D, K, _scale(scale, D), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream(dev))
    _check(st, "qsa_backward")
    return dq, dk, dv


def qsa_select_token_ids(index_queries: torch.Tensor, compressed_keys: torch.Tensor, sequence_lengths: torch.Tensor,
                         token_budget: int, compress_ratio: int, query_position_offset: int = 0,
                         global_sequence_length: Optional[int] = None, query_chunk_size: Optional[int] = None,
                         out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Route selection: int32 token IDs [B, S_q, token_budget + compress_ratio - 1] (-1 = empty slot).

    ``index_queries`` bf16 [B,S_q,H,D], ``compressed_keys`` bf16 [B,n_blocks,1,D] with
    ``n_blocks >= global_sequence_length // compress_ratio``, ``sequence_lengths`` int [B]
    (right-padded logical lengths, global positions; read on the device, no host sync).
    ``global_sequence_length`` defaults to the local query length.  ``query_chunk_size``
    bounds the rows scored per pass (fp32 scores [rows, visible blocks]); ``None`` scores
    every row in one pass.  Chunking changes no result.
    """
    dev = _require_gpu(index_queries, compressed_keys, sequence_lengths)
    iq = _bf16_operand(index_queries, "index_queries")
    ck = _bf16_operand(compressed_keys, "compressed_keys")
    B, S_q, H, D = iq.shape
    c, budget, q_off = int(compress_ratio), int(token_budget), int(query_position_offset)
    S_global = S_q if global_sequence_length is None else int(global_sequence_length)
    if ck.shape[0] != B or ck.shape[2] != 1 or ck.shape[3] != D:
        raise ValueError(f"compressed_keys must be [B, n_blocks, 1, D] = [{B}, n, 1, {D}], got {tuple(ck.shape)}")
    if c >= 1 and ck.shape[1] < S_global // c:
        raise ValueError(f"compressed_keys holds {ck.shape[1]} blocks, fewer than {S_global} // {c}")
    if tuple(sequence_lengths.shape) != (B,):
        raise ValueError(f"sequence_lengths must be [B] = [{B}]")
    lens = sequence_lengths.to(torch.int64).contiguous()
    width = budget + c - 1
    if out is None:
        out = torch.empty((B, S_q, max(width, 0)), dtype=torch.int32, device=dev)
    elif out.dtype != torch.int32 or tuple(out.shape) != (B, S_q, width) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous int32 tensor of shape {(B, S_q, width)}")
    _on_device(out, dev, "out")
    if workspace is None:
        if query_chunk_size is None:
            ws_bytes = qsa_select_workspace_size(B, S_q, H, q_off, c)
        else:
            ws_bytes = qsa_select_chunk_workspace_size(B, S_q, H, q_off, c, max(1, int(query_chunk_size)))
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    _on_device(workspace, dev, "workspace")
    st = lib().qsa_select_token_ids(_ptr(iq), _strides(iq), _ptr(ck), _strides(ck), _ptr(lens), B, S_q, H, D,
                                    S_global, q_off, budget, c, _ptr(out), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(dev))
    _check(st, "qsa_select_token_ids")
    return out


__all__ = [
    "qsa_select_token_ids",
    "qsa_select_workspace_size",
    "qsa_select_chunk_workspace_size",
    "qsa_preprocess",
    "qsa_tile_lists",
    "qsa_forward",
    "qsa_forward_noalloc",
    "qsa_forward_preprocessed",
    "qsa_backward",
    "qsa_forward_workspace_size",
    "qsa_attention_workspace_size",
    "qsa_backward_workspace_size",
    "qsa_status_string",
    "lib",
    "QSAError",
    "QSAHipError",
]
