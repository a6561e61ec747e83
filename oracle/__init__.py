"""CPU oracle for route-sparse GQA attention (fp64, plain C + a thin numpy wrapper).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark may import this package; the product path never does.  It
shares no code with the HIP library; the two meet only at the seeded inputs
from ``workloads``.

Functions (all inputs contiguous numpy arrays; bfloat16 tensors are passed as
their ``uint16`` bit patterns):

* ``route_lists(routes, kv_length)``      -> (int32 [B,S_q,K], int32 [B,S_q])
* ``membership(routes, kv_length)``       -> uint8 [B,S_q,round_up(kv_length,128)]
* ``tile_class(routes, kv_length)``       -> int32 [B,ceil(S_q/128),ceil(kv_length/128)]
* ``forward(q, k, v, routes, scale, rows=None)`` -> float64 [B,rows,Hq,D]
* ``tile_lists(kinds)`` -> dict of int32 arrays: ``partial_count`` [B,1,R],
  ``partial_idx`` [B,1,R,C], ``full_count``, ``full_idx``, and the reverse
  ``rev_partial_count`` [B,1,C], ``rev_partial_idx`` [B,1,C,R], ``rev_full_count``,
  ``rev_full_idx`` (R, C = block rows and columns of ``kinds`` [B,R,C])
* ``select_token_ids(iq, ck, seq_lens, token_budget, compress_ratio, q_offset=0, rows=None)``
  -> int32 [B,rows,token_budget+compress_ratio-1] (iq [B,S_q,H,D], ck [B,n_blocks,D] bf16 bits)
* ``block_scores(iq, ck, rows=None)`` -> float64 [B,rows,n_blocks]: every block's score, visible or not
* ``lse(q, k, routes, scale, rows=None)`` -> float64 [B,rows,Hq] (natural log; -inf for empty rows)
* ``backward(q, k, v, dout, routes, scale, rows=None, keys=None)``
  -> (dq [B,rows,Hq,D], dk [B,keys,Hkv,D], dv [B,keys,Hkv,D]) float64

See ``qsa_oracle.c`` for the definitions and the passages they follow.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qsa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

TILE = 128
TILE_LIST_KEYS = ("partial_count", "partial_idx", "full_count", "full_idx", "rev_partial_count", "rev_partial_idx",
                  "rev_full_count", "rev_full_idx")


def build(force: bool = True) -> str:
    """Compile ``liboracle.so`` with gcc (OpenMP over rows)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
             _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class Oracle:
    """ctypes handle on one build of ``qsa_oracle.c`` (tests may load a variant)."""

    def __init__(self, lib_path: str):
        lib = ctypes.CDLL(lib_path)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_route_lists.argtypes = [p, i64, i64, i64, p, p]
        lib.oracle_membership.argtypes = [p, i64, i64, i64, i64, p]
        lib.oracle_tile_class.argtypes = [p, i64, i64, i64, i64, p]
        lib.oracle_forward.argtypes = [p, p, p, p, i64, i64, i64, i64, i64, i64, i64,
                                       ctypes.c_double, i64, i64, p]
        lib.oracle_tile_lists.argtypes = [p, i64, i64, i64, p, p, p, p, p, p, p, p]
        lib.oracle_tile_lists.restype = None
        lib.oracle_lse.argtypes = [p, p, p, i64, i64, i64, i64, i64, i64, i64, ctypes.c_double, i64, i64, p]
        lib.oracle_backward.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, i64, i64,
                                        ctypes.c_double, i64, i64, i64, i64, p, p, p]
        lib.oracle_select_token_ids.argtypes = [p, p, p, i64, i64, i64, i64, i64, i64, i64, i64, i64, i64, p]
        lib.oracle_block_scores.argtypes = [p, p, i64, i64, i64, i64, i64, i64, i64, p]
        for f in (lib.oracle_route_lists, lib.oracle_membership, lib.oracle_tile_class, lib.oracle_forward,
                  lib.oracle_lse, lib.oracle_backward, lib.oracle_select_token_ids, lib.oracle_block_scores):
            f.restype = None
        self.lib = lib

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def route_lists(self, routes, kv_length):
        r = _routes64(routes)
        B, S_q, K = r.shape
        lst = np.empty((B, S_q, K), dtype=np.int32)
        cnt = np.empty((B, S_q), dtype=np.int32)
        self.lib.oracle_route_lists(_ptr(r), B * S_q, K, int(kv_length), _ptr(lst), _ptr(cnt))
        return lst, cnt

    def membership(self, routes, kv_length):
        r = _routes64(routes)
        B, S_q, K = r.shape
        ldm = ldm_of(kv_length)
        out = np.empty((B, S_q, ldm), dtype=np.uint8)
        self.lib.oracle_membership(_ptr(r), B * S_q, K, int(kv_length), ldm, _ptr(out))
        return out

    def tile_class(self, routes, kv_length):
        r = _routes64(routes)
        B, S_q, K = r.shape
        n_ti, n_tj = (S_q + TILE - 1) // TILE, (int(kv_length) + TILE - 1) // TILE
        out = np.empty((B, n_ti, n_tj), dtype=np.int32)
        self.lib.oracle_tile_class(_ptr(r), B, S_q, K, int(kv_length), _ptr(out))
        return out

    def forward(self, q, k, v, routes, scale, rows=None):
        for name, t in (("q", q), ("k", k), ("v", v)):
            if t.dtype != np.uint16:
                raise TypeError(f"{name} must hold bfloat16 bits as uint16")
        q, k, v = (np.ascontiguousarray(t) for t in (q, k, v))
        r = _routes64(routes)
        B, S_q, Hq, D = q.shape
        _, S_kv, Hkv, _ = k.shape
        K = r.shape[2]
        if Hkv < 1 or Hq % Hkv != 0:
            raise ValueError("Hq must be a positive multiple of Hkv")
        r0, r1 = (0, S_q) if rows is None else (int(rows[0]), int(rows[1]))
        out = np.empty((B, r1 - r0, Hq, D), dtype=np.float64)
        self.lib.oracle_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(r), B, S_q, S_kv, Hq, Hkv, D, K,
                                float(scale), r0, r1, _ptr(out))
        return out

    def tile_lists(self, kinds):
        kinds = np.ascontiguousarray(kinds, dtype=np.int32)
        B, R, C = kinds.shape
        out = {
            "partial_count": np.empty((B, 1, R), np.int32), "partial_idx": np.empty((B, 1, R, C), np.int32),
            "full_count": np.empty((B, 1, R), np.int32), "full_idx": np.empty((B, 1, R, C), np.int32),
            "rev_partial_count": np.empty((B, 1, C), np.int32), "rev_partial_idx": np.empty((B, 1, C, R), np.int32),
            "rev_full_count": np.empty((B, 1, C), np.int32), "rev_full_idx": np.empty((B, 1, C, R), np.int32),
        }
        self.lib.oracle_tile_lists(_ptr(kinds), B, R, C, *(_ptr(out[k]) for k in TILE_LIST_KEYS))
        return out

    def lse(self, q, k, routes, scale, rows=None):
        q, k = _bf16_bits(q=q, k=k)
        r = _routes64(routes)
        B, S_q, Hq, D = q.shape
        _, S_kv, Hkv, _ = k.shape
        if Hkv < 1 or Hq % Hkv != 0:
            raise ValueError("Hq must be a positive multiple of Hkv")
        r0, r1 = (0, S_q) if rows is None else (int(rows[0]), int(rows[1]))
        out = np.empty((B, r1 - r0, Hq), dtype=np.float64)
        self.lib.oracle_lse(_ptr(q), _ptr(k), _ptr(r), B, S_q, S_kv, Hq, Hkv, D, r.shape[2], float(scale),
                            r0, r1, _ptr(out))
        return out

    def backward(self, q, k, v, dout, routes, scale, rows=None, keys=None):
        q, k, v, dout = _bf16_bits(q=q, k=k, v=v, dout=dout)
        r = _routes64(routes)
        B, S_q, Hq, D = q.shape
        _, S_kv, Hkv, _ = k.shape
        if Hkv < 1 or Hq % Hkv != 0:
            raise ValueError("Hq must be a positive multiple of Hkv")
        if dout.shape != q.shape:
            raise ValueError("dout must have the shape of q")
        r0, r1 = (0, S_q) if rows is None else (int(rows[0]), int(rows[1]))
        k0, k1 = (0, S_kv) if keys is None else (int(keys[0]), int(keys[1]))
        dq = np.empty((B, r1 - r0, Hq, D), dtype=np.float64)
        dk = np.empty((B, k1 - k0, Hkv, D), dtype=np.float64)
        dv = np.empty((B, k1 - k0, Hkv, D), dtype=np.float64)
        self.lib.oracle_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(r), B, S_q, S_kv, Hq, Hkv, D,
                                 r.shape[2], float(scale), r0, r1, k0, k1, _ptr(dq), _ptr(dk), _ptr(dv))
        return dq, dk, dv


    def select_token_ids(self, iq, ck, seq_lens, token_budget, compress_ratio, q_offset=0, rows=None):
        iq, ck = _bf16_bits(iq=iq, ck=ck)
        lens = np.ascontiguousarray(seq_lens, dtype=np.int64)
        B, S_q, H, D = iq.shape
        if ck.ndim == 4:  # [B, n_blocks, 1, D]
            ck = np.ascontiguousarray(ck[:, :, 0, :])
        n_blocks = ck.shape[1]
        c, budget, q_offset = int(compress_ratio), int(token_budget), int(q_offset)
        if ck.shape[0] != B or ck.shape[2] != D or lens.shape != (B,):
            raise ValueError("shape mismatch among index queries, block keys and lengths")
        if c < 1 or budget < 1 or q_offset < 0:
            raise ValueError("compress_ratio and token_budget must be >= 1, q_offset >= 0")
        if (q_offset + S_q) // c > n_blocks:
            raise ValueError("fewer block keys than the last query row can see")
        r0, r1 = (0, S_q) if rows is None else (int(rows[0]), int(rows[1]))
        out = np.empty((B, r1 - r0, budget + c - 1), dtype=np.int32)
        self.lib.oracle_select_token_ids(_ptr(iq), _ptr(ck), _ptr(lens), B, S_q, H, D, n_blocks, q_offset,
                                         budget, c, r0, r1, _ptr(out))
        return out

    def block_scores(self, iq, ck, rows=None):
        iq, ck = _bf16_bits(iq=iq, ck=ck)
        if ck.ndim == 4:
            ck = np.ascontiguousarray(ck[:, :, 0, :])
        B, S_q, H, D = iq.shape
        n_blocks = ck.shape[1]
        r0, r1 = (0, S_q) if rows is None else (int(rows[0]), int(rows[1]))
        out = np.empty((B, r1 - r0, n_blocks), dtype=np.float64)
        self.lib.oracle_block_scores(_ptr(iq), _ptr(ck), B, S_q, H, D, n_blocks, r0, r1, _ptr(out))
        return out


def _bf16_bits(**tensors):
    out = []
    for name, t in tensors.items():
        if t.dtype != np.uint16:
            raise TypeError(f"{name} must hold bfloat16 bits as uint16")
        out.append(np.ascontiguousarray(t))
    return out


def _load() -> Oracle:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _lib = Oracle(_LIB_PATH)
    return _lib


def num_threads() -> int:
    return _load().num_threads()


def _routes64(routes: np.ndarray) -> np.ndarray:
    r = np.asarray(routes)
    if r.dtype not in (np.int32, np.int64):
        raise TypeError("routes must be int32 or int64")
    return np.ascontiguousarray(r.astype(np.int64))  # int32 -> int64 sign-extends


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def ldm_of(kv_length: int) -> int:
    return (int(kv_length) + TILE - 1) // TILE * TILE


def route_lists(routes: np.ndarray, kv_length: int):
    return _load().route_lists(routes, kv_length)


def membership(routes: np.ndarray, kv_length: int) -> np.ndarray:
    return _load().membership(routes, kv_length)


def tile_class(routes: np.ndarray, kv_length: int) -> np.ndarray:
    return _load().tile_class(routes, kv_length)


def forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, routes: np.ndarray, scale: float,
            rows: tuple[int, int] | None = None) -> np.ndarray:
    """fp64 attention output [B, rows, Hq, D] for query rows ``rows`` (default: all)."""
    return _load().forward(q, k, v, routes, scale, rows)


def lse(q: np.ndarray, k: np.ndarray, routes: np.ndarray, scale: float,
        rows: tuple[int, int] | None = None) -> np.ndarray:
    """fp64 natural-log log-sum-exp of the scaled scores, [B, rows, Hq]; -inf for empty rows."""
    return _load().lse(q, k, routes, scale, rows)


def backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray, routes: np.ndarray, scale: float,
             rows: tuple[int, int] | None = None, keys: tuple[int, int] | None = None):
    """fp64 (dq [B,rows,Hq,D], dk [B,keys,Hkv,D], dv [B,keys,Hkv,D]) for upstream gradient ``dout``."""
    return _load().backward(q, k, v, dout, routes, scale, rows, keys)


def tile_lists(kinds: np.ndarray) -> dict:
    """Forward and reverse partial/full block lists of a tile-class table [B, R, C]."""
    return _load().tile_lists(kinds)


def select_token_ids(iq: np.ndarray, ck: np.ndarray, seq_lens: np.ndarray, token_budget: int, compress_ratio: int,
                     q_offset: int = 0, rows: tuple[int, int] | None = None) -> np.ndarray:
    """Selected token IDs int32 [B, rows, token_budget + compress_ratio - 1] (-1 = empty slot)."""
    return _load().select_token_ids(iq, ck, seq_lens, token_budget, compress_ratio, q_offset, rows)


def block_scores(iq: np.ndarray, ck: np.ndarray, rows: tuple[int, int] | None = None) -> np.ndarray:
    """fp64 block scores sum_h relu(<iq[b,i,h], ck[b,j]>) / sqrt(D), [B, rows, n_blocks]."""
    return _load().block_scores(iq, ck, rows)
