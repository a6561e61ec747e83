"""Independent reference computations that pin the CPU oracle.

Nothing here calls the oracle or the HIP library.  Each function restates a
definition from the route-sparse GQA pages in a different form from the
oracle's per-row gather loop:

* ``brute_route_set``   - Python ``sorted(set(...))`` over plain ints.
* ``brute_membership``  - dense boolean table filled from those sets.
* ``block_classes``     - numpy block reduction of a membership table.
* ``dense_attention``   - dense [S_q, S_kv] fp64 scores, -inf outside the
                          membership table, textbook softmax (also on
                          float64 arrays: ``dense_attention_f64``).
* ``dense_lse``         - per-row log-sum-exp over the dense masked scores.
"""

from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def brute_route_set(row, kv_length: int) -> list[int]:
    """Valid IDs are 0 <= x < kv_length; a repeated ID counts once; ascending."""
    return sorted({int(x) for x in row if 0 <= int(x) < kv_length})


def brute_lists(routes: np.ndarray, kv_length: int):
    B, S_q, K = routes.shape
    lst = np.full((B, S_q, K), -1, dtype=np.int32)
    cnt = np.zeros((B, S_q), dtype=np.int32)
    for b in range(B):
        for i in range(S_q):
            s = brute_route_set(routes[b, i].tolist(), kv_length)
            lst[b, i, : len(s)] = s
            cnt[b, i] = len(s)
    return lst, cnt


def brute_membership(routes: np.ndarray, kv_length: int, ldm: int | None = None) -> np.ndarray:
    B, S_q, _ = routes.shape
    ldm = kv_length if ldm is None else ldm
    m = np.zeros((B, S_q, ldm), dtype=np.uint8)
    for b in range(B):
        for i in range(S_q):
            for x in brute_route_set(routes[b, i].tolist(), kv_length):
                m[b, i, x] = 1
    return m


def block_classes(member: np.ndarray, kv_length: int, tile: int = 128) -> np.ndarray:
    """Tile classes by reducing a [B, S_q, >=kv_length] 0/1 table over tile x tile blocks."""
    B, S_q, _ = member.shape
    n_ti, n_tj = -(-S_q // tile), -(-kv_length // tile)
    m = np.zeros((B, n_ti * tile, n_tj * tile), dtype=np.int64)
    m[:, :S_q, :kv_length] = member[:, :, :kv_length]
    inrange = np.zeros_like(m)
    inrange[:, :S_q, :kv_length] = 1
    sums = m.reshape(B, n_ti, tile, n_tj, tile).sum(axis=(2, 4))
    size = inrange.reshape(B, n_ti, tile, n_tj, tile).sum(axis=(2, 4))
    return np.where(sums == 0, 0, np.where(sums == size, 2, 1)).astype(np.int32)


def dense_attention_f64(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray, scale: float) -> np.ndarray:
    """Dense masked-softmax attention on float64 arrays; ``mask`` [B,S_q,S_kv] bool; empty rows give zeros."""
    B, S_q, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    out = np.zeros((B, S_q, Hq, D), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            kk, vv = k[b, :, h // G, :], v[b, :, h // G, :]
            s = scale * (q[b, :, h, :] @ kk.T)  # [S_q, S_kv]
            s = np.where(mask[b], s, -np.inf)
            has = mask[b].any(axis=1)
            mx = np.where(has, s.max(axis=1), 0.0)
            w = np.where(mask[b], np.exp(s - mx[:, None]), 0.0)
            den = w.sum(axis=1)
            o = (w @ vv) / np.where(has, den, 1.0)[:, None]
            out[b, :, h, :] = np.where(has[:, None], o, 0.0)
    return out


def dense_attention(q_bits, k_bits, v_bits, routes, scale: float) -> np.ndarray:
    """Dense masked-softmax attention in fp64 on bfloat16 bit inputs; empty rows give zeros."""
    S_kv = k_bits.shape[1]
    mask = brute_membership(routes, S_kv).astype(bool)
    return dense_attention_f64(bf16_to_f64(q_bits), bf16_to_f64(k_bits), bf16_to_f64(v_bits), mask, scale)


def dense_lse(q_bits, k_bits, routes, scale: float) -> np.ndarray:
    """log sum_j exp(s_j) over the membership table, [B,S_q,Hq]; -inf for empty rows."""
    q, k = bf16_to_f64(q_bits), bf16_to_f64(k_bits)
    B, S_q, Hq, D = q.shape
    S_kv, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    mask = brute_membership(routes, S_kv).astype(bool)
    out = np.full((B, S_q, Hq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            s = scale * (q[b, :, h, :] @ k[b, :, h // G, :].T)
            for i in range(S_q):
                if mask[b, i].any():
                    x = s[i][mask[b, i]]
                    mx = x.max()
                    out[b, i, h] = mx + np.log(np.exp(x - mx).sum())
    return out
