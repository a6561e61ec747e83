"""Seeded generators for the five route-sparse GQA workloads.

Every workload is fully determined by its name: ``SeedSequence(1000 + n)``
(``n`` = 1..5 in the order below) is split with ``spawn(4)`` into separate
PCG64 streams for Q, K, V and the routes.  Q/K/V are drawn as float32
N(0, 1) and rounded to bfloat16 (round-to-nearest-even) on the host and
kept as ``uint16`` bit patterns, so every consumer sees identical bits.

Route recipes (one per workload; see each ``_routes_*`` function):

* ``tiny``          - 32 uniform draws with replacement from the causal range
                       ``[0, q]``; 26 of the 256 rows (10 %) are all ``-1``.
* ``right_padded``  - logical lengths 4096 and 3000; own causal 64-token block
                       plus up to 7 distinct earlier blocks; tokens past the
                       query are ``-1``; pad rows all ``-1``.
* ``packed_thd``    - lognormal document lengths (median 1500) packed into
                       one 16384-token row with tail padding; 16 distinct
                       document-relative 64-token blocks per query, clipped to
                       the query; then 51 duplicate and 20 invalid slots per
                       row (``-1``, ``S_kv + U[0, 1000)``, ``2**40``) and a
                       per-row shuffle.
* ``cp_slice``      - 8192 local queries at global offset 24576 against 32768
                       keys; own causal block plus 31 distinct earlier blocks.
* ``long_int64``    - 65536 x 65536; own block, block 0 and 30 distinct blocks
                       from ``[1, j)``.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

BLOCK = 64  # tokens per route block in every block-structured recipe


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    number: int  # 1-based, fixes the seed
    B: int
    S_q: int
    S_kv: int
    Hq: int
    Hkv: int
    D: int
    K: int
    q_offset: int = 0  # global position of local query row 0
    description: str = ""

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def seed(self) -> int:
        return 1000 + self.number


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny", 1, B=1, S_q=256, S_kv=256, Hq=4, Hkv=1, D=64, K=32,
                 description="B=1 S=256 Hq=4 Hkv=1 D=64 K=32, causal uniform draws, 10% empty rows"),
        Workload("right_padded", 2, B=2, S_q=4096, S_kv=4096, Hq=16, Hkv=2, D=256, K=512,
                 description="B=2 S=4096 Hq=16 Hkv=2 D=256 K=512, lengths 4096/3000, 8 causal 64-token blocks"),
        Workload("packed_thd", 3, B=1, S_q=16384, S_kv=16384, Hq=16, Hkv=2, D=256, K=1024,
                 description="B=1 T=16384 lognormal documents (median 1500), K=1024, 5% duplicates, 2% invalid"),
        Workload("cp_slice", 4, B=1, S_q=8192, S_kv=32768, Hq=16, Hkv=2, D=256, K=2048, q_offset=24576,
                 description="B=1 S_q=8192 at offset 24576, S_kv=32768, K=2048, 32 causal 64-token blocks"),
        Workload("long_int64", 5, B=1, S_q=65536, S_kv=65536, Hq=16, Hkv=2, D=256, K=2048,
                 description="B=1 S=65536 (B*S_q*S_kv > 2^31), K=2048, own + first + 30 uniform blocks"),
    ]
}


# --------------------------------------------------------------------------
# bfloat16 bit handling (input preparation only)
# --------------------------------------------------------------------------

def float32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16, nearest-even; returns uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_float32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _streams(w: Workload):
    children = np.random.SeedSequence(w.seed).spawn(4)
    return [np.random.Generator(np.random.PCG64(c)) for c in children]


def _normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    out = np.empty(shape, dtype=np.uint16)
    flat = out.reshape(-1)
    step = 1 << 24  # bounded float32 temporaries
    for s in range(0, flat.size, step):
        n = min(step, flat.size - s)
        flat[s:s + n] = float32_to_bf16_bits(rng.standard_normal(n, dtype=np.float32))
    return out


def make_qkv(w: Workload):
    """Q [B,S_q,Hq,D], K and V [B,S_kv,Hkv,D] as uint16 bfloat16 bits."""
    rq, rk, rv, _ = _streams(w)
    q = _normal_bf16(rq, (w.B, w.S_q, w.Hq, w.D))
    k = _normal_bf16(rk, (w.B, w.S_kv, w.Hkv, w.D))
    v = _normal_bf16(rv, (w.B, w.S_kv, w.Hkv, w.D))
    return q, k, v


def make_dout(w: Workload) -> np.ndarray:
    """Upstream gradient [B,S_q,Hq,D] for the backward: bfloat16 N(0,1) bits from a fifth stream."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(w.seed, spawn_key=(4,))))
    return _normal_bf16(rng, (w.B, w.S_q, w.Hq, w.D))


def random_dout(seed: int, shape) -> np.ndarray:
    """bfloat16 N(0,1) bits of the given shape (upstream gradients of the small cases)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return float32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def random_windowed_routes(seed: int, B: int, S_q: int, S_kv: int, K: int, p_invalid: float = 0.1,
                           p_empty: float = 0.05) -> np.ndarray:
    """int64 routes [B,S_q,K] whose valid IDs lie in one window per row: the window's width is drawn
    log-uniformly from [1, S_kv] and its start uniformly, so rows range from a few neighbouring keys
    to the whole key range; then invalid slots (-1, S_kv, 2**40), and a fraction of empty rows.
    Repeats come from drawing with replacement."""
    rng = np.random.Generator(np.random.PCG64(seed))
    width = np.exp(rng.uniform(0.0, np.log(S_kv), size=(B, S_q))).astype(np.int64).clip(1, S_kv)
    start = (rng.random((B, S_q)) * (S_kv - width + 1)).astype(np.int64)
    routes = start[:, :, None] + (rng.random((B, S_q, K)) * width[:, :, None]).astype(np.int64)
    bad = rng.random((B, S_q, K)) < p_invalid
    pool = np.array([-1, S_kv, 1 << 40], dtype=np.int64)
    routes[bad] = pool[rng.integers(0, pool.size, size=int(bad.sum()))]
    routes[rng.random((B, S_q)) < p_empty] = -1
    return routes


# --------------------------------------------------------------------------
# route recipes
# --------------------------------------------------------------------------

def _sample_distinct(rng: np.random.Generator, rows: int, pool: int, take: int) -> np.ndarray:
    """``rows`` independent uniform samples of ``take`` distinct values from [0, pool)."""
    if take <= 0:
        return np.zeros((rows, 0), dtype=np.int64)
    keys = rng.random((rows, pool))
    if take < pool:
        idx = np.argpartition(keys, take - 1, axis=1)[:, :take]
    else:
        idx = np.argsort(keys, axis=1)
    return idx.astype(np.int64)


def _expand_blocks(blocks: np.ndarray, positions: np.ndarray, first_token: np.ndarray | int = 0) -> np.ndarray:
    """Blocks [rows, nb] (entries < 0 unused) -> token IDs [rows, nb*64], clipped to ``<= position``."""
    rows, nb = blocks.shape
    tok = first_token + blocks[:, :, None] * BLOCK + np.arange(BLOCK, dtype=np.int64)[None, None, :]
    bad = (blocks[:, :, None] < 0) | (tok > positions[:, None, None])
    tok = np.where(bad, -1, tok)
    return tok.reshape(rows, nb * BLOCK)


def _routes_tiny(w: Workload, rng: np.random.Generator) -> np.ndarray:
    q = np.arange(w.S_q, dtype=np.int64)
    routes = rng.integers(0, q[:, None] + 1, size=(w.S_q, w.K), dtype=np.int64)
    empty = rng.choice(w.S_q, size=int(round(0.10 * w.S_q)), replace=False)
    routes[empty] = -1
    return routes[None]


def _routes_right_padded(w: Workload, rng: np.random.Generator) -> np.ndarray:
    lengths = [4096, 3000]
    nb = w.K // BLOCK  # 8 blocks
    routes = np.full((w.B, w.S_q, w.K), -1, dtype=np.int64)
    for b in range(w.B):
        L = lengths[b]
        for j in range((L + BLOCK - 1) // BLOCK):
            q = np.arange(j * BLOCK, min((j + 1) * BLOCK, L), dtype=np.int64)
            blocks = np.full((q.size, nb), -1, dtype=np.int64)
            blocks[:, 0] = j
            take = min(nb - 1, j)
            blocks[:, 1:1 + take] = _sample_distinct(rng, q.size, j, take)
            routes[b, q] = _expand_blocks(blocks, q)
    return routes


def _packed_documents(rng: np.random.Generator, total: int):
    """Lognormal (median 1500, sigma 1) lengths, at least 64, appended while they fit."""
    starts, lengths, pos = [], [], 0
    while True:
        L = max(BLOCK, int(round(rng.lognormal(math.log(1500.0), 1.0))))
        if pos + L > total:
            break
        starts.append(pos)
        lengths.append(L)
        pos += L
    return starts, lengths


def _routes_packed_thd(w: Workload, rng: np.random.Generator) -> np.ndarray:
    nb = w.K // BLOCK  # 16 blocks
    routes = np.full((1, w.S_q, w.K), -1, dtype=np.int64)
    starts, lengths = _packed_documents(rng, w.S_q)
    for d0, L in zip(starts, lengths):
        for j in range((L + BLOCK - 1) // BLOCK):
            p = np.arange(j * BLOCK, min((j + 1) * BLOCK, L), dtype=np.int64)  # document-relative
            pool = j + 1  # blocks whose start is <= p
            take = min(nb, pool)
            blocks = np.full((p.size, nb), -1, dtype=np.int64)
            blocks[:, :take] = _sample_distinct(rng, p.size, pool, take)
            routes[0, d0 + p] = _expand_blocks(blocks, d0 + p, first_token=d0)
    # corruption: 5% duplicate slots, 2% invalid slots, then a per-row shuffle
    n_dup = int(0.05 * w.K)  # 51
    n_bad = int(0.02 * w.K)  # 20
    doc_rows = np.concatenate([np.arange(d0, d0 + L) for d0, L in zip(starts, lengths)])
    r = routes[0]
    for row in doc_rows:
        orig = r[row].copy()
        valid = orig[orig >= 0]
        pick = rng.permutation(w.K)[: n_dup + n_bad]
        r[row, pick[:n_dup]] = valid[rng.integers(0, valid.size, size=n_dup)]
        bad = np.empty(n_bad, dtype=np.int64)
        for t in range(n_bad):
            kind = t % 3
            bad[t] = -1 if kind == 0 else (w.S_kv + int(rng.integers(0, 1000)) if kind == 1 else 1 << 40)
        r[row, pick[n_dup:]] = bad
        r[row] = r[row, rng.permutation(w.K)]
    return routes


def _routes_cp_slice(w: Workload, rng: np.random.Generator) -> np.ndarray:
    nb = w.K // BLOCK  # 32 blocks
    routes = np.empty((1, w.S_q, w.K), dtype=np.int64)
    p_all = w.q_offset + np.arange(w.S_q, dtype=np.int64)
    for j in np.unique(p_all // BLOCK):
        sel = np.nonzero(p_all // BLOCK == j)[0]
        p = p_all[sel]
        blocks = np.empty((sel.size, nb), dtype=np.int64)
        blocks[:, 0] = j
        blocks[:, 1:] = _sample_distinct(rng, sel.size, int(j), nb - 1)
        routes[0, sel] = _expand_blocks(blocks, p)
    return routes


def _routes_long_int64(w: Workload, rng: np.random.Generator) -> np.ndarray:
    nb = w.K // BLOCK  # 32 blocks
    routes = np.empty((1, w.S_q, w.K), dtype=np.int64)
    for j in range(w.S_q // BLOCK):
        q = np.arange(j * BLOCK, (j + 1) * BLOCK, dtype=np.int64)
        blocks = np.full((q.size, nb), -1, dtype=np.int64)
        blocks[:, 0] = j
        if j >= 1:
            blocks[:, 1] = 0
            take = min(nb - 2, j - 1)
            blocks[:, 2:2 + take] = 1 + _sample_distinct(rng, q.size, j - 1, take)
        routes[0, q] = _expand_blocks(blocks, q)
    return routes


_ROUTE_RECIPES = {
    "tiny": _routes_tiny,
    "right_padded": _routes_right_padded,
    "packed_thd": _routes_packed_thd,
    "cp_slice": _routes_cp_slice,
    "long_int64": _routes_long_int64,
}


def make_routes(w: Workload, dtype=np.int64) -> np.ndarray:
    """Route IDs [B, S_q, K] for workload ``w`` (int64; int32 gives the same values)."""
    _, _, _, rr = _streams(w)
    routes = _ROUTE_RECIPES[w.name](w, rr)
    assert routes.shape == (w.B, w.S_q, w.K)
    if np.dtype(dtype) == np.int32:
        if routes.max() > np.iinfo(np.int32).max or routes.min() < np.iinfo(np.int32).min:
            raise ValueError(f"{w.name}: route values do not fit int32")
        return routes.astype(np.int32)
    return routes


def make_inputs(name: str, route_dtype=np.int64, with_qkv: bool = True):
    """Return ``(workload, q, k, v, routes)``; q/k/v are None when ``with_qkv`` is False."""
    w = WORKLOADS[name]
    routes = make_routes(w, route_dtype)
    if not with_qkv:
        return w, None, None, None, routes
    q, k, v = make_qkv(w)
    return w, q, k, v, routes


def random_small_case(seed: int, B: int, S_q: int, S_kv: int, Hq: int, Hkv: int, D: int, K: int,
                      p_invalid: float = 0.2, p_empty: float = 0.1, route_dtype=np.int64,
                      extreme: bool = True, q_zero: Optional[bool] = False):
    """Small random case for parity tests: uniform IDs with invalid/duplicate/empty rows mixed in.

    Invalid slots draw from -1, other negatives, ``S_kv`` itself, values past it and,
    for int64, ``2**40`` and the int64 extremes.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    q = float32_to_bf16_bits(rng.standard_normal((B, S_q, Hq, D), dtype=np.float32))
    if q_zero:
        q[:] = 0
    k = float32_to_bf16_bits(rng.standard_normal((B, S_kv, Hkv, D), dtype=np.float32))
    v = float32_to_bf16_bits(rng.standard_normal((B, S_kv, Hkv, D), dtype=np.float32))
    routes = rng.integers(0, S_kv, size=(B, S_q, K), dtype=np.int64)
    bad_pool = [-1, -2, -(1 << 20), S_kv, S_kv + 1, S_kv + 12345]
    if np.dtype(route_dtype) == np.int64 and extreme:
        bad_pool += [1 << 40, np.iinfo(np.int64).max, np.iinfo(np.int64).min, (1 << 32) + 3]
    elif np.dtype(route_dtype) == np.int32 and extreme:
        bad_pool += [np.iinfo(np.int32).max, np.iinfo(np.int32).min]
    bad = rng.random((B, S_q, K)) < p_invalid
    routes[bad] = np.array(bad_pool, dtype=np.int64)[rng.integers(0, len(bad_pool), size=int(bad.sum()))]
    empty = rng.random((B, S_q)) < p_empty
    routes[empty] = -1
    return q, k, v, routes.astype(route_dtype)


# --------------------------------------------------------------------------
# route-selection inputs: index queries and compressed block keys
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class SelectWorkload:
    """Shapes of one route-selection case (index heads H, index head dim D)."""

    name: str
    number: int  # 1-based, fixes the seed
    B: int
    S_q: int
    S_global: int
    H: int
    D: int
    compress_ratio: int
    token_budget: int
    lengths: tuple
    q_offset: int = 0
    description: str = ""

    @property
    def n_blocks(self) -> int:
        return self.S_global // self.compress_ratio

    @property
    def width(self) -> int:
        return self.token_budget + self.compress_ratio - 1

    @property
    def seed(self) -> int:
        return 2000 + self.number


SELECT_WORKLOADS = {
    w.name: w
    for w in [
        SelectWorkload("sel_tiny", 1, B=2, S_q=256, S_global=256, H=4, D=64, compress_ratio=4, token_budget=32,
                       lengths=(256, 197), description="B=2 S=256 H=4 D=64 c=4 budget=32, lengths 256/197"),
        SelectWorkload("sel_right_padded", 2, B=2, S_q=4096, S_global=4096, H=16, D=128, compress_ratio=4,
                       token_budget=512, lengths=(4096, 3000),
                       description="B=2 S=4096 H=16 D=128 c=4 budget=512, lengths 4096/3000"),
        SelectWorkload("sel_cp_slice", 3, B=1, S_q=8192, S_global=32768, H=16, D=128, compress_ratio=4,
                       token_budget=2048, lengths=(32768,), q_offset=24576,
                       description="B=1 S_q=8192 at offset 24576 of 32768, H=16 D=128 c=4 budget=2048"),
        SelectWorkload("sel_long", 4, B=1, S_q=65536, S_global=65536, H=16, D=128, compress_ratio=4,
                       token_budget=2048, lengths=(65536,),
                       description="B=1 S=65536 H=16 D=128 c=4 budget=2048 (16384 blocks)"),
    ]
}


def _unit_rms_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) vectors along the last axis scaled to unit RMS in float32, rounded to bfloat16 bits."""
    out = np.empty(shape, dtype=np.uint16)
    D = shape[-1]
    flat = out.reshape(-1, D)
    step = max(1, (1 << 22) // D)
    for s in range(0, flat.shape[0], step):
        n = min(step, flat.shape[0] - s)
        x = rng.standard_normal((n, D), dtype=np.float32)
        x /= np.sqrt(np.mean(x * x, axis=1, keepdims=True, dtype=np.float32))
        flat[s:s + n] = float32_to_bf16_bits(x)
    return out


def make_select_inputs(name: str):
    """Return ``(workload, iq [B,S_q,H,D], ck [B,n_blocks,1,D], seq_lens int64 [B])``.

    Index queries and block keys are unit-RMS random vectors (the pages feed
    RMS-normalised, rotated projections; their weights are not available, so
    random directions stand in), as bfloat16 bits.
    """
    w = SELECT_WORKLOADS[name]
    rq, rk = [np.random.Generator(np.random.PCG64(c)) for c in np.random.SeedSequence(w.seed).spawn(2)]
    iq = _unit_rms_bf16(rq, (w.B, w.S_q, w.H, w.D))
    ck = _unit_rms_bf16(rk, (w.B, w.n_blocks, 1, w.D))
    return w, iq, ck, np.array(w.lengths, dtype=np.int64)


def random_select_case(seed: int, B: int, S_q: int, H: int, D: int, n_blocks: int, integer: bool = False):
    """Index queries [B,S_q,H,D] and block keys [B,n_blocks,1,D] as bfloat16 bits.

    ``integer=True`` draws small integers in [-3, 3]: every product and sum is
    then exact in float32, and equal scores (ties) are frequent.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    if integer:
        iq = rng.integers(-3, 4, size=(B, S_q, H, D)).astype(np.float32)
        ck = rng.integers(-3, 4, size=(B, n_blocks, 1, D)).astype(np.float32)
    else:
        iq = rng.standard_normal((B, S_q, H, D), dtype=np.float32)
        ck = rng.standard_normal((B, n_blocks, 1, D), dtype=np.float32)
    return float32_to_bf16_bits(iq), float32_to_bf16_bits(ck)
