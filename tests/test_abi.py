"""The C ABI library loads, exports every entry point its header declares and
rejects bad arguments on the host (CPU only: no call here reaches a launch)."""

from __future__ import annotations

import ctypes
import os
import re

import pytest

import route_sparse_gqa_amd as qsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsa.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|int|size_t)\s*\*?\s*(qsa_\w+)\s*\(", text, flags=re.M)))


def _declared_constants():
    text = open(HEADER).read()
    return {m[0]: int(m[1]) for m in re.findall(r"#define\s+(QSA_\w+)\s+(-?\d+)", text)}


def test_header_declares_the_entry_points():
    assert _declared_functions() == sorted([
        "qsa_preprocess", "qsa_forward", "qsa_forward_preprocessed", "qsa_forward_workspace_size",
        "qsa_attention_workspace_size", "qsa_forward_noalloc",
        "qsa_backward", "qsa_backward_workspace_size", "qsa_tile_lists", "qsa_status_string",
        "qsa_select_token_ids", "qsa_select_workspace_size", "qsa_select_chunk_workspace_size"])


def test_library_exports_every_declared_symbol():
    L = qsa.lib()
    for name in _declared_functions():
        assert hasattr(L, name), f"libqsa.so does not export {name}"


def test_python_constants_match_header():
    c = _declared_constants()
    assert c["QSA_INT32"] == qsa.QSA_INT32 and c["QSA_INT64"] == qsa.QSA_INT64
    assert c["QSA_TILE"] == qsa.TILE and c["QSA_MAX_ROUTES"] == qsa.MAX_ROUTES
    assert c["QSA_MAX_GROUP"] == qsa.MAX_GROUP and c["QSA_ERR_HIP"] == qsa._HIP_ERROR
    text = open(HEADER).read()
    assert re.search(r"#define\s+QSA_NOALLOC_SCRATCH_BYTES\s+\(64u << 20\)", text)
    assert qsa.NOALLOC_SCRATCH_BYTES == 64 << 20


def test_status_strings():
    codes = [v for k, v in _declared_constants().items() if k.startswith("QSA_ERR_") or k == "QSA_OK"]
    texts = [qsa.qsa_status_string(c) for c in codes]
    assert len(set(texts)) == len(codes) and "unknown status" not in texts
    assert qsa.qsa_status_string(12345) == "unknown status"


def test_workspace_size():
    ws, att = qsa.qsa_forward_workspace_size, qsa.qsa_attention_workspace_size
    # key ranges within one XCD's L2 (S_kv * 4 * D <= 4 MiB): lists and counts only
    assert att(2, 4096, 4096, 16, 2, 256, 512) == 0
    assert ws(2, 4096, 4096, 16, 2, 256, 512) == 4 * 2 * 4096 * 512 + 4 * 2 * 4096
    assert ws(1, 3, 9, 2, 1, 64, 5) == 256 + 256  # lists and counts each rounded to 256 bytes
    assert att(1, 10, 65536, 4, 1, 64, 8) == 0     # 65536 * 4 * 64 = 16 MiB: four ranges, no split
    assert att(1, 16384, 16384, 16, 2, 256, 1024) == 0
    for bad in ((0, 10, 9, 2, 1, 64, 10), (1, 1, 9, 2, 1, 64, 0), (1, 1, 9, 2, 1, 96, 4), (1, 1, 9, 3, 2, 64, 4)):
        assert ws(*bad) == 0 and att(*bad) == 0
    assert ws(1 << 40, 1 << 40, 9, 2, 1, 64, 1) == 0  # overflow


def _split_bytes(rows, S_kv, Hq, D, pass_rows):
    """The layout of the attention workspace as include/qsa.h documents it."""
    r256 = lambda x: -(-x // 256) * 256
    W = 1
    while 2 * W * 4 * D <= 4 << 20:
        W *= 2
    while -(-S_kv // W) > 63:
        W *= 2
    P = -(-S_kv // W)
    buffers = 2 if pass_rows < rows else 1  # a pass's partials are merged while the next pass fills the other
    return P, r256(4 * rows * (P + 1)) + buffers * (r256(2 * pass_rows * Hq * P * D) + r256(4 * pass_rows * Hq * P))


def test_attention_workspace_size():
    att, fwd = qsa.qsa_attention_workspace_size, qsa.qsa_forward_workspace_size
    cases = [  # (B, S_q, S_kv, Hq, Hkv, D, K): expected ranges
        ((1, 65536, 65536, 16, 2, 256, 2048), 16),   # W = 4096
        ((1, 8192, 32768, 16, 2, 256, 2048), 8),
        ((2, 100, 16385, 4, 1, 256, 64), 5),         # one key past four ranges
        ((1, 50, 40000, 8, 2, 128, 300), 5),         # W = 8192
        ((1, 30, 90000, 4, 2, 64, 300), 6),          # W = 16384
        ((1, 10, 1 << 31, 4, 2, 256, 64), 32),       # W doubled until at most 63 ranges: 2^26
    ]
    for (B, S_q, S_kv, Hq, Hkv, D, K), P in cases:
        rows = B * S_q
        got_P, want = _split_bytes(rows, S_kv, Hq, D, min(rows, 8192))
        assert got_P == P
        assert att(B, S_q, S_kv, Hq, Hkv, D, K) == want, (B, S_q, S_kv)
        lists = -(-4 * rows * K // 256) * 256 + -(-4 * rows // 256) * 256
        assert fwd(B, S_q, S_kv, Hq, Hkv, D, K) == lists + want


def _call_forward(B=1, S_q=4, S_kv=4, Hq=2, Hkv=1, D=64, K=2, scale=0.1, null_routes=False):
    """Every call made with this helper carries one invalid argument (fake pointers never reach a launch)."""
    L = qsa.lib()
    sq = (ctypes.c_int64 * 4)(S_q * Hq * D, Hq * D, D, 1)
    sk = (ctypes.c_int64 * 4)(S_kv * Hkv * D, Hkv * D, D, 1)
    s3 = (ctypes.c_int64 * 3)(S_q * K, K, 1)
    fq, fk, fv, fr, fo, fw = (ctypes.c_void_p(n << 32) for n in range(1, 7))  # distinct, never dereferenced
    return L.qsa_forward(fq, sq, fk, sk, fv, sk, None if null_routes else fr, 1, s3, B, S_q, S_kv, Hq, Hkv,
                         D, K, scale, fo, fw, 1 << 20, None)


@pytest.mark.parametrize("dims", [dict(B=0), dict(S_q=0), dict(S_kv=0), dict(Hq=0), dict(Hkv=0), dict(D=0),
                                  dict(K=0)])
def test_empty_dimensions_rejected_before_anything_runs(dims):
    assert _call_forward(**dims) == -2


def test_other_host_checks():
    assert _call_forward(Hq=3, Hkv=2) == -4
    assert _call_forward(D=96) == -5
    assert _call_forward(Hq=64, Hkv=2) == -11
    assert _call_forward(K=20000) == -11
    assert _call_forward(S_kv=(1 << 31) + 1) == -3
    assert _call_forward(null_routes=True) == -1
    L = qsa.lib()
    s3 = (ctypes.c_int64 * 3)(1, 1, 1)
    fake = ctypes.c_void_p(1 << 20)
    assert L.qsa_preprocess(fake, 1, 1, 2, 0, s3, 5, fake, fake, None, None, None) == -2
    assert L.qsa_preprocess(fake, 1, 1, 2, 3, s3, 0, fake, fake, None, None, None) == -3
    assert L.qsa_preprocess(fake, 9, 1, 2, 3, s3, 5, fake, fake, None, None, None) == -6
    assert L.qsa_preprocess(None, 1, 1, 2, 3, s3, 5, fake, fake, None, None, None) == -1
    # membership grid: 2048 tile rows x 32768 segments (kv_length 2^31) x 32 row groups = 2^31 workgroups
    S_q, kv = 2048 * 128, 1 << 31
    s_rows = (ctypes.c_int64 * 3)(S_q, 1, 1)
    low = [ctypes.c_void_p(n << 32) for n in (1, 2, 3)]  # routes, list, count; the table lies above them
    assert L.qsa_preprocess(low[0], 1, 1, S_q, 1, s_rows, kv, low[1], low[2], ctypes.c_void_p(4 << 32), None,
                            None) == -11


def test_launches_beyond_one_grid_are_refused():
    """One launch holds fewer than 2^32 work-items per grid dimension; calls whose grids would not fit return
    QSA_ERR_LIMIT before anything runs (fake pointers never reach a launch)."""
    L = qsa.lib()
    fake = [ctypes.c_void_p(n << 32) for n in range(1, 4)]
    s3 = (ctypes.c_int64 * 3)(1, 1, 1)
    # 2^24 rows: route normalisation's bitmap path runs one 256-thread workgroup per row
    assert L.qsa_preprocess(fake[0], 1, 1, 1 << 24, 1, s3, 5, fake[1], fake[2], None, None, None) == -11
    # K = 8193 over 2^20 keys sorts each row with 16 wavefronts (1024 work-items): 2^22 rows do not fit
    sk = (ctypes.c_int64 * 3)((1 << 22) * 8193, 8193, 1)
    assert L.qsa_preprocess(fake[0], 1, 1, 1 << 22, 8193, sk, 1 << 20, fake[1], fake[2], None, None, None) == -11
    assert _call_forward(S_q=1 << 24) == -11
    assert _call_forward(S_q=1 << 22, K=8193, S_kv=1 << 20) == -11
    assert _call_forward(S_q=1 << 22, Hq=16, Hkv=16) == -11          # rows * Hkv = 2^26 wavefronts = 2^32 work-items
    assert _call_backward(S_q=1 << 22, Hq=16, Hkv=16) == -11
    # a top-k row that sees more than 16384 blocks takes a 1024-thread workgroup: at most 2^22 - 1 rows
    assert _call_select(S_q=1 << 22, S_global=1 << 22, c=64, budget=64) == -11


def _bwd_ws(B, S_q, S_kv, Hq, Hkv, D, K):
    """The layout the header documents, from its formula."""
    r = lambda x: -(-x // 256) * 256
    T, n_w, n_c = -(-S_kv // 64), -(-S_q // 32), -(-S_q // 256)
    cap = B * S_q * min(K, T)
    P = max(1, 4096 // Hkv)
    slots = 2 * min(P, -(-cap // 64))
    total = (r(4 * B * S_q * Hq) + r(4 * B * n_w * T) + r(4 * B * n_c * T) + r(4 * B * T) + r(4 * (B * T + 1)) +
             r(16 * cap) + r(4 * (B * T + 1)) + r(4 * B * T) + r(8) + r(512 * D * Hkv * slots))
    Pr, _ = _split_bytes(B * S_q, S_kv, Hq, D, 0)
    if Pr >= 5:  # dq's key-range split: range starts, then fp32 partial sums of passes of up to 4096 rows,
        R = min(B * S_q, 4096)  # in two buffers when there is more than one pass
        total += r(4 * B * S_q * (Pr + 1)) + (2 if R < B * S_q else 1) * r(4 * R * Hq * Pr * D)
    return total


def test_backward_workspace_size():
    ws = qsa.qsa_backward_workspace_size
    for args in [(2, 4096, 4096, 16, 2, 256, 512), (1, 10, 17, 2, 1, 64, 100), (1, 65536, 65536, 16, 2, 256, 2048),
                 (3, 257, 513, 8, 1, 128, 129)]:
        assert ws(*args) == _bwd_ws(*args), args
    assert ws(1, 65536, 65536, 16, 2, 256, 2048) < 6 << 30  # long sequences fit in a few GiB
    assert ws(1, 8192, 32768, 16, 2, 256, 2048) > ws(1, 8192, 16384, 16, 2, 256, 2048) + (1 << 30)  # split dq
    assert ws(0, 1, 1, 1, 1, 64, 1) == 0 and ws(1, 1, 1, 1, 1, 64, 0) == 0
    assert ws(1, 1 << 21, 1 << 24, 16, 2, 256, 2048) == 0  # more than 2^31 - 1 segments


def _call_backward(B=1, S_q=4, S_kv=32, Hq=2, Hkv=1, D=64, K=2, scale=0.1, ws_bytes=1 << 30, alias_dq_q=False,
                   null_lse=False, k_row_stride=None):
    """Every call made with this helper carries one invalid argument (fake pointers never reach a launch)."""
    L = qsa.lib()
    sq = (ctypes.c_int64 * 4)(S_q * Hq * D, Hq * D, D, 1)
    sk = (ctypes.c_int64 * 4)(S_kv * Hkv * D, Hkv * D if k_row_stride is None else k_row_stride, D, 1)
    f = [ctypes.c_void_p(n << 32) for n in range(1, 14)]  # distinct, never dereferenced
    q, k, v, o, g, lse, lst, cnt, dq, dk, dv, ws = f[:12]
    if alias_dq_q:
        dq = q
    return L.qsa_backward(q, sq, k, sk, v, sk, o, g, sq, None if null_lse else lse, lst, cnt, B, S_q, S_kv, Hq,
                          Hkv, D, K, scale, dq, dk, dv, ws, ws_bytes, None)


def test_backward_host_checks():
    assert _call_backward(S_q=0) == -2
    assert _call_backward(Hq=3, Hkv=2) == -4
    assert _call_backward(D=48) == -5
    assert _call_backward(scale=float("nan")) == -7
    assert _call_backward(null_lse=True) == -1
    assert _call_backward(alias_dq_q=True) == -9
    assert _call_backward(ws_bytes=16) == -10
    assert _call_backward(k_row_stride=1 << 61) == -11    # the key tensor's extent overflows 64 bits
    assert _call_backward(k_row_stride=-(1 << 61)) == -11


def test_tile_lists_host_checks():
    L = qsa.lib()
    f = [ctypes.c_void_p(n << 32) for n in range(1, 10)]  # distinct, never dereferenced
    assert L.qsa_tile_lists(f[0], 0, 2, 2, *f[1:9], None) == -2
    assert L.qsa_tile_lists(None, 1, 2, 2, *f[1:9], None) == -1
    assert L.qsa_tile_lists(f[0], 1, 2, 2, f[1], f[1], *f[3:9], None) == -9  # two outputs alias
    assert L.qsa_tile_lists(f[0], 1, 2, 2, f[0], *f[2:9], None) == -9        # output aliases the input
    assert L.qsa_tile_lists(ctypes.c_void_p((1 << 32) + 2), 1, 2, 2, *f[1:9], None) == -8


def test_select_workspace_size():
    ws = qsa.qsa_select_workspace_size
    # 16-row tiles (H <= 16), rows of round_up(floor((q_offset + S_q) / c), 64) floats
    assert ws(1, 65536, 16, 0, 4) == 65536 * 16384 * 4
    assert ws(2, 4096, 16, 0, 4) == 2 * 4096 * 1024 * 4
    assert ws(1, 8192, 16, 24576, 4) == 8192 * 8192 * 4
    assert ws(1, 20, 16, 0, 4) == 32 * 64 * 4           # 20 rows -> two 16-row tiles, 5 blocks -> 64
    assert ws(2, 20, 40, 0, 4) == 2 * 5 * 4 * 64 * 4    # H > 32: 4-row tiles per batch
    assert ws(0, 10, 16, 0, 4) == 0 and ws(1, 10, 0, 0, 4) == 0 and ws(1, 10, 65, 0, 4) == 0
    assert ws(1, 10, 16, -1, 4) == 0 and ws(1, 10, 16, 0, 0) == 0


def test_select_chunk_workspace_size():
    """Passes of at least query_chunk_size rows in whole row tiles, never more than the one-pass size."""
    full, chunk = qsa.qsa_select_workspace_size, qsa.qsa_select_chunk_workspace_size
    assert chunk(1, 65536, 16, 0, 4, 16) == 16 * 16384 * 4          # one 16-row tile
    assert chunk(1, 65536, 16, 0, 4, 17) == 2 * 16 * 16384 * 4      # rounded up to whole tiles
    assert chunk(1, 65536, 16, 0, 4, 1000) == 63 * 16 * 16384 * 4
    assert chunk(2, 20, 40, 0, 4, 5) == 2 * 4 * 64 * 4              # H > 32: 4-row tiles
    for args in ((1, 65536, 16, 0, 4), (2, 4096, 16, 0, 4), (1, 8192, 16, 24576, 4), (2, 20, 40, 0, 4)):
        assert chunk(*args, 1 << 40) == full(*args)                  # a chunk past the rows: one pass
    assert chunk(1, 10, 16, 0, 4, 0) == 0 and chunk(1, 10, 0, 0, 4, 16) == 0


def _call_select(B=1, S_q=64, H=4, D=64, S_global=64, q_offset=0, budget=8, c=4, ws_bytes=1 << 20,
                 null_lens=False, alias_out_q=False, k_last_stride=1, misaligned_ws=False, q_row_stride=None):
    """Every call made with this helper carries one invalid argument (fake pointers never reach a launch)."""
    L = qsa.lib()
    sq = (ctypes.c_int64 * 4)(S_q * H * D, H * D if q_row_stride is None else q_row_stride, D, 1)
    nb = max(S_global // max(c, 1), 1)
    sk = (ctypes.c_int64 * 4)(nb * D, D, D, k_last_stride)
    fq, fk, fl, fo, fw = (ctypes.c_void_p(n << 32) for n in range(1, 6))
    if alias_out_q:
        fo = fq
    if misaligned_ws:
        fw = ctypes.c_void_p((5 << 32) + 64)
    return L.qsa_select_token_ids(fq, sq, fk, sk, None if null_lens else fl, B, S_q, H, D, S_global, q_offset,
                                  budget, c, fo, fw, ws_bytes, None)


def test_select_host_checks():
    assert _call_select(S_q=0) == -2
    assert _call_select(H=0) == -2
    assert _call_select(budget=0) == -13
    assert _call_select(c=0) == -13
    assert _call_select(q_offset=-1) == -13
    assert _call_select(q_offset=8) == -13          # q_offset + S_q > S_global
    assert _call_select(D=96) == -5
    assert _call_select(H=65) == -11
    assert _call_select(budget=4 * 4097) == -11      # more than 4096 kept blocks
    assert _call_select(S_global=4 * 65537, S_q=64) == -11
    assert _call_select(null_lens=True) == -1
    assert _call_select(k_last_stride=2) == -8
    assert _call_select(alias_out_q=True) == -9
    assert _call_select(ws_bytes=16) == -10          # smaller than one 16-row tile of scores
    assert _call_select(misaligned_ws=True) == -10
    assert _call_select(q_row_stride=1 << 60) == -11        # the query tensor's extent overflows 64 bits


def test_noalloc_refuses_calls_beyond_its_scratch():
    """Host checks only: these calls need more than the 64 MiB scratch and return before any HIP call."""
    L = qsa.lib()
    fq, fk, fv, fr, fo = (ctypes.c_void_p(n << 32) for n in range(1, 6))  # distinct, never dereferenced

    def call(B, S_q, S_kv, Hq, Hkv, D, K):
        sq = (ctypes.c_int64 * 4)(S_q * Hq * D, Hq * D, D, 1)
        sk = (ctypes.c_int64 * 4)(S_kv * Hkv * D, Hkv * D, D, 1)
        s3 = (ctypes.c_int64 * 3)(S_q * K, K, 1)
        return L.qsa_forward_noalloc(fq, sq, fk, sk, fv, sk, fr, 1, s3, B, S_q, S_kv, Hq, Hkv, D, K,
                                     ctypes.c_float(0.1), fo, None)

    assert call(1, 8192, 4096, 16, 2, 256, 2048) == -14   # lists alone are 64 MiB, plus the counts
    assert call(1, 300, 1 << 20, 16, 2, 256, 64) == -14   # split: 256 rows x 16 heads x 32 ranges x 516 B
    assert call(1, 300, 1 << 20, 16, 2, 96, 64) == -5     # argument errors come first
    assert "QSA_NOALLOC_SCRATCH_BYTES" in qsa.qsa_status_string(-14)
