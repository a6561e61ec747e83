"""Pins of the oracle's log-sum-exp and gradients against facts outside the oracle.

The gradients are pinned to torch autograd on a dense masked softmax written
with torch CPU float64 ops (a library differentiation, not the oracle's
hand-written Jacobian), to central finite differences of the numpy dense
attention in ``pins``, to closed forms (a single route has zero score
gradients; dv sums the upstream gradients that reach it) and to sum rules
(each row's score gradients sum to zero, so the dk rows of a KV head sum to
zero; each row's probabilities sum to one, so the dv rows sum to the
upstream gradients of the non-empty rows).  ``test_backward_mutants_fail_pins``
plants mistakes in a copy of the oracle and checks that a pin catches each.
"""

from __future__ import annotations

import math
import subprocess

import numpy as np
import pytest
import torch

import oracle
import pins
from workloads.generators import float32_to_bf16_bits, random_small_case


def _dout(seed, shape):
    rng = np.random.Generator(np.random.PCG64(seed))
    return float32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def torch_grads(q_bits, k_bits, v_bits, dout_bits, routes, scale):
    """dq, dk, dv of sum(dout * attention) by torch autograd (CPU, float64)."""
    q, k, v, g = (torch.tensor(pins.bf16_to_f64(t)) for t in (q_bits, k_bits, v_bits, dout_bits))
    for t in (q, k, v):
        t.requires_grad_(True)
    B, S_q, Hq, D = q.shape
    S_kv, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    mask = torch.tensor(pins.brute_membership(routes, S_kv).astype(bool))[:, None]  # [B,1,S_q,S_kv]
    has = mask.any(dim=-1, keepdim=True)
    kk = k.repeat_interleave(G, dim=2).permute(0, 2, 3, 1)  # [B,Hq,D,S_kv]
    vv = v.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)  # [B,Hq,S_kv,D]
    s = torch.matmul(q.permute(0, 2, 1, 3), kk) * scale  # [B,Hq,S_q,S_kv]
    s = s.masked_fill(~mask, -math.inf).masked_fill(~has, 0.0)
    p = torch.softmax(s, dim=-1) * has
    o = torch.matmul(p, vv).permute(0, 2, 1, 3)  # [B,S_q,Hq,D]
    (o * g).sum().backward()
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


def _rel(a, b):
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


CASES = [  # seed, B, S_q, S_kv, Hq, Hkv, D, K
    (11, 1, 12, 16, 2, 1, 64, 6),
    (12, 2, 9, 20, 4, 2, 64, 8),
    (13, 1, 16, 24, 8, 1, 128, 12),
    (14, 2, 7, 11, 6, 3, 64, 5),
    (15, 1, 10, 40, 16, 2, 256, 16),
]


# --------------------------------------------------------------------------
# checks (shared with the mutation test)
# --------------------------------------------------------------------------

def check_torch_autograd(orc):
    for seed, B, S_q, S_kv, Hq, Hkv, D, K in CASES:
        q, k, v, r = random_small_case(seed, B, S_q, S_kv, Hq, Hkv, D, K)
        g = _dout(seed + 100, q.shape)
        scale = 1.0 / math.sqrt(D)
        dq, dk, dv = orc.backward(q, k, v, g, r, scale)
        tq, tk, tv = torch_grads(q, k, v, g, r, scale)
        assert _rel(dq, tq) < 1e-10 and _rel(dk, tk) < 1e-10 and _rel(dv, tv) < 1e-10, seed


def check_finite_differences(orc):
    q, k, v, r = random_small_case(21, 1, 5, 7, 2, 1, 64, 4, p_empty=0.0)
    g = _dout(22, q.shape)
    scale = 0.2
    mask = pins.brute_membership(r, k.shape[1]).astype(bool)
    qf, kf, vf, gf = (pins.bf16_to_f64(t) for t in (q, k, v, g))
    dq, dk, dv = orc.backward(q, k, v, g, r, scale)
    rng = np.random.Generator(np.random.PCG64(23))
    eps = 1e-5

    def loss(qx, kx, vx):
        return float((pins.dense_attention_f64(qx, kx, vx, mask, scale) * gf).sum())

    for which, grad in (("q", dq), ("k", dk), ("v", dv)):
        base = {"q": qf, "k": kf, "v": vf}[which]
        for _ in range(6):
            idx = tuple(int(rng.integers(0, n)) for n in base.shape)
            plus, minus = base.copy(), base.copy()
            plus[idx] += eps
            minus[idx] -= eps
            args_p = {"q": qf, "k": kf, "v": vf, which: plus}
            args_m = {"q": qf, "k": kf, "v": vf, which: minus}
            fd = (loss(args_p["q"], args_p["k"], args_p["v"]) - loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (which, idx, fd, grad[idx])


def check_single_route(orc):
    """One route per row: p = 1, so the score gradients vanish and dv collects dout."""
    rng = np.random.Generator(np.random.PCG64(31))
    B, S_q, S_kv, Hq, Hkv, D = 2, 9, 6, 4, 2, 64
    q, k, v, _ = random_small_case(31, B, S_q, S_kv, Hq, Hkv, D, 3)
    ids = rng.integers(0, S_kv, size=(B, S_q))
    r = np.stack([ids, ids, np.full_like(ids, -1)], axis=-1)  # duplicate + invalid slot
    g = _dout(32, q.shape)
    dq, dk, dv = orc.backward(q, k, v, g, r, 0.3)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    gf = pins.bf16_to_f64(g)
    G = Hq // Hkv
    want = np.zeros_like(dv)
    for b in range(B):
        for i in range(S_q):
            for h in range(Hq):
                want[b, ids[b, i], h // G] += gf[b, i, h]
    assert np.abs(dv - want).max() < 1e-12


def check_sum_rules(orc):
    for seed, B, S_q, S_kv, Hq, Hkv, D, K in CASES[:4]:
        q, k, v, r = random_small_case(seed, B, S_q, S_kv, Hq, Hkv, D, K)
        g = _dout(seed + 200, q.shape)
        dq, dk, dv = orc.backward(q, k, v, g, r, 0.125)
        _, cnt = pins.brute_lists(r, S_kv)
        gf = pins.bf16_to_f64(g) * (cnt > 0)[:, :, None, None]
        G = Hq // Hkv
        want_v = gf.reshape(B, S_q, Hkv, G, D).sum(axis=(1, 3))
        assert np.abs(dv.sum(axis=1) - want_v).max() < 1e-10 * max(1.0, np.abs(want_v).max())
        assert np.abs(dk.sum(axis=1)).max() < 1e-10 * max(1.0, np.abs(dk).max())


def check_empty_rows(orc):
    q, k, v, r = random_small_case(41, 1, 10, 12, 4, 1, 64, 5, p_empty=0.0)
    r[0, [2, 7]] = -1
    g = _dout(42, q.shape)
    dq, dk, dv = orc.backward(q, k, v, g, r, 0.125)
    assert (dq[0, [2, 7]] == 0).all()
    g2 = g.copy()
    g2[0, [2, 7]] = _dout(43, g2[0, [2, 7]].shape)
    _, dk2, dv2 = orc.backward(q, k, v, g2, r, 0.125)
    assert np.abs(dk2 - dk).max() < 1e-13 and np.abs(dv2 - dv).max() < 1e-13


def check_lse(orc):
    for seed, B, S_q, S_kv, Hq, Hkv, D, K in CASES:
        q, k, v, r = random_small_case(seed, B, S_q, S_kv, Hq, Hkv, D, K)
        scale = 1.0 / math.sqrt(D)
        got = orc.lse(q, k, r, scale)
        want = pins.dense_lse(q, k, r, scale)
        assert (np.isneginf(got) == np.isneginf(want)).all()
        fin = np.isfinite(want)
        assert np.abs(got[fin] - want[fin]).max() < 1e-12
    # closed form: q = 0 gives equal scores, so lse = log |R|
    q, k, v, r = random_small_case(51, 1, 8, 16, 2, 1, 64, 6, q_zero=True)
    _, cnt = pins.brute_lists(r, 16)
    got = orc.lse(q, k, r, 0.5)
    for i in range(8):
        want = math.log(cnt[0, i]) if cnt[0, i] else -math.inf
        assert got[0, i, 0] == pytest.approx(want, abs=1e-14) if cnt[0, i] else got[0, i, 0] == want


CHECKS = (check_torch_autograd, check_finite_differences, check_single_route, check_sum_rules,
          check_empty_rows, check_lse)


# --------------------------------------------------------------------------
# the pins
# --------------------------------------------------------------------------

@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_backward_pin(check):
    check(oracle._load())


def test_backward_permuting_and_duplicating_routes_changes_nothing():
    q, k, v, r = random_small_case(61, 1, 8, 12, 4, 2, 64, 6)
    g = _dout(62, q.shape)
    base = oracle.backward(q, k, v, g, r, 0.125)
    rng = np.random.Generator(np.random.PCG64(63))
    r2 = np.concatenate([r, r[:, :, :2]], axis=-1)
    r2 = np.take_along_axis(r2, rng.permuted(np.tile(np.arange(r2.shape[-1]), (1, 8, 1)), axis=-1), axis=-1)
    other = oracle.backward(q, k, v, g, r2, 0.125)
    for a, b in zip(base, other):
        assert np.abs(a - b).max() < 1e-13


def test_backward_row_and_key_ranges_match_full():
    q, k, v, r = random_small_case(71, 2, 12, 20, 4, 2, 64, 8)
    g = _dout(72, q.shape)
    dq, dk, dv = oracle.backward(q, k, v, g, r, 0.125)
    dq2, dk2, dv2 = oracle.backward(q, k, v, g, r, 0.125, rows=(3, 9), keys=(5, 17))
    assert np.abs(dq2 - dq[:, 3:9]).max() < 1e-13
    assert np.abs(dk2 - dk[:, 5:17]).max() < 1e-13 and np.abs(dv2 - dv[:, 5:17]).max() < 1e-13


# --------------------------------------------------------------------------
# planted mistakes: every backward mutant must fail at least one pin
# --------------------------------------------------------------------------

BACKWARD_MUTANTS = {
    "softmax Jacobian without the mean term": ("double ds = p[j] * (dp[j] - pdp);", "double ds = p[j] * dp[j];"),
    "Jacobian sign flipped": ("double ds = p[j] * (dp[j] - pdp);", "double ds = p[j] * (pdp - dp[j]);"),
    "dk without the scale": ("gk[d] += scale * ds * bf16_to_double(qv[d]);", "gk[d] += ds * bf16_to_double(qv[d]);"),
    "dv weighted by ds": ("gw[d] += p[j] * bf16_to_double(gv[d]);", "gw[d] += ds * bf16_to_double(gv[d]);"),
    "dq sign flipped": ("o[d] += scale * ds * bf16_to_double(kv[d]);", "o[d] -= scale * ds * bf16_to_double(kv[d]);"),
    "dp from q instead of dout": ("for (int64_t d = 0; d < D; ++d) dot += bf16_to_double(gv[d]) * bf16_to_double(vv[d]);",
                                  "for (int64_t d = 0; d < D; ++d) dot += bf16_to_double(qv[d]) * bf16_to_double(vv[d]);"),
    "unnormalised probabilities": ("p[j] /= denom;", "p[j] /= 1.0;"),
    "lse without the max": ("n == 0 ? -INFINITY : m + log(sum)", "n == 0 ? -INFINITY : log(sum)"),
}


def _backward_pins_fail(orc) -> bool:
    for check in CHECKS:
        try:
            check(orc)
        except AssertionError:
            return True
    return False


@pytest.mark.parametrize("name", sorted(BACKWARD_MUTANTS))
def test_backward_mutants_fail_pins(name, tmp_path):
    src = open(oracle._SRC).read()
    old, new = BACKWARD_MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name!r} not unique"
    mutant = tmp_path / "mutant.c"
    mutant.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", str(mutant), "-o", str(so), "-lm"])
    assert _backward_pins_fail(oracle.Oracle(str(so))), f"no pin catches mutant: {name}"
