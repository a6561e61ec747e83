"""Helpers shared by the GPU parity tests (no oracle arithmetic here)."""

from __future__ import annotations

import numpy as np
import torch

# Forward acceptance, stated for BF16 outputs against the unrounded fp64 oracle:
#   max |err| <= 1e-2 * max|V| over every checked element, and
#   mean |err| <= 2e-3 over the elements of the checked non-empty rows;
# empty rows must be exactly +0.0 (bit pattern 0x0000).
MAX_ERR_FRACTION_OF_MAX_V = 1e-2
MEAN_ABS_ERR = 2e-3


def device() -> torch.device:
    return torch.device("cuda", 0)


def bf16_to_gpu(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device()).view(torch.bfloat16)


def gpu_bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_forward(got_bits: np.ndarray, ref: np.ndarray, counts: np.ndarray, v_bits: np.ndarray, what: str):
    """got_bits [B,R,Hq,D] uint16; ref fp64 same shape; counts [B,R] route counts of those rows."""
    got = bits_to_f64(got_bits)
    empty = counts == 0
    assert not np.any(got_bits[empty]), f"{what}: empty rows are not exactly +0.0"
    max_v = float(np.abs(bits_to_f64(v_bits)).max())
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    worst = float(err.max()) if err.size else 0.0
    assert worst <= MAX_ERR_FRACTION_OF_MAX_V * max_v, f"{what}: max|err| {worst:.3e} > 1e-2*max|V| ({max_v:.3f})"
    if (~empty).any():
        mean = float(err[~empty].mean())
        assert mean <= MEAN_ABS_ERR, f"{what}: mean|err| {mean:.3e} > {MEAN_ABS_ERR}"
    return worst
