"""Helpers of the GPU parity tests: device copies and the acceptance bars."""
from __future__ import annotations

import os

import numpy as np
import torch

ORACLE_THREADS = max(1, min(16, os.cpu_count() or 1))
SENTINEL = 0x7777  # a BF16 word no kernel writes for these inputs


def dev(a: np.ndarray) -> torch.Tensor:
    """Host array -> device tensor (BF16 bits travel as int16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def host(t: torch.Tensor) -> np.ndarray:
    """Device BF16 bits -> numpy uint16."""
    torch.cuda.synchronize()
    return t.cpu().numpy().view(np.uint16)


def empty_bf16(*shape) -> torch.Tensor:
    return torch.full(shape, SENTINEL, dtype=torch.int16, device="cuda")


def f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


def ordered(h: np.ndarray) -> np.ndarray:
    """BF16 bits -> integers whose differences count BF16 steps (+0 == -0)."""
    h = np.asarray(h, np.uint16).astype(np.int64)
    return np.where(h & 0x8000, -(h & 0x7FFF), h)


def finalize_bar(got: np.ndarray, want: np.ndarray, what: str) -> float:
    """Finalize/combine bar: every element within 1 BF16 step and at least
    99.9% bit-exact.  Returns the bit-exact fraction."""
    assert got.shape == want.shape
    assert not np.any(got == SENTINEL) or np.any(want == SENTINEL), f"{what}: unwritten output"
    ulps = np.abs(ordered(got) - ordered(want))
    exact = float(np.mean(got == want))
    assert ulps.max(initial=0) <= 1, f"{what}: max {ulps.max()} BF16 steps off"
    assert exact >= 0.999, f"{what}: only {exact:.5f} bit-exact"
    assert not np.any(got == 0x8000), f"{what}: -0 written"
    return exact


def gemm_bar(got: np.ndarray, want: np.ndarray, what: str) -> float:
    """Projection bar: |err| <= 2e-2 + 1e-2 |ref| against the FP32 oracle.
    Returns the worst ratio err / bound."""
    assert got.shape == want.shape
    g, w = f32(got).astype(np.float64), f32(want).astype(np.float64)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - w)
    bound = 2e-2 + 1e-2 * np.abs(w)
    worst = float(np.max(err / bound))
    assert worst <= 1.0, f"{what}: error {worst:.3f} x the bound"
    assert not np.any(got == 0x8000), f"{what}: -0 written"
    return worst
