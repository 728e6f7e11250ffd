"""Straight-line FP64 evaluation of the tail's formulas, for pinning the oracle.

Written independently of ``oracle/`` (vectorized numpy in float64, no shared
code): it evaluates the formulas of the MoE tail pages in double precision
and rounds to BF16 only where the formulas round.  A result of the FP32
oracle must lie within the FP32 rounding-error bound of this evaluation; a
dropped term, a wrong sign, a misplaced gain or a transposed operand lands
far outside it.
"""
from __future__ import annotations

import numpy as np

U24 = 2.0 ** -24  # unit roundoff of FP32


def f64(h) -> np.ndarray:
    """float64 values of BF16 bit patterns."""
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_bf16(x) -> np.ndarray:
    """Nearest BF16 value (ties to even) of float64 values, as float64.

    BF16 keeps 8 significant bits; below 2^-126 the quantum stays 2^-133."""
    x = np.asarray(x, np.float64)
    _, e = np.frexp(x)
    q = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.round(x / q) * q  # numpy rounds halves to even
    big = np.abs(r) > 3.3895313892515355e38
    return np.where(big, np.copysign(np.inf, x), r)


def ulp_bf16(x) -> np.ndarray:
    """Spacing of BF16 values at |x| (subnormal quantum below 2^-126)."""
    _, e = np.frexp(np.abs(np.asarray(x, np.float64)))
    return np.ldexp(1.0, np.maximum(e - 8, -133))


def norm_products(x, gain, w, eps, wbn):
    """x [..., P] float64 -> (w * normalized x, |terms| scale) in float64.

    s = x * gain (weight_before_norm) or x; inv = 1/sqrt(mean(s^2) + eps);
    n = s * inv, or (x * inv) * gain without weight_before_norm; p = n * w."""
    s = x * gain if wbn else x
    inv = 1.0 / np.sqrt(np.mean(s * s, axis=-1, keepdims=True) + eps)
    n = s * inv if wbn else (x * inv) * gain
    return n * w


def ep_finalize(rows, idx, w, gamma, gain_center, eps, wbn):
    """Returns (acc [tp,b,P] unrounded partial sums, scale [tp,b,P] = sum of
    |products|) in float64."""
    rows64 = f64(rows)
    gain = f64(gamma) + gain_center
    wv = f64(w) if w.dtype == np.uint16 else w.astype(np.float64)
    tp, R, P = rows.shape
    _, b, K = idx.shape
    acc = np.zeros((tp, b, P))
    scale = np.zeros((tp, b, P))
    for d in range(tp):
        for t in range(b):
            for k in range(K):
                r = idx[d, t, k]
                if 0 <= r < R:
                    p = norm_products(rows64[d, r], gain, wv[t, k], eps, wbn)
                    acc[d, t] += p
                    scale[d, t] += np.abs(p)
    return acc, scale


def tp_finalize(kpart, idx, w, gamma, gain_center, eps, wbn):
    """Returns (acc [b,P] unrounded route sums, scale) in float64; x_r is the
    BF16 rounding of the exact rank sum."""
    k64 = f64(kpart)
    gain = f64(gamma) + gain_center
    wv = f64(w) if w.dtype == np.uint16 else w.astype(np.float64)
    tp, n, P = kpart.shape
    b, K = idx.shape
    acc = np.zeros((b, P))
    scale = np.zeros((b, P))
    for t in range(b):
        for k in range(K):
            r = idx[t, k]
            if 0 <= r < n:
                xr = round_bf16(k64[:, r, :].sum(axis=0))
                p = norm_products(xr, gain, wv[t, k], eps, wbn)
                acc[t] += p
                scale[t] += np.abs(p)
    return acc, scale


def within(oracle_bits, ref, err_bound):
    """True where the oracle's BF16 result lies within err_bound plus one
    BF16 spacing of the float64 reference."""
    got = f64(oracle_bits)
    tol = err_bound + ulp_bf16(np.abs(ref) + err_bound)
    return np.abs(got - ref) <= tol
