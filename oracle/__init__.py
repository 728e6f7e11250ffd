"""CPU oracle of the MoE decode tail -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library
(``expert_finalize_rmsnorm_amd``) never imports, links or runs it, and the two
share no code.

This module builds and loads ``liboracle.so`` (plain C, ``oracle.c``) and
wraps its functions for numpy arrays.  BF16 arrays are ``numpy.uint16`` bit
patterns; every array is C-contiguous host memory.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

W_F32 = 0
W_BF16 = 1
SS_W64 = 0  # the wave64 sum-of-squares tree (default)
SS_SEQ = 1  # plain sequential sum of squares

# -O2 with contraction off and no fast-math: every FP32 operation rounds on
# its own, exactly as the C source is written.
CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
          "-Wall", "-Wextra", "-shared", "-fPIC"]


def build() -> str:
    """Compile liboracle.so with gcc (always recompiles)."""
    tmp = _LIB + ".tmp"
    subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = ctypes.CDLL(_LIB)
        P, I32, I64, F32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
        _lib.oracle_bf16_round.argtypes = [P, P, I64]
        _lib.oracle_sum_of_squares.argtypes = [P, I32]
        _lib.oracle_sum_of_squares.restype = F32
        _lib.oracle_set_ss_order.argtypes = [I32]
        _lib.oracle_set_ss_order.restype = None
        _lib.oracle_inv_rms.argtypes = [F32, I32, F32]
        _lib.oracle_inv_rms.restype = F32
        _lib.oracle_route_products.argtypes = [P, P, F32, F32, F32, I32, I32, P]
        _lib.oracle_route_products.restype = None
        _lib.oracle_finalize.argtypes = [P, I64, P, P, I32, P, F32, F32, I32,
                                         I32, I32, I32, I32, P, P, I32]
        _lib.oracle_finalize_plain.argtypes = [P, I64, P, P, I32, I32, I32, I32, I32, P, P,
                                               I32]
        _lib.oracle_rank_combine.argtypes = [P, I32, I32, I32, P]
        _lib.oracle_tp_finalize.argtypes = [P, I64, P, P, I32, P, F32, F32, I32,
                                            I32, I32, I32, I32, P, I32]
        _lib.oracle_combine_norm_upproj.argtypes = [P, I32, P, F32, P, I32, P,
                                                    I32, I32, P, P, I32]
        _lib.oracle_shared_expert.argtypes = [P, I32, I32, P, P, I32, P, P, P, I32]
        for f in ("oracle_bf16_round", "oracle_finalize", "oracle_finalize_plain",
                  "oracle_rank_combine",
                  "oracle_tp_finalize", "oracle_combine_norm_upproj",
                  "oracle_shared_expert"):
            getattr(_lib, f).restype = None
    return _lib


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _u16(a):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    return a


def _weights(w):
    w = np.ascontiguousarray(w)
    if w.dtype == np.float32:
        return w, W_F32
    if w.dtype == np.uint16:
        return w, W_BF16
    raise TypeError("route weights are float32 or uint16 (BF16 bits)")


def bf16_round(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, np.uint16)
    lib().oracle_bf16_round(_ptr(x), _ptr(y), x.size)
    return y


def f32(h) -> np.ndarray:
    """FP32 values of BF16 bit patterns."""
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


def sum_of_squares(v) -> np.float32:
    v = np.ascontiguousarray(v, dtype=np.float32)
    return np.float32(lib().oracle_sum_of_squares(_ptr(v), v.shape[-1]))


class ss_order:
    """Context manager: the oracle's sum-of-squares order (SS_W64 or SS_SEQ)
    inside the block, the wave64 tree again after it."""

    def __init__(self, order):
        self.order = order

    def __enter__(self):
        lib().oracle_set_ss_order(self.order)
        return self

    def __exit__(self, *exc):
        lib().oracle_set_ss_order(SS_W64)
        return False


def inv_rms(ss, P, eps) -> np.float32:
    """1 / sqrt(ss * fp32(1/P) + eps), correctly rounded to FP32."""
    return np.float32(lib().oracle_inv_rms(float(np.float32(ss)), int(P), float(np.float32(eps))))


def route_products(x, gamma, gain_center, w, eps, weight_before_norm) -> np.ndarray:
    """One BF16 row x [P] -> its weighted, normalized FP32 products [P]."""
    x = _u16(x)
    gamma = _u16(gamma)
    P = x.shape[-1]
    p = np.empty(P, np.float32)
    lib().oracle_route_products(_ptr(x), _ptr(gamma), float(np.float32(gain_center)),
                                float(np.float32(w)), float(np.float32(eps)),
                                int(bool(weight_before_norm)), P, _ptr(p))
    return p


def finalize(rows, idx, w, gamma, gain_center, eps, weight_before_norm,
             combine=True, nthreads=0):
    """rows [tp,R,P] u16, idx [tp,b,K] i32, w [b,K] f32|u16, gamma [P] u16.
    Returns (partials [tp,b,P], out [b,P] or None)."""
    rows = _u16(rows)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    w, wdt = _weights(w)
    gamma = _u16(gamma)
    tp, R, P = rows.shape
    _, b, K = idx.shape
    partials = np.empty((tp, b, P), np.uint16)
    out = np.empty((b, P), np.uint16) if combine else None
    lib().oracle_finalize(_ptr(rows), R, _ptr(idx), _ptr(w), wdt, _ptr(gamma),
                          gain_center, eps, int(bool(weight_before_norm)),
                          b, K, P, tp, _ptr(partials), _ptr(out), nthreads)
    return partials, out


def finalize_plain(rows, idx, w, combine=True, nthreads=0):
    """The finalize without a per-route norm ([tail_runtime] module docstring):
    rows [tp,R,P] u16, idx [tp,b,K] i32, w [b,K] f32|u16.
    Returns (partials [tp,b,P], out [b,P] or None)."""
    rows = _u16(rows)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    w, wdt = _weights(w)
    tp, R, P = rows.shape
    _, b, K = idx.shape
    partials = np.empty((tp, b, P), np.uint16)
    out = np.empty((b, P), np.uint16) if combine else None
    lib().oracle_finalize_plain(_ptr(rows), R, _ptr(idx), _ptr(w), wdt, b, K, P, tp,
                                _ptr(partials), _ptr(out), nthreads)
    return partials, out


def rank_combine(partials):
    partials = _u16(partials)
    tp, b, P = partials.shape
    out = np.empty((b, P), np.uint16)
    lib().oracle_rank_combine(_ptr(partials), tp, b, P, _ptr(out))
    return out


def tp_finalize(kpart, idx, w, gamma, gain_center, eps, weight_before_norm,
                nthreads=0):
    """kpart [tp,num_rows,P] u16, idx [b,K] i32, w [b,K]. Returns out [b,P]."""
    kpart = _u16(kpart)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    w, wdt = _weights(w)
    gamma = _u16(gamma)
    tp, num_rows, P = kpart.shape
    b, K = idx.shape
    out = np.empty((b, P), np.uint16)
    lib().oracle_tp_finalize(_ptr(kpart), num_rows, _ptr(idx), _ptr(w), wdt,
                             _ptr(gamma), gain_center, eps,
                             int(bool(weight_before_norm)), b, K, P, tp,
                             _ptr(out), nthreads)
    return out


def combine_norm_upproj(lat, gamma, eps, w_up, rs=None, nthreads=0):
    """lat [tp,b,L], gamma [L], w_up [N,L], rs [b,N] or None.
    Returns (normed [b,L], out [b,N])."""
    lat = _u16(lat)
    gamma = _u16(gamma)
    w_up = _u16(w_up)
    tp, b, L = lat.shape
    N = w_up.shape[0]
    if rs is not None:
        rs = _u16(rs)
    normed = np.empty((b, L), np.uint16)
    out = np.empty((b, N), np.uint16)
    lib().oracle_combine_norm_upproj(_ptr(lat), tp, _ptr(gamma), eps, _ptr(w_up),
                                     N, _ptr(rs), b, L, _ptr(normed), _ptr(out),
                                     nthreads)
    return normed, out


def shared_expert(x, w_gate, w_up, w_down, nthreads=0):
    """x [b,H], w_gate/w_up [I,H], w_down [H,I]. Returns (h [b,I], rs [b,H])."""
    x = _u16(x)
    w_gate, w_up, w_down = _u16(w_gate), _u16(w_up), _u16(w_down)
    b, H = x.shape
    I = w_gate.shape[0]
    h = np.empty((b, I), np.uint16)
    rs = np.empty((b, H), np.uint16)
    lib().oracle_shared_expert(_ptr(x), b, H, _ptr(w_gate), _ptr(w_up), I,
                               _ptr(w_down), _ptr(h), _ptr(rs), nthreads)
    return h, rs
