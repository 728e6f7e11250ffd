"""Python binding of libmoetail: the MoE decode tail on one MI355X (gfx950).

Thin ctypes marshalling over the C ABI in ``include/moetail.h``: the same
entry-point names, device tensors in, status codes turned into exceptions.
Every step of the tail runs in the library's HIP kernels; PyTorch only owns
device memory and streams.  There is no fallback: if ``libmoetail.so`` is
missing the import of an entry point raises.

BF16 tensors are ``torch.bfloat16`` (or int16/uint16 views of BF16 bits);
route weights ``torch.float32`` or ``torch.bfloat16``; indices
``torch.int32``.  All tensors must be contiguous CUDA (HIP) tensors.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoetail.so")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, -1, -2, -3, -4
F32, BF16 = 0, 1
NORM_GAIN_AFTER, NORM_GAIN_FIRST, NO_NORM = 0, 1, 2  # moetail_finalize norm modes
OP_FINALIZE, OP_TP_FINALIZE, OP_COMBINE_NORM_UPPROJ, OP_SHARED_EXPERT, OP_TAIL = 0, 1, 2, 3, 4
W_ROWS, W_TILED = 0, 1  # weight layouts of the projections

_CALLS = ("moetail_finalize", "moetail_tp_finalize", "moetail_combine_norm_upproj",
          "moetail_shared_expert", "moetail_tail", "moetail_decode_tail", "moetail_pack_weights")
ENTRY_POINTS = _CALLS + ("moetail_workspace_bytes", "moetail_status_string")


class MoetailError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libmoetail.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m expert_finalize_rmsnorm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
        SZ = ctypes.c_size_t
        L.moetail_finalize.argtypes = [P, I64, P, P, I32, P, F, F, I32, I32, I32, I32, I32,
                                       P, P, P]
        L.moetail_tp_finalize.argtypes = [P, I64, P, P, I32, P, F, F, I32, I32, I32, I32, I32,
                                          P, P, SZ, P]
        L.moetail_combine_norm_upproj.argtypes = [P, I32, P, F, P, I32, P, I32, I32, P, P, I32,
                                                  P, SZ, P]
        L.moetail_shared_expert.argtypes = [P, I32, I32, P, P, I32, P, P, P, I32, P, SZ, P]
        L.moetail_tail.argtypes = [P, I32, P, F, P, I32, P, P, P, P, I32, I32, I32, P, P, P, P,
                                   I32, P, SZ, P]
        L.moetail_pack_weights.argtypes = [P, I64, I32, P, P]
        L.moetail_decode_tail.argtypes = [P, I64, P, P, I32, P, F, F, I32, I32, P, I32, P, F, P,
                                          I32, P, P, P, P, I32, I32, I32, P, P, P, P, I32, P, SZ,
                                          P]
        L.moetail_workspace_bytes.argtypes = [I32, I32, I32, I32, I32]
        L.moetail_workspace_bytes.restype = SZ
        L.moetail_status_string.argtypes = [I32]
        L.moetail_status_string.restype = ctypes.c_char_p
        for f in _CALLS:
            getattr(L, f).restype = I32
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moetail_status_string(status).decode()


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("libmoetail takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libmoetail takes contiguous tensors")
    return t.data_ptr()


def _bf16(t, name):
    if t is not None and t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must hold BF16 bits, got {t.dtype}")
    return t


def _weights(w):
    if w.dtype == torch.float32:
        return F32
    if w.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return BF16
    raise TypeError("route weights must be float32 or bfloat16")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status, where):
    if status != OK:
        raise MoetailError(status, where)


def workspace_bytes(op: int, b: int, dim0: int, dim1: int = 0, dim2: int = 0) -> int:
    return int(lib().moetail_workspace_bytes(op, b, dim0, dim1, dim2))


def moetail_finalize(rows, permuted_idx, route_w, gamma, gain_center, eps, weight_before_norm,
                     partials=None, out=None, stream=None):
    """rows [tp, R, P], permuted_idx [tp, b, K], route_w [b, K], gamma [P]
    (or None with NO_NORM); writes partials [tp, b, P] and/or out [b, P].
    weight_before_norm: a bool, or a norm mode (NORM_GAIN_AFTER,
    NORM_GAIN_FIRST, NO_NORM)."""
    _bf16(rows, "rows"), _bf16(gamma, "gamma"), _bf16(partials, "partials"), _bf16(out, "out")
    tp, R, P = rows.shape
    _, b, K = permuted_idx.shape
    if permuted_idx.dtype != torch.int32:
        raise TypeError("permuted_idx must be int32")
    st = lib().moetail_finalize(_ptr(rows), R, _ptr(permuted_idx), _ptr(route_w),
                                _weights(route_w), _ptr(gamma), float(gain_center), float(eps),
                                int(weight_before_norm), b, K, P, tp, _ptr(partials),
                                _ptr(out), _stream(stream))
    _check(st, "moetail_finalize")


def moetail_tp_finalize(kpartials, permuted_idx, route_w, gamma, gain_center, eps,
                        weight_before_norm, out, workspace=None, stream=None):
    """kpartials [tp, num_rows, P], permuted_idx [b, K], route_w [b, K]; writes out [b, P].
    workspace: at least workspace_bytes(OP_TP_FINALIZE, b, K, P) bytes."""
    _bf16(kpartials, "kpartials"), _bf16(gamma, "gamma"), _bf16(out, "out")
    tp, num_rows, P = kpartials.shape
    b, K = permuted_idx.shape
    if permuted_idx.dtype != torch.int32:
        raise TypeError("permuted_idx must be int32")
    ws = _ptr(workspace) if workspace is not None else None
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().moetail_tp_finalize(_ptr(kpartials), num_rows, _ptr(permuted_idx),
                                   _ptr(route_w), _weights(route_w), _ptr(gamma),
                                   float(gain_center), float(eps), int(bool(weight_before_norm)),
                                   b, K, P, tp, _ptr(out), ws, wsb, _stream(stream))
    _check(st, "moetail_tp_finalize")


def moetail_combine_norm_upproj(latent_partials, gamma, eps, w_up, out, rs=None, normed=None,
                                workspace=None, stream=None, w_layout=W_ROWS):
    """latent_partials [tp, b, L], gamma [L], w_up [N, L] (row-major, or its
    pack_weights copy with w_layout=W_TILED), rs [b, N] or None; writes out
    [b, N] and normed [b, L] when given.  workspace: a device tensor of at
    least workspace_bytes(OP_COMBINE_NORM_UPPROJ, b, L, N, tp) bytes."""
    for t, n in ((latent_partials, "latent_partials"), (gamma, "gamma"), (w_up, "w_up"),
                 (out, "out"), (rs, "rs"), (normed, "normed")):
        _bf16(t, n)
    tp, b, L = latent_partials.shape
    N = w_up.shape[0]
    ws = _ptr(workspace) if workspace is not None else None
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().moetail_combine_norm_upproj(_ptr(latent_partials), tp, _ptr(gamma), float(eps),
                                           _ptr(w_up), N, _ptr(rs), b, L, _ptr(normed),
                                           _ptr(out), int(w_layout), ws, wsb, _stream(stream))
    _check(st, "moetail_combine_norm_upproj")


def moetail_shared_expert(x, w_gate, w_up, w_down, rs, h=None, workspace=None, stream=None,
                          w_layout=W_ROWS):
    """x [b, H], w_gate/w_up [I, H], w_down [H, I] (all row-major, or all
    pack_weights copies with w_layout=W_TILED); writes rs [b, H] and h
    [b, I] when given.  workspace: at least
    workspace_bytes(OP_SHARED_EXPERT, b, H, I) bytes."""
    for t, n in ((x, "x"), (w_gate, "w_gate"), (w_up, "w_up"), (w_down, "w_down"), (rs, "rs"),
                 (h, "h")):
        _bf16(t, n)
    b, H = x.shape
    I = w_gate.shape[0]
    ws = _ptr(workspace) if workspace is not None else None
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().moetail_shared_expert(_ptr(x), b, H, _ptr(w_gate), _ptr(w_up), I, _ptr(w_down),
                                     _ptr(h), _ptr(rs), int(w_layout), ws, wsb, _stream(stream))
    _check(st, "moetail_shared_expert")


def moetail_tail(latent_partials, gamma, eps, w_up, x, w_gate, w_up_shared, w_down, out,
                 rs=None, normed=None, h=None, workspace=None, stream=None, w_layout=W_ROWS):
    """The tail after the finalize in one call: rs = shared expert of x,
    out = up projection of the normed rank-combined latent + rs.
    latent_partials [tp, b, L], gamma [L], w_up [H, L]; x [b, H], w_gate and
    w_up_shared [I, H], w_down [H, I]; writes out [b, H] and rs [b, H],
    normed [b, L], h [b, I] when given.  The four weights are all row-major,
    or all pack_weights copies with w_layout=W_TILED.  workspace: at least
    workspace_bytes(OP_TAIL, b, L, H, I) bytes."""
    for t, n in ((latent_partials, "latent_partials"), (gamma, "gamma"), (w_up, "w_up"),
                 (x, "x"), (w_gate, "w_gate"), (w_up_shared, "w_up_shared"), (w_down, "w_down"),
                 (out, "out"), (rs, "rs"), (normed, "normed"), (h, "h")):
        _bf16(t, n)
    tp, b, L = latent_partials.shape
    H = x.shape[1]
    I = w_gate.shape[0]
    ws = _ptr(workspace) if workspace is not None else None
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().moetail_tail(_ptr(latent_partials), tp, _ptr(gamma), float(eps), _ptr(w_up), L,
                            _ptr(x), _ptr(w_gate), _ptr(w_up_shared), _ptr(w_down), H, I, b,
                            _ptr(out), _ptr(rs), _ptr(normed), _ptr(h), int(w_layout), ws,
                            wsb, _stream(stream))
    _check(st, "moetail_tail")


def moetail_decode_tail(rows, permuted_idx, route_w, fin_gamma, gain_center, fin_eps,
                        weight_before_norm, latent_partials, gamma, eps, w_up, x, w_gate,
                        w_up_shared, w_down, out, rs=None, normed=None, h=None, workspace=None,
                        stream=None, w_layout=W_ROWS):
    """The whole tail in one call: latent_partials [tp, b, L] = the EP
    finalize of rows [tp, R, L] (as moetail_finalize with partials only),
    then out [b, H] = moetail_tail(latent_partials, ...).  workspace: at
    least workspace_bytes(OP_TAIL, b, L, H, I) bytes."""
    for t, n in ((rows, "rows"), (fin_gamma, "fin_gamma"), (latent_partials, "latent_partials"),
                 (gamma, "gamma"), (w_up, "w_up"), (x, "x"), (w_gate, "w_gate"),
                 (w_up_shared, "w_up_shared"), (w_down, "w_down"), (out, "out"), (rs, "rs"),
                 (normed, "normed"), (h, "h")):
        _bf16(t, n)
    if permuted_idx.dtype != torch.int32:
        raise TypeError("permuted_idx must be int32")
    tp, R, L = rows.shape
    _, b, K = permuted_idx.shape
    H = x.shape[1]
    I = w_gate.shape[0]
    ws = _ptr(workspace) if workspace is not None else None
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().moetail_decode_tail(_ptr(rows), R, _ptr(permuted_idx), _ptr(route_w),
                                   _weights(route_w), _ptr(fin_gamma), float(gain_center),
                                   float(fin_eps), int(weight_before_norm), K,
                                   _ptr(latent_partials), tp, _ptr(gamma), float(eps),
                                   _ptr(w_up), L, _ptr(x), _ptr(w_gate), _ptr(w_up_shared),
                                   _ptr(w_down), H, I, b, _ptr(out), _ptr(rs), _ptr(normed),
                                   _ptr(h), int(w_layout), ws, wsb, _stream(stream))
    _check(st, "moetail_decode_tail")


def moetail_pack_weights(w, packed, stream=None):
    """packed (same shape and size as w [n, k]) = the tiled copy of the
    row-major weight matrix w, for the projections' w_layout=W_TILED."""
    _bf16(w, "w"), _bf16(packed, "packed")
    if w.dim() != 2 or packed.numel() != w.numel():
        raise ValueError("w must be [n, k] and packed the same size")
    n, k = w.shape
    st = lib().moetail_pack_weights(_ptr(w), n, k, _ptr(packed), _stream(stream))
    _check(st, "moetail_pack_weights")


def pack_weights(w, stream=None):
    """A new tensor shaped like w holding its tiled copy."""
    packed = torch.empty_like(w)
    moetail_pack_weights(w, packed, stream=stream)
    return packed


def new_workspace(op: int, b: int, dim0: int, dim1: int = 0, dim2: int = 0, device="cuda"):
    """A device byte tensor sized for one call of `op` (None when none is needed)."""
    n = workspace_bytes(op, b, dim0, dim1, dim2)
    if n == 0:
        return None
    # the caching allocator hands out blocks aligned to at least 512 bytes
    return torch.empty(n, dtype=torch.uint8, device=device)
