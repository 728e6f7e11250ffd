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
OP_PROJECTION = 5
OP_GATE_UP = 6
W_ROWS, W_TILED = 0, 1  # weight layouts of the projections

PROJ_UPPROJ, PROJ_GATEUP, PROJ_DOWN = 0, 1, 2  # projection kinds for set_projection_tuning

_CALLS = ("moetail_finalize", "moetail_tp_finalize", "moetail_combine_norm_upproj",
          "moetail_shared_expert", "moetail_tail", "moetail_decode_tail", "moetail_pack_weights",
          "moetail_set_projection_tuning", "moetail_decode_tail_noalloc",
          "moetail_projection_partials", "moetail_gate_up")
ENTRY_POINTS = _CALLS + ("moetail_workspace_bytes", "moetail_status_string",
                         "moetail_plan_cache_stats", "moetail_set_tp_wait_limit")


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
        L.moetail_set_projection_tuning.argtypes = [I32] * 7
        L.moetail_plan_cache_stats.argtypes = [ctypes.POINTER(ctypes.c_uint64)] * 2
        L.moetail_plan_cache_stats.restype = None
        L.moetail_set_tp_wait_limit.argtypes = [I64]
        L.moetail_set_tp_wait_limit.restype = None
        L.moetail_decode_tail_noalloc.argtypes = L.moetail_decode_tail.argtypes[:-3] + [P]
        L.moetail_projection_partials.argtypes = [I32, P, P, I32, I32, P, I32, I32, P, SZ, P]
        L.moetail_gate_up.argtypes = [P, I32, I32, P, P, I32, P, P, I32, P, F, I32, P, I32, P, SZ,
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


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def _expect(t, name, shape, dtypes=_BF16, optional=False):
    """Shape and dtype of one argument, checked before anything reaches the
    library (the C ABI takes bare pointers and cannot check sizes)."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}; expected one of {dtypes}")


def _same_device(*tensors):
    """The one device every given tensor is on."""
    devs = {t.device for t in tensors if t is not None}
    if len(devs) != 1:
        raise ValueError(f"all tensors must be on one device, got {sorted(map(str, devs))}")
    return devs.pop()


def _ws(workspace):
    """(pointer, bytes) of an optional workspace tensor (any dtype)."""
    if workspace is None:
        return None, 0
    return _ptr(workspace), workspace.numel() * workspace.element_size()


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


def _weights(w):
    if w.dtype == torch.float32:
        return F32
    if w.dtype in _BF16:
        return BF16
    raise TypeError("route weights must be float32 or bfloat16")


_W_DTYPES = (torch.float32,) + _BF16


def _stream(stream, device=None):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def set_projection_tuning(kind: int, splits: int = 0, waves: int = 0, blocks: int = 0,
                          tiles_per_unit: int = 0, prefetch: int = 0, passes: int = 0) -> None:
    """Plan overrides of one projection kind (PROJ_UPPROJ, PROJ_GATEUP,
    PROJ_DOWN) for measurement runs and tests; all zeros restores the
    library's plan.  An override changes the K slices and so the bits of
    the projection's outputs."""
    _check(lib().moetail_set_projection_tuning(int(kind), int(splits), int(waves), int(blocks),
                                               int(tiles_per_unit), int(prefetch), int(passes)),
           "moetail_set_projection_tuning")


class projection_tuning:
    """Context manager: {kind: dict(splits=.., waves=.., ...)} overrides
    inside the block, the library's plans again after it."""

    def __init__(self, overrides):
        self.overrides = overrides

    def __enter__(self):
        for kind in (PROJ_UPPROJ, PROJ_GATEUP, PROJ_DOWN):
            set_projection_tuning(kind, **self.overrides.get(kind, {}))
        return self

    def __exit__(self, *exc):
        for kind in (PROJ_UPPROJ, PROJ_GATEUP, PROJ_DOWN):
            set_projection_tuning(kind)
        return False


def set_tp_wait_limit(ticks: int = 2000000) -> None:
    """The one-pass expert-TP finalize's wait limit (100 MHz ticks; < 0: no
    wait, each block forms its partner's totals itself)."""
    lib().moetail_set_tp_wait_limit(int(ticks))


def plan_cache_stats():
    """(plan searches, plan-cache hits) so far in this process."""
    a, b = ctypes.c_uint64(0), ctypes.c_uint64(0)
    lib().moetail_plan_cache_stats(ctypes.byref(a), ctypes.byref(b))
    return a.value, b.value


def _check(status, where):
    if status != OK:
        raise MoetailError(status, where)


def workspace_bytes(op: int, b: int, dim0: int, dim1: int = 0, dim2: int = 0) -> int:
    return int(lib().moetail_workspace_bytes(op, b, dim0, dim1, dim2))


def _index(idx, name, shape):
    _expect(idx, name, shape, (torch.int32,))


def moetail_finalize(rows, permuted_idx, route_w, gamma, gain_center, eps, weight_before_norm,
                     partials=None, out=None, stream=None):
    """rows [tp, R, P], permuted_idx [tp, b, K], route_w [b, K], gamma [P]
    (or None with NO_NORM); writes partials [tp, b, P] and/or out [b, P].
    weight_before_norm: a bool, or a norm mode (NORM_GAIN_AFTER,
    NORM_GAIN_FIRST, NO_NORM)."""
    if rows.dim() != 3 or permuted_idx.dim() != 3:
        raise ValueError("rows must be [tp, R, P] and permuted_idx [tp, b, K]")
    tp, R, P = rows.shape
    _, b, K = permuted_idx.shape
    _expect(rows, "rows", (tp, R, P))
    _index(permuted_idx, "permuted_idx", (tp, b, K))
    _expect(route_w, "route_w", (b, K), _W_DTYPES)
    _expect(gamma, "gamma", (P,), optional=True)
    _expect(partials, "partials", (tp, b, P), optional=True)
    _expect(out, "out", (b, P), optional=True)
    dev = _same_device(rows, permuted_idx, route_w, gamma, partials, out)
    st = lib().moetail_finalize(_ptr(rows), R, _ptr(permuted_idx), _ptr(route_w),
                                _weights(route_w), _ptr(gamma), float(gain_center), float(eps),
                                int(weight_before_norm), b, K, P, tp, _ptr(partials),
                                _ptr(out), _stream(stream, dev))
    _check(st, "moetail_finalize")


def moetail_tp_finalize(kpartials, permuted_idx, route_w, gamma, gain_center, eps,
                        weight_before_norm, out, workspace=None, stream=None):
    """kpartials [tp, num_rows, P], permuted_idx [b, K], route_w [b, K],
    gamma [P]; writes out [b, P].  weight_before_norm: a bool (the norm
    modes NORM_GAIN_AFTER / NORM_GAIN_FIRST; NO_NORM is refused by the
    library).  workspace: at least workspace_bytes(OP_TP_FINALIZE, b, K, P)
    bytes."""
    if kpartials.dim() != 3 or permuted_idx.dim() != 2:
        raise ValueError("kpartials must be [tp, num_rows, P] and permuted_idx [b, K]")
    tp, num_rows, P = kpartials.shape
    b, K = permuted_idx.shape
    _expect(kpartials, "kpartials", (tp, num_rows, P))
    _index(permuted_idx, "permuted_idx", (b, K))
    _expect(route_w, "route_w", (b, K), _W_DTYPES)
    _expect(gamma, "gamma", (P,))
    _expect(out, "out", (b, P))
    dev = _same_device(kpartials, permuted_idx, route_w, gamma, out, workspace)
    ws, wsb = _ws(workspace)
    st = lib().moetail_tp_finalize(_ptr(kpartials), num_rows, _ptr(permuted_idx),
                                   _ptr(route_w), _weights(route_w), _ptr(gamma),
                                   float(gain_center), float(eps), int(weight_before_norm),
                                   b, K, P, tp, _ptr(out), ws, wsb, _stream(stream, dev))
    _check(st, "moetail_tp_finalize")


def moetail_combine_norm_upproj(latent_partials, gamma, eps, w_up, out, rs=None, normed=None,
                                workspace=None, stream=None, w_layout=W_ROWS):
    """latent_partials [tp, b, L], gamma [L], w_up [N, L] (row-major, or its
    pack_weights copy with w_layout=W_TILED), rs [b, N] or None; writes out
    [b, N] and normed [b, L] when given.  workspace: a device tensor of at
    least workspace_bytes(OP_COMBINE_NORM_UPPROJ, b, L, N, tp) bytes."""
    if latent_partials.dim() != 3 or w_up.dim() != 2:
        raise ValueError("latent_partials must be [tp, b, L] and w_up [N, L]")
    tp, b, L = latent_partials.shape
    N = w_up.shape[0]
    _expect(latent_partials, "latent_partials", (tp, b, L))
    _expect(gamma, "gamma", (L,))
    _expect(w_up, "w_up", (N, L))
    _expect(out, "out", (b, N))
    _expect(rs, "rs", (b, N), optional=True)
    _expect(normed, "normed", (b, L), optional=True)
    dev = _same_device(latent_partials, gamma, w_up, out, rs, normed, workspace)
    ws, wsb = _ws(workspace)
    st = lib().moetail_combine_norm_upproj(_ptr(latent_partials), tp, _ptr(gamma), float(eps),
                                           _ptr(w_up), N, _ptr(rs), b, L, _ptr(normed),
                                           _ptr(out), int(w_layout), ws, wsb,
                                           _stream(stream, dev))
    _check(st, "moetail_combine_norm_upproj")


def moetail_shared_expert(x, w_gate, w_up, w_down, rs, h=None, workspace=None, stream=None,
                          w_layout=W_ROWS):
    """x [b, H], w_gate/w_up [I, H], w_down [H, I] (all row-major, or all
    pack_weights copies with w_layout=W_TILED); writes rs [b, H] and h
    [b, I] when given.  workspace: at least
    workspace_bytes(OP_SHARED_EXPERT, b, H, I) bytes."""
    if x.dim() != 2 or w_gate.dim() != 2:
        raise ValueError("x must be [b, H] and w_gate [I, H]")
    b, H = x.shape
    I = w_gate.shape[0]
    _expect(x, "x", (b, H))
    for t, n in ((w_gate, "w_gate"), (w_up, "w_up")):
        _expect(t, n, (I, H))
    _expect(w_down, "w_down", (H, I))
    _expect(rs, "rs", (b, H))
    _expect(h, "h", (b, I), optional=True)
    dev = _same_device(x, w_gate, w_up, w_down, rs, h, workspace)
    ws, wsb = _ws(workspace)
    st = lib().moetail_shared_expert(_ptr(x), b, H, _ptr(w_gate), _ptr(w_up), I, _ptr(w_down),
                                     _ptr(h), _ptr(rs), int(w_layout), ws, wsb,
                                     _stream(stream, dev))
    _check(st, "moetail_shared_expert")


def moetail_gate_up(x, w_gate, w_up, h, latent_partials=None, gamma=None, eps=1e-6, normed=None,
                    workspace=None, stream=None, w_layout=W_ROWS):
    """x [b, H], w_gate/w_up [I, H] (row-major, or pack_weights copies with
    w_layout=W_TILED); writes h [b, I] in one launch, and with
    latent_partials [tp, b, L] and gamma [L] also normed [b, L] (the latent
    combine + RMSNorm) in the same launch.  workspace: at least
    workspace_bytes(OP_GATE_UP, b, H, I) bytes, zero before its first use
    (new_workspace)."""
    if x.dim() != 2 or w_gate.dim() != 2:
        raise ValueError("x must be [b, H] and w_gate [I, H]")
    b, H = x.shape
    I = w_gate.shape[0]
    _expect(x, "x", (b, H))
    for t, n in ((w_gate, "w_gate"), (w_up, "w_up")):
        _expect(t, n, (I, H))
    _expect(h, "h", (b, I))
    tp = L = 0
    if latent_partials is not None:
        if latent_partials.dim() != 3:
            raise ValueError("latent_partials must be [tp, b, L]")
        tp, _, L = latent_partials.shape
        _expect(latent_partials, "latent_partials", (tp, b, L))
        _expect(gamma, "gamma", (L,))
        _expect(normed, "normed", (b, L))
    elif normed is not None or gamma is not None:
        raise ValueError("gamma and normed go with latent_partials")
    dev = _same_device(x, w_gate, w_up, h, latent_partials, gamma, normed, workspace)
    ws, wsb = _ws(workspace)
    st = lib().moetail_gate_up(_ptr(x), b, H, _ptr(w_gate), _ptr(w_up), I, _ptr(h),
                               _ptr(latent_partials), tp, _ptr(gamma), float(eps), L,
                               _ptr(normed), int(w_layout), ws, wsb, _stream(stream, dev))
    _check(st, "moetail_gate_up")


def moetail_projection_partials(kind, w0, w1, x, partials, stream=None, w_layout=W_ROWS):
    """One projection's split-K stage: kind PROJ_GATEUP with w0 = w_gate and
    w1 = w_up [N/2, K] each (N = 2 I), or PROJ_DOWN / PROJ_UPPROJ with w0
    [N, K] and w1 None; x [b, K].  Writes the FP32 partial sums into
    partials (a float32 tensor of at least workspace_bytes(OP_PROJECTION, b,
    N, K, kind) bytes) in the layout the C header gives."""
    if x.dim() != 2 or w0.dim() != 2:
        raise ValueError("x must be [b, K] and w0 [rows, K]")
    b, K = x.shape
    rows = w0.shape[0]
    if kind == PROJ_GATEUP:
        _expect(w1, "w1", (rows, K))
        N = 2 * rows
    else:
        if w1 is not None:
            raise ValueError("w1 is the gate/up projection's second matrix only")
        N = rows
    _expect(w0, "w0", (rows, K))
    if not isinstance(partials, torch.Tensor) or partials.dtype != torch.float32:
        raise TypeError("partials must be a float32 tensor")
    dev = _same_device(w0, w1, x, partials)
    st = lib().moetail_projection_partials(int(kind), _ptr(w0), _ptr(w1), N, K, _ptr(x), b,
                                           int(w_layout), _ptr(partials),
                                           partials.numel() * 4, _stream(stream, dev))
    _check(st, "moetail_projection_partials")


def _tail_shapes(latent_partials, gamma, w_up, x, w_gate, w_up_shared, w_down, out, rs, normed,
                 h):
    if latent_partials.dim() != 3 or x.dim() != 2 or w_gate.dim() != 2:
        raise ValueError("latent_partials must be [tp, b, L], x [b, H] and w_gate [I, H]")
    tp, b, L = latent_partials.shape
    H = x.shape[1]
    I = w_gate.shape[0]
    _expect(latent_partials, "latent_partials", (tp, b, L))
    _expect(gamma, "gamma", (L,))
    _expect(w_up, "w_up", (H, L))
    _expect(x, "x", (b, H))
    _expect(w_gate, "w_gate", (I, H))
    _expect(w_up_shared, "w_up_shared", (I, H))
    _expect(w_down, "w_down", (H, I))
    _expect(out, "out", (b, H))
    _expect(rs, "rs", (b, H), optional=True)
    _expect(normed, "normed", (b, L), optional=True)
    _expect(h, "h", (b, I), optional=True)
    return tp, b, L, H, I


def moetail_tail(latent_partials, gamma, eps, w_up, x, w_gate, w_up_shared, w_down, out,
                 rs=None, normed=None, h=None, workspace=None, stream=None, w_layout=W_ROWS):
    """The tail after the finalize in one call: rs = shared expert of x,
    out = up projection of the normed rank-combined latent + rs.
    latent_partials [tp, b, L], gamma [L], w_up [H, L]; x [b, H], w_gate and
    w_up_shared [I, H], w_down [H, I]; writes out [b, H] and rs [b, H],
    normed [b, L], h [b, I] when given.  The four weights are all row-major,
    or all pack_weights copies with w_layout=W_TILED.  workspace: at least
    workspace_bytes(OP_TAIL, b, L, H, I) bytes."""
    tp, b, L, H, I = _tail_shapes(latent_partials, gamma, w_up, x, w_gate, w_up_shared, w_down,
                                  out, rs, normed, h)
    dev = _same_device(latent_partials, gamma, w_up, x, w_gate, w_up_shared, w_down, out, rs,
                       normed, h, workspace)
    ws, wsb = _ws(workspace)
    st = lib().moetail_tail(_ptr(latent_partials), tp, _ptr(gamma), float(eps), _ptr(w_up), L,
                            _ptr(x), _ptr(w_gate), _ptr(w_up_shared), _ptr(w_down), H, I, b,
                            _ptr(out), _ptr(rs), _ptr(normed), _ptr(h), int(w_layout), ws,
                            wsb, _stream(stream, dev))
    _check(st, "moetail_tail")


def moetail_decode_tail(rows, permuted_idx, route_w, fin_gamma, gain_center, fin_eps,
                        weight_before_norm, latent_partials, gamma, eps, w_up, x, w_gate,
                        w_up_shared, w_down, out, rs=None, normed=None, h=None, workspace=None,
                        stream=None, w_layout=W_ROWS):
    """The whole tail in one call: latent_partials [tp, b, L] = the EP
    finalize of rows [tp, R, L] (as moetail_finalize with partials only),
    then out [b, H] = moetail_tail(latent_partials, ...).  workspace: at
    least workspace_bytes(OP_TAIL, b, L, H, I) bytes."""
    tp, b, L, H, I = _tail_shapes(latent_partials, gamma, w_up, x, w_gate, w_up_shared, w_down,
                                  out, rs, normed, h)
    if rows.dim() != 3 or permuted_idx.dim() != 3:
        raise ValueError("rows must be [tp, R, L] and permuted_idx [tp, b, K]")
    R = rows.shape[1]
    K = permuted_idx.shape[2]
    _expect(rows, "rows", (tp, R, L))
    _index(permuted_idx, "permuted_idx", (tp, b, K))
    _expect(route_w, "route_w", (b, K), _W_DTYPES)
    _expect(fin_gamma, "fin_gamma", (L,), optional=True)
    dev = _same_device(rows, permuted_idx, route_w, fin_gamma, latent_partials, gamma, w_up, x,
                       w_gate, w_up_shared, w_down, out, rs, normed, h, workspace)
    ws, wsb = _ws(workspace)
    st = lib().moetail_decode_tail(_ptr(rows), R, _ptr(permuted_idx), _ptr(route_w),
                                   _weights(route_w), _ptr(fin_gamma), float(gain_center),
                                   float(fin_eps), int(weight_before_norm), K,
                                   _ptr(latent_partials), tp, _ptr(gamma), float(eps),
                                   _ptr(w_up), L, _ptr(x), _ptr(w_gate), _ptr(w_up_shared),
                                   _ptr(w_down), H, I, b, _ptr(out), _ptr(rs), _ptr(normed),
                                   _ptr(h), int(w_layout), ws, wsb, _stream(stream, dev))
    _check(st, "moetail_decode_tail")


NOALLOC_SCRATCH_BYTES = 24 << 20  # the library's static scratch per GPU


def moetail_decode_tail_noalloc(rows, permuted_idx, route_w, fin_gamma, gain_center, fin_eps,
                                weight_before_norm, latent_partials, gamma, eps, w_up, x,
                                w_gate, w_up_shared, w_down, out, rs=None, normed=None, h=None,
                                stream=None, w_layout=W_ROWS):
    """moetail_decode_tail without a workspace: the library's static scratch
    (NOALLOC_SCRATCH_BYTES per GPU) serves instead, and the call allocates
    nothing.  Calls on one GPU share that scratch and must not overlap."""
    tp, b, L, H, I = _tail_shapes(latent_partials, gamma, w_up, x, w_gate, w_up_shared, w_down,
                                  out, rs, normed, h)
    if rows.dim() != 3 or permuted_idx.dim() != 3:
        raise ValueError("rows must be [tp, R, L] and permuted_idx [tp, b, K]")
    R = rows.shape[1]
    K = permuted_idx.shape[2]
    _expect(rows, "rows", (tp, R, L))
    _index(permuted_idx, "permuted_idx", (tp, b, K))
    _expect(route_w, "route_w", (b, K), _W_DTYPES)
    _expect(fin_gamma, "fin_gamma", (L,), optional=True)
    dev = _same_device(rows, permuted_idx, route_w, fin_gamma, latent_partials, gamma, w_up, x,
                       w_gate, w_up_shared, w_down, out, rs, normed, h)
    st = lib().moetail_decode_tail_noalloc(
        _ptr(rows), R, _ptr(permuted_idx), _ptr(route_w), _weights(route_w), _ptr(fin_gamma),
        float(gain_center), float(fin_eps), int(weight_before_norm), K, _ptr(latent_partials),
        tp, _ptr(gamma), float(eps), _ptr(w_up), L, _ptr(x), _ptr(w_gate), _ptr(w_up_shared),
        _ptr(w_down), H, I, b, _ptr(out), _ptr(rs), _ptr(normed), _ptr(h), int(w_layout),
        _stream(stream, dev))
    _check(st, "moetail_decode_tail_noalloc")


def moetail_pack_weights(w, packed, stream=None):
    """packed (same shape and size as w [n, k]) = the tiled copy of the
    row-major weight matrix w, for the projections' w_layout=W_TILED."""
    if w.dim() != 2:
        raise ValueError("w must be [n, k]")
    n, k = w.shape
    _expect(w, "w", (n, k))
    _expect(packed, "packed", (n, k))
    dev = _same_device(w, packed)
    st = lib().moetail_pack_weights(_ptr(w), n, k, _ptr(packed), _stream(stream, dev))
    _check(st, "moetail_pack_weights")


def pack_weights(w, stream=None):
    """A new tensor shaped like w holding its tiled copy."""
    packed = torch.empty_like(w)
    moetail_pack_weights(w, packed, stream=stream)
    return packed


def new_workspace(op: int, b: int, dim0: int, dim1: int = 0, dim2: int = 0, device="cuda"):
    """A device byte tensor sized for one call of `op` (None when none is
    needed), zeroed (the expert-TP finalize's flags and the tail's
    output-tile counters must be zero before the first use; every call
    leaves them so)."""
    n = workspace_bytes(op, b, dim0, dim1, dim2)
    if n == 0:
        return None
    # the caching allocator hands out blocks aligned to at least 512 bytes
    return torch.zeros(n, dtype=torch.uint8, device=device)
