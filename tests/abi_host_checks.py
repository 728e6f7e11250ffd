"""Host-side checks of the C ABI (CPU only: no call here reaches a kernel).

The library must load, export every entry point include/moetail.h declares,
and refuse bad arguments with the documented status before it touches a
device.  Pointers below are fake aligned addresses: every call either fails
validation or has b == 0, so nothing is dereferenced or launched.

tests/test_abi.py runs this file in a child process that sees no GPU
(HIP_VISIBLE_DEVICES empty), so that a validation regression fails here on
the host instead of launching a kernel on a fake address.
"""
from __future__ import annotations

import ctypes
import os
import re
import shutil
import subprocess

import pytest

import expert_finalize_rmsnorm_amd as mt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moetail.h")

A = 0x10000  # a 16-byte aligned fake device address (never dereferenced)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moetail_\w+)\s*\(", text)))


def test_header_declares_the_calls():
    names = declared_functions()
    for n in ("moetail_finalize", "moetail_tp_finalize", "moetail_combine_norm_upproj",
              "moetail_shared_expert", "moetail_tail", "moetail_decode_tail",
              "moetail_pack_weights", "moetail_workspace_bytes", "moetail_status_string"):
        assert n in names
    assert set(names) == set(mt.ENTRY_POINTS)


def test_library_exports_every_declared_symbol():
    lib = mt.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_header_has_no_torch_types():
    text = open(HEADER).read()
    assert "torch" not in text.lower().replace("no torch", "")
    assert "at::" not in text and "Tensor" not in text


def test_status_strings():
    for st in (mt.OK, mt.EINVAL, mt.EUNSUPPORTED, mt.EWORKSPACE, mt.EHIP):
        assert mt.status_string(st)
    assert mt.status_string(12345) == "unknown status"


def _fin(**kw):
    a = dict(rows=A, R=16, idx=A, w=A, wdt=mt.F32, gamma=A, gc=1.0, eps=1e-6, wbn=1, b=4, K=4,
             P=512, tp=2, partials=A, out=A)
    a.update(kw)
    return mt.lib().moetail_finalize(a["rows"], a["R"], a["idx"], a["w"], a["wdt"], a["gamma"],
                                     a["gc"], a["eps"], a["wbn"], a["b"], a["K"], a["P"], a["tp"],
                                     a["partials"], a["out"], None)


def test_finalize_validation():
    assert _fin(b=0) == mt.OK  # b == 0: nothing to do, nothing launched
    assert _fin(b=0, rows=None, w=None, eps=-1.0) == mt.OK  # returns before any check
    assert _fin(rows=None) == mt.EINVAL
    assert _fin(rows=A + 8) == mt.EINVAL  # misaligned
    assert _fin(idx=None) == mt.EINVAL
    assert _fin(idx=A + 2) == mt.EINVAL
    assert _fin(w=None) == mt.EINVAL
    assert _fin(w=A + 2) == mt.EINVAL  # FP32 weights need 4-byte alignment
    assert _fin(w=A + 2, wdt=mt.BF16, b=0) == mt.OK
    assert _fin(wdt=7) == mt.EINVAL
    assert _fin(gamma=None) == mt.EINVAL
    assert _fin(partials=None, out=None) == mt.EINVAL
    assert _fin(eps=-1.0) == mt.EINVAL
    assert _fin(eps=float("nan")) == mt.EINVAL
    assert _fin(eps=float("inf")) == mt.EINVAL
    assert _fin(gc=float("inf")) == mt.EINVAL
    assert _fin(K=0) == mt.EINVAL
    assert _fin(tp=0) == mt.EINVAL
    assert _fin(b=-1) == mt.EINVAL
    assert _fin(R=0) == mt.EINVAL
    assert _fin(P=516) == mt.EUNSUPPORTED  # P % 8
    assert _fin(P=8200) == mt.EUNSUPPORTED
    assert _fin(K=33) == mt.EUNSUPPORTED
    assert _fin(tp=33) == mt.EUNSUPPORTED
    assert _fin(b=70000) == mt.EUNSUPPORTED
    assert _fin(partials=None, tp=32, P=8192, b=0) == mt.OK


def _tp(ws=A, wsb=1 << 30, **kw):
    a = dict(kp=A, n=64, idx=A, w=A, wdt=mt.F32, gamma=A, gc=0.0, eps=1e-6, wbn=0, b=4, K=16,
             P=7168, tp=8, out=A)
    a.update(kw)
    return mt.lib().moetail_tp_finalize(a["kp"], a["n"], a["idx"], a["w"], a["wdt"], a["gamma"],
                                        a["gc"], a["eps"], a["wbn"], a["b"], a["K"], a["P"],
                                        a["tp"], a["out"], ws, wsb, None)


def test_tp_finalize_validation():
    assert _tp(b=0) == mt.OK
    assert _tp(kp=None) == mt.EINVAL
    assert _tp(out=None) == mt.EINVAL
    assert _tp(out=A + 4) == mt.EINVAL
    assert _tp(n=0) == mt.EINVAL
    assert _tp(P=7170) == mt.EUNSUPPORTED
    assert _tp(K=40) == mt.EUNSUPPORTED
    assert _tp(ws=None, wsb=0) == mt.EWORKSPACE
    # tp = 8: the generations [4] and tagged block totals [4][16][14] (7424 B)
    assert _tp(wsb=256 + 7168 - 1) == mt.EWORKSPACE
    # tp = 12: the two-pass path's rows and totals as well
    assert _tp(tp=12, wsb=256 + 7168) == mt.EWORKSPACE
    assert _tp(tp=12, wsb=256 + 7168 + 4 * 16 * 7168 * 2 + 3584 - 1) == mt.EWORKSPACE
    assert _tp(ws=A + 128) == mt.EWORKSPACE


def _up(ws=A, wsb=1 << 30, **kw):
    a = dict(lat=A, tp=8, gamma=A, eps=1e-6, w=A, N=7168, rs=None, b=32, L=3584, normed=None,
             out=A, lay=mt.W_ROWS)
    a.update(kw)
    return mt.lib().moetail_combine_norm_upproj(a["lat"], a["tp"], a["gamma"], a["eps"], a["w"],
                                                a["N"], a["rs"], a["b"], a["L"], a["normed"],
                                                a["out"], a["lay"], ws, wsb, None)


def test_upproj_validation():
    assert _up(b=0) == mt.OK
    assert _up(out=None) == mt.EINVAL
    assert _up(w=None) == mt.EINVAL
    assert _up(rs=A + 8) == mt.EINVAL
    assert _up(L=3600) == mt.EUNSUPPORTED
    assert _up(N=7200) == mt.EUNSUPPORTED
    assert _up(b=129) == mt.EUNSUPPORTED
    assert _up(ws=None, wsb=0) == mt.EWORKSPACE  # y needs a home when normed is NULL
    assert _up(wsb=16) == mt.EWORKSPACE
    assert _up(ws=A + 16) == mt.EWORKSPACE  # 256-byte alignment
    assert _up(lay=2) == mt.EINVAL
    assert _up(lay=-1) == mt.EINVAL
    assert _up(lay=2, b=0) == mt.OK


def _sh(ws=A, wsb=1 << 30, **kw):
    a = dict(x=A, b=32, H=7168, wg=A, wu=A, I=6144, wd=A, h=None, rs=A, lay=mt.W_TILED)
    a.update(kw)
    return mt.lib().moetail_shared_expert(a["x"], a["b"], a["H"], a["wg"], a["wu"], a["I"],
                                          a["wd"], a["h"], a["rs"], a["lay"], ws, wsb, None)


def test_shared_validation():
    assert _sh(b=0) == mt.OK
    assert _sh(b=0, x=None, ws=None, wsb=0) == mt.OK  # b == 0 before any check
    assert _sh(x=None) == mt.EINVAL
    assert _sh(rs=None) == mt.EINVAL
    assert _sh(wd=A + 2) == mt.EINVAL
    assert _sh(H=7160) == mt.EUNSUPPORTED
    assert _sh(I=6100) == mt.EUNSUPPORTED
    assert _sh(b=200) == mt.EUNSUPPORTED
    assert _sh(ws=None, wsb=0) == mt.EWORKSPACE
    assert _sh(lay=5) == mt.EINVAL


def _gu(ws=A, wsb=1 << 30, **kw):
    a = dict(x=A, b=64, H=7168, wg=A, wu=A, I=6144, h=A, lat=A, tp=8, g=A, eps=1e-6, L=3584,
             y=A, lay=mt.W_TILED)
    a.update(kw)
    return mt.lib().moetail_gate_up(a["x"], a["b"], a["H"], a["wg"], a["wu"], a["I"], a["h"],
                                    a["lat"], a["tp"], a["g"], a["eps"], a["L"], a["y"],
                                    a["lay"], ws, wsb, None)


def test_gate_up_validation():
    assert _gu(b=0) == mt.OK
    assert _gu(b=0, x=None, ws=None, wsb=0) == mt.OK  # b == 0 before any check
    assert _gu(x=None) == mt.EINVAL
    assert _gu(h=None) == mt.EINVAL
    assert _gu(wu=A + 2) == mt.EINVAL
    assert _gu(lay=3) == mt.EINVAL
    assert _gu(H=7160) == mt.EUNSUPPORTED
    assert _gu(I=6100) == mt.EUNSUPPORTED
    assert _gu(b=129) == mt.EUNSUPPORTED
    # y's arguments are checked only with latent partials
    assert _gu(g=None) == mt.EINVAL
    assert _gu(y=A + 8) == mt.EINVAL
    assert _gu(eps=-1.0) == mt.EINVAL
    assert _gu(tp=0) == mt.EINVAL
    assert _gu(L=3600) == mt.EUNSUPPORTED
    assert _gu(tp=33) == mt.EUNSUPPORTED
    assert _gu(lat=None, g=None, y=None, tp=0, L=0, eps=float("nan"), ws=None,
               wsb=0) == mt.EWORKSPACE
    need = mt.workspace_bytes(mt.OP_GATE_UP, 64, 7168, 6144)
    assert _gu(wsb=need - 1) == mt.EWORKSPACE
    assert _gu(ws=A + 16) == mt.EWORKSPACE  # 256-byte aligned


@pytest.mark.parametrize("b", [1, 32, 64, 128])
def test_gate_up_workspace(b):
    """The h tiles' counters (I/16 words, rounded to 256 bytes), then the
    gate/up partials of the shared expert's plan."""
    gu = mt.workspace_bytes(mt.OP_GATE_UP, b, 7168, 6144)
    part = mt.workspace_bytes(mt.OP_PROJECTION, b, 12288, 7168, mt.PROJ_GATEUP)
    assert gu == (6144 // 16 * 4 + 255) // 256 * 256 + part
    assert mt.workspace_bytes(mt.OP_GATE_UP, b, 7160, 6144) == 0
    assert mt.workspace_bytes(mt.OP_GATE_UP, b, 7168, 6100) == 0


def _proj(**kw):
    a = dict(kind=mt.PROJ_GATEUP, w0=A, w1=A, N=12288, K=7168, x=A, b=64, lay=mt.W_TILED,
             part=A, pb=1 << 31)
    a.update(kw)
    return mt.lib().moetail_projection_partials(a["kind"], a["w0"], a["w1"], a["N"], a["K"],
                                                a["x"], a["b"], a["lay"], a["part"], a["pb"],
                                                None)


def test_projection_partials_validation():
    assert _proj(b=0) == mt.OK
    assert _proj(kind=3) == mt.EINVAL
    assert _proj(kind=-1, b=0) == mt.EINVAL  # the kind first
    assert _proj(w1=None) == mt.EINVAL       # gate/up takes both matrices
    assert _proj(kind=mt.PROJ_DOWN, N=7168, K=6144) == mt.EINVAL  # ... the others one
    assert _proj(x=A + 2) == mt.EINVAL
    assert _proj(part=A + 16) == mt.EINVAL   # 256-byte aligned partials
    assert _proj(lay=7) == mt.EINVAL
    assert _proj(N=12304) == mt.EUNSUPPORTED  # gate/up rows: two halves of whole tiles
    assert _proj(K=7176) == mt.EUNSUPPORTED
    assert _proj(b=129) == mt.EUNSUPPORTED
    need = mt.workspace_bytes(mt.OP_PROJECTION, 64, 12288, 7168, mt.PROJ_GATEUP)
    assert _proj(pb=need - 1) == mt.EWORKSPACE


@pytest.mark.parametrize("b", [1, 16, 64, 128])
def test_projection_partial_bytes(b):
    """The partials are splits x N rows x the padded tokens in FP32, with the
    splits of the composite calls' plans."""
    T = 16 * next(n for n in (1, 2, 4, 8) if b <= 16 * n)
    for kind, N, K in ((mt.PROJ_GATEUP, 12288, 7168), (mt.PROJ_DOWN, 7168, 6144),
                       (mt.PROJ_UPPROJ, 7168, 3584)):
        n = mt.workspace_bytes(mt.OP_PROJECTION, b, N, K, kind)
        assert n > 0 and n % (N * T * 4) == 0, (kind, n)
        assert 1 <= n // (N * T * 4) <= 64
    assert mt.workspace_bytes(mt.OP_PROJECTION, b, 12288, 7168, 7) == 0
    assert mt.workspace_bytes(mt.OP_PROJECTION, b, 12304, 7168, mt.PROJ_GATEUP) == 0


def _tail(ws=A, wsb=1 << 31, **kw):
    a = dict(lat=A, tp=8, gamma=A, eps=1e-6, wup=A, L=3584, x=A, wg=A, wu=A, wd=A, H=7168,
             I=6144, b=64, out=A, rs=None, normed=None, h=None, lay=mt.W_TILED)
    a.update(kw)
    return mt.lib().moetail_tail(a["lat"], a["tp"], a["gamma"], a["eps"], a["wup"], a["L"],
                                 a["x"], a["wg"], a["wu"], a["wd"], a["H"], a["I"], a["b"],
                                 a["out"], a["rs"], a["normed"], a["h"], a["lay"], ws, wsb, None)


def test_finalize_norm_mode_validation():
    lib = mt.lib()
    for mode in (-1, 3):
        assert lib.moetail_finalize(A, 8, A, A, mt.F32, A, 1.0, 1e-6, mode, 4, 16, 3584, 8, A, A,
                                    None) == mt.EINVAL
    # the expert-TP finalize takes the two normalizing modes only
    assert lib.moetail_tp_finalize(A, 64, A, A, mt.F32, A, 1.0, 1e-6, mt.NO_NORM, 4, 16, 3584, 8,
                                   A, A, 1 << 30, None) == mt.EINVAL
    # gamma may be NULL only without a norm (checked before anything launches)
    assert lib.moetail_finalize(A, 8, A, A, mt.F32, None, 1.0, 1e-6, mt.NORM_GAIN_FIRST, 4, 16,
                                3584, 8, A, A, None) == mt.EINVAL


def test_tail_validation():
    # every case is refused before anything launches (the pointers are fake)
    assert _tail(b=0) == mt.OK
    assert _tail(b=0, lat=None, x=None, ws=None, wsb=0) == mt.OK  # b == 0 before any check
    assert _tail(out=None) == mt.EINVAL
    assert _tail(x=None) == mt.EINVAL
    assert _tail(wd=A + 2) == mt.EINVAL
    assert _tail(rs=A + 8) == mt.EINVAL
    assert _tail(eps=-1.0) == mt.EINVAL
    assert _tail(tp=0) == mt.EINVAL
    assert _tail(L=3600) == mt.EUNSUPPORTED
    assert _tail(H=7200) == mt.EUNSUPPORTED
    assert _tail(I=6100) == mt.EUNSUPPORTED
    assert _tail(tp=33) == mt.EUNSUPPORTED
    assert _tail(b=129) == mt.EUNSUPPORTED
    assert _tail(ws=None, wsb=0) == mt.EWORKSPACE
    assert _tail(wsb=16) == mt.EWORKSPACE
    assert _tail(ws=A + 16) == mt.EWORKSPACE
    assert _tail(lay=7) == mt.EINVAL


def test_pack_weights_validation():
    lib = mt.lib()
    assert lib.moetail_pack_weights(A, 0, 7168, A, None) == mt.OK  # nothing to pack
    assert lib.moetail_pack_weights(None, 16, 32, A, None) == mt.EINVAL
    assert lib.moetail_pack_weights(A, 16, 32, None, None) == mt.EINVAL
    assert lib.moetail_pack_weights(A + 8, 16, 32, 1 << 30, None) == mt.EINVAL  # misaligned
    assert lib.moetail_pack_weights(A, -16, 32, 1 << 30, None) == mt.EINVAL
    assert lib.moetail_pack_weights(A, 16, 0, 1 << 30, None) == mt.EINVAL
    assert lib.moetail_pack_weights(A, 24, 32, 1 << 30, None) == mt.EUNSUPPORTED  # n % 16
    assert lib.moetail_pack_weights(A, 16, 48, 1 << 30, None) == mt.EUNSUPPORTED  # k % 32
    # the copy may not overlap its source
    assert lib.moetail_pack_weights(A, 16, 32, A + 512, None) == mt.EINVAL
    assert lib.moetail_pack_weights(A + 512, 16, 32, A, None) == mt.EINVAL


@pytest.mark.parametrize("b", [1, 8, 16, 32, 64, 128])
def test_workspace_query(b):
    tail = mt.workspace_bytes(mt.OP_TAIL, b, 3584, 7168, 6144)
    assert tail >= b * (3584 + 6144) * 2 and tail % 256 == 0
    assert mt.workspace_bytes(mt.OP_TAIL, b, 3600, 7168, 6144) == 0
    up = mt.workspace_bytes(mt.OP_COMBINE_NORM_UPPROJ, b, 3584, 7168, 8)
    assert up >= b * 3584 * 2 and up % 256 == 0
    sh = mt.workspace_bytes(mt.OP_SHARED_EXPERT, b, 7168, 6144)
    assert sh >= b * 6144 * 2 and sh % 256 == 0
    assert mt.workspace_bytes(mt.OP_FINALIZE, b, 3584) == 0
    # the token generations [b] and the tagged block totals [b][16][14] (8 B
    # each; 16 routes' slots for K <= 16, 32 above); for more than 8 ranks (or any tp, 0) also the rank-summed rows
    # [b][16][7168] BF16 and their 14 block totals a route in FP32
    def up256(n):
        return (n + 255) // 256 * 256
    sync = up256(b * 4) + up256(b * 16 * 14 * 8)
    two_pass = b * 16 * 7168 * 2 + up256(b * 16 * 14 * 4)
    assert mt.workspace_bytes(mt.OP_TP_FINALIZE, b, 16, 7168) == sync + two_pass
    assert mt.workspace_bytes(mt.OP_TP_FINALIZE, b, 16, 7168, 8) == sync
    assert mt.workspace_bytes(mt.OP_TP_FINALIZE, b, 16, 7168, 9) == sync + two_pass
    assert mt.workspace_bytes(mt.OP_TP_FINALIZE, b, 16, 7168, 33) == 0
    assert mt.workspace_bytes(99, b, 1, 1, 1) == 0
    assert mt.workspace_bytes(mt.OP_SHARED_EXPERT, 0, 7168, 6144) == 0


def _dt(ws=A, wsb=1 << 31, **kw):
    a = dict(rows=A, R=128, idx=A, w=A, wdt=mt.F32, fg=A, gc=1.0, feps=1e-6, wbn=1, K=16,
             lat=A, tp=8, gamma=A, eps=1e-6, wup=A, L=3584, x=A, wg=A, wu=A, wd=A, H=7168,
             I=6144, b=64, out=A, rs=None, normed=None, h=None, lay=mt.W_TILED)
    a.update(kw)
    return mt.lib().moetail_decode_tail(a["rows"], a["R"], a["idx"], a["w"], a["wdt"], a["fg"],
                                        a["gc"], a["feps"], a["wbn"], a["K"], a["lat"], a["tp"],
                                        a["gamma"], a["eps"], a["wup"], a["L"], a["x"], a["wg"],
                                        a["wu"], a["wd"], a["H"], a["I"], a["b"], a["out"],
                                        a["rs"], a["normed"], a["h"], a["lay"], ws, wsb, None)


def test_decode_tail_validation():
    """Every case is refused before anything launches (the pointers are fake)."""
    assert _dt(b=0) == mt.OK
    assert _dt(b=0, rows=None, x=None, ws=None, wsb=0) == mt.OK  # b == 0 before any check
    # the finalize's checks
    assert _dt(rows=None) == mt.EINVAL
    assert _dt(idx=A + 2) == mt.EINVAL
    assert _dt(w=None) == mt.EINVAL
    assert _dt(fg=None) == mt.EINVAL
    assert _dt(fg=None, wbn=mt.NO_NORM, ws=None, wsb=0) == mt.EWORKSPACE  # gamma may be NULL
    assert _dt(wbn=3) == mt.EINVAL
    assert _dt(feps=-1.0) == mt.EINVAL
    assert _dt(gc=float("nan")) == mt.EINVAL
    assert _dt(lat=None) == mt.EINVAL
    assert _dt(R=0) == mt.EINVAL
    assert _dt(K=33) == mt.EUNSUPPORTED
    assert _dt(tp=33) == mt.EUNSUPPORTED
    # the tail's checks
    assert _dt(out=None) == mt.EINVAL
    assert _dt(wd=A + 2) == mt.EINVAL
    assert _dt(eps=-1.0) == mt.EINVAL
    assert _dt(lay=2) == mt.EINVAL
    assert _dt(L=3600) == mt.EUNSUPPORTED
    assert _dt(H=7200) == mt.EUNSUPPORTED
    assert _dt(b=129) == mt.EUNSUPPORTED
    assert _dt(ws=None, wsb=0) == mt.EWORKSPACE
    assert _dt(ws=A + 16) == mt.EWORKSPACE


def test_no_device_visible():
    """These checks run where no kernel can launch."""
    assert os.environ.get("HIP_VISIBLE_DEVICES", None) == ""


def test_projection_tuning_validation():
    lib = mt.lib()
    assert lib.moetail_set_projection_tuning(3, 0, 0, 0, 0, 0, 0) == mt.EINVAL
    assert lib.moetail_set_projection_tuning(-1, 0, 0, 0, 0, 0, 0) == mt.EINVAL
    assert lib.moetail_set_projection_tuning(mt.PROJ_DOWN, -1, 0, 0, 0, 0, 0) == mt.EINVAL
    assert lib.moetail_set_projection_tuning(mt.PROJ_DOWN, 0, 0, 0, 0, 0, -2) == mt.EINVAL
    for kind in (mt.PROJ_UPPROJ, mt.PROJ_GATEUP, mt.PROJ_DOWN):
        assert lib.moetail_set_projection_tuning(kind, 0, 0, 0, 0, 0, 0) == mt.OK


def test_plans_are_searched_once_per_shape():
    """The per-call path looks its plan up: a second query of the same shape
    searches nothing; an override set empties the cache, and clearing it
    gives back the library's own plan."""
    s0, h0 = mt.plan_cache_stats()
    a = mt.workspace_bytes(mt.OP_TAIL, 48, 3584, 7168, 6144)
    s1, h1 = mt.plan_cache_stats()
    b = mt.workspace_bytes(mt.OP_TAIL, 48, 3584, 7168, 6144)
    s2, h2 = mt.plan_cache_stats()
    assert a == b and a > 0
    assert s1 == s0 + 1 and s2 == s1 and h2 == h1 + 1
    # the call itself takes the same cached plan (refused later for its fake
    # pointers' workspace size, after the lookup)
    assert _tail(b=48, wsb=16) == mt.EWORKSPACE
    assert mt.plan_cache_stats()[0] == s2
    with mt.projection_tuning({mt.PROJ_UPPROJ: dict(splits=2)}):
        c = mt.workspace_bytes(mt.OP_TAIL, 48, 3584, 7168, 6144)
        assert mt.plan_cache_stats()[0] == s2 + 1
    d = mt.workspace_bytes(mt.OP_TAIL, 48, 3584, 7168, 6144)
    assert d == a and mt.plan_cache_stats()[0] == s2 + 2
    assert c > 0


@pytest.mark.skipif(shutil.which("nm") is None, reason="needs nm")
def test_library_reads_no_environment():
    """No environment variable changes what the library computes: it does
    not import getenv at all."""
    r = subprocess.run(["nm", "-D", "--undefined-only", mt.LIB_PATH], capture_output=True,
                       text=True, check=True)
    names = {line.split()[-1].split("@")[0] for line in r.stdout.splitlines() if line.strip()}
    assert "getenv" not in names and "secure_getenv" not in names


# ------------------------------------------------------ the Python binding --

def test_binding_passes_the_norm_mode_through():
    """moetail_tp_finalize hands its norm mode to the library unchanged, so
    NO_NORM is refused there (EINVAL), not turned into the gain-first norm."""
    import inspect
    src = inspect.getsource(mt.moetail_tp_finalize)
    assert "int(weight_before_norm)" in src and "bool(weight_before_norm)" not in src
