"""Argument checks of the Python binding (CPU only: every call here is
refused before the library is asked to do anything).

The C ABI takes bare pointers and cannot see sizes, so the binding checks
every tensor's shape, dtype and device against the dimensions it derives
before it passes a pointer; a wrong shape must never reach a kernel."""
from __future__ import annotations

import pytest
import torch

import expert_finalize_rmsnorm_amd as mt

BF = torch.bfloat16


def z(*shape, dtype=BF):
    return torch.zeros(shape, dtype=dtype)


def ep_args(tp=2, R=8, P=64, b=4, K=4):
    return dict(rows=z(tp, R, P), permuted_idx=z(tp, b, K, dtype=torch.int32),
                route_w=z(b, K, dtype=torch.float32), gamma=z(P), gain_center=1.0, eps=1e-6,
                weight_before_norm=True, partials=z(tp, b, P), out=z(b, P))


def expect_shape_error(fn, name, **kw):
    with pytest.raises(ValueError, match=name):
        fn(**kw)


def test_finalize_shapes():
    good = ep_args()
    with pytest.raises(ValueError, match="device tensors"):
        mt.moetail_finalize(**good)  # every shape right: refused for the host memory only
    for name, bad in (("route_w", z(4, 3, dtype=torch.float32)), ("gamma", z(65)),
                      ("partials", z(2, 4, 32)), ("out", z(5, 64)), ("partials", z(3, 4, 64))):
        expect_shape_error(mt.moetail_finalize, name, **dict(good, **{name: bad}))
    with pytest.raises(TypeError, match="permuted_idx"):
        mt.moetail_finalize(**dict(good, permuted_idx=z(2, 4, 4, dtype=torch.int64)))
    with pytest.raises(TypeError, match="rows"):
        mt.moetail_finalize(**dict(good, rows=z(2, 8, 64, dtype=torch.float32)))


def test_tp_finalize_shapes():
    good = dict(kpartials=z(2, 16, 64), permuted_idx=z(4, 4, dtype=torch.int32),
                route_w=z(4, 4, dtype=torch.float32), gamma=z(64), gain_center=0.0, eps=1e-6,
                weight_before_norm=False, out=z(4, 64))
    with pytest.raises(ValueError, match="device tensors"):
        mt.moetail_tp_finalize(**good)
    for name, bad in (("route_w", z(4, 5, dtype=torch.float32)), ("gamma", z(32)),
                      ("out", z(4, 72))):
        expect_shape_error(mt.moetail_tp_finalize, name, **dict(good, **{name: bad}))


def test_upproj_shapes():
    good = dict(latent_partials=z(2, 4, 64), gamma=z(64), eps=1e-6, w_up=z(128, 64),
                out=z(4, 128), rs=z(4, 128), normed=z(4, 64))
    with pytest.raises(ValueError, match="device tensors"):
        mt.moetail_combine_norm_upproj(**good)
    for name, bad in (("gamma", z(63)), ("out", z(4, 64)), ("rs", z(3, 128)),
                      ("normed", z(4, 128)), ("w_up", z(128, 32))):
        expect_shape_error(mt.moetail_combine_norm_upproj, name, **dict(good, **{name: bad}))


def test_shared_shapes():
    good = dict(x=z(4, 128), w_gate=z(64, 128), w_up=z(64, 128), w_down=z(128, 64),
                rs=z(4, 128), h=z(4, 64))
    with pytest.raises(ValueError, match="device tensors"):
        mt.moetail_shared_expert(**good)
    for name, bad in (("w_up", z(64, 64)), ("w_down", z(64, 128)), ("rs", z(4, 64)),
                      ("h", z(4, 128))):
        expect_shape_error(mt.moetail_shared_expert, name, **dict(good, **{name: bad}))


def test_projection_partials_shapes():
    good = dict(kind=mt.PROJ_GATEUP, w0=z(64, 128), w1=z(64, 128), x=z(4, 128),
                partials=z(1024, dtype=torch.float32))
    with pytest.raises(ValueError, match="device tensors"):
        mt.moetail_projection_partials(**good)
    expect_shape_error(mt.moetail_projection_partials, "w1", **dict(good, w1=z(64, 64)))
    expect_shape_error(mt.moetail_projection_partials, "w1", **dict(good, w1=None))
    with pytest.raises(ValueError, match="second matrix"):
        mt.moetail_projection_partials(**dict(good, kind=mt.PROJ_DOWN))
    with pytest.raises(TypeError, match="float32"):
        mt.moetail_projection_partials(**dict(good, partials=z(1024)))


def tail_args():
    return dict(latent_partials=z(2, 4, 64), gamma=z(64), eps=1e-6, w_up=z(128, 64),
                x=z(4, 128), w_gate=z(64, 128), w_up_shared=z(64, 128), w_down=z(128, 64),
                out=z(4, 128), rs=z(4, 128), normed=z(4, 64), h=z(4, 64))


def test_tail_shapes():
    good = tail_args()
    with pytest.raises(ValueError, match="device tensors"):
        mt.moetail_tail(**good)
    for name, bad in (("w_up", z(64, 64)), ("w_up_shared", z(64, 64)), ("w_down", z(128, 32)),
                      ("out", z(4, 64)), ("normed", z(4, 128)), ("h", z(5, 64)),
                      ("gamma", z(128))):
        expect_shape_error(mt.moetail_tail, name, **dict(good, **{name: bad}))


def test_decode_tail_shapes():
    good = dict(tail_args(), rows=z(2, 8, 64), permuted_idx=z(2, 4, 4, dtype=torch.int32),
                route_w=z(4, 4, dtype=torch.float32), fin_gamma=z(64), gain_center=1.0,
                fin_eps=1e-6, weight_before_norm=True)
    with pytest.raises(ValueError, match="device tensors"):
        mt.moetail_decode_tail(**good)
    for name, bad in (("rows", z(2, 8, 32)), ("permuted_idx", z(3, 4, 4, dtype=torch.int32)),
                      ("route_w", z(4, 5, dtype=torch.float32)), ("fin_gamma", z(32))):
        expect_shape_error(mt.moetail_decode_tail, name, **dict(good, **{name: bad}))


def test_pack_weights_shapes():
    with pytest.raises(ValueError, match="packed"):
        mt.moetail_pack_weights(z(32, 64), z(64, 32))
    with pytest.raises(ValueError, match="device tensors"):
        mt.moetail_pack_weights(z(32, 64), z(32, 64))


def test_one_device():
    good = ep_args()
    good["out"] = torch.zeros((4, 64), dtype=BF, device="meta")
    with pytest.raises(ValueError, match="one device"):
        mt.moetail_finalize(**good)
