"""moetail_decode_tail_noalloc (the library's static scratch instead of a
workspace) against moetail_decode_tail with a workspace: the same bits, on
two calls in a row, the second with a smaller input; a call whose sizes need
more than the static scratch is refused and writes nothing."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import expert_finalize_rmsnorm_amd as mt
import workloads
from tests.gpu_util import SENTINEL, dev, empty_bf16, host

pytestmark = pytest.mark.gpu


def inputs(seed, b, K, tp, L, H, I, layout):
    ep = workloads.ep_finalize(seed, b=b, K=K, P=L, tp=tp)
    up = workloads.upproj(seed, b=b, tp=tp, L=L, N=H)
    sh = workloads.shared(seed, b=b, H=H, I=I)
    wl = (lambda a: mt.pack_weights(dev(a))) if layout == mt.W_TILED else dev
    return dict(rows=dev(ep["rows"]), idx=dev(ep["idx"]), w=dev(ep["w32"]), fg=dev(ep["gamma"]),
                gamma=dev(up["gamma"]), w_up=wl(up["w_up"]), x=dev(sh["x"]),
                wg=wl(sh["w_gate"]), wu=wl(sh["w_up"]), wd=wl(sh["w_down"]), b=b, tp=tp, L=L,
                H=H, I=I)


def outputs(d):
    b, tp, L, H, I = d["b"], d["tp"], d["L"], d["H"], d["I"]
    return dict(lat=empty_bf16(tp, b, L), out=empty_bf16(b, H), rs=empty_bf16(b, H),
                normed=empty_bf16(b, L), h=empty_bf16(b, I))


def call(d, o, noalloc, layout):
    args = (d["rows"], d["idx"], d["w"], d["fg"], 1.0, 1e-6, True, o["lat"], d["gamma"], 1e-6,
            d["w_up"], d["x"], d["wg"], d["wu"], d["wd"], o["out"])
    kw = dict(rs=o["rs"], normed=o["normed"], h=o["h"], w_layout=layout)
    if noalloc:
        mt.moetail_decode_tail_noalloc(*args, **kw)
    else:
        ws = mt.new_workspace(mt.OP_TAIL, d["b"], d["L"], d["H"], d["I"])
        mt.moetail_decode_tail(*args, workspace=ws, **kw)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in o.items()}


def test_noalloc_equals_the_workspace_call_twice_second_smaller():
    cases = [(64, 16, 8, 3584, 7168, 6144, mt.W_TILED), (16, 6, 3, 544, 256, 128, mt.W_ROWS)]
    for seed, (b, K, tp, L, H, I, layout) in enumerate(cases):
        print(f"noalloc case b={b} K={K} tp={tp} L={L} H={H} I={I} layout={layout}", flush=True)
        d = inputs(seed, b, K, tp, L, H, I, layout)
        assert mt.workspace_bytes(mt.OP_TAIL, b, L, H, I) <= mt.NOALLOC_SCRATCH_BYTES
        want = call(d, outputs(d), False, layout)
        got = call(d, outputs(d), True, layout)
        for k in want:
            assert np.array_equal(got[k], want[k]), f"{k} differs at b={b}"
            assert not np.any(got[k] == SENTINEL), f"{k} not written at b={b}"


def test_noalloc_refuses_sizes_beyond_its_scratch():
    b, K, tp, L, H, I = 128, 16, 8, 3584, 7168, 6144
    assert mt.workspace_bytes(mt.OP_TAIL, b, L, H, I) > mt.NOALLOC_SCRATCH_BYTES
    d = inputs(3, b, K, tp, L, H, I, mt.W_ROWS)
    o = outputs(d)
    with pytest.raises(mt.MoetailError) as e:
        call(d, o, True, mt.W_ROWS)
    assert e.value.status == mt.EWORKSPACE
    for k, v in o.items():
        assert np.all(host(v) == SENTINEL), f"{k} was written by a refused call"
