"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Every test here runs on an MI355X.  Inputs are the seeded synthetic
workloads of ``workloads.py``; expected values come from ``oracle/`` on the
same inputs.  Finalize and combine outputs must be within 1 BF16 step of
the oracle and at least 99.9% bit-exact; projection outputs within
2e-2 + 1e-2 |ref|.
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest
import torch

import expert_finalize_rmsnorm_amd as mt
import oracle
import workloads
from tests.gpu_util import (ORACLE_THREADS, SENTINEL, dev, empty_bf16, finalize_bar, gemm_bar,
                            host)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
NT = ORACLE_THREADS


def bits(values):
    return oracle.bf16_round(np.asarray(values, np.float32))


# ------------------------------------------------------------ EP finalize --

def run_ep(inp, wbn, wkey="w32", mode="both", **kw):
    tp, b, P = inp["tp"], inp["b"], inp["P"]
    rows, idx, w, gamma = dev(inp["rows"]), dev(inp["idx"]), dev(inp[wkey]), dev(inp["gamma"])
    partials = empty_bf16(tp, b, P) if mode in ("both", "partials") else None
    out = empty_bf16(b, P) if mode in ("both", "out") else None
    mt.moetail_finalize(rows, idx, w, gamma, inp["gain_center"], inp["eps"], wbn,
                        partials=partials, out=out, **kw)
    return (host(partials) if partials is not None else None,
            host(out) if out is not None else None)


def oracle_ep(inp, wbn, wkey="w32"):
    return oracle.finalize(inp["rows"], inp["idx"], inp[wkey], inp["gamma"], inp["gain_center"],
                           inp["eps"], wbn, nthreads=NT)


@pytest.mark.parametrize("wbn", [True, False])
@pytest.mark.parametrize("wkey", ["w32", "w16"])
def test_ep_tiny(wbn, wkey):
    inp = workloads.tiny_ep_finalize(0)
    want_p, want_o = oracle_ep(inp, wbn, wkey)
    got_p, got_o = run_ep(inp, wbn, wkey)
    assert np.array_equal(got_p, want_p)
    assert np.array_equal(got_o, want_o)


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("wbn", [True, False])
@pytest.mark.parametrize("wkey", ["w32", "w16"])
def test_ep_decode_scale(seed, wbn, wkey):
    """b=64, top-16 over tp=8 ranks (2 local routes each), P=3584, outlier rows."""
    inp = workloads.ep_finalize(seed)
    want_p, want_o = oracle_ep(inp, wbn, wkey)
    got_p, got_o = run_ep(inp, wbn, wkey, "both")
    finalize_bar(got_p, want_p, "partials")
    finalize_bar(got_o, want_o, "out")
    assert np.array_equal(got_p, want_p) and np.array_equal(got_o, want_o)
    # out only (combine fused, partials never written) and partials only
    _, only_o = run_ep(inp, wbn, wkey, "out")
    only_p, _ = run_ep(inp, wbn, wkey, "partials")
    assert np.array_equal(only_o, got_o) and np.array_equal(only_p, got_p)


@pytest.mark.parametrize("b,K,P,tp", [(5, 3, 520, 3), (3, 7, 8, 1), (2, 32, 8192, 4),
                                      (9, 16, 1032, 12), (1, 1, 3584, 8), (4, 4, 512, 2),
                                      (17, 8, 7168, 8), (3, 32, 64, 32)])
@pytest.mark.parametrize("wbn", [True, False])
def test_ep_ragged_and_edges(b, K, P, tp, wbn):
    per = max(1, K // tp)
    if K % tp == 0:
        inp = workloads.ep_finalize(b * 7 + K, b=b, K=K, P=P, tp=tp, outlier_frac=0.05)
    else:
        # routes spread unevenly: rank d holds the routes with k % tp == d
        inp = workloads.ep_finalize(b, b=b, K=K, P=P, tp=1, outlier_frac=0.0)
        rows1 = inp["rows"][0]
        idx = np.full((tp, b, K), -1, np.int32)
        for k in range(K):
            idx[k % tp, :, k] = inp["idx"][0, :, k]
        inp.update(rows=np.ascontiguousarray(np.broadcast_to(rows1, (tp,) + rows1.shape)),
                   idx=idx, tp=tp)
    del per
    want_p, want_o = oracle_ep(inp, wbn)
    got_p, got_o = run_ep(inp, wbn)
    finalize_bar(got_p, want_p, "partials")
    finalize_bar(got_o, want_o, "out")
    assert np.array_equal(got_p, want_p) and np.array_equal(got_o, want_o)
    _, only_o = run_ep(inp, wbn, mode="out")  # the fused kernel
    assert np.array_equal(only_o, want_o)


@pytest.mark.parametrize("wbn", [True, False])
def test_ep_skewed_ranks(wbn):
    """Uneven route ownership: rank 0 holds 13 of 16 routes (more than one
    batch of rows), ranks 1-3 one each, ranks 4-7 none (+0 partials)."""
    inp = workloads.ep_finalize(11, b=6, K=16, P=3584, tp=1, outlier_frac=0.0)
    tp = 8
    rows1 = inp["rows"][0]
    owner = np.array([0] * 13 + [1, 2, 3])
    idx = np.full((tp, 6, 16), -1, np.int32)
    for k in range(16):
        idx[owner[k], :, k] = inp["idx"][0, :, k]
    inp.update(rows=np.ascontiguousarray(np.broadcast_to(rows1, (tp,) + rows1.shape)), idx=idx,
               tp=tp)
    want_p, want_o = oracle_ep(inp, wbn)
    assert not want_p[4:].any()
    for mode in ("both", "partials", "out"):
        got_p, got_o = run_ep(inp, wbn, mode=mode)
        if got_p is not None:
            assert np.array_equal(got_p, want_p), mode
        if got_o is not None:
            assert np.array_equal(got_o, want_o), mode


def test_ep_absent_and_out_of_range_indices():
    inp = workloads.ep_finalize(5, b=6, K=8, P=1024, tp=4)
    idx = inp["idx"].copy()
    idx[idx < 0] = np.where(np.arange((idx < 0).sum()) % 2 == 0, -7, inp["R"] + 3)
    inp["idx"] = idx
    want_p, want_o = oracle_ep(inp, True)
    got_p, got_o = run_ep(inp, True)
    assert np.array_equal(got_p, want_p) and np.array_equal(got_o, want_o)


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)["case"]


def test_ep_golden_rank_and_route_order_and_negzero():
    case = _golden("rank_order.json")
    tp, P = case["tp"], case["P"]
    idx = np.full((tp, 1, tp), -1, np.int32)
    for d in range(tp):
        idx[d, 0, d] = 0
    inp = dict(rows=bits(np.ones((tp, 1, P))), idx=idx, w32=np.array([case["w"]], np.float32),
               gamma=np.zeros(P, np.uint16), gain_center=case["gain_center"], eps=case["eps"],
               tp=tp, b=1, P=P)
    got_p, got_o = run_ep(inp, True)
    assert [f"{int(v):04x}" for v in got_p[:, 0, 0]] == case["expected_partials_hex"]
    assert all(f"{int(v):04x}" == case["expected_out_hex"] for v in got_o.ravel())

    case = _golden("route_order.json")
    K, P = case["K"], case["P"]
    inp = dict(rows=bits(np.ones((1, K, P))), idx=np.arange(K, dtype=np.int32).reshape(1, 1, K),
               w32=np.array([case["w"]], np.float32), gamma=np.zeros(P, np.uint16),
               gain_center=case["gain_center"], eps=case["eps"], tp=1, b=1, P=P)
    for wbn in (True, False):
        _, got_o = run_ep(inp, wbn)
        assert all(f"{int(v):04x}" == case["expected_out_hex"] for v in got_o.ravel())

    case = _golden("negzero.json")
    P = case["P"]
    inp = dict(rows=bits(np.array(case["row"])).reshape(1, 1, P),
               idx=np.zeros((1, 1, 1), np.int32),
               w32=np.array([[case["w_sign"] * 2.0 ** case["w_log2"]]], np.float32),
               gamma=np.zeros(P, np.uint16), gain_center=case["gain_center"], eps=case["eps"],
               tp=1, b=1, P=P)
    got_p, got_o = run_ep(inp, case["weight_before_norm"])
    assert [f"{int(v):04x}" for v in got_o.ravel()] == case["expected_out_hex"]
    assert [f"{int(v):04x}" for v in got_p.ravel()] == case["expected_out_hex"]


def test_ep_b0_and_refused_calls_write_nothing():
    inp = workloads.ep_finalize(0, b=4, K=16, P=3584, tp=8)
    rows, idx, w, gamma = dev(inp["rows"]), dev(inp["idx"]), dev(inp["w32"]), dev(inp["gamma"])
    out = empty_bf16(4, 3584)
    mt.moetail_finalize(rows, idx[:, :0], w[:0], gamma, 1.0, 1e-6, True, out=out[:0])
    with pytest.raises(mt.MoetailError):
        mt.moetail_finalize(rows, idx, w, gamma, 1.0, -1.0, True, out=out)  # eps < 0
    assert np.all(host(out) == SENTINEL)


def test_ep_repeatable_and_graph_replay():
    inp = workloads.ep_finalize(3)
    rows, idx, w, gamma = dev(inp["rows"]), dev(inp["idx"]), dev(inp["w32"]), dev(inp["gamma"])
    out = empty_bf16(64, 3584)
    partials = empty_bf16(8, 64, 3584)
    first = None
    for _ in range(5):
        mt.moetail_finalize(rows, idx, w, gamma, 1.0, 1e-6, True, partials=partials, out=out)
        cur = (host(partials), host(out))
        if first is None:
            first = cur
        assert np.array_equal(cur[0], first[0]) and np.array_equal(cur[1], first[1])
    out.fill_(SENTINEL)
    partials.fill_(SENTINEL)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        mt.moetail_finalize(rows, idx, w, gamma, 1.0, 1e-6, True, partials=partials, out=out)
    for _ in range(3):
        out.fill_(SENTINEL)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out), first[1]) and np.array_equal(host(partials), first[0])


# ------------------------------------------------------------- expert TP --

def run_tp(inp, wbn, wkey="w32"):
    b, K, P = inp["b"], inp["idx"].shape[1], inp["P"]
    out = empty_bf16(b, P)
    ws = mt.new_workspace(mt.OP_TP_FINALIZE, b, K, P)
    mt.moetail_tp_finalize(dev(inp["kpart"]), dev(inp["idx"]), dev(inp[wkey]), dev(inp["gamma"]),
                           inp["gain_center"], inp["eps"], wbn, out, workspace=ws)
    return host(out)


@pytest.mark.parametrize("wbn,wkey", [(False, "w32"), (False, "w16"), (True, "w32")])
def test_tp_full_scale(wbn, wkey):
    """b=128, K=16, P=7168, tp=8 K-partials of every route row (235 MB)."""
    inp = workloads.tp_finalize(0)
    want = oracle.tp_finalize(inp["kpart"], inp["idx"], inp[wkey], inp["gamma"],
                              inp["gain_center"], inp["eps"], wbn, nthreads=NT)
    got = run_tp(inp, wbn, wkey)
    finalize_bar(got, want, "tp out")
    assert np.array_equal(got, want)


@pytest.mark.parametrize("b,K,P,tp", [(7, 5, 1032, 3), (3, 20, 520, 2), (2, 16, 8192, 1),
                                      (5, 1, 8, 32), (4, 32, 3584, 4), (3, 4, 512, 8),
                                      (6, 16, 7168, 8), (3, 7, 2056, 12)])
@pytest.mark.parametrize("wbn", [True, False])
def test_tp_ragged_and_edges(b, K, P, tp, wbn):
    inp = workloads.tp_finalize(b + K, b=b, K=K, P=P, tp=tp, num_rows=b * K + 3)
    idx = inp["idx"].copy()
    idx[0, K // 2] = -1                 # absent route
    idx[b - 1, K - 1] = inp["num_rows"] + 9  # past the end: absent too
    inp["idx"] = idx
    inp["gain_center"] = 0.5
    want = oracle.tp_finalize(inp["kpart"], idx, inp["w32"], inp["gamma"], 0.5, inp["eps"], wbn,
                              nthreads=NT)
    got = run_tp(inp, wbn)
    finalize_bar(got, want, "tp out")
    assert np.array_equal(got, want)


@pytest.mark.parametrize("b,K,P,tp", [(16, 16, 7168, 8), (7, 5, 1032, 3), (4, 32, 3584, 4)])
def test_tp_one_pass_when_the_halves_do_not_meet(b, K, P, tp):
    """With no wait at all every block forms its partner half's block totals
    itself: the same bits as the oracle (the path a block takes when its
    partner does not come within the wait limit)."""
    inp = workloads.tp_finalize(b + P, b=b, K=K, P=P, tp=tp, num_rows=b * K + 2)
    idx = inp["idx"].copy()
    idx[0, 0] = -1
    inp["idx"] = idx
    want = oracle.tp_finalize(inp["kpart"], idx, inp["w32"], inp["gamma"], 0.0, inp["eps"], False,
                              nthreads=NT)
    try:
        mt.set_tp_wait_limit(-1)
        got = run_tp(inp, False)
    finally:
        mt.set_tp_wait_limit()
    assert np.array_equal(got, want)


def test_tp_workspace_reused_and_graph_replay():
    """One workspace serves many calls, eager and replayed from a graph, with
    the same bits: every call raises each token's generation by one, so its
    block-total slots are told apart from the last call's."""
    inp = workloads.tp_finalize(5, b=32, K=16, P=7168, tp=8)
    want = oracle.tp_finalize(inp["kpart"], inp["idx"], inp["w32"], inp["gamma"], 0.0, inp["eps"],
                              False, nthreads=NT)
    kp, idx, w, gamma = dev(inp["kpart"]), dev(inp["idx"]), dev(inp["w32"]), dev(inp["gamma"])
    ws = mt.new_workspace(mt.OP_TP_FINALIZE, 32, 16, 7168, 8)
    out = empty_bf16(32, 7168)

    def call():
        mt.moetail_tp_finalize(kp, idx, w, gamma, 0.0, inp["eps"], False, out, workspace=ws)

    def generations():
        torch.cuda.synchronize()
        return ws[: 4 * 32].view(torch.int32).cpu().numpy().copy()

    for i in range(3):
        out.fill_(SENTINEL)
        call()
        assert np.array_equal(host(out), want)
        assert np.all(generations() == i + 1)
    g, st = torch.cuda.CUDAGraph(), torch.cuda.Stream()
    with torch.cuda.graph(g, stream=st):
        call()
    for _ in range(3):
        out.fill_(SENTINEL)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out), want)
    assert np.all(generations() == 3 + 3)  # three eager calls, three replays


def test_tp_no_norm_mode_is_refused_and_writes_nothing():
    """The expert-TP finalize takes the two normalizing modes only: NO_NORM
    reaches the library unchanged and is refused before any launch."""
    tp = workloads.tp_finalize(0, b=4, K=4, P=1024, tp=4)
    out = empty_bf16(4, 1024)
    with pytest.raises(mt.MoetailError) as e:
        mt.moetail_tp_finalize(dev(tp["kpart"]), dev(tp["idx"]), dev(tp["w32"]),
                               dev(tp["gamma"]), 0.0, tp["eps"], mt.NO_NORM, out,
                               workspace=mt.new_workspace(mt.OP_TP_FINALIZE, 4, 4, 1024))
    assert e.value.status == mt.EINVAL
    assert np.all(host(out) == SENTINEL)


def test_tp_golden_round_before_norm():
    case = _golden("tp_round_before_norm.json")
    P = case["P"]
    kpart = np.zeros((2, 1, P), np.uint16)
    kpart[0, 0] = bits(np.ones(P))
    kpart[1, 0, 0] = bits([2.0 ** -8])[0]
    inp = dict(kpart=kpart, idx=np.array(case["idx"], np.int32),
               w32=np.array([case["w"]], np.float32), gamma=np.zeros(P, np.uint16),
               gain_center=case["gain_center"], eps=case["eps"], b=1, P=P)
    got = run_tp(inp, True)
    assert [f"{int(v):04x}" for v in got.ravel()] == case["expected_out_hex"]


# ------------------------------------ latent combine + norm + up projection --

def weight(w, layout):
    """A weight matrix on the device in the given layout."""
    d = dev(w)
    return mt.pack_weights(d) if layout == mt.W_TILED else d


def run_upproj(inp, rs=None, with_normed=True, layout=mt.W_ROWS):
    b, L, N, tp = inp["b"], inp["L"], inp["N"], inp["tp"]
    out = empty_bf16(b, N)
    normed = empty_bf16(b, L) if with_normed else None
    ws = mt.new_workspace(mt.OP_COMBINE_NORM_UPPROJ, b, L, N, tp)
    mt.moetail_combine_norm_upproj(dev(inp["lat"]), dev(inp["gamma"]), inp["eps"],
                                   weight(inp["w_up"], layout), out,
                                   rs=None if rs is None else dev(rs), normed=normed,
                                   workspace=ws, w_layout=layout)
    return (host(normed) if normed is not None else None), host(out)


@pytest.mark.parametrize("b", [1, 8, 32, 64])
def test_upproj_scale(b):
    """tp=8 latent partials [8,b,3584] -> RMSNorm -> W_up [7168,3584]."""
    inp = workloads.upproj(0, b=b)
    want_n, want_o = oracle.combine_norm_upproj(inp["lat"], inp["gamma"], inp["eps"],
                                                inp["w_up"], nthreads=NT)
    got_n, got_o = run_upproj(inp)
    assert np.array_equal(got_n, want_n)
    gemm_bar(got_o, want_o, f"upproj b={b}")
    _, got_o2 = run_upproj(inp, with_normed=False)  # y kept in the workspace
    assert np.array_equal(got_o2, got_o)


def test_upproj_with_reduce_scatter_partial():
    inp = workloads.upproj(1, b=64, with_rs=True)
    want_n, want_o = oracle.combine_norm_upproj(inp["lat"], inp["gamma"], inp["eps"],
                                                inp["w_up"], inp["rs"], nthreads=NT)
    got_n, got_o = run_upproj(inp, rs=inp["rs"])
    assert np.array_equal(got_n, want_n)
    gemm_bar(got_o, want_o, "upproj + rs")


@pytest.mark.parametrize("b,tp,L,N", [(5, 3, 544, 128), (17, 1, 32, 64), (128, 2, 1024, 256),
                                      (3, 32, 8192, 64)])
def test_upproj_ragged(b, tp, L, N):
    inp = workloads.upproj(b + L, b=b, tp=tp, L=L, N=N, with_rs=True)
    want_n, want_o = oracle.combine_norm_upproj(inp["lat"], inp["gamma"], inp["eps"],
                                                inp["w_up"], inp["rs"], nthreads=NT)
    got_n, got_o = run_upproj(inp, rs=inp["rs"])
    assert np.array_equal(got_n, want_n)
    gemm_bar(got_o, want_o, "upproj ragged")


def test_upproj_unit_rows_and_zero_weights():
    inp = workloads.upproj(2, b=33, tp=4, L=1024, N=192)
    perm = np.random.default_rng(0).integers(0, 1024, 192)
    w = np.zeros((192, 1024), np.float32)
    w[np.arange(192), perm] = 1.0
    inp["w_up"] = bits(w)
    got_n, got_o = run_upproj(inp)
    assert np.array_equal(got_o, got_n[:, perm])  # one exact product per output
    rs = bits(np.random.default_rng(1).standard_normal((33, 192)))
    rs[0, :4] = 0x8000
    inp["w_up"] = np.zeros((192, 1024), np.uint16)
    _, got_o = run_upproj(inp, rs=rs)
    want = rs.copy()
    want[want == 0x8000] = 0
    assert np.array_equal(got_o, want)


def test_upproj_two_unit_weights_per_row():
    """out = bf16(y[a] + y[c]) from the BF16 normed row y, bit for bit with
    the oracle (the sum of two BF16 products is exact in the FP32 sum)."""
    inp = workloads.upproj(4, b=20, tp=4, L=544, N=128)
    rng = np.random.default_rng(2)
    a, c = rng.integers(0, 544, 128), rng.integers(0, 544, 128)
    c = np.where(c == a, (c + 1) % 544, c)
    w = np.zeros((128, 544), np.float32)
    w[np.arange(128), a] = 1.0
    w[np.arange(128), c] = 1.0
    inp["w_up"] = bits(w)
    _, want_o = oracle.combine_norm_upproj(inp["lat"], inp["gamma"], inp["eps"], inp["w_up"])
    for layout in (mt.W_ROWS, mt.W_TILED):
        _, got_o = run_upproj(inp, layout=layout)
        assert np.array_equal(got_o, want_o)


def test_upproj_golden_rs_after_the_k_sum():
    case = json.load(open(os.path.join(GOLDEN, "upproj_rs_order.json")))["case"]
    tp, b, L, N = case["tp"], case["b"], case["L"], case["N"]
    w = np.zeros((N, L), np.float32)
    w[:, 0], w[:, 1] = 2.0 ** 24, -2.0 ** 24
    inp = dict(lat=bits(np.ones((tp, b, L))), gamma=bits(np.ones(L)), eps=case["eps"],
               w_up=bits(w), b=b, tp=tp, L=L, N=N)
    got_n, got_o = run_upproj(inp, rs=bits(np.ones((b, N))))
    assert np.all(got_n == int(case["expected_normed_hex"], 16))
    assert np.all(got_o == int(case["expected_out_hex"], 16))


# ----------------------------------------------------------- shared expert --

def run_shared(inp, with_h=True, layout=mt.W_ROWS):
    b, H, I = inp["b"], inp["H"], inp["I"]
    rs = empty_bf16(b, H)
    h = empty_bf16(b, I) if with_h else None
    ws = mt.new_workspace(mt.OP_SHARED_EXPERT, b, H, I)
    mt.moetail_shared_expert(dev(inp["x"]), weight(inp["w_gate"], layout),
                             weight(inp["w_up"], layout), weight(inp["w_down"], layout), rs, h=h,
                             workspace=ws, w_layout=layout)
    return (host(h) if h is not None else None), host(rs)


def sample_tokens(b):
    return sorted(t for t in {0, 1, 15, 16, b // 2, b - 1} if t < b)


@pytest.mark.parametrize("b", [16, 32, 64, 128])
def test_shared_scale(b):
    """x [b,7168], W_gate/W_up [6144,7168], W_down [7168,6144]; the oracle
    runs on a sample of the tokens (tokens are independent)."""
    inp = workloads.shared(0, b=b)
    got_h, got_rs = run_shared(inp)
    sel = sample_tokens(b)
    want_h, want_rs = oracle.shared_expert(inp["x"][sel], inp["w_gate"], inp["w_up"],
                                           inp["w_down"], nthreads=NT)
    gemm_bar(got_h[sel], want_h, f"h b={b}")
    gemm_bar(got_rs[sel], want_rs, f"rs b={b}")
    _, got_rs2 = run_shared(inp, with_h=False)  # h kept in the workspace
    assert np.array_equal(got_rs2, got_rs)


@pytest.mark.parametrize("b,H,I", [(5, 512, 256), (33, 256, 128), (1, 64, 64), (128, 128, 192),
                                   (128, 32768, 64), (3, 64, 32768)])
def test_shared_small_full(b, H, I):
    inp = workloads.shared(b + H, b=b, H=H, I=I)
    want_h, want_rs = oracle.shared_expert(inp["x"], inp["w_gate"], inp["w_up"], inp["w_down"],
                                           nthreads=NT)
    got_h, got_rs = run_shared(inp)
    gemm_bar(got_h, want_h, "h")
    gemm_bar(got_rs, want_rs, "rs")


def test_shared_unit_rows():
    rng = np.random.default_rng(4)
    b, H, I = 20, 256, 128
    x = bits(rng.standard_normal((b, H)) * 3)
    a, c = rng.integers(0, H, I), rng.integers(0, H, I)
    wg = np.zeros((I, H), np.float32)
    wu = np.zeros((I, H), np.float32)
    wg[np.arange(I), a] = 1.0
    wu[np.arange(I), c] = 1.0
    sel = rng.integers(0, I, H)
    wd = np.zeros((H, I), np.float32)
    wd[np.arange(H), sel] = 1.0
    inp = dict(x=x, w_gate=bits(wg), w_up=bits(wu), w_down=bits(wd), b=b, H=H, I=I)
    got_h, got_rs = run_shared(inp)
    want_h, _ = oracle.shared_expert(x, inp["w_gate"], inp["w_up"], inp["w_down"])
    gemm_bar(got_h, want_h, "unit-row h")
    assert np.array_equal(got_rs, got_h[:, sel])  # one exact product per output
    zh, zrs = run_shared(dict(inp, x=np.zeros_like(x)))
    assert not zh.any() and not zrs.any()


PLAN_OVERRIDES = [dict(WAVES=w, SPLITS=s) for w in (7, 8, 14, 16) for s in (2, 8)] + [
    dict(MR=2, PF=f, WAVES=w, SPLITS=s) for f in (4, 8) for w in (4, 7, 8) for s in (2, 8)] + [
    dict(WAVES=8, SPLITS=2, BLOCKS=100), dict(WAVES=14, SPLITS=8, BLOCKS=37),
    dict(MR=2, PF=4, WAVES=7, SPLITS=8, BLOCKS=37), dict(SPLITS=1)] + [
    # the multi-pass kernel: 2 or 4 LDS slices per split, 8 or 12 waves, 1..4
    # held units; and the single-pass kernel where the plan would pick it
    dict(PASSES=1), dict(PASSES=2), dict(PASSES=2, BLOCKS=64), dict(PASSES=4, BLOCKS=64),
    dict(PASSES=2, SPLITS=1), dict(PASSES=2, WAVES=8, BLOCKS=64), dict(PASSES=2, BLOCKS=16),
    dict(PASSES=2, BLOCKS=4), dict(PASSES=2, WAVES=12, BLOCKS=8)]


_KIND = {"UPPROJ": mt.PROJ_UPPROJ, "GATEUP": mt.PROJ_GATEUP, "DOWN": mt.PROJ_DOWN}
_KNOB = {"SPLITS": "splits", "WAVES": "waves", "BLOCKS": "blocks", "MR": "tiles_per_unit",
         "PF": "prefetch", "PASSES": "passes"}


def tuning_of(ov, kinds=None):
    """{kind: knobs} for mt.projection_tuning from an override dict whose keys
    are KNOB (for every kind in `kinds`) or KIND_KNOB."""
    res = {}
    for key, val in ov.items():
        if "_" in key:
            kind, knob = key.split("_", 1)
            res.setdefault(_KIND[kind], {})[_KNOB[knob]] = val
        else:
            for kind in kinds:
                res.setdefault(_KIND[kind], {})[_KNOB[key]] = val
    return res


@pytest.mark.parametrize("b", [1, 40, 128])
def test_projection_plan_overrides(b):
    """Every kernel shape the plan can pick (waves per block, slice count,
    uneven blocks per slice, LDS passes per slice) against the oracle,
    through the tuning overrides; a slice count that does not fit falls back
    to the default."""
    up = workloads.upproj(70 + b, b=b, tp=2, L=3584, N=512, with_rs=True)
    sh = workloads.shared(80 + b, b=b, H=1024, I=1024)
    want_up = oracle.combine_norm_upproj(up["lat"], up["gamma"], up["eps"], up["w_up"], up["rs"],
                                         nthreads=NT)[1]
    want_h, want_rs = oracle.shared_expert(sh["x"], sh["w_gate"], sh["w_up"], sh["w_down"],
                                           nthreads=NT)
    for ov in PLAN_OVERRIDES:
        with mt.projection_tuning(tuning_of(ov, ("UPPROJ", "GATEUP", "DOWN"))):
            check_overridden_projections(b, ov, up, sh, want_up, want_h, want_rs)


def check_overridden_projections(b, ov, up, sh, want_up, want_h, want_rs):
    _, got_up = run_upproj(up, rs=up["rs"])
    gemm_bar(got_up, want_up, f"upproj b={b} {ov}")
    got_h, got_rs = run_shared(sh)
    gemm_bar(got_h, want_h, f"h b={b} {ov}")
    gemm_bar(got_rs, want_rs, f"rs b={b} {ov}")
    # the tiled weight layout: the same bits in every kernel shape
    assert np.array_equal(run_upproj(up, rs=up["rs"], layout=mt.W_TILED)[1], got_up)
    got_h2, got_rs2 = run_shared(sh, layout=mt.W_TILED)
    assert np.array_equal(got_h2, got_h) and np.array_equal(got_rs2, got_rs)


def test_projections_graph_replay():
    inp = workloads.upproj(4, b=32, with_rs=True)
    sh = workloads.shared(4, b=32)
    lat, gamma, w_up, rs_in = dev(inp["lat"]), dev(inp["gamma"]), dev(inp["w_up"]), dev(inp["rs"])
    x, wg, wu, wd = dev(sh["x"]), dev(sh["w_gate"]), dev(sh["w_up"]), dev(sh["w_down"])
    out, rs = empty_bf16(32, 7168), empty_bf16(32, 7168)
    ws1 = mt.new_workspace(mt.OP_COMBINE_NORM_UPPROJ, 32, 3584, 7168, 8)
    ws2 = mt.new_workspace(mt.OP_SHARED_EXPERT, 32, 7168, 6144)

    def step():
        mt.moetail_shared_expert(x, wg, wu, wd, rs, workspace=ws2)
        mt.moetail_combine_norm_upproj(lat, gamma, 1e-6, w_up, out, rs=rs, workspace=ws1)

    step()
    eager = (host(rs), host(out))
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    for _ in range(3):
        out.fill_(SENTINEL)
        rs.fill_(SENTINEL)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(rs), eager[0]) and np.array_equal(host(out), eager[1])
    del rs_in


def test_tail_chain_fused_combine_equals_partials_path():
    """The rank combine done inside the finalize launch (its out row fed to
    the up projection as a single partial) gives the same bits as writing
    the tp partials and combining them in moetail_combine_norm_upproj."""
    ep = workloads.ep_finalize(6)
    up = workloads.upproj(6, b=64)
    rows, idx, w, gamma = dev(ep["rows"]), dev(ep["idx"]), dev(ep["w32"]), dev(ep["gamma"])
    partials, comb = empty_bf16(8, 64, 3584), empty_bf16(1, 64, 3584)
    mt.moetail_finalize(rows, idx, w, gamma, 1.0, 1e-6, True, partials=partials)
    mt.moetail_finalize(rows, idx, w, gamma, 1.0, 1e-6, True, out=comb[0])
    outs = []
    for lat, tp in ((partials, 8), (comb, 1)):
        out, normed = empty_bf16(64, 7168), empty_bf16(64, 3584)
        mt.moetail_combine_norm_upproj(lat, dev(up["gamma"]), 1e-6, dev(up["w_up"]), out,
                                       normed=normed,
                                       workspace=mt.new_workspace(mt.OP_COMBINE_NORM_UPPROJ, 64,
                                                                  3584, 7168, tp))
        outs.append((host(normed), host(out)))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    want_n, _ = oracle.combine_norm_upproj(oracle.finalize(ep["rows"], ep["idx"], ep["w32"],
                                                           ep["gamma"], 1.0, 1e-6, True,
                                                           nthreads=NT)[0],
                                           up["gamma"], 1e-6, up["w_up"][:64], nthreads=NT)
    assert np.array_equal(outs[0][0], want_n)


def test_tail_step_two_stream_graph_matches_eager():
    """The benchmark's step: finalize on a side stream beside the shared
    expert, joined before the up projection, captured once and replayed."""
    ep, up, sh = workloads.ep_finalize(8), workloads.upproj(8, b=64), workloads.shared(8, b=64)
    rows, idx, w, gamma = dev(ep["rows"]), dev(ep["idx"]), dev(ep["w32"]), dev(ep["gamma"])
    x, wg, wu, wd = dev(sh["x"]), dev(sh["w_gate"]), dev(sh["w_up"]), dev(sh["w_down"])
    lg, wup = dev(up["gamma"]), dev(up["w_up"])
    lat, rs, out = empty_bf16(1, 64, 3584), empty_bf16(64, 7168), empty_bf16(64, 7168)
    ws_sh = mt.new_workspace(mt.OP_SHARED_EXPERT, 64, 7168, 6144)
    ws_up = mt.new_workspace(mt.OP_COMBINE_NORM_UPPROJ, 64, 3584, 7168, 1)
    side = torch.cuda.Stream()

    def step():
        main = torch.cuda.current_stream()
        fork, join = torch.cuda.Event(), torch.cuda.Event()
        fork.record(main)
        with torch.cuda.stream(side):
            side.wait_event(fork)
            mt.moetail_finalize(rows, idx, w, gamma, 1.0, 1e-6, True, out=lat[0])
            join.record(side)
        mt.moetail_shared_expert(x, wg, wu, wd, rs, workspace=ws_sh)
        main.wait_event(join)
        mt.moetail_combine_norm_upproj(lat, lg, 1e-6, wup, out, rs=rs, workspace=ws_up)

    step()
    eager = (host(lat), host(rs), host(out))
    cap = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        step()
    for _ in range(3):
        for t in (lat, rs, out):
            t.fill_(SENTINEL)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert all(np.array_equal(a, b) for a, b in zip((host(lat), host(rs), host(out)), eager))
    # and the step's latent row is the oracle's finalize + combine
    _, want = oracle.finalize(ep["rows"], ep["idx"], ep["w32"], ep["gamma"], 1.0, 1e-6, True,
                              nthreads=NT)
    assert np.array_equal(eager[0][0], want)


# ------------------------------------------------------------- fused tail --

def run_tail_and_calls(up, sh, with_opt=True, layout=mt.W_ROWS, calls_layout=None):
    """moetail_tail (weights in `layout`), and the two calls it stands for
    (weights in `calls_layout`, the same by default), on the same inputs."""
    b, H, I, L, tp = sh["b"], sh["H"], sh["I"], up["L"], up["tp"]
    lat, gamma = dev(up["lat"]), dev(up["gamma"])
    x = dev(sh["x"])
    w_up, wg, wu, wd = (weight(up["w_up"], layout), weight(sh["w_gate"], layout),
                        weight(sh["w_up"], layout), weight(sh["w_down"], layout))
    out = empty_bf16(b, H)
    rs, normed, h = ((empty_bf16(b, H), empty_bf16(b, L), empty_bf16(b, I)) if with_opt
                     else (None, None, None))
    mt.moetail_tail(lat, gamma, up["eps"], w_up, x, wg, wu, wd, out, rs=rs, normed=normed, h=h,
                    workspace=mt.new_workspace(mt.OP_TAIL, b, L, H, I), w_layout=layout)
    cl = layout if calls_layout is None else calls_layout
    if cl != layout:
        w_up, wg, wu, wd = (weight(up["w_up"], cl), weight(sh["w_gate"], cl),
                            weight(sh["w_up"], cl), weight(sh["w_down"], cl))
    rs2, h2, out2, normed2 = empty_bf16(b, H), empty_bf16(b, I), empty_bf16(b, H), empty_bf16(b, L)
    mt.moetail_shared_expert(x, wg, wu, wd, rs2, h=h2,
                             workspace=mt.new_workspace(mt.OP_SHARED_EXPERT, b, H, I),
                             w_layout=cl)
    mt.moetail_combine_norm_upproj(lat, gamma, up["eps"], w_up, out2, rs=rs2, normed=normed2,
                                   workspace=mt.new_workspace(mt.OP_COMBINE_NORM_UPPROJ, b, L, H,
                                                              tp), w_layout=cl)
    fused = dict(out=host(out), rs=host(rs) if rs is not None else None,
                 normed=host(normed) if normed is not None else None,
                 h=host(h) if h is not None else None)
    calls = dict(out=host(out2), rs=host(rs2), normed=host(normed2), h=host(h2))
    return fused, calls


@pytest.mark.parametrize("b", [1, 32, 64, 128])
def test_tail_equals_the_two_calls(b):
    """b tokens of the decode tail: tp=8 latent partials [8, b, 3584], W_up
    [7168, 3584], shared expert 7168 -> 6144 -> 7168."""
    up = workloads.upproj(20 + b, b=b)
    sh = workloads.shared(30 + b, b=b)
    fused, calls = run_tail_and_calls(up, sh)
    for k in ("out", "rs", "normed", "h"):
        assert np.array_equal(fused[k], calls[k]), k
    sel = sample_tokens(b)
    want_h, want_rs = oracle.shared_expert(sh["x"][sel], sh["w_gate"], sh["w_up"], sh["w_down"],
                                           nthreads=NT)
    gemm_bar(fused["rs"][sel], want_rs, f"tail rs b={b}")
    gemm_bar(fused["h"][sel], want_h, f"tail h b={b}")
    want_n, want_o = oracle.combine_norm_upproj(up["lat"][:, sel], up["gamma"], up["eps"],
                                                up["w_up"], want_rs, nthreads=NT)
    assert np.array_equal(fused["normed"][sel], want_n)
    gemm_bar(fused["out"][sel], want_o, f"tail out b={b}")
    fused2, _ = run_tail_and_calls(up, sh, with_opt=False)  # rs, y, h in the workspace
    assert np.array_equal(fused2["out"], fused["out"])


@pytest.mark.parametrize("b,tp,L,H,I", [(5, 3, 544, 256, 128), (17, 1, 32, 64, 64),
                                        (40, 2, 1024, 512, 192), (3, 32, 8192, 128, 1024)])
def test_tail_ragged(b, tp, L, H, I):
    up = workloads.upproj(b + L, b=b, tp=tp, L=L, N=H)
    sh = workloads.shared(b + H, b=b, H=H, I=I)
    fused, calls = run_tail_and_calls(up, sh)
    for k in ("out", "rs", "normed", "h"):
        assert np.array_equal(fused[k], calls[k]), k
    want_h, want_rs = oracle.shared_expert(sh["x"], sh["w_gate"], sh["w_up"], sh["w_down"],
                                           nthreads=NT)
    gemm_bar(fused["rs"], want_rs, "tail rs")
    want_n, want_o = oracle.combine_norm_upproj(up["lat"], up["gamma"], up["eps"], up["w_up"],
                                                want_rs, nthreads=NT)
    assert np.array_equal(fused["normed"], want_n)
    gemm_bar(fused["out"], want_o, "tail out")


TAIL_OVERRIDES = [
    dict(DOWN_PASSES=2, DOWN_BLOCKS=16),                      # down multi-pass, up single-pass
    dict(UPPROJ_PASSES=2, UPPROJ_BLOCKS=16, DOWN_SPLITS=3),   # down single-pass, ragged last slice
    dict(DOWN_PASSES=2, DOWN_BLOCKS=16, UPPROJ_SPLITS=3),     # up single-pass, ragged last slice
    dict(DOWN_PASSES=4, DOWN_BLOCKS=8, UPPROJ_PASSES=2, UPPROJ_BLOCKS=8),
    dict(GATEUP_PASSES=2, GATEUP_BLOCKS=16, DOWN_PASSES=1, UPPROJ_PASSES=1),
    # the single-pass side planned with 2-tile units (run one tile a unit)
    dict(DOWN_PASSES=2, DOWN_BLOCKS=16, UPPROJ_MR=2, UPPROJ_PF=4, UPPROJ_WAVES=7, UPPROJ_SPLITS=2),
]


@pytest.mark.parametrize("b", [8, 40])
def test_tail_plan_overrides(b):
    """The fused tail's grouped launch in its multi-pass form (either side
    multi-pass, the other run as one pass, with a shorter last slice) gives
    the bits of the two calls, and both match the oracle."""
    tp, L, H, I = 2, 1024, 512, 320
    up = workloads.upproj(90 + b, b=b, tp=tp, L=L, N=H)
    sh = workloads.shared(95 + b, b=b, H=H, I=I)
    want_h, want_rs = oracle.shared_expert(sh["x"], sh["w_gate"], sh["w_up"], sh["w_down"],
                                           nthreads=NT)
    want_o = oracle.combine_norm_upproj(up["lat"], up["gamma"], up["eps"], up["w_up"], want_rs,
                                        nthreads=NT)[1]
    for ov in TAIL_OVERRIDES:
        with mt.projection_tuning(tuning_of(ov)):
            fused, calls = run_tail_and_calls(up, sh, layout=mt.W_TILED)
        for k in ("out", "rs", "normed", "h"):
            assert np.array_equal(fused[k], calls[k]), f"{k} {ov}"
        gemm_bar(fused["h"], want_h, f"tail h b={b} {ov}")
        gemm_bar(fused["rs"], want_rs, f"tail rs b={b} {ov}")
        gemm_bar(fused["out"], want_o, f"tail out b={b} {ov}")


def test_tail_graph_replay():
    up = workloads.upproj(5, b=64)
    sh = workloads.shared(5, b=64)
    lat, gamma, w_up = dev(up["lat"]), dev(up["gamma"]), dev(up["w_up"])
    x, wg, wu, wd = dev(sh["x"]), dev(sh["w_gate"]), dev(sh["w_up"]), dev(sh["w_down"])
    out, rs = empty_bf16(64, 7168), empty_bf16(64, 7168)
    ws = mt.new_workspace(mt.OP_TAIL, 64, 3584, 7168, 6144)

    def call():
        mt.moetail_tail(lat, gamma, 1e-6, w_up, x, wg, wu, wd, out, rs=rs, workspace=ws)

    call()
    eager = (host(out), host(rs))
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    for _ in range(3):
        out.fill_(SENTINEL)
        rs.fill_(SENTINEL)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out), eager[0]) and np.array_equal(host(rs), eager[1])


@pytest.mark.parametrize("b,tp,L,H,I,layout", [(64, 8, 3584, 7168, 6144, mt.W_TILED),
                                               (32, 8, 3584, 7168, 6144, mt.W_ROWS),
                                               (5, 3, 544, 256, 128, mt.W_ROWS),
                                               (40, 2, 1024, 512, 192, mt.W_TILED)])
def test_gate_up_is_the_shared_expert_h_and_the_norm(b, tp, L, H, I, layout):
    """moetail_gate_up forms h and y in one launch: the bits of
    moetail_shared_expert's h and moetail_combine_norm_upproj's normed, with
    and without y, and again on the same workspace (its counters back at
    zero)."""
    up = workloads.upproj(b + L + 1, b=b, tp=tp, L=L, N=H)
    sh = workloads.shared(b + H + 1, b=b, H=H, I=I)
    lat, gamma = dev(up["lat"]), dev(up["gamma"])
    x, wg, wu, wd = (dev(sh["x"]), weight(sh["w_gate"], layout), weight(sh["w_up"], layout),
                     weight(sh["w_down"], layout))
    h_ref, rs = empty_bf16(b, I), empty_bf16(b, H)
    mt.moetail_shared_expert(x, wg, wu, wd, rs, h=h_ref,
                             workspace=mt.new_workspace(mt.OP_SHARED_EXPERT, b, H, I),
                             w_layout=layout)
    y_ref, out = empty_bf16(b, L), empty_bf16(b, H)
    mt.moetail_combine_norm_upproj(lat, gamma, up["eps"], weight(up["w_up"], layout), out,
                                   normed=y_ref,
                                   workspace=mt.new_workspace(mt.OP_COMBINE_NORM_UPPROJ, b, L,
                                                              H, tp), w_layout=layout)
    ws = mt.new_workspace(mt.OP_GATE_UP, b, H, I)
    for with_y in (True, False, True):
        h, y = empty_bf16(b, I), empty_bf16(b, L)
        if with_y:
            mt.moetail_gate_up(x, wg, wu, h, lat, gamma, up["eps"], y, workspace=ws,
                               w_layout=layout)
            assert np.array_equal(host(y), host(y_ref))
        else:
            mt.moetail_gate_up(x, wg, wu, h, workspace=ws, w_layout=layout)
        assert np.array_equal(host(h), host(h_ref)), with_y
        assert int(ws[: 4 * (I // 16)].view(torch.int32).abs().sum()) == 0


def test_tail_counters_back_to_zero():
    """The fused tail forms its split sums in its own launches with per-tile
    counters at the start of the workspace (I/16 h-tile words, then H/16
    output-tile words), which must be zero when a call starts.  Every call
    leaves them at zero: back-to-back calls on one workspace, at token counts
    of different plans, give the bits of calls on fresh workspaces."""
    L, H, I, tp = 544, 256, 128, 3
    sizes = (40, 5, 40, 1)
    ws = torch.zeros(max(mt.workspace_bytes(mt.OP_TAIL, b, L, H, I) for b in sizes),
                     dtype=torch.uint8, device="cuda")
    words = I // 16 + H // 16
    for k, b in enumerate(sizes):
        up = workloads.upproj(b + k, b=b, tp=tp, L=L, N=H)
        sh = workloads.shared(b + 7 * k, b=b, H=H, I=I)
        args = (dev(up["lat"]), dev(up["gamma"]), up["eps"], dev(up["w_up"]), dev(sh["x"]),
                dev(sh["w_gate"]), dev(sh["w_up"]), dev(sh["w_down"]))
        out, rs = empty_bf16(b, H), empty_bf16(b, H)
        mt.moetail_tail(*args, out, rs=rs, workspace=ws)
        torch.cuda.synchronize()
        assert int(ws[: 4 * words].view(torch.int32).abs().sum()) == 0, f"b={b}"
        out2, rs2 = empty_bf16(b, H), empty_bf16(b, H)
        mt.moetail_tail(*args, out2, rs=rs2, workspace=mt.new_workspace(mt.OP_TAIL, b, L, H, I))
        assert np.array_equal(host(out), host(out2)) and np.array_equal(host(rs), host(rs2)), b


# ------------------------------- finalize without a per-route norm (Kimi) --

def run_plain(inp, wkey="w32", mode="both", gamma=True):
    tp, b, P = inp["tp"], inp["b"], inp["P"]
    partials = empty_bf16(tp, b, P) if mode in ("both", "partials") else None
    out = empty_bf16(b, P) if mode in ("both", "out") else None
    mt.moetail_finalize(dev(inp["rows"]), dev(inp["idx"]), dev(inp[wkey]),
                        dev(inp["gamma"]) if gamma else None, 0.0, 1e-6, mt.NO_NORM,
                        partials=partials, out=out)
    return (host(partials) if partials is not None else None,
            host(out) if out is not None else None)


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("wkey", ["w32", "w16"])
def test_plain_decode_scale(seed, wkey):
    """b=64, top-16 over tp=8 ranks, P=3584: the route-weighted sum, all modes."""
    inp = workloads.ep_finalize(seed)
    want_p, want_o = oracle.finalize_plain(inp["rows"], inp["idx"], inp[wkey], nthreads=NT)
    got_p, got_o = run_plain(inp, wkey)
    assert np.array_equal(got_p, want_p) and np.array_equal(got_o, want_o)
    _, only_o = run_plain(inp, wkey, "out", gamma=False)
    only_p, _ = run_plain(inp, wkey, "partials", gamma=False)
    assert np.array_equal(only_o, want_o) and np.array_equal(only_p, want_p)


def test_plain_expanded_rows():
    """The Kimi layout: one rank, expanded rows [b*K, P] with row t*K + k."""
    b, K, P = 64, 16, 3584
    rng = np.random.default_rng(31)
    rows = bits(rng.standard_normal((1, b * K, P)) * 2)
    idx = np.arange(b * K, dtype=np.int32).reshape(1, b, K)
    g0 = torch.Generator("cpu").manual_seed(31)
    w32, w16 = workloads.route_weights(g0, b, K)
    inp = dict(rows=rows, idx=idx, w32=w32, w16=w16, gamma=np.zeros(P, np.uint16), tp=1, b=b,
               P=P)
    for wkey in ("w32", "w16"):
        want_p, want_o = oracle.finalize_plain(rows, idx, inp[wkey], nthreads=NT)
        for mode in ("out", "partials"):
            got_p, got_o = run_plain(inp, wkey, mode, gamma=False)
            if got_o is not None:
                assert np.array_equal(got_o, want_o)
            if got_p is not None:
                assert np.array_equal(got_p, want_p)


@pytest.mark.parametrize("b,K,P,tp", [(5, 3, 520, 3), (3, 7, 8, 1), (2, 32, 8192, 4),
                                      (17, 8, 7168, 8), (3, 32, 64, 32)])
def test_plain_ragged(b, K, P, tp):
    if K % tp == 0:
        inp = workloads.ep_finalize(b * 5 + K, b=b, K=K, P=P, tp=tp, outlier_frac=0.05)
    else:
        inp = workloads.ep_finalize(b, b=b, K=K, P=P, tp=1, outlier_frac=0.0)
        rows1 = inp["rows"][0]
        idx = np.full((tp, b, K), -1, np.int32)
        for k in range(K):
            idx[k % tp, :, k] = inp["idx"][0, :, k]
        inp.update(rows=np.ascontiguousarray(np.broadcast_to(rows1, (tp,) + rows1.shape)),
                   idx=idx, tp=tp)
    want_p, want_o = oracle.finalize_plain(inp["rows"], inp["idx"], inp["w32"], nthreads=NT)
    got_p, got_o = run_plain(inp)
    assert np.array_equal(got_p, want_p) and np.array_equal(got_o, want_o)
    _, only_o = run_plain(inp, mode="out")
    assert np.array_equal(only_o, want_o)


def test_plain_route_order():
    P = 8
    inp = dict(rows=bits(np.ones((1, 3, P))), idx=np.arange(3, dtype=np.int32).reshape(1, 1, 3),
               w32=np.array([[2.0 ** 25, -2.0 ** 25, 1.0]], np.float32),
               gamma=np.zeros(P, np.uint16), tp=1, b=1, P=P)
    for mode in ("out", "both"):
        _, got_o = run_plain(inp, mode=mode, gamma=False)
        assert [f"{int(v):04x}" for v in got_o.ravel()] == ["3f80"] * P


# ---------------------------------------------------- tiled weight layout --

def tiled_reference(w: np.ndarray) -> np.ndarray:
    """The tiled layout written out with numpy: block (t, s) of 16 rows and
    32 columns in MFMA operand order, lane l = r + 16 q holding row 16 t + r,
    columns 32 s + 8 q .. 32 s + 8 q + 7."""
    n, k = w.shape
    return w.reshape(n // 16, 16, k // 32, 4, 8).transpose(0, 2, 3, 1, 4).reshape(n, k)


@pytest.mark.parametrize("n,k", [(16, 32), (48, 96), (192, 1024), (7168, 3584)])
def test_pack_weights_layout(n, k):
    w = np.random.default_rng(n + k).integers(0, 1 << 16, (n, k), dtype=np.uint16)
    got = host(mt.pack_weights(dev(w)))
    assert np.array_equal(got, tiled_reference(w))
    # the first fragment, spelled out: lane 17 = row 1, columns 8..15
    assert np.array_equal(got.reshape(-1)[17 * 8:18 * 8], w[1, 8:16])


@pytest.mark.parametrize("b", [1, 32, 64])
def test_tiled_weights_same_bits_upproj(b):
    inp = workloads.upproj(40 + b, b=b, with_rs=True)
    rows = run_upproj(inp, rs=inp["rs"])
    tiled = run_upproj(inp, rs=inp["rs"], layout=mt.W_TILED)
    assert np.array_equal(rows[0], tiled[0]) and np.array_equal(rows[1], tiled[1])


@pytest.mark.parametrize("b,H,I", [(1, 7168, 6144), (64, 7168, 6144), (128, 1024, 2048),
                                   (5, 512, 256), (33, 256, 128)])
def test_tiled_weights_same_bits_shared(b, H, I):
    inp = workloads.shared(50 + b, b=b, H=H, I=I)
    h0, rs0 = run_shared(inp)
    h1, rs1 = run_shared(inp, layout=mt.W_TILED)
    assert np.array_equal(h0, h1) and np.array_equal(rs0, rs1)
    if H * I <= 1 << 20:
        want_h, want_rs = oracle.shared_expert(inp["x"], inp["w_gate"], inp["w_up"],
                                               inp["w_down"], nthreads=NT)
        gemm_bar(h1, want_h, "tiled h")
        gemm_bar(rs1, want_rs, "tiled rs")


@pytest.mark.parametrize("b,tp,L,H,I", [(64, 8, 3584, 7168, 6144), (5, 3, 544, 256, 128),
                                        (128, 2, 1024, 512, 192)])
def test_tiled_weights_same_bits_tail(b, tp, L, H, I):
    """The fused tail on tiled weights = the two calls on row-major weights."""
    up = workloads.upproj(60 + b, b=b, tp=tp, L=L, N=H)
    sh = workloads.shared(70 + b, b=b, H=H, I=I)
    fused, calls = run_tail_and_calls(up, sh, layout=mt.W_TILED, calls_layout=mt.W_ROWS)
    for key in ("out", "rs", "normed", "h"):
        assert np.array_equal(fused[key], calls[key]), key


# ------------------------------------------------ projection partials --

def partial_sums(part, kind_rows, b):
    """The FP32 partials of moetail_projection_partials as [splits][b][N]
    (the accumulator layout the header gives), padded tokens dropped."""
    N = kind_rows
    T = 16 * next(n for n in (1, 2, 4, 8) if b <= 16 * n)
    a = part.reshape(-1, N // 16, T // 16, 4, 16, 4)  # s, tile, tok block, row quad, tok, row
    a = a.transpose(0, 2, 4, 1, 3, 5).reshape(-1, T, N)
    return a[:, :b, :]


@pytest.mark.parametrize("b", [1, 32, 64])
def test_projection_partials_up_against_oracle(b):
    """The up projection's split-K stage alone: the partials added in split
    order, rounded to BF16, are the oracle's out (y = the oracle's normed
    input, no rs) within the GEMM bar."""
    up = workloads.upproj(80 + b, b=b)
    want_n, want_o = oracle.combine_norm_upproj(up["lat"], up["gamma"], up["eps"], up["w_up"],
                                                None, nthreads=NT)
    w = mt.pack_weights(dev(up["w_up"]))
    x = dev(want_n)
    N, K = up["w_up"].shape
    n = mt.workspace_bytes(mt.OP_PROJECTION, b, N, K, mt.PROJ_UPPROJ)
    part = torch.empty(n // 4, dtype=torch.float32, device="cuda")
    mt.moetail_projection_partials(mt.PROJ_UPPROJ, w, None, x, part, w_layout=mt.W_TILED)
    sums = partial_sums(part.cpu().numpy(), N, b)
    acc = np.zeros((b, N), np.float32)
    for s_ in sums:
        acc = acc + s_
    acc[acc == 0] = 0.0  # -0 as +0, as the calls write
    gemm_bar(oracle.bf16_round(acc), want_o, "partials out")


def test_projection_partials_are_the_shared_experts():
    """The down projection's partials of moetail_projection_partials, added
    in split order from +0 and rounded to BF16 (-0 as +0), are the rs that
    moetail_shared_expert returns for the same h: the same stage, the same
    sums, bit for bit."""
    b = 64
    sh = workloads.shared(85, b=b)
    wg, wu, wd = (mt.pack_weights(dev(a)) for a in (sh["w_gate"], sh["w_up"], sh["w_down"]))
    x = dev(sh["x"])
    H, I = sh["H"], sh["I"]
    h, rs = empty_bf16(b, I), empty_bf16(b, H)
    ws = mt.new_workspace(mt.OP_SHARED_EXPERT, b, H, I)
    mt.moetail_shared_expert(x, wg, wu, wd, rs, h=h, workspace=ws, w_layout=mt.W_TILED)
    n = mt.workspace_bytes(mt.OP_PROJECTION, b, H, I, mt.PROJ_DOWN)
    part = torch.empty(n // 4, dtype=torch.float32, device="cuda")
    mt.moetail_projection_partials(mt.PROJ_DOWN, wd, None, h, part, w_layout=mt.W_TILED)
    sums = partial_sums(part.cpu().numpy(), H, b)
    acc = np.zeros((b, H), np.float32)
    for s_ in sums:
        acc = acc + s_
    acc[acc == 0] = 0.0  # -0 as +0
    assert np.array_equal(oracle.bf16_round(acc), host(rs))
    # gate/up: both matrices, the same call shape
    n = mt.workspace_bytes(mt.OP_PROJECTION, b, 2 * I, H, mt.PROJ_GATEUP)
    part = torch.empty(n // 4, dtype=torch.float32, device="cuda")
    mt.moetail_projection_partials(mt.PROJ_GATEUP, wg, wu, x, part, w_layout=mt.W_TILED)
    assert np.isfinite(part.cpu().numpy()).all()


@pytest.mark.parametrize("b,L,N,layout", [(32, 3584, 7168, mt.W_TILED), (17, 3584, 7168, mt.W_ROWS),
                                          (9, 3584, 7168, mt.W_ROWS), (1, 3584, 7168, mt.W_TILED),
                                          (32, 3616, 7168, mt.W_TILED), (5, 128, 256, mt.W_ROWS),
                                          (20, 128, 256, mt.W_TILED), (64, 3584, 7168, mt.W_TILED),
                                          (50, 3616, 7168, mt.W_ROWS), (40, 128, 256, mt.W_TILED)])
def test_upproj_block_sums_are_the_split_k_stage(b, L, N, layout):
    """Up to 64 tokens the up projection adds its K splits inside its blocks
    (one launch after the norm).  Its out is, bit for bit, the split-K
    stage's partials of the same y added in split order from +0, plus rs,
    rounded once (-0 as +0).
    L = 3616: 4 splits of 928 columns, the last one shorter; 128 -> 256: 4
    splits of one k step."""
    up = workloads.upproj(90 + b, b=b, L=L, N=N, with_rs=True)
    w = weight(up["w_up"], layout)
    lat, gamma, rs = dev(up["lat"]), dev(up["gamma"]), dev(up["rs"])
    out, normed = empty_bf16(b, N), empty_bf16(b, L)
    ws = mt.new_workspace(mt.OP_COMBINE_NORM_UPPROJ, b, L, N, up["tp"])
    mt.moetail_combine_norm_upproj(lat, gamma, up["eps"], w, out, rs=rs, normed=normed,
                                   workspace=ws, w_layout=layout)
    n = mt.workspace_bytes(mt.OP_PROJECTION, b, N, L, mt.PROJ_UPPROJ)
    part = torch.empty(n // 4, dtype=torch.float32, device="cuda")
    mt.moetail_projection_partials(mt.PROJ_UPPROJ, w, None, normed, part, w_layout=layout)
    acc = np.zeros((b, N), np.float32)
    for s_ in partial_sums(part.cpu().numpy(), N, b):
        acc = acc + s_
    acc = acc + oracle.f32(up["rs"])
    acc[acc == 0] = 0.0  # -0 as +0
    assert np.array_equal(oracle.bf16_round(acc), host(out))


@pytest.mark.parametrize("b", [1, 11, 20, 32, 50, 64, 100])
def test_shared_down_block_sums_are_the_split_k_stage(b):
    """The shared expert's down projection (summed inside its blocks up to 64
    tokens): rs is, bit for bit, the split-K stage's partials of the same h
    added in split order from +0 and rounded once (-0 as +0)."""
    sh = workloads.shared(95 + b, b=b)
    wg, wu, wd = (mt.pack_weights(dev(a)) for a in (sh["w_gate"], sh["w_up"], sh["w_down"]))
    x = dev(sh["x"])
    H, I = sh["H"], sh["I"]
    h, rs = empty_bf16(b, I), empty_bf16(b, H)
    ws = mt.new_workspace(mt.OP_SHARED_EXPERT, b, H, I)
    mt.moetail_shared_expert(x, wg, wu, wd, rs, h=h, workspace=ws, w_layout=mt.W_TILED)
    n = mt.workspace_bytes(mt.OP_PROJECTION, b, H, I, mt.PROJ_DOWN)
    part = torch.empty(n // 4, dtype=torch.float32, device="cuda")
    mt.moetail_projection_partials(mt.PROJ_DOWN, wd, None, h, part, w_layout=mt.W_TILED)
    acc = np.zeros((b, H), np.float32)
    for s_ in partial_sums(part.cpu().numpy(), H, b):
        acc = acc + s_
    acc[acc == 0] = 0.0  # -0 as +0
    assert np.array_equal(oracle.bf16_round(acc), host(rs))


# ------------------------------------------------- the fused decode tail --

def run_decode_tail(ep, up, sh, mode, wkey="w32", layout=mt.W_TILED):
    """moetail_decode_tail, and moetail_finalize (partials) then moetail_tail,
    on the same inputs: (fused outputs, separate outputs)."""
    tp, b, L = ep["tp"], ep["b"], ep["P"]
    H, I = sh["H"], sh["I"]
    rows, idx, w = dev(ep["rows"]), dev(ep["idx"]), dev(ep[wkey])
    fg = dev(ep["gamma"]) if mode != mt.NO_NORM else None
    gamma, x = dev(up["gamma"]), dev(sh["x"])
    w_up, wg, wu, wd = (weight(up["w_up"], layout), weight(sh["w_gate"], layout),
                        weight(sh["w_up"], layout), weight(sh["w_down"], layout))
    res = []
    for fused in (True, False):
        lat, out = empty_bf16(tp, b, L), empty_bf16(b, H)
        rs, normed, h = empty_bf16(b, H), empty_bf16(b, L), empty_bf16(b, I)
        ws = mt.new_workspace(mt.OP_TAIL, b, L, H, I)
        if fused:
            mt.moetail_decode_tail(rows, idx, w, fg, ep["gain_center"], ep["eps"], mode, lat, gamma,
                                   up["eps"], w_up, x, wg, wu, wd, out, rs=rs, normed=normed, h=h,
                                   workspace=ws, w_layout=layout)
        else:
            mt.moetail_finalize(rows, idx, w, fg, ep["gain_center"], ep["eps"], mode, partials=lat)
            mt.moetail_tail(lat, gamma, up["eps"], w_up, x, wg, wu, wd, out, rs=rs, normed=normed,
                            h=h, workspace=ws, w_layout=layout)
        res.append(dict(lat=host(lat), out=host(out), rs=host(rs), normed=host(normed),
                        h=host(h)))
    return res


@pytest.mark.parametrize("mode,wkey", [(mt.NORM_GAIN_FIRST, "w32"), (mt.NORM_GAIN_AFTER, "w16"),
                                       (mt.NO_NORM, "w32")])
def test_decode_tail_decode_scale(mode, wkey):
    """c2 rows (b=64, K=16, P=3584, tp=8) into c4/c5's tail: the same bits as
    the two calls, and the partials are the oracle's."""
    ep = workloads.ep_finalize(90)
    up = workloads.upproj(91, b=64)
    sh = workloads.shared(92, b=64)
    fused, calls = run_decode_tail(ep, up, sh, mode, wkey)
    for key in ("lat", "out", "rs", "normed", "h"):
        assert np.array_equal(fused[key], calls[key]), key
    if mode == mt.NO_NORM:
        want, _ = oracle.finalize_plain(ep["rows"], ep["idx"], ep[wkey], combine=False,
                                        nthreads=NT)
    else:
        want, _ = oracle.finalize(ep["rows"], ep["idx"], ep[wkey], ep["gamma"], ep["gain_center"],
                                  ep["eps"], mode == mt.NORM_GAIN_FIRST, combine=False,
                                  nthreads=NT)
    assert np.array_equal(fused["lat"], want)


@pytest.mark.parametrize("b,K,tp,L,H,I,layout", [(5, 6, 3, 544, 256, 128, mt.W_ROWS),
                                                 (128, 16, 8, 3584, 512, 192, mt.W_TILED),
                                                 (3, 4, 2, 8192, 128, 64, mt.W_TILED),
                                                 (17, 7, 1, 32, 64, 64, mt.W_ROWS)])
def test_decode_tail_ragged(b, K, tp, L, H, I, layout):
    """Ragged shapes, b = 128 (8 token blocks), and rows too wide for the side
    job (P = 8192: the finalize runs as a launch of its own)."""
    ep = workloads.ep_finalize(b + L, b=b, K=K, P=L, tp=tp)
    up = workloads.upproj(b + H, b=b, tp=tp, L=L, N=H)
    sh = workloads.shared(b + I, b=b, H=H, I=I)
    fused, calls = run_decode_tail(ep, up, sh, mt.NORM_GAIN_FIRST, layout=layout)
    for key in ("lat", "out", "rs", "normed", "h"):
        assert np.array_equal(fused[key], calls[key]), key


@pytest.mark.parametrize("mode", [mt.NORM_GAIN_AFTER, mt.NORM_GAIN_FIRST, mt.NO_NORM])
@pytest.mark.parametrize("wkey", ["w32", "w16"])
def test_decode_tail_finalize_waves_every_mode(mode, wkey):
    """The decode tail at the tail's real sizes (b=16): the rank partials are
    the oracle's bit for bit in every norm mode and route-weight type, and
    every output equals the two separate calls."""
    ep = workloads.ep_finalize(40 + mode, b=16)
    up = workloads.upproj(41, b=16)
    sh = workloads.shared(42, b=16)
    fused, calls = run_decode_tail(ep, up, sh, mode, wkey)
    if mode == mt.NO_NORM:
        want, _ = oracle.finalize_plain(ep["rows"], ep["idx"], ep[wkey], combine=False,
                                        nthreads=NT)
    else:
        want, _ = oracle.finalize(ep["rows"], ep["idx"], ep[wkey], ep["gamma"], ep["gain_center"],
                                  ep["eps"], mode == mt.NORM_GAIN_FIRST, combine=False,
                                  nthreads=NT)
    assert np.array_equal(fused["lat"], want)
    for key in ("lat", "out", "rs", "normed", "h"):
        assert np.array_equal(fused[key], calls[key]), key


def test_decode_tail_bench_config_against_oracle():
    """The benchmark's launch configuration -- moetail_decode_tail at b=64 on
    tiled weights, c2 rows into c4/c5's tail -- against the oracle: the rank
    partials and y bit-exact, h, rs and out within the GEMM bar on a sample of
    tokens (tokens are independent)."""
    ep = workloads.ep_finalize(0)
    up = workloads.upproj(0, b=64)
    sh = workloads.shared(0, b=64)
    fused, _ = run_decode_tail(ep, up, sh, mt.NORM_GAIN_FIRST)
    want_lat, _ = oracle.finalize(ep["rows"], ep["idx"], ep["w32"], ep["gamma"], ep["gain_center"],
                                  ep["eps"], True, combine=False, nthreads=NT)
    assert np.array_equal(fused["lat"], want_lat)
    sel = sample_tokens(64)
    want_h, want_rs = oracle.shared_expert(sh["x"][sel], sh["w_gate"], sh["w_up"], sh["w_down"],
                                           nthreads=NT)
    gemm_bar(fused["h"][sel], want_h, "decode tail h")
    gemm_bar(fused["rs"][sel], want_rs, "decode tail rs")
    want_n, want_o = oracle.combine_norm_upproj(want_lat[:, sel], up["gamma"], up["eps"],
                                                up["w_up"], want_rs, nthreads=NT)
    assert np.array_equal(fused["normed"][sel], want_n)
    gemm_bar(fused["out"][sel], want_o, "decode tail out")


def test_decode_tail_graph_replay():
    """Graph replays of the benchmark's call, with eager work and host
    synchronizations between them: every replay gives the eager bits."""
    ep = workloads.ep_finalize(7)
    up = workloads.upproj(7, b=64)
    sh = workloads.shared(7, b=64)
    rows, idx, w, fg = dev(ep["rows"]), dev(ep["idx"]), dev(ep["w32"]), dev(ep["gamma"])
    gamma, x = dev(up["gamma"]), dev(sh["x"])
    w_up, wg, wu, wd = (mt.pack_weights(dev(a)) for a in (up["w_up"], sh["w_gate"], sh["w_up"],
                                                          sh["w_down"]))
    lat, out, rs = empty_bf16(8, 64, 3584), empty_bf16(64, 7168), empty_bf16(64, 7168)
    ws = mt.new_workspace(mt.OP_TAIL, 64, 3584, 7168, 6144)

    def call():
        mt.moetail_decode_tail(rows, idx, w, fg, ep["gain_center"], ep["eps"], True, lat, gamma,
                               up["eps"], w_up, x, wg, wu, wd, out, rs=rs, workspace=ws,
                               w_layout=mt.W_TILED)

    call()
    eager = (host(lat), host(out), host(rs))
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    for _ in range(3):
        for t in (lat, out, rs):
            t.fill_(SENTINEL)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (host(lat), host(out), host(rs))
        for a, b_ in zip(got, eager):
            assert np.array_equal(a, b_)
