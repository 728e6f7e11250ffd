"""Pins of the CPU oracle against what the pages and the mathematics fix.

CPU only.  Nothing here calls the HIP library: the oracle is checked against
hand-derived golden cases (tests/golden), closed forms, invariants, library
routines (torch's BF16 cast and rms_norm) and an independent FP64
straight-line evaluation (tests/fp64_ref.py) within the FP32 error bound.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import exact_ref as X
from tests import fp64_ref as ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
U24 = ref.U24


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def bits(values):
    return oracle.bf16_round(np.asarray(values, np.float32))


def hexes(a):
    return [f"{int(v):04x}" for v in np.asarray(a).ravel()]


# ------------------------------------------------------------------ BF16 --

def _special_floats():
    rng = np.random.default_rng(1)
    vals = [0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, 3.3895314e38, 3.4e38,
            -3.4e38, 1e-40, -1e-40, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135,
            2.0 ** -149, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20]
    # exact ties and near-ties at many binades
    mant = rng.integers(0, 1 << 23, size=4000, dtype=np.uint32)
    expo = rng.integers(1, 254, size=4000, dtype=np.uint32)
    sign = rng.integers(0, 2, size=4000, dtype=np.uint32)
    u = (sign << 31) | (expo << 23) | mant
    ties = (u & 0xFFFF0000) | 0x8000
    sub = rng.integers(1, 1 << 23, size=500, dtype=np.uint32)
    arr = np.concatenate([np.array(vals, np.float32), u.view(np.float32),
                          ties.view(np.float32), sub.view(np.float32),
                          rng.standard_normal(4000).astype(np.float32)])
    return arr


def test_bf16_round_matches_torch_cast():
    x = _special_floats()
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_round(x)
    assert np.array_equal(got, want)


def test_bf16_round_matches_fp64_definition():
    x = _special_floats()
    x = x[np.isfinite(x) & (np.abs(x) < 3.38e38)]
    got = oracle.f32(oracle.bf16_round(x)).astype(np.float64)
    want = ref.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, want)
    nan = oracle.bf16_round(np.array([np.nan], np.float32))
    assert (int(nan[0]) & 0x7F80) == 0x7F80 and (int(nan[0]) & 0x7F) != 0


# -------------------------------------------------------- sum of squares --

def _golden_row(case):
    if "values" not in case:
        v = np.full(case["P"], case["rest"], np.float32)
        v[0] = case["v0"]
        return v
    v = np.zeros(case["P"], np.float32)
    for cols, val in case["values"].items():
        lo, _, hi = cols.partition("..")
        v[int(lo): int(hi or lo) + 1] = val
    return v


def test_sum_of_squares_golden_tree():
    for case in golden("ss_tree.json")["cases"]:
        assert float(oracle.sum_of_squares(_golden_row(case))) == case["expected"]


def test_sum_of_squares_small_trees_exact():
    """P = 8: lane 0 adds the 8 squares in column order, every other lane
    holds 0.  P = 16: lanes 0 and 1 hold the ordered sums of columns 0..7
    and 8..15, and the butterfly's first level adds them.  Checked in exact
    arithmetic, each step rounded to FP32, on rows where the orders matter."""
    rng = np.random.default_rng(31)
    for _ in range(200):
        v = (rng.standard_normal(16) * rng.choice([1.0, 1e3, 1e-3], 16)).astype(np.float32)
        lanes = []
        for lo in (0, 8):
            s = Fraction(0)
            for c in range(lo, lo + 8):
                s = X.add(s, X.mul(Fraction(float(v[c])), Fraction(float(v[c]))))
            lanes.append(s)
        assert Fraction(float(oracle.sum_of_squares(v[:8]))) == lanes[0]
        assert Fraction(float(oracle.sum_of_squares(v))) == X.add(lanes[0], lanes[1])


def test_sum_of_squares_seq_order():
    """The SEQ order is the plain column-order sum (the 2^24 golden row gives
    2^24: every +1 after the first square ties back)."""
    v = _golden_row(golden("ss_tree.json")["cases"][0])
    with oracle.ss_order(oracle.SS_SEQ):
        assert float(oracle.sum_of_squares(v)) == 2.0 ** 24
        w = np.arange(1, 17, dtype=np.float32) * 1.37
        s = Fraction(0)
        for c in range(16):
            s = X.add(s, X.mul(Fraction(float(w[c])), Fraction(float(w[c]))))
        assert Fraction(float(oracle.sum_of_squares(w))) == s
    assert float(oracle.sum_of_squares(v)) == 2.0 ** 24 + 504  # W64 again after the block


# ---------------------------------------------------- inverse RMS ---------

def _bits32(x):
    return int(np.float32(x).view(np.uint32))


def test_inv_rms_golden():
    for case in golden("inv_rms.json")["cases"]:
        ss = np.uint32(int(case["ss_hex"], 16)).view(np.float32)
        assert float(ss) == case["ss"]
        got = oracle.inv_rms(ss, case["P"], case["eps"])
        assert _bits32(got) == int(case["expected_hex"], 16), case["what"]
        # the derivation, redone in exact arithmetic, and the other reading
        # really gives another value
        m = X.add(X.mul(Fraction(float(ss)), X.rne(Fraction(1, case["P"]))), Fraction(case["eps"]))
        assert X.f32_bits(X.rsqrt(m)) == int(case["expected_hex"], 16)
        ((reading, other),) = case["other_reading"].items()
        if reading.startswith("ss / P"):
            alt = X.rsqrt(X.add(X.div(Fraction(float(ss)), case["P"]), Fraction(case["eps"])))
        else:
            alt = X.div(1, X.sqrt(m))
        assert X.f32_bits(alt) == int(other, 16) != int(case["expected_hex"], 16)


@pytest.mark.parametrize("P", [512, 520, 3584, 7168])
def test_inv_rms_exact(P):
    """1/sqrt(ss * fp32(1/P) + eps) with each step rounded to FP32 and the
    reciprocal square root correctly rounded, in exact arithmetic."""
    rng = np.random.default_rng(P)
    ss = (rng.uniform(0.5, 2.0, 150) * P * rng.choice([1.0, 4.0, 0.01], 150)).astype(np.float32)
    inv_p = X.rne(Fraction(1, P))
    for eps in (0.0, 1e-6):
        e = Fraction(float(np.float32(eps)))
        for s in ss:
            m = X.add(X.mul(Fraction(float(s)), inv_p), e)
            assert _bits32(oracle.inv_rms(s, P, eps)) == X.f32_bits(X.rsqrt(m))


# ---------------------------------------------- normalized route products --

def _bf16_of(vals):
    return oracle.bf16_round(np.asarray(vals, np.float32))


def test_route_products_golden():
    case = golden("route_products.json")["case"]
    x = _bf16_of(case["x"])
    gamma = np.full(case["P"], int(case["gamma_hex"], 16), np.uint16)
    for key, wbn in (("gain_after", False), ("gain_first", True)):
        got = oracle.route_products(x, gamma, case["gain_center"], case["w"], case["eps"], wbn)
        want = [int(h, 16) for h in case[key]["expected_hex"]]
        assert [_bits32(p) for p in got] == want, key
        assert int(case[key]["other_order_col0_hex"], 16) != want[0]


def _exact_route_products(x, gamma, gc, w, eps, wbn):
    """The page order, each step rounded to FP32 (rows of 8 or 16 columns:
    the sum of squares is the P = 8 / 16 tree of the test above)."""
    P = len(x)
    xs = [X.bf16_value(int(h)) for h in x]
    g = [X.add(X.bf16_value(int(h)), Fraction(float(np.float32(gc)))) for h in gamma]
    v = [X.mul(a, b) for a, b in zip(xs, g)] if wbn else xs
    lanes = []
    for lo in range(0, P, 8):
        s = Fraction(0)
        for c in range(lo, lo + 8):
            s = X.add(s, X.mul(v[c], v[c]))
        lanes.append(s)
    ss = lanes[0] if P == 8 else X.add(lanes[0], lanes[1])
    inv = X.rsqrt(X.add(X.mul(ss, X.rne(Fraction(1, P))), Fraction(float(np.float32(eps)))))
    wf = Fraction(float(np.float32(w)))
    if wbn:
        return [X.mul(X.mul(v[c], inv), wf) for c in range(P)]
    return [X.mul(X.mul(X.mul(xs[c], inv), g[c]), wf) for c in range(P)]


@pytest.mark.parametrize("wbn", [False, True])
def test_route_products_exact(wbn):
    rng = np.random.default_rng(41 + wbn)
    for P in (8, 16):
        for _ in range(60):
            x = bits(rng.standard_normal(P) * 2.0)
            gamma = bits(rng.standard_normal(P) * 0.3)
            gc = float(rng.choice([0.0, 1.0]))
            w = float(np.float32(rng.uniform(0.01, 1.0)))
            got = oracle.route_products(x, gamma, gc, w, 1e-6, wbn)
            want = _exact_route_products(x, gamma, gc, w, 1e-6, wbn)
            assert [_bits32(p) for p in got] == [X.f32_bits(p) for p in want]


@pytest.mark.parametrize("P", [8, 64, 512, 520, 1032, 3584, 7168])
def test_sum_of_squares_error_bound(P):
    rng = np.random.default_rng(P)
    v = (rng.standard_normal(P) * rng.choice([1e-3, 1.0, 40.0], P)).astype(np.float32)
    exact = float(np.sum(v.astype(np.float64) ** 2))
    got = float(oracle.sum_of_squares(v))
    depth = 8 + 6 + (P + 511) // 512 + 1
    assert abs(got - exact) <= 2 * depth * U24 * exact


def test_sum_of_squares_every_column_counts():
    # a dropped column or a skipped lane changes an exact integer sum
    for P in (8, 520, 3584):
        v = np.arange(1, P + 1, dtype=np.float32) % 7 + 1
        assert float(oracle.sum_of_squares(v)) == float(np.sum(v.astype(np.float64) ** 2))


# ------------------------------------------------------------ finalize ----

def _random_ep(rng, b, K, P, tp, R_extra=2):
    R = b * K + R_extra
    rows = bits(rng.standard_normal((tp, R, P)) * 2.0)
    idx = np.full((tp, b, K), -1, np.int32)
    for t in range(b):
        for k in range(K):
            d = int(rng.integers(0, tp))
            idx[d, t, k] = int(rng.integers(0, R))
    logits = rng.standard_normal((b, K))
    w = (np.exp(logits) / np.exp(logits).sum(1, keepdims=True)).astype(np.float32)
    gamma = bits(rng.standard_normal(P) * 0.1)
    return rows, idx, w, gamma


def _check_ep(rows, idx, w, gamma, gc, eps, wbn):
    partials, out = oracle.finalize(rows, idx, w, gamma, gc, eps, wbn)
    acc, scale = ref.ep_finalize(rows, idx, w, gamma, gc, eps, wbn)
    E = 64 * U24 * scale
    assert ref.within(partials, acc, E).all()
    tp = rows.shape[0]
    out_ref = acc.sum(axis=0)
    E_out = (E + ref.ulp_bf16(np.abs(acc) + E)).sum(axis=0) + 2 * tp * U24 * np.abs(acc).sum(axis=0)
    assert ref.within(out, out_ref, E_out).all()
    # the partials themselves: the nearest BF16 of the exact sum almost always
    exact_partials = oracle.bf16_round(ref.round_bf16(acc).astype(np.float32))
    assert np.mean(exact_partials == np.where(partials == 0x8000, 0, partials)) > 0.99
    return partials, out


@pytest.mark.parametrize("P,K,tp", [(8, 1, 1), (16, 2, 2), (64, 3, 3), (64, 4, 4),
                                    (520, 4, 2), (1032, 2, 3)])
@pytest.mark.parametrize("wbn", [True, False])
def test_ep_finalize_brute_force_fp64(P, K, tp, wbn):
    rng = np.random.default_rng(P * 100 + K * 10 + tp)
    rows, idx, w, gamma = _random_ep(rng, 3, K, P, tp)
    _check_ep(rows, idx, w, gamma, 1.0, 1e-6, wbn)
    _check_ep(rows, idx, bits(w), gamma, 0.25, 1e-5, wbn)  # BF16 route weights


def test_ep_finalize_tiny_workload_fp64():
    for wbn in (True, False):
        inp = workloads.tiny_ep_finalize(0)
        _check_ep(inp["rows"], inp["idx"], inp["w32"], inp["gamma"],
                  inp["gain_center"], inp["eps"], wbn)


def test_ep_finalize_outlier_rows_fp64():
    inp = workloads.ep_finalize(0, b=4, K=16, P=3584, tp=8, outlier_frac=0.2)
    for wbn in (True, False):
        _check_ep(inp["rows"], inp["idx"], inp["w32"], inp["gamma"],
                  inp["gain_center"], inp["eps"], wbn)


def test_single_route_is_rmsnorm():
    # one route, w = 1, tp = 1, no gain center: textbook RMSNorm x/rms*gamma
    rng = np.random.default_rng(7)
    P = 3584
    x = bits(rng.standard_normal((1, 1, P)) * 3)
    gamma = bits(1 + 0.05 * rng.standard_normal(P))
    idx = np.zeros((1, 1, 1), np.int32)
    w = np.ones((1, 1), np.float32)
    partials, out = oracle.finalize(x, idx, w, gamma, 0.0, 1e-6, False)
    assert np.array_equal(partials[0], out)
    want = torch.nn.functional.rms_norm(torch.from_numpy(ref.f64(x[0])), [P],
                                        weight=torch.from_numpy(ref.f64(gamma)),
                                        eps=1e-6).numpy()
    got = ref.f64(out)
    assert np.all(np.abs(got - want) <= ref.ulp_bf16(want))


def test_zero_route_weights_give_plus_zero():
    rng = np.random.default_rng(3)
    rows, idx, w, gamma = _random_ep(rng, 4, 4, 64, 2)
    for wz in (np.zeros_like(w), -np.zeros_like(w)):
        for wbn in (True, False):
            partials, out = oracle.finalize(rows, idx, wz, gamma, 1.0, 1e-6, wbn)
            assert not partials.any() and not out.any()


def test_rms_of_normalized_row_is_one():
    inp = workloads.ep_finalize(0, b=4, K=8, P=3584, tp=8, outlier_frac=0.1)
    rows = inp["rows"][:1, :4]
    gamma = np.zeros(3584, np.uint16)
    for r in range(4):
        idx = np.array([[[r]]], np.int32)
        for wbn in (True, False):
            _, out = oracle.finalize(rows, idx, np.ones((1, 1), np.float32), gamma,
                                     1.0, 1e-6, wbn)
            n = ref.f64(out)
            assert abs(np.mean(n * n) - 1.0) <= 2.0 ** -8


def test_gain_variants():
    rng = np.random.default_rng(11)
    rows, idx, w, _ = _random_ep(rng, 3, 4, 520, 2)
    zero = np.zeros(520, np.uint16)
    one = bits(np.ones(520))
    # (i) unit gain: both variants identical
    a = oracle.finalize(rows, idx, w, zero, 1.0, 1e-6, True)
    b = oracle.finalize(rows, idx, w, zero, 1.0, 1e-6, False)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # (ii) eps = 0, gain 2 vs 1: before the norm the gain cancels, after it
    # the output doubles exactly
    g1 = oracle.finalize(rows, idx, w, zero, 1.0, 0.0, True)
    g2 = oracle.finalize(rows, idx, w, one, 1.0, 0.0, True)
    assert np.array_equal(g1[0], g2[0]) and np.array_equal(g1[1], g2[1])
    h1 = oracle.finalize(rows, idx, w, zero, 1.0, 0.0, False)
    h2 = oracle.finalize(rows, idx, w, one, 1.0, 0.0, False)
    assert np.array_equal(2 * ref.f64(h1[0]), ref.f64(h2[0]))
    assert np.array_equal(2 * ref.f64(h1[1]), ref.f64(h2[1]))
    # and the two placements really differ for a non-constant gain
    gam = bits(rng.standard_normal(520) * 0.3)
    c = oracle.finalize(rows, idx, w, gam, 1.0, 1e-6, True)
    d = oracle.finalize(rows, idx, w, gam, 1.0, 1e-6, False)
    assert np.mean(c[1] != d[1]) > 0.5


def test_tp1_combine_is_identity():
    rng = np.random.default_rng(5)
    rows, idx, w, gamma = _random_ep(rng, 3, 3, 64, 1)
    partials, out = oracle.finalize(rows, idx, w, gamma, 1.0, 1e-6, True)
    assert np.array_equal(partials[0], out)


def test_rank_order_golden():
    case = golden("rank_order.json")["case"]
    tp, P = case["tp"], case["P"]
    rows = bits(np.ones((tp, 1, P)))
    idx = np.full((tp, 1, tp), -1, np.int32)
    for d in range(tp):
        idx[d, 0, d] = 0
    w = np.array([case["w"]], np.float32)
    gamma = np.zeros(P, np.uint16)
    partials, out = oracle.finalize(rows, idx, w, gamma, case["gain_center"],
                                    case["eps"], case["weight_before_norm"])
    assert [hexes(partials[d])[0] for d in range(tp)] == case["expected_partials_hex"]
    assert set(hexes(partials)) == set(case["expected_partials_hex"])
    assert hexes(out) == [case["expected_out_hex"]] * P


def test_rank_combine_order_direct():
    p = bits([[2.0 ** 25], [-2.0 ** 25], [1.0]]).reshape(3, 1, 1)
    assert hexes(oracle.rank_combine(np.repeat(p, 8, axis=2))) == ["3f80"] * 8
    assert hexes(oracle.rank_combine(np.repeat(p[::-1].copy(), 8, axis=2))) == ["0000"] * 8


def test_absent_routes_equal_zero_rows():
    rng = np.random.default_rng(9)
    rows, idx, w, gamma = _random_ep(rng, 3, 4, 64, 2)
    R = rows.shape[1]
    zrows = np.concatenate([rows, np.zeros((2, 1, 64), np.uint16)], axis=1)
    zidx = np.where(idx < 0, R, idx).astype(np.int32)
    # route k of token t is now "present" in every rank: zero rows where absent
    a = oracle.finalize(rows, idx, w, gamma, 1.0, 1e-6, True)
    b = oracle.finalize(zrows, zidx, w, gamma, 1.0, 1e-6, True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # indices past the end are absent too
    big = np.where(idx < 0, 10 ** 6, idx).astype(np.int32)
    c = oracle.finalize(rows, big, w, gamma, 1.0, 1e-6, True)
    assert np.array_equal(a[1], c[1])


def test_negzero_golden():
    case = golden("negzero.json")["case"]
    P = case["P"]
    rows = bits(np.array(case["row"])).reshape(1, 1, P)
    w = np.array([[case["w_sign"] * 2.0 ** case["w_log2"]]], np.float32)
    assert w[0, 0] < 0
    gamma = np.zeros(P, np.uint16)
    partials, out = oracle.finalize(rows, np.zeros((1, 1, 1), np.int32), w, gamma,
                                    case["gain_center"], case["eps"],
                                    case["weight_before_norm"])
    assert hexes(out) == case["expected_out_hex"]
    assert hexes(partials) == case["expected_out_hex"]
    # -0 input rows also leave as +0
    negz = np.full((1, 1, P), 0x8000, np.uint16)
    partials, out = oracle.finalize(negz, np.zeros((1, 1, 1), np.int32),
                                    np.ones((1, 1), np.float32), gamma, 1.0, 1e-6, True)
    assert not out.any()


def test_threads_do_not_change_results():
    inp = workloads.ep_finalize(1, b=8, K=16, P=3584, tp=8)
    a = oracle.finalize(inp["rows"], inp["idx"], inp["w32"], inp["gamma"], 1.0, 1e-6, True, nthreads=1)
    b = oracle.finalize(inp["rows"], inp["idx"], inp["w32"], inp["gamma"], 1.0, 1e-6, True, nthreads=4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ------------------------------------------------------- expert-TP path ---

@pytest.mark.parametrize("P,K,tp", [(8, 1, 1), (64, 3, 2), (520, 4, 4), (1032, 2, 8)])
@pytest.mark.parametrize("wbn", [True, False])
def test_tp_finalize_brute_force_fp64(P, K, tp, wbn):
    rng = np.random.default_rng(P + 7 * K + 3 * tp)
    b = 3
    n = b * K + 1
    kpart = bits(rng.standard_normal((tp, n, P)) * 0.5)
    idx = rng.permutation(n)[: b * K].reshape(b, K).astype(np.int32)
    idx[0, 0] = -1  # one absent route
    logits = rng.standard_normal((b, K))
    w = (np.exp(logits) / np.exp(logits).sum(1, keepdims=True)).astype(np.float32)
    gamma = bits(1 + 0.05 * rng.standard_normal(P))
    out = oracle.tp_finalize(kpart, idx, w, gamma, 0.5, 1e-6, wbn)
    acc, scale = ref.tp_finalize(kpart, idx, w, gamma, 0.5, 1e-6, wbn)
    assert ref.within(out, acc, 64 * U24 * scale).all()


def test_tp_round_before_norm_golden():
    case = golden("tp_round_before_norm.json")["case"]
    P = case["P"]
    kpart = np.zeros((2, 1, P), np.uint16)
    kpart[0, 0] = bits(np.ones(P))
    kpart[1, 0, 0] = bits([2.0 ** -8])[0]
    out = oracle.tp_finalize(kpart, np.array(case["idx"], np.int32),
                             np.array([case["w"]], np.float32), np.zeros(P, np.uint16),
                             case["gain_center"], case["eps"], True)
    assert hexes(out) == case["expected_out_hex"]


def test_tp1_tp_finalize_equals_ep_finalize():
    rng = np.random.default_rng(13)
    b, K, P = 3, 4, 520
    rows = bits(rng.standard_normal((1, b * K, P)))
    idx = rng.permutation(b * K).reshape(b, K).astype(np.int32)
    w = rng.random((b, K)).astype(np.float32)
    gamma = bits(rng.standard_normal(P) * 0.1)
    for wbn in (True, False):
        tp_out = oracle.tp_finalize(rows, idx, w, gamma, 1.0, 1e-6, wbn)
        _, ep_out = oracle.finalize(rows, idx[None], w, gamma, 1.0, 1e-6, wbn)
        assert np.array_equal(tp_out, ep_out)


# ---------------------------------------- combine + norm + up projection --

def _combined_latent64(lat):
    return ref.round_bf16(ref.f64(lat).sum(axis=0))


def test_normed_latent_is_rmsnorm_of_combined():
    inp = workloads.upproj(0, b=4, tp=8, L=3584, N=16)
    normed, _ = oracle.combine_norm_upproj(inp["lat"], inp["gamma"], inp["eps"], inp["w_up"])
    l = _combined_latent64(inp["lat"])
    want = torch.nn.functional.rms_norm(torch.from_numpy(l), [3584],
                                        weight=torch.from_numpy(ref.f64(inp["gamma"])),
                                        eps=inp["eps"]).numpy()
    assert np.all(np.abs(ref.f64(normed) - want) <= ref.ulp_bf16(want))


def test_latent_rank_order():
    tp, L = 3, 8
    lat = np.zeros((tp, 1, L), np.uint16)
    lat[:, 0, 0] = bits([2.0 ** 25, -2.0 ** 25, 1.0])
    lat[0, 0, 1:] = bits(np.ones(L - 1))
    gamma = bits(np.ones(L))
    w = np.eye(L, dtype=np.float32)
    normed, out = oracle.combine_norm_upproj(lat, gamma, 0.0, bits(w))
    # combined row is all ones in rank order (reverse order would zero column 0)
    assert hexes(normed) == ["3f80"] * L
    assert hexes(out) == ["3f80"] * L


def test_upproj_unit_rows_gather_normed():
    inp = workloads.upproj(2, b=3, tp=2, L=520, N=40)
    perm = np.random.default_rng(0).integers(0, 520, 40)
    w = np.zeros((40, 520), np.float32)
    w[np.arange(40), perm] = 1.0
    normed, out = oracle.combine_norm_upproj(inp["lat"], inp["gamma"], inp["eps"], bits(w))
    assert np.array_equal(out, normed[:, perm])
    # zero weights give back the reduce-scatter partial, -0 as +0
    rs = bits(np.random.default_rng(1).standard_normal((3, 40)))
    rs[0, 0] = 0x8000
    _, out0 = oracle.combine_norm_upproj(inp["lat"], inp["gamma"], inp["eps"],
                                         np.zeros((40, 520), np.uint16), rs)
    want = rs.copy()
    want[0, 0] = 0
    assert np.array_equal(out0, want)


def test_upproj_random_vs_fp64_matmul():
    inp = workloads.upproj(3, b=5, tp=4, L=3584, N=64, with_rs=True)
    normed, out = oracle.combine_norm_upproj(inp["lat"], inp["gamma"], inp["eps"],
                                             inp["w_up"], inp["rs"])
    W, y = ref.f64(inp["w_up"]), ref.f64(normed)
    exact = y @ W.T + ref.f64(inp["rs"])
    E = 2 * 3584 * U24 * (np.abs(y) @ np.abs(W).T + np.abs(ref.f64(inp["rs"])))
    assert ref.within(out, exact, E).all()
    # a transposed or shifted operand is far outside
    assert not ref.within(out, y @ np.roll(W, 1, axis=1).T, E).all()


def test_upproj_rs_after_the_k_sum_golden():
    case = golden("upproj_rs_order.json")["case"]
    tp, b, L, N = case["tp"], case["b"], case["L"], case["N"]
    lat = bits(np.ones((tp, b, L)))
    gamma = bits(np.ones(L))
    w = np.zeros((N, L), np.float32)
    w[:, 0], w[:, 1] = 2.0 ** 24, -2.0 ** 24
    rs = bits(np.ones((b, N)))
    normed, out = oracle.combine_norm_upproj(lat, gamma, case["eps"], bits(w), rs)
    assert hexes(normed) == [case["expected_normed_hex"][2:]] * L
    assert hexes(out) == [case["expected_out_hex"][2:]] * N


def test_upproj_y_is_rounded_before_the_projection():
    """Rows with two unit weights: out = bf16(y[a] + y[b]) where y is the
    BF16 normed row (the sum of two BF16 values is exact in FP64); with y
    left in FP32 most outputs would differ."""
    inp = workloads.upproj(4, b=3, tp=4, L=544, N=96)
    rng = np.random.default_rng(2)
    a, c = rng.integers(0, 544, 96), rng.integers(0, 544, 96)
    c = np.where(c == a, (c + 1) % 544, c)
    w = np.zeros((96, 544), np.float32)
    w[np.arange(96), a] = 1.0
    w[np.arange(96), c] = 1.0
    normed, out = oracle.combine_norm_upproj(inp["lat"], inp["gamma"], inp["eps"], bits(w))
    y = ref.f64(normed)
    want = oracle.bf16_round(ref.round_bf16(y[:, a] + y[:, c]).astype(np.float32))
    assert np.array_equal(out, np.where(want == 0x8000, 0, want))


# -------------------------------------------- the sum-of-squares order -----
#
# The plain sequential sum of squares (SEQ) against the wave64 tree (W64).
# A different order moves an inverse RMS by an FP32 step now and then; where
# a token's route products nearly cancel, that step is many BF16 steps of the
# small result.  So between two orders the bar is: nearly every word
# identical, and every word within the FP32 noise of its terms (32 u times
# the sum of the products' magnitudes) plus one BF16 step -- not within one
# BF16 step of the result itself.  Measured at decode scale: partials
# 99.95-99.98% identical, the combined row 99.89% (gain after the norm) and
# 99.98% (gain first).


def _identical(a, b):
    return float(np.mean(np.asarray(a) == np.asarray(b)))


@pytest.mark.parametrize("wbn", [True, False])
def test_ss_order_seq_against_w64_decode_scale(wbn):
    inp = workloads.ep_finalize(0)
    args = (inp["rows"], inp["idx"], inp["w32"], inp["gamma"], inp["gain_center"], inp["eps"], wbn)
    p64, o64 = oracle.finalize(*args)
    with oracle.ss_order(oracle.SS_SEQ):
        pseq, oseq = oracle.finalize(*args)
    _, scale = ref.ep_finalize(*args)
    E = 32 * U24 * scale
    assert ref.within(pseq, ref.f64(p64), E).all()
    assert _identical(pseq, p64) >= 0.999
    # the combine adds tp partials, each of which may sit one step apart
    E_out = (E + ref.ulp_bf16(ref.f64(p64))).sum(axis=0)
    assert ref.within(oseq, ref.f64(o64), E_out).all()
    assert _identical(oseq, o64) >= 0.998
    assert not np.array_equal(p64, pseq)  # the orders do differ somewhere


def test_ss_order_seq_against_w64_expert_tp():
    """Expert TP (K=16, P=7168, tp=8; 32 of the 128 tokens)."""
    inp = workloads.tp_finalize(0, b=32)
    args = (inp["kpart"], inp["idx"], inp["w32"], inp["gamma"], 0.0, inp["eps"], False)
    o64 = oracle.tp_finalize(*args)
    with oracle.ss_order(oracle.SS_SEQ):
        oseq = oracle.tp_finalize(*args)
    _, scale = ref.tp_finalize(*args)
    assert ref.within(oseq, ref.f64(o64), 32 * U24 * scale).all()
    assert _identical(oseq, o64) >= 0.999
    assert not np.array_equal(o64, oseq)


# ----------------------------------------------------------- shared expert --

def test_shared_zero_input():
    inp = workloads.shared(0, b=2, H=64, I=32)
    h, rs = oracle.shared_expert(np.zeros_like(inp["x"]), inp["w_gate"], inp["w_up"], inp["w_down"])
    assert not h.any() and not rs.any()


def _silu64(z):
    return z / (1.0 + np.exp(-z))


def test_shared_unit_rows_closed_form():
    rng = np.random.default_rng(4)
    b, H, I = 3, 64, 48
    x = bits(rng.standard_normal((b, H)) * 3)
    a, c = rng.integers(0, H, I), rng.integers(0, H, I)
    wg = np.zeros((I, H), np.float32)
    wu = np.zeros((I, H), np.float32)
    wg[np.arange(I), a] = 1.0
    wu[np.arange(I), c] = 1.0
    sel = rng.integers(0, I, H)
    wd = np.zeros((H, I), np.float32)
    wd[np.arange(H), sel] = 1.0
    h, rs = oracle.shared_expert(x, bits(wg), bits(wu), bits(wd))
    xv = ref.f64(x)
    want = _silu64(xv[:, a]) * xv[:, c]
    assert np.all(np.abs(ref.f64(h) - want) <= ref.ulp_bf16(want))
    assert np.array_equal(rs, h[:, sel])


def test_shared_random_vs_fp64():
    inp = workloads.shared(1, b=3, H=512, I=256)
    h, rs = oracle.shared_expert(inp["x"], inp["w_gate"], inp["w_up"], inp["w_down"])
    x = ref.f64(inp["x"])
    G, U = x @ ref.f64(inp["w_gate"]).T, x @ ref.f64(inp["w_up"]).T
    want_h = ref.round_bf16(_silu64(ref.round_bf16(G)) * ref.round_bf16(U))
    # gate/up roundings can flip near ties: nearly all h words agree exactly,
    # every one within a few BF16 spacings
    got_h = ref.f64(h)
    assert np.mean(got_h == want_h) > 0.98
    assert np.all(np.abs(got_h - want_h) <= 4 * ref.ulp_bf16(want_h) + 1e-30)
    Wd = ref.f64(inp["w_down"])
    exact = got_h @ Wd.T
    E = 2 * 256 * U24 * (np.abs(got_h) @ np.abs(Wd).T)
    assert ref.within(rs, exact, E).all()


# ------------------------------------------------------ input generators ---

def test_ep_workload_structure():
    inp = workloads.ep_finalize(0, b=8, K=16, P=64, tp=8)
    idx = inp["idx"]
    present = idx >= 0
    assert np.all(present.sum(axis=0) == 1)  # each route local to one rank
    assert np.all(present.sum(axis=2) == 2)  # two local routes per rank
    for d in range(8):
        assert sorted(idx[d][present[d]].tolist()) == list(range(inp["R"]))
    assert np.allclose(inp["w32"].sum(axis=1), 1.0, atol=1e-6)
    assert np.all(np.diff(inp["w32"], axis=1) <= 0)  # top-k order
    again = workloads.ep_finalize(0, b=8, K=16, P=64, tp=8)
    assert np.array_equal(again["rows"], inp["rows"]) and np.array_equal(again["idx"], idx)


def test_ep_workload_outliers():
    inp = workloads.ep_finalize(0, b=64, K=16, P=64, tp=8)
    mags = np.abs(ref.f64(inp["rows"])).reshape(-1, 64).max(axis=1)
    assert int(np.sum(mags > 30)) == 10


def test_tp_workload_structure():
    inp = workloads.tp_finalize(0, b=4, K=16, P=64, tp=8)
    assert sorted(inp["idx"].ravel().tolist()) == list(range(64))


def test_route_order_golden():
    case = golden("route_order.json")["case"]
    K, P = case["K"], case["P"]
    w = np.array([case["w"]], np.float32)
    gamma = np.zeros(P, np.uint16)
    ones = bits(np.ones((K, P)))
    for wbn in (True, False):
        # EP: all three routes local to the one rank
        _, out = oracle.finalize(ones[None], np.arange(K, dtype=np.int32).reshape(1, 1, K),
                                 w, gamma, case["gain_center"], case["eps"], wbn)
        assert hexes(out) == [case["expected_out_hex"]] * P
        # expert TP: one rank holds the whole rows
        out = oracle.tp_finalize(ones[None], np.arange(K, dtype=np.int32).reshape(1, K),
                                 w, gamma, case["gain_center"], case["eps"], wbn)
        assert hexes(out) == [case["expected_out_hex"]] * P


# ------------------------------- finalize without a per-route norm (Kimi) --

def test_plain_single_route_is_the_row():
    # one route, w = 1, tp = 1: every product is exact, the sum is the row
    rng = np.random.default_rng(21)
    x = bits(rng.standard_normal((1, 1, 3584)) * 5)
    x[0, 0, :3] = [0x8000, 0x0001, 0x8001]  # -0, the smallest denormals
    p, out = oracle.finalize_plain(x, np.zeros((1, 1, 1), np.int32), np.ones((1, 1), np.float32))
    want = x[0].copy()
    want[want == 0x8000] = 0
    assert np.array_equal(out, want) and np.array_equal(p[0], want)


def test_plain_power_of_two_weights_exact():
    # weights 1/2, 1/4, 1/8: products exact; with rows of BF16 values within a
    # few binades the FP32 sum is exact too, so out = bf16 of the FP64 sum
    rng = np.random.default_rng(22)
    K, P = 3, 512
    rows = bits(rng.uniform(1.0, 2.0, (1, K, P)))
    w = np.array([[0.5, 0.25, 0.125]], np.float32)
    _, out = oracle.finalize_plain(rows, np.arange(K, dtype=np.int32).reshape(1, 1, K), w)
    exact = (ref.f64(rows[0]) * w[0][:, None].astype(np.float64)).sum(axis=0)
    assert np.array_equal(out[0], oracle.bf16_round(ref.round_bf16(exact).astype(np.float32)))


def test_plain_route_order_and_rank_order():
    # routes (2^25, -2^25, 1) in order sum to 1.0; a rank per route: the same
    P = 8
    rows = bits(np.ones((1, 3, P)))
    w = np.array([[2.0 ** 25, -2.0 ** 25, 1.0]], np.float32)
    _, out = oracle.finalize_plain(rows, np.arange(3, dtype=np.int32).reshape(1, 1, 3), w)
    assert hexes(out) == ["3f80"] * P
    rows3 = np.repeat(bits(np.ones((1, 1, P))), 3, axis=0)
    idx = np.full((3, 1, 3), -1, np.int32)
    for d in range(3):
        idx[d, 0, d] = 0
    partials, out = oracle.finalize_plain(rows3, idx, w)
    assert [hexes(partials[d])[0] for d in range(3)] == ["4c00", "cc00", "3f80"]
    assert hexes(out) == ["3f80"] * P


def test_plain_zero_weights_and_absent_routes():
    rng = np.random.default_rng(23)
    rows, idx, w, _ = _random_ep(rng, 3, 4, 64, 2)
    p, out = oracle.finalize_plain(rows, idx, np.zeros_like(w))
    assert not p.any() and not out.any()  # +0 everywhere, never 0x8000
    R = rows.shape[1]
    big = np.where(idx < 0, R + 5, idx).astype(np.int32)
    a = oracle.finalize_plain(rows, idx, w)
    c = oracle.finalize_plain(rows, big, w)
    assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])


@pytest.mark.parametrize("P,K,tp", [(8, 1, 1), (64, 3, 3), (520, 4, 2), (3584, 16, 8)])
def test_plain_brute_force_fp64(P, K, tp):
    """FP64 straight-line sum of w_k x_k per rank: the FP32 result lies within
    the FP32 summation bound, and out within the combine's bound."""
    rng = np.random.default_rng(P + K + tp)
    rows, idx, w, _ = _random_ep(rng, 3, K, P, tp)
    partials, out = oracle.finalize_plain(rows, idx, w)
    b = idx.shape[1]
    R = rows.shape[1]
    acc = np.zeros((tp, b, P))
    mag = np.zeros((tp, b, P))
    for d in range(tp):
        for t in range(b):
            for k in range(K):
                r = idx[d, t, k]
                if 0 <= r < R:
                    term = ref.f64(rows[d, r]) * float(w[t, k])
                    acc[d, t] += term
                    mag[d, t] += np.abs(term)
    E = (K + 1) * U24 * mag
    assert ref.within(partials, acc, E).all()
    E_out = (E + ref.ulp_bf16(np.abs(acc) + E)).sum(axis=0) + 2 * tp * U24 * np.abs(acc).sum(axis=0)
    assert ref.within(out, acc.sum(axis=0), E_out).all()
