"""Seeded synthetic inputs of the MoE decode tail (shared by tests and bench).

This module only draws inputs: it holds none of the tail's arithmetic.  All
draws use ``torch.Generator('cpu').manual_seed(seed)``, FP32 ``randn`` in the
fixed order written in each function, scaled by the stated standard
deviation (``N(mu, sigma)``: sigma is the standard deviation), then rounded
to BF16 by torch (round-to-nearest-even).  BF16 arrays are returned as
``numpy.uint16`` bit patterns; indices as int32; FP32 route weights as
float32.

Workloads (shapes and distributions of the MoE tail pages' problem):

* ``ep_finalize``  EP finalize + rank combine: b tokens, K routes/token split
  evenly over tp simulated ranks, rows of width P.
* ``tp_finalize``  expert-TP finalize: tp K-partials of every route row.
* ``upproj``       latent combine + RMSNorm + 3584->7168 up projection.
* ``shared``       shared expert 7168 -> 6144 (gate/up, SiLU) -> 7168.
"""
from __future__ import annotations

import numpy as np
import torch


def _gen(seed: int) -> torch.Generator:
    return torch.Generator("cpu").manual_seed(int(seed))


def _bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.bfloat16).contiguous().view(torch.int16).numpy().view(np.uint16)


def normal_bf16(g, shape, mean=0.0, std=1.0) -> np.ndarray:
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    if mean != 0.0:
        x = x + mean
    return _bf16_bits(x)


def route_weights(g, b, K, top_sorted=True):
    """FP32 softmax over K N(0,1) logits per token (and its BF16 copy).

    With ``top_sorted`` the logits are sorted descending first, so route order
    is top-k order; a softmax over the top K of any larger expert set equals
    this renormalized top-K softmax."""
    logits = torch.randn((b, K), generator=g, dtype=torch.float32)
    if top_sorted:
        logits = torch.sort(logits, dim=1, descending=True).values
    w = torch.softmax(logits, dim=1).to(torch.float32).contiguous()
    return w.numpy().copy(), _bf16_bits(w)


def ep_finalize(seed=0, b=64, K=16, P=3584, tp=8, row_std=2.0,
                outlier_frac=0.01, outlier_scale=50.0, gamma_std=0.1,
                gain_center=1.0, eps=1e-6, top_sorted=True):
    """EP finalize inputs.

    Route -> rank: per token a seeded permutation pi of the K routes; route k
    is local to rank pi(k) // (K // tp).  Rank d's R = b*K/tp rows hold its
    local (token, route) pairs in a seeded shuffled order (an expert-sorted
    GEMM2 output); idx[d][t][k] is the row, or -1 where route k of token t is
    not local to rank d.  ``round(outlier_frac * b * K)`` rows, chosen by a
    seeded permutation over all tp*R rows, are scaled by ``outlier_scale`` in
    FP32 before the BF16 rounding.

    Draw order: rows, outlier choice, logits, gamma, route permutations,
    row shuffles."""
    if K % tp:
        raise ValueError("K must split evenly over the ranks")
    g = _gen(seed)
    per = K // tp
    R = b * per
    rows = torch.randn((tp, R, P), generator=g, dtype=torch.float32) * row_std
    n_out = int(round(outlier_frac * b * K))
    if n_out:
        pick = torch.randperm(tp * R, generator=g)[:n_out]
        flat = rows.view(tp * R, P)
        flat[pick] = flat[pick] * outlier_scale
    w32, w16 = route_weights(g, b, K, top_sorted)
    gamma = normal_bf16(g, (P,), 0.0, gamma_std)
    idx = np.full((tp, b, K), -1, np.int32)
    owner = np.empty((b, K), np.int64)
    for t in range(b):
        pi = torch.randperm(K, generator=g).numpy()
        owner[t] = pi // per
    for d in range(tp):
        pairs = [(t, k) for t in range(b) for k in range(K) if owner[t, k] == d]
        assert len(pairs) == R
        shuffle = torch.randperm(R, generator=g).numpy()
        for pos, (t, k) in enumerate(pairs):
            idx[d, t, k] = shuffle[pos]
    return dict(rows=_bf16_bits(rows), idx=idx, w32=w32, w16=w16, gamma=gamma,
                gain_center=float(gain_center), eps=float(eps), b=b, K=K, P=P,
                tp=tp, R=R)


def tiny_ep_finalize(seed=0):
    """b=4 tokens, 4 routes/token, P=512, tp=2 (2 routes per rank), rows
    N(0,1), FP32 softmax of N(0,1) logits (unsorted), gamma N(0,0.1),
    gain_center 1.0, eps 1e-6; weight_before_norm is the caller's."""
    return ep_finalize(seed=seed, b=4, K=4, P=512, tp=2, row_std=1.0,
                       outlier_frac=0.0, gamma_std=0.1, gain_center=1.0,
                       eps=1e-6, top_sorted=False)


def tp_finalize(seed=0, b=128, K=16, P=7168, tp=8, part_std=0.5,
                gamma_mean=1.0, gamma_std=0.05, eps=1e-6, num_rows=None):
    """Expert-TP finalize inputs: kpart [tp][num_rows][P] ~ N(0, part_std),
    num_rows = b*K (every route present), idx[t][k] = pi(t*K + k) for a
    seeded permutation pi of the rows, top-K FP32 softmax weights, gamma
    N(gamma_mean, gamma_std); gain_center 0, standard RMSNorm.

    Draw order: kpart, pi, logits, gamma."""
    g = _gen(seed)
    n = b * K if num_rows is None else num_rows
    kpart = normal_bf16(g, (tp, n, P), 0.0, part_std)
    pi = torch.randperm(n, generator=g).numpy().astype(np.int32)
    idx = pi[: b * K].reshape(b, K).copy()
    w32, w16 = route_weights(g, b, K, True)
    gamma = normal_bf16(g, (P,), gamma_mean, gamma_std)
    return dict(kpart=kpart, idx=idx, w32=w32, w16=w16, gamma=gamma,
                gain_center=0.0, eps=float(eps), b=b, K=K, P=P, tp=tp,
                num_rows=n)


def upproj(seed=0, b=64, tp=8, L=3584, N=7168, lat_std=1.0, gamma_mean=1.0,
           gamma_std=0.05, w_std=0.02, eps=1e-6, with_rs=False, rs_std=1.0):
    """Latent combine + norm + up projection inputs.

    Draw order: latent partials [tp][b][L], gamma [L], W_up [N][L], then
    (with_rs) a stand-in reduce-scatter partial rs [b][N]."""
    g = _gen(seed)
    lat = normal_bf16(g, (tp, b, L), 0.0, lat_std)
    gamma = normal_bf16(g, (L,), gamma_mean, gamma_std)
    w_up = normal_bf16(g, (N, L), 0.0, w_std)
    rs = normal_bf16(g, (b, N), 0.0, rs_std) if with_rs else None
    return dict(lat=lat, gamma=gamma, w_up=w_up, rs=rs, eps=float(eps), b=b,
                tp=tp, L=L, N=N)


def shared(seed=0, b=64, H=7168, I=6144, x_std=1.0, w_std=0.02):
    """Shared expert inputs.  Draw order: x [b][H], W_gate [I][H],
    W_up [I][H], W_down [H][I]."""
    g = _gen(seed)
    x = normal_bf16(g, (b, H), 0.0, x_std)
    w_gate = normal_bf16(g, (I, H), 0.0, w_std)
    w_up = normal_bf16(g, (I, H), 0.0, w_std)
    w_down = normal_bf16(g, (H, I), 0.0, w_std)
    return dict(x=x, w_gate=w_gate, w_up=w_up, w_down=w_down, b=b, H=H, I=I)
