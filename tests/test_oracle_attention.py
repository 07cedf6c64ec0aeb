"""Pins of the oracle's attention: dense brute-force causal attention, the
sink's closed forms, CSA == HCA when every entry is selected, and the textbook
sliding-window special case."""
import math

import numpy as np

from oracle.attention import attend_one, csa_sparse_attn, hca_dense_attn
from oracle.compress import compress
from oracle.indexer import index_scores_batch
from oracle.rope import apply_rope
from oracle.topk import topk_batch


def _dense_causal(q, k, v, window=None, sink=None):
    """Dense masked softmax attention over raw tokens 0..L-1 with RoPE at the
    token positions; written with a full L x L score matrix and a mask."""
    L, H, D = q.shape
    pos = np.arange(L)
    Qr = apply_rope(q, pos[:, None])                          # [L, H, D]
    Kr = apply_rope(k, pos)                                   # [L, D]
    S = np.einsum("thd,sd->hts", Qr, Kr) / math.sqrt(D)       # [H, L, L]
    mask = pos[None, :] > pos[:, None]
    if window is not None:
        mask |= pos[None, :] < pos[:, None] - window + 1
    S = np.where(mask[None], -np.inf, S)
    if sink is not None:
        S = np.concatenate([S, np.broadcast_to(sink[:, None, None], (H, L, 1))], axis=2)
        V = np.concatenate([v, np.zeros((1, D))], axis=0)
    else:
        V = v
    P = np.exp(S - S.max(axis=2, keepdims=True))
    P = P / P.sum(axis=2, keepdims=True)
    return np.einsum("hts,sd->thd", P, V)


def test_m1_full_selection_equals_dense_causal():
    rng = np.random.default_rng(0)
    L, H, D = 40, 3, 128
    q = rng.standard_normal((1, L, H, D))
    k = rng.standard_normal((L, D))
    v = rng.standard_normal((L, D))
    kc, vc = compress(k, v, rng.standard_normal(D), m=1)
    # indexer + top-k with k >= L selects every visible entry
    qi = rng.standard_normal((1, L, 2, 16))
    wi = rng.standard_normal((1, L, 2))
    ki = rng.standard_normal((1, L, 16))
    idx = topk_batch(index_scores_batch(qi, wi, ki, 0, 1), L, 0, 1)
    out, _ = csa_sparse_attn(q, 0, kc[None], vc[None], idx, np.zeros((1, 0, D)),
                             np.zeros((1, 0, D)), 0, 0, None)
    ref = _dense_causal(q[0], k, v)
    np.testing.assert_allclose(out[0], ref, atol=1e-12)


def test_window_only_equals_sliding_window_with_sink():
    rng = np.random.default_rng(1)
    L, H, D, W = 50, 2, 128, 7
    q = rng.standard_normal((1, L, H, D))
    k = rng.standard_normal((1, L, D))
    v = rng.standard_normal((1, L, D))
    sink = rng.standard_normal(H)
    idx = np.full((1, L, 4), -1)
    out, _ = csa_sparse_attn(q, 0, np.zeros((1, 4, D)), np.zeros((1, 4, D)), idx, k, v, 0, W, sink)
    ref = _dense_causal(q[0], k[0], v[0], window=W, sink=sink)
    np.testing.assert_allclose(out[0], ref, atol=1e-12)


def test_sink_closed_forms():
    rng = np.random.default_rng(2)
    H, D, n = 4, 128, 9
    q = rng.standard_normal((H, D))
    keys = rng.standard_normal((n, D))
    vals = rng.standard_normal((n, D))
    z = rng.standard_normal(H)
    o, lse = attend_one(q, 50, keys, vals, np.zeros((0, D)), [], np.zeros((0, D)), z)
    o0, lse0 = attend_one(q, 50, keys, vals, np.zeros((0, D)), [], np.zeros((0, D)), None)
    S = np.exp(lse0)                                  # sum of exp(logits)
    # row weights add up to S / (S + e^z) = 1 - e^(z - lse) < 1
    np.testing.assert_allclose(1 - np.exp(z - lse), S / (S + np.exp(z)), rtol=1e-13)
    assert np.all(1 - np.exp(z - lse) < 1)
    np.testing.assert_allclose(o, o0 * (S / (S + np.exp(z)))[:, None], atol=1e-13)
    o_lo, _ = attend_one(q, 50, keys, vals, np.zeros((0, D)), [], np.zeros((0, D)), np.full(H, -np.inf))
    np.testing.assert_allclose(o_lo, o0, atol=1e-14)
    o_hi, _ = attend_one(q, 50, keys, vals, np.zeros((0, D)), [], np.zeros((0, D)), np.full(H, 800.0))
    assert np.abs(o_hi).max() < 1e-100


def test_single_source_and_empty():
    D = 128
    q = np.zeros((1, D))
    q[0, 0] = 2.0
    key = np.zeros((1, D))
    key[0, 0] = math.sqrt(D) * math.log(3.0) / 2.0     # logit = ln 3
    val = np.ones((1, D))
    o, lse = attend_one(q, 0, key, val, np.zeros((0, D)), [], np.zeros((0, D)), np.array([0.0]))
    np.testing.assert_allclose(o, np.full((1, D), 0.75), atol=1e-14)   # 3 / (3 + 1)
    assert abs(lse[0] - math.log(4.0)) < 1e-14
    o, lse = attend_one(q, 0, np.zeros((0, D)), np.zeros((0, D)), np.zeros((0, D)), [], np.zeros((0, D)), None)
    assert np.all(o == 0) and np.isneginf(lse).all()


def test_csa_full_selection_equals_hca():
    rng = np.random.default_rng(3)
    B, Lq, H, D, m, N, W = 2, 5, 4, 128, 4, 30, 6
    q0 = 100
    q = rng.standard_normal((B, Lq, H, D))
    kc = rng.standard_normal((B, N, D))
    vc = rng.standard_normal((B, N, D))
    kr = rng.standard_normal((B, 120, D))
    vr = rng.standard_normal((B, 120, D))
    sink = rng.standard_normal(H)
    idx = np.full((B, Lq, 40), -1)
    for i in range(Lq):
        n = (q0 + i + 1) // m
        idx[:, i, :n] = np.arange(n)
    a, la = csa_sparse_attn(q, q0, kc, vc, idx, kr, vr, 0, W, sink)
    b, lb = hca_dense_attn(q, q0, m, kc, vc, kr, vr, 0, W, sink)
    np.testing.assert_allclose(a, b, atol=1e-13)
    np.testing.assert_allclose(la, lb, atol=1e-13)
