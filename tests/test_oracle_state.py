"""Pins of the oracle's encoders (e4m3fn, e2m1 / MXFP4), of the decode state
cache (ring + incremental compression) and of per-sequence positions and ring
reads in the attention, indexer and top-k oracles.

The encoders are checked against torch's CPU float8 cast (an independent
implementation), a brute-force nearest-value search and the OCP e2m1 table;
the state cache against the batch compressor (pinned in
test_oracle_compress_indexer_topk.py) over a token stream; the per-sequence
and ring forms against the uniform, linear forms on the same rows.
"""
import os

import numpy as np
import torch

from oracle import attention, compress, formats, indexer, rope, state, topk

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- e4m3fn
def _finite_e4m3():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    return codes, formats.e4m3fn_to_f64(codes)


def test_e4m3_roundtrip_every_code():
    codes, vals = _finite_e4m3()
    assert np.array_equal(formats.f64_to_e4m3fn(vals), codes)


def test_e4m3_matches_torch_cast():
    rng = np.random.default_rng(5)
    mag = np.exp2(rng.uniform(-12, np.log2(463.9), 20000))
    x = mag * rng.choice([-1.0, 1.0], mag.shape)
    # every midpoint between neighbouring finite codes of one sign (ties)
    _, vals = _finite_e4m3()
    pos = np.unique(vals[vals >= 0])
    mids = (pos[:-1] + pos[1:]) / 2
    x = np.concatenate([x, mids, -mids, [0.0, 448.0, 463.0]])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = formats.f64_to_e4m3fn(x)
    # torch keeps -0.0 for negative values that round to zero, as the encoder does
    assert np.array_equal(got, ref)


def test_e4m3_saturates():
    x = np.array([464.0, 1e6, -500.0, np.inf])
    assert list(formats.f64_to_e4m3fn(x)) == [0x7E, 0x7E, 0xFE, 0x7E]


def test_e4m3_brute_force_nearest():
    _, vals = _finite_e4m3()
    codes = formats.f64_to_e4m3fn(vals)
    rng = np.random.default_rng(6)
    x = rng.uniform(-448, 448, 3000) * np.exp2(rng.integers(-14, 1, 3000))
    got = formats.e4m3fn_to_f64(formats.f64_to_e4m3fn(x))
    for xi, gi in zip(x, got):
        d = np.abs(vals - xi)
        best = d.min()
        assert abs(gi - xi) == best
        if len(np.unique(np.abs(vals[d == best]))) > 1:   # a true tie: even code wins
            assert formats.f64_to_e4m3fn(np.array([xi]))[0] % 2 == 0


# ------------------------------------------------------------------ bf16
def test_bf16_rounding_matches_torch_cast():
    rng = np.random.default_rng(12)
    x = rng.standard_normal(20000) * np.exp2(rng.integers(-30, 30, 20000))
    # exact midpoints between neighbouring bf16 values (ties) and zeros
    c = rng.integers(0, 0x7F7F, 2000).astype(np.uint16)
    lo, hi = formats.bf16_to_f64(c), formats.bf16_to_f64(c + 1)
    x = np.concatenate([x, (lo + hi) / 2, -(lo + hi) / 2, [0.0, -0.0]])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(formats.f64_to_bf16(x), ref)
    assert np.array_equal(formats.round_bf16(x), torch.from_numpy(x).to(torch.bfloat16).double().numpy())


# ------------------------------------------------------------- e2m1 / MX
def test_e2m1_encodes_ocp_table():
    rows = [l.split() for l in open(os.path.join(GOLD, "e2m1_ocp_mx.txt")) if l.strip() and not l.startswith("#")]
    codes = np.array([int(r[0]) for r in rows])
    vals = np.array([float(r[1]) for r in rows])
    got = formats.f64_to_e2m1(np.where(codes == 8, -0.0, vals))
    assert np.array_equal(got, codes)


def test_e2m1_brute_force_nearest_ties_even():
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    x = np.concatenate([np.linspace(-7, 7, 2801), (mags[:-1] + mags[1:]) / 2, -(mags[:-1] + mags[1:]) / 2])
    c = formats.f64_to_e2m1(x)
    v = formats.e2m1_to_f64(c)
    a = np.minimum(np.abs(x), 6.0)
    for ai, vi, ci, xi in zip(a, np.abs(v), c, x):
        d = np.abs(mags - ai)
        assert abs(vi - ai) == d.min()
        if (d == d.min()).sum() > 1:
            assert (ci & 1) == 0          # the even code of a tie
        assert (ci >> 3) == (1 if np.signbit(xi) else 0)


def test_mxfp4_scale_rule_and_roundtrip():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((6, 64)) * np.exp2(rng.integers(-20, 20, (6, 1)))
    packed, sc = formats.f64_to_mxfp4(x)
    amax = np.abs(x.reshape(6, 2, 32)).max(-1)
    r = amax / np.exp2(sc.astype(np.int64) - 127)
    assert np.all((r >= 4) & (r < 8))               # OCP MX: amax at 4..8 scales
    # decode -> encode is the identity on what the encoder produced
    y = formats.mxfp4_to_f64(packed, sc)
    p2, s2 = formats.f64_to_mxfp4(y)
    assert np.array_equal(p2, packed) and np.array_equal(s2, sc)
    # error bound: half the e2m1 step at the element's magnitude (<= 1 scale)
    # up to 6 scales; above that (amax may reach 8 scales) the value clips to 6
    X = np.repeat(np.exp2(sc.astype(np.int64) - 127), 32, axis=-1)
    inside = np.abs(x) <= 6 * X
    assert (np.abs(y - x) / X)[inside].max() <= 1.0
    assert np.array_equal(np.abs(y[~inside]), 6 * X[~inside])
    # a zero block: scale code 0 and zero codes
    pz, sz = formats.f64_to_mxfp4(np.zeros((1, 32)))
    assert sz[0, 0] == 0 and not pz.any()


# --------------------------------------------------------- state cache
def _stream(rng, T, D, d):
    return (rng.standard_normal((T, D)), rng.standard_normal((T, D)), rng.standard_normal((T, d)))


def test_x_fold_is_unrotated_key_fold():
    rng = np.random.default_rng(8)
    k, v, _ = _stream(rng, 12, 128, 8)
    w = rng.standard_normal(128) / np.sqrt(128)
    k_c, v_c, x_c = compress.compress(k, v, w, 4, pos0=8, x_raw=k)
    j = 2 + np.arange(3)
    assert np.allclose(rope.apply_rope(x_c, j * 4 + 3), k_c, atol=1e-12)
    _, _, xv = compress.compress(k, v, w, 4, pos0=8, x_raw=v)
    assert np.allclose(xv, v_c, atol=1e-12)


def test_state_append_stream_equals_batch_compress():
    rng = np.random.default_rng(9)
    B, D, d, m, R, N_cap = 3, 128, 16, 4, 8, 6
    starts = [0, 5, 13]                       # sequences at different positions
    T = 24
    w = rng.standard_normal(D) / np.sqrt(D)
    toks = [_stream(rng, s + T, D, d) for s in starts]
    k_ring = np.zeros((B, R, D)); v_ring = np.zeros((B, R, D)); ki_ring = np.zeros((B, R, d))
    k_c = np.full((B, N_cap, D), 7.0); v_c = np.full((B, N_cap, D), 7.0); ki_c = np.full((B, N_cap, d), 7.0)
    # the ring holds the tokens before each start (as a prefill would leave it)
    for b, s in enumerate(starts):
        for p in range(max(0, s - R), s):
            k_ring[b, p % R], v_ring[b, p % R], ki_ring[b, p % R] = toks[b][0][p], toks[b][1][p], toks[b][2][p]
        nb = s // m
        if nb:
            kc, vc, xc = compress.compress(toks[b][0][:nb * m], toks[b][1][:nb * m], w, m, x_raw=toks[b][2][:nb * m])
            k_c[b, :nb], v_c[b, :nb], ki_c[b, :nb] = kc[:N_cap], vc[:N_cap], xc[:N_cap]
    for step in range(T):
        pos = np.array([s + step for s in starts])
        kn = np.stack([toks[b][0][pos[b]] for b in range(B)])
        vn = np.stack([toks[b][1][pos[b]] for b in range(B)])
        xn = np.stack([toks[b][2][pos[b]] for b in range(B)])
        written = state.state_append(pos, kn, vn, k_ring, v_ring, w, m, k_c, v_c, xn, ki_ring, ki_c)
        for b in range(B):
            t = pos[b]
            # the ring holds the last R tokens
            for p in range(max(0, t - R + 1), t + 1):
                assert np.array_equal(k_ring[b, p % R], toks[b][0][p])
                assert np.array_equal(ki_ring[b, p % R], toks[b][2][p])
            # every complete block below N_cap equals the batch compressor's entry
            nb = min((t + 1) // m, N_cap)
            kc, vc, xc = compress.compress(toks[b][0][:nb * m], toks[b][1][:nb * m], w, m, x_raw=toks[b][2][:nb * m])
            assert np.allclose(k_c[b, :nb], kc, atol=1e-12)
            assert np.allclose(v_c[b, :nb], vc, atol=1e-12)
            assert np.allclose(ki_c[b, :nb], xc, atol=1e-12)
            assert np.all(k_c[b, nb:] == 7.0)    # nothing else written
            assert ((b, (t + 1) // m - 1) in written) == ((t + 1) % m == 0 and (t + 1) // m - 1 < N_cap)


# ------------------------------------------- per-sequence positions, ring
def test_varlen_and_ring_attention_equal_per_sequence_uniform():
    rng = np.random.default_rng(10)
    B, Lq, H, D, N, k, W, R = 3, 2, 2, 128, 12, 4, 5, 8
    q = rng.standard_normal((B, Lq, H, D))
    k_c = rng.standard_normal((B, N, D)); v_c = rng.standard_normal((B, N, D))
    pos = np.array([20, 33, 41])
    T_lin = 64
    k_lin = rng.standard_normal((B, T_lin, D)); v_lin = rng.standard_normal((B, T_lin, D))
    # ring with the same rows for positions [t - R + Lq, t + Lq - 1] of each sequence
    k_ring = np.zeros((B, R, D)); v_ring = np.zeros((B, R, D))
    for b in range(B):
        for p in range(pos[b] + Lq - R, pos[b] + Lq):
            k_ring[b, p % R], v_ring[b, p % R] = k_lin[b, p], v_lin[b, p]
    idx = np.stack([np.stack([rng.permutation(N)[:k] for _ in range(Lq)]) for _ in range(B)])
    idx[0, 1, 2] = -1
    sink = rng.standard_normal(H)
    o_v, l_v = attention.csa_sparse_attn(q, pos, k_c, v_c, idx, k_ring, v_ring, 0, W, sink, ring=True)
    for b in range(B):
        o_u, l_u = attention.csa_sparse_attn(q[b:b + 1], int(pos[b]), k_c[b:b + 1], v_c[b:b + 1], idx[b:b + 1],
                                             k_lin[b:b + 1], v_lin[b:b + 1], 0, W, sink)
        assert np.allclose(o_v[b], o_u[0], atol=1e-12) and np.allclose(l_v[b], l_u[0], atol=1e-12)
    # HCA: per-sequence positions with m = 4 over a cache holding every entry
    Nh = (pos.max() + Lq) // 4
    kh = rng.standard_normal((B, Nh, D)); vh = rng.standard_normal((B, Nh, D))
    oh, lh = attention.hca_dense_attn(q, pos, 4, kh, vh, k_ring, v_ring, 0, W, sink, ring=True)
    for b in range(B):
        ou, lu = attention.hca_dense_attn(q[b:b + 1], int(pos[b]), 4, kh[b:b + 1], vh[b:b + 1],
                                          k_lin[b:b + 1], v_lin[b:b + 1], 0, W, sink)
        assert np.allclose(oh[b], ou[0], atol=1e-12) and np.allclose(lh[b], lu[0], atol=1e-12)


def test_varlen_indexer_and_topk_equal_per_sequence_uniform():
    rng = np.random.default_rng(11)
    B, Lq, HI, dI, m, N, k = 3, 2, 4, 8, 4, 40, 5
    q_i = rng.integers(-2, 3, (B, Lq, HI, dI)).astype(np.float64)
    w_i = rng.integers(-2, 3, (B, Lq, HI)).astype(np.float64)
    k_i = rng.integers(-2, 3, (B, N, dI)).astype(np.float64)
    pos = np.array([9, 30, 150 - 1 - Lq])
    pos[2] = N * m - Lq                     # the last query sees every entry
    s_v = indexer.index_scores_batch(q_i, w_i, k_i, pos, m)
    i_v = topk.topk_batch(np.where(np.isfinite(s_v), s_v, 0.0), k, pos, m)
    for b in range(B):
        s_u = indexer.index_scores_batch(q_i[b:b + 1], w_i[b:b + 1], k_i[b:b + 1], int(pos[b]), m)
        assert np.array_equal(s_v[b], s_u[0])
        i_u = topk.topk_batch(np.where(np.isfinite(s_u), s_u, 0.0), k, int(pos[b]), m)
        assert np.array_equal(i_v[b], i_u[0])
