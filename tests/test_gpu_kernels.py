"""GPU parity of each kernel against the CPU oracle at small sizes that still
span several tiles and ragged tails, through the C ABI."""
import numpy as np
import pytest
import torch

import long_context_attention_16_amd as csa
from long_context_attention_16_amd import workloads as wl
from oracle import attention as oatt
from oracle import compress as ocmp
from oracle import indexer as oidx
from oracle import topk as otopk
from helpers import assert_close, check_ki, dec, ki_alloc, kv_fmt

pytestmark = pytest.mark.gpu
DEV = "cuda"

# output bars: bf16 outputs (the stated bar) and float32 outputs
BAR_BF16 = (2e-2, 1e-3)
BAR_F32 = (1e-4, 1e-5)


def bars(fmt):
    return BAR_BF16 if fmt == "bf16" else BAR_F32


def _gen(seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


# --------------------------------------------------------------- compressor
@pytest.mark.parametrize("fmt,D,m,B,T,pos0,N_cap", [
    ("f32", 128, 4, 2, 66, 8, 40),        # two tail tokens make no entry
    ("bf16", 128, 4, 3, 200, 0, 50),
    ("bf16", 512, 128, 2, 384, 128, 4),
    ("f32", 512, 1, 1, 37, 5, 64),
    ("bf16", 512, 4, 1, 4096, 61440, 16384),
    # D = 128 reads four rows per wave load: m = 1, a partial last quad (m = 7), many quads (m = 128)
    ("bf16", 128, 1, 2, 37, 5, 64),
    ("f32", 128, 7, 1, 100, 14, 40),
    ("bf16", 128, 128, 1, 512, 0, 8),
])
def test_compress(fmt, D, m, B, T, pos0, N_cap):
    g = _gen(11)
    dt = torch.float32 if fmt == "f32" else torch.bfloat16
    k = torch.randn((B, T, D), generator=g, device=DEV).to(dt)
    v = torch.randn((B, T, D), generator=g, device=DEV).to(dt)
    w = (torch.randn((D,), generator=g, device=DEV) / D ** 0.5).contiguous()
    kc = torch.full((B, N_cap, D), 7.0, device=DEV).to(dt)
    vc = torch.full((B, N_cap, D), 7.0, device=DEV).to(dt)
    csa.compress(k, v, w, m, pos0, kc, vc)
    torch.cuda.synchronize()
    K, V, Wg = dec(k, fmt), dec(v, fmt), dec(w, "f32")
    r0, nb = pos0 // m, T // m
    gk, gv = dec(kc, fmt), dec(vc, fmt)
    for b in range(B):
        ek, ev = ocmp.compress(K[b], V[b], Wg, m, pos0)
        assert_close(gk[b, r0:r0 + nb], ek, *bars(fmt), what="k_c b=%d" % b)
        assert_close(gv[b, r0:r0 + nb], ev, *bars(fmt), what="v_c b=%d" % b)
    # rows outside the written range are untouched
    assert np.all(gk[:, :r0] == 7.0) and np.all(gk[:, r0 + nb:] == 7.0)


@pytest.mark.parametrize("kv,D,m,B,T,pos0,N_cap,idx_fmt,d_i", [
    ("bf16", 128, 4, 1, 4096, 61440, 16384, "fp8", 32),   # the prefill chunk's indexer keys
    ("bf16", 512, 4, 2, 200, 8, 60, "bf16", 128),
    ("f32", 128, 7, 2, 100, 14, 40, "f32", 64),           # a partial last quad of rows
    ("bf16", 128, 4, 3, 130, 0, 40, "fp4", 128),          # two tail tokens make no entry
    ("bf16", 512, 128, 1, 384, 128, 4, "fp4", 64),        # the HCA block
    ("f32", 512, 4, 1, 64, 0, 16, "fp8", 128),
])
def test_compress_index_key(kv, D, m, B, T, pos0, N_cap, idx_fmt, d_i):
    """The indexer-key fold of the batch compressor: the raw indexer keys of
    each block folded with the block's own softmax weights (unrotated), stored
    in the indexer's format; K and V as in test_compress."""
    g = _gen(13 + D + m + d_i)
    dt = torch.float32 if kv == "f32" else torch.bfloat16
    k = torch.randn((B, T, D), generator=g, device=DEV).to(dt)
    v = torch.randn((B, T, D), generator=g, device=DEV).to(dt)
    x = torch.randn((B, T, d_i), generator=g, device=DEV).to(dt)
    w = (torch.randn((D,), generator=g, device=DEV) / D ** 0.5).contiguous()
    kc = torch.full((B, N_cap, D), 7.0, device=DEV).to(dt)
    vc = torch.full((B, N_cap, D), 7.0, device=DEV).to(dt)
    ki_c, ki_sc = ki_alloc(B, N_cap, d_i, idx_fmt)
    mark = ki_c.clone()
    csa.compress(k, v, w, m, pos0, kc, vc, ki_raw=x, ki_c=ki_c, ki_scale=ki_sc, idx_fmt=idx_fmt)
    torch.cuda.synchronize()
    K, V, X, Wg = dec(k, kv), dec(v, kv), dec(x, kv), dec(w, "f32")
    r0, nb = pos0 // m, T // m
    want_x = np.zeros((B, N_cap, d_i))
    gk, gv = dec(kc, kv), dec(vc, kv)
    for b in range(B):
        ek, ev, ex = ocmp.compress(K[b], V[b], Wg, m, pos0, x_raw=X[b])
        assert_close(gk[b, r0:r0 + nb], ek, *bars(kv), what="k_c b=%d" % b)
        assert_close(gv[b, r0:r0 + nb], ev, *bars(kv), what="v_c b=%d" % b)
        want_x[b, r0:r0 + nb] = ex
    rows = [(b, j) for b in range(B) for j in range(r0, r0 + nb)]
    check_ki(ki_c, ki_sc, want_x, idx_fmt, kv, rows)
    # rows outside the written range are untouched
    assert torch.equal(ki_c[:, :r0], mark[:, :r0]) and torch.equal(ki_c[:, r0 + nb:], mark[:, r0 + nb:])


@pytest.mark.parametrize("kv,D,idx_fmt,d_i", [("bf16", 128, "fp8", 32), ("f32", 512, "fp4", 128),
                                              ("bf16", 512, "bf16", 64), ("f32", 128, "fp4", 64)])
def test_compress_index_key_exact_m1(kv, D, idx_fmt, d_i):
    # m = 1: each entry is its own row (softmax weight exactly 1), so every
    # code is the oracle encoder's, bit for bit
    g = _gen(17 + d_i)
    dt = torch.float32 if kv == "f32" else torch.bfloat16
    B, T, N_cap = 2, 37, 40
    k = torch.randn((B, T, D), generator=g, device=DEV).to(dt)
    v = torch.randn((B, T, D), generator=g, device=DEV).to(dt)
    x = (torch.randn((B, T, d_i), generator=g, device=DEV) * 3.0).to(dt)
    w = (torch.randn((D,), generator=g, device=DEV) / D ** 0.5).contiguous()
    kc = torch.zeros((B, N_cap, D), device=DEV).to(dt)
    vc = torch.zeros_like(kc)
    ki_c, ki_sc = ki_alloc(B, N_cap, d_i, idx_fmt)
    csa.compress(k, v, w, 1, 3, kc, vc, ki_raw=x, ki_c=ki_c, ki_scale=ki_sc, idx_fmt=idx_fmt)
    torch.cuda.synchronize()
    want = np.zeros((B, N_cap, d_i))
    want[:, 3:3 + T] = dec(x, kv)
    if idx_fmt == "bf16":
        # bf16 KV rows stored as bf16: the very same bits
        assert torch.equal(ki_c[:, 3:3 + T], x)
    check_ki(ki_c, ki_sc, want, idx_fmt, kv, [(b, j) for b in range(B) for j in range(3, 3 + T)], exact=True)


# ------------------------------------------------------------------ indexer
def _exact_indexer(B, Lq, H_i, d_i, N_cap, fmt, seed):
    s = wl.small_shape(B=B, Lq=Lq, H_I=H_i, d_I=d_i, N_cap=N_cap, idx=fmt, exact=True)
    return wl.indexer_inputs(s, _gen(seed), DEV)


def _index_exact_case(fmt, H_i, d_i, B, Lq, q_pos0, m, N_cap, topk, seed):
    x = _exact_indexer(B, Lq, H_i, d_i, N_cap, fmt, seed=seed)
    ws = torch.empty(csa.index_topk_ws_bytes(B, Lq, q_pos0, m, N_cap, topk) // 4 + 4, device=DEV)
    ws.fill_(float("nan"))                  # no initial contents are needed
    idx = csa.index_topk(x["q_i"], x["w_i"], x["k_i"], topk, q_pos0, m, fmt,
                         x["q_i_scale"], x["k_i_scale"], ws=ws)
    scores = csa.index_scores(x["q_i"], x["w_i"], x["k_i"], q_pos0, m, fmt, x["q_i_scale"], x["k_i_scale"])
    torch.cuda.synchronize()
    q = dec(x["q_i"], fmt, x["q_i_scale"])
    k = dec(x["k_i"], fmt, x["k_i_scale"])
    w = dec(x["w_i"], "f32")
    want = oidx.index_scores_batch(q, w, k, q_pos0, m)
    got = scores.cpu().numpy().astype(np.float64)
    vis = np.isfinite(want)
    assert np.array_equal(got[vis], want[vis]), "indexer scores not exact"
    assert np.all(np.isneginf(got[~vis])), "invisible entries written"
    want_idx = otopk.topk_batch(want, topk, q_pos0, m)
    assert np.array_equal(idx.cpu().numpy(), want_idx), "top-k indices differ"
    if (H_i >= 64 or Lq == 1) and topk <= 1024:
        # the fused path's two launches, called alone, give the same indices
        cand = csa.index_candidates(x["q_i"], x["w_i"], x["k_i"], topk, q_pos0, m, fmt,
                                    x["q_i_scale"], x["k_i_scale"])
        idx2 = csa.topk_merge(cand, B, Lq, topk, q_pos0, m)
        torch.cuda.synchronize()
        assert torch.equal(idx2, idx)


@pytest.mark.parametrize("fmt", ["f32", "bf16", "fp8", "fp4"])
@pytest.mark.parametrize("H_i,d_i", [(4, 32), (8, 64), (16, 128), (32, 32), (64, 128), (128, 64)])
def test_index_scores_and_topk_exact(fmt, H_i, d_i):
    # 21 query rows: H_i >= 64 takes the fused per-chunk top-k, smaller H_i the score path
    B, Lq, m, q_pos0, topk = 2, 21, 4, 4000, 100
    N_cap = (q_pos0 + Lq) // m + 3           # 1009: ragged against 32-entry tiles
    _index_exact_case(fmt, H_i, d_i, B, Lq, q_pos0, m, N_cap, topk, seed=H_i * 7 + d_i)


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "fp4"])
@pytest.mark.parametrize("H_i,d_i", [(4, 32), (16, 128), (64, 128), (128, 128)])
def test_index_topk_decode_fused_exact(fmt, H_i, d_i):
    # one query row: every head layout runs fused; 3 chunks of 2048 (the last ragged), heavy ties
    B, Lq, m, topk = 3, 1, 4, 300
    q_pos0 = 4 * 5001 - 1                    # n = 5001
    _index_exact_case(fmt, H_i, d_i, B, Lq, q_pos0, m, 5001 + 7, topk, seed=H_i + d_i)


@pytest.mark.parametrize("n,topk", [(700, 512), (2048, 512), (2049, 512), (4100, 1), (300, 300), (299, 300)])
def test_index_topk_fused_edges(n, topk):
    # chunk lists shorter than k (padding), n exactly at chunk ends, k = 1, n <= k (all selected + -1)
    B, Lq, m = 2, 1, 4
    q_pos0 = 4 * n - 1
    _index_exact_case("bf16", 64, 128, B, Lq, q_pos0, m, n + 40, topk, seed=n + topk)


@pytest.mark.parametrize("fmt", ["f32", "bf16", "fp8", "fp4"])
def test_index_topk_fused_k1024_exact(fmt):
    # 512 < k <= 1024 runs fused over 4096-entry chunks: 4 chunks, the last
    # one (712 entries) shorter than k, so its list is padded
    B, Lq, m, topk = 2, 1, 4, 1024
    n = 13000
    _index_exact_case(fmt, 64, 128, B, Lq, 4 * n - 1, m, n + 5, topk, seed=31)


@pytest.mark.parametrize("n,topk", [
    (4096, 1024),     # one full chunk, n > k: the chunk select
    (4097, 1024),     # a second chunk of one entry
    (1000, 1024),     # n <= k: every entry, then -1 padding
    (9000, 513),      # just above 512: 4096-entry chunks
    (70000, 1024),    # 18 lists: two merge levels (8 lists per workgroup)
    (300000, 1024),   # 74 lists: three merge levels
])
def test_index_topk_fused_k1024_edges(n, topk):
    B, Lq, m = 2, 1, 4
    _index_exact_case("fp4", 64, 128, B, Lq, 4 * n - 1, m, n + 40, topk, seed=n % 1000 + topk)


@pytest.mark.parametrize("B,Lq,m,q_pos0,n_extra,topk", [
    (2, 37, 4, 4 * 9000 - 20, 6, 100),   # 3 chunks of 4096 (last ragged), last query group of 5
    (1, 16, 2, 8191, 0, 1024),           # first query sees exactly one full chunk; N_cap = n
    (1, 64, 4, 0, 3, 100),               # queries 0..2 see nothing, the rest at most 16 entries
])
def test_index_prefill_fp8_exact(B, Lq, m, q_pos0, n_extra, topk):
    # the many-query fp8 kernel (64 heads x 128, at least 16 query rows)
    N_cap = (q_pos0 + Lq) // m + n_extra
    _index_exact_case("fp8", 64, 128, B, Lq, q_pos0, m, N_cap, topk, seed=Lq + m)


@pytest.mark.parametrize("H_i,d_i,Lq,q_pos0", [(64, 128, 1, 0), (64, 128, 1, 2), (128, 64, 1, 1),
                                               (4, 32, 3, 0)])
def test_index_topk_no_visible_entry(H_i, d_i, Lq, q_pos0):
    """Queries that see no compressed entry yet (t < m - 1): every slot is -1
    padding, on the fused path (one query per workgroup), its two launches
    called alone, and the score path (4 heads, 3 query rows)."""
    B, m, topk, N_cap = 2, 4, 512, 64
    x = _exact_indexer(B, Lq, H_i, d_i, N_cap, "bf16", seed=5 + q_pos0)
    out = torch.full((B, Lq, topk), 12345, dtype=torch.int32, device=DEV)
    csa.index_topk(x["q_i"], x["w_i"], x["k_i"], topk, q_pos0, m, "bf16", out=out)
    torch.cuda.synchronize()
    assert torch.all(out == -1)
    if Lq == 1:
        cand = csa.index_candidates(x["q_i"], x["w_i"], x["k_i"], topk, q_pos0, m, "bf16")
        out2 = torch.full((B, Lq, topk), 12345, dtype=torch.int32, device=DEV)
        csa.topk_merge(cand, B, Lq, topk, q_pos0, m, out=out2)
        # per-sequence positions bounded below m - 1
        q_pos = torch.tensor([q_pos0, 0], dtype=torch.int64, device=DEV)
        out3 = torch.full((B, Lq, topk), 12345, dtype=torch.int32, device=DEV)
        csa.index_topk_varlen(x["q_i"], x["w_i"], x["k_i"], topk, q_pos, 2, m, "bf16", out=out3)
        torch.cuda.synchronize()
        assert torch.all(out2 == -1) and torch.all(out3 == -1)


# -------------------------------------------------------------------- top-k
def _topk_case(scores, k, q_pos0, m):
    t = torch.from_numpy(scores.astype(np.float32)).to(DEV)
    idx = csa.topk(t, k, q_pos0, m)
    torch.cuda.synchronize()
    want = otopk.topk_batch(scores.astype(np.float32).astype(np.float64), k, q_pos0, m)
    assert np.array_equal(idx.cpu().numpy(), want)


@pytest.mark.parametrize("N,k,vals", [
    (40, 7, (-1.0, -0.0, 0.0, 1.0)),          # heavy ties and signed zeros
    (3000, 64, (-2.0, -1.0, 0.0, 1.0, 2.0)),
    (32768, 512, None),                        # decode shape, keys in LDS
    (33000, 1024, (0.0, 1.0)),                 # 5 chunks, ties across chunks
    (70000, 1024, None),
    (327680, 1024, None),                      # 40960 candidates: merge reads global keys
    (300000, 2048, (0.0, 1.0)),                # 75776 candidates, 3 compaction rounds, ties
])
def test_topk(N, k, vals):
    rng = np.random.default_rng(N + k)
    B, Lq, m = 2, 3, 4
    q_pos0 = N * m - Lq                        # last row sees all N entries
    if vals is None:
        s = rng.standard_normal((B, Lq, N)).astype(np.float32)
    else:
        s = rng.choice(np.array(vals, dtype=np.float32), size=(B, Lq, N))
    _topk_case(s, k, q_pos0, m)


def test_topk_multichunk_ragged_rows():
    """One launch whose first rows see fewer than k entries and whose last
    rows span two chunks (rows checked by sampling)."""
    rng = np.random.default_rng(8)
    Lq, k, q_pos0 = 6300, 2048, 1999               # n = 2000 .. 8299
    s = rng.integers(-3, 4, size=(1, Lq, 8300)).astype(np.float32)
    t = torch.from_numpy(s).to(DEV)
    idx = csa.topk(t, k, q_pos0, 1).cpu().numpy()
    for i in (0, 1, 47, 2000, 6191, 6192, 6250, 6299):
        n = q_pos0 + i + 1
        want = otopk.topk_select(s[0, i, :n].astype(np.float64), k)
        assert np.array_equal(idx[0, i], want), i


def test_topk_small_n_and_padding():
    rng = np.random.default_rng(3)
    s = rng.standard_normal((1, 12, 64)).astype(np.float32)
    _topk_case(s, 16, 0, 4)                     # n(t) = 0..3: all visible then -1
    _topk_case(s, 16, 40, 4)                    # n = 10..12 < 16


def test_topk_all_equal():
    s = np.zeros((1, 2, 5000), dtype=np.float32)
    s[0, 1, ::2] = -0.0
    _topk_case(s, 700, 5000 * 2 - 2, 2)


# ---------------------------------------------------------------- attention
def _attn_inputs(fmt, B, Lq, H, D, N_cap, T_raw, seed):
    g = _gen(seed)
    dt = torch.float32 if fmt == "f32" else torch.bfloat16
    r = lambda *s: torch.randn(s, generator=g, device=DEV).to(dt)
    return dict(q=r(B, Lq, H, D), k_c=r(B, N_cap, D), v_c=r(B, N_cap, D), k_raw=r(B, T_raw, D),
                v_raw=r(B, T_raw, D), sink=torch.randn((H,), generator=g, device=DEV))


def _rand_idx(B, Lq, k, q_pos0, m, N_cap, seed, pad=True):
    rng = np.random.default_rng(seed)
    idx = np.full((B, Lq, k), -1, dtype=np.int32)
    for b in range(B):
        for i in range(Lq):
            n = min(N_cap, (q_pos0 + i + 1) // m)
            take = min(n, k if not pad else int(rng.integers(max(1, k // 2), k + 1)))
            idx[b, i, :take] = np.sort(rng.choice(n, size=take, replace=False))
    return idx


def _oracle_attn(x, fmt, idx, q_pos0, raw_pos0, W, sink, hca_m=None):
    q, kc, vc = dec(x["q"], fmt), dec(x["k_c"], fmt), dec(x["v_c"], fmt)
    kr, vr = dec(x["k_raw"], fmt), dec(x["v_raw"], fmt)
    s = None if sink is None else dec(sink, "f32")
    if hca_m is None:
        return oatt.csa_sparse_attn(q, q_pos0, kc, vc, idx, kr, vr, raw_pos0, W, s)
    return oatt.hca_dense_attn(q, q_pos0, hca_m, kc, vc, kr, vr, raw_pos0, W, s)


@pytest.mark.parametrize("fmt,B,Lq,H,D,k,W,sink", [
    ("f32", 2, 9, 4, 128, 64, 128, True),     # the 2K prefill head layout
    ("bf16", 2, 5, 4, 128, 100, 16, True),
    ("bf16", 2, 2, 64, 512, 512, 128, True),  # decode head layout, 10 splits
    ("bf16", 1, 3, 16, 512, 40, 0, False),    # no window, no sink
    ("f32", 1, 3, 32, 512, 24, 7, True),
    ("bf16", 1, 2, 128, 128, 300, 33, True),
    ("f32", 1, 2, 8, 512, 300, 64, True),     # f32 rows of 512 split 4 ways: 128 combine threads per row
    ("bf16", 1, 2, 4, 128, 2048, 1024, True),  # 3072 sources: six splits of 576 rows (the staged idx slots full)
    ("f32", 1, 2, 4, 128, 1024, 128, True),    # 1152 sources: two splits of 576 rows
])
def test_sparse_attn(fmt, B, Lq, H, D, k, W, sink):
    m, q_pos0 = 4, 3000
    N_cap = (q_pos0 + Lq) // m
    raw_pos0 = q_pos0 - W - 3 if W else 0
    T_raw = q_pos0 + Lq - raw_pos0 + 2
    x = _attn_inputs(fmt, B, Lq, H, D, N_cap, T_raw, seed=H + D + k)
    idx = _rand_idx(B, Lq, k, q_pos0, m, N_cap, seed=k)
    s = x["sink"] if sink else None
    out, lse = csa.sparse_attn(x["q"], x["k_c"], x["v_c"], torch.from_numpy(idx).to(DEV), x["k_raw"],
                               x["v_raw"], raw_pos0, W, s, q_pos0)
    torch.cuda.synchronize()
    eo, el = _oracle_attn(x, fmt, idx, q_pos0, raw_pos0, W, s)
    assert_close(dec(out, fmt), eo, *bars(fmt), what="out")
    assert_close(lse.cpu().numpy(), el, 5e-3 if fmt == "bf16" else 1e-5, 1e-3, what="lse")


@pytest.mark.parametrize("B,Lq,H,k,W,q_pos0,sink", [
    (1, 1, 32, 1024, 128, 8000, True),     # 1152 sources: 32-dim P V slices, all 1152 rows staged at once
    (20, 1, 16, 1024, 128, 6000, True),    # 20 rows: 32-dim slices, two staged blocks (640 + 512 rows)
    (33, 1, 16, 600, 100, 3000, True),     # 33 rows: 64-dim slices, two staged blocks (640 + 64 rows)
    (2, 2, 48, 200, 128, 50, True),        # window cut at t = 50 < W, padded idx
    (1, 2, 128, 300, 40, 5000, False),     # 128 heads, no sink
    (3, 1, 16, 64, 0, 900, True),          # compressed only
    (1, 2, 16, 2048, 256, 9000, True),     # 2304 sources: the most the two-launch path takes
    (1, 2, 16, 2048, 300, 9000, True),     # 2348 sources: beyond it, the general split kernel
])
def test_sparse_attn_many_heads(B, Lq, H, k, W, q_pos0, sink):
    # bf16, D = 512, H a multiple of 16: the two-launch path (logits, then P V per D slice)
    fmt, D, m = "bf16", 512, 4
    N_cap = (q_pos0 + Lq) // m + 2
    raw_pos0 = max(0, q_pos0 - W - 1)
    T_raw = q_pos0 + Lq - raw_pos0 + 1
    x = _attn_inputs(fmt, B, Lq, H, D, N_cap, T_raw, seed=H + k + W)
    idx = _rand_idx(B, Lq, k, q_pos0, m, N_cap, seed=k + H)
    s = x["sink"] if sink else None
    out, lse = csa.sparse_attn(x["q"], x["k_c"], x["v_c"], torch.from_numpy(idx).to(DEV), x["k_raw"],
                               x["v_raw"], raw_pos0, W, s, q_pos0)
    torch.cuda.synchronize()
    eo, el = _oracle_attn(x, fmt, idx, q_pos0, raw_pos0, W, s)
    assert_close(dec(out, fmt), eo, *bars(fmt), what="out")
    assert_close(lse.cpu().numpy(), el, 5e-3, 1e-3, what="lse")


def test_sparse_attn_many_heads_edges():
    """The two-launch path at t < m-1: no source at all (out 0, lse -inf), a
    sink only (out 0, lse = sink), and a window only."""
    fmt, B, Lq, H, D, k = "bf16", 1, 3, 16, 512, 8
    x = _attn_inputs(fmt, B, Lq, H, D, 16, 8, seed=6)
    idx = np.full((B, Lq, k), -1, dtype=np.int32)
    it = torch.from_numpy(idx).to(DEV)
    out, lse = csa.sparse_attn(x["q"], x["k_c"], x["v_c"], it, x["k_raw"], x["v_raw"], 0, 0, None, 0)
    torch.cuda.synchronize()
    assert torch.all(out.float() == 0) and torch.all(torch.isneginf(lse))
    out, lse = csa.sparse_attn(x["q"], x["k_c"], x["v_c"], it, x["k_raw"], x["v_raw"], 0, 0, x["sink"], 0)
    torch.cuda.synchronize()
    assert torch.all(out.float() == 0)
    assert torch.allclose(lse[0, 0].cpu(), x["sink"].cpu())
    out, lse = csa.sparse_attn(x["q"], x["k_c"], x["v_c"], it, x["k_raw"], x["v_raw"], 0, 5, x["sink"], 0)
    torch.cuda.synchronize()
    eo, el = _oracle_attn(x, fmt, idx, 0, 0, 5, x["sink"])
    assert_close(dec(out, fmt), eo, *BAR_BF16, what="window-only")
    assert_close(lse.cpu().numpy(), el, 5e-3, 1e-3, what="window-only lse")


def test_sparse_attn_edges():
    """t < m-1 with no window and no sink: no source at all -> out 0, lse -inf;
    with a sink only -> out 0, lse = sink; all slots -1 -> window-only."""
    fmt, B, Lq, H, D, k = "bf16", 1, 4, 16, 128, 8
    x = _attn_inputs(fmt, B, Lq, H, D, 16, 8, seed=5)
    idx = np.full((B, Lq, k), -1, dtype=np.int32)
    it = torch.from_numpy(idx).to(DEV)
    out, lse = csa.sparse_attn(x["q"], x["k_c"], x["v_c"], it, x["k_raw"], x["v_raw"], 0, 0, None, 0)
    torch.cuda.synchronize()
    assert torch.all(out.float() == 0) and torch.all(torch.isneginf(lse))
    out, lse = csa.sparse_attn(x["q"], x["k_c"], x["v_c"], it, x["k_raw"], x["v_raw"], 0, 0, x["sink"], 0)
    torch.cuda.synchronize()
    assert torch.all(out.float() == 0)
    assert torch.allclose(lse[0, 0].cpu(), x["sink"].cpu())
    out, lse = csa.sparse_attn(x["q"], x["k_c"], x["v_c"], it, x["k_raw"], x["v_raw"], 0, 5, x["sink"], 0)
    torch.cuda.synchronize()
    eo, el = _oracle_attn(x, fmt, idx, 0, 0, 5, x["sink"])
    assert_close(dec(out, fmt), eo, *BAR_BF16, what="window-only")


@pytest.mark.parametrize("fmt,B,Lq,H,D,m,q_pos0,W", [
    ("bf16", 2, 1, 64, 512, 128, 70000, 128),   # 547 entries + window: several splits
    ("f32", 1, 6, 4, 128, 4, 250, 16),           # prefill rows with ragged n(t)
    ("bf16", 2, 3, 64, 512, 128, 126, 20),       # n(t) = 0 or 1
    ("f32", 1, 2, 16, 512, 4, 3000, 32),         # f32 rows of 512, several splits
    ("bf16", 1, 4, 16, 512, 4, 700, 40),         # one head group (two waves), ragged n(t), 3 splits
    ("bf16", 2, 2, 20, 512, 8, 3000, 64),        # two head groups, the second padded
    ("bf16", 1, 1, 48, 512, 128, 300000, 128),   # three head groups, 2471 sources
    # sources 4600 .. 4609 over the chunk: 16 splits of 288 rows up to 4608,
    # 15 of 320 at 4609 (the split count is not monotonic in the source
    # count), so the grid must be sized for more splits than the last row's
    ("bf16", 1, 41, 4, 128, 4, 17887, 128),
    # a decode batch of 8 at 1M context with m' = 128 (16 splits of 544 rows)
    ("bf16", 8, 1, 64, 512, 128, 1048575, 128),
    # 32 heads, rows beyond 4096 sources, ragged n(t)
    ("bf16", 3, 2, 32, 512, 4, 20001, 128),
    # 32 heads, one split, a window cut at position 0 (fewer window rows than W)
    ("bf16", 2, 2, 32, 512, 128, 900, 1024),
])
def test_hca_attn(fmt, B, Lq, H, D, m, q_pos0, W):
    N_cap = (q_pos0 + Lq) // m + 1
    raw_pos0 = max(0, q_pos0 - W + 1)
    T_raw = q_pos0 + Lq - raw_pos0
    x = _attn_inputs(fmt, B, Lq, H, D, N_cap, T_raw, seed=D + m)
    out, lse = csa.hca_attn(x["q"], x["k_c"], x["v_c"], m, x["k_raw"], x["v_raw"], raw_pos0, W,
                            x["sink"], q_pos0)
    torch.cuda.synchronize()
    eo, el = _oracle_attn(x, fmt, None, q_pos0, raw_pos0, W, x["sink"], hca_m=m)
    assert_close(dec(out, fmt), eo, *bars(fmt), what="out")
    assert_close(lse.cpu().numpy(), el, 5e-3 if fmt == "bf16" else 1e-5, 1e-3, what="lse")


@pytest.mark.parametrize("B", [4, 40])
def test_determinism_and_batch_invariance(B):
    """Same inputs give bitwise-equal outputs; a sequence alone equals itself
    inside a batch (the split structure depends on the query only). At batch
    40 the decode kernel's second launch takes 64-dim slices of D, alone
    32-dim ones: the bits must not change."""
    fmt, Lq, H, D, k, W = "bf16", 1, 64, 512, 512, 128
    q_pos0 = 40000
    N_cap = (q_pos0 + 1) // 4
    raw_pos0 = q_pos0 - W + 1
    x = _attn_inputs(fmt, B, Lq, H, D, N_cap, W, seed=77)
    idx = torch.from_numpy(_rand_idx(B, Lq, k, q_pos0, 4, N_cap, seed=9)).to(DEV)
    a, _ = csa.sparse_attn(x["q"], x["k_c"], x["v_c"], idx, x["k_raw"], x["v_raw"], raw_pos0, W, x["sink"], q_pos0)
    b, _ = csa.sparse_attn(x["q"], x["k_c"], x["v_c"], idx, x["k_raw"], x["v_raw"], raw_pos0, W, x["sink"], q_pos0)
    one, _ = csa.sparse_attn(x["q"][2:3].contiguous(), x["k_c"][2:3].contiguous(), x["v_c"][2:3].contiguous(),
                             idx[2:3].contiguous(), x["k_raw"][2:3].contiguous(), x["v_raw"][2:3].contiguous(),
                             raw_pos0, W, x["sink"], q_pos0)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a[2:3].view(torch.int16), one.view(torch.int16))
