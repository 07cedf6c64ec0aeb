"""GPU parity of the decode state cache (csa_state_append) and of the
per-sequence-position calls (*_varlen) against the CPU oracle, through the C
ABI: ring contents bit-exact, compressed rows to the output bars, quantized
indexer keys to their codes (exact where the fold is exact, m = 1), indexer
top-k exact on integer inputs, attention to the output bars; and a decode loop
whose rings wrap."""
import numpy as np
import pytest
import torch

import long_context_attention_16_amd as csa
from long_context_attention_16_amd import workloads as wl
from oracle import attention as oatt
from oracle import formats as ofmt
from oracle import indexer as oidx
from oracle import state as ostate
from oracle import topk as otopk
from helpers import assert_close, dec, topk_matches_up_to_ties
from helpers import check_ki as _check_ki, ki_alloc as _ki_alloc

pytestmark = pytest.mark.gpu
DEV = "cuda"
BAR_BF16 = (2e-2, 1e-3)
BAR_F32 = (1e-4, 1e-5)


def bars(fmt):
    return BAR_BF16 if fmt == "bf16" else BAR_F32


def _gen(seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


def _dt(fmt):
    return torch.float32 if fmt == "f32" else torch.bfloat16


@pytest.mark.parametrize("kv,D,m,R,idx_fmt,d_i", [
    ("bf16", 512, 4, 128, "bf16", 128),    # the CSA decode cache
    ("f32", 128, 4, 8, "f32", 32),
    ("bf16", 512, 128, 128, "fp8", 128),   # HCA block (the indexer key only for the test)
    ("bf16", 128, 4, 132, "fp4", 64),
    ("f32", 512, 7, 9, "fp8", 128),        # a block that is not a power of two
    ("bf16", 512, 4, 128, None, 0),        # no indexer key
])
def test_state_append(kv, D, m, R, idx_fmt, d_i):
    g = _gen(21 + D + m)
    dt = _dt(kv)
    B, N_cap = 6, 40
    # positions: completes a block, mid-block, inactive, block j >= N_cap, first token, completes block 0
    pos = [m * 9 - 1, m * 9 + 1, -1, m * (N_cap + 1) - 1, 0, m - 1]
    k_new = torch.randn((B, D), generator=g, device=DEV).to(dt)
    v_new = torch.randn((B, D), generator=g, device=DEV).to(dt)
    w = (torch.randn((D,), generator=g, device=DEV) / D ** 0.5).contiguous()
    k_ring = torch.randn((B, R, D), generator=g, device=DEV).to(dt)
    v_ring = torch.randn((B, R, D), generator=g, device=DEV).to(dt)
    k_c = torch.full((B, N_cap, D), 7.0, device=DEV).to(dt)
    v_c = torch.full((B, N_cap, D), 7.0, device=DEV).to(dt)
    ki_new = ki_ring = ki_c = ki_sc = None
    if d_i:
        ki_new = torch.randn((B, d_i), generator=g, device=DEV).to(dt)
        ki_ring = torch.randn((B, R, d_i), generator=g, device=DEV).to(dt)
        ki_c, ki_sc = _ki_alloc(B, N_cap, d_i, idx_fmt)
    rings0 = (k_ring.clone(), v_ring.clone(), None if ki_ring is None else ki_ring.clone())
    pos_t = torch.tensor(pos, dtype=torch.int64, device=DEV)
    csa.state_append(pos_t, k_new, v_new, w, m, k_ring, v_ring, k_c, v_c, ki_new, ki_ring, ki_c, ki_sc,
                     idx_fmt or "bf16")
    torch.cuda.synchronize()

    # oracle on the decoded inputs
    K, V = dec(rings0[0], kv), dec(rings0[1], kv)
    KI = None if not d_i else dec(rings0[2], kv)
    okc, ovc = np.full((B, N_cap, D), 7.0), np.full((B, N_cap, D), 7.0)
    oki = None if not d_i else np.zeros((B, N_cap, d_i))
    active = [b for b in range(B) if pos[b] >= 0]       # a negative position is skipped
    written = []
    for b in active:
        w_b = ostate.state_append(np.array([pos[b]]), dec(k_new, kv)[b:b + 1], dec(v_new, kv)[b:b + 1],
                                  K[b:b + 1], V[b:b + 1], dec(w, "f32"), m, okc[b:b + 1], ovc[b:b + 1],
                                  None if not d_i else dec(ki_new, kv)[b:b + 1],
                                  None if not d_i else KI[b:b + 1], None if not d_i else oki[b:b + 1])
        written += [(b, j) for _, j in w_b]
    assert sorted(written) == sorted([(0, 8), (5, 0)])
    # rings: bit-exact (the oracle's f64 rings hold the decoded bytes)
    assert np.array_equal(dec(k_ring, kv), K) and np.array_equal(dec(v_ring, kv), V)
    if d_i:
        assert np.array_equal(dec(ki_ring, kv), KI)
    gk, gv = dec(k_c, kv), dec(v_c, kv)
    for b, j in written:
        assert_close(gk[b, j], okc[b, j], *bars(kv), what="k_c b=%d" % b)
        assert_close(gv[b, j], ovc[b, j], *bars(kv), what="v_c b=%d" % b)
    mask = np.ones((B, N_cap), dtype=bool)
    for b, j in written:
        mask[b, j] = False
    assert np.all(gk[mask] == 7.0) and np.all(gv[mask] == 7.0), "rows other than completed blocks written"
    if d_i:
        _check_ki(ki_c, ki_sc, oki, idx_fmt, kv, written)
        if idx_fmt in ("fp8", "fp4"):
            assert np.all(ki_c.cpu().numpy()[mask] == 0x77)
        else:
            assert np.all(dec(ki_c, idx_fmt)[mask] == 7.0)


@pytest.mark.parametrize("kv,idx_fmt,d_i", [("f32", "fp8", 128), ("bf16", "fp4", 128), ("bf16", "fp8", 32),
                                            ("f32", "fp4", 64), ("bf16", "bf16", 64)])
def test_state_append_quantization_exact(kv, idx_fmt, d_i):
    """m = 1: the fold of one row is that row exactly, so the stored codes are
    the encoders' codes of the input, bit for bit."""
    g = _gen(33 + d_i)
    dt = _dt(kv)
    B, D, R, N_cap = 8, 128, 4, 64
    k_new = torch.randn((B, D), generator=g, device=DEV).to(dt)
    v_new = torch.randn((B, D), generator=g, device=DEV).to(dt)
    # magnitudes over many binades, exact zeros and values past e4m3's range
    ki_new = (torch.randn((B, d_i), generator=g, device=DEV) *
              torch.exp2(torch.randint(-12, 10, (B, 1), generator=g, device=DEV).float())).to(dt)
    ki_new[0, :5] = 0.0
    ki_new[1, :3] = torch.tensor([600.0, -1000.0, 448.0], device=DEV).to(dt)
    ki_new[2].zero_()                                    # an all-zero MX block
    w = torch.zeros((D,), device=DEV)
    k_ring = torch.zeros((B, R, D), device=DEV).to(dt)
    v_ring = torch.zeros_like(k_ring)
    ki_ring = torch.zeros((B, R, d_i), device=DEV).to(dt)
    k_c = torch.zeros((B, N_cap, D), device=DEV).to(dt)
    v_c = torch.zeros_like(k_c)
    ki_c, ki_sc = _ki_alloc(B, N_cap, d_i, idx_fmt)
    pos = torch.arange(B, dtype=torch.int64, device=DEV) * 5 + 3
    csa.state_append(pos, k_new, v_new, w, 1, k_ring, v_ring, k_c, v_c, ki_new, ki_ring, ki_c, ki_sc, idx_fmt)
    torch.cuda.synchronize()
    x = dec(ki_new, kv)
    p = pos.cpu().numpy()
    if idx_fmt == "fp8":
        assert np.array_equal(ki_c.cpu().numpy()[np.arange(B), p], ofmt.f64_to_e4m3fn(x))
    elif idx_fmt == "fp4":
        pk, sc = ofmt.f64_to_mxfp4(x)
        assert np.array_equal(ki_sc.cpu().numpy()[np.arange(B), p], sc)
        assert np.array_equal(ki_c.cpu().numpy()[np.arange(B), p], pk)
    else:
        assert np.array_equal(dec(ki_c, "bf16")[np.arange(B), p], x)  # bf16 input: exact
    # V is the row itself; K its rotation at the block's position (m = 1)
    assert np.array_equal(dec(v_c, kv)[np.arange(B), p], dec(v_new, kv))


# --------------------------------------------------- per-sequence positions
def _exact_indexer(B, Lq, H_i, d_i, N_cap, fmt, seed):
    s = wl.small_shape(B=B, Lq=Lq, H_I=H_i, d_I=d_i, N_cap=N_cap, idx=fmt, exact=True)
    return wl.indexer_inputs(s, _gen(seed), DEV)


@pytest.mark.parametrize("fmt,H_i,d_i,Lq,m,topk", [
    ("bf16", 64, 128, 1, 4, 512),    # the fused decode path
    ("fp8", 64, 128, 1, 4, 100),
    ("fp4", 64, 128, 1, 4, 64),
    ("fp4", 64, 128, 1, 4, 1024),    # fused over 4096-entry chunks, rows of different lengths
    ("bf16", 4, 32, 3, 4, 50),       # grouped queries, scores + top-k
    ("fp8", 64, 128, 20, 4, 64),     # the many-query fp8 kernel
])
def test_index_topk_varlen_exact(fmt, H_i, d_i, Lq, m, topk):
    B = 4
    pos = [9000, 123, 0, 20000]      # 0: a query that sees no entry (m > 1) or one
    q_pos_max = 20000
    N_cap = (q_pos_max + Lq) // m + 3
    x = _exact_indexer(B, Lq, H_i, d_i, N_cap, fmt, seed=H_i + Lq)
    q_pos = torch.tensor(pos, dtype=torch.int64, device=DEV)
    idx = csa.index_topk_varlen(x["q_i"], x["w_i"], x["k_i"], topk, q_pos, q_pos_max, m, fmt,
                                x["q_i_scale"], x["k_i_scale"])
    torch.cuda.synchronize()
    q = dec(x["q_i"], fmt, x["q_i_scale"])
    k = dec(x["k_i"], fmt, x["k_i_scale"])
    w = dec(x["w_i"], "f32")
    want = oidx.index_scores_batch(q, w, k, np.array(pos), m)
    want_idx = otopk.topk_batch(np.where(np.isfinite(want), want, 0.0), topk, np.array(pos), m)
    assert np.array_equal(idx.cpu().numpy(), want_idx), "per-sequence top-k differs"


def _attn_case(kv, B, Lq, H, D, N_cap, R, seed):
    g = _gen(seed)
    dt = _dt(kv)
    r = lambda *s: torch.randn(s, generator=g, device=DEV).to(dt)
    return dict(q=r(B, Lq, H, D), k_c=r(B, N_cap, D), v_c=r(B, N_cap, D), k_ring=r(B, R, D),
                v_ring=r(B, R, D), sink=torch.randn((H,), generator=g, device=DEV))


@pytest.mark.parametrize("kv,Lq,H,D,k,W,R", [
    ("bf16", 1, 64, 512, 512, 128, 128),   # the two-launch decode kernel
    ("bf16", 2, 32, 512, 200, 100, 105),   # a ring a little longer than the windows
    ("f32", 3, 4, 128, 64, 16, 20),        # the split-KV kernel
    ("bf16", 1, 16, 512, 2048, 256, 260),  # 2304 sources: the most the two-launch kernel takes
    ("bf16", 1, 16, 512, 2048, 400, 400),  # 2448 sources: the split-KV kernel over the rings
])
def test_sparse_attn_varlen(kv, Lq, H, D, k, W, R):
    B, m = 4, 4
    pos = [131071 - Lq, 5000, 60, 2]       # 60 < W for the larger windows; 2: window cut at 0
    q_pos_max = 131071
    N_cap = (q_pos_max + Lq) // m
    x = _attn_case(kv, B, Lq, H, D, N_cap, R, seed=H + R)
    rng = np.random.default_rng(k)
    idx = np.full((B, Lq, k), -1, dtype=np.int32)
    for b in range(B):
        for i in range(Lq):
            n = (pos[b] + i + 1) // m
            take = min(n, int(rng.integers(k // 2, k + 1)))
            idx[b, i, :take] = np.sort(rng.choice(n, size=take, replace=False)) if take else []
    q_pos = torch.tensor(pos, dtype=torch.int64, device=DEV)
    out, lse = csa.sparse_attn_varlen(x["q"], x["k_c"], x["v_c"], torch.from_numpy(idx).to(DEV), x["k_ring"],
                                      x["v_ring"], W, x["sink"], q_pos, q_pos_max)
    torch.cuda.synchronize()
    eo, el = oatt.csa_sparse_attn(dec(x["q"], kv), np.array(pos), dec(x["k_c"], kv), dec(x["v_c"], kv), idx,
                                  dec(x["k_ring"], kv), dec(x["v_ring"], kv), 0, W, dec(x["sink"], "f32"),
                                  ring=True)
    assert_close(dec(out, kv), eo, *bars(kv), what="out")
    assert_close(lse.cpu().numpy(), el, 5e-3 if kv == "bf16" else 1e-5, 1e-3, what="lse")


@pytest.mark.parametrize("kv,Lq,H,D,m,W,R", [
    ("bf16", 1, 64, 512, 128, 128, 128),
    ("f32", 2, 4, 128, 4, 16, 17),
])
def test_hca_attn_varlen(kv, Lq, H, D, m, W, R):
    B = 3
    pos = [70000, 300, 126]                 # 126 + 1 < m' = 128: no entry yet for the first row
    q_pos_max = 70000
    N_cap = (q_pos_max + Lq) // m + 1
    x = _attn_case(kv, B, Lq, H, D, N_cap, R, seed=D + m)
    q_pos = torch.tensor(pos, dtype=torch.int64, device=DEV)
    out, lse = csa.hca_attn_varlen(x["q"], x["k_c"], x["v_c"], m, x["k_ring"], x["v_ring"], W, x["sink"],
                                   q_pos, q_pos_max)
    torch.cuda.synchronize()
    eo, el = oatt.hca_dense_attn(dec(x["q"], kv), np.array(pos), m, dec(x["k_c"], kv), dec(x["v_c"], kv),
                                 dec(x["k_ring"], kv), dec(x["v_ring"], kv), 0, W, dec(x["sink"], "f32"),
                                 ring=True)
    assert_close(dec(out, kv), eo, *bars(kv), what="out")
    assert_close(lse.cpu().numpy(), el, 5e-3 if kv == "bf16" else 1e-5, 1e-3, what="lse")


def test_hca_attn_varlen_split_count_dip():
    """The bound q_pos_max = 17924 gives 4481 + 128 = 4609 sources (15 splits
    of 320 rows); the sequence at 17920 has 4608 (16 splits of 288): the grid
    must hold more splits than the bound's row."""
    kv, Lq, H, D, m, W, R = "bf16", 1, 4, 128, 4, 128, 128
    pos = [17924, 17920, 300]
    q_pos_max = 17924
    N_cap = (q_pos_max + Lq) // m + 1
    x = _attn_case(kv, len(pos), Lq, H, D, N_cap, R, seed=29)
    q_pos = torch.tensor(pos, dtype=torch.int64, device=DEV)
    out, lse = csa.hca_attn_varlen(x["q"], x["k_c"], x["v_c"], m, x["k_ring"], x["v_ring"], W, x["sink"],
                                   q_pos, q_pos_max)
    torch.cuda.synchronize()
    eo, el = oatt.hca_dense_attn(dec(x["q"], kv), np.array(pos), m, dec(x["k_c"], kv), dec(x["v_c"], kv),
                                 dec(x["k_ring"], kv), dec(x["v_ring"], kv), 0, W, dec(x["sink"], "f32"),
                                 ring=True)
    assert_close(dec(out, kv), eo, *bars(kv), what="out")
    assert_close(lse.cpu().numpy(), el, 5e-3, 1e-3, what="lse")


def test_varlen_positions_clamped_to_bound():
    """Positions above q_pos_max act as q_pos_max, negative ones as 0."""
    kv, Lq, H, D, k, W, R, m = "f32", 1, 4, 128, 16, 8, 8, 4
    B, q_pos_max = 2, 100
    N_cap = (q_pos_max + Lq) // m
    x = _attn_case(kv, B, Lq, H, D, N_cap, R, seed=3)
    idx = np.tile(np.arange(k, dtype=np.int32), (B, Lq, 1))
    it = torch.from_numpy(idx).to(DEV)
    o1, l1 = csa.sparse_attn_varlen(x["q"], x["k_c"], x["v_c"], it, x["k_ring"], x["v_ring"], W, x["sink"],
                                    torch.tensor([5000, -7], dtype=torch.int64, device=DEV), q_pos_max)
    o2, l2 = csa.sparse_attn_varlen(x["q"], x["k_c"], x["v_c"], it, x["k_ring"], x["v_ring"], W, x["sink"],
                                    torch.tensor([100, 0], dtype=torch.int64, device=DEV), q_pos_max)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ------------------------------------------------------------- decode loop
def test_decode_loop_state_cache():
    """Twelve decode steps of three sequences at different positions: append
    (rings of 8 slots wrap), indexer top-k and sparse attention with
    per-sequence positions. Each call is checked against the oracle on the
    same inputs, and the caches against the oracle's state kept alongside."""
    kv, D, H, m, R, W, k = "bf16", 512, 16, 4, 8, 6, 8
    H_i, d_i, idx_fmt = 64, 128, "bf16"
    B, N_cap = 3, 64
    g = _gen(77)
    dt = _dt(kv)
    starts = [37, 101, 6]
    q_pos_max = max(starts) + 12
    w = (torch.randn((D,), generator=g, device=DEV) / D ** 0.5).contiguous()
    k_ring = torch.zeros((B, R, D), device=DEV).to(dt)
    v_ring = torch.zeros_like(k_ring)
    ki_ring = torch.zeros((B, R, d_i), device=DEV).to(dt)
    k_c = torch.randn((B, N_cap, D), generator=g, device=DEV).to(dt)   # entries before the start
    v_c = torch.randn((B, N_cap, D), generator=g, device=DEV).to(dt)
    ki_c = torch.randn((B, N_cap, d_i), generator=g, device=DEV).to(dt)
    sink = torch.randn((H,), generator=g, device=DEV)
    # the rows before each start are in the rings (as after a prefill)
    o_kr, o_vr, o_xr = dec(k_ring, kv), dec(v_ring, kv), dec(ki_ring, kv)
    pre = torch.randn((B, R, D), generator=g, device=DEV).to(dt)
    for b, s in enumerate(starts):
        for p in range(max(0, s - R), s):
            k_ring[b, p % R] = pre[b, p % R]
            v_ring[b, p % R] = pre[b, (p + 1) % R]
            ki_ring[b, p % R] = pre[b, p % R, :d_i]
    o_kr, o_vr, o_xr = dec(k_ring, kv), dec(v_ring, kv), dec(ki_ring, kv)
    o_kc, o_vc, o_xc = dec(k_c, kv), dec(v_c, kv), dec(ki_c, kv)
    for step in range(12):
        pos = np.array([s + step for s in starts])
        pos_t = torch.from_numpy(pos).to(DEV)
        k_new = torch.randn((B, D), generator=g, device=DEV).to(dt)
        v_new = torch.randn((B, D), generator=g, device=DEV).to(dt)
        ki_new = torch.randn((B, d_i), generator=g, device=DEV).to(dt)
        csa.state_append(pos_t, k_new, v_new, w, m, k_ring, v_ring, k_c, v_c, ki_new, ki_ring, ki_c, None, idx_fmt)
        written = ostate.state_append(pos, dec(k_new, kv), dec(v_new, kv), o_kr, o_vr, dec(w, "f32"), m, o_kc, o_vc,
                                      dec(ki_new, kv), o_xr, o_xc)
        torch.cuda.synchronize()
        assert np.array_equal(dec(k_ring, kv), o_kr) and np.array_equal(dec(ki_ring, kv), o_xr)
        gk, gx = dec(k_c, kv), dec(ki_c, kv)
        for b, j in written:
            assert_close(gk[b, j], o_kc[b, j], *BAR_BF16, what="k_c step %d" % step)
            assert_close(gx[b, j], o_xc[b, j], *BAR_BF16, what="ki_c step %d" % step)
        # the next calls, and the oracle, read the GPU's caches (same inputs)
        o_kc, o_vc, o_xc = gk, dec(v_c, kv), gx
        q_i = torch.randn((B, 1, H_i, d_i), generator=g, device=DEV).to(dt)
        w_i = torch.randn((B, 1, H_i), generator=g, device=DEV) / H_i ** 0.5
        idx = csa.index_topk_varlen(q_i, w_i, ki_c, k, pos_t, q_pos_max, m, idx_fmt)
        q = torch.randn((B, 1, H, D), generator=g, device=DEV).to(dt)
        out, lse = csa.sparse_attn_varlen(q, k_c, v_c, idx, k_ring, v_ring, W, sink, pos_t, q_pos_max)
        torch.cuda.synchronize()
        sc = oidx.index_scores_batch(dec(q_i, kv), dec(w_i, "f32"), o_xc, pos, m)
        gi = idx.cpu().numpy()
        for b in range(B):
            n = (pos[b] + 1) // m
            topk_matches_up_to_ties(gi[b, 0], sc[b, 0, :n], k)
        eo, el = oatt.csa_sparse_attn(dec(q, kv), pos, o_kc, o_vc, gi, o_kr, o_vr, 0, W, dec(sink, "f32"), ring=True)
        assert_close(dec(out, kv), eo, *BAR_BF16, what="out step %d" % step)
        assert_close(lse.cpu().numpy(), el, 5e-3, 1e-3, what="lse step %d" % step)
