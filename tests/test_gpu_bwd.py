"""GPU parity of the attention backward (csa_sparse_attn_bwd,
hca_dense_attn_bwd) against the fp64 oracle's gradients, through the C ABI:
the GPU forward's out and lse feed the GPU backward, the oracle recomputes
everything from the same decoded inputs. Also: bitwise determinism across
calls and batch invariance (a sequence alone and inside a batch)."""
import numpy as np
import pytest
import torch

import long_context_attention_16_amd as csa
from oracle import attention_bwd as obwd
from helpers import dec

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _gen(seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


def _inputs(fmt, B, Lq, H, D, N_cap, T_raw, seed):
    g = _gen(seed)
    dt = torch.float32 if fmt == "f32" else torch.bfloat16
    r = lambda *s: torch.randn(s, generator=g, device=DEV).to(dt)
    return dict(q=r(B, Lq, H, D), k_c=r(B, N_cap, D), v_c=r(B, N_cap, D), k_raw=r(B, T_raw, D),
                v_raw=r(B, T_raw, D), sink=torch.randn((H,), generator=g, device=DEV), dout=r(B, Lq, H, D))


def _idx(B, Lq, k, q_pos0, m, N_cap, seed):
    rng = np.random.default_rng(seed)
    idx = np.full((B, Lq, k), -1, dtype=np.int32)
    for b in range(B):
        for i in range(Lq):
            n = min(N_cap, (q_pos0 + i + 1) // m)
            take = min(n, int(rng.integers(max(1, k // 2), k + 1)))
            idx[b, i, :take] = np.sort(rng.choice(n, size=take, replace=False))
    return idx


def _close(got, want, rel, rel_mean, what):
    """Two bars: the largest error against the largest gradient (max-abs <=
    rel x max|ref|), and the mean error against the mean gradient (mean-abs
    <= rel_mean x mean|ref|), which a small error repeated over every entry
    (a dropped factor, a biased sum) does not pass."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    scale = max(1e-6, float(np.abs(want).max()))
    diff = np.abs(got - want)
    err = float(diff.max())
    assert err <= rel * scale, "%s: max-abs %.3g > %.3g x max|ref| %.3g" % (what, err, rel, scale)
    mscale = float(np.abs(want).mean())
    if mscale > 0:
        merr = float(diff.mean())
        print("%s: max-abs/max|ref| %.3g, mean-abs/mean|ref| %.3g" % (what, err / scale, merr / mscale))
        assert merr <= rel_mean * mscale, "%s: mean-abs %.3g > %.3g x mean|ref| %.3g (ratio %.3g)" % (
            what, merr, rel_mean, mscale, merr / mscale)


def _check(fmt, g, want):
    rel, rel_mean = (2e-2, 8e-3) if fmt == "bf16" else (2e-4, 5e-6)
    for name, a, b in zip(["dq", "dk_c", "dv_c", "dk_raw", "dv_raw", "dsink"], g, want):
        if a is None:
            continue
        _close(a.cpu().numpy(), b, rel, rel_mean, name)


@pytest.mark.parametrize("fmt,B,Lq,H,D,k,W,q_pos0,sink", [
    ("f32", 1, 9, 4, 128, 64, 16, 300, True),     # prefill rows sharing entries and window rows
    ("f32", 2, 3, 8, 512, 40, 7, 100, False),     # no sink
    ("bf16", 2, 1, 64, 512, 512, 128, 5000, True),  # decode head layout
    ("bf16", 1, 5, 16, 128, 24, 20, 10, True),    # windows cut at position 0, few entries
    ("f32", 1, 4, 4, 128, 16, 0, 200, True),      # no window
    ("bf16", 2, 3, 20, 128, 100, 40, 700, True),  # two 16-head groups (the second padded), tiles across the window
    ("bf16", 1, 7, 4, 128, 64, 128, 3000, True),  # the prefill head layout
])
def test_sparse_attn_bwd(fmt, B, Lq, H, D, k, W, q_pos0, sink):
    m = 4
    N_cap = (q_pos0 + Lq) // m + 3
    raw_pos0 = max(0, q_pos0 - W - 2)
    T_raw = q_pos0 + Lq - raw_pos0 + 1
    x = _inputs(fmt, B, Lq, H, D, N_cap, T_raw, seed=H + D + k)
    idx = _idx(B, Lq, k, q_pos0, m, N_cap, seed=k + Lq)
    it = torch.from_numpy(idx).to(DEV)
    s = x["sink"] if sink else None
    out, lse = csa.sparse_attn(x["q"], x["k_c"], x["v_c"], it, x["k_raw"], x["v_raw"], raw_pos0, W, s, q_pos0)
    g = csa.sparse_attn_bwd(x["q"], x["k_c"], x["v_c"], it, x["k_raw"], x["v_raw"], raw_pos0, W, s, q_pos0, out, lse,
                            x["dout"])
    torch.cuda.synchronize()
    want = obwd.csa_sparse_attn_bwd(dec(x["q"], fmt), q_pos0, dec(x["k_c"], fmt), dec(x["v_c"], fmt), idx,
                                    dec(x["k_raw"], fmt), dec(x["v_raw"], fmt), raw_pos0, W,
                                    None if s is None else dec(s, "f32"), dec(x["dout"], fmt))
    _check(fmt, g, want)


@pytest.mark.parametrize("fmt,B,Lq,H,D,m,q_pos0,W", [
    ("bf16", 1, 1, 16, 512, 128, 70000, 128),
    ("f32", 1, 6, 4, 128, 4, 250, 16),            # prefill rows with ragged n(t)
    ("bf16", 2, 5, 4, 128, 4, 130, 24),           # bf16 D = 128: the MFMA query pass
])
def test_hca_attn_bwd(fmt, B, Lq, H, D, m, q_pos0, W):
    N_cap = (q_pos0 + Lq) // m + 1
    raw_pos0 = max(0, q_pos0 - W + 1)
    T_raw = q_pos0 + Lq - raw_pos0
    x = _inputs(fmt, B, Lq, H, D, N_cap, T_raw, seed=D + m)
    out, lse = csa.hca_attn(x["q"], x["k_c"], x["v_c"], m, x["k_raw"], x["v_raw"], raw_pos0, W, x["sink"], q_pos0)
    g = csa.hca_attn_bwd(x["q"], x["k_c"], x["v_c"], m, x["k_raw"], x["v_raw"], raw_pos0, W, x["sink"], q_pos0, out,
                         lse, x["dout"])
    torch.cuda.synchronize()
    want = obwd.hca_dense_attn_bwd(dec(x["q"], fmt), q_pos0, m, dec(x["k_c"], fmt), dec(x["v_c"], fmt),
                                   dec(x["k_raw"], fmt), dec(x["v_raw"], fmt), raw_pos0, W, dec(x["sink"], "f32"),
                                   dec(x["dout"], fmt))
    _check(fmt, g, want)


def test_bwd_deterministic_and_batch_invariant():
    """Two calls give the same bits; sequence 0 alone gives the same bits as
    inside the batch (its rows get contributions from its own queries only,
    added exactly)."""
    fmt, B, Lq, H, D, k, W, q_pos0, m = "bf16", 3, 6, 8, 128, 48, 16, 400, 4
    N_cap = (q_pos0 + Lq) // m + 1
    raw_pos0 = q_pos0 - W
    T_raw = q_pos0 + Lq - raw_pos0
    x = _inputs(fmt, B, Lq, H, D, N_cap, T_raw, seed=9)
    it = torch.from_numpy(_idx(B, Lq, k, q_pos0, m, N_cap, seed=3)).to(DEV)
    out, lse = csa.sparse_attn(x["q"], x["k_c"], x["v_c"], it, x["k_raw"], x["v_raw"], raw_pos0, W, x["sink"], q_pos0)
    args = (x["q"], x["k_c"], x["v_c"], it, x["k_raw"], x["v_raw"], raw_pos0, W, x["sink"], q_pos0, out, lse, x["dout"])
    g1 = csa.sparse_attn_bwd(*args)
    g2 = csa.sparse_attn_bwd(*args)
    one = lambda t: t[:1].contiguous()
    o1, l1 = csa.sparse_attn(one(x["q"]), one(x["k_c"]), one(x["v_c"]), one(it), one(x["k_raw"]), one(x["v_raw"]),
                             raw_pos0, W, x["sink"], q_pos0)
    g3 = csa.sparse_attn_bwd(one(x["q"]), one(x["k_c"]), one(x["v_c"]), one(it), one(x["k_raw"]), one(x["v_raw"]),
                             raw_pos0, W, x["sink"], q_pos0, o1, l1, one(x["dout"]))
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    for a, b in zip(g1[:5], g3[:5]):
        assert torch.equal(a[:1], b)


def test_sparse_attn_bwd_hot_entry_and_duplicates():
    """Entries 0 and 1 selected by every one of 1100 queries (more pairs than
    the key/value pass stages at once), and queries that list an entry twice
    (two slots, two contributions)."""
    fmt, B, Lq, H, D, k, W, q_pos0, m = "f32", 1, 1100, 4, 128, 6, 4, 64, 4
    N_cap = (q_pos0 + Lq) // m + 1
    raw_pos0 = q_pos0 - W
    T_raw = q_pos0 + Lq - raw_pos0
    x = _inputs(fmt, B, Lq, H, D, N_cap, T_raw, seed=5)
    rng = np.random.default_rng(12)
    idx = np.full((B, Lq, k), -1, dtype=np.int32)
    for i in range(Lq):
        n = (q_pos0 + i + 1) // m
        idx[0, i, :2] = [0, 1]
        idx[0, i, 2:5] = rng.choice(np.arange(2, n), size=3, replace=False)
        idx[0, i, 5] = idx[0, i, 2] if i % 7 == 0 else -1
    it = torch.from_numpy(idx).to(DEV)
    out, lse = csa.sparse_attn(x["q"], x["k_c"], x["v_c"], it, x["k_raw"], x["v_raw"], raw_pos0, W, x["sink"], q_pos0)
    g = csa.sparse_attn_bwd(x["q"], x["k_c"], x["v_c"], it, x["k_raw"], x["v_raw"], raw_pos0, W, x["sink"], q_pos0,
                            out, lse, x["dout"])
    torch.cuda.synchronize()
    want = obwd.csa_sparse_attn_bwd(dec(x["q"], fmt), q_pos0, dec(x["k_c"], fmt), dec(x["v_c"], fmt), idx,
                                    dec(x["k_raw"], fmt), dec(x["v_raw"], fmt), raw_pos0, W, dec(x["sink"], "f32"),
                                    dec(x["dout"], fmt))
    _check(fmt, g, want)


@pytest.mark.parametrize("fmt", ["f32", "bf16"])
def test_sparse_attn_bwd_list_beyond_lds(fmt):
    """Entry 3 listed in 30 slots of each of 300 queries: 9000 (query, slot)
    pairs, more than the key/value pass sorts in LDS, so that entry is summed
    in 64-bit fixed point; the other entries in float32 in sorted order."""
    B, Lq, H, D, k, W, q_pos0, m = 1, 300, 4, 128, 40, 16, 100, 4
    N_cap = (q_pos0 + Lq) // m + 1
    raw_pos0 = q_pos0 - W
    T_raw = q_pos0 + Lq - raw_pos0
    x = _inputs(fmt, B, Lq, H, D, N_cap, T_raw, seed=21)
    rng = np.random.default_rng(4)
    idx = np.full((B, Lq, k), 3, dtype=np.int32)
    for i in range(Lq):
        n = (q_pos0 + i + 1) // m
        idx[0, i, 30:] = rng.choice(np.arange(4, n), size=k - 30, replace=False)
    it = torch.from_numpy(idx).to(DEV)
    out, lse = csa.sparse_attn(x["q"], x["k_c"], x["v_c"], it, x["k_raw"], x["v_raw"], raw_pos0, W, x["sink"], q_pos0)
    args = (x["q"], x["k_c"], x["v_c"], it, x["k_raw"], x["v_raw"], raw_pos0, W, x["sink"], q_pos0, out, lse,
            x["dout"])
    g = csa.sparse_attn_bwd(*args)
    g2 = csa.sparse_attn_bwd(*args)
    torch.cuda.synchronize()
    want = obwd.csa_sparse_attn_bwd(dec(x["q"], fmt), q_pos0, dec(x["k_c"], fmt), dec(x["v_c"], fmt), idx,
                                    dec(x["k_raw"], fmt), dec(x["v_raw"], fmt), raw_pos0, W, dec(x["sink"], "f32"),
                                    dec(x["dout"], fmt))
    _check(fmt, g, want)
    for a, b in zip(g, g2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("hca", [False, True])
def test_attn_bwd_no_query_rows(hca):
    """Lq = 0: no query contributes, so every key/value gradient row and the
    sink gradient are zero (the outputs are written, not left as they were)."""
    import ctypes
    B, H, D, N_cap, T_raw, W, k = 2, 4, 128, 16, 8, 8, 8
    x = _inputs("bf16", B, 1, H, D, N_cap, T_raw, seed=3)  # q, out, dout: one row each, never read
    idx = torch.zeros((B, 1, k), dtype=torch.int32, device=DEV)
    lse = torch.zeros((B, 1, H), device=DEV)
    f = dict(device=DEV, dtype=torch.float32)
    dq = torch.full((B, 1, H, D), 5.0, **f)
    dkc, dvc = torch.full((B, N_cap, D), 5.0, **f), torch.full((B, N_cap, D), 5.0, **f)
    dkr, dvr = torch.full((B, T_raw, D), 5.0, **f), torch.full((B, T_raw, D), 5.0, **f)
    dsink = torch.full((H,), 5.0, **f)
    q_pos0, m = 60, 4
    lib = csa.lib()
    nb = csa.attn_bwd_ws_bytes(B, 0, q_pos0, m if hca else 0, H, D, N_cap, 0 if hca else k, W)
    ws = torch.empty(max(16, nb) // 4 + 4, **f)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    common = [P(x["q"]), N_cap, P(x["k_c"]), P(x["v_c"])]
    tail = [T_raw, q_pos0 - T_raw + 1, P(x["k_raw"]), P(x["v_raw"]), W, P(x["sink"]), P(x["dout"]), P(lse),
            P(x["dout"]), P(dq), P(dkc), P(dvc), P(dkr), P(dvr), P(dsink), P(ws), ws.numel() * 4, st]
    if hca:
        rc = lib.hca_dense_attn_bwd(B, 0, q_pos0, m, H, D, 1, *common, *tail)
    else:
        rc = lib.csa_sparse_attn_bwd(B, 0, q_pos0, H, D, 1, *common, k, P(idx), *tail)
    torch.cuda.synchronize()
    assert rc == 0
    for name, t in (("dk_c", dkc), ("dv_c", dvc), ("dk_raw", dkr), ("dv_raw", dvr), ("dsink", dsink)):
        assert torch.all(t == 0), name
