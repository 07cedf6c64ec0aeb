"""Determinism and batch invariance of every call on the GPU: the same
inputs give the same bits on every call, and a sequence's results do not
depend on the rest of the batch ("DeepSeek V4 重磅開源！…" (InfoQ), section
確定性內核: a token's output must not depend on its position in the batch).
Attention (forward and backward) is covered beside its parity tests; this file
covers the indexer top-k (fused and score paths, f32 and bf16 scores), the
HCA attention and the state-cache append."""
import pytest
import torch

import long_context_attention_16_amd as csa
from long_context_attention_16_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _gen(seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


def _slice(t, b):
    return None if t is None else t[b:b + 1].contiguous()


@pytest.mark.parametrize("fmt,H_i,d_i,Lq,q_pos0,topk,score", [
    ("bf16", 64, 128, 1, 4 * 9000 - 1, 512, "f32"),     # fused: 5 chunks of 2048 and the merge
    ("fp4", 64, 128, 1, 4 * 70000 - 1, 1024, "f32"),    # fused: 18 chunks of 4096, two merge levels
    ("fp4", 64, 128, 1, 4 * 70000 - 1, 2048, "f32"),    # k above 1024: score path, chunked top-k and merge
    ("fp8", 4, 32, 37, 20000, 300, "f32"),              # many query rows, the score path
    ("fp8", 64, 128, 20, 20000, 256, "bf16"),           # the many-query fp8 kernel, bf16 scores
    ("bf16", 64, 128, 1, 4 * 9000 - 1, 512, "bf16"),    # fused, bf16 scores
])
def test_index_topk_deterministic_and_batch_invariant(fmt, H_i, d_i, Lq, q_pos0, topk, score):
    B, m = 4, 4
    N_cap = (q_pos0 + Lq) // m + 5
    s = wl.small_shape(B=B, Lq=Lq, H_I=H_i, d_I=d_i, N_cap=N_cap, idx=fmt, exact=False)
    x = wl.indexer_inputs(s, _gen(H_i + d_i + Lq), DEV)
    args = (x["q_i"], x["w_i"], x["k_i"], topk, q_pos0, m, fmt)
    kw = dict(score_dtype=score, q_scale=x["q_i_scale"], k_scale=x["k_i_scale"])
    a = csa.index_topk_ex(*args, **kw)
    b = csa.index_topk_ex(*args, **kw)
    one = csa.index_topk_ex(_slice(x["q_i"], 2), _slice(x["w_i"], 2), _slice(x["k_i"], 2), topk, q_pos0, m, fmt,
                            score_dtype=score, q_scale=_slice(x["q_i_scale"], 2),
                            k_scale=_slice(x["k_i_scale"], 2))
    sa = csa.index_scores_ex(x["q_i"], x["w_i"], x["k_i"], q_pos0, m, fmt, score_dtype=score,
                             q_scale=x["q_i_scale"], k_scale=x["k_i_scale"])
    sb = csa.index_scores_ex(x["q_i"], x["w_i"], x["k_i"], q_pos0, m, fmt, score_dtype=score,
                             q_scale=x["q_i_scale"], k_scale=x["k_i_scale"])
    torch.cuda.synchronize()
    assert torch.equal(a, b), "two calls select differently"
    assert torch.equal(a[2:3], one), "a sequence alone selects differently from inside the batch"
    assert torch.equal(sa.view(torch.int16) if score == "bf16" else sa.view(torch.int32),
                       sb.view(torch.int16) if score == "bf16" else sb.view(torch.int32))


@pytest.mark.parametrize("B,H,D,m,q_pos0,W", [
    (4, 64, 512, 128, 300000, 128),
    (3, 4, 128, 4, 5000, 16),
    # 1M context, 16 splits per row, a batch of 40 against a sequence alone
    (40, 64, 512, 128, 1048575, 128),
])
def test_hca_deterministic_and_batch_invariant(B, H, D, m, q_pos0, W):
    g = _gen(B + H + m)
    N_cap = (q_pos0 + 1) // m + 1
    raw_pos0 = q_pos0 - W + 1
    r = lambda *sh: torch.randn(sh, generator=g, device=DEV).to(torch.bfloat16)
    q, kc, vc, kr, vr = r(B, 1, H, D), r(B, N_cap, D), r(B, N_cap, D), r(B, W, D), r(B, W, D)
    sink = torch.randn((H,), generator=g, device=DEV)
    a, la = csa.hca_attn(q, kc, vc, m, kr, vr, raw_pos0, W, sink, q_pos0)
    b, lb = csa.hca_attn(q, kc, vc, m, kr, vr, raw_pos0, W, sink, q_pos0)
    one, lo = csa.hca_attn(_slice(q, 1), _slice(kc, 1), _slice(vc, 1), m, _slice(kr, 1), _slice(vr, 1), raw_pos0, W,
                           sink, q_pos0)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)) and torch.equal(la, lb)
    assert torch.equal(a[1:2].view(torch.int16), one.view(torch.int16)) and torch.equal(la[1:2], lo)


@pytest.mark.parametrize("idx_fmt", ["fp4", "fp8"])
def test_state_append_deterministic_and_batch_invariant(idx_fmt):
    g = _gen(31)
    B, D, m, R, N_cap, d_i = 5, 512, 4, 132, 40, 128
    dt = torch.bfloat16
    pos = torch.tensor([4 * 9 - 1, 4 * 9 + 1, -1, 4 * 20 - 1, 3], dtype=torch.int64, device=DEV)
    k_new, v_new, ki_new = (torch.randn((B, n), generator=g, device=DEV).to(dt) for n in (D, D, d_i))
    w = (torch.randn((D,), generator=g, device=DEV) / D ** 0.5).contiguous()
    rings = [torch.randn((B, R, n), generator=g, device=DEV).to(dt) for n in (D, D, d_i)]
    fp4 = idx_fmt == "fp4"

    def state():
        kc = torch.zeros((B, N_cap, D), device=DEV).to(dt)
        ki = torch.zeros((B, N_cap, d_i // 2 if fp4 else d_i), dtype=torch.uint8, device=DEV)
        sc = torch.zeros((B, N_cap, d_i // 32), dtype=torch.uint8, device=DEV) if fp4 else None
        return [r.clone() for r in rings] + [kc, kc.clone(), ki, sc]

    def run(st, sl=None):
        f = (lambda t: t) if sl is None else (lambda t: _slice(t, sl))
        st = [None if t is None else f(t) for t in st]
        kr, vr, xr, kc, vc, ki, sc = st
        csa.state_append(f(pos), f(k_new), f(v_new), w, m, kr, vr, kc, vc, f(ki_new), xr, ki, sc, idx_fmt)
        return st

    a, b = run(state()), run(state())
    one = run(state(), 3)
    torch.cuda.synchronize()
    for ta, tb, t1 in zip(a, b, one):
        if ta is None:
            continue
        ua, ub, u1 = (t.view(torch.uint8) for t in (ta, tb, t1))
        assert torch.equal(ua, ub), "two appends differ"
        assert torch.equal(ua[3:4], u1), "a sequence alone differs from inside the batch"
