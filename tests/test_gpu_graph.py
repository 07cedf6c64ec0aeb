"""The decode step captured in a HIP graph (as bench.py times it) gives the
eager results on every replay, with eager work between the replays."""
from dataclasses import replace

import pytest
import torch

import long_context_attention_16_amd as csa
from long_context_attention_16_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _buffers(s, x):
    x["scores"] = torch.empty((s.B, s.Lq, s.N_cap), dtype=torch.float32, device=DEV)
    x["idx"] = torch.empty((s.B, s.Lq, s.topk), dtype=torch.int32, device=DEV)
    tb = csa.topk_ws_bytes(s.B, s.Lq, s.q_pos0, s.m, s.topk)
    x["topk_ws"] = torch.empty((tb + 15) // 16 * 4, dtype=torch.float32, device=DEV)
    ab = csa.sparse_attn_ws_bytes(s.B, s.Lq, s.H, s.D, s.topk, s.W)
    x["ws"] = torch.empty((ab + 15) // 16 * 4, dtype=torch.float32, device=DEV)
    x["out"] = torch.empty_like(x["q"])
    x["lse"] = torch.empty((s.B, s.Lq, s.H), dtype=torch.float32, device=DEV)


def _step(s, x):
    csa.index_scores(x["q_i"], x["w_i"], x["k_i"], s.q_pos0, s.m, s.idx, x["q_i_scale"], x["k_i_scale"],
                     out=x["scores"])
    csa.topk(x["scores"], s.topk, s.q_pos0, s.m, out=x["idx"], ws=x["topk_ws"])
    csa.sparse_attn(x["q"], x["k_c"], x["v_c"], x["idx"], x["k_raw"], x["v_raw"], s.raw_pos0, s.W, x["sink"],
                    s.q_pos0, ws=x["ws"], out=x["out"], lse=x["lse"])


@pytest.mark.parametrize("shape", [replace(wl.CFG2, B=4), replace(wl.CFG5_CSA, B=2)], ids=["128k", "1m_fp4"])
def test_csa_decode_graph_replays(shape):
    s = shape
    x = wl.make_inputs(s, 11, DEV)
    _buffers(s, x)
    _step(s, x)
    torch.cuda.synchronize()
    ref_idx, ref_out, ref_lse = x["idx"].clone(), x["out"].clone(), x["lse"].clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(s, x)
    for r in range(4):
        x["idx"].fill_(-7)
        x["out"].zero_()
        x["lse"].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(x["idx"], ref_idx), r
        assert torch.equal(x["out"].view(torch.int16), ref_out.view(torch.int16)), r
        assert torch.equal(x["lse"], ref_lse), r


def test_hca_graph_replays():
    s = replace(wl.CFG4, B=2)
    x = wl.make_inputs(s, 12, DEV)
    nb = csa.hca_attn_ws_bytes(s.B, s.Lq, s.q_pos0, s.m, s.H, s.D, s.W)
    ws = torch.empty((nb + 15) // 16 * 4, dtype=torch.float32, device=DEV)
    out = torch.empty_like(x["q"])
    lse = torch.empty((s.B, s.Lq, s.H), dtype=torch.float32, device=DEV)

    def run():
        csa.hca_attn(x["q"], x["k_c"], x["v_c"], s.m, x["k_raw"], x["v_raw"], s.raw_pos0, s.W, x["sink"],
                     s.q_pos0, ws=ws, out=out, lse=lse)

    run()
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for r in range(4):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), r


def test_attn_bwd_graph_replays():
    """The attention backward captured in a HIP graph (its counters and lists
    are cleared by its own kernels, no memsets) gives the eager bits on every
    replay, with its workspace overwritten and eager work between replays."""
    import numpy as np
    B, Lq, H, D, k, W, q_pos0, m = 2, 64, 4, 128, 64, 16, 500, 4
    N_cap = (q_pos0 + Lq) // m + 1
    raw_pos0 = q_pos0 - W
    T_raw = q_pos0 + Lq - raw_pos0
    gen = torch.Generator(device=DEV)
    gen.manual_seed(5)
    r = lambda *shape: torch.randn(shape, generator=gen, device=DEV).to(torch.bfloat16)
    q, k_c, v_c, k_raw, v_raw, dout = r(B, Lq, H, D), r(B, N_cap, D), r(B, N_cap, D), r(B, T_raw, D), \
        r(B, T_raw, D), r(B, Lq, H, D)
    sink = torch.randn((H,), generator=gen, device=DEV)
    rng = np.random.default_rng(2)
    idx = np.full((B, Lq, k), -1, dtype=np.int32)
    for b in range(B):
        for i in range(Lq):
            n = (q_pos0 + i + 1) // m
            idx[b, i] = np.sort(rng.choice(n, size=k, replace=False))
    it = torch.from_numpy(idx).to(DEV)
    out, lse = csa.sparse_attn(q, k_c, v_c, it, k_raw, v_raw, raw_pos0, W, sink, q_pos0)
    nb = csa.attn_bwd_ws_bytes(B, Lq, q_pos0, 0, H, D, N_cap, k, W)
    ws = torch.empty((nb + 15) // 16 * 4, dtype=torch.float32, device=DEV)
    args = (q, k_c, v_c, it, k_raw, v_raw, raw_pos0, W, sink, q_pos0, out, lse, dout)
    ref = [t.clone() for t in csa.sparse_attn_bwd(*args, ws=ws)]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        got = csa.sparse_attn_bwd(*args, ws=ws)
    for rep in range(3):
        for t in got:
            t.fill_(7.0)
        ws.fill_(3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a, b), rep
