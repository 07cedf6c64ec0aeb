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
