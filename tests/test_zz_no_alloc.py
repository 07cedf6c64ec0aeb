"""csa_sparse_attn_noalloc through the C ABI: the same bits as
csa_sparse_attn on two calls in a row (the second smaller, so it runs on what
the first left in the shared scratch), on the two-launch decode kernel and on
the general split kernel; sizes beyond the fixed scratch are refused before
anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import long_context_attention_16_amd as csa

pytestmark = pytest.mark.gpu
DEV = "cuda"
WS_ERR = 5


def _inputs(dt, B, Lq, H, D, N_cap, T_raw, k, q_pos0, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    r = lambda *s: torch.randn(s, generator=g, device=DEV).to(dt)
    rng = np.random.default_rng(seed)
    idx = np.full((B, Lq, k), -1, dtype=np.int32)
    for b in range(B):
        for i in range(Lq):
            n = min(N_cap, (q_pos0 + i + 1) // 4)
            take = min(n, k - (b + i) % 3)
            idx[b, i, :take] = np.sort(rng.choice(n, size=take, replace=False))
    return dict(q=r(B, Lq, H, D), k_c=r(B, N_cap, D), v_c=r(B, N_cap, D), k_raw=r(B, T_raw, D),
                v_raw=r(B, T_raw, D), sink=torch.randn((H,), generator=g, device=DEV),
                idx=torch.from_numpy(idx).to(DEV))


def _noalloc(x, q_pos0, raw_pos0, W):
    B, Lq, H, D = x["q"].shape
    out = torch.full_like(x["q"], float("nan"))
    lse = torch.full((B, Lq, H), float("nan"), device=DEV)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = csa.lib().csa_sparse_attn_noalloc(
        B, Lq, q_pos0, H, D, 0 if x["q"].dtype == torch.float32 else 1, P(x["q"]), x["k_c"].shape[1], P(x["k_c"]),
        P(x["v_c"]), x["idx"].shape[-1], P(x["idx"]), x["k_raw"].shape[1], raw_pos0, P(x["k_raw"]), P(x["v_raw"]),
        W, P(x["sink"]), P(out), P(lse), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, csa.lib().csa_strerror(rc)
    return out, lse


@pytest.mark.parametrize("dt,H,D", [(torch.bfloat16, 64, 512), (torch.bfloat16, 4, 128), (torch.float32, 8, 512)])
def test_noalloc_matches_workspace_call(dt, H, D):
    for B, Lq, k, W, q_pos0, seed in ((6, 2, 512, 128, 40000, 1), (3, 1, 200, 64, 9000, 2)):
        N_cap = (q_pos0 + Lq) // 4 + 3
        raw_pos0 = q_pos0 - W - 1
        T_raw = q_pos0 + Lq - raw_pos0
        x = _inputs(dt, B, Lq, H, D, N_cap, T_raw, k, q_pos0, seed + H)
        want, wlse = csa.sparse_attn(x["q"], x["k_c"], x["v_c"], x["idx"], x["k_raw"], x["v_raw"], raw_pos0, W,
                                     x["sink"], q_pos0)
        got, glse = _noalloc(x, q_pos0, raw_pos0, W)
        torch.cuda.synchronize()
        iv = torch.int16 if dt == torch.bfloat16 else torch.int32
        assert torch.equal(got.view(iv), want.view(iv)), "outputs differ (B=%d)" % B
        assert torch.equal(glse, wlse)


def test_noalloc_refuses_beyond_scratch():
    B, Lq, H, D, k, W = 64, 64, 128, 512, 2048, 256
    assert csa.sparse_attn_ws_bytes(B, Lq, H, D, k, W) > (32 << 20)
    P = ctypes.c_void_p(0x10000)   # never dereferenced: the call returns before any launch
    rc = csa.lib().csa_sparse_attn_noalloc(B, Lq, 100000, H, D, 0, P, 30000, P, P, k, P, W + Lq, 100000 - W,
                                           P, P, W, P, P, P, None)
    assert rc == WS_ERR
