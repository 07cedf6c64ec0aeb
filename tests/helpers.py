"""Test helpers: decode device tensors for the oracle and compare results."""
import numpy as np
import torch

from oracle import formats
from oracle import formats as ofmt


def dec(t, fmt, scale=None):
    """Exact float64 value of a storage tensor (any device) for the oracle."""
    t = t.detach().cpu().contiguous()
    if fmt == "f32":
        return t.numpy().astype(np.float64)
    if fmt == "bf16":
        return formats.bf16_to_f64(t.view(torch.int16).numpy().view(np.uint16))
    if fmt == "fp8":
        return formats.e4m3fn_to_f64(t.numpy())
    if fmt == "fp4":
        return formats.mxfp4_to_f64(t.numpy(), scale.detach().cpu().numpy())
    raise ValueError(fmt)


def kv_fmt(t):
    return "bf16" if t.dtype == torch.bfloat16 else "f32"


def assert_close(got, want, max_abs, mean_abs, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.all(np.isfinite(got) == np.isfinite(want)), what + ": finiteness differs"
    fin = np.isfinite(want)
    if not np.array_equal(got[~fin], want[~fin]):
        raise AssertionError(what + ": non-finite values differ")
    err = np.abs(got[fin] - want[fin])
    if err.size == 0:
        return
    mx, mn = float(err.max()), float(err.mean())
    assert mx <= max_abs and mn <= mean_abs, "%s: max-abs %.3g (bar %.3g), mean-abs %.3g (bar %.3g)" % (
        what, mx, max_abs, mn, mean_abs)


def topk_matches_up_to_ties(gpu_idx, scores, k, rtol=1e-5):
    """For non-integer scores: GPU and exact top-k may differ only among entries
    whose exact scores are within rtol of the k-th largest. Returns the number of
    differing slots; raises if any difference is not such a near-tie."""
    gpu_idx = np.asarray(gpu_idx)
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[0]
    take = min(k, n)
    sel = gpu_idx[gpu_idx >= 0]
    assert len(sel) == take and np.all(np.diff(sel) > 0) and np.all(gpu_idx[take:] == -1)
    if take == n:
        assert np.array_equal(sel, np.arange(n))
        return 0
    thr = np.sort(s)[::-1][take - 1]
    tol = rtol * max(1.0, abs(thr))
    exact = set(np.argsort(-s, kind="stable")[:take].tolist())
    diff = set(sel.tolist()) ^ exact
    for j in diff:
        assert abs(s[j] - thr) <= tol, "top-k differs at j=%d beyond a near-tie (%.9g vs %.9g)" % (j, s[j], thr)
    return len(diff)


def ki_alloc(B, N_cap, d_i, idx_fmt, DEV="cuda"):
    """Compressed indexer-key buffers (and MXFP4 scales) filled with a marker."""
    if idx_fmt == "f32":
        return torch.full((B, N_cap, d_i), 7.0, device=DEV), None
    if idx_fmt == "bf16":
        return torch.full((B, N_cap, d_i), 7.0, device=DEV).to(torch.bfloat16), None
    if idx_fmt == "fp8":
        return torch.full((B, N_cap, d_i), 0x77, dtype=torch.uint8, device=DEV), None
    return (torch.full((B, N_cap, d_i // 2), 0x77, dtype=torch.uint8, device=DEV),
            torch.full((B, N_cap, d_i // 32), 0x77, dtype=torch.uint8, device=DEV))


def codes_ok(got_codes, x, enc, eps=1e-4):
    """Every GPU code equals the oracle's encoding of x or, where x lies
    within a relative eps of a rounding boundary, of x scaled by 1 +- eps
    (the f32 fold and the fp64 oracle may land on either side)."""
    got = np.asarray(got_codes).astype(np.int64)
    ok = np.zeros(got.shape, dtype=bool)
    for f in (1.0, 1.0 - eps, 1.0 + eps):
        ok |= got == enc(x * f).astype(np.int64)
    return ok


def check_ki(ki_c, ki_sc, want, idx_fmt, kv_fmt, rows, exact=False):
    """Compare the written indexer-key rows [(b, j)] with the oracle fold.
    exact: the fold is exact on the GPU too (m = 1: the row itself), so every
    code must be the oracle's encoding of it, bit for bit."""
    if idx_fmt == "f32":
        got = dec(ki_c, idx_fmt)
        for b, j in rows:
            assert_close(got[b, j], want[b, j], 1e-4, 1e-5, what="ki_c")
        return
    if idx_fmt == "bf16":
        # a stored rounding: each bf16 code is the oracle's nearest-even code
        # (within the rounding-boundary rule of codes_ok)
        got = ki_c.detach().cpu().view(torch.int16).numpy().view(np.uint16)
        eps = 0.0 if exact else 1e-3 if kv_fmt == "bf16" else 1e-4
        for b, j in rows:
            ok = codes_ok(got[b, j], want[b, j], ofmt.f64_to_bf16, eps=eps)
            assert ok.all(), "bf16 indexer key codes differ at b=%d j=%d" % (b, j)
        return
    if idx_fmt == "fp8":
        got = ki_c.cpu().numpy()
        for b, j in rows:
            eps = 0.0 if exact else 1e-3 if kv_fmt == "bf16" else 1e-4
            ok = codes_ok(got[b, j], want[b, j], ofmt.f64_to_e4m3fn, eps=eps)
            assert ok.all(), "fp8 indexer key codes differ at b=%d j=%d" % (b, j)
        return
    packed, sc = ki_c.cpu().numpy(), ki_sc.cpu().numpy()
    eps = 0.0 if exact else 1e-3 if kv_fmt == "bf16" else 1e-4
    for b, j in rows:
        x = want[b, j]
        codes = ofmt.unpack_fp4(packed[b, j])
        for blk in range(x.shape[0] // 32):
            xb = x[32 * blk:32 * blk + 32]
            cands = {int(ofmt.f64_to_mxfp4(xb * f)[1][0]) for f in (1.0, 1.0 - eps, 1.0 + eps)}
            s = int(sc[b, j, blk])
            assert s in cands, "fp4 scale differs at b=%d j=%d block %d" % (b, j, blk)
            X = 2.0 ** (s - 127)
            ok = codes_ok(codes[32 * blk:32 * blk + 32], xb / X, ofmt.f64_to_e2m1, eps)
            assert ok.all(), "fp4 element codes differ at b=%d j=%d block %d" % (b, j, blk)
