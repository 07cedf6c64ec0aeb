"""Test helpers: decode device tensors for the oracle and compare results."""
import numpy as np
import torch

from oracle import formats


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
