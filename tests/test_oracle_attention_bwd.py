"""Pins of the attention backward oracle: central finite differences of the
forward oracle (attention.py, itself pinned) for every input, with and
without a sink, for CSA (entries shared between queries) and HCA; and the
closed form sum_r dV_r = sum_h (1 - Pz_h) dO_h of a single query."""
import numpy as np
import pytest

from oracle import attention as oatt
from oracle import attention_bwd as obwd


def _loss(fwd, args, dout):
    out, _ = fwd(*args)
    return float((out * dout).sum())


def _check_fd(fwd, args, names, grads, dout, rng, n_coords=12, h=1e-6, tol=2e-6):
    for name, g in zip(names, grads):
        arr = args_by_name(args, name)
        flat = arr.reshape(-1)
        for c in rng.choice(flat.size, size=min(n_coords, flat.size), replace=False):
            keep = flat[c]
            flat[c] = keep + h
            lp = _loss(fwd, args, dout)
            flat[c] = keep - h
            lm = _loss(fwd, args, dout)
            flat[c] = keep
            fd = (lp - lm) / (2 * h)
            an = g.reshape(-1)[c]
            assert abs(fd - an) <= tol * max(1.0, abs(fd)), (name, c, fd, an)


_NAMES = {}


def args_by_name(args, name):
    return args[_NAMES[name]]


def _inputs(rng, B, Lq, H, D, N, T_raw):
    return (rng.standard_normal((B, Lq, H, D)), rng.standard_normal((B, N, D)), rng.standard_normal((B, N, D)),
            rng.standard_normal((B, T_raw, D)), rng.standard_normal((B, T_raw, D)), rng.standard_normal(H))


@pytest.mark.parametrize("with_sink", [True, False])
def test_csa_backward_matches_finite_differences(with_sink):
    rng = np.random.default_rng(31)
    B, Lq, H, D, N, W, q_pos0 = 2, 3, 2, 64, 8, 4, 2       # t = 2, 3, 4: windows cut at position 0
    q, k_c, v_c, k_raw, v_raw, sink = _inputs(rng, B, Lq, H, D, N, 8)
    sink = sink if with_sink else None
    # entries shared between the queries of a sequence, a padded slot
    idx = np.array([[[0, 3, 5], [3, 5, 7], [1, 3, -1]], [[2, 4, 6], [0, 2, 6], [6, 7, 1]]])
    dout = rng.standard_normal((B, Lq, H, D))
    fwd = lambda q_, kc_, vc_, kr_, vr_, s_: oatt.csa_sparse_attn(q_, q_pos0, kc_, vc_, idx, kr_, vr_, 0, W, s_)
    args = (q, k_c, v_c, k_raw, v_raw, sink)
    _NAMES.clear(); _NAMES.update(q=0, k_c=1, v_c=2, k_raw=3, v_raw=4, sink=5)
    g = obwd.csa_sparse_attn_bwd(q, q_pos0, k_c, v_c, idx, k_raw, v_raw, 0, W, sink, dout)
    names = ["q", "k_c", "v_c", "k_raw", "v_raw"] + (["sink"] if with_sink else [])
    _check_fd(fwd, args, names, g[:len(names)], dout, rng)
    if not with_sink:
        assert np.all(g[5] == 0)


def test_hca_backward_matches_finite_differences():
    rng = np.random.default_rng(32)
    B, Lq, H, D, m, W, q_pos0 = 1, 3, 2, 64, 2, 3, 7       # n(t) = 4, 4, 5 entries
    q, k_c, v_c, k_raw, v_raw, sink = _inputs(rng, B, Lq, H, D, 6, 12)
    dout = rng.standard_normal((B, Lq, H, D))
    fwd = lambda q_, kc_, vc_, kr_, vr_, s_: oatt.hca_dense_attn(q_, q_pos0, m, kc_, vc_, kr_, vr_, 0, W, s_)
    args = (q, k_c, v_c, k_raw, v_raw, sink)
    _NAMES.clear(); _NAMES.update(q=0, k_c=1, v_c=2, k_raw=3, v_raw=4, sink=5)
    g = obwd.hca_dense_attn_bwd(q, q_pos0, m, k_c, v_c, k_raw, v_raw, 0, W, sink, dout)
    _check_fd(fwd, args, ["q", "k_c", "v_c", "k_raw", "v_raw", "sink"], g, dout, rng)
    # entries past n(t) of every query get no gradient
    assert np.all(g[1][0, 5:] == 0)


def test_value_gradient_closed_form():
    """One query: the source weights P_hr sum to 1 - Pz_h, so the value
    gradients add up to sum_h (1 - Pz_h) dO_h."""
    rng = np.random.default_rng(33)
    H, D, n = 3, 64, 5
    q, keys, vals = rng.standard_normal((H, D)), rng.standard_normal((n, D)), rng.standard_normal((n, D))
    wk, wv, pos = rng.standard_normal((2, D)), rng.standard_normal((2, D)), np.array([9, 10])
    sink, dout = rng.standard_normal(H), rng.standard_normal((H, D))
    g = obwd.attend_one_bwd(q, 10, keys, vals, wk, pos, wv, sink, dout)
    _, lse = oatt.attend_one(q, 10, keys, vals, wk, pos, wv, sink)
    pz = np.exp(sink - lse)
    want = ((1 - pz)[:, None] * dout).sum(axis=0)
    assert np.allclose(g[2].sum(axis=0) + g[4].sum(axis=0), want, atol=1e-12)
    # and the sink gradient is -Pz_h <dO_h, o_h>
    out, _ = oatt.attend_one(q, 10, keys, vals, wk, pos, wv, sink)
    assert np.allclose(g[5], -pz * (dout * out).sum(axis=1), atol=1e-12)
