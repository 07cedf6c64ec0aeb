"""Pins of the oracle's compressor, indexer and top-k: closed forms, a worked
example, brute force with plain Python loops and exhaustive tiny cases."""
import itertools
import math

import numpy as np
import pytest

from oracle.compress import compress, n_visible
from oracle.indexer import index_scores, index_scores_batch
from oracle.rope import apply_rope
from oracle.topk import topk_select, topk_batch


# ---------------------------------------------------------------- compressor
def test_m1_is_rotated_identity():
    rng = np.random.default_rng(0)
    k = rng.standard_normal((10, 128))
    v = rng.standard_normal((10, 128))
    kc, vc = compress(k, v, rng.standard_normal(128), m=1, pos0=0)
    for s in range(10):
        np.testing.assert_allclose(kc[s], apply_rope(k[s], s), atol=1e-14)
    np.testing.assert_array_equal(vc, v)


def test_zero_gate_is_block_mean():
    rng = np.random.default_rng(1)
    k = rng.standard_normal((16, 128))
    v = rng.standard_normal((16, 128))
    kc, vc = compress(k, v, np.zeros(128), m=4, pos0=8)
    for i in range(4):
        j = 2 + i                                  # pos0 // m + i
        np.testing.assert_allclose(kc[i], apply_rope(k[4 * i:4 * i + 4].mean(0), 4 * j + 3), atol=1e-14)
        np.testing.assert_allclose(vc[i], v[4 * i:4 * i + 4].mean(0), atol=1e-15)


def test_worked_gate_example():
    # gates 0 and ln 3 -> weights 1/4 and 3/4
    k = np.zeros((2, 64))
    k[1, 0] = math.log(3.0)
    k[0, 5], k[1, 5] = 4.0, 8.0
    v = np.zeros((2, 64))
    v[0, 1], v[1, 1] = 4.0, 8.0
    w = np.zeros(64)
    w[0] = 1.0
    kc, vc = compress(k, v, w, m=2, pos0=0)
    assert abs(vc[0, 1] - 7.0) < 1e-14            # 0.25*4 + 0.75*8
    pre = np.zeros(64)
    pre[0] = 0.75 * math.log(3.0)
    pre[5] = 7.0
    np.testing.assert_allclose(kc[0], apply_rope(pre, 1), atol=1e-14)   # p = 0*2 + 2 - 1


def test_permutation_invariance_and_hull():
    rng = np.random.default_rng(2)
    k = rng.standard_normal((8, 128))
    v = rng.standard_normal((8, 128))
    w = rng.standard_normal(128)
    kc, vc = compress(k, v, w, m=8)
    perm = rng.permutation(8)
    kc2, vc2 = compress(k[perm], v[perm], w, m=8)
    np.testing.assert_allclose(kc, kc2, atol=1e-13)
    np.testing.assert_allclose(vc, vc2, atol=1e-13)
    assert np.all(vc[0] <= v.max(0) + 1e-13) and np.all(vc[0] >= v.min(0) - 1e-13)


def test_block_alignment_and_tail():
    rng = np.random.default_rng(3)
    k = rng.standard_normal((14, 64))
    v = rng.standard_normal((14, 64))
    w = rng.standard_normal(64)
    full_k, full_v = compress(k, v, w, m=4, pos0=0)
    assert full_k.shape == (3, 64)                 # the 2-token tail makes no entry
    part_k, part_v = compress(k[4:], v[4:], w, m=4, pos0=4)
    np.testing.assert_array_equal(part_k, full_k[1:])
    with pytest.raises(AssertionError):
        compress(k[2:], v[2:], w, m=4, pos0=2)
    assert n_visible(2, 4) == 0 and n_visible(3, 4) == 1 and n_visible(131071, 4) == 32768


# ------------------------------------------------------------------- indexer
def _brute_scores(q, w, k):
    n, d = len(k), len(k[0])
    out = []
    for j in range(n):
        tot = 0.0
        for h in range(len(q)):
            dot = 0.0
            for c in range(d):
                dot += q[h][c] * k[j][c]
            tot += w[h] * (dot if dot > 0 else 0.0)
        out.append(tot)
    return out


def test_indexer_worked_example():
    q = np.array([[1.0, 0.0], [0.0, 1.0]])
    w = np.array([2.0, -1.0])
    k = np.array([[3.0, 1.0], [-1.0, 2.0], [-1.0, -1.0]])
    np.testing.assert_array_equal(index_scores(q, w, k), [5.0, -2.0, 0.0])


def test_indexer_brute_force():
    rng = np.random.default_rng(4)
    q = rng.integers(-2, 3, (4, 32)).astype(float)
    w = np.round(rng.standard_normal(4) / math.sqrt(32) * 256) / 256
    k = rng.integers(-2, 3, (37, 32)).astype(float)
    assert index_scores(q, w, k).tolist() == _brute_scores(q.tolist(), w.tolist(), k.tolist())


def test_indexer_batch_visibility():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 3, 2, 8))
    w = rng.standard_normal((1, 3, 2))
    k = rng.standard_normal((1, 6, 8))
    s = index_scores_batch(q, w, k, q_pos0=9, m=4)       # t = 9, 10, 11 -> n = 2, 2, 3
    assert np.isneginf(s[0, 0, 2:]).all() and np.isfinite(s[0, 0, :2]).all()
    assert np.isfinite(s[0, 2, :3]).all() and np.isneginf(s[0, 2, 3:]).all()


# ---------------------------------------------------------------------- top-k
def _ref_topk(s, k):
    order = sorted(range(len(s)), key=lambda j: (-s[j], j))
    sel = sorted(order[:min(k, len(s))])
    return sel + [-1] * (k - len(sel))


def test_topk_exhaustive_tiny():
    vals = (-1.0, -0.0, 0.0, 1.0)
    for n in range(0, 6):
        for s in itertools.product(vals, repeat=n):
            for k in range(0, 8):
                assert topk_select(np.array(s), k).tolist() == _ref_topk(list(s), k)


def test_topk_invariants_random():
    rng = np.random.default_rng(6)
    for trial in range(200):
        n = int(rng.integers(1, 300))
        k = int(rng.integers(0, 64))
        s = rng.integers(-3, 4, n).astype(float)      # many ties
        idx = topk_select(s, k)
        sel = idx[idx >= 0]
        assert len(sel) == min(k, n)
        assert np.all(np.diff(sel) > 0)
        uns = np.setdiff1d(np.arange(n), sel)
        if len(sel) and len(uns):
            thr = s[sel].min()
            assert thr >= s[uns].max()
            # among entries equal to the threshold, the selected ones come first
            tied_sel = sel[s[sel] == thr]
            tied_uns = uns[s[uns] == thr]
            if len(tied_uns):
                assert tied_sel.max() < tied_uns.min()


def test_topk_batch_visibility_and_padding():
    s = np.full((1, 2, 8), -np.inf)
    s[0, 0, :2] = [1.0, 2.0]                     # t = 9, m = 4 -> n = 2
    s[0, 1, :3] = [5.0, 5.0, 5.0]                # t = 11 -> n = 3
    idx = topk_batch(s, 4, q_pos0=9, m=4)
    assert idx[0, 0].tolist() == [0, 1, -1, -1]
    idx = topk_batch(s[:, 1:], 2, q_pos0=11, m=4)
    assert idx[0, 0].tolist() == [0, 1]


def test_topk_bf16_worked_rows():
    """[P1] section FP4 量化: indexer scores rounded from FP32 to BF16 before the
    top-k. Expected selections worked by hand from the bf16 grid (8 significant
    bits: spacing 2^-7 on [1, 2)), with ties between equal rounded scores going
    to the lower index. Sequence 0 sees 7 entries (position 6, m = 1), sequence
    1 sees 6 (position 5); the entries past them hold NaN / -inf and are never
    read."""
    from oracle.topk import topk_batch_bf16
    e = 2.0 ** -10
    row0 = [0.5,                 # -> 0.5
            1.0,                 # -> 1.0
            2.0,                 # -> 2.0
            1.0 + e,             # below the midpoint 1 + 2^-8: -> 1.0
            1.0 + 2.0 ** -8,     # the midpoint itself: ties to the even code, 1.0
            1.0 + 3 * 2.0 ** -8,  # midpoint of 1 + 2^-7 (odd) and 1 + 2^-6 (even): -> 1.015625
            1.0 + 2.0 ** -7 - e,  # above the midpoint 1 + 2^-8: -> 1.0078125
            float("nan")]        # invisible
    row1 = [-1.0 - e,            # -> -1.0, ties with entry 1
            -1.0,
            -0.0,                # -0 counts as +0
            2.0 ** -140,         # far below bf16's smallest subnormal 2^-133: -> +0
            0.0,
            -2.0,
            -float("inf"),       # invisible
            float("nan")]        # invisible
    scores = np.array([[row0], [row1]], dtype=np.float64)
    idx = topk_batch_bf16(scores, 4, np.array([6, 5]), 1)
    # row 0 rounded: [0.5, 1, 2, 1, 1, 1.015625, 1.0078125]; by (-r, j): 2, 5, 6, then 1
    assert idx[0, 0].tolist() == [1, 2, 5, 6]
    # row 1 rounded: [-1, -1, 0, 0, 0, -2]; by (-r, j): 2, 3, 4, then 0
    assert idx[1, 0].tolist() == [0, 2, 3, 4]
    # the f32 order would differ in both rows (a selection made before rounding)
    from oracle.topk import topk_batch
    f32 = topk_batch(np.where(np.isfinite(scores), scores, 0.0), 4, np.array([6, 5]), 1)
    assert f32[0, 0].tolist() == [2, 4, 5, 6] and f32[1, 0].tolist() == [1, 2, 3, 4]
    # fewer visible entries than k: every one, then -1 padding
    idx = topk_batch_bf16(scores, 8, np.array([6, 5]), 1)
    assert idx[0, 0].tolist() == [0, 1, 2, 3, 4, 5, 6, -1]
    assert idx[1, 0].tolist() == [0, 1, 2, 3, 4, 5, -1, -1]
