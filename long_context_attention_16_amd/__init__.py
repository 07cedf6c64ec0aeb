"""MI355X (gfx950) hybrid compressed attention: CSA and HCA.

Thin Python binding of the C-ABI library libcsa.so (declared in include/csa.h).
The functions here only marshal torch tensors (device pointers, sizes and the
current HIP stream) into the C calls; every step of the computation runs in
the library's HIP kernels. There is no fallback: if libcsa.so is missing or the
tensors are not on a GPU, the calls raise.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcsa.so")

CSA_F32, CSA_BF16, CSA_FP8_E4M3, CSA_FP4_E2M1 = 0, 1, 2, 3
IDX_FORMATS = {"f32": CSA_F32, "bf16": CSA_BF16, "fp8": CSA_FP8_E4M3, "fp4": CSA_FP4_E2M1}

# (name, restype, argtypes) of every exported symbol
_I, _L, _P, _Z = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
SIGNATURES = {
    "csa_abi_version": (_I, []),
    "csa_strerror": (ctypes.c_char_p, [_I]),
    "csa_compress": (_I, [_I, _I, _I, _I, _L, _I, _P, _P, _P, _P, _P, _L, _I, _I, _P, _P, _P, _P]),
    "csa_index_topk_ws_bytes": (_Z, [_I, _I, _L, _I, _L, _I]),
    "csa_topk_ws_bytes": (_Z, [_I, _I, _L, _I, _I]),
    "csa_index_topk": (_I, [_I, _I, _L, _I, _L, _I, _I, _I, _P, _P, _P, _P, _P, _I, _P, _P, _Z, _P]),
    "csa_index_scores": (_I, [_I, _I, _L, _I, _L, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P]),
    "csa_topk": (_I, [_I, _I, _L, _I, _L, _P, _I, _P, _P, _Z, _P]),
    "csa_index_candidates_bytes": (_Z, [_I, _I, _L, _I, _I]),
    "csa_index_candidates": (_I, [_I, _I, _L, _I, _L, _I, _I, _I, _P, _P, _P, _P, _P, _I, _P, _Z, _P]),
    "csa_topk_merge": (_I, [_I, _I, _L, _I, _I, _P, _Z, _P, _P]),
    "csa_sparse_attn_ws_bytes": (_Z, [_I, _I, _I, _I, _I, _I]),
    "csa_sparse_attn": (_I, [_I, _I, _L, _I, _I, _I, _P, _L, _P, _P, _I, _P, _I, _L, _P, _P, _I,
                             _P, _P, _P, _P, _Z, _P]),
    "csa_sparse_attn_noalloc": (_I, [_I, _I, _L, _I, _I, _I, _P, _L, _P, _P, _I, _P, _I, _L, _P, _P, _I,
                                     _P, _P, _P, _P]),
    "hca_dense_attn_ws_bytes": (_Z, [_I, _I, _L, _I, _I, _I, _I]),
    "hca_dense_attn": (_I, [_I, _I, _L, _I, _I, _I, _I, _P, _L, _P, _P, _I, _L, _P, _P, _I,
                            _P, _P, _P, _P, _Z, _P]),
    "csa_state_append": (_I, [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _L, _I, _I,
                              _P, _P, _P, _P, _P]),
    "csa_index_topk_varlen": (_I, [_I, _I, _P, _L, _I, _L, _I, _I, _I, _P, _P, _P, _P, _P, _I, _P, _P,
                                   _Z, _P]),
    "csa_sparse_attn_varlen": (_I, [_I, _I, _P, _L, _I, _I, _I, _P, _L, _P, _P, _I, _P, _I, _P, _P, _I,
                                    _P, _P, _P, _P, _Z, _P]),
    "hca_dense_attn_varlen": (_I, [_I, _I, _P, _L, _I, _I, _I, _I, _P, _L, _P, _P, _I, _P, _P, _I,
                                   _P, _P, _P, _P, _Z, _P]),
    "csa_index_topk_ex": (_I, [_I, _I, _P, _L, _I, _L, _I, _I, _I, _P, _P, _P, _P, _P, _I, _I, _P, _P,
                               _Z, _P]),
    "csa_index_scores_ex": (_I, [_I, _I, _P, _L, _I, _L, _I, _I, _I, _P, _P, _P, _P, _P, _I, _P, _P]),
    "csa_sparse_attn_bwd_ws_bytes": (_Z, [_I, _I, _L, _I, _I, _I, _L, _I, _I]),
    "csa_sparse_attn_bwd": (_I, [_I, _I, _L, _I, _I, _I, _P, _L, _P, _P, _I, _P, _I, _L, _P, _P, _I, _P, _P, _P, _P,
                                 _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "hca_dense_attn_bwd": (_I, [_I, _I, _L, _I, _I, _I, _I, _P, _L, _P, _P, _I, _L, _P, _P, _I, _P, _P, _P, _P,
                                _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
}

_lib = None


class CSAError(RuntimeError):
    pass


def lib():
    """Load libcsa.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise CSAError("libcsa.so is not built (run __graft_entry__.build() or "
                           "python -m long_context_attention_16_amd.build_lib)")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib = h
    return _lib


def _check(rc):
    if rc != 0:
        raise CSAError("csa call failed: %d (%s)" % (rc, lib().csa_strerror(rc).decode()))


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise CSAError("tensor is not on a GPU")
    if not t.is_contiguous():
        raise CSAError("tensor is not contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _kv_dtype(t):
    if t.dtype == torch.float32:
        return CSA_F32
    if t.dtype == torch.bfloat16:
        return CSA_BF16
    raise CSAError("KV tensors must be float32 or bfloat16, got %s" % t.dtype)


def _ws(nbytes, device):
    """A workspace for a call made without one (the library needs no initial
    contents, so none are written). Callers in a loop or under graph capture
    pass their own `ws` and allocate nothing per call."""
    return torch.empty((max(16, int(nbytes)) + 15) // 16 * 4, dtype=torch.float32, device=device)


_IDX_ESIZE = {"f32": 4, "bf16": 2, "fp8": 1, "fp4": 1}


def _expect(t, shape, name, dtype=None, esize=None):
    """Shape (and dtype or element size) check of a tensor handed to the
    library, which trusts the sizes it is given; None passes."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise CSAError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if dtype is not None and t.dtype != dtype:
        raise CSAError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if esize is not None and t.element_size() != esize:
        raise CSAError("%s has %d-byte elements, expected %d" % (name, t.element_size(), esize))


def _indexer_shapes(q_i, w_i, k_i, fmt, q_scale, k_scale):
    """(B, Lq, H_i, N_cap, d_i) of the indexer operands, checked against one
    another."""
    if fmt not in IDX_FORMATS:
        raise CSAError("unknown indexer format %r" % (fmt,))
    if w_i.dim() != 3 or k_i.dim() != 3 or q_i.dim() != 4:
        raise CSAError("indexer operands must be q_i [B, Lq, H_i, d], w_i [B, Lq, H_i], k_i [B, N_cap, d]")
    B, Lq, H_i = w_i.shape
    N_cap, dq = k_i.shape[1], q_i.shape[-1]
    d_i = dq * (2 if fmt == "fp4" else 1)
    es = _IDX_ESIZE[fmt]
    _expect(w_i, (B, Lq, H_i), "w_i", dtype=torch.float32)
    _expect(q_i, (B, Lq, H_i, dq), "q_i", esize=es)
    _expect(k_i, (B, N_cap, dq), "k_i", esize=es)
    if fmt == "fp4":
        if q_scale is None or k_scale is None:
            raise CSAError("fp4 operands need q_scale and k_scale")
        _expect(q_scale, (B, Lq, H_i, d_i // 32), "q_scale", esize=1)
        _expect(k_scale, (B, N_cap, d_i // 32), "k_scale", esize=1)
    return B, Lq, H_i, N_cap, d_i


def _attn_shapes(q, k_c, v_c, k_raw, v_raw, sink, out=None, lse=None):
    """(B, Lq, H, D) of an attention call, its other operands checked against
    q (keys, values and out in q's dtype; sink and lse float32)."""
    if q.dim() != 4 or k_c.dim() != 3 or k_raw.dim() != 3:
        raise CSAError("attention operands must be q [B, Lq, H, D], k_c [B, N_cap, D], k_raw [B, T, D]")
    B, Lq, H, D = q.shape
    _kv_dtype(q)
    _expect(k_c, (B, k_c.shape[1], D), "k_c", dtype=q.dtype)
    _expect(v_c, k_c.shape, "v_c", dtype=q.dtype)
    _expect(k_raw, (B, k_raw.shape[1], D), "k_raw (or k_ring)", dtype=q.dtype)
    _expect(v_raw, k_raw.shape, "v_raw (or v_ring)", dtype=q.dtype)
    _expect(sink, (H,), "sink", dtype=torch.float32)
    _expect(out, q.shape, "out", dtype=q.dtype)
    _expect(lse, (B, Lq, H), "lse", dtype=torch.float32)
    return B, Lq, H, D


# ------------------------------------------------------------------ compress
def compress(k_raw, v_raw, w_gate, m, pos0, k_c, v_c, ki_raw=None, ki_c=None, ki_scale=None, idx_fmt="bf16"):
    """Fold [B, T, D] raw rows at absolute positions pos0.. into k_c, v_c
    [B, N_cap, D] (rows pos0//m .. pos0//m + T//m - 1 are written). With
    ki_raw [B, T, d_i] (KV dtype) the indexer keys are folded with the same
    weights into ki_c [B, N_cap, d_i] in idx_fmt ('f32', 'bf16', 'fp8', or
    'fp4': [B, N_cap, d_i/2] bytes plus ki_scale [B, N_cap, d_i/32])."""
    B, T, D = k_raw.shape
    _kv_dtype(k_raw)
    _expect(v_raw, k_raw.shape, "v_raw", dtype=k_raw.dtype)
    _expect(w_gate, (D,), "w_gate", dtype=torch.float32)
    _expect(k_c, (B, k_c.shape[1], D), "k_c", dtype=k_raw.dtype)
    _expect(v_c, k_c.shape, "v_c", dtype=k_raw.dtype)
    d_i = 0
    if ki_raw is not None:
        if idx_fmt not in IDX_FORMATS:
            raise CSAError("unknown indexer format %r" % (idx_fmt,))
        d_i = ki_raw.shape[-1]
        _expect(ki_raw, (B, T, d_i), "ki_raw", dtype=k_raw.dtype)
        fp4 = idx_fmt == "fp4"
        if ki_c is None:
            raise CSAError("ki_raw needs ki_c")
        _expect(ki_c, (B, k_c.shape[1], d_i // 2 if fp4 else d_i), "ki_c", esize=_IDX_ESIZE[idx_fmt])
        if fp4:
            if ki_scale is None:
                raise CSAError("fp4 indexer keys need ki_scale")
            _expect(ki_scale, (B, k_c.shape[1], d_i // 32), "ki_scale", esize=1)
    _check(lib().csa_compress(B, T, D, m, pos0, _kv_dtype(k_raw), _ptr(k_raw), _ptr(v_raw),
                              _ptr(w_gate), _ptr(k_c), _ptr(v_c), k_c.shape[1], d_i, IDX_FORMATS[idx_fmt],
                              _ptr(ki_raw), _ptr(ki_c if d_i else None), _ptr(ki_scale if d_i else None),
                              _stream()))
    return k_c, v_c


# ---------------------------------------------------------- indexer + top-k
def index_topk_ws_bytes(B, Lq, q_pos0, m, N_cap, topk):
    return lib().csa_index_topk_ws_bytes(B, Lq, q_pos0, m, N_cap, topk)


def topk_ws_bytes(B, Lq, q_pos0, m, topk):
    return lib().csa_topk_ws_bytes(B, Lq, q_pos0, m, topk)


def index_topk(q_i, w_i, k_i, topk, q_pos0, m, fmt, q_scale=None, k_scale=None, ws=None, out=None):
    """Indexer scores and per-query top-k.

    q_i [B, Lq, H_i, d_i] (fp4: [..., d_i/2] bytes + q_scale [..., d_i/32]),
    w_i [B, Lq, H_i] f32, k_i [B, N_cap, d_i] (fp4: bytes + k_scale).
    fmt: 'f32' | 'bf16' | 'fp8' | 'fp4'. Returns idx [B, Lq, topk] int32.
    """
    B, Lq, H_i, N_cap, d_i = _indexer_shapes(q_i, w_i, k_i, fmt, q_scale, k_scale)
    if ws is None:
        ws = _ws(index_topk_ws_bytes(B, Lq, q_pos0, m, N_cap, topk), q_i.device)
    if out is None:
        out = torch.empty((B, Lq, topk), dtype=torch.int32, device=q_i.device)
    _expect(out, (B, Lq, topk), "out", dtype=torch.int32)
    _check(lib().csa_index_topk(B, Lq, q_pos0, m, N_cap, H_i, d_i, IDX_FORMATS[fmt], _ptr(q_i),
                                _ptr(q_scale), _ptr(w_i), _ptr(k_i), _ptr(k_scale), topk, _ptr(out),
                                _ptr(ws), ws.numel() * ws.element_size(), _stream()))
    return out


def index_candidates_bytes(B, Lq, q_pos0, m, topk):
    return lib().csa_index_candidates_bytes(B, Lq, q_pos0, m, topk)


def index_candidates(q_i, w_i, k_i, topk, q_pos0, m, fmt, q_scale=None, k_scale=None, cand=None):
    """First launch of the fused index_topk: per-(row, 2048-entry chunk) top-k
    candidate lists, written into (and returned as) the buffer `cand`."""
    B, Lq, H_i, N_cap, d_i = _indexer_shapes(q_i, w_i, k_i, fmt, q_scale, k_scale)
    if cand is None:
        cand = _ws(index_candidates_bytes(B, Lq, q_pos0, m, topk), q_i.device)
    _check(lib().csa_index_candidates(B, Lq, q_pos0, m, N_cap, H_i, d_i, IDX_FORMATS[fmt], _ptr(q_i),
                                      _ptr(q_scale), _ptr(w_i), _ptr(k_i), _ptr(k_scale), topk, _ptr(cand),
                                      cand.numel() * cand.element_size(), _stream()))
    return cand


def topk_merge(cand, B, Lq, topk, q_pos0, m, out=None):
    """Second launch of the fused index_topk: idx [B, Lq, topk] int32 from the
    candidate lists in `cand`."""
    if out is None:
        out = torch.empty((B, Lq, topk), dtype=torch.int32, device=cand.device)
    _expect(out, (B, Lq, topk), "out", dtype=torch.int32)
    _check(lib().csa_topk_merge(B, Lq, q_pos0, m, topk, _ptr(cand), cand.numel() * cand.element_size(),
                                _ptr(out), _stream()))
    return out


def index_scores(q_i, w_i, k_i, q_pos0, m, fmt, q_scale=None, k_scale=None, out=None):
    """Indexer scores only: returns (or fills) scores [B, Lq, N_cap] float32;
    entries not yet visible to a query are left untouched."""
    B, Lq, H_i, N_cap, d_i = _indexer_shapes(q_i, w_i, k_i, fmt, q_scale, k_scale)
    if out is None:
        out = torch.full((B, Lq, N_cap), float("-inf"), dtype=torch.float32, device=q_i.device)
    _expect(out, (B, Lq, N_cap), "out", dtype=torch.float32)
    _check(lib().csa_index_scores(B, Lq, q_pos0, m, N_cap, H_i, d_i, IDX_FORMATS[fmt], _ptr(q_i),
                                  _ptr(q_scale), _ptr(w_i), _ptr(k_i), _ptr(k_scale), _ptr(out), _stream()))
    return out


def topk(scores, k, q_pos0, m, out=None, ws=None):
    """Top-k of caller scores [B, Lq, N_cap] f32 -> idx [B, Lq, k] int32."""
    B, Lq, N_cap = scores.shape
    _expect(scores, (B, Lq, N_cap), "scores", dtype=torch.float32)
    if out is None:
        out = torch.empty((B, Lq, k), dtype=torch.int32, device=scores.device)
    _expect(out, (B, Lq, k), "out", dtype=torch.int32)
    if ws is None:
        ws = _ws(topk_ws_bytes(B, Lq, q_pos0, m, k), scores.device)
    _check(lib().csa_topk(B, Lq, q_pos0, m, N_cap, _ptr(scores), k, _ptr(out), _ptr(ws),
                          ws.numel() * ws.element_size(), _stream()))
    return out


# ---------------------------------------------------------------- attention
def sparse_attn_ws_bytes(B, Lq, H, D, topk, W):
    return lib().csa_sparse_attn_ws_bytes(B, Lq, H, D, topk, W)


def hca_attn_ws_bytes(B, Lq, q_pos0, m, H, D, W):
    return lib().hca_dense_attn_ws_bytes(B, Lq, q_pos0, m, H, D, W)


def _alloc_out(q, out, lse):
    B, Lq, H, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Lq, H), dtype=torch.float32, device=q.device)
    return out, lse


def sparse_attn(q, k_c, v_c, idx, k_raw, v_raw, raw_pos0, W, sink, q_pos0, ws=None, out=None, lse=None):
    """CSA attention. q [B, Lq, H, D]; k_c, v_c [B, N_cap, D]; idx [B, Lq, k];
    k_raw, v_raw [B, T_raw, D] at positions raw_pos0..; sink [H] f32 or None.
    Returns (out [B, Lq, H, D], lse [B, Lq, H])."""
    B, Lq, H, D = _attn_shapes(q, k_c, v_c, k_raw, v_raw, sink, out, lse)
    topk_ = idx.shape[-1]
    _expect(idx, (B, Lq, topk_), "idx", dtype=torch.int32)
    if ws is None:
        ws = _ws(sparse_attn_ws_bytes(B, Lq, H, D, topk_, W), q.device)
    out, lse = _alloc_out(q, out, lse)
    _check(lib().csa_sparse_attn(B, Lq, q_pos0, H, D, _kv_dtype(q), _ptr(q), k_c.shape[1], _ptr(k_c),
                                 _ptr(v_c), topk_, _ptr(idx), k_raw.shape[1], raw_pos0, _ptr(k_raw),
                                 _ptr(v_raw), W, _ptr(sink), _ptr(out), _ptr(lse), _ptr(ws),
                                 ws.numel() * ws.element_size(), _stream()))
    return out, lse


def hca_attn(q, k_c, v_c, m, k_raw, v_raw, raw_pos0, W, sink, q_pos0, ws=None, out=None, lse=None):
    """HCA attention over every visible entry (block m). Shapes as sparse_attn."""
    B, Lq, H, D = _attn_shapes(q, k_c, v_c, k_raw, v_raw, sink, out, lse)
    if ws is None:
        ws = _ws(hca_attn_ws_bytes(B, Lq, q_pos0, m, H, D, W), q.device)
    out, lse = _alloc_out(q, out, lse)
    _check(lib().hca_dense_attn(B, Lq, q_pos0, m, H, D, _kv_dtype(q), _ptr(q), k_c.shape[1], _ptr(k_c),
                                _ptr(v_c), k_raw.shape[1], raw_pos0, _ptr(k_raw), _ptr(v_raw), W,
                                _ptr(sink), _ptr(out), _ptr(lse), _ptr(ws),
                                ws.numel() * ws.element_size(), _stream()))
    return out, lse


# ------------------------------------------------- decode state cache, varlen
def _pos_tensor(pos):
    if pos.dtype != torch.int64:
        raise CSAError("positions must be int64")
    return _ptr(pos)


def state_append(pos, k_new, v_new, w_gate, m, k_ring, v_ring, k_c, v_c,
                 ki_new=None, ki_ring=None, ki_c=None, ki_scale=None, idx_fmt="bf16"):
    """One decode step of the state cache: token rows k_new, v_new [B, D]
    (and ki_new [B, d_i]) at positions pos [B] int64 enter the rings
    k_ring, v_ring [B, R, D] (ki_ring [B, R, d_i]); blocks they complete are
    compressed into k_c, v_c [B, N_cap, D] (ki_c in idx_fmt, + ki_scale for
    fp4). Negative positions are skipped."""
    B, D = k_new.shape
    R = k_ring.shape[1]
    d_i = 0 if ki_new is None else ki_new.shape[1]
    _kv_dtype(k_new)
    _expect(pos, (B,), "pos", dtype=torch.int64)
    _expect(v_new, (B, D), "v_new", dtype=k_new.dtype)
    _expect(w_gate, (D,), "w_gate", dtype=torch.float32)
    _expect(k_ring, (B, R, D), "k_ring", dtype=k_new.dtype)
    _expect(v_ring, (B, R, D), "v_ring", dtype=k_new.dtype)
    _expect(k_c, (B, k_c.shape[1], D), "k_c", dtype=k_new.dtype)
    _expect(v_c, k_c.shape, "v_c", dtype=k_new.dtype)
    if ki_new is not None:
        if idx_fmt not in IDX_FORMATS:
            raise CSAError("unknown indexer format %r" % (idx_fmt,))
        _expect(ki_new, (B, d_i), "ki_new", dtype=k_new.dtype)
        _expect(ki_ring, (B, R, d_i), "ki_ring", dtype=k_new.dtype)
        fp4 = idx_fmt == "fp4"
        _expect(ki_c, (B, k_c.shape[1], d_i // 2 if fp4 else d_i), "ki_c", esize=_IDX_ESIZE[idx_fmt])
        if fp4:
            _expect(ki_scale, (B, k_c.shape[1], d_i // 32), "ki_scale", esize=1)
    _check(lib().csa_state_append(B, D, m, R, _kv_dtype(k_new), _pos_tensor(pos), _ptr(k_new), _ptr(v_new),
                                  _ptr(w_gate), _ptr(k_ring), _ptr(v_ring), _ptr(k_c), _ptr(v_c), k_c.shape[1],
                                  d_i, IDX_FORMATS[idx_fmt], _ptr(ki_new), _ptr(ki_ring), _ptr(ki_c),
                                  _ptr(ki_scale), _stream()))


def index_topk_varlen(q_i, w_i, k_i, topk, q_pos, q_pos_max, m, fmt, q_scale=None, k_scale=None,
                      ws=None, out=None):
    """index_topk with query row 0 of sequence b at q_pos[b] (int64 [B] on
    the GPU, bounded by the host value q_pos_max)."""
    B, Lq, H_i, N_cap, d_i = _indexer_shapes(q_i, w_i, k_i, fmt, q_scale, k_scale)
    if ws is None:
        ws = _ws(index_topk_ws_bytes(B, Lq, q_pos_max, m, N_cap, topk), q_i.device)
    if out is None:
        out = torch.empty((B, Lq, topk), dtype=torch.int32, device=q_i.device)
    _expect(out, (B, Lq, topk), "out", dtype=torch.int32)
    _check(lib().csa_index_topk_varlen(B, Lq, _pos_tensor(q_pos), q_pos_max, m, N_cap, H_i, d_i,
                                       IDX_FORMATS[fmt], _ptr(q_i), _ptr(q_scale), _ptr(w_i), _ptr(k_i),
                                       _ptr(k_scale), topk, _ptr(out), _ptr(ws),
                                       ws.numel() * ws.element_size(), _stream()))
    return out


def sparse_attn_varlen(q, k_c, v_c, idx, k_ring, v_ring, W, sink, q_pos, q_pos_max, ws=None, out=None,
                       lse=None):
    """sparse_attn with per-sequence positions q_pos [B] int64 (bound
    q_pos_max) and the window read from the state cache's rings [B, R, D]."""
    B, Lq, H, D = _attn_shapes(q, k_c, v_c, k_ring, v_ring, sink, out, lse)
    topk_ = idx.shape[-1]
    _expect(idx, (B, Lq, topk_), "idx", dtype=torch.int32)
    _expect(q_pos, (B,), "q_pos", dtype=torch.int64)
    if ws is None:
        ws = _ws(sparse_attn_ws_bytes(B, Lq, H, D, topk_, W), q.device)
    out, lse = _alloc_out(q, out, lse)
    _check(lib().csa_sparse_attn_varlen(B, Lq, _pos_tensor(q_pos), q_pos_max, H, D, _kv_dtype(q), _ptr(q),
                                        k_c.shape[1], _ptr(k_c), _ptr(v_c), topk_, _ptr(idx), k_ring.shape[1],
                                        _ptr(k_ring), _ptr(v_ring), W, _ptr(sink), _ptr(out), _ptr(lse),
                                        _ptr(ws), ws.numel() * ws.element_size(), _stream()))
    return out, lse


def hca_attn_varlen(q, k_c, v_c, m, k_ring, v_ring, W, sink, q_pos, q_pos_max, ws=None, out=None, lse=None):
    """hca_attn with per-sequence positions and the window from the rings."""
    B, Lq, H, D = _attn_shapes(q, k_c, v_c, k_ring, v_ring, sink, out, lse)
    _expect(q_pos, (B,), "q_pos", dtype=torch.int64)
    if ws is None:
        ws = _ws(hca_attn_ws_bytes(B, Lq, q_pos_max, m, H, D, W), q.device)
    out, lse = _alloc_out(q, out, lse)
    _check(lib().hca_dense_attn_varlen(B, Lq, _pos_tensor(q_pos), q_pos_max, m, H, D, _kv_dtype(q), _ptr(q),
                                       k_c.shape[1], _ptr(k_c), _ptr(v_c), k_ring.shape[1], _ptr(k_ring),
                                       _ptr(v_ring), W, _ptr(sink), _ptr(out), _ptr(lse), _ptr(ws),
                                       ws.numel() * ws.element_size(), _stream()))
    return out, lse


def index_topk_ex(q_i, w_i, k_i, topk, q_pos0, m, fmt, score_dtype="bf16", q_pos=None, q_scale=None,
                  k_scale=None, ws=None, out=None):
    """index_topk with the score precision ('f32' or 'bf16': scores rounded
    to bfloat16 before the top-k) and optional per-sequence positions q_pos
    [B] int64 (then q_pos0 is their bound)."""
    B, Lq, H_i, N_cap, d_i = _indexer_shapes(q_i, w_i, k_i, fmt, q_scale, k_scale)
    if ws is None:
        ws = _ws(index_topk_ws_bytes(B, Lq, q_pos0, m, N_cap, topk), q_i.device)
    if out is None:
        out = torch.empty((B, Lq, topk), dtype=torch.int32, device=q_i.device)
    _expect(out, (B, Lq, topk), "out", dtype=torch.int32)
    _check(lib().csa_index_topk_ex(B, Lq, None if q_pos is None else _pos_tensor(q_pos), q_pos0, m, N_cap, H_i,
                                   d_i, IDX_FORMATS[fmt], _ptr(q_i), _ptr(q_scale), _ptr(w_i), _ptr(k_i),
                                   _ptr(k_scale), topk, IDX_FORMATS[score_dtype], _ptr(out), _ptr(ws),
                                   ws.numel() * ws.element_size(), _stream()))
    return out


def index_scores_ex(q_i, w_i, k_i, q_pos0, m, fmt, score_dtype="bf16", q_pos=None, q_scale=None, k_scale=None,
                    out=None):
    """Indexer scores as f32 [B, Lq, N_cap] or bf16 [B, Lq, N_cap rounded up
    to even] (nearest even); optional per-sequence positions q_pos."""
    B, Lq, H_i, N_cap, d_i = _indexer_shapes(q_i, w_i, k_i, fmt, q_scale, k_scale)
    if out is None:
        if score_dtype == "bf16":
            out = torch.zeros((B, Lq, (N_cap + 1) // 2 * 2), dtype=torch.bfloat16, device=q_i.device)
        else:
            out = torch.full((B, Lq, N_cap), float("-inf"), dtype=torch.float32, device=q_i.device)
    if score_dtype == "bf16":
        _expect(out, (B, Lq, (N_cap + 1) // 2 * 2), "out", dtype=torch.bfloat16)
    else:
        _expect(out, (B, Lq, N_cap), "out", dtype=torch.float32)
    _check(lib().csa_index_scores_ex(B, Lq, None if q_pos is None else _pos_tensor(q_pos), q_pos0, m, N_cap, H_i,
                                     d_i, IDX_FORMATS[fmt], _ptr(q_i), _ptr(q_scale), _ptr(w_i), _ptr(k_i),
                                     _ptr(k_scale), IDX_FORMATS[score_dtype], _ptr(out), _stream()))
    return out


# ------------------------------------------------------------------ backward
def attn_bwd_ws_bytes(B, Lq, q_pos0, m, H, D, N_cap, topk, W):
    """Workspace bytes of sparse_attn_bwd (m = 0) or hca_attn_bwd (m > 0, topk 0)."""
    return lib().csa_sparse_attn_bwd_ws_bytes(B, Lq, q_pos0, m, H, D, N_cap, topk, W)


def _bwd_outputs(q, k_c, k_raw, sink):
    B, Lq, H, D = q.shape
    f = dict(dtype=torch.float32, device=q.device)
    return (torch.empty((B, Lq, H, D), **f), torch.empty(k_c.shape, **f), torch.empty(k_c.shape, **f),
            torch.empty(k_raw.shape, **f), torch.empty(k_raw.shape, **f),
            None if sink is None else torch.empty((H,), **f))


def sparse_attn_bwd(q, k_c, v_c, idx, k_raw, v_raw, raw_pos0, W, sink, q_pos0, out, lse, dout, ws=None):
    """Gradients of sparse_attn: (dq, dk_c, dv_c, dk_raw, dv_raw, dsink), f32."""
    B, Lq, H, D = _attn_shapes(q, k_c, v_c, k_raw, v_raw, sink, out, lse)
    _expect(idx, (B, Lq, idx.shape[-1]), "idx", dtype=torch.int32)
    _expect(dout, q.shape, "dout", dtype=q.dtype)
    if ws is None:
        ws = _ws(attn_bwd_ws_bytes(B, Lq, q_pos0, 0, H, D, k_c.shape[1], idx.shape[-1], W), q.device)
    g = _bwd_outputs(q, k_c, k_raw, sink)
    _check(lib().csa_sparse_attn_bwd(B, Lq, q_pos0, H, D, _kv_dtype(q), _ptr(q), k_c.shape[1], _ptr(k_c), _ptr(v_c),
                                     idx.shape[-1], _ptr(idx), k_raw.shape[1], raw_pos0, _ptr(k_raw), _ptr(v_raw), W,
                                     _ptr(sink), _ptr(out), _ptr(lse), _ptr(dout), *[_ptr(x) for x in g], _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream()))
    return g


def hca_attn_bwd(q, k_c, v_c, m, k_raw, v_raw, raw_pos0, W, sink, q_pos0, out, lse, dout, ws=None):
    """Gradients of hca_attn: (dq, dk_c, dv_c, dk_raw, dv_raw, dsink), f32."""
    B, Lq, H, D = _attn_shapes(q, k_c, v_c, k_raw, v_raw, sink, out, lse)
    _expect(dout, q.shape, "dout", dtype=q.dtype)
    if ws is None:
        ws = _ws(attn_bwd_ws_bytes(B, Lq, q_pos0, m, H, D, k_c.shape[1], 0, W), q.device)
    g = _bwd_outputs(q, k_c, k_raw, sink)
    _check(lib().hca_dense_attn_bwd(B, Lq, q_pos0, m, H, D, _kv_dtype(q), _ptr(q), k_c.shape[1], _ptr(k_c),
                                    _ptr(v_c), k_raw.shape[1], raw_pos0, _ptr(k_raw), _ptr(v_raw), W, _ptr(sink),
                                    _ptr(out), _ptr(lse), _ptr(dout), *[_ptr(x) for x in g], _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream()))
    return g
