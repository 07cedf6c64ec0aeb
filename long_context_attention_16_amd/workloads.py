"""Seeded synthetic inputs for the compressed-attention path.

This module only draws random tensors in their storage formats; it holds none
of the method's arithmetic. Both the GPU path and the CPU oracle take their
inputs from here.

Storage formats (torch dtypes):
  f32  -> torch.float32          bf16 -> torch.bfloat16
  fp8  -> torch.uint8 holding OCP e4m3fn codes
  fp4  -> torch.uint8, two e2m1 codes per byte (element 2i in the low nibble),
          plus a torch.uint8 tensor of e8m0 scales, one per 32 elements.

Workload shapes follow the pages' setting: CSA with m = 4 and k = 512..1024,
HCA with m' = 128, RoPE on the last 64 dims, a 128-token window and per-head
sinks, at 64K..1M-token contexts. Values are N(0, 1) unless stated; the gate
weights are N(0, 1/D) and the indexer head weights N(0, 1/d_I). In "exact"
indexer inputs, q_I and k_I are integers in {-2..2} and the head weights are
multiples of 2**-8 in [-1, 1], so every indexer score is exact in float32 in
any summation order and the top-k selection is exactly checkable.

Generation runs on the device given; one torch.Generator per workload, seeded,
drawing the tensors in the order they are listed in each function.
"""
from dataclasses import dataclass, field, replace

import torch


@dataclass(frozen=True)
class CSAShape:
    """Shape of one CSA or HCA attention layer call."""
    name: str
    B: int            # sequences
    Lq: int           # query tokens per sequence
    q_pos0: int       # absolute position of query row 0
    H: int            # query heads (one shared KV head)
    D: int            # head dim (last 64 rotated)
    m: int            # compression block
    N_cap: int        # compressed-cache rows per sequence
    W: int            # sliding window
    T_raw: int        # raw rows held per sequence
    raw_pos0: int     # absolute position of raw row 0
    kv: str           # 'f32' or 'bf16' (q, k, v, out)
    sink: bool = True
    # CSA only (H_I == 0 means HCA)
    H_I: int = 0
    d_I: int = 0
    topk: int = 0
    idx: str = "bf16"  # indexer format: 'f32', 'bf16', 'fp8', 'fp4'
    exact: bool = False
    # raw tokens to compress per sequence in the step (0: none)
    T_comp: int = 0
    comp_pos0: int = 0
    extra: dict = field(default_factory=dict, compare=False)


# The five workloads (plus the wide-indexer reading of the prefill chunk).
CFG1 = CSAShape("csa_prefill_L2048_f32", B=1, Lq=2048, q_pos0=0, H=4, D=128, m=4,
                N_cap=512, W=128, T_raw=2048, raw_pos0=0, kv="f32",
                H_I=4, d_I=32, topk=64, idx="f32", exact=True,
                T_comp=2048, comp_pos0=0)
CFG2 = CSAShape("csa_decode_128k_b32_bf16", B=32, Lq=1, q_pos0=131071, H=64, D=512, m=4,
                N_cap=32768, W=128, T_raw=128, raw_pos0=131071 - 127, kv="bf16",
                H_I=64, d_I=128, topk=512, idx="bf16")
CFG3 = CSAShape("csa_prefill_chunk4096_ctx64k_fp8idx", B=1, Lq=4096, q_pos0=61440, H=4, D=128,
                m=4, N_cap=16384, W=128, T_raw=65536, raw_pos0=0, kv="bf16",
                H_I=4, d_I=32, topk=1024, idx="fp8", exact=True,
                T_comp=4096, comp_pos0=61440)
CFG3M = replace(CFG3, name="csa_prefill_chunk4096_ctx64k_fp8idx_wide", H_I=64, d_I=128)
CFG4 = CSAShape("hca_decode_1m_b16_bf16", B=16, Lq=1, q_pos0=1048575, H=64, D=512, m=128,
                N_cap=8192, W=128, T_raw=128, raw_pos0=1048575 - 127, kv="bf16")
CFG5_CSA = CSAShape("pair_1m_b8_csa_fp4idx", B=8, Lq=1, q_pos0=1048575, H=64, D=512, m=4,
                    N_cap=262144, W=128, T_raw=128, raw_pos0=1048575 - 127, kv="bf16",
                    H_I=64, d_I=128, topk=1024, idx="fp4")
CFG5_HCA = replace(CFG4, name="pair_1m_b8_hca", B=8)

CONFIGS = {"1": CFG1, "2": CFG2, "3": CFG3, "3M": CFG3M, "4": CFG4, "5csa": CFG5_CSA,
           "5hca": CFG5_HCA}
SEEDS = {"1": 0, "2": 1, "3": 2, "3M": 2, "4": 3, "5csa": 4, "5hca": 5}

_KV_DT = {"f32": torch.float32, "bf16": torch.bfloat16}
# e2m1 codes of the integers -2, -1, 0, 1, 2 (sign bit 3; 1.0 = 0b010, 2.0 = 0b100)
_FP4_INT_CODES = (0xC, 0xA, 0x0, 0x2, 0x4)


def _normal(shape, gen, device, std=1.0):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * std


def _store(x, fmt):
    """Round float32 draws to a storage format (library casts only)."""
    if fmt == "f32":
        return x.contiguous()
    if fmt == "bf16":
        return x.to(torch.bfloat16).contiguous()
    if fmt == "fp8":
        return x.to(torch.float8_e4m3fn).view(torch.uint8).contiguous()
    raise ValueError(fmt)


def _int_values(shape, gen, device):
    return torch.randint(-2, 3, shape, generator=gen, device=device).to(torch.float32)


def _fp4_tensor(shape, gen, device, exact):
    """Packed e2m1 codes [..., n/2] and e8m0 scales [..., n/32]."""
    n = shape[-1]
    if exact:
        table = torch.tensor(_FP4_INT_CODES, dtype=torch.uint8, device=device)
        codes = table[torch.randint(0, 5, shape, generator=gen, device=device)]
        scales = torch.full(shape[:-1] + (n // 32,), 127, dtype=torch.uint8, device=device)
    else:
        codes = torch.randint(0, 16, shape, generator=gen, device=device).to(torch.uint8)
        scales = torch.randint(126, 129, shape[:-1] + (n // 32,), generator=gen,
                               device=device).to(torch.uint8)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).contiguous()
    return packed, scales.contiguous()


def indexer_inputs(s: CSAShape, gen, device):
    """q_I, its scales (fp4 only), w_I, k_I, its scales (fp4 only)."""
    qshape = (s.B, s.Lq, s.H_I, s.d_I)
    kshape = (s.B, s.N_cap, s.d_I)
    if s.idx == "fp4":
        q_i, q_s = _fp4_tensor(qshape, gen, device, s.exact)
        k_i, k_s = _fp4_tensor(kshape, gen, device, s.exact)
    else:
        draw = _int_values if s.exact else _normal
        q_i = _store(draw(qshape, gen, device), s.idx)
        k_i = _store(draw(kshape, gen, device), s.idx)
        q_s = k_s = None
    w = _normal((s.B, s.Lq, s.H_I), gen, device, std=(1.0 / s.d_I) ** 0.5)
    if s.exact:
        w = torch.clamp(torch.round(w * 256.0) / 256.0, -1.0, 1.0)
    return dict(q_i=q_i, q_i_scale=q_s, w_i=w.contiguous(), k_i=k_i, k_i_scale=k_s)


def make_inputs(s: CSAShape, seed: int, device="cpu"):
    """All inputs of one layer call, in storage formats, on `device`.

    Keys: q [B,Lq,H,D]; k_c, v_c [B,N_cap,D] (keys treated as already rotated);
    k_raw, v_raw [B,T_raw,D] (pre-RoPE); sink [H] f32 or None; w_gate [D] f32;
    and, for CSA, the indexer inputs of `indexer_inputs`.
    """
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    dt = s.kv
    out = {}
    out["q"] = _store(_normal((s.B, s.Lq, s.H, s.D), gen, device), dt)
    out["k_c"] = _store(_normal((s.B, s.N_cap, s.D), gen, device), dt)
    out["v_c"] = _store(_normal((s.B, s.N_cap, s.D), gen, device), dt)
    out["k_raw"] = _store(_normal((s.B, s.T_raw, s.D), gen, device), dt)
    out["v_raw"] = _store(_normal((s.B, s.T_raw, s.D), gen, device), dt)
    out["sink"] = _normal((s.H,), gen, device) if s.sink else None
    out["w_gate"] = _normal((s.D,), gen, device, std=(1.0 / s.D) ** 0.5).contiguous()
    if s.H_I:
        out.update(indexer_inputs(s, gen, device))
    return out


def chunk_index_keys(s: CSAShape, seed: int, device="cpu"):
    """Raw indexer keys [B, T_comp, d_I] of the tokens a prefill step
    compresses (KV dtype): integers in {-2..2} for exact shapes, else N(0, 1).
    Their folds become the chunk's compressed indexer keys."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed + 7919)
    draw = _int_values if s.exact else _normal
    return _store(draw((s.B, s.T_comp, s.d_I), gen, device), s.kv)


def small_shape(**kw):
    """A CSAShape for tests with defaults that fit the oracle in seconds."""
    base = dict(name="small", B=2, Lq=8, q_pos0=200, H=4, D=128, m=4, N_cap=64, W=16,
                T_raw=240, raw_pos0=0, kv="f32", H_I=4, d_I=32, topk=16, idx="f32",
                exact=True)
    base.update(kw)
    return CSAShape(**base)
