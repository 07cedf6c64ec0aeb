"""Exact decoders of the storage formats the GPU path reads (oracle; test
infrastructure only).

bf16      : the upper 16 bits of an IEEE binary32.
e4m3fn    : OCP 8-bit float, 1 sign, 4 exponent (bias 7), 3 mantissa bits,
            subnormals, no infinities, S.1111.111 is NaN, max 448.
e2m1      : OCP 4-bit float, 1 sign, 2 exponent (bias 1), 1 mantissa bit;
            magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
e8m0      : OCP MX shared scale, 2**(E-127); E = 255 is NaN.
MXFP4     : e2m1 elements, two per byte (element 2i in the low nibble), one
            e8m0 scale per 32 consecutive elements along the last dimension.

Encoders (for compressed indexer keys written in these formats):
  e4m3fn : round to nearest, ties to the even code (mantissa LSB 0), every
           magnitude above 448 saturating to 448; the sign is kept (-0.0 for
           negative values that round to zero).
  MXFP4  : per 32 consecutive elements, amax = max |x|; the e8m0 code is
           floor(log2 amax) - 2 + 127 clamped to 0..254 (0 when amax = 0), i.e.
           the OCP MX rule that puts amax at 4..8 times the scale (e2m1's largest
           exponent is 2); elements x / scale round to nearest e2m1, ties to the
           even code, saturating at 6; the sign bit is x's (-0.0 -> code 8).

Why these formats: [P1] section FP4 量化 says the indexer's QK path runs in FP4
and that dequantising FP4 to FP8 loses nothing because fine-grained sub-block
scales fit in FP8's range. A power-of-two (e8m0) scale makes that statement
exactly true for e2m1 -> e4m3, which is why MXFP4 is the reading taken.
"""
import numpy as np


def bf16_to_f64(bits):
    """uint16 bf16 bit patterns -> float64 (exact)."""
    u = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def e4m3fn_to_f64(bits):
    """uint8 OCP e4m3fn codes -> float64 (exact; NaN code -> nan)."""
    b = np.asarray(bits).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    mant = (b & 0x7).astype(np.float64)
    normal = (1.0 + mant / 8.0) * np.ldexp(1.0, (e - 7).astype(np.int64))
    sub = (mant / 8.0) * 2.0 ** -6
    v = np.where(e == 0, sub, normal)
    v = np.where((e == 15) & ((b & 7) == 7), np.nan, v)
    return sign * v


def e2m1_to_f64(codes):
    """4-bit e2m1 codes (0..15, one per array element) -> float64 (exact)."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    mant = (c & 0x1).astype(np.float64)
    normal = (1.0 + mant / 2.0) * np.ldexp(1.0, (e - 1).astype(np.int64))
    sub = mant * 0.5
    return sign * np.where(e == 0, sub, normal)


def e8m0_to_f64(bits):
    """uint8 e8m0 scale codes -> float64 powers of two (255 -> nan)."""
    b = np.asarray(bits).astype(np.int64)
    v = np.ldexp(1.0, b - 127)
    return np.where(b == 255, np.nan, v)


def unpack_fp4(packed):
    """[..., n/2] uint8 -> [..., n] e2m1 codes; element 2i is the low nibble."""
    p = np.asarray(packed).astype(np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def mxfp4_to_f64(packed, scales):
    """MXFP4 tensor -> float64.

    packed: [..., n/2] uint8 (two e2m1 codes per byte); scales: [..., n/32]
    uint8 e8m0. Element i of a row is e2m1(code_i) * 2**(scale[i // 32] - 127).
    """
    vals = e2m1_to_f64(unpack_fp4(packed))
    s = e8m0_to_f64(scales)
    n = vals.shape[-1]
    assert s.shape[-1] * 32 == n, "one e8m0 scale per 32 elements"
    return vals * np.repeat(s, 32, axis=-1)


def f32_to_f64(x):
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def decode(arr, fmt, scales=None):
    """Decode a storage array by format name: 'f32', 'bf16', 'fp8', 'fp4'."""
    if fmt == "f32":
        return f32_to_f64(arr)
    if fmt == "bf16":
        return bf16_to_f64(np.asarray(arr).view(np.uint16))
    if fmt == "fp8":
        return e4m3fn_to_f64(np.asarray(arr).view(np.uint8))
    if fmt == "fp4":
        assert scales is not None
        return mxfp4_to_f64(np.asarray(arr).view(np.uint8), np.asarray(scales).view(np.uint8))
    raise ValueError(fmt)


# ------------------------------------------------------------------ encoders
def f64_to_bf16(x):
    """float64 -> uint16 bf16 bit patterns, round to nearest even (finite x).

    The value's binade has 8 significant bits in bf16 (7 stored), so x is
    rounded to a multiple of 2**(e-7), e = floor(log2 |x|), with np.rint
    (ties to even); below the smallest normal (2**-126) the step is 2**-133.
    The rounded value is then exactly a float32 whose upper 16 bits are the
    code.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e2 = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(e2 - 1, -126)
    step = np.ldexp(1.0, (e - 7).astype(np.int64))
    q = np.copysign(np.rint(a / step) * step, x)
    return (q.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def round_bf16(x):
    """float64 rounded to the nearest bf16 value (ties to even), as float64."""
    return bf16_to_f64(f64_to_bf16(x))


_E4M3_MAX = 448.0


def f64_to_e4m3fn(x):
    """float64 -> uint8 OCP e4m3fn codes (round to nearest even, saturating).

    Works on the value's binary exponent: a normal result has 3 mantissa
    bits below the leading one, so x is rounded to a multiple of 2**(e-3),
    e = floor(log2 |x|); below 2**-6 the grid is the subnormal step 2**-9.
    """
    x = np.asarray(x, dtype=np.float64)
    assert not np.any(np.isnan(x)), "NaN has no saturating encoding here"
    a = np.minimum(np.abs(x), _E4M3_MAX)
    _, e2 = np.frexp(np.where(a > 0, a, 1.0))       # a = f * 2**e2, f in [0.5, 1)
    e = np.maximum(e2 - 1, -6)                       # exponent of the grid (subnormals share -6)
    step = np.ldexp(1.0, (e - 3).astype(np.int64))
    q = np.rint(a / step) * step                     # np.rint: ties to even multiple of step
    q = np.minimum(q, _E4M3_MAX)
    # encode the rounded magnitude q exactly
    _, qe2 = np.frexp(np.where(q > 0, q, 1.0))
    qe = qe2 - 1
    normal = q >= 2.0 ** -6
    mant_n = np.rint((q / np.ldexp(1.0, qe.astype(np.int64)) - 1.0) * 8).astype(np.int64)
    code_n = ((qe + 7).astype(np.int64) << 3) | mant_n
    code_s = np.rint(q / 2.0 ** -9).astype(np.int64)
    code = np.where(normal, code_n, code_s)
    sign = np.where(np.signbit(x), 0x80, 0)
    return (code | sign).astype(np.uint8)


_E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def f64_to_e2m1(x):
    """float64 (already divided by its scale) -> e2m1 codes 0..15, nearest,
    ties to the even code, saturating at 6; bit 3 = sign bit of x."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    # distance to every magnitude; ties resolved toward the even code (the
    # codes are in value order, so the candidates of a tie differ by one)
    d = np.abs(a[..., None] - _E2M1_VALUES)
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    codes = np.arange(8)
    even_pick = np.where(cand & (codes % 2 == 0), codes, 99).min(axis=-1)
    any_pick = np.where(cand, codes, 99).min(axis=-1)
    c = np.where(even_pick < 99, even_pick, any_pick)
    sign = np.where(np.signbit(x), 8, 0)
    return (c | sign).astype(np.uint8)


def f64_to_mxfp4(x):
    """[..., n] float64 (n a multiple of 32) -> (packed [..., n/2] uint8,
    scales [..., n/32] uint8 e8m0), element 2i in the low nibble."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    assert n % 32 == 0
    blocks = x.reshape(x.shape[:-1] + (n // 32, 32))
    amax = np.abs(blocks).max(axis=-1)
    _, e2 = np.frexp(np.where(amax > 0, amax, 1.0))
    code = np.where(amax > 0, np.clip(e2 - 1 - 2 + 127, 0, 254), 0).astype(np.int64)
    scale = np.ldexp(1.0, code - 127)
    el = f64_to_e2m1(blocks / scale[..., None]).reshape(x.shape)
    packed = (el[..., 0::2] | (el[..., 1::2] << 4)).astype(np.uint8)
    return packed, code.astype(np.uint8)
