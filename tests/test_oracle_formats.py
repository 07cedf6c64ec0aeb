"""Pins of the oracle's format decoders against torch's CPU casts (an
independent implementation) over every code, and against the OCP e2m1 table."""
import os

import numpy as np
import torch

from oracle import formats

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _same(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert np.array_equal(np.isnan(a), np.isnan(b))
    m = ~np.isnan(a)
    assert np.array_equal(a[m], b[m])
    # sign of zero too
    assert np.array_equal(np.signbit(a[m]), np.signbit(b[m]))


def test_bf16_all_codes():
    codes = np.arange(1 << 16, dtype=np.uint16)
    ref = torch.from_numpy(codes.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    _same(formats.bf16_to_f64(codes), ref)


def test_e4m3fn_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    _same(formats.e4m3fn_to_f64(codes), ref)
    assert formats.e4m3fn_to_f64(np.uint8(0x7E)) == 448.0


def test_e8m0_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e8m0fnu).double().numpy()
    _same(formats.e8m0_to_f64(codes), ref)


def test_e2m1_table():
    rows = [l.split() for l in open(os.path.join(GOLD, "e2m1_ocp_mx.txt")) if l.strip() and not l.startswith("#")]
    codes = np.array([int(r[0]) for r in rows])
    vals = np.array([float(r[1]) for r in rows])
    _same(formats.e2m1_to_f64(codes), vals)


def test_fp4_nibble_order_and_scale():
    # byte 0x21: element 0 = low nibble = code 1 (0.5), element 1 = code 2 (1.0)
    packed = np.zeros((1, 16), dtype=np.uint8)
    packed[0, 0] = 0x21
    packed[0, 15] = 0xF7          # element 30 = code 7 (6.0), 31 = code 15 (-6.0)
    v = formats.mxfp4_to_f64(packed, np.array([[129]], dtype=np.uint8))
    assert v[0, 0] == 2.0 and v[0, 1] == 4.0
    assert v[0, 30] == 24.0 and v[0, 31] == -24.0
    assert np.all(v[0, 2:30] == 0.0)


def test_mxfp4_to_e4m3_lossless():
    """FP4 values times any power-of-two scale that stays in e4m3's range are
    exactly representable in e4m3fn: the dequantisation loses nothing."""
    codes = np.arange(16)
    base = formats.e2m1_to_f64(codes)
    for e in range(-8, 7):        # 0.5 * 2^-8 is e4m3's smallest subnormal; 6 * 2^6 <= 448
        v = base * 2.0 ** e
        t = torch.from_numpy(v).to(torch.float8_e4m3fn).double().numpy()
        _same(t, v)
    # one step below the range the smallest magnitude is lost, as expected
    v = base * 2.0 ** -9
    t = torch.from_numpy(v).to(torch.float8_e4m3fn).double().numpy()
    assert not np.array_equal(t, v)
