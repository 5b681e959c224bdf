"""Pins of the oracle's number formats (fp8 e4m3, e2m1 / e8m0, bfloat16).

Independent references: the OCP 8-bit floating point and Microscaling
definitions (values written out below), torch's float8_e4m3fn and bfloat16
casts (library routines), and exhaustive / boundary sweeps.
"""

import numpy as np
import pytest
import torch

from oracle import codecs


# ----------------------------------------------------------------------------
# e4m3
# ----------------------------------------------------------------------------

# (code, value) points fixed by the OCP E4M3FN definition.
OCP_E4M3_POINTS = [
    (0x00, 0.0), (0x80, -0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9),
    (0x08, 2.0 ** -6), (0x38, 1.0), (0x39, 1.125), (0x3F, 1.875), (0x40, 2.0),
    (0x7E, 448.0), (0xFE, -448.0), (0x77, 240.0), (0x70, 128.0), (0xB8, -1.0),
]


def check_e4m3_decode(decode=codecs.e4m3_decode):
    for code, value in OCP_E4M3_POINTS:
        got = decode(np.array([code], dtype=np.uint8))[0]
        assert got == value and np.signbit(got) == np.signbit(value), (hex(code), got, value)
    assert np.isnan(decode(np.array([0x7F, 0xFF], dtype=np.uint8))).all()
    # every code against torch's float8_e4m3fn decode
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = decode(codes)
    same = (mine == ref) | (np.isnan(mine) & np.isnan(ref))
    assert same.all()


def test_e4m3_decode():
    check_e4m3_decode()


def torch_e4m3(v32):
    """torch's cast of clamp(v, +-448): round-half-even with saturation."""
    t = torch.from_numpy(np.asarray(v32, dtype=np.float32)).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def boundary_values():
    """Every midpoint between adjacent e4m3 values, one binary32 ulp either side,
    every e4m3 value and its neighbours, both signs, plus out-of-range values."""
    pos = codecs.e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float32)
    mids = ((pos[:-1].astype(np.float64) + pos[1:]) / 2).astype(np.float32)
    pts = np.concatenate([pos, mids, [449.0, 464.0, 465.0, 1e6, 3e38]]).astype(np.float32)
    up = np.nextafter(pts, np.float32(np.inf))
    dn = np.nextafter(pts, np.float32(0))
    allp = np.concatenate([pts, up, dn]).astype(np.float32)
    return np.concatenate([allp, -allp]).astype(np.float32)


def check_e4m3_encode(encode=codecs.e4m3_encode):
    v = boundary_values()
    assert (encode(v) == torch_e4m3(v)).all()
    rng = np.random.default_rng(1)
    for scale in (1e-4, 1e-2, 1.0, 30.0, 300.0):
        r = (rng.standard_normal(200_000) * scale).astype(np.float32)
        assert (encode(r) == torch_e4m3(r)).all(), scale


def test_e4m3_encode_matches_torch():
    check_e4m3_encode()


def test_e4m3_encode_full_binade_sweep():
    # All binary32 values of two whole binades (one normal, one subnormal for e4m3).
    for lo in (1.0, 2.0 ** -8):
        a = np.float32(lo).view(np.uint32)
        b = np.float32(2 * lo).view(np.uint32)
        v = np.arange(a, b, 7, dtype=np.uint32).view(np.float32)
        assert (codecs.e4m3_encode(v) == torch_e4m3(v)).all()


def test_e4m3_signed_zero_and_saturation():
    v = np.array([0.0, -0.0, 1e9, -1e9, 448.0, 463.99, 464.0], dtype=np.float32)
    assert list(codecs.e4m3_encode(v)) == [0x00, 0x80, 0x7E, 0xFE, 0x7E, 0x7E, 0x7E]


def test_e4m3_roundtrip():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert (codecs.e4m3_encode(codecs.e4m3_decode(codes)) == codes).all()


# ----------------------------------------------------------------------------
# e2m1 / e8m0 / MXFP4
# ----------------------------------------------------------------------------


def test_e2m1_table_and_sign():
    # OCP MX: E2M1 magnitudes for codes 0..7, bit 3 is the sign.
    expect = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = codecs.e2m1_decode(np.arange(16, dtype=np.uint8))
    assert list(got[:8]) == expect
    assert list(got[8:]) == [-x for x in expect]
    assert np.signbit(got[8])


def check_nibble_order(unpack=codecs.e2m1_unpack):
    # Byte 0x21 holds element 0 = code 1 (low nibble) and element 1 = code 2.
    p = np.array([[0x21, 0xF7]], dtype=np.uint8)
    assert list(unpack(p)[0]) == [1, 2, 7, 15]


def test_nibble_order():
    check_nibble_order()


def test_mxfp4_decode_nibbles():
    # Every byte through mxfp4_decode: element 2i is the low nibble's value
    # (OCP E2M1 magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6; bit 3 the sign), element
    # 2i + 1 the high nibble's, times the block scale 2^(b - 127).
    mag = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    val = lambda c: -mag[c & 7] if c & 8 else mag[c & 7]  # noqa: E731
    packed = np.arange(256, dtype=np.uint8).reshape(16, 16)     # 16 rows of K = 32
    for b, f in ((127, 1.0), (125, 0.25)):
        w = codecs.mxfp4_decode(packed, np.full((16, 1), b, dtype=np.uint8))
        want = np.array([[val(int(x) & 15) * f, val(int(x) >> 4) * f] for x in range(256)]).reshape(16, 32)
        assert np.array_equal(w, want)
    # 0x21: element 0 = code 1 = 0.5, element 1 = code 2 = 1.0; 0xF7: 6, -6
    w = codecs.mxfp4_decode(np.array([[0x21, 0xF7] * 16], dtype=np.uint8), np.array([[127, 127]], dtype=np.uint8))
    assert list(w[0, :4]) == [0.5, 1.0, 6.0, -6.0]


def test_e8m0():
    assert list(codecs.e8m0_decode(np.array([127, 128, 126, 0, 254]))) == [1.0, 2.0, 0.5, 2.0 ** -127, 2.0 ** 127]
    with pytest.raises(ValueError):
        codecs.e8m0_decode(np.array([255]))


def test_mxfp4_block_axis():
    # One output row, K = 64: scale of block 1 only touches elements 32..63.
    codes = np.full((1, 64), 2, dtype=np.uint8)                   # value 1.0
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    scales = np.array([[127, 129]], dtype=np.uint8)               # 1, 4
    w = codecs.mxfp4_decode(packed, scales)
    assert (w[0, :32] == 1.0).all() and (w[0, 32:] == 4.0).all()


# ----------------------------------------------------------------------------
# bfloat16
# ----------------------------------------------------------------------------


def check_bf16_encode(encode=codecs.bf16_encode):
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.standard_normal(100_000) * 10.0 ** rng.integers(-30, 30, 100_000),
                        [0.0, -0.0, 1.0, -1.0, 3e38, 1e-40]]).astype(np.float32)
    # binary32 inputs: torch's float32 -> bfloat16 cast (round-half-even)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (encode(v.astype(np.float64)) == ref).all()
    # exact bf16 ties round to even
    ties = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8], dtype=np.float64)
    assert list(encode(ties)) == [0x3F80, 0x3F82]
    # a float64 just above a tie rounds up (a single rounding, not via binary32)
    assert encode(np.array([1.0 + 2.0 ** -8 + 2.0 ** -40]))[0] == 0x3F81


def test_bf16_encode():
    check_bf16_encode()


def test_bf16_decode():
    bits = np.array([0x3F80, 0xBF80, 0x4000, 0x0000, 0x8000, 0x7F7F], dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert (codecs.bf16_decode(bits) == ref).all()
