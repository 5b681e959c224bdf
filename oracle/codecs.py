"""Number formats used by the layer, written out from their definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* fp8 e4m3 ("E4M3FN" of the OCP 8-bit floating point specification):
  1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
  holds subnormals m * 2^-9; the pattern S.1111.111 is NaN; there is no
  infinity; the largest finite magnitude is 448.  The pages name only "fp8"
  for weights and for the per-token activation quantisation
  (*Ling-2.6-1T on TPU*, §5 "activation quantisation" and
  "per-channel direct_scaled_dot"); the scale amax/448 fixes this variant.
* fp4 e2m1 with an e8m0 block scale (OCP Microscaling "MXFP4"): two e2m1
  values per byte and one power-of-two scale byte per 32 elements
  (*sglang-jax gap list*, §4 MXFP4; *Kimi K3 on TPU*, §2.5 quantisation,
  group size 32, uint8 scales, 4.25 bits per element).
* bfloat16: the upper 16 bits of an IEEE binary32.

Encoders choose the nearest representable value and break exact ties toward
the code with an even mantissa (round-half-to-even), saturating at the largest
finite magnitude.  They are written as "nearest entry of the decode table",
i.e. the definition, not as bit tricks.
"""

import numpy as np

# ----------------------------------------------------------------------------
# fp8 e4m3 (OCP E4M3FN)
# ----------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_decode_table():
    """Value of each of the 256 codes (float64; NaN for the two NaN codes)."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = sign * m * 2.0 ** -9
        else:
            vals[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3 = e4m3_decode_table()
# Non-negative finite codes 0x00..0x7E have strictly increasing values.
_E4M3_POS = _E4M3[:0x7F].copy()


def e4m3_decode(codes):
    """uint8 codes -> float64 values."""
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def _nearest_code(mag, table):
    """Index of the nearest entry of an increasing table, ties to the even index.

    ``mag`` must be non-negative and not above ``table[-1]``.  The differences
    below are exact in float64 for binary32 inputs and these tables.
    """
    hi = np.searchsorted(table, mag, side="left")  # table[hi-1] < mag <= table[hi]
    hi = np.minimum(hi, len(table) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - table[lo]
    d_hi = table[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(mag == table[hi], hi, idx)
    return idx


def e4m3_encode(values):
    """Round values (float32 or float64, finite) to e4m3 codes (uint8).

    Round to nearest, ties to even mantissa, saturate at +-448, keep the sign
    of zero (-0.0 encodes as 0x80).
    """
    v = np.asarray(values, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("e4m3_encode: NaN input")
    neg = np.signbit(v)
    mag = np.minimum(np.abs(v), E4M3_MAX)
    idx = _nearest_code(mag, _E4M3_POS).astype(np.uint8)
    return np.where(neg, idx | np.uint8(0x80), idx).astype(np.uint8)


# ----------------------------------------------------------------------------
# fp4 e2m1 and e8m0 (OCP MX)
# ----------------------------------------------------------------------------

E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def e2m1_decode(nibbles):
    """4-bit codes (values 0..15) -> float64.  Bit 3 is the sign."""
    n = np.asarray(nibbles, dtype=np.uint8)
    mag = E2M1_MAG[n & 0x7]
    return np.where(n & 0x8, -mag, mag)


def e2m1_unpack(packed):
    """uint8 [..., K/2] -> nibble codes [..., K]; element 2i is the low nibble."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def e8m0_decode(scales):
    """uint8 biased exponents -> 2^(b-127) as float64.  255 (NaN) is rejected."""
    b = np.asarray(scales, dtype=np.int64)
    if (b == 255).any():
        raise ValueError("e8m0 scale 255 is NaN")
    return np.ldexp(1.0, b - 127)


# byte b -> (value of its low nibble, value of its high nibble): the two
# elements one packed byte holds, in element order
_E2M1_PAIRS = np.stack([e2m1_decode(np.arange(256) & 0xF), e2m1_decode(np.arange(256) >> 4)], axis=-1)


def mxfp4_decode(packed, scales, group=32):
    """MXFP4 matrix [N][K/2] + scales [N][K/group] -> float64 [N][K]."""
    p = np.asarray(packed, dtype=np.uint8)
    vals = _E2M1_PAIRS[p].reshape(p.shape[:-1] + (p.shape[-1] * 2,))   # = e2m1_decode(e2m1_unpack(p))
    sc = e8m0_decode(scales)
    k = vals.shape[-1]
    blocks = vals.reshape(vals.shape[:-1] + (k // group, group))        # a view of vals
    blocks *= sc[..., None]                                             # each element times its block's scale
    return vals


# ----------------------------------------------------------------------------
# bfloat16
# ----------------------------------------------------------------------------


def bf16_decode(bits):
    """uint16 bfloat16 bit patterns -> float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_encode(values):
    """float64 values -> nearest bfloat16 (ties to even), as uint16 bits.

    Rounds once, straight from float64 (no intermediate binary32).  Finite
    results only; magnitudes beyond the bfloat16 range become +-inf.
    """
    v = np.asarray(values, dtype=np.float64)
    out = np.zeros(v.shape, dtype=np.float64)
    nz = (v != 0) & np.isfinite(v)
    m, e = np.frexp(v[nz])            # v = m * 2^e, 0.5 <= |m| < 1
    # bfloat16 keeps 8 significant bits; below 2^-126 the grid is fixed 2^-133.
    step_exp = np.maximum(e - 8, -133)
    q = np.rint(np.ldexp(v[nz], -step_exp))   # half-to-even
    out[nz] = np.ldexp(q, step_exp)
    out[~np.isfinite(v)] = v[~np.isfinite(v)]
    out = np.where(np.signbit(v) & (out == 0), -0.0, out)
    with np.errstate(over="ignore"):
        f32 = out.astype(np.float32)    # exact: every bf16 value is a binary32 value
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
