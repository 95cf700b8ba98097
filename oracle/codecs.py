"""Number-format codecs, written from the format definitions (oracle only).

Encoders are value based: a finite input is snapped to the format's grid
(quantum 2**(max(floor(log2|x|), e_min) - mantissa_bits)) with round to
nearest, ties to even, evaluated exactly in fp64; the bit fields are then
written out from the snapped value.  Decoders evaluate the field formula.

Formats:
* bf16  -- 1 sign, 8 exponent (bias 127), 7 mantissa bits; subnormals kept.
* fp16  -- IEEE binary16: 1, 5 (bias 15), 10; subnormals; max 65504.
* E4M3  -- the OCP 8-bit "E4M3FN" float used for the FP8 base: 1, 4 (bias 7),
  3 bits; subnormals 2**-6 * m/8; no infinities; only S.1111.111 is NaN, so
  the largest finite magnitude is 448.  Encoding saturates to +-448.
* E2M1  -- the 4-bit float element of the OCP Microscaling (MX) formats and of
  NVFP4: 1 sign, 2 exponent (bias 1), 1 mantissa bit; exponent field 0 is
  subnormal (0.5 * m); no infinities or NaN, so the largest magnitude is 6.
  Encoding saturates to +-6.
"""

import numpy as np


def _snap(x64, e_min, mant_bits):
    """Round fp64 values to the grid of a binary format, ties to even (exact)."""
    _, e = np.frexp(x64)  # x = f * 2**e with 0.5 <= |f| < 1, so floor(log2|x|) = e - 1
    e = np.maximum(e.astype(np.int64) - 1, e_min)
    quantum = np.ldexp(1.0, (e - mant_bits).astype(np.int32))
    return np.rint(x64 / quantum) * quantum


def _fields(v64, bias, mant_bits, e_min):
    """Biased exponent and mantissa fields of values already on the grid."""
    a = np.abs(v64)
    _, e = np.frexp(a)
    e = e.astype(np.int64) - 1
    normal = a >= np.ldexp(1.0, e_min)
    ebits = np.where(normal, e + bias, 0)
    scale_e = np.where(normal, e, e_min).astype(np.int32)
    frac = a / np.ldexp(1.0, scale_e)  # in [1, 2) for normals, [0, 1) for subnormals
    mbits = np.rint(np.where(normal, frac - 1.0, frac) * (1 << mant_bits))
    ebits = np.where(a == 0, 0, ebits)
    return ebits.astype(np.int64), mbits.astype(np.int64)


# ----------------------------------------------------------------------------- bf16

def bf16_encode(x):
    """fp32 values -> bf16 bit patterns (uint16), round to nearest even."""
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    r = _snap(x64, -126, 7)
    out = np.empty(x64.shape, dtype=np.uint16)
    fin = np.isfinite(x64)
    over = fin & (np.abs(r) >= 2.0 ** 128)
    r32 = np.where(fin & ~over, r, 0.0).astype(np.float32)
    out[...] = (r32.view(np.uint32) >> 16).astype(np.uint16)
    sign = np.signbit(x64).astype(np.uint16) << 15
    inf_bits = sign | np.uint16(0x7F80)
    out = np.where(over | np.isinf(x64), inf_bits, out)
    out = np.where(np.isnan(x64), np.uint16(0x7FC0), out)
    return out.astype(np.uint16)


def bf16_decode(bits):
    """bf16 bit patterns -> fp32 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def bf16_round(x):
    """fp32 -> nearest bf16 value, returned as fp32."""
    return bf16_decode(bf16_encode(x))


# ----------------------------------------------------------------------------- fp16

def fp16_encode(x):
    """fp32 values -> IEEE binary16 bit patterns, round to nearest even.

    Returns (bits, overflowed): a finite input whose rounded value exceeds
    65504 in magnitude is flagged (and encoded as infinity).
    """
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    fin = np.isfinite(x64)
    r = np.where(fin, _snap(np.where(fin, x64, 0.0), -14, 10), 0.0)
    over = fin & (np.abs(r) > 65504.0)
    r = np.where(over, 0.0, r)
    ebits, mbits = _fields(r, 15, 10, -14)
    sign = np.signbit(x64).astype(np.int64)
    bits = (sign << 15) | (ebits << 10) | mbits
    bits = np.where(over | np.isinf(x64), (sign << 15) | 0x7C00, bits)
    bits = np.where(np.isnan(x64), 0x7E00, bits)
    return bits.astype(np.uint16), over


def fp16_decode(bits):
    """IEEE binary16 bit patterns -> fp32 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    s = np.where((b >> 15) & 1, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    m = (b & 0x3FF).astype(np.float64)
    val = np.where(e == 0, m * 2.0 ** -24,
                   (1.0 + m / 1024.0) * np.ldexp(1.0, (e - 15).astype(np.int32)))
    val = np.where(e == 31, np.where(m == 0, np.inf, np.nan), val)
    return (s * val).astype(np.float32)


# ----------------------------------------------------------------------------- E4M3

E4M3_MAX = 448.0


def e4m3_encode(x):
    """fp32 values -> OCP E4M3FN codes (uint8): nearest even, saturating to +-448.

    Zero keeps its sign (-0.0 -> 0x80; a negative value that rounds to zero is
    0x80 too).  NaN -> 0x7F.  Infinities saturate like any large value.
    """
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    fin = np.isfinite(x64)
    xx = np.where(fin, x64, np.copysign(E4M3_MAX, x64))
    r = _snap(xx, -6, 3)
    r = np.clip(r, -E4M3_MAX, E4M3_MAX)
    ebits, mbits = _fields(r, 7, 3, -6)
    sign = np.signbit(x64).astype(np.int64)
    bits = (sign << 7) | (ebits << 3) | mbits
    bits = np.where(np.isnan(x64), 0x7F, bits)
    return bits.astype(np.uint8)


def e4m3_decode(codes):
    """OCP E4M3FN codes -> fp32 values (exact); S.1111.111 -> NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6,
                   (1.0 + m / 8.0) * np.ldexp(1.0, (e - 7).astype(np.int32)))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return (s * val).astype(np.float32)


# ----------------------------------------------------------------------------- E2M1

E2M1_MAX = 6.0


def e2m1_encode(x):
    """Real values (fp32 or fp64) -> E2M1 codes (uint8, 0..15): nearest, ties to
    even, saturating to +-6.

    The sign bit is the input's sign bit, so a negative value that rounds to
    zero gives 0x8 (negative zero).  Inputs must be finite.
    """
    x64 = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x64)):
        raise ValueError("E2M1 encode of a non-finite value")
    r = np.clip(_snap(x64, 0, 1), -E2M1_MAX, E2M1_MAX)
    ebits, mbits = _fields(r, 1, 1, 0)
    sign = np.signbit(x64).astype(np.int64)
    return ((sign << 3) | (ebits << 1) | mbits).astype(np.uint8)


def e2m1_decode(codes):
    """E2M1 codes (low 4 bits) -> fp32 values (exact)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64) & 0xF
    s = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 0x1).astype(np.float64)
    val = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.ldexp(1.0, (e - 1).astype(np.int32)))
    return (s * val).astype(np.float32)
