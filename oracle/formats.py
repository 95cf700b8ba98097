"""Base-weight formats: NF4 code book, pack and dequant (oracle only).

The base weight W is fp32 [N, K] (row n = output feature, K = input features,
the nn.Linear convention).  Blocks run along K.  Packing decisions are taken
in IEEE fp32 (numpy float32 arithmetic is correctly rounded), ties to even.

4-bit code layout (Q4_0-style and NF4): each row's codes are cut into groups
of 32 consecutive elements; a group occupies 16 bytes, and byte j of the group
holds element j in its low nibble and element j + 16 in its high nibble.
Codes are u8 [N, K/2]; scales are a separate array (structure of arrays).

MXFP4 codes use the other common 4-bit packing: byte i of a row holds element
2i in its low nibble and element 2i + 1 in its high nibble.

Formats (the legacy-GGUF 4-bit type that the GGUF-recipe page names, the
bitsandbytes NF4 base named on the Surogate pages and the Soup page, the
FP8 E4M3 base of the Surogate FP8 recipe, and the FP4 base behind the
Surogate pages' NVFP4 (E2M1) recipes and MXFP4 checkpoints):

* Q4_0-style: block of 32, fp16 scale d = fp16(absmax / 7), code
  q = clamp(rint(w / d) + 8, 0, 15), value (q - 8) * d.  A zero block stores
  code 8 everywhere.
* NF4: block of 64, fp32 scale a = absmax, code = index of the nearest entry
  of the 16-level code book (ties go to the lower code), value c[q] * a.  A
  zero block stores code 7 (the exact zero of the book).  No double
  quantization.
* FP8: per-tensor fp32 scale s = absmax / 448, code = E4M3(w / s) with
  saturation; value E4M3(q) * s.  A zero tensor has s = 0 and codes 0.
* Q8_0-style (the 8-bit member of the same legacy GGUF family; the plain
  reading of "GGUF Q8_0", which the GGUF-recipe page names as a base but does
  not define): block of 32, fp16 scale d = fp16(absmax / 127), code
  q = clamp(rint(w / d), -127, 127) (ties to even), stored as a two's
  complement byte, one per element (u8 [N, K]); value q * d, exact in fp32.
  A zero block stores d = 0 and codes 0.  While d is a normal fp16 number
  |w / d| <= 127 (1 + 2**-11), so the clamp acts only on blocks whose scale
  rounded down to an fp16 subnormal; -128 is never written, and dequant still
  accepts it.
* MXFP4 (the OCP Microscaling definition, which the pages name but do not
  spell out): block of 32, one E8M0 scale byte e per block standing for
  X = 2**(e - 127); X = 2**(floor(log2 absmax) - 2), the exponent clamped to
  [-127, 127] (2 is the largest exponent of E2M1), so the block's largest
  magnitude lands in [4, 8) before saturation; element code = E2M1(w / X),
  nearest even, saturating to +-6; value E2M1(q) * X, exact in fp32 and bf16.
  A zero block stores e = 0 and codes 0.  e = 255 (NaN in E8M0) is never
  written and decodes to NaN.
* NVFP4 (the FP4 format of the Surogate pages' Blackwell recipe, "NVFP4
  (E2M1)" in the review page's highlights; the pages name it without
  defining it, and the reading taken is NVIDIA's published structure): E2M1
  element codes in blocks of 16, one E4M3 scale byte per block and one fp32
  scale per tensor.  Decisions:
    g   = fl32(amax / 2688)            the tensor scale (2688 = 6 * 448, the
                                       largest E2M1 magnitude times the
                                       largest E4M3 one)
    sb  = E4M3(fl32(fl32(amax_b / 6) / g))   per block, nearest even,
                                       saturating at 448; 0 when g = 0
    X_b = fl32(E4M3(sb) * g)           the block's decode scale
    q   = the E2M1 value nearest to the exact quotient w / X_b, ties to the
          even mantissa, saturating at +-6, sign bit from w; 0 when X_b = 0
  and the value is fl32(E2M1(q) * X_b).  Codes use the split-nibble groups of
  32 of Q4_0 and NF4, so a group's low nibbles are one block of 16 and its
  high nibbles the next.  The stored scale image is 16 header bytes (g's
  fp32 bits little-endian, then 12 zero bytes) followed by the E4M3 bytes
  u8 [N, K/16].  A zero tensor stores g = 0, zero scales and zero codes.
"""

import statistics

import numpy as np

from . import codecs

FMT_Q4_0, FMT_NF4, FMT_FP8, FMT_MXFP4, FMT_Q8_0, FMT_NVFP4 = 1, 2, 3, 4, 5, 6
BLOCK = {FMT_Q4_0: 32, FMT_NF4: 64, FMT_MXFP4: 32, FMT_Q8_0: 32, FMT_NVFP4: 16}


# ----------------------------------------------------------------------------- NF4 book

def nf4_codebook_f64(inv_cdf=None):
    """The 16 NF4 levels in fp64 (QLoRA paper, section "4-bit NormalFloat").

    The levels are quantiles of N(0, 1): 8 for the positive half and 7 for the
    negative half, taken at equally spaced probabilities from an offset delta
    down to 1/2 (the 1/2 endpoint, i.e. zero, is dropped from each half and a
    single exact zero is added), then normalised so the largest magnitude is 1.
    delta is the mean of 1 - 1/(2*15) and 1 - 1/(2*16), the two outermost
    quantile positions for 15 and 16 levels.
    """
    if inv_cdf is None:
        inv_cdf = statistics.NormalDist().inv_cdf
    delta = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0))
    pos = [inv_cdf(delta - i * (delta - 0.5) / 8.0) for i in range(8)]
    neg = [-inv_cdf(delta - i * (delta - 0.5) / 7.0) for i in range(7)]
    levels = sorted(pos + neg + [0.0])
    top = max(abs(v) for v in levels)
    return np.array([v / top for v in levels], dtype=np.float64)


def nf4_codebook(inv_cdf=None):
    """NF4 levels rounded once to fp32."""
    return nf4_codebook_f64(inv_cdf).astype(np.float32)


def nf4_thresholds(book=None):
    """Decision thresholds m_i = fl32(fl32(c_i + c_{i+1}) * 0.5), i = 0..14."""
    c = nf4_codebook() if book is None else np.asarray(book, np.float32)
    return ((c[:-1] + c[1:]) * np.float32(0.5)).astype(np.float32)


# ----------------------------------------------------------------------------- nibbles

def nibbles_to_bytes(q):
    """Codes u8 [N, K] (values 0..15) -> packed bytes u8 [N, K/2], split-half groups of 32."""
    q = np.asarray(q, dtype=np.uint8)
    n, k = q.shape
    assert k % 32 == 0
    g = q.reshape(n, k // 32, 32)
    lo, hi = g[:, :, :16], g[:, :, 16:]
    return (lo | (hi << 4)).astype(np.uint8).reshape(n, k // 2)


def bytes_to_nibbles(b):
    """Packed bytes u8 [N, K/2] -> codes u8 [N, K]."""
    b = np.asarray(b, dtype=np.uint8)
    n, kh = b.shape
    g = b.reshape(n, kh // 16, 16)
    q = np.concatenate([g & 0x0F, g >> 4], axis=2)
    return q.reshape(n, kh * 2).astype(np.uint8)


def pairs_to_bytes(q):
    """Codes u8 [N, K] (values 0..15) -> packed bytes u8 [N, K/2]: element 2i low, 2i + 1 high."""
    q = np.asarray(q, dtype=np.uint8)
    n, k = q.shape
    assert k % 2 == 0
    return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)


def bytes_to_pairs(b):
    """Packed bytes u8 [N, K/2] -> codes u8 [N, K] (inverse of pairs_to_bytes)."""
    b = np.asarray(b, dtype=np.uint8)
    n, kh = b.shape
    q = np.empty((n, 2 * kh), dtype=np.uint8)
    q[:, 0::2] = b & 0x0F
    q[:, 1::2] = b >> 4
    return q


def _check_w(w):
    w = np.asarray(w)
    if w.dtype != np.float32:
        raise TypeError("base weight must be fp32")
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite base weight")
    return w


# ----------------------------------------------------------------------------- Q4_0-style

def pack_q4_0(w):
    """fp32 W [N, K] -> (codes u8 [N, K/2], scales fp16 bits u16 [N, K/32])."""
    w = _check_w(w)
    n, k = w.shape
    if k % 32:
        raise ValueError("K must be a multiple of 32")
    blk = w.reshape(n, k // 32, 32)
    amax = np.max(np.abs(blk), axis=2)                      # exact
    d32 = (amax / np.float32(7.0)).astype(np.float32)       # IEEE fp32 divide
    d_bits, over = codecs.fp16_encode(d32)
    if np.any(over):
        raise OverflowError("Q4_0 scale overflows fp16")
    d = codecs.fp16_decode(d_bits)                          # the stored scale, as fp32
    q = np.full(blk.shape, 8, dtype=np.int64)
    nz = d != 0
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = (blk / d[:, :, None]).astype(np.float32)    # IEEE fp32 divide
    ratio = np.where(nz[:, :, None], ratio, np.float32(0.0))
    qq = np.clip(np.rint(ratio).astype(np.int64) + 8, 0, 15)
    q = np.where(nz[:, :, None], qq, q)
    codes = nibbles_to_bytes(q.reshape(n, k).astype(np.uint8))
    return codes, d_bits


def dequant_q4_0(codes, scales_fp16_bits):
    """(codes, fp16 scale bits) -> fp32 W [N, K]: (q - 8) * d, exact in fp32."""
    q = bytes_to_nibbles(codes).astype(np.float32)
    n, k = q.shape
    d = codecs.fp16_decode(scales_fp16_bits).astype(np.float32)
    w = (q.reshape(n, k // 32, 32) - np.float32(8.0)) * d[:, :, None]
    return w.reshape(n, k).astype(np.float32)


# ----------------------------------------------------------------------------- Q8_0

def pack_q8_0(w):
    """fp32 W [N, K] -> (codes u8 [N, K] (int8 two's complement), scales fp16 bits u16 [N, K/32])."""
    w = _check_w(w)
    n, k = w.shape
    if k % 32:
        raise ValueError("K must be a multiple of 32")
    blk = w.reshape(n, k // 32, 32)
    amax = np.max(np.abs(blk), axis=2)                      # exact
    d32 = (amax / np.float32(127.0)).astype(np.float32)     # IEEE fp32 divide
    d_bits, over = codecs.fp16_encode(d32)
    if np.any(over):
        raise OverflowError("Q8_0 scale overflows fp16")
    d = codecs.fp16_decode(d_bits)                          # the stored scale, as fp32
    nz = d != 0
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = (blk / d[:, :, None]).astype(np.float32)    # IEEE fp32 divide
    ratio = np.where(nz[:, :, None], ratio, np.float32(0.0))
    q = np.clip(np.rint(ratio).astype(np.int64), -127, 127)
    codes = q.reshape(n, k).astype(np.int8).view(np.uint8)
    return codes, d_bits


def dequant_q8_0(codes, scales_fp16_bits):
    """(codes, fp16 scale bits) -> fp32 W [N, K]: q * d, exact in fp32."""
    q = np.asarray(codes, dtype=np.uint8).view(np.int8).astype(np.float32)
    n, k = q.shape
    d = codecs.fp16_decode(scales_fp16_bits).astype(np.float32)
    w = q.reshape(n, k // 32, 32) * d[:, :, None]
    return w.reshape(n, k).astype(np.float32)


# ----------------------------------------------------------------------------- NF4

def pack_nf4(w, book=None):
    """fp32 W [N, K] -> (codes u8 [N, K/2], absmax scales fp32 [N, K/64])."""
    w = _check_w(w)
    n, k = w.shape
    if k % 64:
        raise ValueError("K must be a multiple of 64")
    mids = nf4_thresholds(book)
    blk = w.reshape(n, k // 64, 64)
    amax = np.max(np.abs(blk), axis=2).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = (blk / amax[:, :, None]).astype(np.float32)     # IEEE fp32 divide
    v = np.where((amax == 0)[:, :, None], np.float32(0.0), v)
    q = np.zeros(blk.shape, dtype=np.int64)
    for m in mids:                                          # q = #{i : v > m_i}
        q += (v > m)
    q = np.where((amax == 0)[:, :, None], 7, q)
    codes = nibbles_to_bytes(q.reshape(n, k).astype(np.uint8))
    return codes, amax


def dequant_nf4(codes, absmax, book=None):
    """(codes, fp32 absmax) -> fp32 W [N, K]: fl32(c[q] * a)."""
    c = nf4_codebook() if book is None else np.asarray(book, np.float32)
    q = bytes_to_nibbles(codes)
    n, k = q.shape
    vals = c[q].reshape(n, k // 64, 64)
    w = vals * np.asarray(absmax, np.float32)[:, :, None]   # one fp32 rounding
    return w.reshape(n, k).astype(np.float32)


# ----------------------------------------------------------------------------- FP8

def pack_fp8(w):
    """fp32 W [N, K] -> (E4M3 codes u8 [N, K], per-tensor fp32 scale)."""
    w = _check_w(w)
    amax = np.float32(np.max(np.abs(w))) if w.size else np.float32(0.0)
    s = np.float32(amax / np.float32(448.0))
    if s == 0:
        return np.zeros(w.shape, dtype=np.uint8), s
    ratio = (w / s).astype(np.float32)
    return codecs.e4m3_encode(ratio), s


def dequant_fp8(codes, scale):
    """(E4M3 codes, fp32 scale) -> fp32 W: fl32(E4M3(q) * s)."""
    return (codecs.e4m3_decode(codes) * np.float32(scale)).astype(np.float32)


# ----------------------------------------------------------------------------- MXFP4

def mxfp4_shared_exponent(amax):
    """Block exponent of the MX conversion: floor(log2 amax) - 2, clamped to
    [-127, 127]; -127 for a zero block."""
    a = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(a)                           # a = f * 2**e, 0.5 <= f < 1: floor(log2 a) = e - 1
    shared = np.where(a > 0, e.astype(np.int64) - 1 - 2, -127)
    return np.clip(shared, -127, 127)


def pack_mxfp4(w):
    """fp32 W [N, K] -> (codes u8 [N, K/2] pair-packed, E8M0 scales u8 [N, K/32])."""
    w = _check_w(w)
    n, k = w.shape
    if k % 32:
        raise ValueError("K must be a multiple of 32")
    blk = w.reshape(n, k // 32, 32).astype(np.float64)
    shared = mxfp4_shared_exponent(np.max(np.abs(blk), axis=2))
    x = np.ldexp(1.0, shared.astype(np.int32))   # the block scale X
    q = codecs.e2m1_encode(blk / x[:, :, None])  # division by a power of two: exact in fp64
    return pairs_to_bytes(q.reshape(n, k)), (shared + 127).astype(np.uint8)


def dequant_mxfp4(codes, e8):
    """(codes, E8M0 scale bytes) -> fp32 W [N, K]: E2M1(q) * 2**(e - 127), exact."""
    v = codecs.e2m1_decode(bytes_to_pairs(codes)).astype(np.float64)
    n, k = v.shape
    e = np.asarray(e8, dtype=np.uint8).astype(np.int64)
    x = np.where(e == 255, np.nan, np.ldexp(1.0, (e - 127).astype(np.int32)))
    w = v.reshape(n, k // 32, 32) * x[:, :, None]
    return w.reshape(n, k).astype(np.float32)


# ----------------------------------------------------------------------------- NVFP4

NVFP4_HEADER = 16          # bytes before the block scales in the stored image


def nvfp4_tensor_scale(amax):
    """g = fl32(amax / 2688) (IEEE fp32 division)."""
    return np.float32(np.float32(amax) / np.float32(2688.0))


def nvfp4_block_scale_codes(block_amax, g):
    """E4M3 scale byte of each block: E4M3(fl32(fl32(amax_b / 6) / g)); 0 if g = 0."""
    a = np.asarray(block_amax, dtype=np.float32)
    g = np.float32(g)
    if g == 0:
        return np.zeros(a.shape, np.uint8)
    t = ((a / np.float32(6.0)).astype(np.float32) / g).astype(np.float32)
    return codecs.e4m3_encode(t)


def nvfp4_decode_scales(sb, g):
    """X_b = fl32(E4M3(sb) * g) for every scale byte."""
    return (codecs.e4m3_decode(sb) * np.float32(g)).astype(np.float32)


def pack_nvfp4_parts(w):
    """fp32 W [N, K] -> (codes u8 [N, K/2] split-nibble, g fp32, E4M3 scale bytes u8 [N, K/16])."""
    w = _check_w(w)
    n, k = w.shape
    if k % 32:
        raise ValueError("K must be a multiple of 32")
    g = nvfp4_tensor_scale(np.max(np.abs(w)) if w.size else 0.0)
    blk = w.reshape(n, k // 16, 16)
    sb = nvfp4_block_scale_codes(np.max(np.abs(blk), axis=2), g)
    x = nvfp4_decode_scales(sb, g).astype(np.float64)
    # the fp64 quotient of two fp32 numbers decides the E2M1 rounding as the
    # exact quotient would: a midpoint of the E2M1 grid has at most 3
    # significant bits, so w - m X, when not zero, is at least about 2^-27 of
    # |w| and the fp64 rounding (2^-53 relative) cannot carry a quotient onto
    # or across a midpoint
    safe = np.where(x == 0, 1.0, x)
    q = codecs.e2m1_encode(blk.astype(np.float64) / safe[:, :, None])
    q = np.where((x == 0)[:, :, None], 0, q).astype(np.uint8)
    return nibbles_to_bytes(q.reshape(n, k)), g, sb


def nvfp4_scale_image(g, sb):
    """The stored scale array: g's fp32 bytes, 12 zero bytes, then the E4M3 bytes row by row."""
    head = np.zeros(NVFP4_HEADER, np.uint8)
    head[:4] = np.frombuffer(np.float32(g).tobytes(), np.uint8)
    return np.concatenate([head, np.asarray(sb, np.uint8).ravel()])


def nvfp4_split_image(image, n, k):
    """Inverse of nvfp4_scale_image: (g fp32, E4M3 bytes u8 [n, k/16])."""
    image = np.asarray(image, np.uint8).ravel()
    g = np.frombuffer(image[:4].tobytes(), np.float32)[0]
    return g, image[NVFP4_HEADER:NVFP4_HEADER + n * (k // 16)].reshape(n, k // 16)


def pack_nvfp4(w):
    """fp32 W [N, K] -> (codes u8 [N, K/2], the scale image u8 [16 + N K / 16])."""
    codes, g, sb = pack_nvfp4_parts(w)
    return codes, nvfp4_scale_image(g, sb)


def dequant_nvfp4_parts(codes, g, sb):
    """(codes, g, E4M3 scale bytes) -> fp32 W [N, K]: fl32(E2M1(q) * fl32(E4M3(sb) * g))."""
    v = codecs.e2m1_decode(bytes_to_nibbles(codes))
    n, k = v.shape
    x = nvfp4_decode_scales(sb, g)
    w = (v.reshape(n, k // 16, 16) * x[:, :, None]).astype(np.float32)
    return w.reshape(n, k)


def dequant_nvfp4(codes, image):
    codes = np.asarray(codes, np.uint8)
    n, k = codes.shape[0], codes.shape[1] * 2
    g, sb = nvfp4_split_image(image, n, k)
    return dequant_nvfp4_parts(codes, g, sb)


# ----------------------------------------------------------------------------- dispatch

def pack(fmt, w):
    if fmt == FMT_Q4_0:
        return pack_q4_0(w)
    if fmt == FMT_NF4:
        return pack_nf4(w)
    if fmt == FMT_FP8:
        return pack_fp8(w)
    if fmt == FMT_MXFP4:
        return pack_mxfp4(w)
    if fmt == FMT_Q8_0:
        return pack_q8_0(w)
    if fmt == FMT_NVFP4:
        return pack_nvfp4(w)
    raise ValueError(f"unknown format {fmt}")


def dequant(fmt, codes, scales):
    if fmt == FMT_Q4_0:
        return dequant_q4_0(codes, scales)
    if fmt == FMT_NF4:
        return dequant_nf4(codes, scales)
    if fmt == FMT_FP8:
        return dequant_fp8(codes, scales)
    if fmt == FMT_MXFP4:
        return dequant_mxfp4(codes, scales)
    if fmt == FMT_Q8_0:
        return dequant_q8_0(codes, scales)
    if fmt == FMT_NVFP4:
        return dequant_nvfp4(codes, scales)
    raise ValueError(f"unknown format {fmt}")


def bf16_tile_values(w_f32):
    """The bf16 operand values a GEMM feeds to the matrix cores: one RNE rounding."""
    return codecs.bf16_round(w_f32)
