"""Pins for the oracle's NF4 code book, the pack rules and dequant of every base
format (Q4_0-style, NF4, FP8, MXFP4).  CPU only."""

import os
import statistics

import numpy as np
import pytest
import scipy.stats
import torch

from oracle import codecs, formats

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- NF4 code book

def test_nf4_book_two_independent_inverse_cdfs_agree():
    a = formats.nf4_codebook(statistics.NormalDist().inv_cdf)
    b = formats.nf4_codebook(lambda p: float(scipy.stats.norm.ppf(p)))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_nf4_book_invariants():
    c = formats.nf4_codebook().astype(np.float64)
    assert c.shape == (16,)
    assert np.all(np.diff(c) > 0)
    assert c[0] == -1.0 and c[7] == 0.0 and c[15] == 1.0
    assert (c < 0).sum() == 7 and (c > 0).sum() == 8
    gaps = np.diff(c)
    assert abs(gaps.min() - 0.0796) < 5e-4 and abs(gaps.max() - 0.3038) < 5e-4
    # smallest positive level: Phi^-1(1/2 + (delta - 1/2)/8) / Phi^-1(delta)
    delta = 0.5 * ((1 - 1 / 30) + (1 - 1 / 32))
    ppf = scipy.stats.norm.ppf
    assert abs(c[8] - ppf(0.5 + (delta - 0.5) / 8) / ppf(delta)) < 1e-7
    assert abs(c[6] + ppf(0.5 + (delta - 0.5) / 7) / ppf(delta)) < 1e-7


def test_nf4_book_bits_from_exact_rational_offset():
    """Every level, bit for bit, from an independent route: delta as the exact
    rational (29/30 + 31/32) / 2, probabilities built upward from 1/2, scipy's
    inverse CDF.  A rounded delta (e.g. 0.9677083) moves levels by 1-2 ulps."""
    from fractions import Fraction
    delta = (Fraction(29, 30) + Fraction(31, 32)) / 2
    ppf = scipy.stats.norm.ppf
    top = ppf(float(delta))
    pos = [ppf(float(Fraction(1, 2) + (delta - Fraction(1, 2)) * j / 8)) / top for j in range(1, 9)]
    neg = [-ppf(float(Fraction(1, 2) + (delta - Fraction(1, 2)) * j / 7)) / top for j in range(7, 0, -1)]
    want = np.array(neg + [0.0] + pos, dtype=np.float64).astype(np.float32)
    assert np.array_equal(formats.nf4_codebook().view(np.uint32), want.view(np.uint32))


def test_nf4_thresholds_between_levels():
    c = formats.nf4_codebook()
    m = formats.nf4_thresholds()
    assert np.all(c[:-1] < m) and np.all(m < c[1:])


# ----------------------------------------------------------------------------- nibbles

def test_nibble_layout_round_trip_and_positions():
    g = np.random.default_rng(0)
    q = g.integers(0, 16, size=(3, 96), dtype=np.uint8)
    b = formats.nibbles_to_bytes(q)
    assert b.shape == (3, 48)
    assert np.array_equal(formats.bytes_to_nibbles(b), q)
    # byte j of group t: element 32t + j low, element 32t + j + 16 high
    for t in range(3):
        for j in range(16):
            assert b[1, 16 * t + j] == q[1, 32 * t + j] | (q[1, 32 * t + j + 16] << 4)


# ----------------------------------------------------------------------------- Q4_0-style

def _read_q40_golden():
    vals, codes, scale, byts = [], [], None, None
    with open(os.path.join(GOLDEN, "q4_0_block.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            if line.startswith("scale_fp16_bits"):
                scale = int(line.split()[1], 16)
            elif line.startswith("bytes"):
                byts = [int(t, 16) for t in line.split()[1:]]
            else:
                _, v, c = line.split()
                vals.append(np.float32(v))
                codes.append(int(c))
    return np.array(vals, np.float32), np.array(codes), scale, np.array(byts, np.uint8)


def test_q40_golden_block():
    w, codes, scale, byts = _read_q40_golden()
    c, s = formats.pack_q4_0(w.reshape(1, 32))
    assert int(s[0, 0]) == scale
    assert np.array_equal(formats.bytes_to_nibbles(c)[0], codes)
    assert np.array_equal(c[0], byts)
    deq = formats.dequant_q4_0(c, s)[0]
    d = np.float64(np.uint16(scale).view(np.float16))
    assert np.array_equal(deq.astype(np.float64), (codes - 8) * d)


def test_q40_dequant_exhaustive_codes_times_all_fp16_scales():
    d_bits = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16)    # every finite d >= +0
    d = d_bits.view(np.float16).astype(np.float64)
    for q in range(16):
        codes = formats.nibbles_to_bytes(np.full((d_bits.size, 32), q, np.uint8))
        w = formats.dequant_q4_0(codes, d_bits[:, None])
        assert np.array_equal(w.astype(np.float64), np.repeat(((q - 8) * d)[:, None], 32, 1))


def test_q40_pack_error_bound_and_code_range():
    g = np.random.default_rng(5)
    w = (g.standard_normal((64, 256)) * 0.02).astype(np.float32)
    c, s = formats.pack_q4_0(w)
    q = formats.bytes_to_nibbles(c)
    assert q.min() >= 1 and q.max() <= 15                               # |w/d| < 7.5 never clamps
    d = np.repeat(codecs.fp16_decode(s).astype(np.float64), 32, axis=1)
    err = np.abs(formats.dequant_q4_0(c, s).astype(np.float64) - w)
    assert np.all(err <= d * (0.5 + 1e-6))


def test_q40_zero_and_tiny_blocks():
    w = np.zeros((2, 64), np.float32)
    w[1, 32:] = 1e-12                                                   # absmax/7 underflows fp16
    c, s = formats.pack_q4_0(w)
    assert np.all(formats.bytes_to_nibbles(c) == 8)
    assert np.all(s == 0)
    assert np.all(formats.dequant_q4_0(c, s) == 0)


def test_q40_overflow_rejected_and_nonfinite_rejected():
    with pytest.raises(OverflowError):
        formats.pack_q4_0(np.full((1, 32), 1e6, np.float32))
    w = np.zeros((1, 32), np.float32)
    w[0, 3] = np.nan
    with pytest.raises(ValueError):
        formats.pack_q4_0(w)


# ----------------------------------------------------------------------------- NF4

def test_nf4_pack_matches_brute_force_nearest_code():
    """The threshold rule equals 'nearest level, ties to the lower code' except
    inside the fp32 rounding sliver of a midpoint, where the rounded threshold
    decides.  Checked against a brute-force nearest-level search."""
    g = np.random.default_rng(7)
    book = formats.nf4_codebook().astype(np.float64)
    mids = formats.nf4_thresholds().astype(np.float64)
    w = (g.standard_normal((32, 640)) * 0.02).astype(np.float32)
    w[0, :15] = mids.astype(np.float32)                                 # exact threshold values
    w[0, 63] = 1.0
    c, a = formats.pack_nf4(w)
    q = formats.bytes_to_nibbles(c).reshape(32, 10, 64)
    v = (w.reshape(32, 10, 64) / a[:, :, None]).astype(np.float32).astype(np.float64)
    dist = np.abs(v[..., None] - book)                                   # exact in fp64
    brute = np.argmin(dist, axis=-1)                                     # first minimum = lower code
    diff = brute != q
    if diff.any():
        vv = v[diff]
        true_mid = (book[q[diff]] + book[brute[diff]]) / 2
        assert np.all(np.abs(vv - true_mid) <= 2 ** -24)
    # a value equal to a rounded threshold goes to the lower code
    assert np.array_equal(q[0, 0, :15], np.arange(15))


def test_nf4_levels_times_scale_recover_codes():
    book = formats.nf4_codebook()
    w = np.tile(book, 4).reshape(1, 64) * np.float32(0.0371)
    c, a = formats.pack_nf4(w.astype(np.float32))
    assert a[0, 0] == np.float32(0.0371) * np.float32(1.0)
    assert np.array_equal(formats.bytes_to_nibbles(c)[0], np.tile(np.arange(16), 4))


def test_nf4_dequant_product_rounded_once():
    book = formats.nf4_codebook().astype(np.float64)
    g = np.random.default_rng(11)
    scales = np.concatenate([2.0 ** np.arange(-20, 5), g.uniform(1e-4, 0.2, 200),
                             [1.1754944e-38, 3e-38]]).astype(np.float32)
    q = np.tile(np.arange(16, dtype=np.uint8), 4)
    codes = formats.nibbles_to_bytes(np.tile(q, (scales.size, 1)))
    w = formats.dequant_nf4(codes, scales[:, None])
    ref = (book[q][None, :] * scales.astype(np.float64)[:, None]).astype(np.float32)
    assert np.array_equal(w, ref)
    p2 = scales[:25].astype(np.float64)
    assert np.array_equal(w[:25].astype(np.float64), book.astype(np.float32)[q][None, :] * p2[:, None])


def test_nf4_zero_block_and_error_bound():
    g = np.random.default_rng(9)
    w = (g.standard_normal((16, 128)) * 0.02).astype(np.float32)
    w[3, 64:] = 0
    c, a = formats.pack_nf4(w)
    q = formats.bytes_to_nibbles(c)
    assert np.all(q[3, 64:] == 7) and a[3, 1] == 0
    book = formats.nf4_codebook().astype(np.float64)
    maxgap = np.max(np.diff(book))
    err = np.abs(formats.dequant_nf4(c, a).astype(np.float64) - w)
    assert np.all(err <= np.repeat(a.astype(np.float64), 64, 1) * (maxgap / 2 + 1e-6))


# ----------------------------------------------------------------------------- FP8

def test_fp8_dequant_all_codes_times_scales():
    import torch
    c = np.arange(256, dtype=np.uint8)
    ok = (c != 0x7F) & (c != 0xFF)
    dec = torch.from_numpy(c).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    for s in np.float32([1.0, 0.02 / 448, 3.3e-5, 7.77e-3]):
        w = formats.dequant_fp8(c[ok].reshape(1, -1), s)[0]
        assert np.array_equal(w, (dec[ok] * np.float64(s)).astype(np.float32))


def test_fp8_pack_properties():
    g = np.random.default_rng(13)
    w = (g.standard_normal((32, 256)) * 0.02).astype(np.float32)
    c, s = formats.pack_fp8(w)
    assert s == np.float32(np.max(np.abs(w)) / np.float32(448.0))
    dq = formats.dequant_fp8(c, s).astype(np.float64)
    rel = np.abs(dq - w) / np.maximum(np.abs(w), 2.0 ** -6 * s)
    assert rel.max() <= 2 ** -4 + 1e-6                                   # 3 mantissa bits
    c0, s0 = formats.pack_fp8(np.zeros((2, 32), np.float32))
    assert s0 == 0 and not c0.any()


# ----------------------------------------------------------------------------- re-pack

@pytest.mark.parametrize("fmt", [formats.FMT_Q4_0, formats.FMT_NF4, formats.FMT_MXFP4])
def test_repack_is_idempotent_4bit(fmt):
    g = np.random.default_rng(17 + fmt)
    w = (g.standard_normal((40, 512)) * 0.02).astype(np.float32)
    c1, s1 = formats.pack(fmt, w)
    c2, s2 = formats.pack(fmt, formats.dequant(fmt, c1, s1))
    assert np.array_equal(c1, c2) and np.array_equal(np.asarray(s1), np.asarray(s2))


def test_repack_fp8_codes_identical():
    g = np.random.default_rng(19)
    w = (g.standard_normal((40, 512)) * 0.02).astype(np.float32)
    c1, s1 = formats.pack_fp8(w)
    c2, s2 = formats.pack_fp8(formats.dequant_fp8(c1, s1))
    assert np.array_equal(c1, c2)
    assert abs(float(s2) - float(s1)) <= float(np.spacing(s1))


# ----------------------------------------------------------------------------- MXFP4

def test_pair_layout_round_trip_and_positions():
    g = np.random.default_rng(1)
    q = g.integers(0, 16, size=(3, 96), dtype=np.uint8)
    b = formats.pairs_to_bytes(q)
    assert b.shape == (3, 48)
    assert np.array_equal(formats.bytes_to_pairs(b), q)
    for i in range(48):
        assert b[2, i] == q[2, 2 * i] | (q[2, 2 * i + 1] << 4)


def _read_mxfp4_golden():
    vals, codes, e8, byts = [], [], None, None
    with open(os.path.join(GOLDEN, "mxfp4_block.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            if line.startswith("scale_e8m0"):
                e8 = int(line.split()[1])
            elif line.startswith("bytes"):
                byts = [int(t, 16) for t in line.split()[1:]]
            else:
                _, v, c = line.split()
                vals.append(np.float32(v))
                codes.append(int(c))
    return np.array(vals, np.float32), np.array(codes), e8, np.array(byts, np.uint8)


def test_mxfp4_golden_block():
    w, codes, e8, byts = _read_mxfp4_golden()
    c, e = formats.pack_mxfp4(w.reshape(1, 32))
    assert int(e[0, 0]) == e8
    assert np.array_equal(formats.bytes_to_pairs(c)[0], codes)
    assert np.array_equal(c[0], byts)


def test_mxfp4_scale_decode_vs_torch_e8m0():
    """Every E8M0 byte decodes to torch's float8_e8m0fnu value (255 is NaN)."""
    e = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(e.copy()).view(torch.float8_e8m0fnu).float().numpy()
    codes = np.full((256, 16), 0x22, np.uint8)            # every element E2M1 1.0
    got = formats.dequant_mxfp4(codes, e[:, None])
    assert np.array_equal(got[:, 0], ref, equal_nan=True)
    assert np.array_equal(got[:, 31], ref, equal_nan=True)


def _shared_exp_brute(amax):
    """The integer s with 4 <= amax / 2^s < 8 (search), clamped to [-127, 127]."""
    if amax == 0:
        return -127
    s = -200
    while not (amax / 2.0 ** s < 8):
        s += 1
    assert amax / 2.0 ** s >= 4
    return min(max(s, -127), 127)


def test_mxfp4_pack_vs_brute_force():
    """Scale by exhaustive search over exponents, each code by exhaustive search
    over the 16 E2M1 values times that scale (ties to the even mantissa)."""
    g = np.random.default_rng(23)
    n = 24
    mags = np.exp2(g.uniform(-30, 30, size=(n, 1)))
    w = (g.standard_normal((n, 64)) * mags).astype(np.float32)
    w[3, :32] = 0.0
    w[4, 5] = -0.0
    c, e = formats.pack_mxfp4(w)
    table = codecs.e2m1_decode(np.arange(16, dtype=np.uint8)).astype(np.float64)
    q = formats.bytes_to_pairs(c)
    for row in range(n):
        for blk in range(2):
            v = w[row, 32 * blk:32 * blk + 32].astype(np.float64)
            s = _shared_exp_brute(float(np.max(np.abs(v))))
            assert int(e[row, blk]) == s + 127
            x = 2.0 ** s
            for j in range(32):
                cands = [cc for cc in range(16) if (cc >> 3) == int(np.signbit(v[j]))]
                best = min(cands, key=lambda cc: (abs(abs(v[j]) - abs(table[cc]) * x), cc & 1))
                assert q[row, 32 * blk + j] == best, (row, blk, j)


def test_mxfp4_round_trip_is_exact():
    """W built from random codes and scales, each block holding a +-4 or +-6
    element: packing recovers the codes and scale bytes, dequant is exact."""
    g = np.random.default_rng(29)
    n, k = 16, 128
    q = g.integers(0, 16, size=(n, k), dtype=np.uint8)
    q[:, ::32] = g.choice([6, 7, 14, 15], size=(n, k // 32))
    e = g.integers(1, 253, size=(n, k // 32)).astype(np.uint8)
    w = formats.dequant_mxfp4(formats.pairs_to_bytes(q), e)
    c2, e2 = formats.pack_mxfp4(w)
    assert np.array_equal(e2, e)
    assert np.array_equal(formats.bytes_to_pairs(c2), q)
    table = codecs.e2m1_decode(np.arange(16, dtype=np.uint8)).astype(np.float64)
    x = np.exp2(e.astype(np.float64) - 127)
    want = table[q].reshape(n, k // 32, 32) * x[:, :, None]
    assert np.array_equal(w.astype(np.float64), want.reshape(n, k))


def test_mxfp4_power_of_two_scaling_moves_only_the_scale():
    g = np.random.default_rng(31)
    w = (g.standard_normal((8, 256)) * 0.02).astype(np.float32)
    c0, e0 = formats.pack_mxfp4(w)
    for j in (-20, -1, 1, 17):
        c1, e1 = formats.pack_mxfp4((w * np.float32(2.0 ** j)).astype(np.float32))
        assert np.array_equal(c1, c0)
        assert np.array_equal(e1.astype(int), e0.astype(int) + j)


def test_mxfp4_zero_and_subnormal_blocks():
    w = np.zeros((2, 64), np.float32)
    w[1, 32] = np.float32(2.0 ** -128)                    # 0.5 X at the clamped exponent
    w[1, 33] = np.float32(-(2.0 ** -126))                 # 2 X
    w[1, 34] = np.float32(2.0 ** -140)                    # far below 0.25 X: zero
    c, e = formats.pack_mxfp4(w)
    assert np.array_equal(e, np.array([[0, 0], [0, 0]], np.uint8))
    q = formats.bytes_to_pairs(c)
    assert not q[0].any() and not q[1, :32].any()
    assert list(q[1, 32:35]) == [1, 12, 0]
    d = formats.dequant_mxfp4(c, e)
    assert d[1, 32] == np.float32(2.0 ** -128) and d[1, 33] == np.float32(-(2.0 ** -126))


def test_mxfp4_error_bound_and_largest_element():
    """|w - deq| <= X below the saturation point 6 X and < 2 X above it; the
    largest element of a block codes to the top binade (4 or 6)."""
    g = np.random.default_rng(37)
    w = (g.standard_normal((32, 512)) * np.exp2(g.uniform(-10, 5, (32, 1)))).astype(np.float32)
    c, e = formats.pack_mxfp4(w)
    d = formats.dequant_mxfp4(c, e).astype(np.float64)
    x = np.repeat(np.exp2(e.astype(np.float64) - 127), 32, axis=1)
    err = np.abs(d - w)
    small = np.abs(w) <= 6 * x
    assert np.all(err[small] <= x[small]) and np.all(err[~small] < 2 * x[~small])
    q = formats.bytes_to_pairs(c).reshape(32, 16, 32) & 7
    top = np.argmax(np.abs(w).reshape(32, 16, 32), axis=2)
    assert np.all(np.take_along_axis(q, top[:, :, None], 2) >= 6)


# ----------------------------------------------------------------------------- Q8_0

def _read_q80_golden():
    scale, vals, codes = None, [], []
    for line in open(os.path.join(GOLDEN, "q8_0_block.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        if line.startswith("scale_fp16_bits"):
            scale = int(line.split()[1], 16)
            continue
        _, v, c = line.split()
        vals.append(np.float32(v))
        codes.append(int(c, 16))
    return np.array(vals, np.float32).reshape(1, 32), np.array(codes, np.uint8).reshape(1, 32), scale


def test_q80_golden_block():
    w, want, scale = _read_q80_golden()
    codes, s = formats.pack_q8_0(w)
    assert int(s[0, 0]) == scale
    assert np.array_equal(codes, want)
    d = codecs.fp16_decode(np.uint16(scale))
    assert np.array_equal(formats.dequant_q8_0(codes, s), want.view(np.int8).astype(np.float32) * d)


def test_q80_dequant_exhaustive_codes_and_scales():
    """Every code byte against every finite fp16 scale: w / d == q exactly
    (an 8-bit integer times an 11-bit significand is exact in fp32)."""
    d_bits = np.arange(0, 0x7C00, dtype=np.uint16)
    d_bits = np.concatenate([d_bits, d_bits | 0x8000])
    n = d_bits.size
    q = np.tile(np.arange(256, dtype=np.uint8), (1, 1))
    for lo in range(0, n, 4096):
        db = d_bits[lo:lo + 4096]
        codes = np.tile(np.arange(256, dtype=np.uint8), (db.size, 1))[:, :256]
        w = formats.dequant_q8_0(codes, np.repeat(db.reshape(-1, 1), 8, axis=1))
        d = codecs.fp16_decode(db).astype(np.float64).reshape(-1, 1)
        qv = codes.view(np.int8).astype(np.float64)
        assert np.array_equal(w.astype(np.float64), qv * d)


def test_q80_pack_is_nearest_with_ties_to_even():
    """Against a brute-force search over all 255 codes of each element, given
    the stored scale; equal distances go to the even code."""
    g = np.random.default_rng(17)
    w = (g.standard_normal((16, 256)) * 0.02).astype(np.float32)
    w[3, :32] = (np.arange(32, dtype=np.float32) - 15.5) * np.float32(2.0 ** -7)   # half-integer ties
    w[3, 0] = np.float32(127 * 2.0 ** -7)
    codes, s = formats.pack_q8_0(w)
    d = codecs.fp16_decode(s).astype(np.float64)
    cand = np.arange(-127, 128, dtype=np.float64)
    for i in range(w.shape[0]):
        for b in range(w.shape[1] // 32):
            blk = w[i, 32 * b:32 * b + 32].astype(np.float64)
            ratio = (w[i, 32 * b:32 * b + 32] / np.float32(d[i, b])).astype(np.float32).astype(np.float64)
            dist = np.abs(ratio[:, None] - cand[None, :])
            best = dist.min(axis=1, keepdims=True)
            ok = dist == best
            pick = np.where(ok.sum(axis=1) > 1, cand[np.argmax(ok & (cand % 2 == 0), axis=1)], cand[np.argmax(ok, axis=1)])
            got = codes[i, 32 * b:32 * b + 32].view(np.int8).astype(np.float64)
            assert np.array_equal(got, pick), (i, b)
            assert np.all(np.abs(blk - got * d[i, b]) <= d[i, b] / 2 * (1 + 1e-6))


def test_q80_zero_tiny_and_subnormal_scale_blocks():
    w = np.zeros((3, 64), np.float32)
    w[1, :32] = np.float32(8.5e-8 * 127) * np.linspace(-1, 1, 32, dtype=np.float32)   # scale rounds down to 2^-24
    w[2, 32:] = np.float32(1e-12)                                                       # scale rounds to 0
    codes, s = formats.pack_q8_0(w)
    assert np.all(s[0] == 0) and not codes[0].any()
    assert int(s[1, 0]) == 0x0001                            # the smallest fp16 subnormal
    q = codes[1, :32].view(np.int8)
    assert q.max() == 127 and q.min() == -127                # the clamp acts here
    assert int(s[2, 1]) == 0 and not codes[2, 32:].any()


def test_q80_repack_is_idempotent():
    g = np.random.default_rng(23)
    w = (g.standard_normal((32, 512)) * 0.02).astype(np.float32)
    c, s = formats.pack_q8_0(w)
    c2, s2 = formats.pack_q8_0(formats.dequant_q8_0(c, s))
    assert np.array_equal(c, c2) and np.array_equal(s, s2)


def test_q80_scale_overflow_and_nonfinite():
    with pytest.raises(OverflowError):
        formats.pack_q8_0(np.full((1, 32), 1e7, np.float32))
    w = np.zeros((1, 32), np.float32)
    w[0, 3] = np.inf
    with pytest.raises(ValueError):
        formats.pack_q8_0(w)


# ----------------------------------------------------------------------------- FP8 pack golden

def _read_fp8_golden():
    scale, vals, codes = None, [], []
    for line in open(os.path.join(GOLDEN, "fp8_block.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        if line.startswith("scale_fp32_bits"):
            scale = int(line.split()[1], 16)
            continue
        _, v, c = line.split()
        vals.append(np.float32(v))
        codes.append(int(c, 16))
    return np.array(vals, np.float32).reshape(1, 32), np.array(codes, np.uint8).reshape(1, 32), scale


def test_fp8_golden_block():
    """The hand-packed FP8 tensor: the scale rule (absmax / 448), every code
    including ties to even in the normal and subnormal ranges, a negative
    value rounding to zero, and a ratio that is not exact in fp32."""
    w, want, scale = _read_fp8_golden()
    codes, s = formats.pack_fp8(w)
    assert np.float32(s).view(np.uint32) == scale
    assert np.array_equal(codes, want)
    # decoded values: the code's E4M3 value times 2^-7, e.g. 0x79 -> 288 / 128
    d = formats.dequant_fp8(codes, s)
    assert d[0, 8] == np.float32(2.25) and d[0, 9] == np.float32(2.5) and d[0, 10] == np.float32(13 / 128)
    assert d[0, 0] == np.float32(3.5) and d[0, 11] == np.float32(-0.125)
    assert np.signbit(d[0, 7]) and d[0, 7] == 0
