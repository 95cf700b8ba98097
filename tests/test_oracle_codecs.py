"""Pins for the oracle's number codecs: library routines, exhaustive where the
format is small, and every rounding tie.  CPU only."""

import os

import numpy as np
import pytest
import torch

from oracle import codecs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _dense_f32(n, seed):
    g = np.random.default_rng(seed)
    bits = g.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    return x[np.isfinite(x)]


def _torch_bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


# ----------------------------------------------------------------------------- bf16

def test_bf16_decode_exhaustive_vs_torch():
    bits = np.arange(2 ** 16, dtype=np.uint32).astype(np.uint16)
    ours = codecs.bf16_decode(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_encode_dense_vs_torch():
    x = _dense_f32(400_000, 1)
    x = np.concatenate([x, np.float32([0.0, -0.0, 1e-40, -1e-40, 3.4e38, -3.4e38])])
    assert np.array_equal(codecs.bf16_encode(x), _torch_bf16_bits(x))


def test_bf16_encode_every_tie_goes_to_even():
    # midpoints between consecutive bf16 values: fp32 bits (b << 16) | 0x8000
    b = np.arange(0, 0x7F7F, dtype=np.uint32)
    mid = ((b << 16) | 0x8000).view(np.float32)
    ours = codecs.bf16_encode(mid).astype(np.uint32)
    want = np.where(b % 2 == 0, b, b + 1)
    assert np.array_equal(ours, want)
    assert np.array_equal(codecs.bf16_encode(mid), _torch_bf16_bits(mid))
    assert np.array_equal(codecs.bf16_encode(-mid), _torch_bf16_bits(-mid))


# ----------------------------------------------------------------------------- fp16

def test_fp16_decode_exhaustive_vs_numpy():
    bits = np.arange(2 ** 16, dtype=np.uint32).astype(np.uint16)
    ours = codecs.fp16_decode(bits)
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_fp16_encode_dense_vs_numpy():
    g = np.random.default_rng(2)
    x = np.concatenate([
        (g.standard_normal(200_000) * 10.0 ** g.uniform(-9, 5, 200_000)).astype(np.float32),
        np.float32([0.0, -0.0, 6.0e-8, 2.9e-8, 3.0e-8, 65504.0, 65519.0, -65519.0]),
    ])
    bits, over = codecs.fp16_encode(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16)
    assert np.array_equal(over, np.isinf(ref))
    assert np.array_equal(bits[~over], ref[~over].view(np.uint16))


def test_fp16_encode_every_tie_goes_to_even():
    # all midpoints between consecutive finite fp16 values (normal and subnormal)
    h = np.arange(0, 0x7BFF, dtype=np.uint32)
    lo = h.astype(np.uint16).view(np.float16).astype(np.float64)
    hi = (h + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)  # midpoints exact in fp32
    bits, _ = codecs.fp16_encode(mid)
    want = np.where(h % 2 == 0, h, h + 1)
    assert np.array_equal(bits.astype(np.uint32), want)
    assert np.array_equal(bits, mid.astype(np.float16).view(np.uint16))


def test_fp16_overflow_flagged():
    _, over = codecs.fp16_encode(np.float32([65504.0, 65519.99, 65520.0, 1e9, -70000.0]))
    assert over.tolist() == [False, False, True, True, True]


# ----------------------------------------------------------------------------- E4M3

def _torch_e4m3_decode(codes):
    return torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()


def test_e4m3_decode_exhaustive_vs_torch():
    c = np.arange(256, dtype=np.uint8)
    ours = codecs.e4m3_decode(c)
    ref = _torch_e4m3_decode(c)
    nan = np.isnan(ref)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))
    assert np.nanmax(ours) == 448.0


def test_e4m3_encode_in_range_vs_torch():
    g = np.random.default_rng(3)
    x = (g.standard_normal(300_000) * 10.0 ** g.uniform(-4, 2.6, 300_000)).astype(np.float32)
    x = x[np.abs(x) <= 448.0]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codecs.e4m3_encode(x), ref)


def test_e4m3_encode_every_tie_goes_to_even():
    c = np.arange(0, 0x7E, dtype=np.uint8)           # all finite non-negative codes but the top
    lo = codecs.e4m3_decode(c).astype(np.float64)
    hi = codecs.e4m3_decode(c + 1).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)
    ours = codecs.e4m3_encode(mid).astype(np.int64)
    want = np.where(c % 2 == 0, c, c + 1)
    assert np.array_equal(ours, want)
    ref = torch.from_numpy(mid).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    assert np.array_equal(codecs.e4m3_encode(-mid).astype(np.int64), want | 0x80)


def test_e4m3_saturates():
    x = np.float32([448.0, 463.99, 464.0, 465.0, 1e6, np.inf, -1e6, -np.inf])
    assert codecs.e4m3_encode(x).tolist() == [0x7E] * 6 + [0xFE] * 2
    assert codecs.e4m3_encode(np.float32([np.nan]))[0] == 0x7F


def test_e4m3_golden_points():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_points.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                v, c = line.split()
                rows.append((np.float32(float(v)), int(c, 16)))
    vals = np.array([r[0] for r in rows], dtype=np.float32)
    codes = np.array([r[1] for r in rows], dtype=np.uint8)
    assert np.array_equal(codecs.e4m3_encode(vals), codes)
    exact = np.abs(vals) <= 448.0
    dec = codecs.e4m3_decode(codes)
    on_grid = exact & np.isin(vals, dec)
    assert np.array_equal(dec[on_grid], vals[on_grid])
    assert on_grid.sum() >= 12


@pytest.mark.parametrize("x", [0.0, -0.0, 1e-30, -1e-30])
def test_e4m3_zero_keeps_sign(x):
    code = codecs.e4m3_encode(np.float32([x]))[0]
    assert code == (0x80 if np.signbit(np.float32(x)) else 0x00)


# ----------------------------------------------------------------------------- E2M1

def _e2m1_table():
    vals = []
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                c, v = line.split()
                vals.append((int(c), float(v)))
    assert [c for c, _ in vals] == list(range(16))
    return np.array([v for _, v in vals]), [np.signbit(v) for _, v in vals]


def test_e2m1_decode_matches_published_table():
    table, neg = _e2m1_table()
    got = codecs.e2m1_decode(np.arange(16, dtype=np.uint8)).astype(np.float64)
    assert np.array_equal(got, table)
    assert list(np.signbit(got)) == neg                   # code 8 is negative zero


def _e2m1_brute(x):
    """Nearest of the 16 E2M1 values by exhaustive search; a tie takes the code
    whose mantissa bit (bit 0) is 0; magnitudes above 6 saturate."""
    table, _ = _e2m1_table()
    out = []
    for v in np.asarray(x, np.float64):
        best = None
        for c in range(16):
            if (c >> 3) != int(np.signbit(v)):             # same sign half, zero included
                continue
            d = abs(abs(v) - abs(table[c]))
            key = (d, c & 1)
            if best is None or key < best[0]:
                best = (key, c)
        out.append(best[1])
    return np.array(out, np.uint8)


def test_e2m1_encode_every_tie_goes_to_even():
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    want = np.array([0, 2, 2, 4, 4, 6, 6], np.uint8)      # 0, 1, 1, 2, 2, 4, 4
    assert np.array_equal(codecs.e2m1_encode(mids), want)
    assert np.array_equal(codecs.e2m1_encode(-mids), want | 8)
    assert np.array_equal(_e2m1_brute(np.concatenate([mids, -mids])),
                          np.concatenate([want, want | 8]))


def test_e2m1_encode_vs_exhaustive_search():
    g = np.random.default_rng(5)
    x = np.concatenate([g.uniform(-8, 8, 4000), g.uniform(-1, 1, 2000),
                        np.arange(-64, 65) / 8.0])         # every multiple of 1/8 in [-8, 8]
    assert np.array_equal(codecs.e2m1_encode(x), _e2m1_brute(x))


@pytest.mark.parametrize("x,code", [(6.0, 7), (6.5, 7), (7.999, 7), (1e30, 7), (-1e30, 15),
                                    (0.0, 0), (-0.0, 8), (-1e-30, 8), (0.2499, 0), (0.2501, 1)])
def test_e2m1_saturation_and_zero_sign(x, code):
    assert int(codecs.e2m1_encode([x])[0]) == code


def test_e2m1_rejects_non_finite():
    with pytest.raises(ValueError):
        codecs.e2m1_encode([np.nan])
