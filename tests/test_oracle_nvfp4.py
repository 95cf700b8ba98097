"""Pins of the oracle's NVFP4 base format against what its definition fixes
(no GPU): a block packed by hand, exhaustive decoding against torch's E4M3
type, brute-force nearest codes in exact rational arithmetic, exact round
trips, power-of-two invariance, error bounds and the degenerate blocks."""

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import codecs, formats

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]           # magnitudes by code 0..7


def _read_golden():
    w = np.zeros((2, 32), np.float32)
    q = np.zeros((2, 32), np.uint8)
    g_bits, sb, deq = None, None, []
    for line in open(os.path.join(GOLDEN, "nvfp4_block.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        t = line.split()
        if t[0] == "tensor_scale_fp32_bits":
            g_bits = int(t[1], 16)
        elif t[0] == "block_scales":
            sb = np.array([int(v, 16) for v in t[1:]], np.uint8).reshape(2, 2)
        elif t[0] == "dequant":
            deq.append((int(t[1]), int(t[2]), float(t[3])))
        else:
            r, e = int(t[0]), int(t[1])
            w[r, e] = np.float32(t[2])
            q[r, e] = int(t[3])
    return w, q, g_bits, sb, deq


def test_nvfp4_golden_block():
    w, q, g_bits, sb, deq = _read_golden()
    codes, g, s = formats.pack_nvfp4_parts(w)
    assert np.float32(g).view(np.uint32) == g_bits
    assert np.array_equal(s, sb)
    assert np.array_equal(formats.bytes_to_nibbles(codes), q)
    # the stored image: g's bytes, 12 zero bytes, the scale bytes row by row
    c2, image = formats.pack_nvfp4(w)
    assert np.array_equal(c2, codes)
    assert image.size == 16 + 4
    assert int.from_bytes(bytes(image[:4]), "little") == g_bits
    assert not image[4:16].any()
    assert list(image[16:]) == [0x7E, 0x63, 0x62, 0x00]
    d = formats.dequant_nvfp4(codes, image)
    for r, e, v in deq:
        assert d[r, e] == np.float32(v), (r, e)
    assert formats.dequant(formats.FMT_NVFP4, codes, image).tobytes() == d.tobytes()


def test_nvfp4_dequant_exhaustive_codes_and_scales_vs_torch_e4m3():
    """Every code times every E4M3 scale byte, g = 1 and g = 2^-20: the value
    is E2M1(q) * E4M3(s) * g, an exact product (at most 6 significant bits)."""
    s = np.arange(256, dtype=np.uint8)
    e4 = torch.from_numpy(s.copy()).view(torch.float8_e4m3fn).double().numpy()
    q = np.arange(16, dtype=np.uint8)
    e2 = np.array(E2M1 + [-v for v in E2M1])
    for g in (1.0, 2.0 ** -20):
        # row i: 32 elements whose codes run 0..15 twice; block scales s[i] and s[255 - i]
        codes = formats.nibbles_to_bytes(np.tile(q, (256, 2)))
        sb = np.stack([s, s[::-1]], axis=1)
        got = formats.dequant_nvfp4_parts(codes, np.float32(g), sb).astype(np.float64)
        want = np.concatenate([e2[None, :] * e4[:, None], e2[None, :] * e4[::-1, None]], axis=1) * g
        assert np.array_equal(got, want, equal_nan=True)
    # NaN scale bytes decode to NaN
    assert np.isnan(formats.dequant_nvfp4_parts(formats.nibbles_to_bytes(np.ones((1, 32), np.uint8)),
                                                np.float32(1.0), np.array([[0x7F, 0xFF]], np.uint8))).all()


def test_nvfp4_dequant_rounds_the_block_scale_before_the_element():
    """With g = fl32(0.1) the block scale X = fl32(E4M3(s) g) is rounded once,
    then E2M1(q) X once more: compared with exact rational arithmetic."""
    g = np.float32(0.1)
    s = np.arange(1, 127, dtype=np.uint8)                   # the positive finite E4M3 bytes
    e4 = torch.from_numpy(s.copy()).view(torch.float8_e4m3fn).double().numpy()
    codes = formats.nibbles_to_bytes(np.tile(np.arange(16, dtype=np.uint8), (s.size, 2)))
    got = formats.dequant_nvfp4_parts(codes, g, np.stack([s, s], axis=1))
    for i in range(s.size):
        x = np.float32(Fraction(float(e4[i])) * Fraction(float(g)))     # one rounding of the exact product
        for j in range(32):
            c = (E2M1 + [-v for v in E2M1])[j % 16]
            assert got[i, j] == np.float32(Fraction(c) * Fraction(float(x))), (i, j)


def _e4m3_brute(t):
    """Nearest non-negative finite E4M3 value to t (>= 0) by search, ties to the
    even code, saturating at 448: the code byte."""
    vals = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    t = Fraction(float(t))
    best = min(range(127), key=lambda c: (abs(Fraction(float(vals[c])) - t), c & 1))
    return best


def _code_brute(w, x):
    """The code whose value E2M1(q) X is nearest to w (exact), ties to the even
    mantissa, sign bit from w."""
    sign = 8 if np.signbit(w) else 0
    wf = abs(Fraction(float(w)))
    xf = Fraction(float(x))
    best = min(range(8), key=lambda c: (abs(Fraction(E2M1[c]) * xf - wf), c & 1))
    return best | sign


@pytest.mark.parametrize("seed", [3, 4])
def test_nvfp4_pack_vs_brute_force(seed):
    g_rng = np.random.default_rng(seed)
    n, k = 6, 64
    mags = np.exp2(g_rng.uniform(-12, 12, size=(n, 4, 1)))  # blocks of very different size
    w = (g_rng.standard_normal((n, 4, 16)) * mags).astype(np.float32).reshape(n, k)
    w[2, 16:32] = 0.0
    w[3, 5] = -0.0
    w[4, 40] = np.float32(w[4, 32:48].max() * 0.999)       # near-equal block maxima
    codes, g, sb = formats.pack_nvfp4_parts(w)
    assert g == np.float32(np.float32(np.abs(w).max()) / np.float32(2688))
    q = formats.bytes_to_nibbles(codes)
    for r in range(n):
        for b in range(k // 16):
            blk = w[r, 16 * b:16 * b + 16]
            t = np.float32(np.float32(np.abs(blk).max()) / np.float32(6)) / g
            assert sb[r, b] == _e4m3_brute(np.float32(t)), (r, b)
            x = np.float32(torch.tensor([int(sb[r, b])], dtype=torch.uint8).view(torch.float8_e4m3fn).float().item()
                           * g)
            for j in range(16):
                want = 0 if x == 0 else _code_brute(blk[j], x)
                assert q[r, 16 * b + j] == want, (r, b, j)


def test_nvfp4_codes_at_exact_midpoints_and_just_beside_them():
    """Inputs one fp32 ulp either side of each E2M1 midpoint times X: the code
    moves across the midpoint exactly there (the fp64 quotient decides as the
    exact one would)."""
    # a block with amax 6 X (X = E4M3(0x38) g = g, sb = 1.0) and a second block holding the tensor maximum
    g = np.float32(2.0 ** -8)
    for xb in (0x38, 0x3B, 0x55, 0x6B):                     # X = E4M3 value of the byte times g
        e4 = torch.tensor([xb], dtype=torch.uint8).view(torch.float8_e4m3fn).double().item()
        x = np.float32(e4 * float(g))
        rows = []
        mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
        for m in mids:
            c = np.float32(m * float(x))                    # exact: at most 3 + 4 significant bits
            assert float(c) == m * float(x)
            rows += [np.nextafter(c, np.float32(0)), c, np.nextafter(c, np.float32(100))]
        # mids 0-3 in block 0, mids 4-6 in block 1; each block's element 15 is
        # 6 X, so amax_b = 6 X and t = E4M3(xb) exactly
        blk = np.zeros(32, np.float32)
        blk[:12] = rows[:12]
        blk[16:25] = rows[12:]
        blk[15] = blk[31] = np.float32(6 * float(x))
        big = np.zeros(32, np.float32)
        big[0] = np.float32(2688 * float(g))                # tensor amax -> g
        w = np.stack([blk, big]).astype(np.float32)
        codes, gg, sb = formats.pack_nvfp4_parts(w)
        assert gg == g and sb[0, 0] == xb and sb[0, 1] == xb
        q = formats.bytes_to_nibbles(codes)[0]
        pos = list(range(12)) + list(range(16, 25))
        for i, m in enumerate(mids):
            lo_c = E2M1.index(max(v for v in E2M1 if v < m))
            hi_c = E2M1.index(min(v for v in E2M1 if v > m))
            even = lo_c if lo_c % 2 == 0 else hi_c
            assert [q[pos[3 * i + j]] for j in range(3)] == [lo_c, even, hi_c], (xb, m)


def test_nvfp4_round_trip_is_exact():
    """W built from random codes and scales with g a power of two, every block
    holding a +-6 element and one block the scale 448: packing recovers g,
    every scale byte and every code, and dequant is exact."""
    rng = np.random.default_rng(41)
    n, k = 12, 128
    q = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    q[:, ::16] = rng.choice([7, 15], size=(n, k // 16))
    sb = rng.integers(1, 127, size=(n, k // 16)).astype(np.uint8)
    sb[5, 3] = 0x7E
    g = np.float32(2.0 ** -13)
    w = formats.dequant_nvfp4_parts(formats.nibbles_to_bytes(q), g, sb)
    c2, g2, sb2 = formats.pack_nvfp4_parts(w)
    assert g2 == g
    assert np.array_equal(sb2, sb)
    assert np.array_equal(formats.bytes_to_nibbles(c2), q)
    e4 = torch.from_numpy(sb.copy()).view(torch.float8_e4m3fn).double().numpy()
    e2 = np.array(E2M1 + [-v for v in E2M1])[q]
    want = e2.reshape(n, k // 16, 16) * (e4 * float(g))[:, :, None]
    assert np.array_equal(w.astype(np.float64), want.reshape(n, k))


def test_nvfp4_power_of_two_scaling_moves_only_the_tensor_scale():
    rng = np.random.default_rng(43)
    w = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32)
    c0, g0, s0 = formats.pack_nvfp4_parts(w)
    for j in (-30, -1, 1, 40):
        c1, g1, s1 = formats.pack_nvfp4_parts((w * np.float32(2.0 ** j)).astype(np.float32))
        assert np.array_equal(c1, c0) and np.array_equal(s1, s0)
        assert g1 == np.float32(g0 * np.float32(2.0 ** j))


def test_nvfp4_error_bound_and_block_maximum():
    """Below 6 X the error is at most half a step of the E2M1 grid (at most X,
    X / 4 below 2 X) plus the value's fp32 rounding; above 6 X (a scale that
    rounded down) it is the saturation gap, under 6 X / 16.  While the block
    scale is a normal E4M3 number the block's largest element codes to +-6."""
    rng = np.random.default_rng(47)
    w = (rng.standard_normal((32, 512)) * np.exp2(rng.uniform(-6, 6, (32, 1)))).astype(np.float32)
    codes, g, sb = formats.pack_nvfp4_parts(w)
    d = formats.dequant_nvfp4_parts(codes, g, sb).astype(np.float64)
    x = np.repeat(formats.nvfp4_decode_scales(sb, g).astype(np.float64), 16, axis=1)
    a = np.abs(w.astype(np.float64))
    err = np.abs(d - w)
    step = np.where(a <= 2 * x, 0.25 * x, np.where(a <= 4 * x, 0.5 * x, x))
    inside = a <= 6 * x
    assert np.all(err[inside] <= step[inside] * (1 + 2.0 ** -22))
    assert np.all(err[~inside] <= a[~inside] - 6 * x[~inside] * (1 - 2.0 ** -23))   # d = fl32(6 X)
    assert np.all(a[~inside] <= 6 * x[~inside] * (1 + 1 / 16) * (1 + 2.0 ** -20))
    q = formats.bytes_to_nibbles(codes).reshape(32, 32, 16) & 7
    top = np.argmax(np.abs(w).reshape(32, 32, 16), axis=2)
    normal = codecs.e4m3_decode(sb) >= 2.0 ** -6
    assert np.all(np.take_along_axis(q, top[:, :, None], 2)[:, :, 0][normal] == 7)


def test_nvfp4_zero_tensor_zero_block_and_vanishing_block():
    w = np.zeros((2, 64), np.float32)
    c, g, sb = formats.pack_nvfp4_parts(w)
    assert g == 0 and not sb.any() and not c.any()
    assert not formats.dequant_nvfp4_parts(c, g, sb).any()
    # a block so small against the tensor maximum that its E4M3 scale is 0
    w[0, 0] = 2688.0                                        # g = 1
    w[1, 16] = 2.0 ** -12                                   # t = 2^-12 / 6 < 2^-10: rounds to 0
    w[1, 33] = -(2.0 ** -9) * 6                             # t = 2^-9: the smallest subnormal scale
    c, g, sb = formats.pack_nvfp4_parts(w)
    assert g == 1.0
    assert sb[1, 1] == 0 and sb[1, 2] == 0x01 and sb[0, 1] == 0
    q = formats.bytes_to_nibbles(c)
    assert not q[1, 16:32].any()                            # X = 0: codes 0
    assert q[1, 33] == 15                                   # -6 X
    d = formats.dequant_nvfp4_parts(c, g, sb)
    assert d[1, 33] == np.float32(-(2.0 ** -9) * 6) and d[1, 16] == 0


def test_nvfp4_rejects_bad_input():
    with pytest.raises(ValueError):
        formats.pack_nvfp4(np.zeros((2, 48), np.float32))   # K not a multiple of 32
    w = np.zeros((2, 64), np.float32)
    w[1, 3] = np.inf
    with pytest.raises(ValueError):
        formats.pack_nvfp4(w)


def _e4m3_values():
    return torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def test_nvfp4_element_codes_where_an_fp32_quotient_would_land_on_a_midpoint():
    """Near each E2M1 midpoint m X there are inputs whose fp32 quotient
    fl32(w / X) is exactly m although w / X is not: the code must follow the
    exact quotient (brute force), not the rounded one."""
    e4 = _e4m3_values()
    g = np.float32(np.float32(1.0) / np.float32(2688))
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    hits = tested = 0
    for sbyte in range(8, 127):
        if tested == 6:
            break
        x = np.float32(np.float32(e4[sbyte]) * g)
        cands = []
        for m in mids:
            c = np.float32(m * float(x))
            lo = hi = c
            for _ in range(3):
                lo, hi = np.nextafter(lo, np.float32(0)), np.nextafter(hi, np.float32(1e30))
                for w in (lo, hi):
                    if np.float32(w / x) == np.float32(m):
                        cands.append(w)
        if not cands:
            continue
        tested += 1
        hits += len(cands)
        cands = cands[:30]
        w = np.zeros((2, 32), np.float32)
        w[0, 0] = 1.0                                        # tensor maximum: g = fl32(1 / 2688)
        w[1, :len(cands[:15])] = cands[:15]
        w[1, 16:16 + len(cands[15:])] = cands[15:]
        w[1, 15] = w[1, 31] = np.float32(6 * e4[sbyte] * float(g))
        codes, gg, sb = formats.pack_nvfp4_parts(w)
        assert gg == g and sb[1, 0] == sbyte and sb[1, 1] == sbyte
        q = formats.bytes_to_nibbles(codes)[1]
        for j in range(32):
            assert q[j] == _code_brute(w[1, j], x), (sbyte, j)
    assert tested == 6 and hits >= 12


def test_nvfp4_block_scale_follows_the_two_fp32_divisions():
    """Block maxima where E4M3 of fl32(fl32(amax_b / 6) / g) and E4M3 of the
    exact amax_b / (6 g) differ: the scale byte is the former (the stated
    reading), found here by brute force over the E4M3 values."""
    e4 = _e4m3_values()
    g = np.float32(np.float32(1.0) / np.float32(2688))
    picked = []
    for mi in range(8, 126):
        mid = (Fraction(float(e4[mi])) + Fraction(float(e4[mi + 1]))) / 2
        a0 = np.float32(float(mid * 6 * Fraction(float(g))))
        for a in (a0, np.nextafter(a0, np.float32(0)), np.nextafter(a0, np.float32(1e30))):
            t2 = np.float32(np.float32(a / np.float32(6)) / g)
            exact = Fraction(float(a)) / (6 * Fraction(float(g)))
            two = _e4m3_brute(t2)
            one = min(range(127), key=lambda c: (abs(Fraction(float(e4[c])) - exact), c & 1))
            if two != one:
                picked.append((a, two))
    assert len(picked) >= 4
    picked = picked[:8]
    w = np.zeros((2, 16 * len(picked)), np.float32)
    w[0, 0] = 1.0
    for b, (a, _) in enumerate(picked):
        w[1, 16 * b + 3] = a
    w = np.pad(w, ((0, 0), (0, (-w.shape[1]) % 32)))
    _, gg, sb = formats.pack_nvfp4_parts(w)
    assert gg == g
    assert [int(sb[1, b]) for b in range(len(picked))] == [two for _, two in picked]
