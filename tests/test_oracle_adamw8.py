"""Pins of the 8-bit-state AdamW oracle (oracle/adamw8.py) against things
other than itself: hand-worked levels and a hand-quantized block
(tests/golden/dyn8_levels.txt), an independent decoding of the code bits,
brute-force nearest-level search, the closed form of a first step from zero
state, the fp32-state AdamW oracle (itself pinned to torch.optim.AdamW) over
many steps, and error bounds of the block quantization."""

import os

import numpy as np
import pytest

from oracle import adamw, adamw8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "dyn8_levels.txt")
F32 = np.float32


def read_golden():
    levels, block, codes = [], None, None
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        t, rest = line.split(None, 1)
        if t in ("s", "u"):
            c, v = rest.split()
            levels.append((t == "s", int(c, 16), F32(float(v))))
        elif t == "block":
            block = np.array([float(v) for v in rest.split()], dtype=F32)
        elif t == "codes":
            codes = np.array([int(v, 16) for v in rest.split()], dtype=np.uint8)
    return levels, block, codes


def decode_bits(code, signed):
    """Independent decoding of one code from its bit description."""
    neg = signed and bool(code & 0x80)
    bits = 7 if signed else 8
    mag = code & ((1 << bits) - 1)
    if mag == 0:
        return 0.0
    s = format(mag, f"0{bits}b")
    z = s.index("1")
    frac_bits = s[z + 1:]
    f = len(frac_bits)
    q = int(frac_bits, 2) if f else 0
    v = (0.1 + 0.9 * (q + 1) / 2 ** f) / 10.0 ** z
    return -v if neg else v


def test_golden_levels():
    levels, _, _ = read_golden()
    for signed, code, want in levels:
        got = adamw8.dequantize(np.array([code], np.uint8), np.array([1.0], F32), signed)[0]
        assert got == want, (signed, hex(code), got, want)


def test_golden_block():
    _, block, want = read_golden()
    codes, absmax = adamw8.quantize(block, True)
    assert absmax[0] == 1.0
    assert np.array_equal(codes, want), [hex(c) for c in codes]


@pytest.mark.parametrize("signed", [True, False])
def test_levels_structure(signed):
    lv = adamw8.dynamic_levels(signed).astype(np.float64)
    b = 7 if signed else 8
    assert lv.size == 1 << b and lv[0] == 0 and lv[-1] == 1.0
    assert np.all(np.diff(lv) > 0)                       # the magnitude bits order the values
    assert lv[1] == F32(10.0 ** -(b - 1))                # smallest magnitude
    for z in range(b):                                   # 2^f evenly spaced levels per decade
        f = b - 1 - z
        sl = lv[1 << f:1 << (f + 1)]
        assert sl.size == 1 << f
        assert np.isclose(sl[-1], 10.0 ** -z, rtol=1e-7) and sl[0] > 0.1 * 10.0 ** -z
        if f >= 2:
            np.testing.assert_allclose(np.diff(sl), 0.9 / 2 ** f / 10.0 ** z, rtol=2e-5)
    for code in range(1 << (b + (1 if signed else 0))):
        got = adamw8.dequantize(np.array([code], np.uint8), np.array([1.0], F32), signed)[0]
        assert got == F32(decode_bits(code, signed)), hex(code)


@pytest.mark.parametrize("signed", [True, False])
def test_quantize_is_nearest_level(signed):
    """Brute force over every level in fp64: the code's level is a nearest one
    (ties and the fp32 sliver around each threshold aside)."""
    g = np.random.default_rng(3)
    n = 3 * adamw8.BLOCK + 77
    x = (g.standard_normal(n) * 10.0 ** g.uniform(-7, 0, n)).astype(F32)
    if not signed:
        x = np.abs(x)
    x[5] = 0
    codes, absmax = adamw8.quantize(x, signed)
    lv = adamw8.dynamic_levels(signed).astype(np.float64)
    a = np.repeat(absmax, adamw8.BLOCK)[:n].astype(np.float64)
    r = (x.astype(np.float32) / a.astype(np.float32)).astype(np.float64)
    best = np.argmin(np.abs(np.abs(r)[:, None] - lv[None, :]), axis=1)
    mag = codes & 0x7F if signed else codes
    diff = np.abs(np.abs(r) - lv[mag]) - np.abs(np.abs(r) - lv[best])
    assert np.all(diff <= 1e-7 * np.maximum(np.abs(r), 1e-7))
    if signed:
        assert np.all(((codes & 0x80) != 0) == ((x < 0) & (mag > 0)))
    # the block's largest element gets the top code; an all-zero block stores zeros
    for bi in range(len(absmax)):
        blk = np.abs(x[bi * adamw8.BLOCK:(bi + 1) * adamw8.BLOCK])
        assert absmax[bi] == blk.max() and mag[bi * adamw8.BLOCK + np.argmax(blk)] == (0x7F if signed else 0xFF)
    zc, za = adamw8.quantize(np.zeros(100, F32), signed)
    assert not zc.any() and not za.any()


@pytest.mark.parametrize("signed", [True, False])
def test_value_on_a_threshold_takes_the_lower_code(signed):
    """Inputs exactly on the decision thresholds (absmax 1, so r = x): each
    takes the lower of its two codes; just above it takes the upper one."""
    th = adamw8.thresholds(adamw8.dynamic_levels(signed))
    x = np.concatenate([[1.0], th]).astype(F32)
    c, a = adamw8.quantize(x, signed)
    assert a[0] == 1.0
    assert np.array_equal(c[1:].astype(np.int64), np.arange(th.size))
    up = np.nextafter(th, np.float32(2)).astype(F32)
    c2, _ = adamw8.quantize(np.concatenate([[1.0], up]).astype(F32), signed)
    assert np.array_equal(c2[1:].astype(np.int64), np.arange(1, th.size + 1))


def test_quantization_error_bound():
    """Within the [0.1, 1] decade the levels are 0.9/64 apart (signed): the
    dequantized value is within half a gap of the input, relative to absmax."""
    g = np.random.default_rng(4)
    x = g.uniform(-1, 1, 5000).astype(F32)
    x[0] = 1.0
    c, a = adamw8.quantize(x, True)
    d = adamw8.dequantize(c, a, True)
    big = np.abs(x) >= 0.1
    assert np.max(np.abs(d - x)[big]) <= 0.9 / 64 / 2 * (1 + 1e-5)


def test_first_step_from_zero_state():
    """From zero moments the parameter moves with the fp32 moments, which are
    the closed form (1 - b1) g and (1 - b2) g^2: the first step equals the
    fp32-state AdamW step (oracle/adamw.py, fp64) up to fp32 rounding, and its
    sign-descent limit lr * sign(g) for eps -> 0."""
    g = np.random.default_rng(5)
    n = 4096 + 512
    p = (g.standard_normal(n) * 0.02).astype(F32)
    gr = (g.standard_normal(n) * 1e-3).astype(F32)
    z8 = np.zeros(n, np.uint8)
    za = np.zeros(-(-n // adamw8.BLOCK), F32)
    th, mc, ma, vc, va, m, v = adamw8.adamw8_step(p, gr, z8, za, z8, za, 1, 1e-3, 0.9, 0.999, 1e-8, 0.01)
    rp, rm, rv = adamw.adamw_step(p, gr, np.zeros(n), np.zeros(n), 1, 1e-3, 0.9, 0.999, 1e-8, 0.01)
    np.testing.assert_allclose(m, rm, rtol=2e-7)
    np.testing.assert_allclose(v, rv, rtol=3e-7)
    np.testing.assert_allclose(th, rp, rtol=0, atol=2.5e-8)      # a few fp32 roundings of |p| < 0.1
    th0, *_ = adamw8.adamw8_step(p, gr, z8, za, z8, za, 1, 1e-3, 0.9, 0.999, 0.0, 0.0)
    np.testing.assert_allclose(th0, p - F32(1e-3) * np.sign(gr), rtol=0, atol=1e-8)   # 2 ulp of |p| < 0.1
    # the stored state is the quantized fp32 moments
    assert np.array_equal(mc, adamw8.quantize(m, True)[0]) and np.array_equal(ma, adamw8.quantize(m, True)[1])
    assert np.array_equal(vc, adamw8.quantize(v, False)[0])


@pytest.mark.parametrize("t,lr,b1,b2,eps,wd,gs", [(1, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1.0),
                                                  (7, 2e-4, 0.8, 0.95, 1e-6, 0.01, 0.5),
                                                  (40, 5e-2, 0.5, 0.9, 1e-3, 0.1, 2.0)])
def test_step_is_adamw_on_the_dequantized_state(t, lr, b1, b2, eps, wd, gs):
    """One step from an arbitrary 8-bit state equals the fp32-state AdamW step
    (oracle/adamw.py in fp64, pinned to torch.optim.AdamW) started from the
    dequantized moments, up to fp32 rounding; the new state is the
    quantization of the new fp32 moments."""
    g = np.random.default_rng(10 + t)
    n = adamw8.BLOCK + 1000
    p = (g.standard_normal(n) * 0.02).astype(F32)
    gr = (g.standard_normal(n) * 1e-3).astype(F32)
    mc = g.integers(0, 256, n).astype(np.uint8)
    vc = g.integers(0, 256, n).astype(np.uint8)
    ma = np.array([2e-4, 5e-4], F32)
    va = np.array([3e-7, 1e-6], F32)
    th, mc2, ma2, vc2, va2, m, v = adamw8.adamw8_step(p, gr, mc, ma, vc, va, t, lr, b1, b2, eps, wd, gs)
    md, vd = adamw8.dequantize(mc, ma, True), adamw8.dequantize(vc, va, False)
    rp, rm, rv = adamw.adamw_step(p, gr, md, vd, t, lr, b1, b2, eps, wd, grad_scale=gs)
    # fp32 rounding bounds: a few units in the last place of the terms summed
    # (the moment updates can cancel)
    gg = gr.astype(np.float64) * gs
    assert np.all(np.abs(m - rm) <= 3e-7 * (np.abs(b1 * md) + np.abs((1 - b1) * gg)) + 1e-30)
    assert np.all(np.abs(v - rv) <= 3e-7 * (np.abs(b2 * vd) + np.abs((1 - b2) * gg * gg)) + 1e-30)
    np.testing.assert_allclose(th, rp, rtol=0, atol=2.5e-8 + 5e-7 * lr)
    assert np.array_equal(mc2, adamw8.quantize(m, True)[0]) and np.array_equal(ma2, adamw8.quantize(m, True)[1])
    assert np.array_equal(vc2, adamw8.quantize(v, False)[0]) and np.array_equal(va2, adamw8.quantize(v, False)[1])


def test_tracks_fp32_state_adamw():
    """Over 30 steps the 8-bit-state optimizer stays near the fp32-state one
    (the parameter displacement agrees to within 10 %: the quantization noise
    of the moments), and each stored moment is within its quantization bound
    of the fp32 moment it was quantized from."""
    g = np.random.default_rng(6)
    n = 2 * adamw8.BLOCK
    p0 = (g.standard_normal(n) * 0.02).astype(F32)
    p8, mc, ma, vc, va = p0.copy(), np.zeros(n, np.uint8), np.zeros(2, F32), np.zeros(n, np.uint8), np.zeros(2, F32)
    pr, mr, vr = p0.astype(np.float64), np.zeros(n), np.zeros(n)
    scale = np.exp(g.standard_normal(n)).astype(F32) * F32(1e-3)
    for t in range(1, 31):
        gr = (g.standard_normal(n).astype(F32) * scale + F32(2e-4)).astype(F32)
        p8, mc, ma, vc, va, m, v = adamw8.adamw8_step(p8, gr, mc, ma, vc, va, t, 1e-3, 0.9, 0.999, 1e-8, 0.0)
        pr, mr, vr = adamw.adamw_step(pr, gr, mr, vr, t, 1e-3, 0.9, 0.999, 1e-8, 0.0)
        md = adamw8.dequantize(mc, ma, True)
        assert np.max(np.abs(md - m)) <= np.max(np.abs(m)) * 0.9 / 64 / 2 * 1.001 + 1e-12
    d8, dr = p8.astype(np.float64) - p0, pr - p0
    assert np.linalg.norm(d8 - dr) / np.linalg.norm(dr) < 0.1


def test_bf16_copy():
    x = np.array([1.0, 1.00390625, 1.005859375, -2.5], F32)
    assert list(adamw8.bf16_copy(x)) == [0x3F80, 0x3F80, 0x3F81, 0xC020]
