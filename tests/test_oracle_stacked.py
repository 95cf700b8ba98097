"""Pins of the stacked-adapter oracle (oracle/stacked.py): one adapter reduces
to the single-adapter oracle, a zero adapter drops out, the merged-weight
route agrees, and finite differences of L = sum(G * y) give dX, dA_top and
dB_top (y is linear in each of x, A_top and B_top)."""

import numpy as np

from oracle import lora, stacked


def _case(seed, m=5, k=64, n=48, ranks=(4, 8)):
    g = np.random.default_rng(seed)
    x = g.standard_normal((m, k))
    w = g.standard_normal((n, k)) * 0.1
    ads = [(g.standard_normal((r, k)) / np.sqrt(k), g.standard_normal((n, r)) * 0.1, float(2 * r)) for r in ranks]
    dy = g.standard_normal((m, n))
    return x, w, ads, dy


def test_single_adapter_is_the_lora_oracle():
    x, w, ads, dy = _case(1, ranks=(8,))
    a, b, alpha = ads[0]
    y, _ = lora.forward(x, w, a, b, alpha)
    assert np.allclose(stacked.forward(x, w, ads), y, rtol=1e-14, atol=1e-14)
    dx, da, db = lora.backward(x, dy, w, a, b, alpha)
    sdx, sda, sdb = stacked.backward(x, dy, w, ads)
    assert np.allclose(sdx, dx, rtol=1e-14, atol=1e-13)
    assert np.array_equal(sda, da) and np.array_equal(sdb, db)


def test_zero_frozen_adapter_drops_out():
    x, w, ads, dy = _case(2)
    a0, b0, al0 = ads[0]
    zeroed = [(a0, np.zeros_like(b0), al0), ads[1]]
    y1, _ = lora.forward(x, w, ads[1][0], ads[1][1], ads[1][2])
    assert np.allclose(stacked.forward(x, w, zeroed), y1, rtol=1e-14, atol=1e-14)
    dx1, _, _ = lora.backward(x, dy, w, ads[1][0], ads[1][1], ads[1][2])
    assert np.allclose(stacked.backward(x, dy, w, zeroed)[0], dx1, rtol=1e-14, atol=1e-13)


def test_merged_weight_route():
    x, w, ads, _ = _case(3, ranks=(4, 8, 4))
    merged = w.copy()
    for a, b, alpha in ads:
        merged = merged + (alpha / a.shape[0]) * (b @ a)
    assert np.allclose(stacked.forward(x, w, ads), x @ merged.T, rtol=1e-12, atol=1e-12)


def test_finite_differences_of_the_top_adapter_and_input():
    x, w, ads, g = _case(4, m=3, k=32, n=20, ranks=(4, 2))
    dx, da, db = stacked.backward(x, g, w, ads)
    loss = lambda xx, aa, bb: float(np.sum(g * stacked.forward(xx, w, ads[:-1] + [(aa, bb, ads[-1][2])])))
    a, b = ads[-1][0], ads[-1][1]
    h = 0.5    # y is linear in each argument: the central difference is exact up to rounding
    for (i, j) in [(0, 0), (2, 31), (1, 7)]:
        e = np.zeros_like(x); e[i, j] = h
        assert abs((loss(x + e, a, b) - loss(x - e, a, b)) / (2 * h) - dx[i, j]) <= 1e-10 * max(1, abs(dx[i, j]))
    for (i, j) in [(0, 0), (1, 31)]:
        e = np.zeros_like(a); e[i, j] = h
        assert abs((loss(x, a + e, b) - loss(x, a - e, b)) / (2 * h) - da[i, j]) <= 1e-10 * max(1, abs(da[i, j]))
    for (i, j) in [(0, 0), (19, 1)]:
        e = np.zeros_like(b); e[i, j] = h
        assert abs((loss(x, a, b + e) - loss(x, a, b - e)) / (2 * h) - db[i, j]) <= 1e-10 * max(1, abs(db[i, j]))
