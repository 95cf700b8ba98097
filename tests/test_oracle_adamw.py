"""Pins of the AdamW oracle (oracle/adamw.py) against things other than itself:
PyTorch's AdamW run in fp64, closed forms of the first step and of a constant
gradient, scale invariance, and the fixed point of a zero gradient."""

import numpy as np
import pytest
import torch

from oracle import adamw, codecs


def torch_adamw(p0, grads, lr, betas, eps, wd):
    """torch.optim.AdamW over a list of gradients, in fp64."""
    p = torch.nn.Parameter(torch.from_numpy(np.array(p0, dtype=np.float64)))
    opt = torch.optim.AdamW([p], lr=lr, betas=betas, eps=eps, weight_decay=wd, foreach=False)
    for g in grads:
        p.grad = torch.from_numpy(np.array(g, dtype=np.float64))
        opt.step()
    st = opt.state[p]
    return p.detach().numpy(), st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()


@pytest.mark.parametrize("lr,betas,eps,wd,gs", [
    (2e-4, (0.9, 0.999), 1e-8, 0.0, 1.0),
    (1e-3, (0.8, 0.95), 1e-6, 0.01, 0.25),
    (5e-2, (0.5, 0.9), 1e-3, 0.1, 3.0),
])
def test_matches_torch_adamw_over_steps(lr, betas, eps, wd, gs):
    g = np.random.default_rng(7)
    n = 257
    p0 = g.standard_normal(n) * 0.02
    grads = [g.standard_normal(n) * 10.0 ** g.uniform(-4, 0) for _ in range(6)]
    grads[2][:9] = 0.0
    rp, rm, rv = torch_adamw(p0, [gr * gs for gr in grads], lr, betas, eps, wd)
    p, m, v = p0, np.zeros(n), np.zeros(n)
    for t, gr in enumerate(grads, start=1):
        p, m, v = adamw.adamw_step(p, gr, m, v, t, lr, betas[0], betas[1], eps, wd, grad_scale=gs)
    np.testing.assert_allclose(m, rm, rtol=1e-13, atol=0)
    np.testing.assert_allclose(v, rv, rtol=1e-13, atol=0)
    np.testing.assert_allclose(p, rp, rtol=1e-13, atol=1e-16)


def test_first_step_is_sign_descent():
    """t = 1 from zero moments with eps = 0: m_hat = g and v_hat = g^2, so the
    Adam term is lr * sign(g); the decay multiplies theta by 1 - lr * lambda."""
    g = np.random.default_rng(3)
    p0 = g.standard_normal(100)
    gr = g.standard_normal(100)
    gr[5] = 0.0
    lr, wd = 1e-2, 0.05
    p, m, v = adamw.adamw_step(p0, gr, np.zeros(100), np.zeros(100), 1, lr, 0.9, 0.999, 0.0, wd)
    nz = gr != 0
    want = p0 * (1 - lr * wd) - lr * np.sign(gr)
    np.testing.assert_allclose(p[nz], want[nz], rtol=1e-14, atol=1e-16)
    assert np.isnan(p[5])          # 0 / (0 + 0): eps = 0 is only for this closed form
    np.testing.assert_allclose(m, 0.1 * gr, rtol=1e-14)
    np.testing.assert_allclose(v, 0.001 * gr * gr, rtol=1e-14)


def test_constant_gradient_moves_by_lr_per_step():
    """With a constant gradient the bias-corrected moments equal g and g^2 at
    every step, so theta falls by lr * g / (|g| + eps) per step (no decay)."""
    g = np.random.default_rng(4)
    n, lr, eps = 64, 1e-3, 1e-8
    p0 = g.standard_normal(n)
    gr = g.standard_normal(n)
    p, m, v = p0, np.zeros(n), np.zeros(n)
    for t in range(1, 21):
        p, m, v = adamw.adamw_step(p, gr, m, v, t, lr, 0.9, 0.999, eps)
    np.testing.assert_allclose(p, p0 - 20 * lr * gr / (np.abs(gr) + eps), rtol=0, atol=1e-13)


def test_gradient_scale_invariance():
    """With eps = 0 the update does not depend on the gradient's scale."""
    g = np.random.default_rng(5)
    n = 50
    p0 = g.standard_normal(n)
    grads = [g.standard_normal(n) for _ in range(4)]
    pa, ma, va = p0, np.zeros(n), np.zeros(n)
    pb, mb, vb = p0, np.zeros(n), np.zeros(n)
    for t, gr in enumerate(grads, start=1):
        pa, ma, va = adamw.adamw_step(pa, gr, ma, va, t, 1e-3, 0.9, 0.99, 0.0, 0.01)
        pb, mb, vb = adamw.adamw_step(pb, gr * 1024.0, mb, vb, t, 1e-3, 0.9, 0.99, 0.0, 0.01)
    np.testing.assert_allclose(pa, pb, rtol=1e-14)


def test_zero_gradient_without_decay_is_a_fixed_point():
    p0 = np.random.default_rng(6).standard_normal(32)
    p, m, v = adamw.adamw_step(p0, np.zeros(32), np.zeros(32), np.zeros(32), 1, 1e-2, 0.9, 0.999, 1e-8)
    assert np.array_equal(p, p0) and not m.any() and not v.any()


def test_bf16_copy_matches_torch_cast():
    x = np.random.default_rng(8).standard_normal(4096).astype(np.float32) * np.float32(0.05)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(adamw.bf16_copy(x), want)
    assert np.array_equal(adamw.bf16_copy(x), codecs.bf16_encode(x))


def test_rejects_step_zero():
    with pytest.raises(ValueError):
        adamw.adamw_step(np.zeros(4), np.zeros(4), np.zeros(4), np.zeros(4), 0, 1e-3)
