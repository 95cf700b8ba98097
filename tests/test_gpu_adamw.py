"""GPU parity of the fused AdamW adapter step (ql_adamw_step) against the
oracle (oracle/adamw.py, fp64), through the C ABI.

Bar, derived from the arithmetic: the kernel takes about ten fp32 roundings
per element and step, so over a few steps the moments stay within 1e-5 of
their largest magnitude; the parameter is rounded to fp32 twice per step
(after the decay and after the update), so it stays within 2 steps 2^-23
max|param| plus 1e-5 of the largest total update; the bf16 copy is bit-exact
against nearest-even rounding of the kernel's own fp32 parameters (both sides
decide the rounding on the same value)."""


def param_bound(steps, p_ref, p0):
    return 2 * steps * 2.0 ** -23 * np.max(np.abs(p_ref)) + 1e-5 * np.max(np.abs(p_ref - p0))

import sys

import numpy as np
import pytest
import torch

from oracle import adamw as oadamw
from oracle import codecs

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel(got, ref, scale):
    return float(np.max(np.abs(got.astype(np.float64) - ref)) / scale) if ref.size else 0.0


@pytest.mark.parametrize("hp", [
    dict(lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, grad_scale=1.0),
    dict(lr=1e-3, beta1=0.8, beta2=0.95, eps=1e-6, weight_decay=0.01, grad_scale=0.25),
])
def test_adamw_parity_multi_tensor(lib, hp):
    from quantized_base_lora_amd import binding as B
    g = np.random.default_rng(11)
    # adapter shapes of a Llama-3.1-8B gate projection (A [16, 4096], B [14336, 16]),
    # a small ragged one, an empty one; the last without a bf16 copy
    sizes = [16 * 4096, 14336 * 16, 8 * 36, 0, 1028]
    say(f"adamw parity sizes={sizes} hp={hp}")
    p0 = [(g.standard_normal(n) * 0.02).astype(np.float32) for n in sizes]
    dev = [dict(p=torch.from_numpy(a.copy()).cuda(), m=torch.zeros(n, device="cuda"),
                v=torch.zeros(n, device="cuda"),
                pb=torch.empty(n, dtype=torch.bfloat16, device="cuda") if i != 4 else None)
           for i, (a, n) in enumerate(zip(p0, sizes))]
    ref = [dict(p=a.astype(np.float64), m=np.zeros(n), v=np.zeros(n)) for a, n in zip(p0, sizes)]
    for t in range(1, 6):
        grads = [(g.standard_normal(n) * 10.0 ** g.uniform(-5, -1)).astype(np.float32) for n in sizes]
        if sizes[0]:
            grads[0][:64] = 0.0
        gd = [torch.from_numpy(x).cuda() for x in grads]
        B.adamw_step([(d["p"], gr, d["m"], d["v"], d["pb"]) for d, gr in zip(dev, gd)], t, **hp)
        for r, gr in zip(ref, grads):
            r["p"], r["m"], r["v"] = oadamw.adamw_step(r["p"], gr, r["m"], r["v"], t, hp["lr"], hp["beta1"],
                                                       hp["beta2"], hp["eps"], hp["weight_decay"],
                                                       grad_scale=hp["grad_scale"])
    torch.cuda.synchronize()
    for i, (d, r, a0) in enumerate(zip(dev, ref, p0)):
        if sizes[i] == 0:
            continue
        p, m, v = d["p"].cpu().numpy(), d["m"].cpu().numpy(), d["v"].cpu().numpy()
        ep = rel(p, r["p"], param_bound(5, r["p"], a0))
        em = rel(m, r["m"], np.max(np.abs(r["m"])))
        ev = rel(v, r["v"], np.max(np.abs(r["v"])))
        say(f"  tensor {i} n={sizes[i]}: param {ep:.2e} (of its bound), exp_avg {em:.2e}, exp_avg_sq {ev:.2e}")
        assert ep <= 1.0 and em <= 1e-5 and ev <= 1e-5, (i, ep, em, ev)
        if d["pb"] is not None:
            got = d["pb"].view(torch.int16).cpu().numpy().view(np.uint16)
            assert np.array_equal(got, codecs.bf16_encode(p)), i


def test_adamw_after_layer_backward(lib):
    """The step consumes the layer's own dA / dB in place and its bf16 copy
    feeds the next forward: parity on the gradients the layer produced."""
    from quantized_base_lora_amd import binding as B
    import helpers as H
    from oracle import formats as ofmt
    m, k, n, r, alpha = 96, 256, 192, 16, 32.0
    c = H.make_case(m, k, n, r, seed=5)
    qw = B.quant_pack(ofmt.FMT_NF4, torch.from_numpy(c["W"]).cuda())
    x, dy = H.bits_to_bf16_tensor(c["x"]), H.bits_to_bf16_tensor(c["dY"])
    a16, b16 = H.bits_to_bf16_tensor(c["A"]), H.bits_to_bf16_tensor(c["B"])
    a32, b32 = a16.float().contiguous(), b16.float().contiguous()
    y, u = B.linear_fwd(qw, x, a16, b16, alpha)
    _, da, db = B.linear_bwd(qw, x, dy, u, a16, b16, alpha)
    torch.cuda.synchronize()
    da_np, db_np, a0, b0 = da.cpu().numpy(), db.cpu().numpy(), a32.cpu().numpy(), b32.cpu().numpy()
    st = [torch.zeros_like(a32), torch.zeros_like(a32), torch.zeros_like(b32), torch.zeros_like(b32)]
    B.adamw_step([(a32, da, st[0], st[1], a16), (b32, db, st[2], st[3], b16)], 1, lr=1e-3, weight_decay=0.01)
    y2, _ = B.linear_fwd(qw, x, a16, b16, alpha)
    torch.cuda.synchronize()
    for got, g0, w0 in ((a32, da_np, a0), (b32, db_np, b0)):
        rp, _, _ = oadamw.adamw_step(w0, g0, np.zeros_like(w0), np.zeros_like(w0), 1, 1e-3, weight_decay=0.01)
        assert rel(got.cpu().numpy(), rp, param_bound(1, rp, w0)) <= 1.0
    assert torch.equal(a16.view(torch.int16).cpu(),
                       torch.from_numpy(codecs.bf16_encode(a32.cpu().numpy()).view(np.int16)).view(a16.shape))
    assert not torch.equal(y2.view(torch.int16), y.view(torch.int16))   # the adapters moved


def test_adamw_deterministic(lib):
    from quantized_base_lora_amd import binding as B
    g = torch.Generator(device="cuda").manual_seed(3)
    n = 65536
    base = [torch.randn(n, device="cuda", generator=g) for _ in range(4)]
    outs = []
    for _ in range(2):
        p, gr, m, v = (t.clone() for t in base)
        v.abs_()
        pb = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        B.adamw_step([(p, gr, m, v, pb)], 7, lr=3e-4, weight_decay=0.1, grad_scale=0.5)
        torch.cuda.synchronize()
        outs.append((p, m, v, pb))
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                           b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16))
