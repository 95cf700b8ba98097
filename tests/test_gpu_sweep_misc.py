"""Seeded sweeps of the other calls against the oracle, bit for bit: packing
(every format, random shapes, rows spread over 60 decades of magnitude, heavy
tails, zero runs and integer-valued rows), the FP8 activation split (both of
its kernels: rows up to 4096 and longer ones) and the 8-bit AdamW step
(random tensor sizes, three steps)."""

import sys

import numpy as np
import pytest
import torch

import helpers as H
from oracle import adamw8, formats as ofmt, lora as olora
from quantized_base_lora_amd import synth

pytestmark = pytest.mark.gpu

FMTS = [ofmt.FMT_Q4_0, ofmt.FMT_NF4, ofmt.FMT_FP8, ofmt.FMT_MXFP4, ofmt.FMT_Q8_0, ofmt.FMT_NVFP4]


def weights(fmt, seed):
    g = np.random.default_rng(seed)
    kb = 64 if fmt == ofmt.FMT_NF4 else 32
    n = 32 * int(g.integers(1, 9))
    k = kb * int(g.integers(1, 2048 // kb + 1))
    w = g.standard_normal((n, k)).astype(np.float32)
    # per-row magnitudes over 60 decades (kept inside each format's range below)
    lo, hi = (-12, 4) if fmt in (ofmt.FMT_Q4_0, ofmt.FMT_Q8_0) else (-30, 30)
    if fmt in (ofmt.FMT_FP8, ofmt.FMT_NVFP4):
        lo, hi = -3, 3                               # one tensor scale: rows within a few decades
    w *= (10.0 ** g.uniform(lo, hi, (n, 1))).astype(np.float32)
    w[0] = np.trunc(w[0] / np.abs(w[0]).max() * 7)   # integer-valued row
    w[1, : k // 2] = 0                               # a zero run
    w[2] = (g.standard_t(2, k) * 0.02).astype(np.float32)   # heavy tails
    return w.astype(np.float32)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("seed", range(6))
def test_sweep_pack_bitexact(lib, fmt, seed):
    from quantized_base_lora_amd import binding as B
    w = weights(fmt, 500 + 10 * fmt + seed)
    print(f"pack sweep fmt={fmt} seed={seed} shape={w.shape}", flush=True)
    qw = B.quant_pack(fmt, torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    c, s = ofmt.pack(fmt, w)
    assert np.array_equal(H.tensor_bytes(qw.codes), np.ascontiguousarray(c).ravel())
    assert np.array_equal(H.tensor_bytes(qw.scales), H.scales_bytes(fmt, s))


@pytest.mark.parametrize("seed", range(8))
def test_sweep_act_split_bitexact(lib, seed):
    from quantized_base_lora_amd import binding as B
    g = np.random.default_rng(700 + seed)
    m = int(g.integers(1, 80))
    k = 16 * int(g.integers(1, 257)) if seed % 2 else 16 * int(g.integers(257, 801))   # <= 4096 / longer rows
    x = (g.standard_normal((m, k)) * (10.0 ** g.uniform(-20, 20, (m, 1)))).astype(np.float32)
    x[0] = 0
    print(f"act split sweep m={m} k={k}", flush=True)
    bits = synth.to_bf16_bits(x)
    hi, lo, s = B.act_quant_e4m3(H.bits_to_bf16_tensor(bits))
    rh, rl, rs = olora.act_split_e4m3(synth.bf16_bits_to_f32(bits))
    assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(hi.cpu().numpy(), rh)
    assert np.array_equal(lo.cpu().numpy(), rl)


@pytest.mark.parametrize("seed", range(4))
def test_sweep_adamw8_bitexact(lib, seed):
    from quantized_base_lora_amd import binding as B
    g = np.random.default_rng(900 + seed)
    sizes = [8 * int(g.integers(1, 3000)) for _ in range(int(g.integers(1, 5)))]
    hp = dict(lr=float(10.0 ** g.uniform(-4, -2)), beta1=0.9, beta2=float(g.choice([0.95, 0.999])),
              eps=1e-8, weight_decay=float(g.choice([0.0, 0.01])), grad_scale=float(g.choice([1.0, 0.5])))
    print(f"adamw8 sweep sizes={sizes} hp={hp}", flush=True)
    params = [(g.standard_normal(n) * 0.02).astype(np.float32) for n in sizes]
    dev = [torch.from_numpy(p.copy()).cuda() for p in params]
    states = [B.Adamw8State(n) for n in sizes]
    grads = [torch.empty(n, dtype=torch.float32, device="cuda") for n in sizes]
    bf = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for n in sizes]
    plan = B.Adamw8Plan([(dev[i], grads[i], states[i], bf[i]) for i in range(len(sizes))])
    ref = [(params[i], np.zeros(n, np.uint8), np.zeros(-(-n // 2048), np.float32), np.zeros(n, np.uint8),
            np.zeros(-(-n // 2048), np.float32)) for i, n in enumerate(sizes)]
    for t in range(1, 4):
        gn = [(g.standard_normal(n) * (10.0 ** g.uniform(-6, 0))).astype(np.float32) for n in sizes]
        for i in range(len(sizes)):
            grads[i].copy_(torch.from_numpy(gn[i]))
        plan.step(t, **hp)
        torch.cuda.synchronize()
        for i, n in enumerate(sizes):
            p, mc, ma, vc, va = ref[i]
            p, mc, ma, vc, va, _, _ = adamw8.adamw8_step(p, gn[i], mc, ma, vc, va, t, **hp)
            ref[i] = (p, mc, ma, vc, va)
            st = states[i]
            assert np.array_equal(dev[i].cpu().numpy().view(np.uint32), p.view(np.uint32)), (t, i)
            assert np.array_equal(st.m.cpu().numpy(), mc) and np.array_equal(st.v.cpu().numpy(), vc), (t, i)
            assert np.array_equal(st.m_absmax.cpu().numpy().view(np.uint32), ma.view(np.uint32)), (t, i)
            assert np.array_equal(st.v_absmax.cpu().numpy().view(np.uint32), va.view(np.uint32)), (t, i)
