"""GPU parity of the 8-bit-state AdamW step (ql_adamw8_step) against the
oracle (oracle/adamw8.py), through the C ABI: several tensors in one launch
(ragged last blocks, a tensor of one block, an all-zero gradient block),
several steps in a row; every code, every block scale, every parameter and
bf16 copy equal bit for bit (the codes are fp32 decisions taken in the same
order on both sides)."""

import sys

import numpy as np
import pytest
import torch

from oracle import adamw8
from quantized_base_lora_amd import binding as B

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("hp", [dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, grad_scale=1.0),
                                dict(lr=5e-3, beta1=0.8, beta2=0.95, eps=1e-6, weight_decay=0.01, grad_scale=0.25)])
def test_adamw8_bitwise_over_steps(lib, hp):
    g = np.random.default_rng(17)
    sizes = [16 * 4096, 5000 - 5000 % 8 + 8, 2048, 24]
    params = [(g.standard_normal(n) * 0.02).astype(np.float32) for n in sizes]
    dev = [torch.from_numpy(p.copy()).cuda() for p in params]
    states = [B.Adamw8State(n) for n in sizes]
    grads = [torch.empty(n, dtype=torch.float32, device="cuda") for n in sizes]
    bf = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for n in sizes]
    plan = B.Adamw8Plan([(dev[i], grads[i], states[i], bf[i]) for i in range(len(sizes))])
    ref = [(params[i], np.zeros(n, np.uint8), np.zeros(-(-n // 2048), np.float32), np.zeros(n, np.uint8),
            np.zeros(-(-n // 2048), np.float32)) for i, n in enumerate(sizes)]
    for t in range(1, 6):
        gnp = []
        for i, n in enumerate(sizes):
            gr = (g.standard_normal(n) * np.exp(g.standard_normal(n)) * 1e-3).astype(np.float32)
            if i == 0 and t == 2:
                gr[:2048] = 0.0                      # a block whose new moments only decay
            gnp.append(gr)
            grads[i].copy_(torch.from_numpy(gr))
        plan.step(t, **hp)
        torch.cuda.synchronize()
        for i, n in enumerate(sizes):
            p, mc, ma, vc, va = ref[i]
            p, mc, ma, vc, va, _, _ = adamw8.adamw8_step(p, gnp[i], mc, ma, vc, va, t, **hp)
            ref[i] = (p, mc, ma, vc, va)
            st = states[i]
            assert np.array_equal(dev[i].cpu().numpy().view(np.uint32), p.view(np.uint32)), (t, i, "param")
            assert np.array_equal(st.m.cpu().numpy(), mc), (t, i, "m codes")
            assert np.array_equal(st.v.cpu().numpy(), vc), (t, i, "v codes")
            assert np.array_equal(st.m_absmax.cpu().numpy().view(np.uint32), ma.view(np.uint32)), (t, i, "m scale")
            assert np.array_equal(st.v_absmax.cpu().numpy().view(np.uint32), va.view(np.uint32)), (t, i, "v scale")
            assert np.array_equal(bf[i].view(torch.int16).cpu().numpy().view(np.uint16), adamw8.bf16_copy(p))
        say(f"step {t}: every code, scale, parameter and bf16 copy equal to the oracle's")
