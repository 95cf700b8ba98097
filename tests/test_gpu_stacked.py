"""Stacked adapters on the GPU against the stacked oracle: the concatenation
kernel (ql_stack_adapters) bit for bit, then forward / backward through the
layer's own kernels with the concatenated adapter, to the layer tolerance."""

import sys

import numpy as np
import pytest
import torch

import helpers as H
from oracle import codecs, formats as ofmt, stacked
from quantized_base_lora_amd import synth

pytestmark = pytest.mark.gpu

CASES = [
    # name, fmt, m, k, n, [(r, alpha), ...] top last
    ("nf4_split_2x8", ofmt.FMT_NF4, 64, 512, 384, [(8, 16.0), (8, 16.0)]),
    ("mxfp4_tiles_4_12", ofmt.FMT_MXFP4, 300, 320, 224, [(4, 8.0), (12, 36.0)]),
    ("q40_m16_3_adapters", ofmt.FMT_Q4_0, 16, 1024, 160, [(8, 8.0), (16, 64.0), (8, 32.0)]),
]


def random_cases(count=10):
    """Seeded stacks: 2-4 adapters whose ranks sum to 8, 16 or 32, alphas with
    non-power-of-two ratios, every format, token counts on every path."""
    g = np.random.default_rng(77)
    fmts = [ofmt.FMT_Q4_0, ofmt.FMT_NF4, ofmt.FMT_FP8, ofmt.FMT_MXFP4, ofmt.FMT_Q8_0, ofmt.FMT_NVFP4]
    out = []
    for i in range(count):
        fmt = fmts[i % len(fmts)]
        R = int(g.choice([8, 16, 32]))
        parts = int(g.integers(2, 5))
        cuts = sorted(int(x) for x in g.choice(np.arange(1, R), size=parts - 1, replace=False))
        ranks = [b - a for a, b in zip([0] + cuts, cuts + [R])]
        # alphas cross the C ABI as fp32: draw them as fp32 values
        spec = [(r, float(np.float32(np.round(g.uniform(0.5, 4.0) * r, 2)))) for r in ranks]
        m = int(g.choice([5, 16, 40, 96, 300]))
        k = (64 if fmt == ofmt.FMT_NF4 else 32) * int(g.integers(2, 17))
        n = 32 * int(g.integers(1, 13))
        out.append((f"random{i}_fmt{fmt}_m{m}_R{R}_{parts}", fmt, m, k, n, spec))
    return out


CASES += random_cases()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_stacked_parity(lib, case):
    from quantized_base_lora_amd import binding as B
    name, fmt, m, k, n, spec = case
    print(f"stacked {name}: m={m} k={k} n={n} adapters={spec}", flush=True)
    g = np.random.default_rng(len(name))
    c = H.make_case(m, k, n, 8, seed=len(name) + 7)
    ads_bits = []
    for r, alpha in spec:
        a = synth.to_bf16_bits((g.standard_normal((r, k)) / np.sqrt(k)).astype(np.float32))
        b = synth.to_bf16_bits((g.standard_normal((n, r)) * 0.01).astype(np.float32))
        ads_bits.append((a, b, alpha))
    ads = [(H.bits_to_bf16_tensor(a), H.bits_to_bf16_tensor(b), alpha) for a, b, alpha in ads_bits]
    a_cat, b_cat, alpha_cat = B.stack_adapters(ads)
    torch.cuda.synchronize()
    # the concatenation, bit for bit: A rows and the top block copied, frozen blocks scaled once
    R = sum(r for r, _ in spec)
    s_top = np.float64(spec[-1][1]) / spec[-1][0]
    want_a = np.concatenate([a for a, _, _ in ads_bits], axis=0)
    assert np.array_equal(H.bf16_tensor_bits(a_cat).reshape(R, k), want_a)
    blocks = []
    for i, (a, b, alpha) in enumerate(ads_bits):
        if i == len(ads_bits) - 1:
            blocks.append(b)
        else:
            ci = np.float32((np.float64(alpha) / a.shape[0]) / s_top)
            blocks.append(codecs.bf16_encode((synth.bf16_bits_to_f32(b) * ci).astype(np.float32)))
    assert np.array_equal(H.bf16_tensor_bits(b_cat).reshape(n, R), np.concatenate(blocks, axis=1))
    assert alpha_cat == np.float32(s_top) * np.float32(R)
    # the layer with the concatenated adapter against the stacked definition
    qw = B.quant_pack(fmt, torch.from_numpy(c["W"]).cuda())
    x, dy = H.bits_to_bf16_tensor(c["x"]), H.bits_to_bf16_tensor(c["dY"])
    y, u = B.linear_fwd(qw, x, a_cat, b_cat, alpha_cat)
    dx, da, db = B.linear_bwd(qw, x, dy, u, a_cat, b_cat, alpha_cat)
    da_top, db_top = B.top_grads(da, db, spec[-1][0])
    torch.cuda.synchronize()
    _, _, wd = H.oracle_packed(fmt, c["W"])
    f32 = synth.bf16_bits_to_f32
    oads = [(f32(a), f32(b), alpha) for a, b, alpha in ads_bits]
    ry = stacked.forward(f32(c["x"]), wd, oads)
    rdx, rda, rdb = stacked.backward(f32(c["x"]), f32(c["dY"]), wd, oads)
    for key, got, ref in (("y", y, ry), ("dX", dx, rdx), ("dA_top", da_top, rda), ("dB_top", db_top, rdb)):
        e = H.rel(got.float().cpu().numpy(), ref)
        print(f"  {key}: rel err {e:.3e}", flush=True)
        assert e <= H.FWD_TOL, (key, e)
