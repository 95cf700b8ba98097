"""The 32-layer Llama-3.1-8B NF4 stack at full size, base streamed from pinned
host memory through two device slots, against the same stack resident in
HBM: every output of every layer bitwise equal (max abs difference 0.0), at
2048 tokens (256-row tiles) and 16 tokens (split path), with the grouped
calls the benchmark uses, and at 32 tokens one call per projection (the
split path whose reduction also writes dA and dB).  The oracle checks layers
0 and 31: their packed bytes bit for bit and every output on every row.
(Soup page, "Correctness" paragraph: a streamed run must equal the resident
run with the same numerics exactly.)"""

import sys

import numpy as np
import pytest
import torch

import helpers as H
from oracle import formats as ofmt
from quantized_base_lora_amd import stack, synth

pytestmark = pytest.mark.gpu

WL = synth.WORKLOADS["llama3.1_8b_nf4_stack32"]
L = 32
CHECKED = (0, L - 1)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def base(lib):
    say(f"building {L} packed Llama-3.1-8B NF4 layers in pinned host memory")
    layout, host, kept = stack.build_host_images(WL, L, keep_w=CHECKED)
    ref = {}
    for layer in CHECKED:
        for pi, p in enumerate(WL.projs):
            w = kept[(layer, pi)].numpy()
            c, s = ofmt.pack(WL.fmt, w)
            co, cb, so, sb = layout.offsets[pi]
            img = host[layer]
            assert H.packed_equal(WL.fmt, img[co:co + cb].numpy(), img[so:so + sb].numpy(), c, s), (layer, p.name)
            ref[(layer, pi)] = ofmt.dequant(WL.fmt, c, s)
        say(f"  layer {layer}: packed bytes equal the oracle's")
    yield layout, host, ref


@pytest.mark.parametrize("m,grouped", [(2048, True), (16, True), (32, False)],
                         ids=["m2048-grouped", "m16-grouped", "m32-single-calls"])
def test_stack_streamed_equals_resident_full_size(base, m, grouped):
    layout, host, ref = base
    say(f"stack of {L} layers, {m} tokens, {'grouped' if grouped else 'single'} calls")
    acts = stack.layer_inputs(WL, m, L)
    groups = stack.layer_groups(WL.projs) if grouped else None
    dev_imgs = [h.to("cuda") for h in host]
    o_res = stack.layer_outputs(WL, m, L)
    stack.Stack(layout, WL.r, WL.alpha, images_dev=dev_imgs).run(acts, o_res, groups)
    torch.cuda.synchronize()
    del dev_imgs
    st = stack.Stack(layout, WL.r, WL.alpha, images_host=host, n_slots=2)
    o_st = stack.layer_outputs(WL, m, L)
    st.run(acts, o_st, groups)
    torch.cuda.synchronize()
    stats = st.pool.stats()
    st.close()
    equal, first, worst = stack.compare_outputs(o_res, o_st)
    say(f"  streamed vs resident: equal={equal} max abs difference {worst}")
    assert equal and worst == 0.0, first
    assert stats["copies"] == 2 * L - 2 and stats["bytes"] == stats["copies"] * layout.nbytes, stats
    for layer in CHECKED:
        for pi, p in enumerate(WL.projs):
            a, o = acts[layer][pi], o_st[layer][pi]
            r = H.oracle_outputs(a["x"], a["dy"], a["a"], a["b"], ref[(layer, pi)], WL.alpha)
            got = {"y": o["y"], "U": o["u"], "dX": o["dx"], "dA": o["da"], "dB": o["db"]}
            for key in ("y", "U", "dX", "dA", "dB"):
                e = H.rel(H.f32_host(got[key]), r[key])
                assert e <= H.FWD_TOL, (layer, p.name, key, e)
        say(f"  layer {layer}: every output within {H.FWD_TOL} of the oracle on all {m} rows")
