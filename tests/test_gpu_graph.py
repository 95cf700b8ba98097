"""A layer step captured into a HIP graph, with independent projections on
parallel streams, replays bit for bit like eager launches.

The step is captured once and replayed several times, with eager work and
synchronizations between the replays (the outputs are poisoned with NaN each
time), and every replay is compared with the eager result.  Covers the split
path (at most 64 tokens, partials in the workspace), the 256-row tiles, and
the FP8 base on fp8 matrix cores."""

import sys

import numpy as np
import pytest
import torch

import helpers as H
from oracle import formats as ofmt
from quantized_base_lora_amd import binding as B

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# name, fmt, m, [(k, n), ...] (the projections run side by side), r, alpha
CASES = [
    ("nf4_m40", ofmt.FMT_NF4, 40, [(256, 512), (512, 256), (256, 256)], 16, 32.0),
    ("q40_m300", ofmt.FMT_Q4_0, 300, [(256, 384), (384, 256)], 8, 16.0),
    ("fp8_m200", ofmt.FMT_FP8, 200, [(256, 320), (320, 256)], 32, 64.0),
]


def setup(fmt, m, shapes, r, seed):
    projs = []
    for i, (k, n) in enumerate(shapes):
        c = H.make_case(m, k, n, r, seed=seed + i)
        d = {"qw": B.quant_pack(fmt, torch.from_numpy(c["W"]).cuda()),
             "x": H.bits_to_bf16_tensor(c["x"]), "dy": H.bits_to_bf16_tensor(c["dY"]),
             "a": H.bits_to_bf16_tensor(c["A"]), "b": H.bits_to_bf16_tensor(c["B"]),
             "y": torch.empty((m, n), dtype=torch.bfloat16, device="cuda"),
             "u": torch.empty((m, r), dtype=torch.float32, device="cuda"),
             "dx": torch.empty((m, k), dtype=torch.bfloat16, device="cuda"),
             "da": torch.empty((r, k), dtype=torch.float32, device="cuda"),
             "db": torch.empty((n, r), dtype=torch.float32, device="cuda"),
             "wsf": torch.empty(max(256, B.workspace_bytes(B.OP_FWD, fmt, n, k, m, r)), dtype=torch.uint8,
                                device="cuda"),
             "ws": torch.empty(max(256, B.workspace_bytes(B.OP_BWD, fmt, n, k, m, r)), dtype=torch.uint8,
                               device="cuda")}
        projs.append(d)
    return projs


OUTS = ("y", "u", "dx", "da", "db")


def step(projs, alpha, main, side):
    """forward of every projection on its own stream, join, then backward likewise"""
    for phase in ("fwd", "bwd"):
        fork = torch.cuda.Event()
        fork.record(main)
        for d, st in zip(projs, side):
            st.wait_event(fork)
            if phase == "fwd":
                B.linear_fwd(d["qw"], d["x"], d["a"], d["b"], alpha, y=d["y"], u=d["u"], ws=d["wsf"], stream=st)
            else:
                B.linear_bwd(d["qw"], d["x"], d["dy"], d["u"], d["a"], d["b"], alpha, dx=d["dx"], da=d["da"],
                             db=d["db"], ws=d["ws"], stream=st)
        for st in side[:len(projs)]:
            join = torch.cuda.Event()
            join.record(st)
            main.wait_event(join)


def poison(projs):
    for d in projs:
        for k in OUTS:
            d[k].fill_(float("nan"))


def snapshot(projs):
    return [{k: d[k].detach().clone() for k in OUTS} for d in projs]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_graph_replay_bitwise(lib, case):
    name, fmt, m, shapes, r, alpha = case
    say(f"graph replay {name}: fmt={fmt} m={m} shapes={shapes} r={r}")
    projs = setup(fmt, m, shapes, r, seed=len(name) * 7)
    main = torch.cuda.Stream()
    side = [torch.cuda.Stream() for _ in projs]
    with torch.cuda.stream(main):
        poison(projs)
        step(projs, alpha, main, side)
    torch.cuda.synchronize()
    ref = snapshot(projs)
    for d, rf in zip(projs, ref):
        for k in OUTS:
            assert torch.isfinite(rf[k].float()).all(), (name, k)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=main):
        step(projs, alpha, main, side)
    torch.cuda.synchronize()
    for rep in range(3):
        with torch.cuda.stream(main):
            poison(projs)                       # eager work between replays
            junk = torch.randn(1 << 16, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for i, (d, rf) in enumerate(zip(projs, ref)):
            for k in OUTS:
                a = d[k].view(torch.int16) if d[k].dtype == torch.bfloat16 else d[k].view(torch.int32)
                b = rf[k].view(torch.int16) if rf[k].dtype == torch.bfloat16 else rf[k].view(torch.int32)
                assert torch.equal(a, b), (name, rep, i, k)
    say(f"  3 replays bitwise equal to eager")
