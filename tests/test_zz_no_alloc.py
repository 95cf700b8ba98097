"""The allocation-free backward (qlora_linear_bwd_noalloc) against the
workspace backward it mirrors, through the C ABI: two calls in a row, the
second with a smaller input, on a tile-path shape and then a split-path one;
every output bitwise equal to qlora_linear_bwd's on the same inputs (same
kernels, same launch configuration, fixed reduction order) and within 1e-2
of the oracle."""

import sys

import numpy as np
import pytest
import torch

import helpers as H
from oracle import formats as ofmt
from quantized_base_lora_amd import binding as B

pytestmark = pytest.mark.gpu

# (fmt, m, k, n, r, alpha): the second call is smaller than the first
CALLS = [(ofmt.FMT_NF4, 1536, 2048, 3072, 16, 32.0), (ofmt.FMT_Q4_0, 24, 1024, 320, 32, 64.0)]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


def test_noalloc_backward_matches_workspace_backward(lib):
    for i, (fmt, m, k, n, r, alpha) in enumerate(CALLS):
        say(f"call {i}: fmt={fmt} m={m} k={k} n={n} r={r}")
        c = H.make_case(m, k, n, r, seed=700 + i)
        qw = B.quant_pack(fmt, torch.from_numpy(c["W"]).cuda())
        x, dy = H.bits_to_bf16_tensor(c["x"]), H.bits_to_bf16_tensor(c["dY"])
        a, b = H.bits_to_bf16_tensor(c["A"]), H.bits_to_bf16_tensor(c["B"])
        _, u = B.linear_fwd(qw, x, a, b, alpha)
        dx0, da0, db0 = B.linear_bwd(qw, x, dy, u, a, b, alpha)
        dx = torch.full((m, k), float("nan"), dtype=torch.bfloat16, device="cuda")
        da = torch.full((r, k), float("nan"), dtype=torch.float32, device="cuda")
        db = torch.full((n, r), float("nan"), dtype=torch.float32, device="cuda")
        B.linear_bwd_noalloc(qw, x, dy, u, a, b, alpha, dx, da, db)
        torch.cuda.synchronize()
        for name, got, want in (("dX", dx, dx0), ("dA", da, da0), ("dB", db, db0)):
            assert torch.equal(bits(got), bits(want)), (i, name)
        _, _, wd = H.oracle_packed(fmt, c["W"])
        ref = H.oracle_layer(c, wd, alpha)
        for name, got in (("dX", dx), ("dA", da), ("dB", db)):
            e = H.rel(H.f32_host(got), ref[name])
            say(f"  {name}: bitwise equal to the workspace call, rel err {e:.2e}")
            assert e <= H.FWD_TOL, (i, name, e)
