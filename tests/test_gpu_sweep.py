"""A seeded sweep of layer shapes against the oracle: for every base format,
ten shapes drawn from a fixed generator (token counts on both sides of every
path boundary: 1..16 the 16-token kernels, 17..32 and 33..64 the split path's
32- and 64-row tiles, above 64 the tile kernels; contraction and output widths
with ragged tiles; ranks 8, 16 and 32), each forward and backward compared
output by output (y, U, dX, dA, dB) with the fp64 oracle at 1e-2 of the
largest reference magnitude."""

import sys

import numpy as np
import pytest
import torch

import helpers as H
from oracle import formats as ofmt

pytestmark = pytest.mark.gpu

FMTS = [ofmt.FMT_Q4_0, ofmt.FMT_NF4, ofmt.FMT_FP8, ofmt.FMT_MXFP4, ofmt.FMT_Q8_0, ofmt.FMT_NVFP4]
MS = [1, 3, 8, 16, 17, 24, 32, 33, 48, 64, 65, 96, 129, 256, 300, 513]


def shapes(fmt):
    g = np.random.default_rng(1000 + fmt)
    out = []
    for i in range(10):
        m = int(MS[(i * 7 + fmt) % len(MS)])
        k = 64 * int(g.integers(1, 25))
        n = 32 * int(g.integers(1, 33))
        r = int(g.choice([8, 16, 32]))
        out.append((fmt, m, k, n, r, int(g.integers(0, 1 << 30))))
    return out


CASES = [c for f in FMTS for c in shapes(f)]


@pytest.mark.parametrize("case", CASES, ids=[f"fmt{c[0]}-m{c[1]}-k{c[2]}-n{c[3]}-r{c[4]}" for c in CASES])
def test_sweep_parity(lib, case):
    from quantized_base_lora_amd import binding as B
    fmt, m, k, n, r, seed = case
    print(f"sweep fmt={fmt} m={m} k={k} n={n} r={r} seed={seed}", flush=True)
    sys.stdout.flush()
    alpha = 2.0 * r
    c = H.make_case(m, k, n, r, seed=seed)
    qw = B.quant_pack(fmt, torch.from_numpy(c["W"]).cuda())
    t = {key: H.bits_to_bf16_tensor(c[key]) for key in ("x", "dY", "A", "B")}
    y, u = B.linear_fwd(qw, t["x"], t["A"], t["B"], alpha)
    dx, da, db = B.linear_bwd(qw, t["x"], t["dY"], u, t["A"], t["B"], alpha)
    torch.cuda.synchronize()
    _, _, wd = H.oracle_packed(fmt, c["W"])
    ref = H.oracle_layer(c, wd, alpha)
    got = {"y": y.float().cpu().numpy(), "U": u.cpu().numpy(), "dX": dx.float().cpu().numpy(),
           "dA": da.cpu().numpy(), "dB": db.cpu().numpy()}
    for key, v in got.items():
        e = H.rel(v, ref[key])
        assert e <= H.FWD_TOL, (key, e)
