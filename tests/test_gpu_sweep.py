"""A seeded sweep of layer shapes against the oracle: for every base format,
24 shapes drawn from a fixed generator (token counts on both sides of every
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


def shapes(fmt, count=24):
    g = np.random.default_rng(1000 + fmt)
    out = []
    for i in range(count):
        m = int(MS[(i * 7 + fmt) % len(MS)])
        # mostly short contractions; every fourth up to 4096 (long split slices);
        # formats with 32-element blocks also take odd multiples of 32 (a half
        # contraction step at the end)
        k = 64 * int(g.integers(1, 65 if i % 4 == 3 else 25))
        if fmt != ofmt.FMT_NF4 and i % 3 == 1:
            k -= 32
        n = 32 * int(g.integers(1, 33))
        r = int(g.choice([8, 16, 32]))
        out.append((fmt, m, k, n, r, int(g.integers(0, 1 << 30))))
    return out


CASES = [c for f in FMTS for c in shapes(f)]


@pytest.mark.parametrize("case", CASES, ids=[f"fmt{c[0]}-m{c[1]}-k{c[2]}-n{c[3]}-r{c[4]}" for c in CASES])
def test_sweep_parity(lib, case):
    _parity(case)

def groups(fmt, count=2):
    g = np.random.default_rng(2000 + fmt)
    out = []
    for i in range(count):
        m = int(MS[(i * 5 + 3 * fmt) % len(MS)])
        r = int(g.choice([8, 16, 32]))
        kb = 64 if fmt == ofmt.FMT_NF4 else 32
        probs = [(kb * int(g.integers(1, 49)), 32 * int(g.integers(1, 33))) for _ in range(int(g.integers(2, 4)))]
        out.append((fmt, m, r, probs, int(g.integers(0, 1 << 30))))
    return out


GROUPS = [c for f in FMTS for c in groups(f)]


@pytest.mark.parametrize("grp", GROUPS, ids=[f"fmt{c[0]}-m{c[1]}-r{c[2]}-n{len(c[3])}" for c in GROUPS])
def test_sweep_groups(lib, grp):
    """Random groups (2-3 problems of one token count and rank): every output
    bitwise that of the same call made alone, and within 1e-2 of the oracle."""
    from quantized_base_lora_amd import binding as B
    fmt, m, r, probs, seed = grp
    print(f"sweep group fmt={fmt} m={m} r={r} problems={probs}", flush=True)
    alpha = 2.0 * r
    single, fi, bi, cases = [], [], [], []
    for i, (k, n) in enumerate(probs):
        c = H.make_case(m, k, n, r, seed=seed + i)
        cases.append(c)
        qw = B.quant_pack(fmt, torch.from_numpy(c["W"]).cuda())
        t = {key: H.bits_to_bf16_tensor(c[key]) for key in ("x", "dY", "A", "B")}
        y, u = B.linear_fwd(qw, t["x"], t["A"], t["B"], alpha)
        dx, da, db = B.linear_bwd(qw, t["x"], t["dY"], u, t["A"], t["B"], alpha)
        single.append({"y": y, "u": u, "dx": dx, "da": da, "db": db})
        o = {key: torch.empty_like(v) for key, v in single[-1].items()}
        wsf = torch.empty(max(256, B.workspace_bytes(B.OP_FWD, fmt, n, k, m, r)), dtype=torch.uint8, device="cuda")
        wsb = torch.empty(max(256, B.workspace_bytes(B.OP_BWD, fmt, n, k, m, r)), dtype=torch.uint8, device="cuda")
        fi.append((qw, t["x"], t["A"], t["B"], alpha, o["y"], o["u"], wsf))
        bi.append((qw, t["x"], t["dY"], o["u"], t["A"], t["B"], alpha, o["dx"], o["da"], o["db"], wsb, False))
    B.linear_fwd_group(fi)
    B.linear_bwd_group(bi)
    torch.cuda.synchronize()
    for j, (c, sg) in enumerate(zip(cases, single)):
        got = {"y": fi[j][5], "u": fi[j][6], "dx": bi[j][7], "da": bi[j][8], "db": bi[j][9]}
        for key, v in sg.items():
            iv = torch.int16 if v.dtype == torch.bfloat16 else torch.int32
            assert torch.equal(got[key].view(iv), v.view(iv)), (j, key)
        _, _, wd = H.oracle_packed(fmt, c["W"])
        ref = H.oracle_layer(c, wd, alpha)
        for key, rk in (("y", "y"), ("u", "U"), ("dx", "dX"), ("da", "dA"), ("db", "dB")):
            g_ = got[key].float().cpu().numpy() if got[key].dtype == torch.bfloat16 else got[key].cpu().numpy()
            e = H.rel(g_, ref[rk])
            assert e <= H.FWD_TOL, (j, key, e)


@pytest.mark.parametrize("case", CASES[::3], ids=[f"fmt{c[0]}-m{c[1]}-k{c[2]}-n{c[3]}-r{c[4]}" for c in CASES[::3]])
def test_sweep_backward_variants(lib, case):
    """The backward's other forms on the sweep's shapes: without dX (dA, dB
    within 1e-2 of the oracle), accumulating into given dA / dB (bitwise the
    given values plus the fresh gradients), and the allocation-free call
    (bitwise the workspace call's outputs)."""
    from quantized_base_lora_amd import binding as B
    fmt, m, k, n, r, seed = case
    print(f"sweep backward variants fmt={fmt} m={m} k={k} n={n} r={r}", flush=True)
    alpha = 2.0 * r
    c = H.make_case(m, k, n, r, seed=seed)
    qw = B.quant_pack(fmt, torch.from_numpy(c["W"]).cuda())
    t = {key: H.bits_to_bf16_tensor(c[key]) for key in ("x", "dY", "A", "B")}
    _, u = B.linear_fwd(qw, t["x"], t["A"], t["B"], alpha)
    dx, da, db = B.linear_bwd(qw, t["x"], t["dY"], u, t["A"], t["B"], alpha)
    _, da_n, db_n = B.linear_bwd(qw, t["x"], t["dY"], u, t["A"], t["B"], alpha, need_dx=False)
    g = np.random.default_rng(seed)
    da0 = torch.from_numpy(g.standard_normal((r, k)).astype(np.float32)).cuda()
    db0 = torch.from_numpy(g.standard_normal((n, r)).astype(np.float32)).cuda()
    _, da_a, db_a = B.linear_bwd(qw, t["x"], t["dY"], u, t["A"], t["B"], alpha, accumulate=True,
                                 da=da0.clone(), db=db0.clone())
    torch.cuda.synchronize()
    _, _, wd = H.oracle_packed(fmt, c["W"])
    ref = H.oracle_layer(c, wd, alpha)
    assert H.rel(da_n.cpu().numpy(), ref["dA"]) <= H.FWD_TOL
    assert H.rel(db_n.cpu().numpy(), ref["dB"]) <= H.FWD_TOL
    assert torch.equal(da_a, da0 + da) and torch.equal(db_a, db0 + db)
    if B.workspace_bytes(B.OP_BWD, fmt, n, k, m, r) <= B.NOALLOC_SCRATCH_BYTES:
        dx2 = torch.empty_like(dx)
        da2 = torch.empty_like(da)
        db2 = torch.empty_like(db)
        B.linear_bwd_noalloc(qw, t["x"], t["dY"], u, t["A"], t["B"], alpha, dx2, da2, db2)
        torch.cuda.synchronize()
        assert torch.equal(dx2.view(torch.int16), dx.view(torch.int16))
        assert torch.equal(da2, da) and torch.equal(db2, db)


def large_shapes(count=12):
    g = np.random.default_rng(3000)
    out = []
    for i in range(count):
        fmt = FMTS[i % len(FMTS)]
        m = int(g.integers(600, 3100))
        kb = 64 if fmt == ofmt.FMT_NF4 else 32
        k = kb * int(g.integers(2, 2048 // kb + 1))
        n = 32 * int(g.integers(2, 41))
        out.append((fmt, m, k, n, int(g.choice([8, 16, 32])), int(g.integers(0, 1 << 30))))
    return out


LARGE = large_shapes()


@pytest.mark.parametrize("case", LARGE, ids=[f"fmt{c[0]}-m{c[1]}-k{c[2]}-n{c[3]}-r{c[4]}" for c in LARGE])
def test_sweep_large_m(lib, case):
    """600-3100 tokens: several waves of row tiles, two to seven gradient
    partitions, ragged last tiles in every dimension; all five outputs
    against the oracle on every row."""
    _parity(case)


def _parity(case):
    from quantized_base_lora_amd import binding as B
    fmt, m, k, n, r, seed = case
    print(f"sweep fmt={fmt} m={m} k={k} n={n} r={r} seed={seed}", flush=True)
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
