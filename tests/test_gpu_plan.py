"""Launch plans (ql_plan_*): a recorded sequence of forward / backward calls,
enqueued by one library call, gives bitwise the results of the same calls
issued one by one (same kernels, same launch configuration), run after run."""

import sys

import numpy as np
import pytest
import torch

import helpers as H
from oracle import formats as ofmt

pytestmark = pytest.mark.gpu

CASES = [
    # fmt, m, k, n, r: split path with fused gradients, split path, 128x128 tiles, fp8 matrix cores
    (ofmt.FMT_NF4, 16, 512, 384, 16),
    (ofmt.FMT_MXFP4, 64, 1024, 256, 8),
    (ofmt.FMT_Q4_0, 200, 256, 320, 32),
    (ofmt.FMT_FP8, 130, 256, 224, 16),
]


def test_plan_matches_direct_calls(lib):
    from quantized_base_lora_amd import binding as B
    alpha = 32.0
    items = []
    for i, (fmt, m, k, n, r) in enumerate(CASES):
        print(f"plan case fmt={fmt} m={m} k={k} n={n} r={r}", flush=True)
        c = H.make_case(m, k, n, r, seed=60 + i)
        qw = B.quant_pack(fmt, torch.from_numpy(c["W"]).cuda())
        t = {key: H.bits_to_bf16_tensor(c[key]) for key in ("x", "dY", "A", "B")}
        y, u = B.linear_fwd(qw, t["x"], t["A"], t["B"], alpha)
        dx, da, db = B.linear_bwd(qw, t["x"], t["dY"], u, t["A"], t["B"], alpha)
        out = {"y": torch.empty_like(y), "u": torch.empty_like(u), "dx": torch.empty_like(dx),
               "da": torch.empty_like(da), "db": torch.empty_like(db),
               "wsf": torch.empty(max(256, B.workspace_bytes(B.OP_FWD, fmt, n, k, m, r)), dtype=torch.uint8,
                                  device="cuda"),
               "wsb": torch.empty(max(256, B.workspace_bytes(B.OP_BWD, fmt, n, k, m, r)), dtype=torch.uint8,
                                  device="cuda")}
        items.append((qw, t, {"y": y, "u": u, "dx": dx, "da": da, "db": db}, out))
    torch.cuda.synchronize()
    pl = B.Plan()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pl.add_event(e0, stream)
    for qw, t, _, o in items:
        pl.add_fwd(qw, t["x"], t["A"], t["B"], alpha, o["y"], o["u"], o["wsf"])
    for qw, t, _, o in reversed(items):
        pl.add_bwd(qw, t["x"], t["dY"], o["u"], t["A"], t["B"], alpha, o["dx"], o["da"], o["db"], o["wsb"])
    pl.add_event(e1, stream)
    assert len(pl) == 2 * len(items) + 2
    for run in range(3):
        for _, _, _, o in items:
            for key in ("y", "u", "dx", "da", "db"):
                o[key].fill_(float("nan"))
        pl.run()
        torch.cuda.synchronize()
        assert e0.elapsed_time(e1) > 0
        for j, (_, _, ref, o) in enumerate(items):
            for key in ("y", "u", "dx", "da", "db"):
                a, b = o[key], ref[key]
                iv = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
                assert torch.equal(a.view(iv), b.view(iv)), (run, j, key)
    pl.close()


GROUPS = [
    # fmt, m, r, [(k, n), ...]: split path with fused gradients, split path at 64 tokens,
    # 33 tokens (separate gradient launch), then tile-kernel groups (one launch per
    # group): ragged row and column tiles, contractions of different lengths in both
    # directions (the table is reordered, longest first), a q|k|v-shaped group whose
    # tile counts are multiples of 8 (per-problem XCD remap), and the FP8 base above
    # 64 tokens (one fp8 GEMM launch, reordered longest contraction first)
    (ofmt.FMT_NF4, 16, 16, [(512, 384), (512, 128), (512, 128)]),
    # 16 tokens, one problem for the streaming kernel and one whose scale rows
    # (11 fp16 entries) rule it out: each runs the kernel of its own call
    (ofmt.FMT_Q4_0, 16, 8, [(352, 224), (768, 512)]),
    (ofmt.FMT_MXFP4, 3, 16, [(96, 160), (896, 864)]),
    (ofmt.FMT_MXFP4, 64, 8, [(1024, 256), (256, 1024)]),
    (ofmt.FMT_Q4_0, 33, 32, [(96, 224), (1056, 64), (256, 96)]),
    (ofmt.FMT_FP8, 24, 16, [(256, 160), (512, 96)]),
    (ofmt.FMT_NF4, 200, 16, [(256, 192), (128, 64)]),
    (ofmt.FMT_MXFP4, 300, 8, [(256, 448), (512, 128), (128, 320)]),
    (ofmt.FMT_Q8_0, 520, 32, [(192, 96), (640, 288)]),
    (ofmt.FMT_Q4_0, 129, 16, [(64, 64), (320, 1088), (64, 256), (128, 32)]),
    (ofmt.FMT_NF4, 2048, 16, [(1024, 2048), (1024, 1024), (1024, 1024)]),
    (ofmt.FMT_FP8, 96, 16, [(256, 160), (512, 96)]),
    (ofmt.FMT_FP8, 600, 32, [(256, 512), (512, 256), (768, 128)]),
]


@pytest.mark.parametrize("grp", GROUPS, ids=[f"fmt{g[0]}-m{g[1]}-r{g[2]}-n{len(g[3])}" for g in GROUPS])
def test_group_matches_single_calls(lib, grp):
    """A group (direct call and through a plan) gives bitwise the results of
    its calls made one by one."""
    from quantized_base_lora_amd import binding as B
    fmt, m, r, shapes = grp
    print(f"group fmt={fmt} m={m} r={r} shapes={shapes}", flush=True)
    alpha = 16.0
    ref, fi, bi = [], [], []
    for i, (k, n) in enumerate(shapes):
        c = H.make_case(m, k, n, r, seed=80 + i)
        qw = B.quant_pack(fmt, torch.from_numpy(c["W"]).cuda())
        t = {key: H.bits_to_bf16_tensor(c[key]) for key in ("x", "dY", "A", "B")}
        y, u = B.linear_fwd(qw, t["x"], t["A"], t["B"], alpha)
        dx, da, db = B.linear_bwd(qw, t["x"], t["dY"], u, t["A"], t["B"], alpha)
        ref.append({"y": y, "u": u, "dx": dx, "da": da, "db": db})
        o = {key: torch.empty_like(v) for key, v in ref[-1].items()}
        wsf = torch.empty(max(256, B.workspace_bytes(B.OP_FWD, fmt, n, k, m, r)), dtype=torch.uint8, device="cuda")
        wsb = torch.empty(max(256, B.workspace_bytes(B.OP_BWD, fmt, n, k, m, r)), dtype=torch.uint8, device="cuda")
        fi.append((qw, t["x"], t["A"], t["B"], alpha, o["y"], o["u"], wsf))
        # the backward reads the group forward's own U
        bi.append((qw, t["x"], t["dY"], o["u"], t["A"], t["B"], alpha, o["dx"], o["da"], o["db"], wsb, False))
    torch.cuda.synchronize()

    def check(tag):
        torch.cuda.synchronize()
        for j, (rf, it) in enumerate(zip(ref, bi)):
            got = {"y": fi[j][5], "u": fi[j][6], "dx": it[7], "da": it[8], "db": it[9]}
            for key, v in rf.items():
                iv = torch.int16 if v.dtype == torch.bfloat16 else torch.int32
                assert torch.equal(got[key].view(iv), v.view(iv)), (tag, j, key)

    B.linear_fwd_group(fi)
    B.linear_bwd_group(bi)
    check("direct")
    pl = B.Plan()
    pl.add_fwd_group(fi)
    pl.add_bwd_group(bi)
    for run in range(2):
        for it in fi:
            it[5].fill_(float("nan"))
        pl.run()
        check(f"plan run {run}")
    pl.close()


# FP8: the two-term split made once for the group, the projections' and the
# dA launches' workgroups of one row block or tile side by side (ragged row
# blocks at 300 tokens); NF4 on the bf16 tiles, the dA runs with tile x
# partition counts that are not multiples of 8 (k = 320: 5 tiles at rank 16,
# 3 at rank 32)
@pytest.mark.parametrize("fmt,r,k,m", [(ofmt.FMT_FP8, 16, 512, 300), (ofmt.FMT_FP8, 16, 512, 1030),
                                       (ofmt.FMT_NF4, 32, 320, 600), (ofmt.FMT_NF4, 16, 320, 1100)])
def test_group_shared_activation(lib, fmt, r, k, m):
    """q|k|v-shaped group above 64 tokens whose calls share one input x: y, U,
    dX, dA and dB bitwise those of single calls."""
    from quantized_base_lora_amd import binding as B
    alpha = 32.0
    ns = [512, 128, 128]
    print(f"shared-activation group fmt={fmt} r={r} k={k} m={m}", flush=True)
    x = H.bits_to_bf16_tensor(H.make_case(m, k, 32, r, seed=120)["x"])
    items = []
    for i, n in enumerate(ns):
        c = H.make_case(m, k, n, r, seed=121 + i)
        qw = B.quant_pack(fmt, torch.from_numpy(c["W"]).cuda())
        t = {key: H.bits_to_bf16_tensor(c[key]) for key in ("dY", "A", "B")}
        items.append((qw, t, n))
    ref, fi, bi = [], [], []
    for qw, t, n in items:
        y, u = B.linear_fwd(qw, x, t["A"], t["B"], alpha)
        dx, da, db = B.linear_bwd(qw, x, t["dY"], u, t["A"], t["B"], alpha)
        ref.append(dict(y=y, u=u, dx=dx, da=da, db=db))
        o = {key: torch.empty_like(v) for key, v in ref[-1].items()}
        wsf = torch.empty(max(256, B.workspace_bytes(B.OP_FWD, fmt, n, k, m, r)), dtype=torch.uint8, device="cuda")
        wsb = torch.empty(max(256, B.workspace_bytes(B.OP_BWD, fmt, n, k, m, r)), dtype=torch.uint8, device="cuda")
        fi.append((qw, x, t["A"], t["B"], alpha, o["y"], o["u"], wsf))
        bi.append((qw, x, t["dY"], o["u"], t["A"], t["B"], alpha, o["dx"], o["da"], o["db"], wsb, False))
    torch.cuda.synchronize()
    B.linear_fwd_group(fi)
    B.linear_bwd_group(bi)
    torch.cuda.synchronize()
    for j, rf in enumerate(ref):
        got = {"y": fi[j][5], "u": fi[j][6], "dx": bi[j][7], "da": bi[j][8], "db": bi[j][9]}
        for key, v in rf.items():
            iv = torch.int16 if v.dtype == torch.bfloat16 else torch.int32
            assert torch.equal(got[key].view(iv), v.view(iv)), (m, j, key)


def test_group_edge_cases(lib):
    """Groups with accumulate, with one call, without dX, and with no tokens
    behave as the same single calls."""
    from quantized_base_lora_amd import binding as B
    fmt, r, alpha = ofmt.FMT_NF4, 16, 32.0
    shapes = [(256, 128), (128, 192)]

    def setup(m, seed):
        items = []
        for i, (k, n) in enumerate(shapes):
            c = H.make_case(max(m, 1), k, n, r, seed=seed + i)
            qw = B.quant_pack(fmt, torch.from_numpy(c["W"]).cuda())
            t = {key: H.bits_to_bf16_tensor(c[key])[:m] if key in ("x", "dY") else H.bits_to_bf16_tensor(c[key])
                 for key in ("x", "dY", "A", "B")}
            items.append((qw, t, k, n))
        return items

    for m in (24, 48, 0):
        print(f"group edge cases m={m}", flush=True)
        items = setup(m, 90)
        # reference: single calls, accumulating onto given dA / dB, and a call without dX
        ref = []
        for qw, t, k, n in items:
            y, u = B.linear_fwd(qw, t["x"], t["A"], t["B"], alpha)
            da0 = torch.full((r, k), 0.25, device="cuda")
            db0 = torch.full((n, r), -0.5, device="cuda")
            dx, da, db = B.linear_bwd(qw, t["x"], t["dY"], u, t["A"], t["B"], alpha, accumulate=True,
                                      da=da0.clone(), db=db0.clone())
            _, da2, db2 = B.linear_bwd(qw, t["x"], t["dY"], u, t["A"], t["B"], alpha, need_dx=False)
            ref.append(dict(y=y, u=u, dx=dx, da=da, db=db, da2=da2, db2=db2))
        got = []
        fi, bi, bn = [], [], []
        for (qw, t, k, n), rf in zip(items, ref):
            o = dict(y=torch.empty_like(rf["y"]), u=torch.empty_like(rf["u"]), dx=torch.empty_like(rf["dx"]),
                     da=torch.full((r, k), 0.25, device="cuda"), db=torch.full((n, r), -0.5, device="cuda"),
                     da2=torch.empty((r, k), device="cuda"), db2=torch.empty((n, r), device="cuda"),
                     wsf=torch.empty(max(256, B.workspace_bytes(B.OP_FWD, fmt, n, k, m, r)), dtype=torch.uint8,
                                     device="cuda"),
                     wsb=torch.empty(max(256, B.workspace_bytes(B.OP_BWD, fmt, n, k, m, r)), dtype=torch.uint8,
                                     device="cuda"),
                     wsb2=torch.empty(max(256, B.workspace_bytes(B.OP_BWD, fmt, n, k, m, r)), dtype=torch.uint8,
                                      device="cuda"))
            got.append(o)
            fi.append((qw, t["x"], t["A"], t["B"], alpha, o["y"], o["u"], o["wsf"]))
            bi.append((qw, t["x"], t["dY"], o["u"], t["A"], t["B"], alpha, o["dx"], o["da"], o["db"], o["wsb"], True))
            bn.append((qw, t["x"], t["dY"], o["u"], t["A"], t["B"], alpha, None, o["da2"], o["db2"], o["wsb2"], False))
        B.linear_fwd_group(fi[:1])            # a group of one
        B.linear_fwd_group(fi[1:])
        B.linear_bwd_group(bi)                # accumulate into the given dA / dB
        B.linear_bwd_group(bn)                # no dX
        torch.cuda.synchronize()
        for j, (rf, o) in enumerate(zip(ref, got)):
            for key in ("y", "u", "dx", "da", "db", "da2", "db2"):
                a, b = o[key], rf[key]
                iv = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
                assert torch.equal(a.view(iv), b.view(iv)), (m, j, key)


HELD_SPECS = {
    # 1100 tokens: three partitions of M; 600: two (the reductions are held back)
    "reductions": [(1100, 256, 192), (1100, 128, 320), (1100, 320, 64), (1100, 192, 128), (1100, 64, 256),
                   (1100, 256, 64), (1100, 128, 128), (1100, 64, 192), (1100, 192, 96), (600, 128, 192)],
    # 48 tokens: the small-token path, whose gradient launches are held back
    # themselves (one partition); the last call has 40 tokens, another plan
    "gradient_launches": [(48, 256, 192), (48, 128, 320), (48, 320, 64), (48, 192, 128), (48, 64, 256),
                          (48, 256, 64), (48, 128, 128), (48, 64, 192), (48, 192, 96), (40, 128, 192)],
}


@pytest.mark.parametrize("held", list(HELD_SPECS))
def test_plan_held_back_reductions(lib, held):
    """A plan holds the adapter-gradient work of its backward steps back and
    runs it as one launch: the reductions of partial sums (more than 512
    tokens), and on the small-token path (33-64 tokens) the gradient launches
    themselves.  Each rule that launches them early is hit here: a later step
    accumulating into the same dA / dB, later forward and backward steps
    reusing a held step's workspace, an event, another partition count or
    token count, a set that is full (16 reductions, or 8 calls) and the end of
    the plan.  Every output must equal, bit for bit, the same calls made one
    by one."""
    from quantized_base_lora_amd import binding as B
    fmt, r, alpha = ofmt.FMT_NF4, 16, 16.0
    specs = HELD_SPECS[held]
    calls = []
    wsb = max(256, max(B.workspace_bytes(B.OP_BWD, fmt, n, k, m, r) for m, k, n in specs))
    for i, (m, k, n) in enumerate(specs):
        print(f"held reductions call {i}: m={m} k={k} n={n}", flush=True)
        c = H.make_case(m, k, n, r, seed=120 + i)
        qw = B.quant_pack(fmt, torch.from_numpy(c["W"]).cuda())
        t = {key: H.bits_to_bf16_tensor(c[key]) for key in ("x", "dY", "A", "B")}
        _, u = B.linear_fwd(qw, t["x"], t["A"], t["B"], alpha)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        calls.append({"qw": qw, "t": t, "u": u, "ws": ws, "m": m, "k": k, "n": n})
    torch.cuda.synchronize()

    def outs(c):
        return {"dx": torch.empty((c["m"], c["k"]), dtype=torch.bfloat16, device="cuda"),
                "da": torch.empty((r, c["k"]), dtype=torch.float32, device="cuda"),
                "db": torch.empty((c["n"], r), dtype=torch.float32, device="cuda")}

    def item(i, o, ws=None, acc=False):
        c = calls[i]
        t = c["t"]
        return (c["qw"], t["x"], t["dY"], c["u"], t["A"], t["B"], alpha, o["dx"], o["da"], o["db"],
                ws if ws is not None else c["ws"], acc)

    # the sequence: (kind, [(call, output slot, workspace of call or None, accumulate)])
    seq = [
        ("bwd", [(0, "a", None, False)]),
        ("group", [(1, "b", None, False), (2, "c", None, False)]),
        ("bwd", [(0, "a", None, True)]),                  # accumulates into held dA / dB of step 1
        ("bwd", [(3, "d", None, False)]),
        ("fwd", [(5, "F", 3, False)]),                    # a forward whose workspace is call 3's, held
        ("bwd", [(4, "e", 3, False)]),                    # reuses the held workspace of call 3
        ("event", []),
        ("group", [(5, "f", None, False), (6, "g", None, False), (7, "h", None, False)]),
        ("bwd", [(9, "j", None, False)]),                 # two partitions, not three
        ("group", [(1, "k", None, False), (2, "l", None, False), (3, "m", None, False), (4, "n", None, False),
                   (5, "o", None, False), (6, "p", None, False), (7, "q", None, False), (8, "r", None, False)]),
        ("bwd", [(0, "s", None, False)]),                 # the set above is full
    ]
    def fouts(c):
        return {"y": torch.empty((c["m"], c["n"]), dtype=torch.bfloat16, device="cuda"),
                "u": torch.empty((c["m"], r), dtype=torch.float32, device="cuda")}

    def fitem(i, o, ws):
        c = calls[i]
        t = c["t"]
        return (c["qw"], t["x"], t["A"], t["B"], alpha, o["y"], o["u"], ws)

    slots = {}
    for kind, its in seq:
        for ci, slot, _, _ in its:
            slots.setdefault(slot, fouts(calls[ci]) if kind == "fwd" else outs(calls[ci]))
    ref = {}
    # one by one (direct calls), in the same order and with the same workspaces
    for kind, its in seq:
        for ci, slot, wsi, acc in its:
            c = calls[ci]
            if kind == "fwd":
                o = ref.setdefault(slot, fouts(c))
                B.linear_fwd(c["qw"], c["t"]["x"], c["t"]["A"], c["t"]["B"], alpha, y=o["y"], u=o["u"],
                             ws=calls[wsi]["ws"])
                continue
            o = ref.setdefault(slot, outs(c))
            it = item(ci, o, calls[wsi]["ws"] if wsi is not None else None, acc)
            B.linear_bwd(c["qw"], c["t"]["x"], c["t"]["dY"], c["u"], c["t"]["A"], c["t"]["B"], alpha,
                         accumulate=acc, dx=o["dx"], da=o["da"], db=o["db"], ws=it[10])
    torch.cuda.synchronize()
    pl = B.Plan()
    stream = torch.cuda.current_stream()
    ev = torch.cuda.Event()
    for kind, its in seq:
        if kind == "event":
            pl.add_event(ev, stream)
        elif kind == "fwd":
            ci, slot, wsi, _ = its[0]
            pl.add_fwd(*fitem(ci, slots[slot], calls[wsi]["ws"]))
        elif kind == "bwd":
            ci, slot, wsi, acc = its[0]
            pl.add_bwd(*item(ci, slots[slot], calls[wsi]["ws"] if wsi is not None else None, acc))
        else:
            pl.add_bwd_group([item(ci, slots[slot], calls[wsi]["ws"] if wsi is not None else None, acc)
                              for ci, slot, wsi, acc in its])
    for run in range(2):
        for o in slots.values():
            for v in o.values():
                v.fill_(float("nan"))
        pl.run()
        torch.cuda.synchronize()
        for slot, o in slots.items():
            for key, v in o.items():
                iv = torch.int16 if v.dtype == torch.bfloat16 else torch.int32
                assert torch.equal(v.view(iv), ref[slot][key].view(iv)), (run, slot, key)
    pl.close()


BENCH_LAYERS = [("qwen3_0.6b_nf4", 8192), ("llama3.1_8b_mxfp4", 16), ("llama3.1_8b_q8_0", 64)]


@pytest.mark.parametrize("wname,m", BENCH_LAYERS, ids=[f"{w}-m{m}" for w, m in BENCH_LAYERS])
def test_bench_launch_configuration_matches_single_calls(lib, wname, m):
    """The layer step exactly as the benchmark times it (a launch plan: the
    forward of q|k|v, o, gate|up, down as grouped calls, then their backward
    in reverse, gradient reductions held back) gives bit for bit the outputs
    of the seven projections called one by one, which the full-size parity
    tests compare with the oracle."""
    from quantized_base_lora_amd import binding as B, synth
    wl = synth.WORKLOADS[wname]
    say_ = lambda *a: print(*a, flush=True)  # noqa: E731
    say_(f"bench configuration {wname} m={m}")
    d = []
    for pi, p in enumerate(wl.projs):
        c = synth.layer_tensors(wl, pi, m=m)
        qw = B.quant_pack(wl.fmt, torch.from_numpy(c["W"]).cuda())
        del c["W"]
        t = {key: H.bits_to_bf16_tensor(c[key]) for key in ("x", "dY", "A", "B")}
        e = {"p": p, "qw": qw, "t": t}
        for tag in ("ref", "got"):
            e[tag] = {"y": torch.empty((m, p.n), dtype=torch.bfloat16, device="cuda"),
                      "u": torch.empty((m, wl.r), dtype=torch.float32, device="cuda"),
                      "dx": torch.empty((m, p.k), dtype=torch.bfloat16, device="cuda"),
                      "da": torch.empty((wl.r, p.k), dtype=torch.float32, device="cuda"),
                      "db": torch.empty((p.n, wl.r), dtype=torch.float32, device="cuda"),
                      "wsf": torch.empty(max(256, B.workspace_bytes(B.OP_FWD, wl.fmt, p.n, p.k, m, wl.r)),
                                         dtype=torch.uint8, device="cuda"),
                      "ws": torch.empty(max(256, B.workspace_bytes(B.OP_BWD, wl.fmt, p.n, p.k, m, wl.r)),
                                        dtype=torch.uint8, device="cuda")}
        d.append(e)
    by = {e["p"].name: e for e in d}
    groups = [[by[n] for n in g] for g in (["q", "k", "v"], ["o"], ["gate", "up"], ["down"])]
    for e in d:                                    # one by one
        t, o = e["t"], e["ref"]
        B.linear_fwd(e["qw"], t["x"], t["A"], t["B"], wl.alpha, y=o["y"], u=o["u"], ws=o["wsf"])
    for e in reversed(d):
        t, o = e["t"], e["ref"]
        B.linear_bwd(e["qw"], t["x"], t["dY"], o["u"], t["A"], t["B"], wl.alpha, dx=o["dx"], da=o["da"],
                     db=o["db"], ws=o["ws"])
    pl = B.Plan()                                  # as the benchmark records a step
    for g in groups:
        pl.add_fwd_group([(e["qw"], e["t"]["x"], e["t"]["A"], e["t"]["B"], wl.alpha, e["got"]["y"], e["got"]["u"],
                           e["got"]["wsf"]) for e in g])
    for g in reversed(groups):
        pl.add_bwd_group([(e["qw"], e["t"]["x"], e["t"]["dY"], e["got"]["u"], e["t"]["A"], e["t"]["B"], wl.alpha,
                           e["got"]["dx"], e["got"]["da"], e["got"]["db"], e["got"]["ws"], False)
                          for e in reversed(g)])
    for run in range(2):
        for e in d:
            for key in ("y", "u", "dx", "da", "db"):
                e["got"][key].fill_(float("nan"))
        pl.run()
        torch.cuda.synchronize()
        for e in d:
            for key in ("y", "u", "dx", "da", "db"):
                a, b = e["got"][key], e["ref"][key]
                iv = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
                assert torch.equal(a.view(iv), b.view(iv)), (run, e["p"].name, key)
    pl.close()


@pytest.mark.parametrize("seed", range(12))
def test_plan_random_sequences(lib, seed):
    """Random launch plans of forward, backward and grouped backward steps and
    events over a pool of calls at three of 24, 48, 96, 600 and 1100 tokens (the fused,
    held-back, single-partition and several-partition gradient paths), with workspaces
    borrowed from other calls and backward steps accumulating into earlier
    outputs: every output bitwise that of the same calls made one by one, on
    two runs of the plan."""
    from quantized_base_lora_amd import binding as B
    g = np.random.default_rng(4200 + seed)
    fmt = [ofmt.FMT_NF4, ofmt.FMT_MXFP4, ofmt.FMT_Q4_0, ofmt.FMT_NVFP4, ofmt.FMT_Q8_0, ofmt.FMT_FP8][seed % 6]
    r, alpha = int(g.choice([8, 16, 32])), 16.0
    pool = []
    for m in [int(x) for x in g.choice([24, 48, 96, 600, 1100], size=3, replace=False)]:
        for _ in range(3):                                # three calls per token count (groups share it)
            pool.append((m, 64 * int(g.integers(1, 6)), 32 * int(g.integers(1, 9))))
    print(f"random plan seed={seed} fmt={fmt} r={r} pool={pool}", flush=True)
    wsb = max(256, max(max(B.workspace_bytes(B.OP_BWD, fmt, n, k, m, r), B.workspace_bytes(B.OP_FWD, fmt, n, k, m, r))
                       for m, k, n in pool))
    calls = []
    for i, (m, k, n) in enumerate(pool):
        c = H.make_case(m, k, n, r, seed=4300 + 10 * seed + i)
        qw = B.quant_pack(fmt, torch.from_numpy(c["W"]).cuda())
        t = {key: H.bits_to_bf16_tensor(c[key]) for key in ("x", "dY", "A", "B")}
        _, u = B.linear_fwd(qw, t["x"], t["A"], t["B"], alpha)
        calls.append({"qw": qw, "t": t, "u": u, "m": m, "k": k, "n": n,
                      "ws": torch.empty(wsb, dtype=torch.uint8, device="cuda")})
    torch.cuda.synchronize()
    # steps: ("fwd"|"bwd", [(call, slot, workspace owner, accumulate)]) or ("event", [])
    seq, slot_of = [], {}
    for _ in range(12):
        kind = g.choice(["fwd", "bwd", "bwd", "group", "group", "event"])
        if kind == "event":
            seq.append(("event", []))
            continue
        if kind == "group":
            m0 = int(g.integers(0, 3))                   # one token count for the group
            cis = [3 * m0 + int(x) for x in g.choice(3, size=int(g.integers(2, 4)), replace=False)]
            items = [(ci, f"b{ci}", ci, False) for ci in cis]   # own slots and workspaces: independent
            seq.append(("group", items))
            continue
        ci = int(g.integers(0, len(calls)))
        wsi = int(g.integers(0, len(calls))) if g.random() < 0.4 else ci
        if kind == "fwd":
            seq.append(("fwd", [(ci, f"f{ci}", wsi, False)]))
        else:
            acc = bool(f"b{ci}" in slot_of and g.random() < 0.5)
            seq.append(("bwd", [(ci, f"b{ci}", wsi, acc)]))
        for it in seq[-1][1]:
            slot_of[it[1]] = it[0]
    for kind, its in seq:
        for ci, slot, _, _ in its:
            slot_of[slot] = ci

    def new_out(slot):
        c = calls[slot_of[slot]]
        if slot[0] == "f":
            return {"y": torch.empty((c["m"], c["n"]), dtype=torch.bfloat16, device="cuda"),
                    "u": torch.empty((c["m"], r), dtype=torch.float32, device="cuda")}
        return {"dx": torch.empty((c["m"], c["k"]), dtype=torch.bfloat16, device="cuda"),
                "da": torch.zeros((r, c["k"]), dtype=torch.float32, device="cuda"),
                "db": torch.zeros((c["n"], r), dtype=torch.float32, device="cuda")}

    def bitem(ci, o, wsi, acc):
        c = calls[ci]
        t = c["t"]
        return (c["qw"], t["x"], t["dY"], c["u"], t["A"], t["B"], alpha, o["dx"], o["da"], o["db"],
                calls[wsi]["ws"], acc)

    ref = {s: new_out(s) for s in slot_of}
    for kind, its in seq:
        for ci, slot, wsi, acc in its:
            c = calls[ci]
            o = ref[slot]
            if kind == "fwd":
                B.linear_fwd(c["qw"], c["t"]["x"], c["t"]["A"], c["t"]["B"], alpha, y=o["y"], u=o["u"],
                             ws=calls[wsi]["ws"])
            elif kind in ("bwd", "group"):
                B.linear_bwd(c["qw"], c["t"]["x"], c["t"]["dY"], c["u"], c["t"]["A"], c["t"]["B"], alpha,
                             accumulate=acc, dx=o["dx"], da=o["da"], db=o["db"], ws=calls[wsi]["ws"])
    torch.cuda.synchronize()
    got = {s: new_out(s) for s in slot_of}
    pl = B.Plan()
    stream = torch.cuda.current_stream()
    ev = torch.cuda.Event()
    for kind, its in seq:
        if kind == "event":
            pl.add_event(ev, stream)
        elif kind == "fwd":
            ci, slot, wsi, _ = its[0]
            c = calls[ci]
            pl.add_fwd(c["qw"], c["t"]["x"], c["t"]["A"], c["t"]["B"], alpha, got[slot]["y"], got[slot]["u"],
                       calls[wsi]["ws"])
        elif kind == "bwd":
            ci, slot, wsi, acc = its[0]
            pl.add_bwd(*bitem(ci, got[slot], wsi, acc))
        else:
            pl.add_bwd_group([bitem(ci, got[slot], wsi, acc) for ci, slot, wsi, acc in its])
    for run in range(2):
        for s, o in got.items():
            for key, v in o.items():
                if key in ("da", "db"):
                    v.zero_()                              # the starting values of accumulating steps
                else:
                    v.fill_(float("nan"))
        pl.run()
        torch.cuda.synchronize()
        for s, o in got.items():
            for key, v in o.items():
                iv = torch.int16 if v.dtype == torch.bfloat16 else torch.int32
                assert torch.equal(v.view(iv), ref[s][key].view(iv)), (run, s, key)
    pl.close()
