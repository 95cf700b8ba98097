"""Benchmark: QLoRA linear layer forward + backward on one MI355X.

One step = forward of every projection of a decoder layer (7 LoRA linears over
a frozen quantized base), then backward of every projection (dX, dA, dB), on
synthetic seeded inputs resident in HBM.  Reported value: tokens/s per layer.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--m M]

Prints ONE JSON line.  Besides the headline value it carries the roofline of
the dominant kernel (its launches bracketed by HIP events on the stream they
run on) and the CPU oracle timed on this host on a bounded sample.
"""

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QLoRA-linear fwd+bwd tokens/s per layer; % bf16 MFMA peak, % HBM BW"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
FMT_NAME = {1: "q4_0", 2: "nf4", 3: "fp8_e4m3", 4: "mxfp4", 5: "q8_0"}
BPW = {1: 18 / 32, 2: 0.5 + 4 / 64, 3: 1.0, 4: 17 / 32, 5: 34 / 32}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen3_0.6b_nf4")
    ap.add_argument("--m", type=int, default=None, help="tokens (default: the workload's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=0, help="tokens in the CPU oracle sample (0: all)")
    ap.add_argument("--copies", type=int, default=0, help="packed weight copies rotated per step (0: auto)")
    ap.add_argument("--proj", default=None, help="run only this projection (profiling)")
    ap.add_argument("--exclude", default="",
                    help="comma-separated projections left out of the layer (e.g. o), in the timing and in "
                         "every per-layer figure")
    ap.add_argument("--phase", default="both", choices=["both", "fwd", "bwd"], help="profiling: one pass only")
    ap.add_argument("--graph", action="store_true",
                    help="time HIP-graph replays of the step instead of eager launches")
    ap.add_argument("--streams", action="store_true",
                    help="run projections that are independent in a decoder layer (q|k|v, gate|up) "
                         "on parallel streams")
    ap.add_argument("--no-plan", action="store_true",
                    help="issue each layer call from Python instead of through a recorded launch plan")
    ap.add_argument("--optimizer", action="store_true",
                    help="time the fused AdamW step on the layer's adapters instead of the layer step")
    ap.add_argument("--layers", type=int, default=0,
                    help="stack mode: this many layers, resident vs streamed from pinned host")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device-to-device (a plain copy kernel of known size, "
                         "to calibrate HBM byte counters) and exit")
    return ap.parse_args()


def layer_flops(wl, m):
    return sum(m * (4 * p.n * p.k + 6 * wl.r * (p.k + p.n)) for p in wl.projs)


def layer_bytes(wl, m):
    bpw = BPW[wl.fmt]
    sk = sum(p.k for p in wl.projs)
    sn = sum(p.n for p in wl.projs)
    snk = sum(p.n * p.k for p in wl.projs)
    return 2 * bpw * snk + 8 * wl.r * (sk + sn) + m * (6 * sk + 4 * sn) + 12 * m * wl.r * len(wl.projs)


def fwd_kernel_flops(wl, p, m):
    return m * (2 * p.n * p.k + 2 * wl.r * (p.k + p.n))


def source_hash():
    h = hashlib.sha256()
    with open(os.path.join(ROOT, "quantized_base_lora_amd", "csrc", "kernels_gemm.hip"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload, m):
    """HBM bytes per dominant-kernel launch from committed rocprofv3 counters,
    if they were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "qgemm_fwd_counters.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha") != source_hash():
        return None
    e = d.get("workloads", {}).get(f"{workload}@{m}")
    return None if e is None else e.get("hbm_bytes_per_launch")


def optimizer_bench(args, wl):
    """The fused AdamW step over all adapter tensors of one layer (A and B of
    every projection, fp32 masters and moments, bf16 copies), one launch per
    step; state copies rotated over >= 512 MB so the MALL cannot serve them.
    Algorithmic bytes per element: param, grad, m, v read (16) and param, m, v
    (12) plus the bf16 copy (2) written."""
    import torch
    from quantized_base_lora_amd import binding as B
    dev = torch.device("cuda:0")
    sizes = []
    for p in wl.projs:
        sizes += [wl.r * p.k, p.n * wl.r]
    n_el = sum(sizes)
    per_el = 30
    copies = max(1, int(np.ceil(512e6 / (n_el * 18))))
    gen = torch.Generator(device=dev).manual_seed(1)
    sets = []
    for _ in range(copies):
        ts = []
        for n in sizes:
            ts.append((torch.randn(n, device=dev, generator=gen) * 0.02, torch.randn(n, device=dev, generator=gen) * 1e-3,
                       torch.zeros(n, device=dev), torch.zeros(n, device=dev),
                       torch.empty(n, dtype=torch.bfloat16, device=dev)))
        sets.append(ts)
    plans = [B.AdamwPlan(ts) for ts in sets]
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    for i in range(args.warmup):
        plans[i % copies].step(i + 1, lr=2e-4, weight_decay=0.01, stream=stream)
    torch.cuda.synchronize()
    # the launches captured in a HIP graph and replayed, so host-side call
    # overhead (larger than the kernel itself) stays out of the timing
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(args.steps):
            plans[i % copies].step(args.warmup + i + 1, lr=2e-4, weight_decay=0.01, stream=stream)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    gbs = n_el * per_el / (us / 1e6) / 1e9
    out = {"metric": "fused AdamW adapter step, algorithmic HBM GB/s", "value": gbs, "unit": "GB/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "us_per_step": us,
           "higher_is_better": True, "dtype": "f32", "data": "synthetic",
           "config": {"workload": f"adapters of one {wl.notes}", "tensors": len(sizes), "elements": n_el,
                      "bytes_per_element": per_el, "state_copies_rotated": copies,
                      "step_mode": "HIP graph of the launches, replayed"},
           "roofline": {"kernel": "adamw_kernel", "bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS, "traffic": None}}
    print(json.dumps(out), flush=True)


def cpu_baseline(wl, tokens, min_seconds=10.0):
    """The oracle (numpy, fp64 products) on `tokens` tokens of the same layer:
    W dequantized once beforehand, then forward + backward of every
    projection, repeated until at least min_seconds of wall time."""
    from threadpoolctl import threadpool_info

    from oracle import formats as ofmt, lora as olora
    from quantized_base_lora_amd import synth
    f32 = synth.bf16_bits_to_f32
    prep = []
    for pi, _ in enumerate(wl.projs):
        c = synth.layer_tensors(wl, pi, m=tokens)
        codes, scales = ofmt.pack(wl.fmt, c["W"])
        wd = ofmt.dequant(wl.fmt, codes, scales)
        prep.append((f32(c["x"]), f32(c["dY"]), wd, f32(c["A"]), f32(c["B"])))
    passes, dt = 0, 0.0
    while dt < min_seconds and passes < 50:
        t0 = time.perf_counter()
        for x, dy, wd, a, b in prep:
            olora.forward(x, wd, a, b, wl.alpha)
            olora.backward(x, dy, wd, a, b, wl.alpha)
        dt += time.perf_counter() - t0
        passes += 1
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": tokens * passes / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{tokens} tokens of the same layer (all {len(wl.projs)} projections, fwd+bwd, "
                      f"fp64 products, W dequantized beforehand), {passes} passes in {dt:.2f} s wall; "
                      f"BLAS threads {threads}, host cpus visible {len(os.sched_getaffinity(0))}"}


def bench_stack(args, wl, m):
    """The layer stack: L Llama-shaped layers, forward 0..L-1 then backward
    L-1..0, with the packed bases resident in VRAM or streamed from pinned
    host memory through two device slots (one layer ahead on a side stream).
    Bases are random normal W packed on the GPU; activations and adapters are
    seeded normals generated on the GPU (their values do not affect timing)."""
    import torch

    from quantized_base_lora_amd import binding as B, stack

    dev = torch.device("cuda:0")
    L = args.layers
    layout = stack.LayerLayout(wl.fmt, wl.projs)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    host = []
    t0 = time.time()
    for layer in range(L):
        qws = []
        for p in wl.projs:
            w = torch.randn((p.n, p.k), generator=gen, device=dev, dtype=torch.float32) * 0.02
            qws.append(B.quant_pack(wl.fmt, w))
            del w
        img = layout.image_from(qws)
        h = torch.empty(layout.nbytes, dtype=torch.uint8, pin_memory=True)
        h.copy_(img)
        host.append(h)
        del img, qws
    torch.cuda.synchronize()
    prep_s = time.time() - t0

    def bf16(shape, std):
        return (torch.randn(shape, generator=gen, device=dev, dtype=torch.float32) * std).to(torch.bfloat16)

    acts, outs = [], []
    for layer in range(L):
        al, ol = [], []
        for p in wl.projs:
            al.append({"x": bf16((m, p.k), 1.0), "dy": bf16((m, p.n), 1.0),
                       "a": bf16((wl.r, p.k), p.k ** -0.5), "b": bf16((p.n, wl.r), 0.01)})
            ol.append({"y": torch.empty((m, p.n), dtype=torch.bfloat16, device=dev),
                       "u": torch.empty((m, wl.r), dtype=torch.float32, device=dev),
                       "dx": torch.empty((m, p.k), dtype=torch.bfloat16, device=dev),
                       "da": torch.empty((wl.r, p.k), dtype=torch.float32, device=dev),
                       "db": torch.empty((p.n, wl.r), dtype=torch.float32, device=dev),
                       "ws": torch.empty(max(256, B.workspace_bytes(B.OP_BWD, wl.fmt, p.n, p.k, m, wl.r)),
                                         dtype=torch.uint8, device=dev),
                       "wsf": torch.empty(max(256, B.workspace_bytes(B.OP_FWD, wl.fmt, p.n, p.k, m, wl.r)),
                                          dtype=torch.uint8, device=dev)})
        acts.append(al)
        outs.append(ol)
    stream = torch.cuda.current_stream()
    # independent projections of a decoder layer as grouped calls (q|k|v, gate|up)
    names = [p.name for p in wl.projs]
    groups = [[names.index(n) for n in g if n in names] for g in (["q", "k", "v"], ["o"], ["gate", "up"], ["down"])]
    groups = [g for g in groups if g]
    if sorted(i for g in groups for i in g) != list(range(len(names))):
        groups = None

    def timed(st, steps, warmup):
        for _ in range(warmup):
            st.run(acts, outs, groups)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            st.run(acts, outs, groups)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    # pinned host -> device bandwidth, 1 GiB, in the same process
    hb = torch.empty(1 << 30, dtype=torch.uint8, pin_memory=True)
    db = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    db.copy_(hb, non_blocking=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(3):
        db.copy_(hb, non_blocking=True)
    e1.record(stream)
    torch.cuda.synchronize()
    h2d_gbs = 3 * (1 << 30) / (e0.elapsed_time(e1) / 1e3) / 1e9
    del hb, db

    dev_imgs = [h.to(dev) for h in host]
    res = stack.Stack(layout, wl.r, wl.alpha, images_dev=dev_imgs)
    ms_res = timed(res, args.steps, args.warmup)
    del res, dev_imgs
    torch.cuda.empty_cache()
    st = stack.Stack(layout, wl.r, wl.alpha, images_host=host, n_slots=2)
    ms_st = timed(st, args.steps, args.warmup)
    stats = st.pool.stats()
    st.close()
    copies_per_step = 2 * L - 2
    copy_ms = copies_per_step * layout.nbytes / (h2d_gbs * 1e9) * 1e3
    out = {
        "metric": "QLoRA stack fwd+bwd tokens/s, base streamed from pinned host",
        "value": m / (ms_st / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_st,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.notes, "name": wl.name, "tokens": m, "layers": L,
                   "base_format": FMT_NAME[wl.fmt], "rank": wl.r, "alpha": wl.alpha,
                   "layer_image_bytes": layout.nbytes, "slots": 2,
                   "calls": "grouped q|k|v, o, gate|up, down" if groups else "one call per projection"},
        "stack": {"resident_ms_per_step": ms_res, "resident_tokens_per_s": m / (ms_res / 1e3),
                  "streamed_over_resident": ms_st / ms_res,
                  "copies_per_step": copies_per_step,
                  "streamed_bytes_per_step": copies_per_step * layout.nbytes,
                  "pinned_h2d_gbs": h2d_gbs,
                  "copy_ms_at_measured_h2d": copy_ms,
                  "overlap_efficiency": max(copy_ms, ms_res) / ms_st,
                  "pool_stats_total": stats, "host_prep_s": prep_s},
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    import torch

    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20)
        a = torch.ones(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n}), flush=True)
        return

    from quantized_base_lora_amd import binding as B, synth

    B.load()
    wl = synth.WORKLOADS[args.workload]
    m = args.m or wl.m
    if args.layers:
        return bench_stack(args, wl, m)
    if args.optimizer:
        return optimizer_bench(args, wl)
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream()             # default priority; capturable (not the legacy stream)
    torch.cuda.set_stream(stream)

    def t(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    # inputs, packed bases and preallocated outputs / workspaces
    projs = []
    packed_bytes = 0
    excluded = set(filter(None, args.exclude.split(",")))
    for pi, p in enumerate(wl.projs):
        if (args.proj and p.name != args.proj) or p.name in excluded:
            continue
        c = synth.layer_tensors(wl, pi, m=m)
        qw = B.quant_pack(wl.fmt, torch.from_numpy(c["W"]).to(dev))
        packed_bytes += qw.nbytes()
        d = {"p": p, "qws": [qw], "x": t(c["x"]), "dy": t(c["dY"]), "a": t(c["A"]), "b": t(c["B"]),
             "y": torch.empty((m, p.n), dtype=torch.bfloat16, device=dev),
             "u": torch.empty((m, wl.r), dtype=torch.float32, device=dev),
             "dx": torch.empty((m, p.k), dtype=torch.bfloat16, device=dev),
             "da": torch.empty((wl.r, p.k), dtype=torch.float32, device=dev),
             "db": torch.empty((p.n, wl.r), dtype=torch.float32, device=dev),
             "ws": torch.empty(max(256, B.workspace_bytes(B.OP_BWD, wl.fmt, p.n, p.k, m, wl.r)),
                               dtype=torch.uint8, device=dev),
             "wsf": torch.empty(max(256, B.workspace_bytes(B.OP_FWD, wl.fmt, p.n, p.k, m, wl.r)),
                                dtype=torch.uint8, device=dev)}
        projs.append(d)
    if excluded:
        # per-layer accounting over the projections that run (inputs keep their seeds)
        wl = dataclasses.replace(wl, projs=tuple(p for p in wl.projs if p.name not in excluded))
    # rotate packed copies so weight reads come from HBM, not the 256 MB MALL
    copies = args.copies or max(1, min(8, int(np.ceil(512e6 / packed_bytes))))
    for d in projs:
        base = d["qws"][0]
        for _ in range(copies - 1):
            q2 = B.QWeight(base.fmt, base.n, base.k, base.codes.clone(), base.scales.clone())
            d["qws"].append(q2)
    torch.cuda.synchronize()

    ev_pairs = []

    def fwd(d, i, st):
        B.linear_fwd(d["qws"][i % copies], d["x"], d["a"], d["b"], wl.alpha, y=d["y"], u=d["u"], ws=d["wsf"],
                     stream=st)

    def bwd(d, i, st):
        B.linear_bwd(d["qws"][i % copies], d["x"], d["dy"], d["u"], d["a"], d["b"], wl.alpha, dx=d["dx"],
                     da=d["da"], db=d["db"], ws=d["ws"], stream=st)

    def eager_step(i, timed):
        """One stream; each forward launch bracketed by events (the roofline's kernel timing)."""
        for d in (projs if args.phase != "bwd" else []):
            if timed:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            fwd(d, i, stream)
            if timed:
                e1.record(stream)
                ev_pairs.append((d["p"], e0, e1))
        for d in (reversed(projs) if args.phase != "fwd" else []):
            bwd(d, i, stream)

    # groups of projections with no data dependence in a decoder layer
    by_name = {d["p"].name: d for d in projs}
    order = [g for g in (["q", "k", "v"], ["o"], ["gate", "up"], ["down"])]
    groups = [[by_name[n] for n in g if n in by_name] for g in order]
    groups = [g for g in groups if g] or [[d] for d in projs]
    side = [torch.cuda.Stream() for _ in range(max(len(g) for g in groups))]

    def layer_step(i):
        """fwd groups in order, then bwd groups in reverse; a group's members on parallel streams."""
        phases = []
        if args.phase != "bwd":
            phases.append((groups, fwd))
        if args.phase != "fwd":
            phases.append((list(reversed(groups)), bwd))
        for gs, fn in phases:
            for g in gs:
                if len(g) == 1 or not args.streams:
                    for d in g:
                        fn(d, i, stream)
                    continue
                fork = torch.cuda.Event()
                fork.record(stream)
                for d, st in zip(g, side):
                    st.wait_event(fork)
                    fn(d, i, st)
                for st in side[:len(g)]:
                    join = torch.cuda.Event()
                    join.record(st)
                    stream.wait_event(join)

    # Launch plans (the default for eager launches on one stream): the whole
    # step recorded once per rotated weight copy and enqueued by one library
    # call, so host-side call overhead never idles the GPU between launches;
    # the timing plans bracket each forward call with events.
    use_plan = not (args.no_plan or args.streams or args.graph)
    if use_plan:
        def record(pl, i):
            # calls grouped as a decoder layer allows: q|k|v and gate|up read one input
            for g in (groups if args.phase != "bwd" else []):
                pl.add_fwd_group([(d["qws"][i], d["x"], d["a"], d["b"], wl.alpha, d["y"], d["u"], d["wsf"])
                                  for d in g])
            for g in (reversed(groups) if args.phase != "fwd" else []):
                pl.add_bwd_group([(d["qws"][i], d["x"], d["dy"], d["u"], d["a"], d["b"], wl.alpha, d["dx"],
                                   d["da"], d["db"], d["ws"], False) for d in reversed(g)])
        step_plans = []
        for i in range(copies):
            pl = B.Plan()
            record(pl, i)
            step_plans.append(pl)
        # the roofline's kernel timing: the forward launches of K steps back to back
        # (weight copies rotated as the steps rotate them), one event pair around
        # all of them, so the event markers' own cost (a few microseconds each)
        # is spread over every launch instead of falling on each step's four
        fwd_projs = projs if args.phase != "bwd" else []
        if fwd_projs:
            roof = B.Plan()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            roof.add_event(e0, stream)
            for i in range(args.steps):
                for g in groups:
                    roof.add_fwd_group([(d["qws"][i % copies], d["x"], d["a"], d["b"], wl.alpha, d["y"], d["u"],
                                         d["wsf"]) for d in g])
            roof.add_event(e1, stream)
            # a group is one launch (pair) unless the FP8 base above 64 tokens runs call by call
            nl = (len(fwd_projs) if (wl.fmt == 3 and m > 64) else len(groups)) * args.steps
        torch.cuda.synchronize()
        for i in range(args.warmup):
            step_plans[i % copies].run(stream)
        if fwd_projs:
            roof.run(stream)                   # untimed pass
            roof.run(stream)
            torch.cuda.synchronize()
            ev_pairs.append(([d["p"] for d in fwd_projs] * args.steps, nl, e0.elapsed_time(e1)))
    else:
        # the roofline's kernel timing: eager launches on one stream
        for i in range(args.warmup):
            eager_step(i, False)
        torch.cuda.synchronize()
        for i in range(args.steps):
            eager_step(i, True)
        torch.cuda.synchronize()
        ev_pairs[:] = [([pp], 1, e0.elapsed_time(e1)) for pp, e0, e1 in ev_pairs]

    # the step itself: HIP-graph replays (one graph per rotated weight copy) or eager launches
    graphs = []
    if args.graph:
        for i in range(copies):
            layer_step(i)                      # warm the side streams outside capture
        torch.cuda.synchronize()
        for i in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                layer_step(i)
            graphs.append(g)
        torch.cuda.synchronize()

    def run(i):
        if graphs:
            graphs[i % copies].replay()
        elif use_plan:
            step_plans[i % copies].run(stream)
        else:
            layer_step(i)

    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        run(i)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    # spread of single steps, from a separate pass with an event between steps
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record(stream)
    for i in range(args.steps):
        run(i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per_step = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])
    spread = {"p10": float(np.percentile(per_step, 10)), "median": float(np.median(per_step)),
              "p90": float(np.percentile(per_step, 90)), "pass": "separate, one event between steps"}

    fwd_ms = sum(t for _, _, t in ev_pairs)
    fwd_flops = sum(fwd_kernel_flops(wl, p, m) for ps, _, _ in ev_pairs for p in ps)
    n_launch = max(1, sum(nl for _, nl, _ in ev_pairs))
    n_calls = max(1, sum(len(ps) for ps, _, _ in ev_pairs))
    fwd_ms = fwd_ms or float("nan")
    avg_launch_ms = fwd_ms / n_launch
    achieved = fwd_flops / (fwd_ms / 1e3) / 1e12
    traffic = traffic_from_profile(args.workload, m)

    flops = layer_flops(wl, m)
    nbytes = layer_bytes(wl, m)
    out = {
        "metric": METRIC,
        "value": m / (ms / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_spread": spread,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.notes, "name": wl.name, "tokens": m, "base_format": FMT_NAME[wl.fmt],
                   "rank": wl.r, "alpha": wl.alpha, "projections": [f"{p.name}:{p.k}->{p.n}" for p in wl.projs],
                   "packed_copies_rotated": copies, "excluded_projections": sorted(excluded),
                   "step_mode": ("HIP graph replay" if args.graph else
                                 "eager launches, one library call per step (recorded launch plan; "
                                 "q|k|v and gate|up as grouped calls)" if use_plan
                                 else "eager launches, one library call per layer call") + (
                       ", q|k|v and gate|up on parallel streams" if args.streams else ", one stream")},
        "layer": {"tflops": flops / (ms / 1e3) / 1e12, "frac_bf16_peak": flops / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
                  "algorithmic_bytes": nbytes, "hbm_gbs": nbytes / (ms / 1e3) / 1e9,
                  "frac_hbm_peak": nbytes / (ms / 1e3) / 1e9 / PEAK_HBM_GBS},
        "roofline": {"kernel": "qgemm_kernel (forward: dequant GEMM + fused LoRA)", "bound": "mfma",
                     "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                     "avg_launch_us": avg_launch_ms * 1e3, "launches_timed": n_launch, "calls_timed": n_calls,
                     "timing": ("one HIP event pair around the forward launches of K steps, enqueued back "
                                "to back by one launch plan (q|k|v and gate|up one launch each), total / launches"
                                if use_plan else
                                "HIP events around each forward call"),
                     "flops_per_launch_avg": fwd_flops / n_launch},
    }
    if wl.fmt == 3 and m > 64 and ev_pairs:
        # the FP8 base above 64 tokens: activation split, rank-r projection and the
        # fp8 GEMM (two E4M3 products per output, hi and lo terms) per call; the
        # algorithmic FLOPs against the fp8 peak
        out["dtype"] = "fp8_e4m3"
        out["roofline"].update({"kernel": "qgemm8_kernel (forward: fp8 GEMM over the two-term E4M3 activation "
                                          "split, with act_quant_kernel and rproj_kernel per call)",
                                "peak": PEAK_FP8_TFLOPS, "frac": achieved / PEAK_FP8_TFLOPS,
                                "executed_fp8_flops_per_algorithmic": 2})
    if m <= 64:
        fwd_bytes = sum(BPW[wl.fmt] * p.n * p.k + m * 2 * (p.k + p.n) for ps, _, _ in ev_pairs for p in ps) / n_launch
        gbs = fwd_bytes / (avg_launch_ms / 1e3) / 1e9
        out["roofline"].update({"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                "frac": gbs / PEAK_HBM_GBS, "bytes_per_launch_avg": fwd_bytes})
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, min(args.cpu_tokens, m) if args.cpu_tokens else m)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
