"""Benchmark: QLoRA linear layer forward + backward on one MI355X.

One step = forward of every projection of a decoder layer (7 LoRA linears over
a frozen quantized base), then backward of every projection (dX, dA, dB), on
synthetic seeded inputs resident in HBM, issued in the launch configuration
of layer.LayerStep (a recorded launch plan, q|k|v and gate|up grouped).
Reported value: tokens/s per layer.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
        every workload in one JSON line: the headline is the largest layer,
        the Qwen3-8B layer with an FP8 E4M3 base at 8192 tokens; the single
        256->256 linear, the Qwen3-0.6B NF4 layer (8192 tokens), the
        Llama-3.1-8B NF4 layer (4096, 64, 16 tokens) and the 32-layer
        Llama-3.1-8B stack streamed from pinned host memory (2048 and 16
        tokens, checked bit for bit against the resident stack) are
        sub-records under "configs"
    python bench.py --workload NAME [--m M] [--layers L]   one workload only
    python bench.py --optimizer --workload NAME            the fused AdamW step

Each record carries the roofline of its dominant kernel (the forward
launches of its steps, back to back, bracketed by one HIP event pair on the
stream they run on); the headline also carries the CPU oracle timed on this
host (one thread and all cores) on a bounded sample.
"""

import argparse
import hashlib
import json
import math
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
FMT_NAME = {1: "q4_0", 2: "nf4", 3: "fp8_e4m3", 4: "mxfp4", 5: "q8_0", 6: "nvfp4"}
BPW = {1: 18 / 32, 2: 0.5 + 4 / 64, 3: 1.0, 4: 17 / 32, 5: 34 / 32, 6: 0.5 + 1 / 16}
ROTATE_BYTES = 512e6           # packed weight copies rotated per config (the MALL is 256 MB)
MAX_CFG_STEPS = 20000          # sub-record steps: enough to pass over every rotated copy

HEADLINE = ("qwen3_8b_fp8", 8192)
LAYER_CONFIGS = [("single256_q40", 64), ("qwen3_0.6b_nf4", 8192), ("llama3.1_8b_nf4", 4096),
                 ("llama3.1_8b_nf4", 64), ("llama3.1_8b_nf4", 16), ("qwen3_8b_fp8", 8192)]
STACK_WORKLOAD, STACK_LAYERS, STACK_TOKENS = "llama3.1_8b_nf4_stack32", 32, (2048, 16)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None, help="one workload only (default: every workload)")
    ap.add_argument("--m", type=int, default=None, help="tokens (default: the workload's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=64, help="tokens in the CPU oracle sample")
    ap.add_argument("--copies", type=int, default=0, help="packed weight copies rotated (0: >= 512 MB)")
    ap.add_argument("--proj", default=None, help="run only this projection (profiling)")
    ap.add_argument("--exclude", default="",
                    help="comma-separated projections left out of the layer (e.g. o), in the timing and in "
                         "every per-layer figure")
    ap.add_argument("--phase", default="both", choices=["both", "fwd", "bwd"], help="profiling: one pass only")
    ap.add_argument("--no-stack", action="store_true", help="leave the streamed stack out of the full run")
    ap.add_argument("--optimizer", action="store_true",
                    help="time the fused AdamW step on the layer's adapters instead of the layer step")
    ap.add_argument("--state8", action="store_true", help="with --optimizer: the 8-bit block-wise state")
    ap.add_argument("--layers", type=int, default=0,
                    help="stack mode: this many layers, resident vs streamed from pinned host")
    ap.add_argument("--hbm-ceiling", action="store_true",
                    help="only measure plain streaming kernels (device copy, read-only reduction) over 4 GiB "
                         "and exit: the HBM ceiling the kernels are compared with")
    ap.add_argument("--counters-json", default=None, metavar="DIR",
                    help="build profiles/fwd_counters.json from the rocprofv3 FETCH_SIZE / WRITE_SIZE runs in DIR "
                         "(fetch_<workload>_m<tokens>, write_..., fetch_copy, write_copy) and exit; needs no GPU")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device-to-device (a plain copy kernel of known size, "
                         "to calibrate HBM byte counters) and exit")
    return ap.parse_args()


# ----------------------------------------------------------------------------- accounting

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


def fwd_kernel_bytes(wl, p, m):
    """Algorithmic bytes of one forward call: the packed base, x and A read,
    y written (bf16), U written (fp32), B read."""
    return BPW[wl.fmt] * p.n * p.k + 2 * m * (p.k + p.n) + 4 * m * wl.r + 2 * wl.r * (p.k + p.n)


def source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_base_lora_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(key):
    """HBM bytes per dominant-kernel launch from committed rocprofv3 counters,
    if they were taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "fwd_counters.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha") != source_hash():
        return None
    e = d.get("configs", {}).get(key)
    return None if e is None else e.get("hbm_bytes_per_launch")


def fwd_launches_per_step(wl, m):
    """Forward GEMM launches of one layer step, as layer.LayerStep issues
    them: one per group of calls (q|k|v, o, gate|up, down; one per call when
    the layer's projections do not form those groups)."""
    from quantized_base_lora_amd.layer import GROUPS
    names = [p.name for p in wl.projs]
    groups = [g for g in ([n for n in grp if n in names] for grp in GROUPS) if g]
    if sum(len(g) for g in groups) != len(names):
        groups = [[n] for n in names]
    return len(groups)


MAIN_FWD_KERNELS = ("qgemm_kernel", "qgemm8_kernel", "qstream16_kernel", "qsplit16_kernel", "qsplit_kernel")
SETUP_KERNELS = ("pack4_kernel", "pack_nvfp4_kernel", "absmax_kernel", "quant_fp8_kernel", "fill_u32_kernel")


def _kernel_base(name):
    n = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return n.split("(")[0].split("<")[0].split("::")[-1]


def _counter_rows(path, counter):
    """(kernel base name, value) per dispatch of one counter in a rocprofv3 CSV."""
    import csv
    out = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                out.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    out.sort()
    return [(n, v) for _, n, v in out]


def counters_json(art):
    """HBM bytes per forward launch of every layer config, from rocprofv3
    counter runs of `bench.py --workload W --m M --phase fwd` (only forward
    launches run after the bases are packed): every library kernel but the
    packing ones is summed, FETCH_SIZE and WRITE_SIZE (KiB per dispatch)
    scaled by what the same counters read for a plain 1 GiB device copy, and
    divided by the number of forward launches (dispatches of the GEMM kernel,
    one per group of calls; the reduction, activation-split and projection
    kernels belong to their launch)."""
    def path(tag):
        return os.path.join(art, f"{tag}_counter_collection.csv")
    copy = 1 << 30
    fk = max(v for n, v in _counter_rows(path("fetch_copy"), "FETCH_SIZE") if "copyBuffer" in n)
    wk = max(v for n, v in _counter_rows(path("write_copy"), "WRITE_SIZE") if "copyBuffer" in n)
    ff, wf = copy / (fk * 1024), copy / (wk * 1024)
    from quantized_base_lora_amd import synth
    entries, cmds = {}, []
    for name, m in LAYER_CONFIGS:
        tag = f"{name}_m{m}"
        if not os.path.exists(path(f"fetch_{tag}")):
            continue
        wl = synth.WORKLOADS[name]
        per = {}
        for cname, tagp in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
            rows = [(n, v) for n, v in _counter_rows(path(f"{tagp}_{tag}"), cname)
                    if "ql::" in n and _kernel_base(n) not in SETUP_KERNELS]
            launches = sum(1 for n, _ in rows if _kernel_base(n) in MAIN_FWD_KERNELS)
            per[cname] = (sum(v for _, v in rows), launches, sorted({_kernel_base(n) for n, _ in rows}))
        (fs, nl, kern), (ws, nl2, _) = per["FETCH_SIZE"], per["WRITE_SIZE"]
        assert nl == nl2 and nl > 0, (tag, nl, nl2)
        hbm = (fs * 1024 * ff + ws * 1024 * wf) / nl
        alg = sum(fwd_kernel_bytes(wl, p, m) for p in wl.projs) / fwd_launches_per_step(wl, m)
        entries[f"{name}@{m}"] = {"hbm_bytes_per_launch": hbm, "algorithmic_bytes_per_launch": alg,
                                  "hbm_over_algorithmic": hbm / alg, "launches_counted": nl,
                                  "FETCH_SIZE_KiB_per_launch": fs / nl, "WRITE_SIZE_KiB_per_launch": ws / nl,
                                  "kernels": kern}
        for tagp, cname in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
            cmds.append(f"rocprofv3 --pmc {cname} --output-format csv -d {art} -o {tagp}_{tag} -- python3 bench.py "
                        f"--workload {name} --m {m} --phase fwd --steps 2 --warmup 1 --no-cpu-baseline")
    for tagp, cname in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        cmds.append(f"rocprofv3 --pmc {cname} --output-format csv -d {art} -o {tagp}_copy -- python3 bench.py "
                    f"--calibrate-copy 1024")
    out = {"what": "HBM bytes per forward launch (a launch: one group of calls, with its reduction, or for the FP8 "
                   "base above 64 tokens with its activation splits and projections)",
           "kernel_source_sha": source_hash(), "commands": cmds,
           "calibration": {"copy_bytes": copy, "FETCH_SIZE_KiB": fk, "WRITE_SIZE_KiB": wk,
                           "fetch_factor": ff, "write_factor": wf},
           "configs": entries}
    dst = os.path.join(ROOT, "profiles", "fwd_counters.json")
    with open(dst, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps({"written": dst, "configs": sorted(entries)}), flush=True)


def copies_for(packed_bytes, override=0):
    return override or max(1, math.ceil(ROTATE_BYTES / max(1, packed_bytes)))


def roofline_kind(wl, m):
    if m <= 64:
        return {"kernel": "qstream16_kernel (16 tokens, 4-bit) / qsplit_kernel + split_reduce_kernel (forward: split-contraction "
                          "dequant GEMM, fixed-order reduction with the fused LoRA term)",
                "bound": "hbm", "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    if wl.fmt == 3:
        return {"kernel": "qgemm8_kernel with act_quant_kernel and rproj_kernel (forward: fp8 GEMM over the "
                          "two-term E4M3 activation split, rank-r projection, fused LoRA term)",
                "bound": "mfma", "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                "executed_fp8_flops_per_algorithmic": 2}
    return {"kernel": "qgemm_kernel (forward: dequant GEMM + fused LoRA)", "bound": "mfma",
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}


# ----------------------------------------------------------------------------- one layer

def bench_layer(args, wl, m, steps, exclude=(), only=None):
    """Time one layer config; returns its record (without cpu_baseline)."""
    import torch

    from quantized_base_lora_amd import binding as B, layer

    est = sum(BPW[wl.fmt] * p.n * p.k for p in wl.projs
              if p.name not in exclude and (only is None or p.name == only))
    copies = copies_for(est, args.copies)
    ls = layer.LayerStep(wl, m, copies=copies, exclude=exclude, only=only)
    packed = ls.packed_bytes()
    if exclude or only:
        import dataclasses
        wl = dataclasses.replace(wl, projs=tuple(d["p"] for d in ls.projs))
    stream = torch.cuda.Stream()             # default priority
    torch.cuda.set_stream(stream)
    plans = ls.plans(args.phase)
    torch.cuda.synchronize()

    # the roofline's kernel timing: the forward launches of `steps` steps back to
    # back, weight copies rotated as the steps rotate them, one event pair around
    # all of them (an event per step would add its own cost to every step)
    roof = None
    if args.phase != "bwd":
        roof = B.Plan()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        roof.add_event(e0, stream)
        for i in range(steps):
            for g in ls.groups:
                roof.add_fwd_group(ls.fwd_items(g, i))
        roof.add_event(e1, stream)

    for i in range(args.warmup):
        plans[i % copies].run(stream)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        plans[i % copies].run(stream)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    # spread of single steps, from a separate pass with an event between steps
    ns = min(steps, 200)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(ns + 1)]
    evs[0].record(stream)
    for i in range(ns):
        plans[i % copies].run(stream)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per_step = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(ns)])
    spread = {"p10": float(np.percentile(per_step, 10)), "median": float(np.median(per_step)),
              "p90": float(np.percentile(per_step, 90)), "steps": ns,
              "pass": "separate, one event between steps"}

    rec = {"workload": wl.notes, "name": wl.name, "tokens": m, "base_format": FMT_NAME[wl.fmt],
           "rank": wl.r, "alpha": wl.alpha, "projections": [f"{p.name}:{p.k}->{p.n}" for p in wl.projs],
           "steps": steps, "warmup": args.warmup, "ms_per_step": ms, "tokens_per_s": m / (ms / 1e3),
           "ms_per_step_spread": spread, "packed_bytes_per_copy": packed, "packed_copies_rotated": copies,
           "rotated_bytes": packed * copies, "copies_touched_in_timed_steps": min(copies, steps),
           "step_mode": "eager launches, one library call per step (recorded launch plan; q|k|v and "
                        "gate|up as grouped calls), one stream"}
    flops, nbytes = layer_flops(wl, m), layer_bytes(wl, m)
    rec["layer"] = {"tflops": flops / (ms / 1e3) / 1e12, "frac_bf16_peak": flops / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
                    "algorithmic_bytes": nbytes, "hbm_gbs": nbytes / (ms / 1e3) / 1e9,
                    "frac_hbm_peak": nbytes / (ms / 1e3) / 1e9 / PEAK_HBM_GBS}
    if roof is not None:
        roof.run(stream)                       # untimed pass
        roof.run(stream)
        torch.cuda.synchronize()
        fwd_ms = e0.elapsed_time(e1)
        n_launch = ls.fwd_launches_per_step() * steps
        n_calls = len(ls.projs) * steps
        avg_ms = fwd_ms / n_launch
        r = roofline_kind(wl, m)
        if r["bound"] == "hbm":
            per_launch = sum(fwd_kernel_bytes(wl, d["p"], m) for d in ls.projs) * steps / n_launch
            achieved = per_launch / (avg_ms / 1e3) / 1e9
            r["bytes_per_launch_avg"] = per_launch
        else:
            per_launch = sum(fwd_kernel_flops(wl, d["p"], m) for d in ls.projs) * steps / n_launch
            achieved = per_launch / (avg_ms / 1e3) / 1e12
            r["flops_per_launch_avg"] = per_launch
        r.update({"achieved": achieved, "frac": achieved / r["peak"],
                  "traffic": traffic_from_profile(f"{wl.name}@{m}"),
                  "avg_launch_us": avg_ms * 1e3, "launches_timed": n_launch, "calls_timed": n_calls,
                  "timing": "one HIP event pair around the forward launches of the config's steps, enqueued "
                            "back to back by one launch plan, total / launches"})
        rec["roofline"] = r
        roof.close()
    ls.close()
    del ls, plans
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


# ----------------------------------------------------------------------------- the streamed stack

def h2d_bandwidth(stream):
    """Pinned host -> device bandwidth, 1 GiB copies, in this process."""
    import torch
    hb = torch.empty(1 << 30, dtype=torch.uint8, pin_memory=True)
    db = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    db.copy_(hb, non_blocking=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(3):
        db.copy_(hb, non_blocking=True)
    e1.record(stream)
    torch.cuda.synchronize()
    return 3 * (1 << 30) / (e0.elapsed_time(e1) / 1e3) / 1e9


def bench_stack(args, wl, n_layers, tokens, steps):
    """The layer stack: L layers, forward 0..L-1 then backward L-1..0, the
    packed bases resident in HBM or streamed from pinned host memory through
    two device slots (one layer ahead on a side stream).  The streamed run's
    outputs (every output of every layer, from its last timed step) are
    compared bit for bit with the resident run's.  Returns one record per
    token count."""
    import torch

    from quantized_base_lora_amd import stack

    t0 = time.time()
    layout, host, _ = stack.build_host_images(wl, n_layers)
    prep_s = time.time() - t0
    stream = torch.cuda.current_stream()
    h2d_gbs = h2d_bandwidth(stream)
    groups = stack.layer_groups(wl.projs)

    def timed(st, acts, outs):
        for _ in range(args.warmup):
            st.run(acts, outs, groups)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            st.run(acts, outs, groups)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    recs = []
    for m in tokens:
        acts = stack.layer_inputs(wl, m, n_layers)
        o_res = stack.layer_outputs(wl, m, n_layers)
        dev_imgs = [h.to("cuda") for h in host]
        ms_res = timed(stack.Stack(layout, wl.r, wl.alpha, images_dev=dev_imgs), acts, o_res)
        del dev_imgs
        torch.cuda.empty_cache()
        o_st = stack.layer_outputs(wl, m, n_layers)
        st = stack.Stack(layout, wl.r, wl.alpha, images_host=host, n_slots=2)
        ms_st = timed(st, acts, o_st)
        stats = st.pool.stats()
        st.close()
        equal, first, worst = stack.compare_outputs(o_res, o_st)
        n_out = n_layers * len(wl.projs) * len(stack.OUTPUT_KEYS)
        del acts, o_res, o_st
        torch.cuda.empty_cache()
        copies_per_step = 2 * n_layers - 2
        copy_ms = copies_per_step * layout.nbytes / (h2d_gbs * 1e9) * 1e3
        recs.append({
            "workload": wl.notes, "name": wl.name, "tokens": m, "layers": n_layers,
            "base_format": FMT_NAME[wl.fmt], "rank": wl.r, "alpha": wl.alpha,
            "steps": steps, "warmup": args.warmup, "ms_per_step": ms_st, "tokens_per_s": m / (ms_st / 1e3),
            "layer_image_bytes": layout.nbytes, "slots": 2,
            "calls": "grouped q|k|v, o, gate|up, down" if groups else "one call per projection",
            "resident_ms_per_step": ms_res, "resident_tokens_per_s": m / (ms_res / 1e3),
            "streamed_over_resident": ms_st / ms_res, "copies_per_step": copies_per_step,
            "streamed_bytes_per_step": copies_per_step * layout.nbytes, "pinned_h2d_gbs": h2d_gbs,
            "copy_ms_at_measured_h2d": copy_ms, "overlap_efficiency": max(copy_ms, ms_res) / ms_st,
            "roofline": {"kernel": "host-to-device copies of the layer images (PCIe)", "bound": "pcie",
                         "achieved": copies_per_step * layout.nbytes / (ms_st / 1e3) / 1e9,
                         "peak": h2d_gbs, "unit": "GB/s",
                         "frac": copies_per_step * layout.nbytes / (ms_st / 1e3) / 1e9 / h2d_gbs,
                         "peak_is": "pinned H2D bandwidth measured in this run"},
            "check": {"streamed_equals_resident_bitwise": bool(equal), "max_abs_diff": worst,
                      "outputs_compared": n_out, "first_mismatch": first,
                      "what": "every y, U, dX, dA, dB of every layer, last timed step of each run"},
            "pool_stats_total": stats, "host_prep_s": prep_s})
    del host
    return recs


# ----------------------------------------------------------------------------- oracle on the host

def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, m, tokens, min_seconds=5.0):
    """The oracle (numpy, fp64 products) on a bounded sample of the layer:
    the first `tokens` tokens of the same seeded inputs (drawn on the GPU and
    copied to the host), every projection's base packed and dequantized by the
    oracle beforehand (untimed); then forward + backward of every projection,
    repeated until min_seconds of wall time, once on one thread and once on
    every core the process may use."""
    import torch
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import formats as ofmt, lora as olora
    from quantized_base_lora_amd import synth

    t0 = time.time()
    prep = []
    for pi in range(len(wl.projs)):
        t = synth.layer_tensors_torch(wl, pi, m=m)
        w = t["W"].cpu().numpy()
        codes, scales = ofmt.pack(wl.fmt, w)
        wd = ofmt.dequant(wl.fmt, codes, scales)
        del w, codes, scales
        prep.append(tuple(t[k][:tokens].float().cpu().numpy() if k in ("x", "dY") else t[k].float().cpu().numpy()
                          for k in ("x", "dY", "A", "B")) + (wd,))
        del t
    torch.cuda.empty_cache()
    prep_s = time.time() - t0

    def run(limit):
        passes, dt = 0, 0.0
        with threadpool_limits(limit):
            while dt < min_seconds and passes < 50:
                t1 = time.perf_counter()
                for x, dy, a, b, wd in prep:
                    olora.forward(x, wd, a, b, wl.alpha)
                    olora.backward(x, dy, wd, a, b, wl.alpha)
                dt += time.perf_counter() - t1
                passes += 1
        return tokens * passes / dt, passes, dt

    one, p1, d1 = run(1)
    cores = len(os.sched_getaffinity(0))
    allc, pa, da = run(cores)
    threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] + [1])
    return {"value": allc, "unit": "tokens/s", "cores": int(min(cores, threads)), "kind": "oracle",
            "single_thread": {"value": one, "unit": "tokens/s", "cores": 1, "passes": p1, "seconds": d1},
            "all_cores": {"value": allc, "unit": "tokens/s", "cores": cores, "passes": pa, "seconds": da},
            "cpu_model": cpu_model(), "host_cpus_visible": cores, "untimed_prep_s": prep_s,
            "sample": f"first {tokens} of the {m} tokens of the same layer (all {len(wl.projs)} projections, "
                      f"forward + backward, fp64 products; every base packed and dequantized by the oracle "
                      f"beforehand, untimed); tokens/s scales linearly in tokens"}


# ----------------------------------------------------------------------------- AdamW mode

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
    # 8-bit state: param, grad read (8), codes read (2), param and codes written (6), bf16 copy (2);
    # fp32 state: param, grad, m, v read (16), param, m, v written (12), bf16 copy (2)
    per_el = 18 if args.state8 else 30
    copies = max(1, int(np.ceil(ROTATE_BYTES / (n_el * (10 if args.state8 else 18)))))
    gen = torch.Generator(device=dev).manual_seed(1)
    sets = []
    for _ in range(copies):
        ts = []
        for n in sizes:
            p0 = torch.randn(n, device=dev, generator=gen) * 0.02
            g0 = torch.randn(n, device=dev, generator=gen) * 1e-3
            pb = torch.empty(n, dtype=torch.bfloat16, device=dev)
            if args.state8:
                ts.append((p0, g0, B.Adamw8State(n, device=dev), pb))
            else:
                ts.append((p0, g0, torch.zeros(n, device=dev), torch.zeros(n, device=dev), pb))
        sets.append(ts)
    plans = [(B.Adamw8Plan(ts) if args.state8 else B.AdamwPlan(ts)) for ts in sets]
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
    out = {"metric": "fused AdamW adapter step" + (" (8-bit block-wise state)" if args.state8 else "") +
                     ", algorithmic HBM GB/s", "value": gbs, "unit": "GB/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "us_per_step": us,
           "higher_is_better": True, "dtype": "f32", "data": "synthetic",
           "config": {"workload": f"adapters of one {wl.notes}", "tensors": len(sizes), "elements": n_el,
                      "bytes_per_element": per_el, "state_copies_rotated": copies,
                      "step_mode": "HIP graph of the launches, replayed"},
           "roofline": {"kernel": "adamw8_kernel" if args.state8 else "adamw_kernel", "bound": "hbm",
                        "achieved": gbs, "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS, "traffic": None}}
    print(json.dumps(out), flush=True)


# ----------------------------------------------------------------------------- HBM ceiling

def hbm_ceiling(args):
    """Plain streaming kernels on 4 GiB (16x the MALL): the library's
    streaming read (ql_stream_read, one pass, every word read once), a
    device-to-device copy (read + write) and a read-only reduction (torch's
    sum), each timed with HIP events over several repetitions; bytes moved /
    time.  The streaming read's XOR of all words is checked against the
    host's on a 64 MB prefix first."""
    import torch

    from quantized_base_lora_amd import binding as B
    n = 4 << 30
    a = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    a[:: 4097] = 3.0                                   # a pattern whose XOR is not zero
    b = torch.empty_like(a)
    sink = torch.empty(B.STREAM_READ_THREADS, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    chk = a[: 1 << 24]                                 # 64 MB: every word read once, checked on the host
    B.stream_read(chk, sink, stream)
    got = int(np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)))
    want = int(np.bitwise_xor.reduce(chk.cpu().numpy().view(np.uint32)))
    if got != want:
        raise SystemExit(f"stream read check failed: XOR {got:#x} != {want:#x}")
    out = {}
    for name, fn, nbytes in (("read_kernel", lambda: B.stream_read(a, sink, stream), n),
                             ("copy", lambda: b.copy_(a), 2 * n), ("read_sum", lambda: a.sum(), n)):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = {"gbs": nbytes / (ms / 1e3) / 1e9, "ms": ms, "bytes": nbytes,
                     "frac_of_8000": nbytes / (ms / 1e3) / 1e9 / PEAK_HBM_GBS}
    print(json.dumps({"hbm_ceiling": out, "buffer_bytes": n}), flush=True)


# ----------------------------------------------------------------------------- main

def line_from(rec, args, steps):
    """The JSON line's top level from one layer record."""
    dtype = "fp8_e4m3 base on fp8 MFMA, bf16 activations and adapters" if rec["base_format"] == "fp8_e4m3" \
        else "bf16"
    return {"metric": METRIC, "value": rec["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": steps,
            "warmup": args.warmup, "ms_per_step": rec["ms_per_step"],
            "ms_per_step_spread": rec.get("ms_per_step_spread"), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": dtype, "data": "synthetic",
            "config": {k: rec[k] for k in ("workload", "name", "tokens", "base_format", "rank", "alpha",
                                           "projections", "packed_copies_rotated", "rotated_bytes",
                                           "step_mode") if k in rec},
            "layer": rec.get("layer"), "roofline": rec.get("roofline")}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    if args.counters_json:
        return counters_json(args.counters_json)
    import torch

    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20)
        a = torch.ones(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n}), flush=True)
        return

    if args.hbm_ceiling:
        return hbm_ceiling(args)

    from quantized_base_lora_amd import binding as B, synth

    B.load()
    if args.workload is not None:
        wl = synth.WORKLOADS[args.workload]
        m = args.m or wl.m
        if args.optimizer:
            return optimizer_bench(args, wl)
        if args.layers:
            for rec in bench_stack(args, wl, args.layers, (m,), args.steps):
                out = {"metric": "QLoRA stack fwd+bwd tokens/s, base streamed from pinned host",
                       "value": rec["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
                       "warmup": args.warmup, "ms_per_step": rec["ms_per_step"], "higher_is_better": True,
                       "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
                       "config": {"workload": rec["workload"], "tokens": m, "layers": args.layers}, "stack": rec}
                print(json.dumps(out), flush=True)
            return
        excluded = tuple(filter(None, args.exclude.split(",")))
        rec = bench_layer(args, wl, m, args.steps, exclude=excluded, only=args.proj)
        out = line_from(rec, args, args.steps)
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline(wl, m, min(args.cpu_tokens, m))
        print(json.dumps(out), flush=True)
        return

    # every workload: the headline layer timed with exactly --steps steps, the
    # others with enough steps to pass over every rotated weight copy
    configs = {}
    head = None
    for name, m in LAYER_CONFIGS:
        wl = synth.WORKLOADS[name]
        key = f"{name}@{m}"
        if (name, m) == HEADLINE:
            steps = args.steps
        else:
            probe_bytes = sum(BPW[wl.fmt] * p.n * p.k for p in wl.projs)
            steps = min(MAX_CFG_STEPS, max(args.steps, copies_for(probe_bytes, args.copies)))
        print(f"[bench] {key}: {steps} steps", file=sys.stderr, flush=True)
        rec = bench_layer(args, wl, m, steps)
        configs[key] = rec
        if (name, m) == HEADLINE:
            head = rec
    if not args.no_stack:
        wl = synth.WORKLOADS[STACK_WORKLOAD]
        print(f"[bench] {STACK_WORKLOAD}: {STACK_LAYERS} layers at {STACK_TOKENS} tokens", file=sys.stderr,
              flush=True)
        for rec in bench_stack(args, wl, STACK_LAYERS, STACK_TOKENS, min(args.steps, 5)):
            configs[f"{STACK_WORKLOAD}@{rec['tokens']}"] = rec
    out = line_from(head, args, args.steps)
    out["config"]["headline"] = "the largest single-GPU layer config (6.44 TFLOP per step)"
    out["configs"] = configs
    if not args.no_cpu_baseline:
        print("[bench] cpu oracle sample", file=sys.stderr, flush=True)
        wl = synth.WORKLOADS[HEADLINE[0]]
        out["cpu_baseline"] = cpu_baseline(wl, HEADLINE[1], min(args.cpu_tokens, HEADLINE[1]))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
