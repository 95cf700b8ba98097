"""Full-size parity in the launch configuration the benchmark times: one
decoder layer's seven projections (q|k|v and gate|up as grouped calls, the
step recorded as a launch plan, layer.LayerStep), every output of every
projection compared with the oracle on every row at the workloads' own
sizes, so every output tile, including the per-XCD tile order and the
grouped row blocks that only large shapes reach, is checked element by
element.  The packed bases are compared with the oracle's bit for bit, and a
second run of the step must reproduce every output bit for bit.

Bars: max|err| / max|ref| <= 1e-2; 3e-2 on y and dX for the FP8 base."""

import sys

import numpy as np
import pytest
import torch

import helpers as H
from oracle import formats as ofmt
from quantized_base_lora_amd import layer, synth

pytestmark = pytest.mark.gpu

CONFIGS = [
    ("single256_q40", 64),
    ("qwen3_0.6b_nf4", 8192),
    ("llama3.1_8b_nf4", 4096), ("llama3.1_8b_nf4", 64), ("llama3.1_8b_nf4", 16),
    ("qwen3_8b_fp8", 8192),
    ("llama3.1_8b_mxfp4", 4096), ("llama3.1_8b_mxfp4", 64), ("llama3.1_8b_mxfp4", 16),
    ("llama3.1_8b_q8_0", 4096), ("llama3.1_8b_q8_0", 64), ("llama3.1_8b_q8_0", 16),
    ("llama3.1_8b_nvfp4", 4096), ("llama3.1_8b_nvfp4", 64), ("llama3.1_8b_nvfp4", 16),
]

_oracle_cache = {}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def oracle_base(wname, pi, w_host):
    """Oracle codes, scales and dequantized base of a projection (the bases
    do not depend on the token count, so one workload's are packed once)."""
    key = (wname, pi)
    if key not in _oracle_cache:
        if any(k[0] != wname for k in _oracle_cache):
            _oracle_cache.clear()
        wl = synth.WORKLOADS[wname]
        c, s = ofmt.pack(wl.fmt, w_host.numpy())
        _oracle_cache[key] = (c, s, ofmt.dequant(wl.fmt, c, s))
    return _oracle_cache[key]


def snapshot(ls):
    return [{k: d[k].clone() for k in ("y", "u", "dx", "da", "db")} for d in ls.projs]


@pytest.mark.parametrize("wname,m", CONFIGS, ids=[f"{w}-m{m}" for w, m in CONFIGS])
def test_layer_step_full_size(lib, wname, m):
    wl = synth.WORKLOADS[wname]
    say(f"full-size layer step {wname} at {m} tokens")
    ls = layer.LayerStep(wl, m, copies=1, keep_w=True)
    ls.run(0)
    torch.cuda.synchronize()
    first = snapshot(ls)
    ls.run(0)
    torch.cuda.synchronize()
    for d, f in zip(ls.projs, first):
        for key in f:
            v = torch.int16 if f[key].dtype == torch.bfloat16 else torch.int32
            assert torch.equal(d[key].view(v), f[key].view(v)), (d["p"].name, key, "second run differs")
    tol_base = H.FP8_TOL if wl.fmt == ofmt.FMT_FP8 else H.FWD_TOL
    for d in ls.projs:
        p = d["p"]
        c, s, wd = oracle_base(wname, d["pi"], d["W"])
        qw = d["qws"][0]
        assert np.array_equal(H.tensor_bytes(qw.codes), np.ascontiguousarray(c).ravel()), p.name
        assert np.array_equal(H.tensor_bytes(qw.scales), H.scales_bytes(wl.fmt, s)), p.name
        ref = H.oracle_outputs(d["x"], d["dy"], d["a"], d["b"], wd, wl.alpha)
        got = {"y": d["y"], "U": d["u"], "dX": d["dx"], "dA": d["da"], "dB": d["db"]}
        errs = {}
        for key, tol in (("y", tol_base), ("U", H.FWD_TOL), ("dX", tol_base), ("dA", H.FWD_TOL),
                         ("dB", H.FWD_TOL)):
            errs[key] = H.rel(H.f32_host(got[key]), ref[key])
            assert errs[key] <= tol, (p.name, key, errs[key])
        say(f"  {p.name} K={p.k} N={p.n}: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    ls.close()
