"""Seeded synthetic inputs and workload shapes.

This module only draws random numbers and describes shapes; it holds none of
the layer's arithmetic.  Both the GPU tests and the CPU oracle are fed from it.

Every tensor comes from ``numpy.random.default_rng([workload, layer, proj,
tensor])`` with tensor ids W=0, A=1, B=2, x=3, dY=4.  Draws are fp32 standard
normals times a standard deviation; activations and adapters are then rounded
to bf16 (nearest even) because that is the dtype the layer takes them in:

* base W  ~ N(0, 0.02^2), fp32, packed by the library's quant_pack;
* A       ~ N(0, 1/K), bf16;     B ~ N(0, 0.01^2), bf16;
* x, dY   ~ N(0, 1), bf16.

The shapes are those of the model layers the pages train (Qwen3-0.6B,
Llama-3.1-8B and Qwen3-8B decoder layers, all seven projections as LoRA
linears) plus a single 256x256 layer.  No checkpoint or dataset is used.
"""

from dataclasses import dataclass, field

import numpy as np

FMT_Q4_0, FMT_NF4, FMT_FP8, FMT_MXFP4, FMT_Q8_0, FMT_NVFP4 = 1, 2, 3, 4, 5, 6
TID_W, TID_A, TID_B, TID_X, TID_DY = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class Proj:
    name: str
    k: int   # in_features
    n: int   # out_features


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    fmt: int
    projs: tuple
    m: int
    r: int
    alpha: float
    notes: str = ""
    extra_m: tuple = field(default_factory=tuple)

    @property
    def scale(self):
        return self.alpha / self.r


def _projs(rows):
    return tuple(Proj(*t) for t in rows)


QWEN3_06B = _projs([("q", 1024, 2048), ("k", 1024, 1024), ("v", 1024, 1024),
                    ("o", 2048, 1024), ("gate", 1024, 3072), ("up", 1024, 3072),
                    ("down", 3072, 1024)])
LLAMA31_8B = _projs([("q", 4096, 4096), ("k", 4096, 1024), ("v", 4096, 1024),
                     ("o", 4096, 4096), ("gate", 4096, 14336), ("up", 4096, 14336),
                     ("down", 14336, 4096)])
QWEN3_8B = _projs([("q", 4096, 4096), ("k", 4096, 1024), ("v", 4096, 1024),
                   ("o", 4096, 4096), ("gate", 4096, 12288), ("up", 4096, 12288),
                   ("down", 12288, 4096)])

WORKLOADS = {
    "single256_q40": Workload(0, "single256_q40", FMT_Q4_0, _projs([("lin", 256, 256)]),
                              64, 8, 16.0, "one 256->256 LoRA linear, Q4_0-style base"),
    "qwen3_0.6b_nf4": Workload(1, "qwen3_0.6b_nf4", FMT_NF4, QWEN3_06B, 8192, 16, 32.0,
                               "Qwen3-0.6B decoder layer, NF4 base, 4x2048 tokens"),
    "llama3.1_8b_nf4": Workload(2, "llama3.1_8b_nf4", FMT_NF4, LLAMA31_8B, 4096, 16, 16.0,
                                "Llama-3.1-8B decoder layer, NF4 base", extra_m=(16, 64)),
    "qwen3_8b_fp8": Workload(3, "qwen3_8b_fp8", FMT_FP8, QWEN3_8B, 8192, 32, 64.0,
                             "Qwen3-8B decoder layer, FP8 E4M3 per-tensor base"),
    "llama3.1_8b_nf4_stack32": Workload(4, "llama3.1_8b_nf4_stack32", FMT_NF4, LLAMA31_8B,
                                        2048, 16, 16.0,
                                        "32 Llama-3.1-8B layers, base streamed from pinned host",
                                        extra_m=(16,)),
    "llama3.1_8b_mxfp4": Workload(5, "llama3.1_8b_mxfp4", FMT_MXFP4, LLAMA31_8B, 4096, 16, 16.0,
                                  "Llama-3.1-8B decoder layer, MXFP4 base (E2M1, E8M0 per 32)",
                                  extra_m=(16, 64)),
    "llama3.1_8b_q8_0": Workload(6, "llama3.1_8b_q8_0", FMT_Q8_0, LLAMA31_8B, 4096, 16, 16.0,
                                 "Llama-3.1-8B decoder layer, Q8_0-style base (int8, fp16 per 32)",
                                 extra_m=(16, 64)),
    "llama3.1_8b_nvfp4": Workload(7, "llama3.1_8b_nvfp4", FMT_NVFP4, LLAMA31_8B, 4096, 16, 16.0,
                                  "Llama-3.1-8B decoder layer, NVFP4 base (E2M1, E4M3 per 16, fp32 per tensor)",
                                  extra_m=(16, 64)),
}


def torch_seed(wid, layer, proj, tid):
    """Seed of one tensor's draw on the GPU (distinct per workload, layer,
    projection and tensor id)."""
    return 1 + int(tid) + 10 * (int(proj) + 100 * (int(layer) + 1000 * int(wid)))


def layer_tensors_torch(w: Workload, proj_idx: int, m: int = None, layer: int = 0, device="cuda",
                        want=("W", "A", "B", "x", "dY")):
    """The inputs of one projection drawn on the GPU with torch's seeded
    generator (same distributions as layer_tensors; fast at full model sizes):
    dict of torch tensors W fp32 [N, K], and bf16 A [r, K], B [N, r], x [m, K],
    dY [m, N] (fp32 draws rounded to bf16, nearest even).  The oracle gets the
    same values by copying these tensors to the host."""
    import torch

    p = w.projs[proj_idx]
    m = w.m if m is None else m

    def draw(tid, shape, std):
        g = torch.Generator(device=device)
        g.manual_seed(torch_seed(w.wid, layer, proj_idx, tid))
        return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * float(std)

    spec = {"W": (TID_W, (p.n, p.k), 0.02, False), "A": (TID_A, (w.r, p.k), np.sqrt(1.0 / p.k), True),
            "B": (TID_B, (p.n, w.r), 0.01, True), "x": (TID_X, (m, p.k), 1.0, True),
            "dY": (TID_DY, (m, p.n), 1.0, True)}
    out = {}
    for name in want:
        tid, shape, std, bf16 = spec[name]
        t = draw(tid, shape, std)
        out[name] = t.to(torch.bfloat16) if bf16 else t
    return out


def rng(wid, layer, proj, tid):
    return np.random.default_rng([int(wid), int(layer), int(proj), int(tid)])


def normal_f32(wid, layer, proj, tid, shape, std):
    g = rng(wid, layer, proj, tid)
    return (g.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def to_bf16_bits(a_f32):
    """fp32 -> bf16 bit patterns (uint16), nearest even, via torch's cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def layer_tensors(w: Workload, proj_idx: int, m: int = None, layer: int = 0):
    """All inputs of one projection: dict with W (fp32), and bf16 bit arrays A, B, x, dY."""
    p = w.projs[proj_idx]
    m = w.m if m is None else m
    out = {"W": normal_f32(w.wid, layer, proj_idx, TID_W, (p.n, p.k), 0.02)}
    out["A"] = to_bf16_bits(normal_f32(w.wid, layer, proj_idx, TID_A, (w.r, p.k), np.sqrt(1.0 / p.k)))
    out["B"] = to_bf16_bits(normal_f32(w.wid, layer, proj_idx, TID_B, (p.n, w.r), 0.01))
    out["x"] = to_bf16_bits(normal_f32(w.wid, layer, proj_idx, TID_X, (m, p.k), 1.0))
    out["dY"] = to_bf16_bits(normal_f32(w.wid, layer, proj_idx, TID_DY, (m, p.n), 1.0))
    return out
