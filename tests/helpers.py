"""Shared helpers for the GPU tests: seeded inputs on both sides, comparisons."""

import numpy as np
import torch

from oracle import formats as ofmt
from oracle import lora as olora
from quantized_base_lora_amd import synth

FWD_TOL = 1e-2
FP8_TOL = 3e-2


def bits_to_bf16_tensor(bits, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def bf16_tensor_bits(t):
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def make_case(m, k, n, r, seed, w_std=0.02, b_std=0.01):
    """Seeded inputs of one projection: fp32 W, bf16 bit arrays A, B, x, dY."""
    g = np.random.default_rng(seed)
    w = (g.standard_normal((n, k), dtype=np.float32) * np.float32(w_std)).astype(np.float32)
    a = synth.to_bf16_bits(g.standard_normal((r, k), dtype=np.float32) * np.float32(np.sqrt(1.0 / k)))
    b = synth.to_bf16_bits(g.standard_normal((n, r), dtype=np.float32) * np.float32(b_std))
    x = synth.to_bf16_bits(g.standard_normal((m, k), dtype=np.float32))
    dy = synth.to_bf16_bits(g.standard_normal((m, n), dtype=np.float32))
    return {"W": w, "A": a, "B": b, "x": x, "dY": dy}


def oracle_packed(fmt, w):
    c, s = ofmt.pack(fmt, w)
    return c, s, ofmt.dequant(fmt, c, s)


def scales_bytes(fmt, s):
    """Oracle scales as raw bytes in the library's layout."""
    if fmt in (ofmt.FMT_Q4_0, ofmt.FMT_Q8_0):
        return np.ascontiguousarray(s, dtype=np.uint16).view(np.uint8).ravel()
    if fmt == ofmt.FMT_NF4:
        return np.ascontiguousarray(s, dtype=np.float32).view(np.uint8).ravel()
    if fmt in (ofmt.FMT_MXFP4, ofmt.FMT_NVFP4):
        return np.ascontiguousarray(s, dtype=np.uint8).ravel()
    return np.array([s], dtype=np.float32).view(np.uint8)


def tensor_bytes(t):
    return t.detach().contiguous().view(torch.uint8).cpu().numpy().ravel()


def oracle_layer(case, wd, alpha, rows=None):
    """fp64 reference outputs (y, U, dX, dA, dB).  With rows, y / U / dX are
    computed for those rows only (each row depends on its own inputs alone);
    dA and dB always cover every row."""
    x = synth.bf16_bits_to_f32(case["x"])
    dy = synth.bf16_bits_to_f32(case["dY"])
    a = synth.bf16_bits_to_f32(case["A"])
    b = synth.bf16_bits_to_f32(case["B"])
    xs = x if rows is None else x[rows]
    dys = dy if rows is None else dy[rows]
    y, u = olora.forward(xs, wd, a, b, alpha)
    dx, _, _ = olora.backward(xs, dys, wd, a, b, alpha)
    da, db = olora.adapter_grads(x, dy, a, b, alpha)
    return {"y": y, "U": u, "dX": dx, "dA": da, "dB": db}


def rel(got, ref):
    return olora.rel_err(got, ref)


def f32_host(t):
    """A device tensor's values as a host fp32 array (bf16 widens exactly)."""
    return t.detach().float().cpu().numpy()


def oracle_outputs(x, dy, a, b, wd, alpha):
    """fp64 oracle outputs of one projection from device inputs (x, dY, A, B
    bf16 tensors) and the dequantized base wd (host fp32): y, U, dX, dA, dB."""
    xf, dyf, af, bf = (f32_host(t) for t in (x, dy, a, b))
    y, u = olora.forward(xf, wd, af, bf, alpha)
    dx, da, db = olora.backward(xf, dyf, wd, af, bf, alpha)
    return {"y": y, "U": u, "dX": dx, "dA": da, "dB": db}


def packed_equal(fmt, codes_bytes, scales_bytes_, c, s):
    """Library-packed bytes against the oracle's codes and scales."""
    return (np.array_equal(np.asarray(codes_bytes).ravel(), np.ascontiguousarray(c).ravel())
            and np.array_equal(np.asarray(scales_bytes_).ravel(), scales_bytes(fmt, s)))
