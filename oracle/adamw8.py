"""AdamW with 8-bit block-wise quantized moments (oracle only: test
infrastructure, imported by tests/ and bench.py's CPU baseline alone).

The Surogate README page lists "AdamW 8-bit" among its optimizers
("Optimizers & monitoring" row) and the GGUF-recipe page ("How it works")
trains its adapters with an 8-bit AdamW; neither defines the state format.
The definition taken is the published one: Dettmers, Lewis, Shleifer and
Zettlemoyer, "8-bit Optimizers via Block-wise Quantization" (ICLR 2022):

* Block-wise quantization (their Section 2.1): each state tensor is cut into
  blocks of 2048 consecutive elements; a block stores one fp32 scale, its
  largest magnitude a, and per element an 8-bit code c standing for the value
  level[c] * a, with level[c] in [-1, 1].
* Dynamic tree quantization (their Section 2.2): a code's magnitude bits, read
  from the most significant, are a run of z zero bits, a one bit that ends
  the run, and f remaining bits holding an integer q; the run length sets a
  decimal exponent and q a linear fraction: value 10^-z * fraction.  The
  paper leaves the placement of the 2^f fraction levels open; the reading
  taken here puts them evenly in (0.1, 1] with the top one at 1:
      fraction = 0.1 + 0.9 * (q + 1) / 2^f,
  so the largest code is exactly 1 (the block's largest element is stored
  exactly) and levels of neighbouring exponents never coincide.  All-zero
  magnitude bits stand for 0.  Read as an unsigned integer the magnitude
  bits order the values, so the code of a value is its rank.
  - first moment (signed): bit 7 is the sign, 7 magnitude bits, z in 0..6,
    magnitudes 10^-6 .. 1;
  - second moment (never negative): all 8 bits are magnitude, z in 0..7,
    10^-7 .. 1.
  Each level is computed in fp64 as (0.1 + 0.9 (q + 1) / 2^f) / 10^z and
  rounded once to fp32.
* Quantizing: r = fl32(x / a) (IEEE divide); the magnitude code is the number
  of decision thresholds t_i = fl32(fl32(level_i + level_{i+1}) * 0.5) that
  |r| exceeds (a value equal to a threshold takes the lower code); the sign
  bit is set for negative values with a non-zero magnitude code.  A block
  whose largest magnitude is 0 stores a = 0 and codes 0.
* The step (their Section 2: dequantize, update in 32 bits, quantize): the
  moments are dequantized, the AdamW update of oracle/adamw.py runs in fp32 on
  them (the parameter moves with the updated fp32 moments), then each moment
  is quantized again with its block's new largest magnitude.

Every operation is fp32 with one rounding each, in the order written in
adamw8_step (no fused multiply-add): the quantization decisions are integer
results decided by floating point, so the oracle takes them in the precision
the GPU kernel takes them in.  The per-step constants (1 - lr wd, 1 - beta,
lr / (1 - beta1^t), 1 / sqrt(1 - beta2^t)) are formed in fp64 and rounded to
fp32 once.
"""

import math

import numpy as np

from . import codecs

BLOCK = 2048
F32 = np.float32


def dynamic_levels(signed):
    """The 2^b non-negative levels of the dynamic tree type (b = 7 magnitude
    bits when signed, 8 when not), indexed by the magnitude bits: fp32."""
    b = 7 if signed else 8
    out = np.zeros(1 << b, dtype=np.float64)
    for code in range(1, 1 << b):
        z = b - code.bit_length()            # leading zero bits of the magnitude
        f = b - 1 - z                        # fraction bits after the indicator
        q = code & ((1 << f) - 1)
        out[code] = (0.1 + 0.9 * (q + 1) / float(1 << f)) / (10.0 ** z)
    return out.astype(F32)


def thresholds(levels):
    """Decision thresholds between consecutive levels: fl32(fl32(l_i + l_i+1) * 0.5)."""
    lv = np.asarray(levels, dtype=F32)
    return ((lv[:-1] + lv[1:]).astype(F32) * F32(0.5)).astype(F32)


def _blocks(n):
    return (n + BLOCK - 1) // BLOCK


def quantize(x, signed):
    """fp32 array -> (codes u8 [n], absmax fp32 [ceil(n / BLOCK)])."""
    x = np.asarray(x, dtype=F32).ravel()
    n = x.size
    lv = dynamic_levels(signed)
    th = thresholds(lv)
    codes = np.zeros(n, dtype=np.uint8)
    absmax = np.zeros(_blocks(n), dtype=F32)
    for bi in range(_blocks(n)):
        blk = x[bi * BLOCK:(bi + 1) * BLOCK]
        a = F32(np.max(np.abs(blk))) if blk.size else F32(0)
        absmax[bi] = a
        if a == 0:
            continue
        r = (blk / a).astype(F32)
        k = np.searchsorted(th, np.abs(r), side="left").astype(np.uint32)   # thresholds strictly below |r|
        if signed:
            k = np.where((r < 0) & (k > 0), k | 0x80, k)
        codes[bi * BLOCK:(bi + 1) * BLOCK] = k.astype(np.uint8)
    return codes, absmax


def dequantize(codes, absmax, signed):
    """(codes, absmax) -> fp32 values level[c] * a."""
    codes = np.asarray(codes, dtype=np.uint8).ravel()
    lv = dynamic_levels(signed)
    a = np.repeat(np.asarray(absmax, dtype=F32), BLOCK)[:codes.size]
    if signed:
        mag = lv[codes & 0x7F]
        val = np.where(codes & 0x80, -mag, mag).astype(F32)
    else:
        val = lv[codes]
    return (val * a).astype(F32)


def step_constants(step, lr, beta1, beta2, eps, weight_decay, grad_scale):
    """The fp32 constants of step t, each formed in fp64 and rounded once."""
    t = float(int(step))
    return {"decay": F32(1.0 - lr * weight_decay), "b1": F32(beta1), "omb1": F32(1.0 - beta1),
            "b2": F32(beta2), "omb2": F32(1.0 - beta2), "step_size": F32(lr / (1.0 - beta1 ** t)),
            "inv_bc2_sqrt": F32(1.0 / math.sqrt(1.0 - beta2 ** t)), "eps": F32(eps), "gs": F32(grad_scale)}


def adamw8_step(param, grad, m_codes, m_absmax, v_codes, v_absmax, step, lr, beta1=0.9, beta2=0.999,
                eps=1e-8, weight_decay=0.0, grad_scale=1.0):
    """One AdamW step with 8-bit block-wise moments.  Returns (param fp32,
    m_codes, m_absmax, v_codes, v_absmax, m fp32, v fp32): the new parameter,
    the new quantized state, and the fp32 moments before quantization."""
    if int(step) < 1:
        raise ValueError("step must be >= 1")
    c = step_constants(step, lr, beta1, beta2, eps, weight_decay, grad_scale)
    p = np.asarray(param, dtype=F32).ravel()
    g = (np.asarray(grad, dtype=F32).ravel() * c["gs"]).astype(F32)
    m = dequantize(m_codes, m_absmax, True)
    v = dequantize(v_codes, v_absmax, False)
    th = (p * c["decay"]).astype(F32)
    m = ((c["b1"] * m).astype(F32) + (c["omb1"] * g).astype(F32)).astype(F32)
    v = ((c["b2"] * v).astype(F32) + (c["omb2"] * (g * g).astype(F32)).astype(F32)).astype(F32)
    denom = ((np.sqrt(v).astype(F32) * c["inv_bc2_sqrt"]).astype(F32) + c["eps"]).astype(F32)
    th = (th - (c["step_size"] * (m / denom).astype(F32)).astype(F32)).astype(F32)
    mc, ma = quantize(m, True)
    vc, va = quantize(v, False)
    return th, mc, ma, vc, va, m, v


def bf16_copy(param_f32):
    """bf16 bit patterns of the fp32 parameters (nearest even)."""
    return codecs.bf16_encode(np.asarray(param_f32, dtype=F32))
