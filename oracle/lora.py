"""Forward and backward of the LoRA linear layer over a frozen base (oracle only).

Shapes (row-major, nn.Linear convention): W [N, K] (already dequantized, fp32),
x [M, K], A [r, K], B [N, r], y and dY [M, N], U = x.A^T [M, r],
V = dY.B [M, r], s = alpha / r (the LoRA scaling; alpha / r, not alpha /
sqrt(r)).

Forward   y  = x.W^T + s.(x.A^T).B^T                         (U is saved)
Backward  dX = dY.W + s.(dY.B).A
          dA = s.(dY.B)^T.x          = s.V^T.x
          dB = s.dY^T.(x.A^T)        = s.dY^T.U
The base W is frozen: it gets no gradient and is never written.

The Soup page states the frozen base is read and never written; the GGUF
recipe page's "fast backward formulas" for LoRA are read here as reusing the
rank-r intermediates U and V instead of forming B.A.

Inputs are exact fp32 values (bf16 activations and adapters decode exactly)
or fp64 values (finite-difference checks); products are evaluated in ``dtype`` (fp64 by default) with plain
library matmuls, in the order the formulas are written.
"""

import numpy as np

from . import codecs


def _f(a, dtype):
    a = np.asarray(a)
    if a.dtype not in (np.float32, np.float64):
        a = a.astype(np.float32)
    return a.astype(dtype)


def lora_scale(alpha, r):
    return float(alpha) / float(r)


def forward(x, w, a, b, alpha, dtype=np.float64):
    """Returns (y, U): y = x.W^T + s.U.B^T with U = x.A^T."""
    r = np.asarray(a).shape[0]
    s = lora_scale(alpha, r)
    xf, wf, af, bf = (_f(t, dtype) for t in (x, w, a, b))
    u = xf @ af.T
    base = xf @ wf.T
    y = base + s * (u @ bf.T)
    return y, u


def forward_base(x, w, dtype=np.float64):
    """Base term only: x.W^T."""
    return _f(x, dtype) @ _f(w, dtype).T


def forward_merged(x, w, a, b, alpha, dtype=np.float64):
    """Textbook re-parametrisation: y = x.(W + s.B.A)^T (same value, other route)."""
    r = np.asarray(a).shape[0]
    s = lora_scale(alpha, r)
    wf, af, bf = (_f(t, dtype) for t in (w, a, b))
    return _f(x, dtype) @ (wf + s * (bf @ af)).T


def adapter_grads(x, dy, a, b, alpha, dtype=np.float64):
    """(dA, dB): dA = s.(dY.B)^T.x and dB = s.dY^T.(x.A^T); W does not enter."""
    r = np.asarray(a).shape[0]
    s = lora_scale(alpha, r)
    xf, dyf, af, bf = (_f(t, dtype) for t in (x, dy, a, b))
    u = xf @ af.T
    v = dyf @ bf
    return s * (v.T @ xf), s * (dyf.T @ u)


def backward(x, dy, w, a, b, alpha, dtype=np.float64):
    """Returns (dX, dA, dB) for upstream gradient dY."""
    r = np.asarray(a).shape[0]
    s = lora_scale(alpha, r)
    dyf, wf, af, bf = (_f(t, dtype) for t in (dy, w, a, b))
    v = dyf @ bf
    dx = dyf @ wf + s * (v @ af)
    da, db = adapter_grads(x, dy, a, b, alpha, dtype)
    return dx, da, db


def rel_err(got, ref):
    """max|got - ref| / max|ref|; when ref is all zero, 0 if got is too, else inf."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(got - ref)) if ref.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


# ----------------------------------------------------------------------------- FP8 activations

LO_SHIFT = 16.0   # the low term is stored 16x finer than the high term


def act_row_exponent(amax):
    """Smallest integer e with 448 * 2^e >= amax (amax > 0), by exact
    comparisons (448 * 2^e is exact in fp64 over the whole fp32 range)."""
    a = float(amax)
    e = int(np.floor(np.log2(a))) - 8
    while 448.0 * 2.0 ** e < a:
        e += 1
    while 448.0 * 2.0 ** (e - 1) >= a:
        e -= 1
    return e


def act_split_e4m3(x):
    """Per-token two-term E4M3 split of activations for the FP8-base GEMM.

    For each row m with a = max|x_m| > 0 the scale is the power of two
    s_m = 2^e, e the smallest integer with 448 * 2^e >= a, so t = x / s_m is
    exact in fp32 and |t| <= 448; then hi = E4M3(t) and
    lo = E4M3(fl32(t - E4M3(hi)) * 16) (the difference and the factor 16 are
    exact too), so that x ~= s_m * (hi + lo / 16) with the two E4M3
    roundings as the only ones.  A zero row has s_m = 0 and zero codes.
    Returns (hi u8 [M, K], lo u8 [M, K], s fp32 [M]).

    The pages quantize activations for their FP8 recipe without saying how:
    the per-token scale, its power-of-two form (the form of the matrix cores'
    E8M0 block-scale operand) and the second term are this implementation's
    reading.  It is an approximation, checked by its error bound.
    """
    xf = np.asarray(x, dtype=np.float32)
    m = xf.shape[0]
    amax = np.max(np.abs(xf), axis=1) if xf.shape[1] else np.zeros(m, np.float32)
    s = np.zeros(m, np.float32)
    t = np.zeros_like(xf)
    for i in range(m):
        if amax[i] > 0:
            e = act_row_exponent(amax[i])
            s[i] = np.float32(np.ldexp(1.0, e))
            t[i] = np.ldexp(xf[i].astype(np.float64), -e).astype(np.float32)   # exact
    hi = codecs.e4m3_encode(t)
    res = (t - codecs.e4m3_decode(hi)).astype(np.float32)
    lo = codecs.e4m3_encode((res * np.float32(LO_SHIFT)).astype(np.float32))
    nz = amax > 0
    hi = np.where(nz[:, None], hi, np.uint8(0)).astype(np.uint8)
    lo = np.where(nz[:, None], lo, np.uint8(0)).astype(np.uint8)
    return hi, lo, s


def act_join_e4m3(hi, lo, s, dtype=np.float64):
    """Value represented by a two-term split: s_m * (hi + lo / 16)."""
    h = codecs.e4m3_decode(hi).astype(dtype)
    l_ = codecs.e4m3_decode(lo).astype(dtype)
    return np.asarray(s, dtype)[:, None] * (h + l_ / LO_SHIFT)
