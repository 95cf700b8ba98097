"""Stacked adapters over one frozen base (oracle only).

The Surogate review page lists stacked LoRA (adapters trained on top of
other adapters, with no offline merge) and the README page's "LoRA & QLoRA"
row names stacked LoRA adapters: frozen lower adapters under one trainable
top adapter.  Written from the plain definition, adapter i with factors A_i [r_i, K], B_i [N, r_i] and scale
s_i = alpha_i / r_i, the top one last:

    y  = x.W^T + sum_i s_i.(x.A_i^T).B_i^T
    dX = dY.W  + sum_i s_i.(dY.B_i).A_i
    dA_top = s_top.(dY.B_top)^T.x,   dB_top = s_top.dY^T.(x.A_top^T)

(no gradient for W or for the frozen adapters).  Products in fp64 by
default, in the order written.
"""

import numpy as np

from . import lora


def forward(x, w, adapters, dtype=np.float64):
    """adapters: list of (A, B, alpha), top last.  Returns y."""
    y = lora.forward_base(x, w, dtype)
    for a, b, alpha in adapters:
        s = lora.lora_scale(alpha, np.asarray(a).shape[0])
        xf, af, bf = (lora._f(t, dtype) for t in (x, a, b))
        y = y + s * ((xf @ af.T) @ bf.T)
    return y


def backward(x, dy, w, adapters, dtype=np.float64):
    """Returns (dX, dA_top, dB_top)."""
    dyf = lora._f(dy, dtype)
    dx = dyf @ lora._f(w, dtype)
    for a, b, alpha in adapters:
        s = lora.lora_scale(alpha, np.asarray(a).shape[0])
        af, bf = lora._f(a, dtype), lora._f(b, dtype)
        dx = dx + s * ((dyf @ bf) @ af)
    a, b, alpha = adapters[-1]
    da, db = lora.adapter_grads(x, dy, a, b, alpha, dtype)
    return dx, da, db
