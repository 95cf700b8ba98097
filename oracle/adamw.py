"""AdamW step on the LoRA adapters (oracle only).

The Surogate README page lists "AdamW 8-bit" among its optimizers and the
GGUF-recipe page ("How it works") trains its adapters with bitsandbytes'
8-bit AdamW; neither page defines the update.  The definition taken is
decoupled weight decay as in Loshchilov & Hutter, "Decoupled Weight Decay
Regularization" (Algorithm 2, Adam with decoupled weight decay), with the
convention PyTorch's and bitsandbytes' AdamW implementations share: the
decay is multiplied by the learning rate (schedule multiplier 1, alpha = lr)
and applied to the parameter before the Adam term.  One step t >= 1, for
every element, given the gradient g (times a gradient scale, e.g. 1 / the
number of accumulated micro-batches):

    theta <- theta * (1 - lr * lambda)
    m     <- beta1 * m + (1 - beta1) * g
    v     <- beta2 * v + (1 - beta2) * g^2
    m_hat  = m / (1 - beta1^t)
    v_hat  = v / (1 - beta2^t)
    theta <- theta - lr * m_hat / (sqrt(v_hat) + eps)

The moments are kept in full precision here (the 8-bit state quantization of
the pages' optimizer is a storage format the pages do not define).  The
adapters the layer reads are bf16: the step also returns bf16_RNE(theta),
the copy the next forward takes.

Arithmetic in fp64 by default, written in the order above.
"""

import numpy as np

from . import codecs


def adamw_step(param, grad, exp_avg, exp_avg_sq, step, lr, beta1=0.9, beta2=0.999, eps=1e-8,
               weight_decay=0.0, grad_scale=1.0, dtype=np.float64):
    """One AdamW step.  Returns (param, exp_avg, exp_avg_sq) as new arrays of
    ``dtype``; the inputs are not modified.  ``step`` is the 1-based step
    number t after this update."""
    if int(step) < 1:
        raise ValueError("step must be >= 1")
    t = int(step)
    theta = np.asarray(param).astype(dtype)
    g = np.asarray(grad).astype(dtype) * dtype(grad_scale)
    m = np.asarray(exp_avg).astype(dtype)
    v = np.asarray(exp_avg_sq).astype(dtype)
    lr, b1, b2 = dtype(lr), dtype(beta1), dtype(beta2)
    theta = theta * (dtype(1) - lr * dtype(weight_decay))
    m = b1 * m + (dtype(1) - b1) * g
    v = b2 * v + (dtype(1) - b2) * g * g
    m_hat = m / (dtype(1) - b1 ** t)
    v_hat = v / (dtype(1) - b2 ** t)
    theta = theta - lr * m_hat / (np.sqrt(v_hat) + dtype(eps))
    return theta, m, v


def bf16_copy(param_f32):
    """bf16 bit patterns of fp32 parameters (nearest even): the adapter copy
    the layer's kernels read."""
    return codecs.bf16_encode(np.asarray(param_f32, dtype=np.float32))
