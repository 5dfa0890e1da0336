"""LoRA linear on a frozen weight: forward and backward, as plain matrix definitions.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

What is computed.  The frozen base weight W' is [out, in] (a PyTorch Linear
weight; NF4-decoded, or bf16 as stored).  The adapters are A [r, in] and
B [out, r] with scale s, and are the only trainable tensors: low-rank matrices
inserted next to the frozen weights (the 20B-RLHF-on-24GB article, section
"Low-rank adaptation via PEFT"; the S-LoRA news article on LoRA's
freeze-and-learn-the-change idea).  Scale s = alpha / r from the adapter
config (``r=8, lora_alpha=32`` in the 20B-RLHF article's step 2); the caller
supplies s.

Forward       y  = x W'^T + s (x A^T) B^T,       u = x A^T      [T, r]
Backward      v  = dy B                                         [T, r]
              dx = dy W' + s v A  (the frozen weight must be on hand again in
                   backward because the input gradient is W^T applied to the
                   output gradient: the Soup deep dive, "How layer streaming
                   works")
              dA = s v^T x                                      [r, in]
              dB = s dy^T u                                     [out, r]
W' gets no gradient.  With the adapters disabled (A, B absent, or r = 0) the
module is the frozen base linear: y = x W'^T and dx = dy W' (the 20B-RLHF
article, step 3: the same model with the adapters switched off gives the
reference logits).

All inputs arrive as fp64 arrays holding exactly the bf16 values the GPU
reads; every product and sum is fp64 (numpy matmul as the primitive), and
nothing is rounded on the way out.
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def adapters_on(A, B, r: int | None = None) -> bool:
    if A is None or B is None:
        return False
    return (A.shape[0] if r is None else r) > 0


def linear_fwd(x, Wd, A=None, B=None, scale: float = 0.0):
    """Return (y, u): y = x W'^T + s (x A^T) B^T; u = x A^T, or None with adapters off."""
    x, Wd, A, B = _f64(x), _f64(Wd), _f64(A), _f64(B)
    y = x @ Wd.T
    if not adapters_on(A, B):
        return y, None
    u = x @ A.T
    return y + scale * (u @ B.T), u


def linear_bwd(x, dy, Wd, A=None, B=None, scale: float = 0.0):
    """Return (dx, dA, dB); dA and dB are None with adapters off."""
    x, dy, Wd, A, B = _f64(x), _f64(dy), _f64(Wd), _f64(A), _f64(B)
    dx = dy @ Wd
    if not adapters_on(A, B):
        return dx, None, None
    v = dy @ B
    u = x @ A.T
    dx = dx + scale * (v @ A)
    dA = scale * (v.T @ x)
    dB = scale * (dy.T @ u)
    return dx, dA, dB


def trainable_params(shapes, r: int) -> int:
    """Adapter parameter count r * (in + out) summed over adapted [out, in] projections."""
    return sum(r * (o + i) for (o, i) in shapes)
