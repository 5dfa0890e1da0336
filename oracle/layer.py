"""One decoder layer's seven frozen projections composed into a layer step.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

The Soup deep dive ("How layer streaming works") describes a step as: each
layer read for the forward, then read again in backward, where its forward is
recomputed from the checkpointed input and the input gradient is formed.  Only
the linear projections are on this path; attention, norms and activations
between them are not, so each projection group gets its own input.

Reading (the pages do not list the projections): the seven projections of a
Llama/Qwen decoder layer in the order q, k, v, o, gate, up, down.  q, k and v
read the same input (the attention input), gate and up read the same input
(the MLP input), o and down read their own.  In backward the input gradient of
a group is the sum over its projections.  The forward runs the groups in order
qkv, o, gate-up, down; backward runs them in reverse.  For a DPO step an
adapter-off forward of all groups comes first (the same streamed base with the
adapters off gives the reference pass: the 4 GB-laptop article, "Memory-free
reference model").
"""
from __future__ import annotations

from . import lora

PROJ_ORDER = ("q", "k", "v", "o", "gate", "up", "down")
GROUPS = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))


def group_fwd(names, weights, adapters, x, adapters_enabled=True):
    """Forward of one group sharing input x; returns {name: (y, u)}."""
    out = {}
    for n in names:
        ad = adapters.get(n) if adapters_enabled else None
        if ad is None:
            out[n] = lora.linear_fwd(x, weights[n])
        else:
            A, B, s = ad
            out[n] = lora.linear_fwd(x, weights[n], A, B, s)
    return out


def group_bwd(names, weights, adapters, x, dys):
    """Backward of one group: dx summed over the group, and per-projection (dA, dB)."""
    dx = None
    grads = {}
    for n in names:
        ad = adapters.get(n)
        if ad is None:
            d, dA, dB = lora.linear_bwd(x, dys[n], weights[n])
        else:
            A, B, s = ad
            d, dA, dB = lora.linear_bwd(x, dys[n], weights[n], A, B, s)
        dx = d if dx is None else dx + d
        grads[n] = (dA, dB)
    return dx, grads


def layer_step(weights, adapters, xs, dys, dpo=False):
    """One layer-step: [adapter-off fwd,] fwd, recompute, bwd in reverse group order.

    weights: {name: W' [out, in] fp64}; adapters: {name: (A, B, s)} for adapted
    projections; xs: {group index: x}; dys: {name: dy}.
    Returns dict with 'ref' (adapter-off outputs or None), 'fwd', 'recompute'
    ({name: y}), 'dx' ({group index: dx}) and 'grads' ({name: (dA, dB)}).
    """
    res = {"ref": None}
    if dpo:
        res["ref"] = {}
        for gi, g in enumerate(GROUPS):
            for n, (y, _) in group_fwd(g, weights, adapters, xs[gi], adapters_enabled=False).items():
                res["ref"][n] = y
    for key in ("fwd", "recompute"):
        res[key] = {}
        for gi, g in enumerate(GROUPS):
            for n, (y, _) in group_fwd(g, weights, adapters, xs[gi]).items():
                res[key][n] = y
    res["dx"], res["grads"] = {}, {}
    for gi in reversed(range(len(GROUPS))):
        dx, grads = group_bwd(GROUPS[gi], weights, adapters, xs[gi], dys)
        res["dx"][gi] = dx
        res["grads"].update(grads)
    return res
