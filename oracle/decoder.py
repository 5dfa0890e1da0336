"""A whole decoder layer and a small whole-model training step, in plain fp64 numpy.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

The Llama-3.1-8B and Qwen2.5 workloads are decoder layers made of RMSNorm, grouped-query
attention with 32 query and 8 KV heads of dim 128 (or 14 / 2 of dim 64), a SwiGLU MLP and
residual connections (the Soup deep dive, "Core feature: how layer streaming works", names
the per-layer checkpoint recompute).  The pages give no
formulas for them; the readings are the standard Llama definitions:

  RMSNorm   y = x / sqrt(mean(x^2) + eps) * g                         (g frozen)
  RoPE      rotate-half pairs (i, i + D/2) by pos * base^(-2i/D), pos = t mod seq_len
  attention per sequence of seq_len tokens, causal, softmax(q k^T / sqrt(D)) v;
            q head h reads kv head h // (n_heads / n_kv)
  SwiGLU    s = silu(g) * u,  silu(z) = z / (1 + e^-z)
  layer     a = norm1(x); q,k,v = a W^T (+ LoRA); q,k = rope; o = attn;
            h = x + o W_o^T (+ LoRA); m = norm2(h); g,u = m W^T; s = swiglu;
            out = h + s W_down^T (+ LoRA)
  model     x0 = embed[ids]; layers; logits = norm_f(x_L) W_lm^T; mean token CE

Backward is written out by hand from these definitions (the chain rule, no autodiff).

``rnd=True`` rounds every tensor the GPU path stores in bf16 at the point where it is
stored (each call's output is bf16 by definition of the call), so that the comparison
with the GPU isolates accumulation-order differences; ``rnd=False`` keeps everything
fp64 for the finite-difference pins.
"""
from __future__ import annotations

import contextlib

import numpy as np

from . import head as ohead
from . import lora
from . import nf4


_JITTER = None  # (rng, rel) while storage_jitter is active


@contextlib.contextmanager
def storage_jitter(rng, rel: float):
    """Inside this block every value is perturbed by a relative N(0, rel) error before its
    bf16 storage.  With rel the size of an fp32 accumulation error (~1e-6) this measures
    the model's own sensitivity: how far two exact-up-to-fp32 computations drift apart
    once bf16 roundings flip and the flips propagate (tolerances of whole-model checks)."""
    global _JITTER
    old, _JITTER = _JITTER, (rng, float(rel))
    try:
        yield
    finally:
        _JITTER = old


def q16(a, rnd: bool = True):
    """bf16 storage of a tensor (fp64 -> fp32 -> bf16 RNE), or the identity."""
    a = np.asarray(a, dtype=np.float64)
    if not rnd:
        return a
    if _JITTER is not None:
        rng, rel = _JITTER
        a = a * (1.0 + rel * rng.standard_normal(a.shape))
    return nf4.bf16_bits_to_f64(nf4.bf16_rne_bits(a))


# ------------------------------------------------------------------ RMSNorm
def rmsnorm(x, g, eps):
    x = np.asarray(x, np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps)
    return x * r * g[None, :], r[:, 0]


def rmsnorm_bwd(x, g, r, dy):
    """d/dx of y = x r g with r = (mean(x^2) + eps)^-1/2: r g dy - x r^3 mean(x g dy)."""
    x = np.asarray(x, np.float64)
    gdy = g[None, :] * dy
    return r[:, None] * gdy - x * (r ** 3)[:, None] * np.mean(x * gdy, axis=1, keepdims=True)


# ------------------------------------------------------------------ RoPE
def rope_angles(T, seq_len, D, base):
    pos = (np.arange(T) % seq_len).astype(np.float64)
    inv = base ** (-np.arange(0, D // 2, dtype=np.float64) * 2.0 / D)
    ang = pos[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


def rope(x, cos, sin, n_heads, D, inverse=False):
    """Rotate-half RoPE on [T, n_heads*D]; inverse=True rotates by -angle (the backward)."""
    T = x.shape[0]
    xh = np.asarray(x, np.float64).reshape(T, n_heads, D)
    a, b = xh[:, :, : D // 2], xh[:, :, D // 2:]
    c, s = cos[:, None, :], (-sin if inverse else sin)[:, None, :]
    out = np.concatenate([a * c - b * s, b * c + a * s], axis=2)
    return out.reshape(T, n_heads * D)


# ------------------------------------------------------------------ attention
def _heads(x, n, D):
    T = x.shape[0]
    return np.asarray(x, np.float64).reshape(T, n, D).transpose(1, 0, 2)  # [n, T, D]


def attention(q, k, v, n_heads, n_kv, D, seq_len):
    """Causal GQA attention per sequence.  Returns o [T, n_heads*D] and lse [n_heads, T]
    (natural-log log-sum-exp of each query's scaled scores)."""
    T = q.shape[0]
    Q, K, V = _heads(q, n_heads, D), _heads(k, n_kv, D), _heads(v, n_kv, D)
    rep = n_heads // n_kv
    O = np.zeros((n_heads, T, D))
    lse = np.zeros((n_heads, T))
    mask = np.tril(np.ones((seq_len, seq_len), dtype=bool))
    for h in range(n_heads):
        kv = h // rep
        for s0 in range(0, T, seq_len):
            sl = slice(s0, s0 + seq_len)
            S = Q[h, sl] @ K[kv, sl].T / np.sqrt(D)
            S = np.where(mask, S, -np.inf)
            m = S.max(axis=1, keepdims=True)
            e = np.exp(S - m)
            z = e.sum(axis=1, keepdims=True)
            O[h, sl] = (e / z) @ V[kv, sl]
            lse[h, sl] = (m + np.log(z))[:, 0]
    return O.transpose(1, 0, 2).reshape(T, n_heads * D), lse


def attention_bwd(q, k, v, o, lse, do, n_heads, n_kv, D, seq_len):
    """dq, dk, dv of the attention above: P = exp(S - lse), dV = P^T dO, dP = dO V^T,
    dS = P (dP - rowsum(dO o O)), dQ = dS K / sqrt(D), dK = dS^T Q / sqrt(D); a kv
    head's gradients sum over the query heads that read it."""
    T = q.shape[0]
    Q, K, V = _heads(q, n_heads, D), _heads(k, n_kv, D), _heads(v, n_kv, D)
    O, dO = _heads(o, n_heads, D), _heads(do, n_heads, D)
    rep = n_heads // n_kv
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    mask = np.tril(np.ones((seq_len, seq_len), dtype=bool))
    sc = 1.0 / np.sqrt(D)
    for h in range(n_heads):
        kv = h // rep
        for s0 in range(0, T, seq_len):
            sl = slice(s0, s0 + seq_len)
            S = Q[h, sl] @ K[kv, sl].T * sc
            P = np.where(mask, np.exp(S - lse[h, sl][:, None]), 0.0)
            dV[kv, sl] += P.T @ dO[h, sl]
            dP = dO[h, sl] @ V[kv, sl].T
            Dl = np.sum(dO[h, sl] * O[h, sl], axis=1, keepdims=True)
            dS = P * (dP - Dl)
            dQ[h, sl] = dS @ K[kv, sl] * sc
            dK[kv, sl] += dS.T @ Q[h, sl] * sc
    back = lambda X, n: X.transpose(1, 0, 2).reshape(T, n * D)
    return back(dQ, n_heads), back(dK, n_kv), back(dV, n_kv)


# ------------------------------------------------------------------ SwiGLU
def silu(z):
    return z / (1.0 + np.exp(-z))


def swiglu(g, u):
    return silu(g) * u


def swiglu_bwd(g, u, ds):
    sig = 1.0 / (1.0 + np.exp(-g))
    return ds * u * sig * (1.0 + g * (1.0 - sig)), ds * g * sig   # (dg, du)


# ------------------------------------------------------------------ layer and model
def _lin(x, W, ad):
    if ad is None:
        return lora.linear_fwd(x, W)[0]
    A, B, s = ad
    return lora.linear_fwd(x, W, A, B, s)[0]


def _lin_bwd(x, dy, W, ad):
    if ad is None:
        return lora.linear_bwd(x, dy, W)[0], None
    A, B, s = ad
    dx, dA, dB = lora.linear_bwd(x, dy, W, A, B, s)
    return dx, (dA, dB)


def layer_fwd(P, cfg, x, rnd=True):
    """P: {"W": {proj: [out, in]}, "ad": {proj: (A, B, s)}, "g1": [H], "g2": [H]}."""
    nh, nkv, D, S = cfg["n_heads"], cfg["n_kv"], cfg["head_dim"], cfg["seq_len"]
    W, ad = P["W"], P["ad"]
    c = {"x": x}
    a, c["r1"] = rmsnorm(x, P["g1"], cfg["eps"])
    c["a"] = a = q16(a, rnd)
    qp = q16(_lin(a, W["q"], ad.get("q")), rnd)
    kp = q16(_lin(a, W["k"], ad.get("k")), rnd)
    c["v"] = v = q16(_lin(a, W["v"], ad.get("v")), rnd)
    cos, sin = rope_angles(x.shape[0], S, D, cfg["rope_base"])
    c["cos"], c["sin"] = cos, sin
    c["q"] = q = q16(rope(qp, cos, sin, nh, D), rnd)
    c["k"] = k = q16(rope(kp, cos, sin, nkv, D), rnd)
    o, c["lse"] = attention(q, k, v, nh, nkv, D, S)
    c["o"] = o = q16(o, rnd)
    po = q16(_lin(o, W["o"], ad.get("o")), rnd)
    c["h"] = h = q16(x + po, rnd)
    m, c["r2"] = rmsnorm(h, P["g2"], cfg["eps"])
    c["m"] = m = q16(m, rnd)
    c["g"] = g = q16(_lin(m, W["gate"], ad.get("gate")), rnd)
    c["u"] = u = q16(_lin(m, W["up"], ad.get("up")), rnd)
    c["s"] = s = q16(swiglu(g, u), rnd)
    dn = q16(_lin(s, W["down"], ad.get("down")), rnd)
    return q16(h + dn, rnd), c


def layer_bwd(P, cfg, c, dout, rnd=True):
    """Returns dx and {proj: (dA, dB)} for the adapted projections."""
    nh, nkv, D, S = cfg["n_heads"], cfg["n_kv"], cfg["head_dim"], cfg["seq_len"]
    W, ad = P["W"], P["ad"]
    grads = {}
    ds, grads["down"] = _lin_bwd(c["s"], dout, W["down"], ad.get("down"))
    ds = q16(ds, rnd)
    dg, du = swiglu_bwd(c["g"], c["u"], ds)
    dg, du = q16(dg, rnd), q16(du, rnd)
    dm_g, grads["gate"] = _lin_bwd(c["m"], dg, W["gate"], ad.get("gate"))
    dm_u, grads["up"] = _lin_bwd(c["m"], du, W["up"], ad.get("up"))
    dm = q16(dm_g + dm_u, rnd)
    dh = q16(dout + rmsnorm_bwd(c["h"], P["g2"], c["r2"], dm), rnd)
    do, grads["o"] = _lin_bwd(c["o"], dh, W["o"], ad.get("o"))
    do = q16(do, rnd)
    dq, dk, dv = attention_bwd(c["q"], c["k"], c["v"], c["o"], c["lse"], do, nh, nkv, D, S)
    dq, dk, dv = q16(dq, rnd), q16(dk, rnd), q16(dv, rnd)
    dq = q16(rope(dq, c["cos"], c["sin"], nh, D, inverse=True), rnd)
    dk = q16(rope(dk, c["cos"], c["sin"], nkv, D, inverse=True), rnd)
    da_q, grads["q"] = _lin_bwd(c["a"], dq, W["q"], ad.get("q"))
    da_k, grads["k"] = _lin_bwd(c["a"], dk, W["k"], ad.get("k"))
    da_v, grads["v"] = _lin_bwd(c["a"], dv, W["v"], ad.get("v"))
    da = q16(da_q + da_k + da_v, rnd)
    dx = q16(dh + rmsnorm_bwd(c["x"], P["g1"], c["r1"], da), rnd)
    return dx, {k_: v_ for k_, v_ in grads.items() if v_ is not None}


def model_step(M, cfg, ids, labels, rnd=True):
    """One SFT step of the whole model: returns loss (mean over tokens), per-token
    log-probs, the per-layer adapter gradients, and the embedding-output gradient dx0.
    M: {"embed": [V, H], "layers": [P], "g_final": [H], "lm_head": [V, H]}."""
    x = M["embed"][np.asarray(ids)]
    caches = []
    for P in M["layers"]:
        x, c = layer_fwd(P, cfg, x, rnd)
        caches.append(c)
    hN, rf = rmsnorm(x, M["g_final"], cfg["eps"])
    hN = q16(hN, rnd)
    logits = q16(lora.linear_fwd(hN, M["lm_head"])[0], rnd)
    logp, loss, dlogits = ohead.cross_entropy(logits, labels)
    dlogits = q16(dlogits, rnd)
    dhN = q16(lora.linear_bwd(hN, dlogits, M["lm_head"])[0], rnd)
    dx = q16(rmsnorm_bwd(x, M["g_final"], rf, dhN), rnd)
    grads = [None] * len(M["layers"])
    for li in range(len(M["layers"]) - 1, -1, -1):
        dx, grads[li] = layer_bwd(M["layers"][li], cfg, caches[li], dx, rnd)
    return {"loss": float(np.mean(loss)), "logp": logp, "grads": grads, "dx0": dx, "logits": logits,
            "x_last": x, "dhN": dhN}
