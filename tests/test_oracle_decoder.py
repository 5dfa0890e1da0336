"""Pins of the decoder-layer oracle (RMSNorm, RoPE, causal GQA attention, SwiGLU, the
layer and the whole-model step) against closed forms, invariants, a loop brute force
and central finite differences in fp64."""
import math

import numpy as np
import pytest

from oracle import decoder as od

RS = np.random.default_rng(123)


def fd(f, x, h=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        a, b = x.copy(), x.copy()
        a[i] += h
        b[i] -= h
        g[i] = (f(a) - f(b)) / (2 * h)
    return g


# ------------------------------------------------------------------ RMSNorm
def test_rmsnorm_unit_rms_and_scale_invariance():
    x = RS.normal(size=(5, 16)) * 3
    y, r = od.rmsnorm(x, np.ones(16), 0.0)
    assert np.allclose(np.mean(y * y, axis=1), 1.0, atol=1e-14)
    y2, _ = od.rmsnorm(7.5 * x, np.ones(16), 0.0)
    assert np.allclose(y, y2, atol=1e-14)
    assert np.allclose(r, 1 / np.sqrt(np.mean(x * x, axis=1)))


def test_rmsnorm_backward_finite_differences():
    x = RS.normal(size=(3, 8))
    g = RS.normal(size=8)
    dy = RS.normal(size=(3, 8))
    _, r = od.rmsnorm(x, g, 1e-5)
    num = fd(lambda z: np.sum(od.rmsnorm(z, g, 1e-5)[0] * dy), x)
    assert np.allclose(od.rmsnorm_bwd(x, g, r, dy), num, atol=1e-8)


# ------------------------------------------------------------------ RoPE
def test_rope_two_dim_rotation_and_identity_at_zero():
    # D = 2: the pair (x0, x1) turns by pos * base^0 = pos radians
    cos, sin = od.rope_angles(4, 4, 2, 10000.0)
    x = np.tile([[1.0, 0.0]], (4, 1))
    y = od.rope(x, cos, sin, 1, 2)
    assert np.allclose(y, np.stack([np.cos(np.arange(4)), np.sin(np.arange(4))], axis=1), atol=1e-15)
    x = RS.normal(size=(1, 3 * 8))
    c0, s0 = od.rope_angles(1, 1, 8, 500000.0)
    assert np.array_equal(od.rope(x, c0, s0, 3, 8), x)


def test_rope_norms_inverse_and_relative_positions():
    T, D, nh = 12, 16, 2
    cos, sin = od.rope_angles(T, T, D, 10000.0)
    x = RS.normal(size=(T, nh * D))
    y = od.rope(x, cos, sin, nh, D)
    xa, ya = x.reshape(T, nh, 2, D // 2), y.reshape(T, nh, 2, D // 2)
    assert np.allclose(np.hypot(xa[:, :, 0], xa[:, :, 1]), np.hypot(ya[:, :, 0], ya[:, :, 1]))
    assert np.allclose(od.rope(y, cos, sin, nh, D, inverse=True), x, atol=1e-13)
    # <R(p) q, R(p') k> depends on p - p' only
    q, k = RS.normal(size=D), RS.normal(size=D)
    Q = od.rope(np.tile(q, (T, 1)), cos, sin, 1, D)
    K = od.rope(np.tile(k, (T, 1)), cos, sin, 1, D)
    assert math.isclose(Q[5] @ K[2], Q[9] @ K[6], rel_tol=1e-12)
    # positions restart with every sequence
    c2, s2 = od.rope_angles(2 * T, T, D, 10000.0)
    assert np.array_equal(c2[T:], c2[:T]) and np.array_equal(s2[T:], s2[:T])


# ------------------------------------------------------------------ attention
def _brute_attention(q, k, v, nh, nkv, D, S):
    T = q.shape[0]
    o = np.zeros((T, nh * D))
    for h in range(nh):
        kv = h // (nh // nkv)
        for t in range(T):
            s0 = (t // S) * S
            w = [math.exp(float(q[t, h * D:(h + 1) * D] @ k[j, kv * D:(kv + 1) * D]) / math.sqrt(D))
                 for j in range(s0, t + 1)]
            z = sum(w)
            for j, wj in zip(range(s0, t + 1), w):
                o[t, h * D:(h + 1) * D] += wj / z * v[j, kv * D:(kv + 1) * D]
    return o


def test_attention_matches_loop_brute_force():
    T, S, nh, nkv, D = 10, 5, 4, 2, 4
    q, k, v = RS.normal(size=(T, nh * D)), RS.normal(size=(T, nkv * D)), RS.normal(size=(T, nkv * D))
    o, lse = od.attention(q, k, v, nh, nkv, D, S)
    assert np.allclose(o, _brute_attention(q, k, v, nh, nkv, D, S), atol=1e-13)
    # first token of each sequence attends to itself only
    for t in (0, S):
        assert np.allclose(o[t, :D], v[t, :D], atol=1e-15)
        assert math.isclose(lse[0, t], float(q[t, :D] @ k[t, :D]) / 2.0, rel_tol=1e-12, abs_tol=1e-15)


def test_attention_zero_queries_average_the_prefix():
    T, S, D = 6, 6, 4
    v = RS.normal(size=(T, D))
    o, lse = od.attention(np.zeros((T, D)), RS.normal(size=(T, D)), v, 1, 1, D, S)
    assert np.allclose(o, np.cumsum(v, axis=0) / np.arange(1, T + 1)[:, None], atol=1e-14)
    assert np.allclose(lse[0], np.log(np.arange(1, T + 1)), atol=1e-14)


def test_attention_backward_finite_differences():
    T, S, nh, nkv, D = 6, 3, 2, 1, 4
    q, k, v = RS.normal(size=(T, nh * D)), RS.normal(size=(T, nkv * D)), RS.normal(size=(T, nkv * D))
    do = RS.normal(size=(T, nh * D))
    o, lse = od.attention(q, k, v, nh, nkv, D, S)
    dq, dk, dv = od.attention_bwd(q, k, v, o, lse, do, nh, nkv, D, S)
    f = lambda qq, kk, vv: np.sum(od.attention(qq, kk, vv, nh, nkv, D, S)[0] * do)
    assert np.allclose(dq, fd(lambda z: f(z, k, v), q), atol=1e-8)
    assert np.allclose(dk, fd(lambda z: f(q, z, v), k), atol=1e-8)
    assert np.allclose(dv, fd(lambda z: f(q, k, z), v), atol=1e-8)


# ------------------------------------------------------------------ SwiGLU
def test_swiglu_values_and_backward():
    assert od.silu(np.array([0.0]))[0] == 0.0
    assert math.isclose(od.silu(np.array([40.0]))[0], 40.0, rel_tol=1e-15)
    assert math.isclose(od.silu(np.array([1.0]))[0], 1.0 / (1.0 + math.exp(-1.0)), rel_tol=1e-15)
    g, u, ds = RS.normal(size=(3, 5)), RS.normal(size=(3, 5)), RS.normal(size=(3, 5))
    dg, du = od.swiglu_bwd(g, u, ds)
    assert np.allclose(dg, fd(lambda z: np.sum(od.swiglu(z, u) * ds), g), atol=1e-8)
    assert np.allclose(du, fd(lambda z: np.sum(od.swiglu(g, z) * ds), u), atol=1e-8)


# ------------------------------------------------------------------ layer and model
CFG = {"n_heads": 4, "n_kv": 2, "head_dim": 4, "seq_len": 3, "eps": 1e-5, "rope_base": 10000.0}


def _layer_params(H=8, inter=12, r=2, seed=0):
    rs = np.random.default_rng(seed)
    nh, nkv, D = CFG["n_heads"], CFG["n_kv"], CFG["head_dim"]
    shapes = {"q": (nh * D, H), "k": (nkv * D, H), "v": (nkv * D, H), "o": (H, nh * D),
              "gate": (inter, H), "up": (inter, H), "down": (H, inter)}
    W = {p: rs.normal(size=s) * 0.3 for p, s in shapes.items()}
    ad = {p: (rs.normal(size=(r, s[1])) * 0.3, rs.normal(size=(s[0], r)) * 0.3, 1.5) for p, s in shapes.items()}
    return {"W": W, "ad": ad, "g1": 1 + 0.1 * rs.normal(size=H), "g2": 1 + 0.1 * rs.normal(size=H)}


def test_layer_backward_finite_differences():
    P = _layer_params()
    T, H = 6, 8
    x, dout = RS.normal(size=(T, H)), RS.normal(size=(T, H))
    y, c = od.layer_fwd(P, CFG, x, rnd=False)
    dx, grads = od.layer_bwd(P, CFG, c, dout, rnd=False)
    obj = lambda: np.sum(od.layer_fwd(P, CFG, x_, rnd=False)[0] * dout)
    x_ = x
    assert np.allclose(dx, fd(lambda z: np.sum(od.layer_fwd(P, CFG, z, rnd=False)[0] * dout), x), atol=1e-7)
    for p in ("q", "k", "v", "o", "gate", "down"):
        A, B, s = P["ad"][p]

        def with_A(z):
            P["ad"][p] = (z, B, s)
            out = obj()
            P["ad"][p] = (A, B, s)
            return out

        def with_B(z):
            P["ad"][p] = (A, z, s)
            out = obj()
            P["ad"][p] = (A, B, s)
            return out

        assert np.allclose(grads[p][0], fd(with_A, A), atol=1e-7), p
        assert np.allclose(grads[p][1], fd(with_B, B), atol=1e-7), p


def test_model_step_finite_differences_and_rounding_stays_close():
    V, H, T = 11, 8, 6
    rs = np.random.default_rng(7)
    M = {"embed": rs.normal(size=(V, H)), "layers": [_layer_params(seed=1), _layer_params(seed=2)],
         "g_final": 1 + 0.1 * rs.normal(size=H), "lm_head": rs.normal(size=(V, H)) * 0.5}
    ids, labels = rs.integers(0, V, size=T), rs.integers(0, V, size=T)
    out = od.model_step(M, CFG, ids, labels, rnd=False)
    P = M["layers"][0]
    A, B, s = P["ad"]["v"]

    def loss_with(z):
        P["ad"]["v"] = (z, B, s)
        val = od.model_step(M, CFG, ids, labels, rnd=False)["loss"]
        P["ad"]["v"] = (A, B, s)
        return val

    assert np.allclose(out["grads"][0]["v"][0], fd(loss_with, A), atol=1e-8)
    # the embedding output's gradient: perturb the embedding rows the ids select
    E = M["embed"].copy()

    def loss_emb(z):
        M["embed"] = z
        val = od.model_step(M, CFG, ids, labels, rnd=False)["loss"]
        M["embed"] = E
        return val

    gE = fd(loss_emb, E)
    want = np.zeros_like(E)
    np.add.at(want, ids, out["dx0"])
    assert np.allclose(gE, want, atol=1e-8)
    # bf16 storage at every call output changes the result only at bf16 scale
    r = od.model_step(M, CFG, ids, labels, rnd=True)
    assert abs(r["loss"] - out["loss"]) < 2e-2 * abs(out["loss"])


def test_attention_gqa_equals_repeated_kv_heads():
    T, S, nh, nkv, D = 8, 4, 4, 2, 4
    q, k, v = RS.normal(size=(T, nh * D)), RS.normal(size=(T, nkv * D)), RS.normal(size=(T, nkv * D))
    rep = lambda a: np.repeat(a.reshape(T, nkv, D), nh // nkv, axis=1).reshape(T, nh * D)
    o1, l1 = od.attention(q, k, v, nh, nkv, D, S)
    o2, l2 = od.attention(q, rep(k), rep(v), nh, nh, D, S)
    assert np.allclose(o1, o2, atol=1e-15) and np.allclose(l1, l2, atol=1e-15)


def test_layer_with_zero_output_projections_is_the_identity():
    P = _layer_params()
    P["W"]["o"][:] = 0.0
    P["W"]["down"][:] = 0.0
    for p in ("o", "down"):
        A, B, s = P["ad"][p]
        P["ad"][p] = (A, np.zeros_like(B), s)
    x = RS.normal(size=(6, 8))
    y, _ = od.layer_fwd(P, CFG, x, rnd=False)
    assert np.array_equal(y, x)


def test_storage_jitter_is_scoped_and_small():
    x = RS.normal(size=(400, 400))
    base = od.q16(x)
    with od.storage_jitter(np.random.default_rng(0), 1e-6):
        j = od.q16(x)
        assert np.array_equal(od.q16(x, rnd=False), x)      # no storage, no jitter
    assert np.array_equal(od.q16(x), base)                   # restored on exit
    # a 1e-6 relative perturbation moves an element by at most one bf16 step, rarely
    step = np.abs(j - base) / np.abs(base)
    assert step.max() <= 2.0 ** -7 and 0 < np.count_nonzero(j != base) < x.size // 50
