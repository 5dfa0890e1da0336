"""Pins for the oracle's LoRA linear: closed forms, finite differences, brute force,
special cases and the counts printed on the pages."""
import json
import os

import numpy as np

from oracle import layer, lora
import synthgen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")


def _case(seed=0, T=5, out_f=6, in_f=7, r=3):
    rs = np.random.default_rng(seed)
    x = rs.standard_normal((T, in_f))
    W = rs.standard_normal((out_f, in_f))
    A = rs.standard_normal((r, in_f))
    B = rs.standard_normal((out_f, r))
    dy = rs.standard_normal((T, out_f))
    return x, W, A, B, dy


def test_forward_brute_force_loops():
    x, W, A, B, _ = _case()
    s = 1.75
    y, u = lora.linear_fwd(x, W, A, B, s)
    T, in_f = x.shape
    out_f, r = B.shape
    for t in range(T):
        for o in range(out_f):
            acc = sum(x[t, i] * W[o, i] for i in range(in_f))
            for k in range(r):
                acc += s * sum(x[t, i] * A[k, i] for i in range(in_f)) * B[o, k]
            assert abs(acc - y[t, o]) < 1e-12


def test_merge_identity():
    # merging the adapter into the base gives the same linear map
    x, W, A, B, _ = _case(1, 8, 16, 12, 4)
    s = 2.5
    y, _ = lora.linear_fwd(x, W, A, B, s)
    y_merged = x @ (W + s * B @ A).T
    assert np.allclose(y, y_merged, rtol=1e-13, atol=1e-13)


def test_backward_brute_force_dx_is_wT_dy():
    # dL/dx = W^T dL/dy, checked with explicit loops (adapters off)
    x, W, _, _, dy = _case(2)
    dx, dA, dB = lora.linear_bwd(x, dy, W)
    assert dA is None and dB is None
    T, out_f = dy.shape
    in_f = W.shape[1]
    for t in range(T):
        for i in range(in_f):
            ref = sum(W[o, i] * dy[t, o] for o in range(out_f))
            assert abs(ref - dx[t, i]) < 1e-12


def test_adjoint_identity():
    # y is linear in x, so <dy, y(x)> == <dx, x>
    x, W, A, B, dy = _case(3, 9, 10, 11, 2)
    s = 4.0
    y, _ = lora.linear_fwd(x, W, A, B, s)
    dx, _, _ = lora.linear_bwd(x, dy, W, A, B, s)
    assert abs(np.sum(dy * y) - np.sum(dx * x)) < 1e-10 * np.sum(np.abs(dy * y))


def test_finite_differences():
    rs = np.random.default_rng(4)
    T, in_f, out_f, r, s = 4, 64, 64, 2, 3.0
    x = rs.standard_normal((T, in_f))
    W = rs.standard_normal((out_f, in_f)) * 0.05
    A = rs.standard_normal((r, in_f)) * 0.1
    B = rs.standard_normal((out_f, r)) * 0.1
    dy = rs.standard_normal((T, out_f))

    def loss(x_, A_, B_):
        return float(np.sum(dy * lora.linear_fwd(x_, W, A_, B_, s)[0]))

    dx, dA, dB = lora.linear_bwd(x, dy, W, A, B, s)
    h = 1e-6
    for (arr, grad, which) in ((x, dx, 0), (A, dA, 1), (B, dB, 2)):
        idx = [tuple(rs.integers(0, n) for n in arr.shape) for _ in range(12)]
        for ix in idx:
            p, m = arr.copy(), arr.copy()
            p[ix] += h
            m[ix] -= h
            args_p = [x, A, B]
            args_m = [x, A, B]
            args_p[which], args_m[which] = p, m
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - grad[ix]) < 1e-6 * max(1.0, abs(grad[ix])), (which, ix, fd, grad[ix])


def test_second_route_through_full_weight_gradient():
    # with G = dy^T x the full-weight gradient: dA = s B^T G, dB = s G A^T
    x, W, A, B, dy = _case(5, 7, 9, 8, 3)
    s = 0.5
    _, dA, dB = lora.linear_bwd(x, dy, W, A, B, s)
    G = dy.T @ x
    assert np.allclose(dA, s * B.T @ G, rtol=1e-12, atol=1e-12)
    assert np.allclose(dB, s * G @ A.T, rtol=1e-12, atol=1e-12)


def test_adapter_off_and_zero_b_equal_base_exactly():
    x, W, A, B, dy = _case(6)
    y_base, u0 = lora.linear_fwd(x, W)
    assert u0 is None
    assert np.array_equal(y_base, x @ W.T)
    y0, _ = lora.linear_fwd(x, W, A, np.zeros_like(B), 2.0)
    assert np.array_equal(y0, y_base)
    dx_base, _, _ = lora.linear_bwd(x, dy, W)
    assert np.array_equal(dx_base, dy @ W)
    # r = 0 adapters are "off"
    y_r0, u_r0 = lora.linear_fwd(x, W, A[:0], B[:, :0], 2.0)
    assert u_r0 is None and np.array_equal(y_r0, y_base)


def test_trainable_params_match_page():
    g = json.load(open(GOLDEN))
    wl = synthgen.WORKLOADS["qwen05b"]
    per_layer = lora.trainable_params([wl.shapes[n] for n in ("q", "v")], 16)
    assert per_layer * wl.layers == g["trainable_params"]["value"]
    pct = 100.0 * g["trainable_params"]["value"] / g["total_params_approx"]["value"]
    assert round(pct, 2) == g["trainable_percent"]["value"]


def test_layer_size_matches_page_preflight():
    g = json.load(open(GOLDEN))
    wl = synthgen.WORKLOADS["qwen05b"]
    P = sum(o * i for (o, i) in wl.shapes.values())
    assert P == 14_909_440
    bpp = g["ram_store"]["bytes_per_param"]
    assert round(P * bpp * g["ram_store"]["layers"] / 1e9, 2) == g["ram_store"]["gb"]
    assert round(P * bpp / 1e6) == g["layer_buffers"]["mb_each"]


def test_layer_step_composition():
    rs = np.random.default_rng(7)
    shapes = {"q": (8, 6), "k": (4, 6), "v": (4, 6), "o": (6, 8), "gate": (10, 6), "up": (10, 6), "down": (6, 10)}
    W = {n: rs.standard_normal(s) for n, s in shapes.items()}
    ad = {n: (rs.standard_normal((2, shapes[n][1])), rs.standard_normal((shapes[n][0], 2)), 1.5) for n in ("q", "v")}
    T = 3
    xs = {0: rs.standard_normal((T, 6)), 1: rs.standard_normal((T, 8)), 2: rs.standard_normal((T, 6)),
          3: rs.standard_normal((T, 10))}
    dys = {n: rs.standard_normal((T, shapes[n][0])) for n in shapes}
    res = layer.layer_step(W, ad, xs, dys, dpo=True)
    for n in shapes:
        assert np.array_equal(res["fwd"][n], res["recompute"][n])
    # reference pass = base linear; dx of a group sums its projections
    assert np.array_equal(res["ref"]["q"], xs[0] @ W["q"].T)
    A, B, s = ad["q"]
    Av, Bv, sv = ad["v"]
    dx0 = dys["q"] @ W["q"] + s * dys["q"] @ B @ A + dys["k"] @ W["k"] + dys["v"] @ W["v"] + sv * dys["v"] @ Bv @ Av
    assert np.allclose(res["dx"][0], dx0, rtol=1e-12, atol=1e-12)
    assert res["grads"]["k"] == (None, None)
