"""Pins of the oracle's output-side functions (embedding gather, token cross-entropy,
sequence sums, sigmoid DPO) against closed forms, invariants and finite differences."""
import math

import numpy as np
import pytest

from oracle import head


def test_embed_gather_identity_and_repeats():
    rs = np.random.default_rng(0)
    table = rs.integers(0, 1 << 16, size=(11, 5), dtype=np.uint16)
    assert np.array_equal(head.embed_gather(table, np.arange(11)), table)
    ids = np.array([3, 3, 0, 10, 3])
    out = head.embed_gather(table, ids)
    for t, i in enumerate(ids):
        assert np.array_equal(out[t], table[i])
    with pytest.raises(ValueError):
        head.embed_gather(table, np.array([11]))


def test_uniform_logits_give_log_vocab():
    T, V = 4, 9
    logp, loss, d = head.cross_entropy(np.full((T, V), 1.25), np.array([0, 3, 8, 3]))
    assert np.allclose(loss, math.log(V), rtol=0, atol=1e-15)
    expect = np.full((T, V), 1.0 / V)
    expect[np.arange(T), [0, 3, 8, 3]] -= 1.0
    assert np.allclose(d, expect / T, rtol=0, atol=1e-15)


def test_two_classes_is_softplus():
    l = np.array([[0.3, -1.7], [2.0, 5.5]])
    _, loss, _ = head.cross_entropy(l, np.array([0, 0]))
    assert np.allclose(loss, np.log1p(np.exp(l[:, 1] - l[:, 0])), rtol=1e-14)


def test_gradient_rows_sum_to_zero_and_shift_invariance():
    rs = np.random.default_rng(1)
    l = rs.normal(size=(5, 13)) * 3
    lab = rs.integers(0, 13, size=5)
    logp, _, d = head.cross_entropy(l, lab)
    assert np.allclose(d.sum(axis=1), 0.0, atol=1e-15)
    logp2, _, _ = head.cross_entropy(l + rs.normal(size=(5, 1)) * 40, lab)
    assert np.allclose(logp, logp2, rtol=0, atol=1e-12)


def test_dominant_logit_loss():
    V = 6
    l = np.zeros((1, V))
    l[0, 2] = 50.0
    _, loss, _ = head.cross_entropy(l, np.array([2]))
    assert loss[0] == pytest.approx(math.log1p((V - 1) * math.exp(-50.0)), rel=1e-12)


def test_cross_entropy_finite_differences():
    rs = np.random.default_rng(2)
    T, V = 3, 7
    l = rs.normal(size=(T, V))
    lab = np.array([1, 6, 0])
    g = np.array([0.5, -1.25, 2.0])
    _, _, d = head.cross_entropy(l, lab, grad_scale=g)
    h = 1e-6
    num = np.zeros_like(l)
    for t in range(T):
        for j in range(V):
            lp, lm = l.copy(), l.copy()
            lp[t, j] += h
            lm[t, j] -= h
            fp = np.dot(g, head.cross_entropy(lp, lab)[1])
            fm = np.dot(g, head.cross_entropy(lm, lab)[1])
            num[t, j] = (fp - fm) / (2 * h)
    assert np.allclose(d, num, rtol=0, atol=1e-8)


def test_sequence_sums():
    assert np.array_equal(head.sequence_sums(np.arange(12), 4), [6, 22, 38])
    with pytest.raises(ValueError):
        head.sequence_sums(np.arange(10), 4)


def test_dpo_at_zero_margin():
    beta, P = 0.1, 3
    s = np.random.default_rng(3).normal(size=2 * P)
    loss, g = head.dpo_loss(s, s, beta)
    assert loss == pytest.approx(math.log(2.0), rel=1e-15)
    assert np.allclose(g, np.tile([-beta / (2 * P), beta / (2 * P)], P), rtol=1e-14)


def test_dpo_finite_differences_and_limits():
    rs = np.random.default_rng(4)
    beta = 0.7
    pol, ref = rs.normal(size=4) * 3, rs.normal(size=4) * 3
    _, g = head.dpo_loss(pol, ref, beta)
    h = 1e-6
    for i in range(4):
        a, b = pol.copy(), pol.copy()
        a[i] += h
        b[i] -= h
        num = (head.dpo_loss(a, ref, beta)[0] - head.dpo_loss(b, ref, beta)[0]) / (2 * h)
        assert g[i] == pytest.approx(num, abs=1e-9)
    # large positive margin -> loss -> 0; large negative -> loss ~ -m
    big = np.array([1000.0, 0.0])
    assert head.dpo_loss(big, np.zeros(2), 1.0)[0] == pytest.approx(0.0, abs=1e-300)
    assert head.dpo_loss(-big, np.zeros(2), 1.0)[0] == pytest.approx(1000.0, rel=1e-12)


def test_dpo_chain_to_logits_finite_differences():
    """End-to-end sign check: logits -> token log-probs -> sequence sums -> DPO loss,
    differentiated through cross_entropy with the per-token scale dpo_token_scale."""
    rs = np.random.default_rng(5)
    S, V, beta = 2, 5, 0.9
    T = 2 * S                                   # one pair: chosen then rejected
    l = rs.normal(size=(T, V))
    lab = rs.integers(0, V, size=T)
    ref = rs.normal(size=2)

    def objective(logits):
        logp, _, _ = head.cross_entropy(logits, lab)
        return head.dpo_loss(head.sequence_sums(logp, S), ref, beta)[0]

    logp, _, _ = head.cross_entropy(l, lab)
    _, coef = head.dpo_loss(head.sequence_sums(logp, S), ref, beta)
    _, _, d = head.cross_entropy(l, lab, grad_scale=head.dpo_token_scale(coef, S))
    h = 1e-6
    for t in range(T):
        for j in range(V):
            a, b = l.copy(), l.copy()
            a[t, j] += h
            b[t, j] -= h
            assert d[t, j] == pytest.approx((objective(a) - objective(b)) / (2 * h), abs=1e-8)
