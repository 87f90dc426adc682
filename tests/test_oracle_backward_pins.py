"""Pins for the oracle's gradients (oracle/backward.py).

``grads`` (autograd of the definition) is tied to central finite differences of the already
pinned forward ``softmax_attention``, to closed forms (all-zero keys, constant values) and to
invariants of softmax attention that hold for any input:
  * shifting every key by one vector u adds q_i.u to every score of row i, which the softmax
    ignores, so the key gradients sum to zero over the keys;
  * each row's probabilities sum to one, so the value gradients sum to the sum of dO over the
    rows that see at least one key;
  * scores are bilinear in (q, k), so sum_i q_i.dq_i = sum_j k_j.dk_j.
The hand-written per-pair chain rule (``round_grads`` / ``ring_backward``) is pinned to the
autograd result on every layout, mask and device count, and planted mistakes in it must be
caught.
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle import attention as A
from oracle import backward as G
from oracle import ring as R

LAYOUTS = [R.CONTIGUOUS, R.STRIPED]


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _loss(q, k, v, dout, bias, scale):
    o, _ = A.softmax_attention(q, k, v, bias, scale)
    return float((o * dout).sum())


@pytest.mark.parametrize("causal,offset", [(False, 0), (True, 0), (True, 2)])
def test_grads_match_finite_differences(causal, offset):
    m, n, d = 5, 7, 3
    q, k, v, dout = _rand((m, d), 1), _rand((n, d), 2), _rand((n, 4), 3), _rand((m, 4), 4)
    pos_q = np.arange(m) + offset
    pos_k = np.arange(n)
    bias = A.causal_bias(pos_q, pos_k) if causal else None
    scale = 0.7
    dq, dk, dv = G.grads(q, k, v, dout, causal, pos_q, pos_k, scale)
    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + h
            up = _loss(q, k, v, dout, bias, scale)
            x[idx] = keep - h
            dn = _loss(q, k, v, dout, bias, scale)
            x[idx] = keep
            fd[idx] = (up - dn) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-7)


def test_zero_keys_closed_form():
    # K = 0, no mask: uniform weights 1/N, O = mean(V).  dV_j = (1/N) sum_i dO_i, dQ = 0,
    # dK_j = (scale/N) sum_i (dO_i . (v_j - mean V)) q_i.
    m, n, d = 6, 9, 4
    q, v, dout = _rand((m, d), 5), _rand((n, d), 6), _rand((m, d), 7)
    k = np.zeros((n, d))
    scale = 0.3
    dq, dk, dv = G.grads(q, k, v, dout, False, scale=scale)
    np.testing.assert_allclose(dq, 0.0, atol=1e-14)
    np.testing.assert_allclose(dv, np.tile(dout.sum(0) / n, (n, 1)), rtol=1e-12)
    ref_dk = scale / n * ((v - v.mean(0)) @ dout.T) @ q
    np.testing.assert_allclose(dk, ref_dk, rtol=1e-10, atol=1e-12)


def test_constant_values_give_zero_score_gradients():
    m, n, d = 5, 8, 4
    q, k, dout = _rand((m, d), 8), _rand((n, d), 9), _rand((m, d), 10)
    v = np.tile(_rand((1, d), 11), (n, 1))
    dq, dk, dv = G.grads(q, k, v, dout, True, np.arange(m) + 3, np.arange(n))
    np.testing.assert_allclose(dq, 0.0, atol=1e-12)
    np.testing.assert_allclose(dk, 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(0), dout.sum(0), rtol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_invariants(causal):
    m, n, d = 12, 12, 6
    q, k, v, dout = (_rand((m if i in (0, 3) else n, d), 20 + i) for i in range(4))
    dq, dk, dv = G.grads(q, k, v, dout, causal)
    np.testing.assert_allclose(dk.sum(0), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(0), dout.sum(0), rtol=1e-12, atol=1e-12)
    assert np.sum(q * dq) == pytest.approx(np.sum(k * dk), rel=1e-12, abs=1e-12)


def test_single_visible_key_row():
    # Query 0 sees key 0 only: O_0 = v_0 for any scores, so row 0 adds nothing to dQ or dK
    # and all of dO_0 lands on dV_0.
    n, d = 4, 3
    q, k, v = _rand((n, d), 30), _rand((n, d), 31), _rand((n, d), 32)
    dout = np.zeros((n, d))
    dout[0] = _rand((d,), 33)
    dq, dk, dv = G.grads(q, k, v, dout, True)
    np.testing.assert_allclose(dq, 0.0, atol=1e-14)
    np.testing.assert_allclose(dk, 0.0, atol=1e-14)
    np.testing.assert_allclose(dv[0], dout[0], rtol=1e-14)
    np.testing.assert_allclose(dv[1:], 0.0, atol=1e-14)


def test_delta_is_rowwise_dot():
    o, dout = _rand((3, 5), 40), _rand((3, 5), 41)
    np.testing.assert_allclose(G.delta(o, dout), [o[i] @ dout[i] for i in range(3)], rtol=1e-14)


@pytest.mark.parametrize("P", [1, 2, 4])
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("causal", [False, True])
def test_ring_backward_equals_autograd(P, layout, causal):
    n, d = 16, 4
    q, k, v, dout = (_rand((n, d), 50 + i) for i in range(4))
    order = R.layout_order(n, P, layout)
    pos = order                                # token position of each layout row
    ref = G.grads(q[order], k[order], v[order], dout[order], causal, pos, pos, 0.5)
    got = G.ring_backward(q[order], k[order], v[order], dout[order], P, layout, causal, 0.5)
    for g, r in zip(got, ref):
        np.testing.assert_allclose(g, r, rtol=1e-10, atol=1e-12)


def test_striped_gradients_are_permuted_contiguous_gradients():
    n, d, P = 24, 4, 4
    q, k, v, dout = (_rand((n, d), 60 + i) for i in range(4))
    base = G.ring_backward(q, k, v, dout, P, R.CONTIGUOUS, True, 0.4)
    order = R.layout_order(n, P, R.STRIPED)
    got = G.ring_backward(q[order], k[order], v[order], dout[order], P, R.STRIPED, True, 0.4)
    for g, b in zip(got, base):
        np.testing.assert_allclose(R.from_layout(g, order, axis=0), b, rtol=1e-10, atol=1e-12)


def test_fully_masked_rows_contribute_nothing():
    c, d = 4, 3
    qb, kb, vb, dob = (_rand((c, d), 70 + i) for i in range(4))
    bias = np.full((c, c), -np.inf)
    gq, gk, gv = G.round_grads(qb, kb, vb, dob, np.full(c, -np.inf), np.zeros(c), bias)
    for g in (gq, gk, gv):
        assert np.all(g == 0.0)


# ------------------------------------------------------------------- planted mistakes
def _check_ring():
    test_ring_backward_equals_autograd(4, R.STRIPED, True)


def test_planted_mistakes_are_caught(monkeypatch):
    orig = G.round_grads

    def no_delta(qb, kb, vb, dob, lse_b, delta_b, bias, scale=None):
        return orig(qb, kb, vb, dob, lse_b, np.zeros_like(delta_b), bias, scale)

    def dk_unscaled(qb, kb, vb, dob, lse_b, delta_b, bias, scale=None):
        dq, dk, dv = orig(qb, kb, vb, dob, lse_b, delta_b, bias, scale)
        return dq, dk / scale, dv

    def dq_from_v(qb, kb, vb, dob, lse_b, delta_b, bias, scale=None):
        dq, dk, dv = orig(qb, kb, vb, dob, lse_b, delta_b, bias, scale)
        dq2, _, _ = orig(qb, vb, vb, dob, lse_b, delta_b, bias, scale)
        return dq2, dk, dv

    def bias_transposed(qb, kb, vb, dob, lse_b, delta_b, bias, scale=None):
        return orig(qb, kb, vb, dob, lse_b, delta_b, bias.T, scale)

    orig_kv = R.kv_block
    orig_sa = G.softmax_attention

    def lse_dropped(q, k, v, bias, scale):          # probabilities left unnormalised
        o, lse = orig_sa(q, k, v, bias, scale)
        return o, np.zeros_like(lse)

    planted = [
        (G, "round_grads", no_delta),
        (G, "round_grads", dk_unscaled),
        (G, "round_grads", dq_from_v),
        (G, "round_grads", bias_transposed),
        (G, "kv_block", lambda p, r, P: (p + 2 * r) % P),
        (G, "softmax_attention", lse_dropped),
    ]
    _check_ring()
    for mod, name, bad in planted:
        good = getattr(mod, name)
        monkeypatch.setattr(mod, name, bad)
        with pytest.raises(AssertionError):
            _check_ring()
        monkeypatch.setattr(mod, name, good)
    _check_ring()
    assert R.kv_block is orig_kv
