"""Pins for the oracle's rotary embedding (oracle/rope.py).

RoPE is tied to what defines it: the score between a rotated query at position m and a rotated
key at position n depends only on n - m; rotations compose (m1 then m2 is m1 + m2) and keep
every pair's norm; position 0 is the identity; d = 2 is a plain planar rotation by m.  The two
pairings are tied to each other by a fixed permutation of the head dim.  The striped form is
tied to the page's rule that RoPE sees the permuted position IDs, and the whole path
(RoPE, striped attention, un-permute) to plain token-order attention.
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle import attention as A
from oracle import ring as R
from oracle import rope as RP

STYLES = ["interleaved", "half"]


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_theta_values():
    np.testing.assert_allclose(RP.angles([3], 4, 10000.0), [[3.0, 0.03]], rtol=1e-15)
    np.testing.assert_allclose(RP.angles([1], 8, 16.0), [[1.0, 0.5, 0.25, 0.125]], rtol=1e-15)


@pytest.mark.parametrize("style", STYLES)
def test_position_zero_is_identity(style):
    x = _rand((3, 5, 8), 1)
    np.testing.assert_array_equal(RP.rope(x, np.zeros(5), style=style), x)


def test_two_dims_is_a_planar_rotation():
    x = _rand((7, 2), 2)
    pos = np.arange(7) * 3 + 1
    got = RP.rope(x, pos)
    c, s = np.cos(pos), np.sin(pos)
    np.testing.assert_allclose(got[:, 0], x[:, 0] * c - x[:, 1] * s, rtol=1e-14)
    np.testing.assert_allclose(got[:, 1], x[:, 0] * s + x[:, 1] * c, rtol=1e-14)


@pytest.mark.parametrize("style", STYLES)
def test_scores_depend_on_relative_position_only(style):
    d = 16
    q, k = _rand((1, d), 3), _rand((1, d), 4)
    for m, n in [(0, 5), (7, 12), (1000, 1005), (123456, 123461)]:
        s = (RP.rope(q, [m], style=style) @ RP.rope(k, [n], style=style).T).item()
        s0 = (RP.rope(q, [0], style=style) @ RP.rope(k, [n - m], style=style).T).item()
        assert s == pytest.approx(s0, rel=1e-9, abs=1e-9)


@pytest.mark.parametrize("style", STYLES)
def test_rotations_compose_and_keep_norms(style):
    x = _rand((4, 6, 12), 5)
    m1, m2 = np.arange(6) * 11, np.arange(6) * 7 + 2
    np.testing.assert_allclose(RP.rope(RP.rope(x, m1, style=style), m2, style=style),
                               RP.rope(x, m1 + m2, style=style), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(RP.rope(RP.rope(x, m1, style=style), m1, style=style, inverse=True), x,
                               rtol=1e-12, atol=1e-12)
    a, b = RP.pair_index(12, style)
    y = RP.rope(x, m1, style=style)
    np.testing.assert_allclose(y[..., a] ** 2 + y[..., b] ** 2, x[..., a] ** 2 + x[..., b] ** 2, rtol=1e-12)


def test_half_pairing_is_a_permuted_interleaved_pairing():
    d = 10
    x = _rand((5, d), 6)
    pos = np.arange(5) * 13
    perm = np.empty(d, dtype=np.int64)                 # half-pairing element -> interleaved slot
    perm[: d // 2] = 2 * np.arange(d // 2)
    perm[d // 2:] = 2 * np.arange(d // 2) + 1
    xi = np.empty_like(x)
    xi[:, perm] = x
    got = RP.rope(xi, pos, style="interleaved")[:, perm]
    np.testing.assert_allclose(RP.rope(x, pos, style="half"), got, rtol=1e-14)


@pytest.mark.parametrize("style", STYLES)
def test_striped_rope_uses_the_permuted_position_ids(style):
    n, P, d = 24, 4, 8
    x = _rand((2, n, d), 7)
    pos = np.arange(n) + 100
    order = R.layout_order(n, P, "striped")
    want = RP.rope(R.to_layout(x, order), pos[order], style=style)     # rotate in the layout with permuted IDs
    np.testing.assert_allclose(RP.rope_permute(x, P, "striped", pos, style=style), want, rtol=1e-14)
    back = RP.rope_permute(want, P, "striped", pos, style=style, inverse=True)
    np.testing.assert_allclose(back, x, rtol=1e-12, atol=1e-12)


def test_inverse_is_the_adjoint():
    # <rope_permute(x), y> = <x, rope_permute^T(y)>: inverse=True is the gradient map
    n, P, d = 16, 4, 6
    x, y = _rand((n, d), 8), _rand((n, d), 9)
    lhs = np.sum(RP.rope_permute(x, P, "striped", style="half") * y)
    rhs = np.sum(x * RP.rope_permute(y, P, "striped", style="half", inverse=True))
    assert lhs == pytest.approx(rhs, rel=1e-12)


def test_striped_attention_with_rope_equals_token_order():
    n, P, d = 32, 4, 8
    q, k, v = _rand((1, 1, n, d), 10), _rand((1, 1, n, d), 11), _rand((1, 1, n, d), 12)
    o_tok, _ = A.attention(RP.rope(q, np.arange(n)), RP.rope(k, np.arange(n)), v, True)
    order = R.layout_order(n, P, "striped")
    qs = RP.rope_permute(q, P, "striped")
    ks = RP.rope_permute(k, P, "striped")
    o_s, _ = A.attention(qs, ks, R.to_layout(v, order), True, pos_q=order, pos_k=order)
    np.testing.assert_allclose(R.from_layout(o_s, order), o_tok, rtol=1e-12, atol=1e-12)


def test_planted_mistakes_are_caught(monkeypatch):
    def check():
        test_theta_values()
        for st in STYLES:
            test_scores_depend_on_relative_position_only(st)
            test_striped_rope_uses_the_permuted_position_ids(st)
        test_half_pairing_is_a_permuted_interleaved_pairing()
        test_two_dims_is_a_planar_rotation()

    check()
    orig_angles, orig_pairs = RP.angles, RP.pair_index

    def theta_half_rate(pos, d, base):              # base^(-i/d) instead of base^(-2i/d)
        return np.asarray(pos, np.float64)[:, None] * float(base) ** (-np.arange(d // 2) / d)[None, :]

    def pairs_swapped(d, style):                    # rotation direction flipped
        a, b = orig_pairs(d, style)
        return b, a

    def half_as_interleaved(d, style):
        return orig_pairs(d, "interleaved")

    def unpermuted_ids(pos, d, base):               # angles from the layout row, not the token
        return orig_angles(np.arange(len(pos)), d, base)

    for name, bad in (("angles", theta_half_rate), ("pair_index", pairs_swapped),
                      ("pair_index", half_as_interleaved)):
        monkeypatch.setattr(RP, name, bad)
        with pytest.raises(AssertionError):
            check()
        monkeypatch.setattr(RP, name, orig_angles if name == "angles" else orig_pairs)
    monkeypatch.setattr(RP, "angles", unpermuted_ids)
    with pytest.raises(AssertionError):
        test_striped_rope_uses_the_permuted_position_ids("interleaved")
    monkeypatch.setattr(RP, "angles", orig_angles)
    check()
