"""Pins for the CPU oracle: each check ties the oracle to something other than itself.

The pins are closed forms, a library routine (torch's scaled_dot_product_attention in fp64),
brute force on tiny inputs, invariants the pages state (blockwise online softmax equals full
attention; striped outputs are a permutation of contiguous outputs), and the worked partition
example printed in the Striped Attention review (tests/golden/).  The last group plants
mistakes in the oracle and checks that a pin catches each one.
"""
from __future__ import annotations

import itertools
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import ring as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
LAYOUTS = [R.CONTIGUOUS, R.STRIPED]


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ------------------------------------------------------------------- layouts and permutation
def test_partition_matches_page_example():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "striped_partition_n16_p4.txt"))
            if ln.strip() and not ln.startswith("#")]
    assert rows
    for layout, dev, *tokens in rows:
        order = R.layout_order(16, 4, layout)
        c = 4
        dev = int(dev)
        assert order[dev * c:(dev + 1) * c].tolist() == [int(t) for t in tokens]


@pytest.mark.parametrize("n,P", [(16, 4), (32, 4), (48, 8), (12, 3), (64, 64), (7, 1)])
def test_permutation_closed_form(n, P):
    c = n // P
    pi = R.layout_position(n, P, R.STRIPED)
    t = np.arange(n)
    assert np.array_equal(pi, (t % P) * c + t // P)            # token t -> slot t//P of device t%P
    order = R.layout_order(n, P, R.STRIPED)
    assert np.array_equal(pi[order], np.arange(n))             # pi o order = id
    assert np.array_equal(order[pi], np.arange(n))
    assert np.array_equal(R.layout_order(n, P, R.CONTIGUOUS), np.arange(n))
    if P in (1, n):                                            # P=1 and P=n: striped is the identity
        assert np.array_equal(order, np.arange(n))


def test_layout_roundtrip():
    x = _rand((2, 3, 24, 5), 1)
    order = R.layout_order(24, 4, R.STRIPED)
    assert np.array_equal(R.from_layout(R.to_layout(x, order), order), x)


def test_schedule_matches_explicit_ring_passing():
    # simulate the ring: in each round every device passes the block it holds to rank + 1
    for P in (1, 2, 3, 4, 8):
        held = list(range(P))                     # round 0: own block
        for r in range(P):
            for p in range(P):
                assert R.kv_block(p, r, P) == held[p]
            held = [held[(p - 1) % P] for p in range(P)]   # receive from rank - 1
        assert sorted(R.kv_block(0, r, P) for r in range(P)) == list(range(P))


# ------------------------------------------------------------------- full attention
@pytest.mark.parametrize("n,d,causal", [(17, 8, True), (33, 16, False), (64, 64, True), (5, 3, True)])
def test_attention_matches_torch_sdpa_fp64(n, d, causal):
    q, k, v = (_rand((1, 2, n, d), s) for s in (2, 3, 4))
    o, lse = A.attention(q, k, v, causal)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(t) for t in (q, k, v)), is_causal=causal)
    assert np.abs(o - ref.numpy()).max() < 1e-12
    # LSE: torch.logsumexp over explicitly masked scores (library reduction, not our formula)
    s = torch.from_numpy(q) @ torch.from_numpy(k).transpose(-1, -2) / math.sqrt(d)
    if causal:
        s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
    assert np.abs(lse - torch.logsumexp(s, -1).numpy()).max() < 1e-12


def test_attention_with_permuted_positions_matches_sdpa_mask():
    n, d, P = 24, 8, 4
    q, k, v = (_rand((1, 1, n, d), s) for s in (5, 6, 7))
    order = R.layout_order(n, P, R.STRIPED)
    ql, kl, vl = (R.to_layout(t, order) for t in (q, k, v))
    o, _ = A.attention(ql, kl, vl, True, pos_q=order, pos_k=order)
    allowed = torch.from_numpy(order[None, :] <= order[:, None])   # key pos <= query pos
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(t) for t in (ql, kl, vl)), attn_mask=allowed)
    assert np.abs(o - ref.numpy()).max() < 1e-12


@pytest.mark.parametrize("causal", [True, False])
def test_zero_keys_closed_form(causal):
    # K = 0: every visible score is 0, so O_i is the mean of the visible V rows and
    # LSE_i = ln(#visible keys) = ln(i + 1) (causal) or ln(n).
    n, d = 40, 6
    v = _rand((1, 1, n, d), 8)
    o, lse = A.attention(_rand((1, 1, n, d), 9), np.zeros((1, 1, n, d)), v, causal)
    cnt = np.arange(1, n + 1) if causal else np.full(n, n)
    mean = np.cumsum(v[0, 0], 0) / cnt[:, None] if causal else np.broadcast_to(v[0, 0].mean(0), (n, d))
    assert np.abs(o[0, 0] - mean).max() < 1e-13
    assert np.abs(lse[0, 0] - np.log(cnt)).max() < 1e-13


def test_naive_loops_tiny():
    n, d = 9, 4
    q, k, v = (_rand((n, d), s) for s in (10, 11, 12))
    o, lse = A.softmax_attention(q, k, v, A.causal_bias(range(n), range(n)))
    for i in range(n):
        scores = [sum(q[i][t] * k[j][t] for t in range(d)) / math.sqrt(d) for j in range(i + 1)]
        w = [math.exp(s) for s in scores]
        z = sum(w)
        for t in range(d):
            assert abs(o[i][t] - sum(w[j] * v[j][t] for j in range(i + 1)) / z) < 1e-12
        assert abs(lse[i] - math.log(z)) < 1e-12


def test_identity_values_give_probabilities():
    n = 16
    q, k = (_rand((n, n), s) for s in (13, 14))
    o, _ = A.softmax_attention(q, k, np.eye(n), A.causal_bias(range(n), range(n)))
    assert np.abs(o.sum(1) - 1).max() < 1e-13
    assert (o >= 0).all() and np.all(np.triu(o, 1) == 0)      # no weight on future keys


def test_fully_masked_row_is_merge_identity():
    o, lse = A.softmax_attention(_rand((3, 4), 1), _rand((5, 4), 2), _rand((5, 4), 3),
                                 np.full((3, 5), -np.inf))
    assert np.all(o == 0) and np.all(lse == -np.inf)


# ------------------------------------------------------------------- blockwise == full
@pytest.mark.parametrize("P", [1, 2, 4, 8])
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("causal", [True, False])
def test_blockwise_equals_full(P, layout, causal):
    n, d = 64, 16
    q, k, v = (_rand((n, d), s) for s in (20, 21, 22))
    order = R.layout_order(n, P, layout)
    ql, kl, vl = (R.to_layout(t, order, 0) for t in (q, k, v))
    o_blk, lse_blk = R.blockwise_all(ql, kl, vl, P, layout, causal)
    o_full, lse_full = A.softmax_attention(q, k, v, A.causal_bias(range(n), range(n)) if causal else None)
    assert np.abs(R.from_layout(o_blk, order, 0) - o_full).max() < 1e-12
    assert np.abs(R.from_layout(lse_blk[:, None], order, 0)[:, 0] - lse_full).max() < 1e-12


def test_round_order_does_not_matter():
    n, d, P = 48, 8, 4
    q, k, v = (_rand((n, d), s) for s in (23, 24, 25))
    order = R.layout_order(n, P, R.STRIPED)
    ql, kl, vl = (R.to_layout(t, order, 0) for t in (q, k, v))
    ref = R.blockwise_device(ql, kl, vl, 2, P, R.STRIPED, True)
    rng = np.random.default_rng(0)
    for _ in range(5):
        got = R.blockwise_device(ql, kl, vl, 2, P, R.STRIPED, True, rounds=rng.permutation(P))
        assert np.abs(got[0] - ref[0]).max() < 1e-12 and np.abs(got[1] - ref[1]).max() < 1e-12


def test_striped_equivariance():
    n, d, P = 64, 8, 8
    q, k, v = (_rand((n, d), s) for s in (26, 27, 28))
    outs = {}
    for layout in LAYOUTS:
        order = R.layout_order(n, P, layout)
        o, _ = R.blockwise_all(*(R.to_layout(t, order, 0) for t in (q, k, v)), P, layout, True)
        outs[layout] = R.from_layout(o, order, 0)
    assert np.abs(outs[R.STRIPED] - outs[R.CONTIGUOUS]).max() < 1e-12


def test_local_only_attention_is_wrong():
    # the flawed scheme (each device attends to its own segment only) must differ
    n, d, P = 32, 8, 4
    q, k, v = (_rand((n, d), s) for s in (29, 30, 31))
    o_full, _ = A.softmax_attention(q, k, v, A.causal_bias(range(n), range(n)))
    assert np.abs(R.local_only(q, k, v, P, R.CONTIGUOUS, True) - o_full).max() > 1e-2


# ------------------------------------------------------------------- merge
def _partials(seed, rows=6, dv=5, nkeys=(4, 7, 3)):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((rows, 4))
    ks = [rng.standard_normal((m, 4)) for m in nkeys]
    vs = [rng.standard_normal((m, dv)) for m in nkeys]
    parts = [A.softmax_attention(q, kk, vv) for kk, vv in zip(ks, vs)]
    full = A.softmax_attention(q, np.concatenate(ks), np.concatenate(vs))
    return parts, full


def test_merge_of_key_partition_equals_full():
    parts, (o_full, l_full) = _partials(40)
    o, l = parts[0]
    for po, pl in parts[1:]:
        o, l = R.merge(o, l, po, pl)
    assert np.abs(o - o_full).max() < 1e-12 and np.abs(l - l_full).max() < 1e-12


def test_merge_assoc_comm_identity():
    (a, b, c), _ = _partials(41)
    ab_c = R.merge(*R.merge(*a, *b), *c)
    a_bc = R.merge(*a, *R.merge(*b, *c))
    ba = R.merge(*b, *a)
    ab = R.merge(*a, *b)
    for x, y in ((ab_c, a_bc), (ab, ba)):
        assert np.abs(x[0] - y[0]).max() < 1e-12 and np.abs(x[1] - y[1]).max() < 1e-12
    empty = (np.zeros_like(a[0]), np.full_like(a[1], -np.inf))
    e = R.merge(*a, *empty)
    assert np.array_equal(e[0], a[0]) and np.array_equal(e[1], a[1])
    ee = R.merge(*empty, *empty)
    assert np.all(ee[0] == 0) and np.all(ee[1] == -np.inf)


def test_streamed_rounds_with_stop_and_resume():
    # per-round partials merged one by one (stopping after 2 rounds and resuming from the saved
    # accumulator) equal the fused online-softmax device result
    n, d, P, p = 64, 8, 8, 6
    q, k, v = (_rand((n, d), s) for s in (42, 43, 44))
    order = R.layout_order(n, P, R.STRIPED)
    ql, kl, vl = (R.to_layout(t, order, 0) for t in (q, k, v))
    c = n // P
    acc = (np.zeros((c, d)), np.full(c, -np.inf))
    saved = None
    for r in range(P):
        kk = R.kv_block(p, r, P)
        part = R.round_partial(ql[p * c:(p + 1) * c], kl[kk * c:(kk + 1) * c], vl[kk * c:(kk + 1) * c],
                               R.STRIPED, p, kk, True)
        acc = R.merge(*acc, *part)
        if r == 1:
            saved = (acc[0].copy(), acc[1].copy())
            acc = None
            acc = saved
    ref = R.blockwise_device(ql, kl, vl, p, P, R.STRIPED, True)
    assert np.abs(acc[0] - ref[0]).max() < 1e-12 and np.abs(acc[1] - ref[1]).max() < 1e-12


# ------------------------------------------------------------------- GetMask and counts
def _divisor_pairs(max_n=64):
    for n in (8, 12, 16, 24, 32, 48, 64):
        if n > max_n:
            continue
        for P in range(1, n + 1):
            if n % P == 0 and n // P >= 1 and P <= 16:
                yield n, P


@pytest.mark.parametrize("layout", LAYOUTS)
def test_getmask_equals_position_mask(layout):
    for n, P in _divisor_pairs():
        c = n // P
        order = R.layout_order(n, P, layout)
        for j, k in itertools.product(range(P), range(P)):
            want = A.causal_bias(order[j * c:(j + 1) * c], order[k * c:(k + 1) * c])
            assert np.array_equal(R.round_bias(layout, j, k, c, True), want), (n, P, j, k)


def test_getmask_transposed_reading_is_wrong():
    n, P = 16, 4
    c = n // P
    order = R.layout_order(n, P, R.STRIPED)
    bad = 0
    for j, k in itertools.product(range(P), range(P)):
        want = A.causal_bias(order[j * c:(j + 1) * c], order[k * c:(k + 1) * c])
        bad += not np.array_equal(R.get_mask(R.STRIPED, j, k, c), want)  # MASK used as [y, x]
    assert bad > 0


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("causal", [True, False])
def test_pair_counts_closed_form(layout, causal):
    for n, P in _divisor_pairs():
        c = n // P
        total = 0
        for p, r in itertools.product(range(P), range(P)):
            k = R.kv_block(p, r, P)
            got = R.visible_pairs(layout, p, k, c, causal)
            assert got == R.work_closed_form(layout, p, k, c, causal)
            total += got
        assert total == (n * (n + 1) // 2 if causal else n * n)


def test_per_round_work_shapes():
    # contiguous rounds r >= 1 are all-or-nothing; striped rounds are always triangles
    c, P = 6, 4
    for p, r in itertools.product(range(P), range(1, P)):
        k = R.kv_block(p, r, P)
        assert R.visible_pairs(R.CONTIGUOUS, p, k, c, True) in (0, c * c)
        assert R.visible_pairs(R.STRIPED, p, k, c, True) in (c * (c + 1) // 2, c * (c - 1) // 2)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("c,tq,tk", [(16, 4, 4), (16, 4, 8), (24, 8, 4), (20, 8, 6), (13, 4, 4), (9, 16, 16), (32, 32, 8)])
def test_tile_counts_closed_form_equals_brute(layout, c, tq, tk):
    for P in (1, 3, 4):
        for j, k in itertools.product(range(P), range(P)):
            for causal in (True, False):
                assert R.tile_counts_closed_form(layout, j, k, c, tq, tk, causal) == \
                    R.tile_counts_brute(layout, j, k, c, tq, tk, causal)


def test_tile_counts_example_values():
    # c = 2048 with 128 x 128 tiles: a 16 x 16 tile grid; a triangular block gives 120 full, 16
    # diagonal and 120 skipped tiles; 128 x 64 tiles give 240 + 32 + 240
    for layout, j, k in ((R.CONTIGUOUS, 2, 2), (R.STRIPED, 2, 1), (R.STRIPED, 1, 2)):
        assert R.tile_counts_closed_form(layout, j, k, 2048, 128, 128, True) == (120, 16, 120)
        assert R.tile_counts_closed_form(layout, j, k, 2048, 128, 64, True) == (240, 32, 240)
    assert R.tile_counts_brute(R.STRIPED, 1, 2, 256, 32, 32, True) == (28, 8, 28)
    assert R.tile_counts_closed_form(R.CONTIGUOUS, 3, 1, 2048, 128, 128, True) == (256, 0, 0)
    assert R.tile_counts_closed_form(R.CONTIGUOUS, 1, 3, 2048, 128, 128, True) == (0, 0, 256)


def test_speedup_bound_approaches_two():
    # slowest device per round: contiguous c^2 vs striped c(c+1)/2 -> 2c/(c+1) -> 2
    for c, P in ((64, 4), (2048, 4), (32768, 8)):
        p = P - 1
        for r in range(1, P):
            k = R.kv_block(p, r, P)
            ratio = R.work_closed_form(R.CONTIGUOUS, p, k, c, True) / \
                max(R.work_closed_form(R.STRIPED, q, R.kv_block(q, r, P), c, True) for q in range(P))
            assert ratio == pytest.approx(2 * c / (c + 1), rel=1e-15)
        tot_c = sum(R.work_closed_form(R.CONTIGUOUS, p, R.kv_block(p, r, P), c, True) for r in range(P))
        tot_s = max(sum(R.work_closed_form(R.STRIPED, q, R.kv_block(q, r, P), c, True) for r in range(P))
                    for q in range(P))
        assert tot_c / tot_s == pytest.approx((c * (c + 1) / 2 + (P - 1) * c * c) / (P * c * (c + 1) / 2))
    assert 2 * 32768 / 32769 > 1.9999


# ------------------------------------------------------------------- planted mistakes
def _check_blockwise_equals_full():
    test_blockwise_equals_full(4, R.STRIPED, True)


def _check_sdpa():
    test_attention_matches_torch_sdpa_fp64(17, 8, True)


def _check_getmask():
    test_getmask_equals_position_mask(R.STRIPED)
    test_getmask_equals_position_mask(R.CONTIGUOUS)


def _check_merge():
    test_merge_of_key_partition_equals_full()


def test_planted_mistakes_are_caught(monkeypatch):
    cases = []

    # 1. scale dropped in the definition
    orig_default = A.default_scale
    cases.append(("scale", lambda: monkeypatch.setattr(A, "default_scale", lambda d: 1.0), _check_sdpa,
                  lambda: monkeypatch.setattr(A, "default_scale", orig_default)))

    # 2. GetMask transposed (MASK read as [query, key])
    orig_rb = R.round_bias
    cases.append(("mask-transpose",
                  lambda: monkeypatch.setattr(R, "round_bias",
                                              lambda lay, j, k, c, causal: R.get_mask(lay, j, k, c) if causal else np.zeros((c, c))),
                  _check_getmask, lambda: monkeypatch.setattr(R, "round_bias", orig_rb)))

    # 3. striped strict/inclusive swapped
    orig_gm = R.get_mask

    def swapped(layout, j, k, c):
        return orig_gm(layout, k, j, c) if layout == R.STRIPED else orig_gm(layout, j, k, c)
    cases.append(("strict-swap", lambda: monkeypatch.setattr(R, "get_mask", swapped), _check_getmask,
                  lambda: monkeypatch.setattr(R, "get_mask", orig_gm)))

    # 4. online softmax forgets to rescale the normaliser
    orig_update = R.OnlineState.update

    def no_l_rescale(self, s, v):
        m_new = np.maximum(self.m, s.max(axis=1))
        ref = np.where(np.isfinite(m_new), m_new, 0.0)
        alpha = np.exp(self.m - ref)
        p = np.exp(s - ref[:, None])
        self.l = self.l + p.sum(axis=1)
        self.acc = alpha[:, None] * self.acc + p @ v
        self.m = m_new
    cases.append(("l-rescale", lambda: monkeypatch.setattr(R.OnlineState, "update", no_l_rescale),
                  _check_blockwise_equals_full,
                  lambda: monkeypatch.setattr(R.OnlineState, "update", orig_update)))

    # 5. merge drops the second partial's weight
    orig_merge = R.merge

    def bad_merge(o_a, l_a, o_b, l_b):
        o, l = orig_merge(o_a, l_a, o_b, l_b)
        return o_a * np.exp(l_a - l)[..., None] + o_b, l
    cases.append(("merge-weight", lambda: monkeypatch.setattr(R, "merge", bad_merge), _check_merge,
                  lambda: monkeypatch.setattr(R, "merge", orig_merge)))

    # 6. ring direction reversed: kv_block(p, r) = (p + r) mod P breaks the explicit ring
    orig_kv = R.kv_block
    cases.append(("ring-direction", lambda: monkeypatch.setattr(R, "kv_block", lambda p, r, P: (p + r) % P),
                  test_schedule_matches_explicit_ring_passing,
                  lambda: monkeypatch.setattr(R, "kv_block", orig_kv)))

    for name, plant, check, undo in cases:
        check()                       # passes on the real oracle
        plant()
        with pytest.raises(AssertionError):
            check()
        undo()
        check()
