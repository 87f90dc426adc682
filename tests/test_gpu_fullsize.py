"""GPU parity at full workload sizes, in the launch configuration bench.py times.

* 256K-token share (n = 262144, P = 8, H = 32, d = 128, bf16): device 7's query block against all
  8 K/V blocks with ra_forward, contiguous and striped (the striped inputs through ra_permute
  first), and striped read straight from the token-order tensors, as in the timed step.  Every device of both layouts is also run once, so
  the whole sequence's striped output, un-permuted on the GPU, can be compared with the
  contiguous one.
* The backward of device 7's share (ra_backward), both layouts: dQ on sampled rows against the
  oracle, dK and dV through identities that hold at any size; the same share streamed round by
  round through ra_backward_round equals the fused result; from token-order tensors it equals
  the permuted path bit for bit; and the backward of the 1M stress
  share (device 31) under the same checks.
* 1M-token stress (n = 1048576, P = 32, H = 8, 1% of K rows x8): device 31, striped, all 32
  rounds streamed through ra_round + ra_merge, and the same share fused with ra_forward.

Floating-point outputs are checked against the fp64 oracle on sampled query rows (the oracle
computes each sampled row against all keys in token order; attention does not depend on the
order of the keys, only on their positions).  Integer outputs (permutation, work counters) are
checked exactly.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads
from oracle import attention as OA
from oracle import ring as OR
from tests._gpu_util import compare, compare_grad, need_gpu, np64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ra():
    need_gpu()
    import striped_blockwise_amd as m
    return m


def _sel(t: torch.Tensor, heads, rows) -> torch.Tensor:
    """t[0, heads][:, rows] for a GPU tensor with numpy/list indices."""
    return t[0].index_select(0, torch.tensor(heads, device=t.device)).index_select(
        1, torch.as_tensor(np.asarray(rows), device=t.device))


def _sample_rows(c: int, k: int = 58, seed: int = 1234) -> np.ndarray:
    fixed = np.array([0, 1, 2, c // 2, c - 2, c - 1])
    rnd = np.random.default_rng(seed).choice(c, size=k, replace=False)
    return np.unique(np.concatenate([fixed, rnd]))


def _oracle_rows(w, heads, tokens):
    """fp64 attention for the given query tokens (global positions), per head, all keys."""
    o_ref, l_ref = [], []
    for h in heads:
        q, k, v = workloads.qkv(w, heads=[h])
        o, l = OA.attention(q[:, :, torch.from_numpy(tokens)], k, v, True, pos_q=tokens, pos_k=np.arange(w.n))
        o_ref.append(o[0, 0])
        l_ref.append(l[0, 0])
    return np.stack(o_ref), np.stack(l_ref)


def _expected_stats_row(layout, P, c, p, BH, tq, tk):
    out = np.zeros((P, 4), dtype=np.int64)
    for r in range(P):
        kk = OR.kv_block(p, r, P)
        pairs = OR.work_closed_form(layout, p, kk, c, True)
        full, diag, skip = OR.tile_counts_closed_form(layout, p, kk, c, tq, tk, True)
        out[r] = [pairs * BH, full * BH, diag * BH, skip * BH]
    return out


@pytest.fixture(scope="module")
def share(ra):
    w = workloads.get("share_n256k")
    print(f"[fullsize] generating {w.name}", flush=True)
    q, k, v = (t.cuda() for t in workloads.qkv(w))
    torch.cuda.synchronize()
    yield w, q, k, v
    del q, k, v
    torch.cuda.empty_cache()


@pytest.mark.parametrize("layout", ["contiguous", "striped"])
def test_share256k_device7(ra, share, layout):
    w, q, k, v = share
    P, c, p = w.P, w.c, w.device
    order = OR.layout_order(w.n, P, layout)
    if layout == "striped":
        qs, ks, vs = (ra.permute(t, P) for t in (q, k, v))
        ids = ra.permute_ids(workloads.positions(w.n).cuda(), P)
        torch.cuda.synchronize()
        idx = torch.from_numpy(order).cuda()
        assert torch.equal(ids.cpu(), torch.from_numpy(order)), "position-ID permutation"
        assert torch.equal(qs[:, 5], q[:, 5].index_select(1, idx)), "Q permutation (head 5)"
        assert torch.equal(vs[:, 31], v[:, 31].index_select(1, idx)), "V permutation (head 31)"
    else:
        qs, ks, vs = q, k, v
    stats = ra.new_stats(P)
    o, lse = ra.forward(qs, ks, vs, P, layout, True, p_begin=p, p_end=p + 1, stats=stats)
    torch.cuda.synchronize()
    tq, tk = ra.tile_shape(ra.BF16, w.d)
    got = stats.cpu().numpy()
    assert np.array_equal(got[p], _expected_stats_row(layout, P, c, p, w.B * w.H, tq, tk)), got[p]
    assert not got[:p].any() and not got[p + 1:].any()
    rows = _sample_rows(c)
    heads = [0, 9, 22, 31]
    tokens = order[p * c + rows]
    o_ref, l_ref = _oracle_rows(w, heads, tokens)
    compare(_sel(o, heads, rows).float(), _sel(lse, heads, rows), o_ref, l_ref, "bf16",
            f"share256k {layout} device {p}")
    del qs, ks, vs


def test_share256k_device7_token_order(ra, share):
    """The timed step exactly as bench.py launches it: device 7's share read straight from the
    token-order tensors (RA_STRIPED_TOKENS), no counters, preallocated outputs.  Bit-exact
    against the permuted path, sampled rows against the oracle.  Then the counting variant of
    the same launch, with a counter buffer pre-filled with garbage: the call clears device 7's
    row and writes the closed-form counts there, leaves the other rows alone, and its O and LSE
    equal the non-counting launch's bit for bit."""
    w, q, k, v = share
    P, c, p = w.P, w.c, w.device
    o = torch.empty((w.B, w.H, w.n, w.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.H, w.n), dtype=torch.float32, device="cuda")
    ra.forward(q, k, v, P, "striped_tokens", True, p_begin=p, p_end=p + 1, out=(o, lse))
    qs, ks, vs = (ra.permute(t, P) for t in (q, k, v))
    o_s, l_s = ra.forward(qs, ks, vs, P, "striped", True, p_begin=p, p_end=p + 1)
    del qs, ks, vs
    torch.cuda.synchronize()
    assert torch.equal(o[:, :, p::P], o_s) and torch.equal(lse[:, :, p::P], l_s), "token order vs permuted"
    rows = _sample_rows(c, seed=99)
    heads = [3, 17, 30]
    tokens = rows * P + p
    o_ref, l_ref = _oracle_rows(w, heads, tokens)
    compare(_sel(o, heads, tokens).float(), _sel(lse, heads, tokens), o_ref, l_ref, "bf16",
            "share256k token order device 7 (timed launch)")

    stats = ra.new_stats(P).fill_(12345)
    o2, l2 = ra.forward(q, k, v, P, "striped_tokens", True, p_begin=p, p_end=p + 1, stats=stats)
    torch.cuda.synchronize()
    tq, tk = ra.tile_shape(ra.BF16, w.d)
    got = stats.cpu().numpy()
    assert np.array_equal(got[p], _expected_stats_row("striped", P, c, p, w.B * w.H, tq, tk)), got[p]
    assert (got[:p] == 12345).all() and (got[p + 1:] == 12345).all(), "rows of other devices were touched"
    assert torch.equal(o2[:, :, p::P], o_s) and torch.equal(l2[:, :, p::P], l_s), "counting variant"
    del o, lse, o2, l2, o_s, l_s


def test_share256k_whole_sequence_equivariance(ra, share):
    """Striped over all devices, un-permuted, equals contiguous over all devices."""
    w, q, k, v = share
    P = w.P
    o_c, l_c = ra.forward(q, k, v, P, "contiguous", True, o_dtype=torch.float32)
    qs, ks, vs = (ra.permute(t, P) for t in (q, k, v))
    o_s, l_s = ra.forward(qs, ks, vs, P, "striped", True, o_dtype=torch.float32)
    del qs, ks, vs
    o_u = ra.permute(o_s, P, inverse=True)
    l_u = ra.permute(l_s, P, dim=-1, inverse=True)
    del o_s, l_s
    torch.cuda.synchronize()
    err_o = float((o_u - o_c).abs().max())
    err_l = float((l_u - l_c).abs().max())
    assert err_o <= 2e-2 and err_l <= 1e-3, (err_o, err_l)
    # and both against the oracle on a few tokens spread over the sequence
    tokens = np.array([0, 1, 7, 8, 4095, 32767, 32768, 131071, 200003, w.n - 2, w.n - 1])
    heads = [3, 17]
    o_ref, l_ref = _oracle_rows(w, heads, tokens)
    compare(_sel(o_u, heads, tokens), _sel(l_u, heads, tokens), o_ref, l_ref, "bf16", "whole-sequence striped")
    compare(_sel(o_c, heads, tokens), _sel(l_c, heads, tokens), o_ref, l_ref, "bf16", "whole-sequence contiguous")


@pytest.mark.parametrize("layout", ["contiguous", "striped"])
def test_share256k_device7_backward(ra, share, layout):
    """ra_backward of device 7's share at full size, as bench.py --backward runs it.

    dQ is checked against the oracle on sampled query rows (a row's dQ needs only that row
    against all keys).  dK and dV hold what device 7's queries send to all 262144 keys; the
    oracle cannot form them at this size, so they are checked through identities that hold for
    any input: the key gradients sum to zero over the keys (softmax ignores a shift of every key),
    the value gradients sum to the sum of dO over the rows (each row's probabilities sum to one),
    and sum_i q_i.dq_i = sum_j k_j.dk_j (scores are bilinear in q and k).
    """
    from oracle import backward as OB
    w, q, k, v = share
    P, c, p = w.P, w.c, w.device
    order = OR.layout_order(w.n, P, layout)
    (g_tok,) = workloads.qkv(w, "g")
    if layout == "striped":
        qs, ks, vs = (ra.permute(t, P) for t in (q, k, v))
    else:
        qs, ks, vs = q, k, v
    dout = g_tok[:, :, torch.from_numpy(order[p * c:(p + 1) * c])].contiguous().cuda()
    o, lse = ra.forward(qs, ks, vs, P, layout, True, p_begin=p, p_end=p + 1)
    dq, dk, dv = ra.backward(qs, ks, vs, dout, lse, P, layout, True, p, p + 1, o=o)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(dq).all()) and bool(torch.isfinite(dk).all()) and bool(torch.isfinite(dv).all())

    # identities, per head and head-dim column, in fp64 on the GPU
    qd = qs[:, :, p * c:(p + 1) * c].double()
    sum_dk = dk.double().sum(2)
    assert float((sum_dk.abs() / dk.double().abs().sum(2)).max()) <= 1e-2, "sum_j dK_j = 0"
    sum_dv = dv.double().sum(2)
    sum_do = dout.double().sum(2)
    assert float(((sum_dv - sum_do).abs() / dout.double().abs().sum(2)).max()) <= 1e-2, "sum_j dV_j = sum_i dO_i"
    lhs = (qd * dq.double()).sum((2, 3))
    rhs = (ks.double() * dk.double()).sum((2, 3))
    scale = (qd * dq.double()).abs().sum((2, 3))
    assert float(((lhs - rhs).abs() / scale).max()) <= 1e-2, "sum q.dq = sum k.dk"
    del qd, sum_dk, sum_dv, lhs, rhs

    # dQ on sampled rows against the oracle (keys in token order, positions = token index)
    rows = _sample_rows(c, k=10)
    heads = [0, 13, 31]
    tokens = order[p * c + rows]
    for i, h in enumerate(heads):
        qh, kh, vh, gh = workloads.qkv(w, "qkvg", heads=[h])
        t = torch.from_numpy(tokens)
        ref, _, _ = OB.grads(qh[0, 0, t], kh[0, 0], vh[0, 0], gh[0, 0, t], True, tokens, np.arange(w.n))
        got = _sel(dq, [h], rows)[0]
        compare_grad(got, ref, "bf16", f"share256k {layout} dQ head {h}")
    del qs, ks, vs, dq, dk, dv, dout, o, lse
    torch.cuda.empty_cache()


def test_share256k_backward_rounds_equal_fused(ra, share):
    """ra_backward_round over device 7's 8 rounds (dQ accumulated in place, dK/dV per block, as
    the travelling ring buffers would hold them) against the fused ra_backward, striped."""
    w, q, k, v = share
    P, c, p = w.P, w.c, w.device
    qs, ks, vs = (ra.permute(t, P) for t in (q, k, v))
    gen = torch.Generator(device="cuda").manual_seed(11)
    dout = torch.randn((w.B, w.H, c, w.d), device="cuda", generator=gen).to(torch.bfloat16)
    o, lse = ra.forward(qs, ks, vs, P, "striped", True, p_begin=p, p_end=p + 1)
    delta = ra.bwd_delta(o, dout)
    dq, dk, dv = ra.backward(qs, ks, vs, dout, lse, P, "striped", True, p, p + 1, delta=delta)
    dq_r = torch.zeros_like(dq)
    rows = slice(p * c, (p + 1) * c)
    worst = 0.0
    for r in range(P):
        kb = OR.kv_block(p, r, P)
        keys = slice(kb * c, (kb + 1) * c)
        acc = (dq_r, torch.zeros_like(dk[:, :, keys]), torch.zeros_like(dv[:, :, keys]))
        ra.backward_round(qs[:, :, rows], ks[:, :, keys], vs[:, :, keys], dout, lse, delta, P, p, kb,
                          "striped", True, grads=acc)
        for name, a_, b_ in (("dk", acc[1], dk[:, :, keys]), ("dv", acc[2], dv[:, :, keys])):
            diff = float((a_ - b_).abs().max())
            worst = max(worst, diff / max(1e-30, float(b_.abs().max())))
            assert diff <= 1e-5 * float(b_.abs().max()), (name, kb, diff)
        del acc
    torch.cuda.synchronize()
    diff = float((dq_r - dq).abs().max())
    assert diff <= 1e-5 * float(dq.abs().max()), diff
    print(f"[fullsize] streamed backward vs fused: worst relative max diff {worst:.2e}", flush=True)
    del qs, ks, vs, dq, dk, dv, dq_r, dout, o, lse, delta
    torch.cuda.empty_cache()


def test_share256k_backward_token_order(ra, share):
    """The backward of device 7's share from token-order tensors (RA_STRIPED_TOKENS): dQ on device
    7's token rows and every dK/dV row equal, bit for bit, the permuted path's gradients mapped
    back to token order."""
    w, q, k, v = share
    P, c, p = w.P, w.c, w.device
    gen = torch.Generator(device="cuda").manual_seed(23)
    dout_t = torch.randn((w.B, w.H, w.n, w.d), device="cuda", generator=gen).to(torch.bfloat16)
    o_t, lse_t = ra.forward(q, k, v, P, "striped_tokens", True, p_begin=p, p_end=p + 1)
    delta_t = ra.bwd_delta(o_t, dout_t)
    dq_t, dk_t, dv_t = ra.backward(q, k, v, dout_t, lse_t, P, "striped_tokens", True, p, p + 1, delta=delta_t)
    torch.cuda.synchronize()
    del o_t
    qs, ks, vs = (ra.permute(t, P) for t in (q, k, v))
    dout_s = dout_t[:, :, p::P].contiguous()
    o_s, lse_s = ra.forward(qs, ks, vs, P, "striped", True, p_begin=p, p_end=p + 1)
    delta_s = ra.bwd_delta(o_s, dout_s)
    dq_s, dk_s, dv_s = ra.backward(qs, ks, vs, dout_s, lse_s, P, "striped", True, p, p + 1, delta=delta_s)
    del qs, ks, vs, o_s
    torch.cuda.synchronize()
    assert torch.equal(delta_t[:, :, p::P], delta_s), "delta"
    assert torch.equal(dq_t[:, :, p::P], dq_s), "dq"
    assert torch.equal(dk_t, ra.permute(dk_s, P, inverse=True)), "dk"
    assert torch.equal(dv_t, ra.permute(dv_s, P, inverse=True)), "dv"
    del dq_t, dk_t, dv_t, dq_s, dk_s, dv_s, dout_t, dout_s
    torch.cuda.empty_cache()


def test_stress1m_backward(ra):
    """Backward of device 31's share of the 1M-token stress sequence (1% of K rows x8): dQ on
    sampled rows against the oracle, dK/dV through the key-shift, row-sum and bilinearity
    identities (see test_share256k_device7_backward)."""
    from oracle import backward as OB
    w = workloads.get("stress_n1m")
    P, c, p = w.P, w.c, w.device
    print(f"[fullsize] generating {w.name} with dO", flush=True)
    q, k, v, g = workloads.qkv(w, "qkvg")
    order = OR.layout_order(w.n, P, "striped")
    qs, ks, vs = (ra.permute(t.cuda(), P) for t in (q, k, v))
    dout = g[:, :, torch.from_numpy(order[p * c:(p + 1) * c])].contiguous().cuda()
    del g
    o, lse = ra.forward(qs, ks, vs, P, "striped", True, p_begin=p, p_end=p + 1)
    dq, dk, dv = ra.backward(qs, ks, vs, dout, lse, P, "striped", True, p, p + 1, o=o)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(dq).all()) and bool(torch.isfinite(dk).all()) and bool(torch.isfinite(dv).all())
    qd = qs[:, :, p * c:(p + 1) * c].double()
    assert float((dk.double().sum(2).abs() / dk.double().abs().sum(2)).max()) <= 1e-2
    assert float(((dv.double().sum(2) - dout.double().sum(2)).abs() / dout.double().abs().sum(2)).max()) <= 1e-2
    lhs = (qd * dq.double()).sum((2, 3))
    rhs = (ks.double() * dk.double()).sum((2, 3))
    assert float(((lhs - rhs).abs() / (qd * dq.double()).abs().sum((2, 3))).max()) <= 1e-2
    del qd, dk, dv, qs, ks, vs
    rows = _sample_rows(c, k=10)
    tokens = order[p * c + rows]
    t = torch.from_numpy(tokens)
    for h in (0, 5):
        ref, _, _ = OB.grads(q[0, h, t], k[0, h], v[0, h], dout[0, h, torch.from_numpy(rows).cuda()].cpu(),
                             True, tokens, np.arange(w.n))
        compare_grad(_sel(dq, [h], rows)[0], ref, "bf16", f"stress1m dQ head {h}")
    del dq, dout, o, lse
    torch.cuda.empty_cache()


def test_stress1m_streamed_rounds_and_merge(ra):
    w = workloads.get("stress_n1m")
    P, c, p = w.P, w.c, w.device
    print(f"[fullsize] generating {w.name}", flush=True)
    q, k, v = (t.cuda() for t in workloads.qkv(w))
    qs, ks, vs = (ra.permute(t, P) for t in (q, k, v))
    del q, k, v
    acc_o = torch.zeros((w.B, w.H, c, w.d), dtype=torch.float32, device="cuda")
    acc_l = torch.full((w.B, w.H, c), float("-inf"), device="cuda")
    tq, tk = ra.tile_shape(ra.BF16, w.d)
    exp_stats = _expected_stats_row("striped", P, c, p, w.B * w.H, tq, tk)
    for r in range(P):
        kk = OR.kv_block(p, r, P)
        st = torch.zeros(4, dtype=torch.int64, device="cuda")
        po, pl = ra.round(qs[:, :, p * c:(p + 1) * c], ks[:, :, kk * c:(kk + 1) * c], vs[:, :, kk * c:(kk + 1) * c],
                          P, p, kk, "striped", True, stats=st)
        ra.merge(acc_o, acc_l, po, pl)
        assert st.cpu().numpy().tolist() == exp_stats[r].tolist(), r
    o_f, l_f = ra.forward(qs, ks, vs, P, "striped", True, p_begin=p, p_end=p + 1, o_dtype=torch.float32)
    torch.cuda.synchronize()
    del qs, ks, vs
    order = OR.layout_order(w.n, P, "striped")
    rows = _sample_rows(c, k=26)
    heads = [0, 3, 7]
    tokens = order[p * c + rows]
    o_ref, l_ref = _oracle_rows(w, heads, tokens)
    compare(_sel(acc_o, heads, rows), _sel(acc_l, heads, rows), o_ref, l_ref, "bf16", "stress1m streamed")
    compare(_sel(o_f, heads, rows), _sel(l_f, heads, rows), o_ref, l_ref, "bf16", "stress1m fused")
    assert float((acc_o - o_f).abs().max()) <= 2e-2
    assert float((acc_l - l_f).abs().max()) <= 1e-3
    del acc_o, acc_l, o_f, l_f
    torch.cuda.empty_cache()
