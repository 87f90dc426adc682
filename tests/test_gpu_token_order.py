"""GPU parity of the token-order striped layout (RA_STRIPED_TOKENS) of ra_forward and ra_backward.

The partition, ring schedule and GetMask are those of the striped layout (Striped Attention
review, "分区策略对比" and "GetMask 函数"); only the addressing differs: the kernels read and write
row y of device p's block at token y*P + p of token-order tensors, so no permutation pass runs.
Checked here:
* against the fp64 oracle's attention in token order (natural positions), element by element,
  at sizes that span several tiles and a ragged tail, for bf16 and f32 inputs;
* bit-exact against the permuted path (ra_permute, ra_forward on RA_STRIPED, inverse ra_permute
  of O and LSE): both run the same arithmetic in the same order on the same values;
* the work counters equal the striped layout's closed forms;
* a device range writes only its own rows (token t with p_begin <= t mod P < p_end);
* the backward: gradients against the oracle's fp64 autograd in token order, and bit-exact
  against the permuted path (permute, backward on RA_STRIPED, inverse permute of dQ, dK, dV).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads
from oracle import attention as OA
from oracle import backward as OB
from oracle import ring as OR
from tests._gpu_util import compare, compare_grad, need_gpu, np64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ra():
    need_gpu()
    import striped_blockwise_amd as m
    return m


def _expected_stats(P, c, BH, causal, tq, tk, devices):
    exp = np.zeros((P, P, 4), dtype=np.int64)
    for p in devices:
        for r in range(P):
            kk = OR.kv_block(p, r, P)
            pairs = OR.work_closed_form("striped", p, kk, c, causal)
            full, diag, skip = OR.tile_counts_closed_form("striped", p, kk, c, tq, tk, causal)
            exp[p, r] = [pairs * BH, full * BH, diag * BH, skip * BH]
    return exp


def _permuted_path(ra, q, k, v, P, causal, o_dtype):
    qs, ks, vs = (ra.permute(t, P) for t in (q, k, v))
    o, lse = ra.forward(qs, ks, vs, P, "striped", causal, o_dtype=o_dtype)
    return ra.permute(o, P, inverse=True), ra.permute(lse, P, dim=-1, inverse=True)


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 64), (torch.float32, 128)])
@pytest.mark.parametrize("P,c", [(4, 1), (4, 37), (8, 200), (3, 512), (1, 300), (64, 1)])
def test_token_order_matches_oracle(ra, dtype, d, P, c):
    B, H = 1, 2
    n = P * c
    g = torch.Generator().manual_seed(1000 + 7 * c + P + d)
    q, k, v = (torch.randn((B, H, n, d), generator=g).mul(0.5).to(dtype) for _ in range(3))
    o_ref, l_ref = OA.attention(q, k, v, True)                     # token order, positions 0..n-1
    kind = "f32" if dtype == torch.float32 else "bf16"
    qg, kg, vg = (t.cuda() for t in (q, k, v))
    stats = ra.new_stats(P)
    o, lse = ra.forward(qg, kg, vg, P, "striped_tokens", True, o_dtype=torch.float32, stats=stats)
    torch.cuda.synchronize()
    compare(o, lse, o_ref, l_ref, kind, f"token order P={P} c={c} {dtype}")
    tq, tk = ra.tile_shape(ra.F32 if kind == "f32" else ra.BF16, d)
    assert np.array_equal(stats.cpu().numpy(), _expected_stats(P, c, B * H, True, tq, tk, range(P)))
    o_p, l_p = _permuted_path(ra, qg, kg, vg, P, True, torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o, o_p) and torch.equal(lse, l_p), "token order differs from the permuted path"


def test_token_order_seq8k_bf16(ra):
    w = workloads.get("seq_n8k")
    q, k, v = workloads.qkv(w)
    o_ref, l_ref = OA.attention(q, k, v, True)
    qg, kg, vg = (t.cuda() for t in (q, k, v))
    for o_dtype in (torch.float32, torch.bfloat16):
        o, lse = ra.forward(qg, kg, vg, w.P, "striped_tokens", True, o_dtype=o_dtype)
        torch.cuda.synchronize()
        compare(o.float(), lse, o_ref, l_ref, "bf16", f"seq8k token order, {o_dtype} out")
        o_p, l_p = _permuted_path(ra, qg, kg, vg, w.P, True, o_dtype)
        torch.cuda.synchronize()
        assert torch.equal(o, o_p) and torch.equal(lse, l_p)


@pytest.mark.parametrize("P,c", [(4, 100), (64, 1)])
def test_token_order_not_causal(ra, P, c):
    """Unmasked rounds in token order.  With P = 64 and c = 1 every round has one key tile, so
    three of the four key splits of the small-grid workgroups own none while their rows lie 64
    tokens apart: a split must not fetch a tile it does not own (it would start past the
    block)."""
    H = 2
    g = torch.Generator().manual_seed(77 + P)
    q, k, v = (torch.randn((1, H, P * c, 128), generator=g).to(torch.bfloat16) for _ in range(3))
    o_ref, l_ref = OA.attention(q, k, v, False)
    o, lse = ra.forward(q.cuda(), k.cuda(), v.cuda(), P, "striped_tokens", False, o_dtype=torch.float32)
    torch.cuda.synchronize()
    compare(o, lse, o_ref, l_ref, "bf16", f"token order, no mask, P={P} c={c}")


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_token_order_device_range_writes_only_its_rows(ra, dtype, d):
    P, c, H = 4, 130, 2
    n = P * c
    g = torch.Generator().manual_seed(5 + d)
    q, k, v = (torch.randn((1, H, n, d), generator=g).to(dtype) for _ in range(3))
    o_ref, l_ref = OA.attention(q, k, v, True)
    kind = "f32" if dtype == torch.float32 else "bf16"
    o = torch.full((1, H, n, d), float("nan"), device="cuda")
    lse = torch.full((1, H, n), float("nan"), device="cuda")
    stats = ra.new_stats(P)
    ra.forward(q.cuda(), k.cuda(), v.cuda(), P, "striped_tokens", True, p_begin=1, p_end=3,
               o_dtype=torch.float32, stats=stats, out=(o, lse))
    torch.cuda.synchronize()
    mine = np.isin(np.arange(n) % P, [1, 2])
    on, ln = np64(o), np64(lse)
    assert np.isnan(on[:, :, ~mine]).all() and np.isnan(ln[:, :, ~mine]).all(), "rows of other devices written"
    compare(on[:, :, mine], ln[:, :, mine], o_ref[:, :, mine], l_ref[:, :, mine], kind, "device range 1..3")
    tq, tk = ra.tile_shape(ra.F32 if kind == "f32" else ra.BF16, d)
    assert np.array_equal(stats.cpu().numpy(), _expected_stats(P, c, H, True, tq, tk, [1, 2]))
    # out=None allocates zeros for the rows outside the range
    o2, l2 = ra.forward(q.cuda(), k.cuda(), v.cuda(), P, "striped_tokens", True, p_begin=1, p_end=3,
                        o_dtype=torch.float32)
    torch.cuda.synchronize()
    assert not np64(o2)[:, :, ~mine].any() and not np64(l2)[:, :, ~mine].any()
    assert torch.equal(o2[:, :, torch.from_numpy(mine).cuda()], o[:, :, torch.from_numpy(mine).cuda()])


def test_token_order_rejected_where_unsupported(ra):
    x = torch.zeros((1, 1, 256, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(NotImplementedError, match="layout order"):
        ra.round(x[:, :, :64], x[:, :, :64], x[:, :, :64], 4, 1, 0, "striped_tokens", True)
    o = torch.empty((1, 1, 128, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="out\\[0\\]"):                     # o must hold all n rows
        ra.forward(x, x, x, 4, "striped_tokens", True, p_begin=0, p_end=2, out=(o, None))


# --------------------------------------------------------------------------- backward
def _grads_via_permutes(ra, q, k, v, g, P, causal):
    """The permuted path: ra_permute, forward and backward on RA_STRIPED, gradients back to token
    order with the inverse permutation."""
    qs, ks, vs, gs = (ra.permute(t, P) for t in (q, k, v, g))
    o, lse = ra.forward(qs, ks, vs, P, "striped", causal)
    dq, dk, dv = ra.backward(qs, ks, vs, gs, lse, P, "striped", causal, o=o)
    return tuple(ra.permute(t, P, inverse=True) for t in (dq, dk, dv))


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 64)])
@pytest.mark.parametrize("P,c", [(4, 37), (8, 200), (3, 512), (1, 96), (64, 2)])
def test_token_order_backward_matches_oracle(ra, dtype, d, P, c):
    B, H = 1, 2
    n = P * c
    gen = torch.Generator().manual_seed(3000 + 11 * c + P + d)
    q, k, v, g = (torch.randn((B, H, n, d), generator=gen).mul(0.5 if i < 3 else 1.0).to(dtype) for i in range(4))
    ref = OB.attention_grads(q, k, v, g, True)                   # token order, positions 0..n-1
    kind = "f32" if dtype == torch.float32 else "bf16"
    qg, kg, vg, gg = (t.cuda() for t in (q, k, v, g))
    o, lse = ra.forward(qg, kg, vg, P, "striped_tokens", True)
    got = ra.backward(qg, kg, vg, gg, lse, P, "striped_tokens", True, o=o)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        compare_grad(a, b, kind, f"token order P={P} c={c} {name}")
    via = _grads_via_permutes(ra, qg, kg, vg, gg, P, True)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, via):
        assert torch.equal(a, b), f"token-order {name} differs from the permuted path"


def test_token_order_backward_device_range(ra):
    """Devices 1..2 of 4: dq only on their rows (others untouched), dk and dv everywhere, equal to
    the oracle's gradient of those queries' loss."""
    P, c, H, d = 4, 130, 2, 128
    n = P * c
    gen = torch.Generator().manual_seed(41)
    q, k, v, g = (torch.randn((1, H, n, d), generator=gen).to(torch.bfloat16) for _ in range(4))
    mine = np.isin(np.arange(n) % P, [1, 2])
    sel = torch.from_numpy(np.nonzero(mine)[0])
    ref = OB.attention_grads(q[:, :, sel], k, v, g[:, :, sel], True, pos_q=sel.numpy(), pos_k=np.arange(n))
    qg, kg, vg, gg = (t.cuda() for t in (q, k, v, g))
    o, lse = ra.forward(qg, kg, vg, P, "striped_tokens", True, p_begin=1, p_end=3)
    dq = torch.full((1, H, n, d), float("nan"), device="cuda")
    dk = torch.empty((1, H, n, d), device="cuda")
    dv = torch.empty((1, H, n, d), device="cuda")
    ra.backward(qg, kg, vg, gg, lse, P, "striped_tokens", True, 1, 3, o=o, out=(dq, dk, dv))
    torch.cuda.synchronize()
    dqn = np64(dq)
    assert np.isnan(dqn[:, :, ~mine]).all(), "dq rows of other devices written"
    compare_grad(dqn[:, :, mine], ref[0], "bf16", "range dq")
    compare_grad(dk, ref[1], "bf16", "range dk")
    compare_grad(dv, ref[2], "bf16", "range dv")


@pytest.mark.parametrize("layout", ["contiguous", "striped", "striped_tokens"])
def test_batch_of_two_forward_and_backward(ra, layout):
    """B = 2, H = 3: the kernels flatten (b, h) into one stride; every (b, h) matrix must match."""
    B, H, P, c, d = 2, 3, 4, 70, 128
    n = P * c
    gen = torch.Generator().manual_seed(555)
    q, k, v, g = (torch.randn((B, H, n, d), generator=gen).mul(0.5 if i < 3 else 1.0).to(torch.bfloat16)
                  for i in range(4))
    o_ref, l_ref = OA.attention(q, k, v, True)
    dq_ref, dk_ref, dv_ref = OB.attention_grads(q, k, v, g, True)
    order = OR.layout_order(n, P, "striped" if layout == "striped" else "contiguous")
    idx = torch.from_numpy(order)
    to_l = (lambda t: t[:, :, idx].contiguous()) if layout == "striped" else (lambda t: t)
    qg, kg, vg, gg = (to_l(t).cuda() for t in (q, k, v, g))
    o, lse = ra.forward(qg, kg, vg, P, layout, True, o_dtype=torch.float32)
    dq, dk, dv = ra.backward(qg, kg, vg, gg, lse, P, layout, True, o=o)
    torch.cuda.synchronize()
    back = (lambda t: t[:, :, torch.from_numpy(np.argsort(order))]) if layout == "striped" else (lambda t: t)
    compare(back(o.cpu()), back(lse.cpu()), o_ref, l_ref, "bf16", f"B=2 {layout}")
    for name, got, ref in (("dq", dq, dq_ref), ("dk", dk, dk_ref), ("dv", dv, dv_ref)):
        compare_grad(back(got.cpu()), ref, "bf16", f"B=2 {layout} {name}")
