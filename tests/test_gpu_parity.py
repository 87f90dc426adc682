"""GPU parity: libra.so (through the C ABI) against the fp64 CPU oracle, element by element.

Integer outputs (permutations, position IDs, work counters) must be bit-exact; floating-point
outputs must meet the tolerances in tests/_gpu_util.py on the same rounded inputs.
"""
from __future__ import annotations

import itertools

import numpy as np
import pytest
import torch

import workloads
from oracle import attention as OA
from oracle import ring as OR
from tests._gpu_util import compare, need_gpu, np64

pytestmark = pytest.mark.gpu

LAYOUTS = ["contiguous", "striped"]


@pytest.fixture(scope="module")
def ra():
    need_gpu()
    import striped_blockwise_amd as m
    return m


def _oracle_layout(w_or_tensors, P, layout):
    """Inputs in layout order for the oracle (numpy fp64) plus the layout order."""
    q, k, v = w_or_tensors
    n = q.shape[2]
    order = OR.layout_order(n, P, layout)
    return [OR.to_layout(np64(t), order) for t in (q, k, v)], order


def _expected_stats(layout, P, c, BH, causal, tq, tk, devices=None, rounds=None):
    exp = np.zeros((P, P, 4), dtype=np.int64)
    for p in (range(P) if devices is None else devices):
        for r in (range(P) if rounds is None else rounds):
            kk = OR.kv_block(p, r, P)
            pairs = OR.work_closed_form(layout, p, kk, c, causal)
            full, diag, skip = OR.tile_counts_closed_form(layout, p, kk, c, tq, tk, causal)
            exp[p, r] = [pairs * BH, full * BH, diag * BH, skip * BH]
    return exp


# --------------------------------------------------------------------------- permutation
@pytest.mark.parametrize("B,H,n,P,d,dtype", [
    (1, 8, 8192, 4, 128, torch.bfloat16), (2, 3, 96, 8, 64, torch.float32),
    (1, 1, 64, 64, 128, torch.bfloat16), (1, 2, 30, 3, 6, torch.float32), (1, 1, 16, 1, 8, torch.bfloat16)])
def test_permute_bit_exact(ra, B, H, n, P, d, dtype):
    x = torch.randn((B, H, n, d), generator=torch.Generator().manual_seed(n + P)).to(dtype)
    xg = x.cuda()
    order = torch.from_numpy(OR.layout_order(n, P, "striped"))
    y = ra.permute(xg, P)
    torch.cuda.synchronize()
    assert torch.equal(y.cpu(), x[:, :, order]), "forward permutation"
    z = ra.permute(y, P, inverse=True)
    torch.cuda.synchronize()
    assert torch.equal(z.cpu(), x), "inverse permutation"


def test_permute_ids_and_lse_rows(ra):
    n, P = 8192, 4
    ids = workloads.positions(n)
    order = torch.from_numpy(OR.layout_order(n, P, "striped"))
    got = ra.permute_ids(ids.cuda(), P)
    torch.cuda.synchronize()
    assert torch.equal(got.cpu(), ids[order])
    assert torch.equal(ra.permute_ids(got, P, inverse=True).cpu(), ids)
    lse = torch.randn((2, 8, n), generator=torch.Generator().manual_seed(5))       # 4-byte rows
    got = ra.permute(lse.cuda(), P, dim=-1)
    torch.cuda.synchronize()
    assert torch.equal(got.cpu(), lse[:, :, order])


# --------------------------------------------------------------------------- tiny fp32
@pytest.fixture(scope="module")
def tiny():
    w = workloads.get("tiny_n256")
    return w, workloads.qkv(w)


@pytest.mark.parametrize("layout,causal", [("contiguous", False), ("contiguous", True), ("striped", True)])
def test_tiny_f32_every_round(ra, tiny, layout, causal):
    w, (q, k, v) = tiny
    P, c = w.P, w.c
    (ql, kl, vl), order = _oracle_layout((q, k, v), P, layout)
    qg, kg, vg = (ra.permute(t.cuda(), P) if layout == "striped" else t.cuda() for t in (q, k, v))
    tq, tk = ra.tile_shape(ra.F32, w.d)
    for p, r in itertools.product(range(P), range(P)):
        kk = OR.kv_block(p, r, P)
        stats = torch.zeros(4, dtype=torch.int64, device="cuda")
        o, lse = ra.round(qg[:, :, p * c:(p + 1) * c], kg[:, :, kk * c:(kk + 1) * c],
                          vg[:, :, kk * c:(kk + 1) * c], P, p, kk, layout, causal, stats=stats)
        torch.cuda.synchronize()
        o_ref, l_ref = OR.round_partial(ql[0, 0, p * c:(p + 1) * c], kl[0, 0, kk * c:(kk + 1) * c],
                                        vl[0, 0, kk * c:(kk + 1) * c], layout, p, kk, causal)
        compare(o[0, 0], lse[0, 0], o_ref, l_ref, "f32", f"round p={p} r={r}")
        exp = _expected_stats(layout, P, c, 1, causal, tq, tk, [p], [r])[p, r]
        assert stats.cpu().numpy().tolist() == exp.tolist(), (p, r)


@pytest.mark.parametrize("layout,causal", [("contiguous", False), ("contiguous", True), ("striped", True)])
def test_tiny_f32_forward_and_stream(ra, tiny, layout, causal):
    w, (q, k, v) = tiny
    P, c = w.P, w.c
    (ql, kl, vl), order = _oracle_layout((q, k, v), P, layout)
    o_ref, l_ref = OA.attention(ql, kl, vl, causal, pos_q=order, pos_k=order)
    qg, kg, vg = (ra.permute(t.cuda(), P) if layout == "striped" else t.cuda() for t in (q, k, v))
    stats = ra.new_stats(P)
    o, lse = ra.forward(qg, kg, vg, P, layout, causal, stats=stats)
    torch.cuda.synchronize()
    compare(o, lse, o_ref, l_ref, "f32", "forward")
    tq, tk = ra.tile_shape(ra.F32, w.d)
    assert np.array_equal(stats.cpu().numpy(), _expected_stats(layout, P, c, 1, causal, tq, tk))
    # streamed: every round through ra_round, merged with ra_merge, per device
    for p in range(P):
        acc_o = torch.zeros((1, 1, c, w.d), dtype=torch.float32, device="cuda")
        acc_l = torch.full((1, 1, c), float("-inf"), device="cuda")
        for r in range(P):
            kk = OR.kv_block(p, r, P)
            po, pl = ra.round(qg[:, :, p * c:(p + 1) * c], kg[:, :, kk * c:(kk + 1) * c],
                              vg[:, :, kk * c:(kk + 1) * c], P, p, kk, layout, causal)
            ra.merge(acc_o, acc_l, po, pl)
        torch.cuda.synchronize()
        compare(acc_o, acc_l, o_ref[:, :, p * c:(p + 1) * c], l_ref[:, :, p * c:(p + 1) * c], "f32",
                f"stream p={p}")


def test_tiny_f32_bf16_output(ra, tiny):
    w, (q, k, v) = tiny
    o_ref, _ = OA.attention(q, k, v, True)
    o, _ = ra.forward(q.cuda(), k.cuda(), v.cuda(), w.P, "contiguous", True, o_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16
    # one bf16 rounding of the output: relative 2^-8 of |O| <= 4
    assert np.abs(np64(o) - o_ref).max() <= 4 * 2.0 ** -8


# --------------------------------------------------------------------------- bf16, 8K tokens
@pytest.fixture(scope="module")
def seq8k():
    w = workloads.get("seq_n8k")
    q, k, v = workloads.qkv(w)
    refs = {}
    for layout in LAYOUTS:
        (ql, kl, vl), order = _oracle_layout((q, k, v), w.P, layout)
        refs[layout] = OA.attention(ql, kl, vl, True, pos_q=order, pos_k=order) + (order,)
    return w, (q, k, v), refs


@pytest.mark.parametrize("layout", LAYOUTS)
def test_bf16_seq8k_forward(ra, seq8k, layout):
    w, (q, k, v), refs = seq8k
    o_ref, l_ref, order = refs[layout]
    qg, kg, vg = (ra.permute(t.cuda(), w.P) if layout == "striped" else t.cuda() for t in (q, k, v))
    stats = ra.new_stats(w.P)
    o, lse = ra.forward(qg, kg, vg, w.P, layout, True, o_dtype=torch.float32, stats=stats)
    torch.cuda.synchronize()
    compare(o, lse, o_ref, l_ref, "bf16", f"forward {layout}")
    tq, tk = ra.tile_shape(ra.BF16, w.d)
    assert np.array_equal(stats.cpu().numpy(), _expected_stats(layout, w.P, w.c, w.B * w.H, True, tq, tk))
    o16, lse16 = ra.forward(qg, kg, vg, w.P, layout, True)              # bf16 output
    torch.cuda.synchronize()
    compare(o16, lse16, o_ref, l_ref, "bf16", f"forward {layout} bf16 out")


def test_bf16_seq8k_striped_unpermuted_equals_contiguous(ra, seq8k):
    w, (q, k, v), refs = seq8k
    qg, kg, vg = (t.cuda() for t in (q, k, v))
    o_c, l_c = ra.forward(qg, kg, vg, w.P, "contiguous", True, o_dtype=torch.float32)
    qs, ks, vs = (ra.permute(t, w.P) for t in (qg, kg, vg))
    o_s, l_s = ra.forward(qs, ks, vs, w.P, "striped", True, o_dtype=torch.float32)
    o_u = ra.permute(o_s, w.P, inverse=True)
    l_u = ra.permute(l_s, w.P, dim=-1, inverse=True)
    torch.cuda.synchronize()
    o_ref, l_ref, _ = refs["contiguous"]
    compare(o_u, l_u, o_ref, l_ref, "bf16", "striped un-permuted vs oracle")
    assert float((o_u - o_c).abs().max()) <= 2e-2
    assert float((l_u - l_c).abs().max()) <= 1e-3


@pytest.mark.parametrize("layout", LAYOUTS)
def test_bf16_seq8k_rounds_and_merge(ra, seq8k, layout):
    w, (q, k, v), refs = seq8k
    P, c = w.P, w.c
    o_ref, l_ref, order = refs[layout]
    (ql, kl, vl), _ = _oracle_layout((q[:, :2], k[:, :2], v[:, :2]), P, layout)
    qg, kg, vg = (ra.permute(t.cuda(), P) if layout == "striped" else t.cuda() for t in (q, k, v))
    tq, tk = ra.tile_shape(ra.BF16, w.d)
    for p in range(P):
        acc_o = torch.zeros((w.B, w.H, c, w.d), dtype=torch.float32, device="cuda")
        acc_l = torch.full((w.B, w.H, c), float("-inf"), device="cuda")
        for r in range(P):
            kk = OR.kv_block(p, r, P)
            stats = torch.zeros(4, dtype=torch.int64, device="cuda")
            po, pl = ra.round(qg[:, :, p * c:(p + 1) * c], kg[:, :, kk * c:(kk + 1) * c],
                              vg[:, :, kk * c:(kk + 1) * c], P, p, kk, layout, True, stats=stats)
            torch.cuda.synchronize()
            exp = _expected_stats(layout, P, c, w.B * w.H, True, tq, tk, [p], [r])[p, r]
            assert stats.cpu().numpy().tolist() == exp.tolist(), (p, r)
            if p in (0, P - 1):             # element check of the round partial on 2 heads
                for h in range(2):
                    ro, rl = OR.round_partial(ql[0, h, p * c:(p + 1) * c], kl[0, h, kk * c:(kk + 1) * c],
                                              vl[0, h, kk * c:(kk + 1) * c], layout, p, kk, True)
                    compare(po[0, h], pl[0, h], ro, rl, "bf16", f"round p={p} r={r} h={h}")
            ra.merge(acc_o, acc_l, po, pl)
        torch.cuda.synchronize()
        compare(acc_o, acc_l, o_ref[:, :, p * c:(p + 1) * c], l_ref[:, :, p * c:(p + 1) * c], "bf16",
                f"streamed p={p}")


# --------------------------------------------------------------------------- edge cases
@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 64)])
@pytest.mark.parametrize("c", [1, 2, 37, 200])
@pytest.mark.parametrize("layout,causal", [("contiguous", True), ("striped", True), ("contiguous", False)])
def test_ragged_blocks(ra, dtype, d, c, layout, causal):
    P, B, H = 4, 1, 2
    n = P * c
    g = torch.Generator().manual_seed(c * 7 + d)
    q, k, v = (torch.randn((B, H, n, d), generator=g).mul(0.5).to(dtype) for _ in range(3))
    (ql, kl, vl), order = _oracle_layout((q, k, v), P, layout)
    o_ref, l_ref = OA.attention(ql, kl, vl, causal, pos_q=order, pos_k=order)
    kind = "f32" if dtype == torch.float32 else "bf16"
    qg, kg, vg = (ra.permute(t.cuda(), P) if layout == "striped" else t.cuda() for t in (q, k, v))
    stats = ra.new_stats(P)
    o, lse = ra.forward(qg, kg, vg, P, layout, causal, o_dtype=torch.float32, stats=stats)
    torch.cuda.synchronize()
    compare(o, lse, o_ref, l_ref, kind, f"ragged c={c}")
    tq, tk = ra.tile_shape(ra.F32 if kind == "f32" else ra.BF16, d)
    assert np.array_equal(stats.cpu().numpy(), _expected_stats(layout, P, c, B * H, causal, tq, tk))
    # one round with empty rows (striped, later device: query row 0 sees no key)
    p, kk = 1, 3
    o_r, l_r = ra.round(qg[:, :, p * c:(p + 1) * c], kg[:, :, kk * c:(kk + 1) * c], vg[:, :, kk * c:(kk + 1) * c],
                        P, p, kk, layout, causal)
    torch.cuda.synchronize()
    for h in range(H):
        ro, rl = OR.round_partial(ql[0, h, p * c:(p + 1) * c], kl[0, h, kk * c:(kk + 1) * c],
                                  vl[0, h, kk * c:(kk + 1) * c], layout, p, kk, causal)
        compare(o_r[0, h], l_r[0, h], ro, rl, kind, f"ragged round c={c} h={h}")


def test_single_device_and_one_token_blocks(ra):
    for P, n in ((1, 300), (64, 64)):
        q, k, v = (torch.randn((1, 1, n, 128), generator=torch.Generator().manual_seed(P + i)).to(torch.bfloat16)
                   for i in range(3))
        o_ref, l_ref = OA.attention(q, k, v, True)
        for layout in LAYOUTS:
            order = OR.layout_order(n, P, layout)
            qg, kg, vg = (ra.permute(t.cuda(), P) if layout == "striped" else t.cuda() for t in (q, k, v))
            o, lse = ra.forward(qg, kg, vg, P, layout, True, o_dtype=torch.float32)
            o = ra.permute(o, P, inverse=True) if layout == "striped" else o
            lse = ra.permute(lse, P, dim=-1, inverse=True) if layout == "striped" else lse
            torch.cuda.synchronize()
            compare(o, lse, o_ref, l_ref, "bf16", f"P={P} n={n} {layout}")
            del order


def test_empty_problems_are_noops(ra):
    z = torch.empty((1, 2, 0, 128), dtype=torch.bfloat16, device="cuda")
    o, lse = ra.forward(z, z, z, 4, "striped", True)
    assert o.numel() == 0
    zb = torch.empty((0, 2, 64, 128), dtype=torch.bfloat16, device="cuda")
    o, lse = ra.forward(zb, zb, zb, 4, "contiguous", True)
    assert o.numel() == 0
    torch.cuda.synchronize()


def test_sharp_scores_and_determinism(ra):
    # large-magnitude scores (std ~ 8) stress the running-max rescale
    n, P, H = 2048, 4, 2
    g = torch.Generator().manual_seed(11)
    q, k, v = (torch.randn((1, H, n, 128), generator=g).mul(s).to(torch.bfloat16) for s in (3.0, 3.0, 1.0))
    o_ref, l_ref = OA.attention(q, k, v, True)
    qg, kg, vg = (t.cuda() for t in (q, k, v))
    o1, l1 = ra.forward(qg, kg, vg, P, "contiguous", True, o_dtype=torch.float32)
    o2, l2 = ra.forward(qg, kg, vg, P, "contiguous", True, o_dtype=torch.float32)
    torch.cuda.synchronize()
    compare(o1, l1, o_ref, l_ref, "bf16", "sharp")
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "run-to-run results differ"


def test_output_guard_bands_untouched(ra):
    n, P, H, c = 1024, 4, 2, 256
    g = torch.Generator().manual_seed(12)
    q, k, v = (torch.randn((1, H, n, 128), generator=g).to(torch.bfloat16).cuda() for _ in range(3))
    for h in range(H):                      # per head, into NaN-guarded buffers
        buf = torch.full((3 * c * 128 + 2 * 4096,), float("nan"), device="cuda")
        oh = buf[4096:4096 + 3 * c * 128].view(1, 1, 3 * c, 128)
        lbuf = torch.full((3 * c + 64,), float("nan"), device="cuda")
        lh = lbuf[32:32 + 3 * c].view(1, 1, 3 * c)
        ra.forward(q[:, h:h + 1].contiguous(), k[:, h:h + 1].contiguous(), v[:, h:h + 1].contiguous(),
                   P, "contiguous", True, p_begin=1, p_end=4, o_dtype=torch.float32, out=(oh, lh))
        torch.cuda.synchronize()
        assert torch.isnan(buf[:4096]).all() and torch.isnan(buf[4096 + 3 * c * 128:]).all()
        assert torch.isnan(lbuf[:32]).all() and torch.isnan(lbuf[32 + 3 * c:]).all()
        assert torch.isfinite(oh).all() and torch.isfinite(lh).all()


def test_invalid_arguments_raise_before_launch(ra):
    q = torch.zeros((1, 1, 100, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        ra.forward(q, q, q, 3, "striped", True)                  # n % P != 0
    with pytest.raises(NotImplementedError):
        x = torch.zeros((1, 1, 64, 96), dtype=torch.bfloat16, device="cuda")
        ra.forward(x, x, x, 4, "contiguous", True)               # unsupported head dim
    with pytest.raises(ValueError):
        ra.forward(q, q, q, 4, "contiguous", True, p_begin=3, p_end=3)


def test_wrong_outputs_raise_before_launch(ra):
    """Caller-provided outputs whose shape, dtype or device differ from what the kernels write are
    refused on the host (the library sizes its writes from the problem, not from the buffers)."""
    n, P, d = 256, 4, 128
    c = n // P
    q = torch.zeros((1, 2, n, d), dtype=torch.bfloat16, device="cuda")
    small = torch.empty((1, 2, c - 1, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, 2, c), device="cuda")
    with pytest.raises(ValueError, match="out\\[0\\]"):
        ra.forward(q, q, q, P, "striped", True, p_begin=1, p_end=2, out=(small, lse))
    with pytest.raises(ValueError, match="out\\[1\\]"):
        ra.forward(q, q, q, P, "striped", True, p_begin=1, p_end=2,
                   out=(torch.empty((1, 2, c, d), dtype=torch.bfloat16, device="cuda"), lse[:, :, :-1]))
    with pytest.raises(ValueError, match="stats"):
        ra.forward(q, q, q, P, "striped", True, stats=torch.zeros((P, P, 4), dtype=torch.int64))     # on the CPU
    blk = q[:, :, :c]
    with pytest.raises(ValueError, match="out\\[0\\]"):
        ra.round(blk, blk, blk, P, 1, 0, "striped", True,
                 out=(torch.empty((1, 2, c, d), dtype=torch.bfloat16, device="cuda"), lse))   # o must be f32
    with pytest.raises(ValueError, match="out"):
        ra.permute_ids(torch.arange(n, device="cuda"), P, out=torch.empty(n - 1, dtype=torch.int64, device="cuda"))
    o = torch.zeros((1, 2, c, d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="out"):
        ra.bwd_delta(o, o, out=torch.empty((1, 2, c)))                                             # on the CPU
    dq = torch.empty((1, 2, c, d), device="cuda")
    dkv = torch.empty((1, 2, n, d), device="cuda")
    with pytest.raises(ValueError, match="dk"):
        ra.backward(q, q, q, o, lse, P, "striped", True, 1, 2, delta=lse, out=(dq, dkv[:, :, :-1], dkv))
    with pytest.raises(ValueError, match="dq_acc"):
        ra.backward_round(blk, blk, blk, blk, lse, lse, P, 1, 0, "striped", True,
                          grads=(dq[:, :1], dq, dq))
    torch.cuda.synchronize()


@pytest.mark.parametrize("layout", ["contiguous", "striped", "striped_tokens"])
def test_wide_workgroup_path(ra, layout):
    """A grid large enough for the 12-wave workgroups (at least two per CU: 128 heads x 2 devices
    x 4 query tiles of 384 rows), with ragged query and key tiles (c = 1500).  Element-wise on 8
    heads against the oracle, counters on all of them, and one round per direction."""
    B, H, P, c, d = 1, 128, 2, 1500, 128
    n = P * c
    g = torch.Generator().manual_seed(2024)
    q, k, v = (torch.randn((B, H, n, d), generator=g).mul(0.5).to(torch.bfloat16) for _ in range(3))
    heads = [0, 1, 2, 3, 124, 125, 126, 127]
    base = "striped" if layout == "striped_tokens" else layout
    qh, kh, vh = (t[:, heads] for t in (q, k, v))
    if layout == "striped_tokens":
        o_ref, l_ref = OA.attention(qh, kh, vh, True)
    else:
        (ql, kl, vl), order = _oracle_layout((qh, kh, vh), P, layout)
        o_ref, l_ref = OA.attention(ql, kl, vl, True, pos_q=order, pos_k=order)
    qg, kg, vg = (ra.permute(t.cuda(), P) if layout == "striped" else t.cuda() for t in (q, k, v))
    stats = ra.new_stats(P)
    o, lse = ra.forward(qg, kg, vg, P, layout, True, o_dtype=torch.float32, stats=stats)
    torch.cuda.synchronize()
    idx = torch.tensor(heads, device="cuda")
    compare(o.index_select(1, idx), lse.index_select(1, idx), o_ref, l_ref, "bf16", f"wide {layout}")
    tq, tk = ra.tile_shape(ra.BF16, d)
    assert np.array_equal(stats.cpu().numpy(), _expected_stats(base, P, c, B * H, True, tq, tk))
    if layout == "striped_tokens":
        return
    (ql, kl, vl), _ = _oracle_layout((qh, kh, vh), P, layout)
    for p, kk in ((1, 0), (0, 1), (1, 1)):
        po, pl = ra.round(qg[:, :, p * c:(p + 1) * c], kg[:, :, kk * c:(kk + 1) * c], vg[:, :, kk * c:(kk + 1) * c],
                          P, p, kk, layout, True)
        torch.cuda.synchronize()
        for j, h in enumerate(heads[::3]):
            jj = heads.index(h)
            ro, rl = OR.round_partial(ql[0, jj, p * c:(p + 1) * c], kl[0, jj, kk * c:(kk + 1) * c],
                                      vl[0, jj, kk * c:(kk + 1) * c], layout, p, kk, True)
            compare(po[0, h], pl[0, h], ro, rl, "bf16", f"wide round p={p} kv={kk} h={h}")


@pytest.mark.parametrize("H,P,c", [(2, 4, 1000), (64, 2, 600), (96, 2, 700)])
def test_small_grid_workgroup_shapes(ra, H, P, c):
    """Grids below two 12-wave workgroups per CU pick their workgroup shape by the number of
    32-row groups G in the launch; on a 256-CU device these three cases take 2 row groups x 4 key
    splits (G = 256; the striped launches and the contiguous diagonal round, whose row groups'
    work grows with their position, take the paired mode instead), 2 x 2 (G = 2432) and 4 row
    groups with three LDS stages (G = 4224), all with a ragged last tile.  The split workgroups merge their partial softmax states in LDS;
    element-wise against the oracle on three heads, counters on all, token-order tensors
    bit-identical to the permuted path, and one round per direction (whose single-device grids
    take the split shapes too)."""
    B, d = 1, 128
    n = P * c
    g = torch.Generator().manual_seed(4100 + H + c)
    q, k, v = (torch.randn((B, H, n, d), generator=g).mul(0.5).to(torch.bfloat16) for _ in range(3))
    heads = [0, 1, H - 1]
    qh, kh, vh = (t[:, heads] for t in (q, k, v))
    tq, tk = ra.tile_shape(ra.BF16, d)
    for layout in ("contiguous", "striped"):
        (ql, kl, vl), order = _oracle_layout((qh, kh, vh), P, layout)
        o_ref, l_ref = OA.attention(ql, kl, vl, True, pos_q=order, pos_k=order)
        qg, kg, vg = (ra.permute(t.cuda(), P) if layout == "striped" else t.cuda() for t in (q, k, v))
        stats = ra.new_stats(P)
        o, lse = ra.forward(qg, kg, vg, P, layout, True, o_dtype=torch.float32, stats=stats)
        torch.cuda.synchronize()
        idx = torch.tensor(heads, device="cuda")
        compare(o.index_select(1, idx), lse.index_select(1, idx), o_ref, l_ref, "bf16", f"H={H} c={c} {layout}")
        assert np.array_equal(stats.cpu().numpy(), _expected_stats(layout, P, c, B * H, True, tq, tk))
        if layout == "striped":
            # token-order tensors (rows P apart in every tile) take the same shape: bit-identical
            o_t, l_t = ra.forward(q.cuda(), k.cuda(), v.cuda(), P, "striped_tokens", True, o_dtype=torch.float32)
            torch.cuda.synchronize()
            assert torch.equal(o_t, ra.permute(o, P, inverse=True))
            assert torch.equal(l_t, ra.permute(lse, P, dim=-1, inverse=True))
        for p, kk in ((P - 1, 0), (0, P - 1), (P - 1, P - 1)):
            po, pl = ra.round(qg[:, :, p * c:(p + 1) * c], kg[:, :, kk * c:(kk + 1) * c], vg[:, :, kk * c:(kk + 1) * c],
                              P, p, kk, layout, True)
            torch.cuda.synchronize()
            for jj, h in enumerate(heads):
                ro, rl = OR.round_partial(ql[0, jj, p * c:(p + 1) * c], kl[0, jj, kk * c:(kk + 1) * c],
                                          vl[0, jj, kk * c:(kk + 1) * c], layout, p, kk, True)
                compare(po[0, h], pl[0, h], ro, rl, "bf16", f"H={H} c={c} {layout} round p={p} kv={kk} h={h}")


@pytest.mark.parametrize("H", [2, 128])          # split and 12-wave workgroups
def test_rising_scores_take_the_rescale_path(ra, H):
    """Scores that grow with the key position by about 3 log2 units per 32-key tile (more for
    some heads), so that the running reference falls behind again and again and the kernel's
    max-and-rescale path runs in the middle of the sweep, not only on a row's first tile."""
    B, P, c, d = 1, 2, 768, 128
    n = P * c
    g = torch.Generator().manual_seed(99)
    q = torch.randn((B, H, n, d), generator=g).mul(0.1)
    k = torch.randn((B, H, n, d), generator=g).mul(0.1)
    v = torch.randn((B, H, n, d), generator=g)
    rate = torch.linspace(0.5, 2.0, H).view(1, H, 1)           # per-head growth factor
    q[..., 0] = 8.0
    k[..., 0] = 0.092 * rate * torch.arange(n, dtype=torch.float32).view(1, 1, n)
    q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    heads = [0, 1] if H == 2 else [0, 1, 63, 127]
    for layout in ("contiguous", "striped"):
        qh, kh, vh = (t[:, heads] for t in (q, k, v))
        (ql, kl, vl), order = _oracle_layout((qh, kh, vh), P, layout)
        o_ref, l_ref = OA.attention(ql, kl, vl, True, pos_q=order, pos_k=order)
        qg, kg, vg = (ra.permute(t.cuda(), P) if layout == "striped" else t.cuda() for t in (q, k, v))
        o, lse = ra.forward(qg, kg, vg, P, layout, True, o_dtype=torch.float32)
        torch.cuda.synchronize()
        idx = torch.tensor(heads, device="cuda")
        compare(o.index_select(1, idx), lse.index_select(1, idx), o_ref, l_ref, "bf16", f"rising H={H} {layout}")


@pytest.mark.parametrize("H,c", [(256, 383), (256, 384), (256, 385), (2, 127), (2, 128), (2, 129)])
def test_workgroup_tile_boundaries(ra, H, c):
    """Block sizes at and around a workgroup's query tile: 384 rows for the 12-wave kernel (the
    256-head cases, whose grids of at least two 12-wave workgroups per CU select it), and around
    four 32-key tiles, one per key split of the small-grid workgroups (the 2-head cases)."""
    B, P, d = 1, 2, 128
    n = P * c
    g = torch.Generator().manual_seed(7000 + c + H)
    q, k, v = (torch.randn((B, H, n, d), generator=g).mul(0.5).to(torch.bfloat16) for _ in range(3))
    heads = [0, H - 1]
    for layout in ("contiguous", "striped"):
        (ql, kl, vl), order = _oracle_layout(tuple(t[:, heads] for t in (q, k, v)), P, layout)
        o_ref, l_ref = OA.attention(ql, kl, vl, True, pos_q=order, pos_k=order)
        qg, kg, vg = (ra.permute(t.cuda(), P) if layout == "striped" else t.cuda() for t in (q, k, v))
        stats = ra.new_stats(P)
        o, lse = ra.forward(qg, kg, vg, P, layout, True, o_dtype=torch.float32, stats=stats)
        torch.cuda.synchronize()
        idx = torch.tensor(heads, device="cuda")
        compare(o.index_select(1, idx), lse.index_select(1, idx), o_ref, l_ref, "bf16", f"c={c} H={H} {layout}")
        tq, tk = ra.tile_shape(ra.BF16, d)
        assert np.array_equal(stats.cpu().numpy(), _expected_stats(layout, P, c, B * H, True, tq, tk))


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 64)])
@pytest.mark.parametrize("scale", [0.3, 1.0])
def test_explicit_score_scale(ra, dtype, d, scale):
    """A caller-given score scale replaces 1/sqrt(d), in the fused forward and in one round."""
    P, c, H = 4, 96, 2
    n = P * c
    g = torch.Generator().manual_seed(int(scale * 100) + d)
    q, k, v = (torch.randn((1, H, n, d), generator=g).mul(0.5).to(dtype) for _ in range(3))
    kind = "f32" if dtype == torch.float32 else "bf16"
    for layout in LAYOUTS:
        (ql, kl, vl), order = _oracle_layout((q, k, v), P, layout)
        o_ref, l_ref = OA.attention(ql, kl, vl, True, pos_q=order, pos_k=order, scale=scale)
        qg, kg, vg = (ra.permute(t.cuda(), P) if layout == "striped" else t.cuda() for t in (q, k, v))
        o, lse = ra.forward(qg, kg, vg, P, layout, True, o_dtype=torch.float32, scale=scale)
        torch.cuda.synchronize()
        compare(o, lse, o_ref, l_ref, kind, f"scale={scale} {layout}")
        p, kk = 3, 1
        po, pl = ra.round(qg[:, :, p * c:(p + 1) * c], kg[:, :, kk * c:(kk + 1) * c], vg[:, :, kk * c:(kk + 1) * c],
                          P, p, kk, layout, True, scale=scale)
        torch.cuda.synchronize()
        for h in range(H):
            ro, rl = OR.round_partial(ql[0, h, p * c:(p + 1) * c], kl[0, h, kk * c:(kk + 1) * c],
                                      vl[0, h, kk * c:(kk + 1) * c], layout, p, kk, True, scale=scale)
            compare(po[0, h], pl[0, h], ro, rl, kind, f"round scale={scale} {layout} h={h}")
