"""GPU parity of the backward pass: libra.so (ra_bwd_delta, ra_backward, ra_backward_round)
against the oracle's fp64 gradients (oracle/backward.py), element by element.

The GPU side runs its own forward (ra_forward) for O and LSE, then the backward; the oracle
differentiates the plain definition on the identical rounded inputs.  Tolerances are in
tests/_gpu_util.py.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads
from oracle import backward as OB
from oracle import ring as OR
from tests._gpu_util import compare_grad, need_gpu, np64

pytestmark = pytest.mark.gpu

LAYOUTS = ["contiguous", "striped"]


@pytest.fixture(scope="module")
def ra():
    need_gpu()
    import striped_blockwise_amd as m
    return m


def _inputs(w, heads=None, n=None, P=None):
    """Q, K, V, dO of a workload in token order (CPU), optionally truncated to n tokens."""
    q, k, v, g = workloads.qkv(w, "qkvg", heads=heads)
    if n is not None:
        q, k, v, g = (t[:, :, :n].contiguous() for t in (q, k, v, g))
    return q, k, v, g


def _to_layout(ts, P, layout):
    n = ts[0].shape[2]
    order = OR.layout_order(n, P, layout)
    idx = torch.from_numpy(order)
    return [t[:, :, idx].contiguous() for t in ts], order


def _gpu_fwd_bwd(ra, q, k, v, g, P, layout, causal, p_begin=0, p_end=None, o_dtype=None, scale=0.0):
    """q, k, v, g: CPU tensors in layout order.  Returns GPU (dq, dk, dv) of the device range."""
    p_end = P if p_end is None else p_end
    c = q.shape[2] // P
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    o, lse = ra.forward(qg, kg, vg, P, layout, causal, p_begin, p_end, o_dtype=o_dtype, scale=scale)
    dout = g[:, :, p_begin * c:p_end * c].contiguous().cuda()
    dq, dk, dv = ra.backward(qg, kg, vg, dout, lse, P, layout, causal, p_begin, p_end, o=o, scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


def _oracle(q, k, v, g, P, order, causal, p_begin=0, p_end=None, scale=None):
    """Oracle gradients for the queries of devices [p_begin, p_end) (inputs in layout order)."""
    p_end = P if p_end is None else p_end
    c = q.shape[2] // P
    rows = slice(p_begin * c, p_end * c)
    return OB.attention_grads(q[:, :, rows], k, v, g[:, :, rows], causal, order[rows], order, scale)


def _check(got, ref, kind, label):
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        compare_grad(a, b, kind, f"{label} {name}")


# --------------------------------------------------------------------------- row term D
@pytest.mark.parametrize("shape,odt,gdt", [
    ((2, 3, 100, 128), torch.bfloat16, torch.bfloat16), ((1, 2, 77, 128), torch.float32, torch.bfloat16),
    ((1, 1, 50, 6), torch.float32, torch.float32), ((1, 1, 33, 64), torch.bfloat16, torch.float32)])
def test_delta_matches_oracle(ra, shape, odt, gdt):
    gen = torch.Generator().manual_seed(sum(shape))
    o = torch.randn(shape, generator=gen).to(odt)
    g = torch.randn(shape, generator=gen).to(gdt)
    got = ra.bwd_delta(o.cuda(), g.cuda())
    torch.cuda.synchronize()
    ref = OB.delta(np64(o), np64(g))
    np.testing.assert_allclose(np64(got), ref, rtol=1e-5, atol=1e-5)


# --------------------------------------------------------------------------- tiny fp32
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("causal", [False, True])
def test_tiny_f32_backward(ra, layout, causal):
    w = workloads.get("tiny_n256")
    (q, k, v, g), order = _to_layout(_inputs(w), w.P, layout)
    got = _gpu_fwd_bwd(ra, q, k, v, g, w.P, layout, causal)
    _check(got, _oracle(q, k, v, g, w.P, order, causal), "f32", f"tiny {layout} causal={causal}")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_tiny_f32_rounds_accumulate(ra, layout):
    """ra_backward_round over every (device, round) pair, in ring order, adds up to the gradient."""
    w = workloads.get("tiny_n256")
    P, c = w.P, w.c
    (q, k, v, g), order = _to_layout(_inputs(w), P, layout)
    qg, kg, vg, gg = q.cuda(), k.cuda(), v.cuda(), g.cuda()
    o, lse = ra.forward(qg, kg, vg, P, layout, True)
    delta = ra.bwd_delta(o, gg)
    dq = torch.zeros_like(qg)
    dk = torch.zeros_like(kg)
    dv = torch.zeros_like(vg)
    for p in range(P):
        rows = slice(p * c, (p + 1) * c)
        for r in range(P):
            kv = OR.kv_block(p, r, P)
            keys = slice(kv * c, (kv + 1) * c)
            acc = (torch.zeros_like(dq[:, :, rows]), torch.zeros_like(dk[:, :, keys]), torch.zeros_like(dv[:, :, keys]))
            ra.backward_round(qg[:, :, rows], kg[:, :, keys], vg[:, :, keys], gg[:, :, rows], lse[:, :, rows],
                              delta[:, :, rows], P, p, kv, layout, True, grads=acc)
            dq[:, :, rows] += acc[0]
            dk[:, :, keys] += acc[1]
            dv[:, :, keys] += acc[2]
    torch.cuda.synchronize()
    _check((dq, dk, dv), _oracle(q, k, v, g, P, order, True), "f32", f"tiny rounds {layout}")


# --------------------------------------------------------------------------- bf16, 8K tokens
@pytest.mark.parametrize("layout", LAYOUTS)
def test_bf16_seq8k_backward(ra, layout):
    w = workloads.get("seq_n8k")
    (q, k, v, g), order = _to_layout(_inputs(w, heads=[0, 5]), w.P, layout)
    got = _gpu_fwd_bwd(ra, q, k, v, g, w.P, layout, True, o_dtype=torch.bfloat16, scale=w.input_scale)
    _check(got, _oracle(q, k, v, g, w.P, order, True, scale=w.input_scale), "bf16", f"seq8k {layout}")


def test_bf16_device_range_and_noncausal(ra):
    w = workloads.get("seq_n8k")
    n, P = 4096, 4
    (q, k, v, g), order = _to_layout(_inputs(w, heads=[3], n=n), P, "striped")
    got = _gpu_fwd_bwd(ra, q, k, v, g, P, "striped", True, p_begin=1, p_end=3)
    _check(got, _oracle(q, k, v, g, P, order, True, 1, 3), "bf16", "striped devices 1..2")
    (q, k, v, g), order = _to_layout(_inputs(w, heads=[4], n=n), P, "contiguous")
    got = _gpu_fwd_bwd(ra, q, k, v, g, P, "contiguous", False, p_begin=2, p_end=4, scale=0.3)
    _check(got, _oracle(q, k, v, g, P, order, False, 2, 4, scale=0.3), "bf16", "non-causal devices 2..3")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_bf16_rounds_equal_fused(ra, layout):
    """Per-round backward (every pair, ring order) matches the fused backward and the oracle."""
    w = workloads.get("seq_n8k")
    n, P = 2048, 4
    c = n // P
    (q, k, v, g), order = _to_layout(_inputs(w, heads=[1, 2], n=n), P, layout)
    qg, kg, vg, gg = q.cuda(), k.cuda(), v.cuda(), g.cuda()
    o, lse = ra.forward(qg, kg, vg, P, layout, True)
    delta = ra.bwd_delta(o, gg)
    fused = ra.backward(qg, kg, vg, gg, lse, P, layout, True, delta=delta)
    dq = torch.zeros(fused[0].shape, dtype=torch.float32, device="cuda")
    dk = torch.zeros_like(dq)
    dv = torch.zeros_like(dq)
    for p in range(P):
        rows = slice(p * c, (p + 1) * c)
        dq_p = torch.zeros_like(dq[:, :, rows])
        for r in range(P):
            kv = OR.kv_block(p, r, P)
            keys = slice(kv * c, (kv + 1) * c)
            acc = (dq_p, torch.zeros_like(dk[:, :, keys]), torch.zeros_like(dv[:, :, keys]))
            ra.backward_round(qg[:, :, rows], kg[:, :, keys], vg[:, :, keys], gg[:, :, rows], lse[:, :, rows],
                              delta[:, :, rows], P, p, kv, layout, True, grads=acc)
            dk[:, :, keys] += acc[1]
            dv[:, :, keys] += acc[2]
        dq[:, :, rows] = dq_p
    torch.cuda.synchronize()
    for a, b, name in zip((dq, dk, dv), fused, ("dq", "dk", "dv")):
        diff = float((a - b).abs().max())
        assert diff <= 1e-5 * max(1.0, float(b.abs().max())), f"{layout} {name}: rounds vs fused {diff:.3e}"
    _check((dq, dk, dv), _oracle(q, k, v, g, P, order, True), "bf16", f"rounds {layout}")


# --------------------------------------------------------------------------- edge cases
@pytest.mark.parametrize("c", [1, 2, 37, 200])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_blocks(ra, c, dtype):
    P = 4
    n = c * P
    d = 128 if dtype == "bf16" else 64
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    gen = torch.Generator().manual_seed(1000 + c)
    q, k, v, g = (torch.randn((1, 2, n, d), generator=gen).mul(0.5).to(tdt) for _ in range(4))
    for layout in LAYOUTS:
        (ql, kl, vl, gl), order = _to_layout((q, k, v, g), P, layout)
        got = _gpu_fwd_bwd(ra, ql, kl, vl, gl, P, layout, True)
        _check(got, _oracle(ql, kl, vl, gl, P, order, True), dtype, f"c={c} {dtype} {layout}")


@pytest.mark.parametrize("n,P", [(96, 1), (64, 64), (256, 8)])
def test_device_count_extremes(ra, n, P):
    gen = torch.Generator().manual_seed(n * 7 + P)
    q, k, v, g = (torch.randn((1, 1, n, 128), generator=gen).mul(0.5).to(torch.bfloat16) for _ in range(4))
    for layout in LAYOUTS:
        (ql, kl, vl, gl), order = _to_layout((q, k, v, g), P, layout)
        got = _gpu_fwd_bwd(ra, ql, kl, vl, gl, P, layout, True)
        _check(got, _oracle(ql, kl, vl, gl, P, order, True), "bf16", f"n={n} P={P} {layout}")


def test_striped_gradients_equivariant(ra):
    """Striped gradients, un-permuted, equal the contiguous ones (same tokens, same math)."""
    w = workloads.get("seq_n8k")
    n, P = 4096, 4
    q, k, v, g = _inputs(w, heads=[6], n=n)
    base = _gpu_fwd_bwd(ra, q, k, v, g, P, "contiguous", True)
    (ql, kl, vl, gl), order = _to_layout((q, k, v, g), P, "striped")
    st = _gpu_fwd_bwd(ra, ql, kl, vl, gl, P, "striped", True)
    for name, a, b in zip(("dq", "dk", "dv"), st, base):
        a_tok = ra.permute(a.contiguous(), P, inverse=True)
        torch.cuda.synchronize()
        compare_grad(a_tok, np64(b), "bf16", f"equivariance {name}")


def test_backward_deterministic(ra):
    w = workloads.get("seq_n8k")
    (q, k, v, g), _ = _to_layout(_inputs(w, heads=[2], n=4096), 4, "striped")
    a = _gpu_fwd_bwd(ra, q, k, v, g, 4, "striped", True)
    b = _gpu_fwd_bwd(ra, q, k, v, g, 4, "striped", True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_invalid_args(ra):
    q = torch.zeros((1, 1, 64, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((1, 1, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):                    # dout rows do not match the device range
        ra.backward(q, q, q, q, lse, 4, "striped", True, p_begin=0, p_end=2, delta=lse[:, :, :32])
    with pytest.raises(ValueError):                    # neither delta nor o
        ra.backward(q, q, q, q, lse, 4)
    out = torch.zeros((1, 1, 64, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):                    # dq and dk alias
        ra.backward(q, q, q, q, lse, 4, delta=lse, out=(out, out, torch.zeros_like(out)))
    q48 = torch.zeros((1, 1, 64, 48), dtype=torch.float32, device="cuda")
    with pytest.raises(NotImplementedError):           # f32 head dim 48
        ra.backward(q48, q48, q48, q48, lse, 4, delta=lse)
    with pytest.raises(ValueError):
        ra.bwd_delta(q, q[:, :, :32])


@pytest.mark.parametrize("c", [127, 129, 255, 257])
def test_backward_workgroup_boundaries(ra, c):
    """Block sizes around the backward kernels' workgroup tiles (128 key rows for dK/dV; for dQ,
    whose small grids take 2 row groups x 4 key splits, around multiples of four 32-key tiles),
    both layouts, against the oracle."""
    P, H, d = 2, 2, 128
    n = P * c
    gen = torch.Generator().manual_seed(9000 + c)
    q, k, v, g = (torch.randn((1, H, n, d), generator=gen).mul(0.5 if i < 3 else 1.0).to(torch.bfloat16)
                  for i in range(4))
    for layout in LAYOUTS:
        (ql, kl, vl, gl), order = _to_layout((q, k, v, g), P, layout)
        got = _gpu_fwd_bwd(ra, ql, kl, vl, gl, P, layout, True)
        ref = _oracle(ql, kl, vl, gl, P, order, True)
        _check(got, ref, "bf16", f"c={c} {layout}")


@pytest.mark.parametrize("H,P,c", [(2, 4, 1000), (64, 2, 600), (128, 2, 1500)])
def test_backward_dq_workgroup_shapes(ra, H, P, c):
    """The dQ kernel picks its workgroup shape by grid size; on a 256-CU device these cases take
    2 row groups x 4 key splits (2 x 4 x 32 = 256 row groups), 4 x 2 (2432 row groups) and the
    8-wave workgroups without splits (1536 of them), all with ragged tiles.  The split shapes add
    their partial dQ sums in LDS.  Gradients of three heads against the oracle, both layouts."""
    d = 128
    n = P * c
    gen = torch.Generator().manual_seed(9500 + H + c)
    q, k, v, g = (torch.randn((1, H, n, d), generator=gen).mul(0.5 if i < 3 else 1.0).to(torch.bfloat16)
                  for i in range(4))
    heads = [0, 1, H - 1]
    for layout in LAYOUTS:
        (ql, kl, vl, gl), order = _to_layout((q, k, v, g), P, layout)
        dq, dk, dv = _gpu_fwd_bwd(ra, ql, kl, vl, gl, P, layout, True)
        idx = torch.tensor(heads, device="cuda")
        got = tuple(t.index_select(1, idx) for t in (dq, dk, dv))
        ref = _oracle(*(t[:, heads].contiguous() for t in (ql, kl, vl, gl)), P, order, True)
        _check(got, ref, "bf16", f"H={H} c={c} {layout}")


@pytest.mark.parametrize("layout,H,P,c,p_begin,p_end", [
    ("striped", 128, 2, 700, 0, 2),          # 3 query tiles of 256 rows: pairs (0, 2) and (1, 1)
    ("striped", 64, 4, 1100, 1, 4),          # 5 tiles, three devices, ragged last tile
    ("contiguous", 128, 2, 1500, 0, 1),      # device 0 alone: diagonal round, then a skipped one
])
def test_backward_dq_paired_query_tiles(ra, layout, H, P, c, p_begin, p_end):
    """Wide dQ launches whose rounds are all causal-triangular pair query tiles i and nqt-1-i in
    one workgroup and add each (round, tile) partial into dq: an odd tile count (a tile paired
    with itself), a device range, and a contiguous launch with a round that skips every key.
    Gradients of three heads against the oracle."""
    d = 128
    n = P * c
    gen = torch.Generator().manual_seed(9700 + H + c)
    q, k, v, g = (torch.randn((1, H, n, d), generator=gen).mul(0.5 if i < 3 else 1.0).to(torch.bfloat16)
                  for i in range(4))
    heads = [0, 5, H - 1]
    (ql, kl, vl, gl), order = _to_layout((q, k, v, g), P, layout)
    dq, dk, dv = _gpu_fwd_bwd(ra, ql, kl, vl, gl, P, layout, True, p_begin, p_end)
    idx = torch.tensor(heads, device="cuda")
    got = tuple(t.index_select(1, idx) for t in (dq, dk, dv))
    ref = _oracle(*(t[:, heads].contiguous() for t in (ql, kl, vl, gl)), P, order, True, p_begin, p_end)
    _check(got, ref, "bf16", f"paired dQ {layout} H={H} c={c} devices {p_begin}..{p_end - 1}")
