"""GPU robustness of the boundary.

* ra_merge on ragged row counts (tails of the vector kernel's row groups) and on every head-dim
  path (the vector kernel for d = 64 and 128, the general kernel for any other d), with rows
  where one side or both sides are empty (LSE = -inf) and rows with a NaN LSE, against the
  oracle's merge in fp64.
* NaN inputs: no kernel loops on data, so NaN entries in Q, K or V must neither hang nor leak
  into rows that do not use them.  A NaN in Q reaches its own row only; a NaN in K reaches the
  rows that see that key; a NaN in V reaches the O of the rows that see it (their LSE stays
  finite) and at most the rows of the same 32 x 32 tile that mask it (0 x NaN in the matrix
  product), never any other row.  Rows it does not reach match the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import ring as OR
from tests._gpu_util import F32_LSE_ABS, F32_O_ABS, compare, need_gpu, np64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ra():
    need_gpu()
    import striped_blockwise_amd as m
    return m


# ------------------------------------------------------------------------------------- merge
@pytest.mark.parametrize("d", [6, 32, 64, 128])
@pytest.mark.parametrize("rows", [1, 3, 13, 1001])
def test_merge_ragged_rows_and_empty_sides(ra, rows, d):
    print(f"[robust] merge rows={rows} d={d}", flush=True)
    g = np.random.default_rng(1000 * rows + d)
    o_a = g.standard_normal((rows, d)).astype(np.float32)
    o_b = g.standard_normal((rows, d)).astype(np.float32)
    l_a = g.uniform(-6, 6, rows).astype(np.float32)
    l_b = g.uniform(-6, 6, rows).astype(np.float32)
    # empty sides: row 0 both, then (if present) acc only and partial only
    l_a[0] = l_b[0] = -np.inf
    o_a[0] = 0.0
    o_b[0] = 0.0
    if rows > 1:
        l_a[1] = -np.inf
        o_a[1] = 0.0
    if rows > 2:
        l_b[2] = -np.inf
        o_b[2] = 0.0
    o_ref, l_ref = OR.merge(o_a, l_a, o_b, l_b)
    acc_o, acc_l = torch.from_numpy(o_a).cuda(), torch.from_numpy(l_a).cuda()
    po, pl = torch.from_numpy(o_b).cuda(), torch.from_numpy(l_b).cuda()
    ra.merge(acc_o, acc_l, po, pl)
    torch.cuda.synchronize()
    o, l = np64(acc_o), np64(acc_l)
    assert l[0] == -np.inf and np.all(o[0] == 0.0), "both sides empty must stay (0, -inf)"
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(l), fin)
    assert np.abs(l[fin] - l_ref[fin]).max(initial=0.0) <= F32_LSE_ABS
    assert np.abs(o[fin] - o_ref[fin]).max(initial=0.0) <= F32_O_ABS
    # the partial is unchanged
    assert np.array_equal(np64(po), o_b.astype(np.float64)) and np.array_equal(np64(pl), l_b.astype(np.float64))


@pytest.mark.parametrize("d", [6, 128])
def test_merge_nan_lse_propagates(ra, d):
    rows = 9
    o_a = np.ones((rows, d), np.float32)
    o_b = np.full((rows, d), 2.0, np.float32)
    l_a = np.zeros(rows, np.float32)
    l_b = np.zeros(rows, np.float32)
    l_b[3] = np.nan                        # NaN partial against a live accumulator
    l_a[5] = np.nan                        # NaN accumulator against an empty partial
    l_b[5] = -np.inf
    acc_o, acc_l = torch.from_numpy(o_a).cuda(), torch.from_numpy(l_a).cuda()
    ra.merge(acc_o, acc_l, torch.from_numpy(o_b).cuda(), torch.from_numpy(l_b).cuda())
    torch.cuda.synchronize()
    o, l = np64(acc_o), np64(acc_l)
    for r in (3, 5):
        assert np.isnan(l[r]) and np.isnan(o[r]).all(), r
    ok = [r for r in range(rows) if r not in (3, 5)]
    assert np.allclose(l[ok], np.log(2.0)) and np.allclose(o[ok], 1.5)


# --------------------------------------------------------------------------------- NaN inputs
def _inputs(dtype, d, n, H, seed):
    g = torch.Generator().manual_seed(seed)
    return [torch.randn((1, H, n, d), generator=g).mul(0.5).to(dtype) for _ in range(3)]


@pytest.mark.parametrize("which", ["q", "k", "v"])
@pytest.mark.parametrize("layout", ["contiguous", "striped", "striped_tokens"])
@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_nan_inputs_reach_only_the_rows_that_use_them(ra, which, layout, dtype, d):
    n, P, H = 2048, 4, 2
    c = n // P
    print(f"[robust] NaN in {which}, {layout}, {dtype}", flush=True)
    q, k, v = _inputs(dtype, d, n, H, seed=77)
    tok = 1234                              # token position of the NaN entry (head 1, element 5)
    clean_o, clean_l = OA.attention(q, k, v, True)          # token order, all rows
    bad = {"q": q, "k": k, "v": v}[which].clone()
    bad[0, 1, tok, 5] = float("nan")
    q2, k2, v2 = (bad if which == name else t for name, t in (("q", q), ("k", k), ("v", v)))
    base = "striped" if layout != "contiguous" else "contiguous"
    order = OR.layout_order(n, P, base)
    if layout == "striped":
        args = [ra.permute(t.cuda(), P) for t in (q2, k2, v2)]
    else:
        args = [t.cuda() for t in (q2, k2, v2)]
    o, lse = ra.forward(*args, P, layout, True, o_dtype=torch.float32)
    torch.cuda.synchronize()
    o, lse = np64(o)[0], np64(lse)[0]
    if layout == "striped":                 # back to token order
        o, lse = OR.from_layout(o, order), OR.from_layout(lse[..., None], order)[..., 0]
    pos = np.arange(n)
    if which == "q":
        hit = np.zeros((H, n), bool)
        hit[1, tok] = True
    else:                                    # rows that see key `tok`
        hit = np.zeros((H, n), bool)
        hit[1] = pos >= tok
    kind = "f32" if dtype == torch.float32 else "bf16"
    if which == "v":
        # LSE does not depend on V: every row matches the oracle
        assert np.isfinite(lse).all()
        assert np.abs(lse - clean_l[0]).max() <= (1e-4 if kind == "f32" else 1e-3)
        assert np.isnan(o[hit]).any(axis=-1).all(), "rows that see the NaN value must be NaN"
        leak = np.isnan(o).any(axis=-1) & ~hit
        # rows that mask the key but share its 32-key tile: at most 32 rows per K/V block tile
        assert leak.sum() <= 32 * P, leak.sum()
        assert not leak[0].any(), "the other head is untouched"
        keep = ~hit & ~leak
    else:
        assert np.isnan(lse[hit]).all() and np.isnan(o[hit]).all(), "rows that use the NaN must be NaN"
        assert not np.isnan(lse[~hit]).any() and not np.isnan(o[~hit]).any(), "NaN leaked into other rows"
        keep = ~hit
    compare(o[keep], lse[keep], clean_o[0][keep], clean_l[0][keep], kind, f"NaN in {which}, {layout}")


def test_nan_query_backward_ends_and_keeps_other_rows(ra):
    """The backward with a NaN query entry: the launch ends, dQ of that row is NaN and dQ of
    every other row matches a clean run's within the gradient tolerance."""
    from tests._gpu_util import compare_grad
    n, P, H, d = 1024, 4, 2, 128
    q, k, v = _inputs(torch.bfloat16, d, n, H, seed=5)
    dout = torch.randn((1, H, n, d), generator=torch.Generator().manual_seed(6)).to(torch.bfloat16)
    qg, kg, vg, dog = (t.cuda() for t in (q, k, v, dout))
    o, lse = ra.forward(qg, kg, vg, P, "contiguous", True)
    clean = ra.backward(qg, kg, vg, dog, lse, P, "contiguous", True, o=o)
    tok = 700
    qn = qg.clone()
    qn[0, 0, tok, 3] = float("nan")
    o2, lse2 = ra.forward(qn, kg, vg, P, "contiguous", True)
    dq, dk, dv = ra.backward(qn, kg, vg, dog, lse2, P, "contiguous", True, o=o2)
    torch.cuda.synchronize()
    dq = np64(dq)
    assert np.isnan(dq[0, 0, tok]).all()
    mask = np.ones(dq.shape[:3], bool)
    mask[0, 0, tok] = False
    assert not np.isnan(dq[mask]).any(), "NaN leaked into other query rows' dQ"
    compare_grad(dq[mask], np64(clean[0])[mask], "bf16", "dQ of the other rows")
    assert np.isnan(np64(dk)[0, 0, :tok + 1]).any(axis=-1).all(), "keys the NaN row sees"
    assert not np.isnan(np64(dk)[0, 1]).any() and not np.isnan(np64(dv)[0, 1]).any(), "other head"
