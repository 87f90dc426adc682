"""GPU parity of ra_permute_rope (rotary embedding fused with the striped permutation) against
the oracle (oracle/rope.py): RoPE applied in token order with the tokens' positions, then the
rows moved to the layout -- the Striped Attention review's rule that RoPE sees the permuted
position IDs, checked as equivariance.

The kernel forms angles, cosines, sines and the rotation in fp64 and rounds once to fp32 (then
once more to bf16), as the reference rounding below does.  The two fp64 computations differ
only through the last bit of theta_i and of the trigonometric functions, so an angle m*theta
differs by at most ~2 eps64 * m and an output by that times the input's magnitude; the bound is
one unit in the last place of the rounded result plus 4 * 2^-53 * (max position + 1) * max|x|
(that term only matters where a rotation cancels to a value far below its inputs).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads
from oracle import rope as RP
from tests._gpu_util import need_gpu, np64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ra():
    need_gpu()
    import striped_blockwise_amd as m
    return m


def _rounded(ref: np.ndarray, dtype: torch.dtype) -> np.ndarray:
    """fp64 -> fp32 (nearest even) -> dtype (nearest even), widened back to fp64."""
    t = torch.from_numpy(np.asarray(ref, np.float64).astype(np.float32))
    return t.to(dtype).to(torch.float64).numpy()


def _check(got: torch.Tensor, ref: np.ndarray, label: str, x=None, max_pos: float = 0.0):
    g = np64(got)
    r = _rounded(ref, got.dtype)
    ulp = np.spacing(np.abs(r).astype(np.float32)).astype(np.float64)
    if got.dtype == torch.bfloat16:
        ulp = ulp * 2.0 ** 16                      # bf16 keeps 8 of fp32's 24 significand bits
    xmax = float(np.abs(np64(x) if isinstance(x, torch.Tensor) else np.abs(ref)).max()) if g.size else 0.0
    atol = 4.0 * 2.0 ** -53 * (max_pos + 1.0) * xmax
    diff = np.abs(g - r)
    assert np.all(diff <= ulp + atol), f"{label}: max diff {diff.max():.3e} beyond one ulp + {atol:.1e}"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("style", ["interleaved", "half"])
@pytest.mark.parametrize("layout", ["striped", "contiguous"])
@pytest.mark.parametrize("B,H,n,P,d", [(1, 4, 256, 4, 128), (2, 3, 96, 8, 64), (1, 2, 30, 3, 6), (1, 1, 64, 64, 130)])
def test_rope_permute_matches_oracle(ra, dtype, style, layout, B, H, n, P, d):
    gen = torch.Generator().manual_seed(n * d + P)
    x = torch.randn((B, H, n, d), generator=gen).to(dtype)
    got = ra.permute_rope(x.cuda(), P, layout, style=style)
    torch.cuda.synchronize()
    ref = RP.rope_permute(np64(x), P, layout, style=style)
    _check(got, ref, f"{dtype} {style} {layout} n={n} P={P} d={d}", x, n)
    back = ra.permute_rope(got, P, layout, style=style, inverse=True)
    torch.cuda.synchronize()
    _check(back, RP.rope_permute(np64(got), P, layout, style=style, inverse=True), "inverse", got, n)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_rope_large_and_custom_positions(ra, dtype):
    """Positions around 10^6 (where an fp32 angle has no fraction left) and arbitrary IDs."""
    n, P, d = 512, 8, 128
    gen = torch.Generator().manual_seed(7)
    x = torch.randn((1, 2, n, d), generator=gen).to(dtype)
    for pos in (torch.arange(n, dtype=torch.int64) + 1_000_000,
                torch.randint(0, 4_000_000, (n,), generator=gen, dtype=torch.int64)):
        got = ra.permute_rope(x.cuda(), P, "striped", pos=pos.cuda())
        torch.cuda.synchronize()
        _check(got, RP.rope_permute(np64(x), P, "striped", pos.numpy()), f"{dtype} pos from {int(pos[0])}",
               x, float(pos.max()))


def test_rope_then_striped_attention_equals_token_order(ra):
    """The whole path: RoPE fused into the striped permutation, striped attention, un-permute,
    against RoPE'd token-order (contiguous) attention on the same data."""
    w = workloads.get("seq_n8k")
    n, P = 4096, 4
    q, k, v = (t[:, :2, :n].contiguous().cuda() for t in workloads.qkv(w, heads=[0, 1]))
    qs, ks = (ra.permute_rope(t, P, "striped") for t in (q, k))
    vs = ra.permute(v, P)
    qc, kc = (ra.permute_rope(t, P, "contiguous") for t in (q, k))
    o_s, l_s = ra.forward(qs, ks, vs, P, "striped", True, o_dtype=torch.float32)
    o_c, l_c = ra.forward(qc, kc, v, P, "contiguous", True, o_dtype=torch.float32)
    o_u = ra.permute(o_s, P, inverse=True)
    l_u = ra.permute(l_s, P, dim=-1, inverse=True)
    torch.cuda.synchronize()
    assert float((o_u - o_c).abs().max()) <= 2e-2 and float((l_u - l_c).abs().max()) <= 1e-3


def test_rope_full_size_share(ra):
    """bench.py's configuration: Q of the 256K share (32 heads), striped, default positions;
    sampled rows against the oracle, and the round trip on every element."""
    w = workloads.get("share_n256k")
    (q,) = workloads.qkv(w, "q")
    qg = q.cuda()
    got = ra.permute_rope(qg, w.P, "striped")
    back = ra.permute_rope(got, w.P, "striped", inverse=True)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 7, 8, 32767, 32768, 131071, 200003, w.n - 1])     # layout rows
    from oracle import ring as R
    order = R.layout_order(w.n, w.P, "striped")
    for h in (0, 31):
        ref = RP.rope(np64(q[0, h, torch.from_numpy(order[rows])]), order[rows])
        _check(got[0, h, torch.from_numpy(rows).cuda()], ref, f"share head {h}", qg[0, h], w.n)
    err = float((back.float() - qg.float()).abs().max())
    assert err <= 2 * 2.0 ** -8 * float(qg.float().abs().max()), err
