"""Seeded random forward and backward problems against the oracle, across the launchers'
workgroup shapes.

Each case draws a device count, block size (ragged), head count, layout (contiguous, striped
on permuted tensors, striped in token order), mask, device range, output dtype and score scale
from a fixed generator.  The grids this spans take every bf16 forward shape: the 12-wave
workgroups, the three key-split shapes and the paired mode of small triangular launches.  The
GPU runs every head; the oracle checks the first and the last.
"""
from __future__ import annotations

import zlib

import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import backward as OB
from oracle import ring as OR
from tests._gpu_util import compare, compare_grad, need_gpu, np64

pytestmark = pytest.mark.gpu

LAYOUTS = ["contiguous", "striped", "striped_tokens"]


def _cases(count=24, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        P = int(rng.choice([1, 2, 3, 4, 8, 16]))
        c = int(rng.integers(1, 700))
        H = int(rng.choice([1, 2, 3, 8, 40, 96, 160]))
        if P * c > 4096 or H * P * c > 600_000:
            continue
        layout = LAYOUTS[int(rng.integers(0, 3))]
        causal = bool(rng.random() < 0.8)
        p0 = int(rng.integers(0, P)) if rng.random() < 0.4 else 0
        p1 = int(rng.integers(p0 + 1, P + 1)) if p0 > 0 or rng.random() < 0.3 else P
        bf16_out = bool(rng.random() < 0.3)
        scale = float(rng.uniform(0.03, 0.2)) if rng.random() < 0.3 else 0.0
        out.append((P, c, H, layout, causal, p0, p1, bf16_out, scale))
    # grids of at least two 12-wave workgroups per CU (on 256 CUs), and one past the key splits
    out += [(2, 700, 160, "striped", True, 0, 2, False, 0.0),
            (2, 650, 160, "striped_tokens", True, 0, 2, True, 0.1),
            (2, 690, 160, "contiguous", True, 0, 2, False, 0.0),
            (4, 300, 96, "contiguous", True, 0, 4, False, 0.0)]
    return out


@pytest.fixture(scope="module")
def ra():
    need_gpu()
    import striped_blockwise_amd as m
    return m


@pytest.mark.parametrize("case", _cases(), ids=lambda t: "P{}-c{}-H{}-{}-{}-d{}:{}-{}-s{:.3f}".format(
    t[0], t[1], t[2], t[3], "causal" if t[4] else "full", t[5], t[6], "bf16" if t[7] else "f32", t[8]))
def test_random_forward_problem(ra, case):
    P, c, H, layout, causal, p0, p1, bf16_out, scale = case
    n, d = P * c, 128
    g = torch.Generator().manual_seed(zlib.crc32(repr(case).encode()))
    q, k, v = (torch.randn((1, H, n, d), generator=g).mul(0.5).to(torch.bfloat16) for _ in range(3))
    heads = sorted({0, H - 1})
    sc = scale if scale > 0 else None
    o_dtype = torch.bfloat16 if bf16_out else torch.float32
    label = f"P={P} c={c} H={H} {layout} causal={causal} devices {p0}..{p1 - 1}"
    idx = torch.tensor(heads, device="cuda")
    if layout == "striped_tokens":
        o, lse = ra.forward(q.cuda(), k.cuda(), v.cuda(), P, layout, causal, p0, p1, o_dtype=o_dtype, scale=scale)
        torch.cuda.synchronize()
        rows = np.nonzero((np.arange(n) % P >= p0) & (np.arange(n) % P < p1))[0]
        o_ref, l_ref = OA.attention(q[:, heads][:, :, rows], k[:, heads], v[:, heads], causal,
                                    pos_q=rows, scale=sc)
        got_o = np64(o.index_select(1, idx).float())[:, :, rows]
        got_l = np64(lse.index_select(1, idx))[:, :, rows]
        compare(got_o, got_l, o_ref, l_ref, "bf16", label)
        return
    order = OR.layout_order(n, P, layout)
    ql, kl, vl = (OR.to_layout(np64(t[:, heads]), order) for t in (q, k, v))
    rows = slice(p0 * c, p1 * c)
    o_ref, l_ref = OA.attention(ql[:, :, rows], kl, vl, causal, pos_q=order[rows], pos_k=order, scale=sc)
    qg, kg, vg = (ra.permute(t.cuda(), P) if layout == "striped" else t.cuda() for t in (q, k, v))
    o, lse = ra.forward(qg, kg, vg, P, layout, causal, p0, p1, o_dtype=o_dtype, scale=scale)
    torch.cuda.synchronize()
    compare(o.index_select(1, idx).float(), lse.index_select(1, idx), o_ref, l_ref, "bf16", label)


def _bwd_cases(count=12, seed=20261204):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        P = int(rng.choice([1, 2, 3, 4, 8]))
        c = int(rng.integers(1, 600))
        H = int(rng.choice([1, 2, 8, 40, 96]))
        if P * c > 3072 or H * P * c > 400_000:
            continue
        layout = LAYOUTS[int(rng.integers(0, 3))]
        causal = bool(rng.random() < 0.8)
        p0 = int(rng.integers(0, P)) if rng.random() < 0.4 else 0
        p1 = int(rng.integers(p0 + 1, P + 1)) if p0 > 0 or rng.random() < 0.3 else P
        scale = float(rng.uniform(0.03, 0.2)) if rng.random() < 0.3 else 0.0
        out.append((P, c, H, layout, causal, p0, p1, scale))
    # the dQ kernel's 4 x 2 split (more than 4 row groups of 32 per CU) and its 8-wave shape
    out += [(2, 600, 96, "striped", True, 0, 2, 0.0), (2, 1500, 128, "striped_tokens", True, 0, 2, 0.0)]
    return out


@pytest.mark.parametrize("case", _bwd_cases(), ids=lambda t: "P{}-c{}-H{}-{}-{}-d{}:{}-s{:.3f}".format(
    t[0], t[1], t[2], t[3], "causal" if t[4] else "full", t[5], t[6], t[7]))
def test_random_backward_problem(ra, case):
    P, c, H, layout, causal, p0, p1, scale = case
    n, d = P * c, 128
    g = torch.Generator().manual_seed(zlib.crc32(repr(case).encode()))
    q, k, v, go = (torch.randn((1, H, n, d), generator=g).mul(0.5 if i < 3 else 1.0).to(torch.bfloat16)
                   for i in range(4))
    heads = sorted({0, H - 1})
    sc = scale if scale > 0 else None
    label = f"P={P} c={c} H={H} {layout} causal={causal} devices {p0}..{p1 - 1}"
    idx = torch.tensor(heads, device="cuda")
    if layout == "striped_tokens":
        qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
        o, lse = ra.forward(qg, kg, vg, P, layout, causal, p0, p1, scale=scale)
        dq, dk, dv = ra.backward(qg, kg, vg, go.cuda(), lse, P, layout, causal, p0, p1, o=o, scale=scale)
        torch.cuda.synchronize()
        rows = np.nonzero((np.arange(n) % P >= p0) & (np.arange(n) % P < p1))[0]
        ref = OB.attention_grads(q[:, heads][:, :, rows], k[:, heads], v[:, heads], go[:, heads][:, :, rows],
                                 causal, rows, np.arange(n), sc)
        got = (np64(dq.index_select(1, idx))[:, :, rows], dk.index_select(1, idx), dv.index_select(1, idx))
    else:
        order = OR.layout_order(n, P, layout)
        ql, kl, vl, gl = (OR.to_layout(np64(t[:, heads]), order) for t in (q, k, v, go))
        rows = slice(p0 * c, p1 * c)
        ref = OB.attention_grads(ql[:, :, rows], kl, vl, gl[:, :, rows], causal, order[rows], order, sc)
        qg, kg, vg, gg = (ra.permute(t.cuda(), P) if layout == "striped" else t.cuda() for t in (q, k, v, go))
        o, lse = ra.forward(qg, kg, vg, P, layout, causal, p0, p1, scale=scale)
        dq, dk, dv = ra.backward(qg, kg, vg, gg[:, :, rows].contiguous(), lse, P, layout, causal, p0, p1, o=o,
                                 scale=scale)
        torch.cuda.synchronize()
        got = tuple(t.index_select(1, idx) for t in (dq, dk, dv))
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        compare_grad(a, b, "bf16", f"{label} {name}")
