"""Graph capture of the path (torch.cuda.CUDAGraph over the library's launches).

The forward with counters, D, the backward, and the streamed form (accumulator init, P x
(ra_round + ra_merge)) are captured once and replayed several times.  Before each replay every
output and the counter buffer are overwritten with garbage and unrelated eager work runs; each
replay must then reproduce the eager results bit for bit (same kernels, same order), and the
counters must come back exact, which they can only do if the forward clears its counter rows
inside the graph itself (it does so with a fill kernel, not a memset node).
"""
from __future__ import annotations

import pytest
import torch

from tests._gpu_util import need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ra():
    need_gpu()
    import striped_blockwise_amd as m
    return m


def _rows_of_range(n: int, P: int, p0: int, p1: int, tokens: bool, dev) -> torch.Tensor:
    """Row indices that the device range writes: token rows t with p0 <= t mod P < p1 in token
    order, else all rows of the (already range-sized) output."""
    t = torch.arange(n if tokens else (p1 - p0) * (n // P), device=dev)
    return t[(t % P >= p0) & (t % P < p1)] if tokens else t


@pytest.mark.parametrize("layout,p0,p1", [("striped_tokens", 1, 3), ("contiguous", 0, 4), ("striped", 3, 4)])
def test_captured_path_replays_match_eager(ra, layout, p0, p1):
    print(f"[graph] {layout} devices {p0}..{p1 - 1}", flush=True)
    dev = torch.device("cuda:0")
    B, H, n, d, P = 1, 4, 4096, 128, 4
    c = n // P
    tokens = layout == "striped_tokens"
    g = torch.Generator(device=dev).manual_seed(11)
    q, k, v = (torch.randn((B, H, n, d), generator=g, device=dev).mul_(0.5).to(torch.bfloat16) for _ in range(3))
    if layout == "striped":
        q, k, v = (ra.permute(t, P) for t in (q, k, v))
    m = n if tokens else (p1 - p0) * c
    dout = torch.randn((B, H, m, d), generator=g, device=dev).to(torch.bfloat16)
    rows = _rows_of_range(n, P, p0, p1, tokens, dev)

    # eager reference
    st_e = ra.new_stats(P)
    o_e, l_e = ra.forward(q, k, v, P, layout, True, p0, p1, stats=st_e)
    dl_e = ra.bwd_delta(o_e, dout)
    dq_e, dk_e, dv_e = ra.backward(q, k, v, dout, l_e, P, layout, True, p0, p1, delta=dl_e)
    stream_layout = "striped" if layout != "contiguous" else "contiguous"
    qs, ks, vs = (q, k, v) if layout != "striped_tokens" else (ra.permute(t, P) for t in (q, k, v))
    p = p1 - 1                                         # the streamed form for the last device
    po = torch.empty((B, H, c, d), dtype=torch.float32, device=dev)
    pl = torch.empty((B, H, c), dtype=torch.float32, device=dev)

    def streamed(acc_o, acc_l):
        acc_o.zero_()
        acc_l.fill_(float("-inf"))
        for r in range(P):
            kb = (p - r) % P
            ra.round(qs[:, :, p * c:(p + 1) * c], ks[:, :, kb * c:(kb + 1) * c], vs[:, :, kb * c:(kb + 1) * c],
                     P, p, kb, stream_layout, True, out=(po, pl))
            ra.merge(acc_o, acc_l, po, pl)

    so_e = torch.empty((B, H, c, d), dtype=torch.float32, device=dev)
    sl_e = torch.empty((B, H, c), dtype=torch.float32, device=dev)
    streamed(so_e, sl_e)
    torch.cuda.synchronize()

    # static buffers of the graph
    o_g, l_g = torch.empty_like(o_e), torch.empty_like(l_e)
    st_g = ra.new_stats(P)
    dl_g = torch.empty_like(dl_e)
    dq_g, dk_g, dv_g = torch.empty_like(dq_e), torch.empty_like(dk_e), torch.empty_like(dv_e)
    so_g, sl_g = torch.empty_like(so_e), torch.empty_like(sl_e)

    def path():
        ra.forward(q, k, v, P, layout, True, p0, p1, stats=st_g, out=(o_g, l_g))
        ra.bwd_delta(o_g, dout, out=dl_g)
        ra.backward(q, k, v, dout, l_g, P, layout, True, p0, p1, delta=dl_g, out=(dq_g, dk_g, dv_g))
        streamed(so_g, sl_g)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                      # warm-up outside the capture
        path()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        path()

    for rep in range(3):
        for t in (o_g, l_g, dl_g, dq_g, dk_g, dv_g, so_g, sl_g):
            t.fill_(float("nan"))
        st_g.fill_(987654321 + rep)
        x = torch.randn((1024, 1024), device=dev)
        (x @ x).sum().item()                           # unrelated eager work and a synchronization
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(st_g[p0:p1], st_e[p0:p1]), f"replay {rep}: counters"
        assert torch.equal(o_g[:, :, rows], o_e[:, :, rows]), f"replay {rep}: O"
        assert torch.equal(l_g[:, :, rows], l_e[:, :, rows]), f"replay {rep}: LSE"
        assert torch.equal(dl_g[:, :, rows], dl_e[:, :, rows]), f"replay {rep}: D"
        assert torch.equal(dq_g[:, :, rows], dq_e[:, :, rows]), f"replay {rep}: dQ"
        assert torch.equal(dk_g, dk_e) and torch.equal(dv_g, dv_e), f"replay {rep}: dK, dV"
        assert torch.equal(so_g, so_e) and torch.equal(sl_g, sl_e), f"replay {rep}: streamed O, LSE"
