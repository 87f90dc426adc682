"""Ring / Striped blockwise attention, emulated step by step in fp64 on the CPU.

TEST INFRASTRUCTURE (see the package docstring): never imported by the GPU library.

What each function follows (pages cited by title and section; see the package docstring):

* Layouts.  Contiguous: device p owns tokens [p*c, (p+1)*c), c = n/P (Ring Attention review,
  step 1).  Striped: token t goes to device t mod P and each device keeps its tokens in
  increasing order, e.g. with 4 devices device 0 holds 0, 4, 8, 12 and device 1 holds 1, 5, 9,
  13 (Striped Attention review, "分区策略对比").  Position IDs get the same permutation
  (Striped Attention review, "位置编码处理").
* Schedule.  Each device keeps its Q block; K/V blocks move one hop per round from rank i to
  rank i+1, so after r rounds device p holds the block that started on device (p - r) mod P,
  and P rounds visit every block (Ring Attention review, step 2 and the sketch's send/receive
  ranks).
* GetMask.  The Striped Attention review's "GetMask 函数" procedures, with j = the device that
  owns the query block and k = the device the K/V block came from.  The procedures index
  MASK[x, y]; the reading taken is x = key index inside the K/V block and y = query index inside
  the Q block.  It is the only orientation under which the procedures agree with the causal
  matrix C (query position < key position is masked) and with the work formulas; the tests
  check that agreement by brute force.  The contiguous procedure never initialises MASK; the
  reading taken is the striped procedure's initial value 0 (everything visible).
* Online softmax across rounds (Ring Attention review, step 3).  The printed equation lacks the
  normaliser recurrence and the exp(m_{j-1} - m_j) rescale; the reading taken is the recurrence
  the same page's PyTorch sketch runs: m_j = max(m_{j-1}, rowmax S_j),
  l_j = exp(m_{j-1} - m_j) l_{j-1} + rowsum exp(S_j - m_j),
  acc_j = exp(m_{j-1} - m_j) acc_{j-1} + exp(S_j - m_j) V_j, and O = acc / l after the last round.
* Merge of per-round partials: the softmax denominator of a query is the sum of the per-node
  sums of exp over each node's keys ("Computing Attention Weights in Sequence Parallelism").
  With normalised partials (O_a, L_a), (O_b, L_b): L = ln(e^{L_a} + e^{L_b}),
  O = e^{L_a - L} O_a + e^{L_b - L} O_b.
* Work per (device, round): Striped Attention review, "核心公式": the contiguous layout gives
  c^2 for a K/V block from an earlier device and 0 for a later one; the page also counts the
  diagonal (own) block as c^2, but that block is only partly visible (the review's "算法行为对比":
  round 0 is partly masked) and holds c(c+1)/2 visible pairs -- the reading taken.  The striped
  layout gives c(c+1)/2 when the block's device index is not larger than the query device's and
  c(c-1)/2 otherwise.
* Tiles: a block is cut into tiles; a tile whose pairs are all masked is skipped
  (Striped Attention review, "分块与分瓦片").  The tile shape is the kernel's own.
"""
from __future__ import annotations

import numpy as np

from .attention import softmax_attention, default_scale

__all__ = [
    "CONTIGUOUS", "STRIPED", "layout_order", "layout_position", "kv_block", "get_mask",
    "round_bias", "round_partial", "merge", "OnlineState", "blockwise_device", "blockwise_all",
    "local_only", "visible_pairs", "work_closed_form", "tile_counts_brute",
    "tile_counts_closed_form", "to_layout", "from_layout",
]

CONTIGUOUS = "contiguous"
STRIPED = "striped"


# ----------------------------------------------------------------------------- layouts
def layout_order(n: int, P: int, layout: str) -> np.ndarray:
    """order[pos] = token index stored at layout position pos (device p owns [p*c, (p+1)*c))."""
    if n % P:
        raise ValueError("n must be a multiple of P")
    if layout == CONTIGUOUS:
        return np.arange(n, dtype=np.int64)
    if layout != STRIPED:
        raise ValueError(layout)
    per_device = [[] for _ in range(P)]
    for t in range(n):                       # token t -> device t mod P, kept in increasing order
        per_device[t % P].append(t)
    return np.array([t for dev in per_device for t in dev], dtype=np.int64)


def layout_position(n: int, P: int, layout: str) -> np.ndarray:
    """pi[t] = layout position of token t (inverse of ``layout_order``)."""
    order = layout_order(n, P, layout)
    pi = np.empty(n, dtype=np.int64)
    pi[order] = np.arange(n, dtype=np.int64)
    return pi


def to_layout(x: np.ndarray, order: np.ndarray, axis: int = -2) -> np.ndarray:
    """Rows in layout order: out[..., pos, :] = x[..., order[pos], :]."""
    return np.take(x, order, axis=axis)


def from_layout(x: np.ndarray, order: np.ndarray, axis: int = -2) -> np.ndarray:
    """Inverse of ``to_layout``: rows back in token order."""
    out = np.empty_like(x)
    idx = [slice(None)] * x.ndim
    idx[axis] = order
    out[tuple(idx)] = x
    return out


# ----------------------------------------------------------------------------- schedule, mask
def kv_block(p: int, r: int, P: int) -> int:
    """Origin device of the K/V block that device p holds in round r."""
    return (p - r) % P


def get_mask(layout: str, j: int, k: int, c: int) -> np.ndarray:
    """MASK[x, y] (x: key index in block k, y: query index in block j) with 0 / -inf entries."""
    mask = np.zeros((c, c))
    x = np.arange(c)[:, None]
    y = np.arange(c)[None, :]
    if layout == CONTIGUOUS:
        if j < k:
            mask[:, :] = -np.inf
        elif j == k:
            mask[np.broadcast_to(y < x, (c, c))] = -np.inf
    elif layout == STRIPED:
        if j < k:
            mask[np.broadcast_to(y <= x, (c, c))] = -np.inf
        else:
            mask[np.broadcast_to(y < x, (c, c))] = -np.inf
    else:
        raise ValueError(layout)
    return mask


def round_bias(layout: str, j: int, k: int, c: int, causal: bool) -> np.ndarray:
    """Additive bias in [query, key] orientation for device j's Q block against block k."""
    if not causal:
        return np.zeros((c, c))
    return get_mask(layout, j, k, c).T


# ----------------------------------------------------------------------------- one round
def round_partial(qb, kb, vb, layout: str, j: int, k: int, causal: bool, scale=None):
    """Normalised attention of Q block j over K/V block k alone: (O_r [c, dv], LSE_r [c])."""
    c = qb.shape[0]
    return softmax_attention(qb, kb, vb, round_bias(layout, j, k, c, causal), scale)


def merge(o_a, lse_a, o_b, lse_b):
    """Combine two normalised partials over disjoint key sets (rows with -inf are empty)."""
    o_a, lse_a, o_b, lse_b = (np.asarray(t, dtype=np.float64) for t in (o_a, lse_a, o_b, lse_b))
    lse = np.logaddexp(lse_a, lse_b)                       # (-inf, -inf) -> -inf
    ref = np.where(np.isfinite(lse), lse, 0.0)             # an empty side gets weight exp(-inf)=0
    w_a = np.exp(lse_a - ref)
    w_b = np.exp(lse_b - ref)
    o = w_a[..., None] * o_a + w_b[..., None] * o_b
    return o, lse


# ----------------------------------------------------------------------------- online softmax
class OnlineState:
    """Running max m, running normaliser l and unnormalised output acc for one Q block."""

    def __init__(self, rows: int, dv: int):
        self.m = np.full(rows, -np.inf)
        self.l = np.zeros(rows)
        self.acc = np.zeros((rows, dv))

    def update(self, s: np.ndarray, v: np.ndarray) -> None:
        """Fold in one round: s = masked scaled scores [rows, keys], v = that block's values."""
        m_new = np.maximum(self.m, s.max(axis=1))
        ref = np.where(np.isfinite(m_new), m_new, 0.0)     # no key seen yet: keep zeros
        alpha = np.exp(self.m - ref)                       # exp(-inf) = 0 on the first round
        p = np.exp(s - ref[:, None])
        self.l = alpha * self.l + p.sum(axis=1)
        self.acc = alpha[:, None] * self.acc + p @ v
        self.m = m_new

    def finish(self):
        live = self.l > 0
        o = np.zeros_like(self.acc)
        o[live] = self.acc[live] / self.l[live, None]
        lse = np.full(self.l.shape, -np.inf)
        lse[live] = self.m[live] + np.log(self.l[live])
        return o, lse


def blockwise_device(q_lay, k_lay, v_lay, p: int, P: int, layout: str, causal: bool,
                     scale=None, rounds=None):
    """Device p of the emulated ring, one head; q/k/v [n, d] already in layout order.

    Runs the rounds r in ``rounds`` (default 0..P-1, the ring order) with the K/V block
    ``kv_block(p, r, P)`` and the round's GetMask.  Returns (O [c, dv], LSE [c]).
    """
    q_lay, k_lay, v_lay = (np.asarray(t, dtype=np.float64) for t in (q_lay, k_lay, v_lay))
    n, d = q_lay.shape
    c = n // P
    if scale is None:
        scale = default_scale(d)
    qb = q_lay[p * c:(p + 1) * c]
    st = OnlineState(c, v_lay.shape[1])
    for r in (range(P) if rounds is None else rounds):
        k = kv_block(p, r, P)
        s = (qb @ k_lay[k * c:(k + 1) * c].T) * scale + round_bias(layout, p, k, c, causal)
        st.update(s, v_lay[k * c:(k + 1) * c])
    return st.finish()


def blockwise_all(q_lay, k_lay, v_lay, P: int, layout: str, causal: bool, scale=None):
    """Every device of the ring, one head: (O [n, dv], LSE [n]) in layout order."""
    outs = [blockwise_device(q_lay, k_lay, v_lay, p, P, layout, causal, scale) for p in range(P)]
    return np.concatenate([o for o, _ in outs]), np.concatenate([l for _, l in outs])


def local_only(q_lay, k_lay, v_lay, P: int, layout: str, causal: bool, scale=None):
    """The flawed scheme where each device attends only to its own K/V block (negative test)."""
    return np.concatenate([
        blockwise_device(q_lay, k_lay, v_lay, p, P, layout, causal, scale, rounds=[0])[0]
        for p in range(P)])


# ----------------------------------------------------------------------------- integer counts
def visible_pairs(layout: str, j: int, k: int, c: int, causal: bool) -> int:
    """Unmasked (query, key) pairs of Q block j against K/V block k, counted from the mask."""
    if not causal:
        return c * c
    return int(np.count_nonzero(get_mask(layout, j, k, c) == 0.0))


def work_closed_form(layout: str, j: int, k: int, c: int, causal: bool) -> int:
    """The work formulas of the Striped Attention review, with the diagonal block's true count."""
    if not causal:
        return c * c
    if layout == CONTIGUOUS:
        if k < j:
            return c * c
        if k == j:
            return c * (c + 1) // 2
        return 0
    return c * (c + 1) // 2 if k <= j else c * (c - 1) // 2


def _band_visible(layout, j, k, c, causal, y0, y1):
    """Boolean visibility for query rows [y0, y1) of block j against all c keys of block k."""
    if not causal:
        return np.ones((y1 - y0, c), dtype=bool)
    y = np.arange(y0, y1)[:, None]
    x = np.arange(c)[None, :]
    if layout == CONTIGUOUS:
        if j < k:
            return np.zeros((y1 - y0, c), dtype=bool)
        if j > k:
            return np.ones((y1 - y0, c), dtype=bool)
        return ~(y < x)
    return ~(y <= x) if j < k else ~(y < x)


def tile_counts_brute(layout: str, j: int, k: int, c: int, tq: int, tk: int, causal: bool):
    """(full, diag, skipped) tiles of a tq x tk grid over the c x c block, from the mask itself.

    Edge tiles of a ragged grid are classified on their in-range part.
    """
    full = diag = skipped = 0
    for y0 in range(0, c, tq):
        y1 = min(c, y0 + tq)
        vis = _band_visible(layout, j, k, c, causal, y0, y1)
        for x0 in range(0, c, tk):
            t = vis[:, x0:min(c, x0 + tk)]
            if t.all():
                full += 1
            elif not t.any():
                skipped += 1
            else:
                diag += 1
    return full, diag, skipped


def tile_counts_closed_form(layout: str, j: int, k: int, c: int, tq: int, tk: int, causal: bool):
    """Same counts as ``tile_counts_brute`` by arithmetic on the tile corners.

    Within a causal block the visible pairs are exactly key index x <= query index y - delta,
    with delta = 0 (contiguous own block, striped earlier-or-same device) or 1 (striped later
    device).  A tile [y0, y1) x [x0, x1) is then fully visible iff x1 - 1 <= y0 - delta and
    fully masked iff x0 > y1 - 1 - delta.
    """
    nt_q = -(-c // tq)
    nt_k = -(-c // tk)
    total = nt_q * nt_k
    if not causal or (layout == CONTIGUOUS and j > k):
        return total, 0, 0
    if layout == CONTIGUOUS and j < k:
        return 0, 0, total
    delta = 1 if (layout == STRIPED and j < k) else 0
    y0 = np.arange(nt_q, dtype=np.int64)[:, None] * tq          # tile rows  [y0, y1)
    y1 = np.minimum(c, y0 + tq)
    x0 = np.arange(nt_k, dtype=np.int64)[None, :] * tk          # tile cols  [x0, x1)
    x1 = np.minimum(c, x0 + tk)
    is_full = (x1 - 1) <= (y0 - delta)
    is_diag = ~is_full & (x0 <= (y1 - 1 - delta))
    full = int(is_full.sum())
    diag = int(is_diag.sum())
    return full, diag, total - full - diag
