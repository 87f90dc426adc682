"""Exact softmax attention, written out from its definition, in fp64 on the CPU.

TEST INFRASTRUCTURE (see the package docstring): never imported by the GPU library.

Definition (Striped Attention review, section 三 "核心公式", causal self-attention):
    O = softmax(S + C) V,   S = Q K^T * scale,
    C[i, j] = -inf when the query's position is smaller than the key's position, else 0.
The scale is 1/sqrt(d) (Ring Attention review, step 3: the scores are Q_p K_j^T / sqrt(d); the
PyTorch sketch multiplies by d_k ** -0.5).  The Striped Attention review writes the definition
without the scale; the reading taken is that the scale is part of S.

The log-sum-exp of a row is LSE_i = ln sum_j exp(S_ij + C_ij) (natural log), computed as
max + ln(sum exp(. - max)).  A row whose keys are all masked has no softmax; the reading taken
for it (needed only for single-round partials) is O_i = 0 and LSE_i = -inf, so that it is the
identity of the log-sum-exp merge.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["causal_bias", "softmax_attention", "attention", "default_scale"]


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def causal_bias(pos_q, pos_k) -> np.ndarray:
    """C[i, j] = -inf if pos_q[i] < pos_k[j] else 0 (query i may see key j iff pos_k <= pos_q)."""
    pq = np.asarray(pos_q, dtype=np.int64)[:, None]
    pk = np.asarray(pos_k, dtype=np.int64)[None, :]
    return np.where(pq < pk, -np.inf, 0.0)


def softmax_attention(q, k, v, bias=None, scale=None):
    """One head: q [m, d], k [N, d], v [N, dv], bias [m, N] (0 or -inf) or None.

    Returns (O [m, dv], LSE [m]) in float64.  Rows with every key masked give O = 0,
    LSE = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if scale is None:
        scale = default_scale(q.shape[1])
    s = (q @ k.T) * scale
    if bias is not None:
        s = s + bias
    m = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    live = np.isfinite(m)
    ref = np.where(live, m, 0.0)
    e = np.exp(s - ref[:, None])          # masked entries: exp(-inf) = 0
    l = e.sum(axis=1)
    o = np.zeros((q.shape[0], v.shape[1]), dtype=np.float64)
    o[live] = (e[live] @ v) / l[live, None]
    lse = np.full(q.shape[0], -np.inf)
    lse[live] = m[live] + np.log(l[live])
    return o, lse


def attention(q, k, v, causal: bool, pos_q=None, pos_k=None, scale=None, row_chunk: int = 4096):
    """Batched heads: q [B, H, m, d], k/v [B, H, N, d] (numpy or torch, any float dtype).

    ``pos_q`` / ``pos_k`` are the tokens' global positions (default 0..m-1 / 0..N-1); the
    causal mask compares them, so permuted (striped) rows are handled by passing the permuted
    position IDs.  Returns (O [B, H, m, dv], LSE [B, H, m]) as float64 numpy arrays.
    """
    q, k, v = (_np64(t) for t in (q, k, v))
    B, H, m, _ = q.shape
    N = k.shape[2]
    pos_q = np.arange(m) if pos_q is None else np.asarray(pos_q, dtype=np.int64)
    pos_k = np.arange(N) if pos_k is None else np.asarray(pos_k, dtype=np.int64)
    o = np.empty((B, H, m, v.shape[3]), dtype=np.float64)
    lse = np.empty((B, H, m), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, m, row_chunk):
                r1 = min(m, r0 + row_chunk)
                bias = causal_bias(pos_q[r0:r1], pos_k) if causal else None
                o[b, h, r0:r1], lse[b, h, r0:r1] = softmax_attention(
                    q[b, h, r0:r1], k[b, h], v[b, h], bias, scale)
    return o, lse


def _np64(t) -> np.ndarray:
    if hasattr(t, "detach"):  # torch tensor (CPU): widen exactly to fp64
        import torch
        return t.detach().to(torch.float64).cpu().numpy()
    return np.asarray(t, dtype=np.float64)
