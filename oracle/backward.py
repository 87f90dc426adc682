"""Gradients of blockwise ring / striped attention, in fp64 on the CPU.

TEST INFRASTRUCTURE (see the package docstring): never imported by the GPU library.

The pages give no backward pass; they only report training speedups (Striped Attention review,
section 五), so the gradients of the method are those of its forward definition,
O = softmax(Q K^T * scale + C) V (Striped Attention review, "核心公式"; Ring Attention review,
step 3 for the scale).  Two independent formulations:

* ``grads``: reverse-mode differentiation of that definition by torch autograd in float64.  No
  hand-written derivative is involved.
* ``round_grads`` / ``ring_backward``: the chain rule written out per (query block, K/V block)
  pair, the form a ring runs.  With the final log-sum-exp L of each query row (saved by the
  forward) the probabilities of one pair are P = exp(S + C - L) without any cross-block
  rescaling, and with D_i = sum_c dO_ic O_ic:
      dV_k += P^T dO_p,   dP = dO_p V_k^T,   dS = P * (dP - D_p),
      dQ_p += dS K_k * scale,   dK_k += dS^T Q_p * scale.
  Each device keeps dQ of its queries while dK, dV travel with their K/V block around the ring
  (Ring Attention review, step 2), so block k's gradients collect one contribution per device.
"""
from __future__ import annotations

import numpy as np
import torch

from .attention import causal_bias, default_scale, softmax_attention
from .ring import kv_block, round_bias

__all__ = ["grads", "attention_grads", "delta", "round_grads", "ring_backward"]


def grads(q, k, v, dout, causal: bool, pos_q=None, pos_k=None, scale=None):
    """One head: q [m, d], k/v [N, d], dout [m, dv] (numpy or torch, any float dtype) ->
    (dq, dk, dv) as float64 numpy arrays."""
    q, k, v, dout = (torch.tensor(_np64(t)) for t in (q, k, v, dout))
    q.requires_grad_(True)
    k.requires_grad_(True)
    v.requires_grad_(True)
    m, d = q.shape
    n = k.shape[0]
    if scale is None:
        scale = default_scale(d)
    s = (q @ k.T) * scale
    if causal:
        pq = np.arange(m) if pos_q is None else np.asarray(pos_q)
        pk = np.arange(n) if pos_k is None else np.asarray(pos_k)
        s = s + torch.tensor(causal_bias(pq, pk))
    o = torch.softmax(s, dim=1) @ v
    o.backward(dout)
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


def delta(o, dout):
    """D_i = sum over the head dim of O_i * dO_i."""
    return (np.asarray(o, dtype=np.float64) * np.asarray(dout, dtype=np.float64)).sum(axis=-1)


def round_grads(qb, kb, vb, dob, lse_b, delta_b, bias, scale=None):
    """Contributions of one (query block, K/V block) pair: (dq, dk, dv) in float64.

    lse_b and delta_b belong to the query rows; bias is the pair's 0 / -inf mask [rows, keys].
    """
    qb, kb, vb, dob = (np.asarray(t, dtype=np.float64) for t in (qb, kb, vb, dob))
    if scale is None:
        scale = default_scale(qb.shape[1])
    s = (qb @ kb.T) * scale + bias
    lse = np.asarray(lse_b, dtype=np.float64)[:, None]
    p = np.where(np.isfinite(lse), np.exp(s - np.where(np.isfinite(lse), lse, 0.0)), 0.0)
    dv = p.T @ dob
    dp = dob @ vb.T
    ds = p * (dp - np.asarray(delta_b, dtype=np.float64)[:, None])
    dq = ds @ kb * scale
    dk = ds.T @ qb * scale
    return dq, dk, dv


def ring_backward(q_lay, k_lay, v_lay, dout_lay, P: int, layout: str, causal: bool, scale=None):
    """Whole-sequence gradients by the ring's per-pair contributions, one head, layout order.

    The forward's O and LSE come from the plain definition; returns (dq, dk, dv) [n, d].
    """
    q_lay, k_lay, v_lay, dout_lay = (np.asarray(t, dtype=np.float64) for t in (q_lay, k_lay, v_lay, dout_lay))
    n, d = q_lay.shape
    c = n // P
    dq = np.zeros_like(q_lay)
    dk = np.zeros_like(k_lay)
    dv = np.zeros_like(v_lay)
    for p in range(P):
        rows = slice(p * c, (p + 1) * c)
        bias_full = np.concatenate([round_bias(layout, p, kk, c, causal) for kk in range(P)], axis=1)
        o, lse = softmax_attention(q_lay[rows], k_lay, v_lay, bias_full, scale)
        dlt = delta(o, dout_lay[rows])
        for r in range(P):
            kk = kv_block(p, r, P)
            keys = slice(kk * c, (kk + 1) * c)
            gq, gk, gv = round_grads(q_lay[rows], k_lay[keys], v_lay[keys], dout_lay[rows], lse, dlt,
                                     round_bias(layout, p, kk, c, causal), scale)
            dq[rows] += gq
            dk[keys] += gk
            dv[keys] += gv
    return dq, dk, dv


def attention_grads(q, k, v, dout, causal: bool, pos_q=None, pos_k=None, scale=None):
    """Batched heads [B, H, m, d] (numpy or torch, any float dtype) -> (dq, dk, dv) float64.

    Gradients of the definition with respect to every input, head by head (``grads``).
    """
    q, k, v, dout = (_np64(t) for t in (q, k, v, dout))
    B, H = q.shape[:2]
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = grads(q[b, h], k[b, h], v[b, h], dout[b, h], causal,
                                                 pos_q, pos_k, scale)
    return dq, dk, dv


def _np64(t) -> np.ndarray:
    if hasattr(t, "detach"):
        return t.detach().to(torch.float64).cpu().numpy()
    return np.asarray(t, dtype=np.float64)
