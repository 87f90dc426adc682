"""Rotary position embedding (RoPE) applied with the striped permutation, in fp64 on the CPU.

TEST INFRASTRUCTURE (see the package docstring): never imported by the GPU library.

The Striped Attention review ("位置编码处理") says that position encodings such as RoPE must see
the position IDs permuted exactly like the tokens.  The pages do not define RoPE itself; the
reading taken is the rotary embedding of RoFormer: the head dim is split into d/2 pairs, pair i
of a token at position m is rotated by the angle m * theta_i with theta_i = base^(-2i/d), so
that the score <R(m) q, R(n) k> depends on the positions only through n - m.  Two pairings of
the head dim are in common use and both are supported:
  * "interleaved": pair i = elements (2i, 2i + 1);
  * "half":        pair i = elements (i, i + d/2).

``rope_permute`` is what the fused kernel computes: RoPE applied in token order, then the rows
moved to the layout (or, with inverse=True, the adjoint: rows moved back to token order, then
rotated by -m * theta_i, which is the map that carries gradients back through the forward).
"""
from __future__ import annotations

import numpy as np

from .ring import from_layout, layout_order, to_layout

__all__ = ["pair_index", "angles", "rope", "rope_permute"]


def pair_index(d: int, style: str):
    """(first, second) element indices of the d/2 pairs."""
    if d % 2:
        raise ValueError("head dim must be even")
    i = np.arange(d // 2)
    if style == "interleaved":
        return 2 * i, 2 * i + 1
    if style == "half":
        return i, i + d // 2
    raise ValueError(style)


def angles(pos, d: int, base: float) -> np.ndarray:
    """[len(pos), d/2] rotation angles m * base^(-2i/d) in float64."""
    theta = float(base) ** (-2.0 * np.arange(d // 2, dtype=np.float64) / d)
    return np.asarray(pos, dtype=np.float64)[:, None] * theta[None, :]


def rope(x, pos, base: float = 10000.0, style: str = "interleaved", inverse: bool = False) -> np.ndarray:
    """Rotate rows of x [..., n, d] (token order) by their positions pos [n]."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    a, b = pair_index(d, style)
    ang = angles(pos, d, base)
    c, s = np.cos(ang), np.sin(ang)
    if inverse:
        s = -s
    out = np.empty_like(x)
    out[..., a] = x[..., a] * c - x[..., b] * s
    out[..., b] = x[..., a] * s + x[..., b] * c
    return out


def rope_permute(x, P: int, layout: str, pos=None, base: float = 10000.0, style: str = "interleaved",
                 inverse: bool = False) -> np.ndarray:
    """x [..., n, d]: token order -> rotated rows in layout order (inverse: layout -> token order,
    rotated back).  pos: positions of the tokens in token order (default 0..n-1)."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-2]
    pos = np.arange(n) if pos is None else np.asarray(pos)
    order = layout_order(n, P, layout)
    if inverse:
        return rope(from_layout(x, order), pos, base, style, inverse=True)
    return to_layout(rope(x, pos, base, style), order)
