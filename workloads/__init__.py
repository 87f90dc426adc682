"""Workload shapes and seeded synthetic inputs for blockwise ring / striped attention.

This module holds no attention arithmetic: only shapes, seeds and random-number generation.
It is the one piece of code that both the CPU oracle (``oracle/``) and the GPU path
(``striped_blockwise_amd``) may use, so that both sides see bit-identical inputs.

Recipe (every tensor is [B, H, n, d], token order, row-major, d contiguous):

* Q, K and V are drawn independently.  Each (tensor, batch, head) matrix [n, d] comes from its
  own torch CPU generator seeded with the first word of NumPy's
  ``SeedSequence([seed, tensor_id, b, h])`` (tensor_id 0/1/2 for Q/K/V), as iid standard
  normals in float32 (``torch.randn``), multiplied by ``input_scale`` (1 or 1/2, both exact in
  binary) and rounded to the compute dtype with round-to-nearest-even (torch's
  ``.to(torch.bfloat16)``).  Per-head streams let the oracle regenerate only the heads it needs.
  Both sides of every comparison use the same generated tensor in one process.
* The million-token stress workload scales K at 1% of token positions (all heads) by 8 to force
  large jumps of the running row maximum.  The positions are ``round(0.01 * n)`` distinct token
  indices drawn from ``SeedSequence([seed, 3])``.  The scaling is applied in float32 before the
  bf16 rounding; a power-of-two factor commutes with that rounding, so the stored K row equals
  8x the unscaled bf16 row.
* Position IDs are the global token indices 0..n-1 (int64).
* For the backward pass, the upstream gradient dO ("g") is drawn like Q, K, V with tensor_id 4,
  as unscaled iid standard normals rounded to the compute dtype.

Workload sizes follow the pages' settings: 8K, 256K and ~1M-token sequences, head dim 128, 2
to 32 sequence-parallel devices (Striped Attention review, section 5 "experimental setup";
Ring Attention review, "applications": million-token contexts).  The pages train language
models on text; an attention kernel only sees the score distribution, so Gaussian inputs of the
same shapes stand in for that data.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "get", "qkv", "positions", "outlier_rows"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n: int               # total tokens in the sequence
    P: int               # sequence-parallel (virtual) devices
    B: int               # batch
    H: int               # heads
    d: int               # head dim
    dtype: str           # "f32" or "bf16": storage/compute dtype of Q, K, V
    input_scale: float   # N(0,1) samples are multiplied by this
    seed: int = 0
    device: int | None = None     # the one device whose share is computed (None: all devices)
    outlier_frac: float = 0.0     # fraction of K rows multiplied by outlier_gain
    outlier_gain: float = 1.0

    @property
    def c(self) -> int:
        """Tokens per device (block size)."""
        return self.n // self.P

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


WORKLOADS = {
    # tiny exact check: fp32, every device and round
    "tiny_n256": Workload("tiny_n256", n=256, P=4, B=1, H=1, d=64, dtype="f32", input_scale=1.0),
    # 8K-token sequence over 4 devices, all devices x all rounds, contiguous and striped
    "seq_n8k": Workload("seq_n8k", n=8192, P=4, B=1, H=8, d=128, dtype="bf16", input_scale=0.5),
    # one device's share of a 256K-token sequence over 8 devices (the last device: most causal
    # work under the contiguous layout)
    "share_n256k": Workload("share_n256k", n=262144, P=8, B=1, H=32, d=128, dtype="bf16",
                            input_scale=0.5, device=7),
    # one device's share of a 1M-token sequence over 32 devices, K outlier rows
    "stress_n1m": Workload("stress_n1m", n=1048576, P=32, B=1, H=8, d=128, dtype="bf16",
                           input_scale=0.5, device=31, outlier_frac=0.01, outlier_gain=8.0),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


_TENSOR_ID = {"q": 0, "k": 1, "v": 2, "g": 4}


def _draw(seed: int, tid: int, b: int, h: int, n: int, d: int, scale: float) -> torch.Tensor:
    s = int(np.random.SeedSequence([seed, tid, b, h]).generate_state(1, np.uint64)[0])
    x = torch.randn((n, d), generator=torch.Generator().manual_seed(s), dtype=torch.float32)
    if scale != 1.0:
        x.mul_(scale)
    return x


def outlier_rows(w: Workload) -> np.ndarray:
    """Sorted token indices whose K rows are scaled by ``w.outlier_gain`` (empty if none)."""
    if w.outlier_frac <= 0.0:
        return np.zeros(0, dtype=np.int64)
    m = int(round(w.outlier_frac * w.n))
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, 3])))
    return np.sort(rng.choice(w.n, size=m, replace=False)).astype(np.int64)


def qkv(w: Workload | str, which: str = "qkv", heads=None, dtype: torch.dtype | None = None):
    """Generate the workload's inputs on the CPU, in token order.

    Returns a tuple of torch tensors, one per letter of ``which`` (letters of "qkvg"; g is the
    upstream gradient dO of the backward pass), each
    [B, len(heads), n, d] in the workload dtype (or ``dtype`` if given: float32/float64 return
    the exactly-rounded workload-dtype values widened).  ``heads`` selects head indices (default
    all).  Deterministic for a given workload regardless of which heads are requested.
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    heads = list(range(w.H)) if heads is None else [int(h) for h in heads]
    out_rows = outlier_rows(w)
    results = []
    for letter in which:
        tid = _TENSOR_ID[letter]
        t = torch.empty((w.B, len(heads), w.n, w.d), dtype=w.torch_dtype)
        rows = torch.from_numpy(out_rows)
        for b in range(w.B):
            for i, h in enumerate(heads):
                x = _draw(w.seed, tid, b, h, w.n, w.d, 1.0 if letter == "g" else w.input_scale)
                if letter == "k" and rows.numel():
                    x[rows] *= w.outlier_gain
                t[b, i].copy_(x)                      # round-to-nearest-even to the dtype
        if dtype is not None and dtype != t.dtype:
            t = t.to(dtype)
        results.append(t)
    return tuple(results)


def positions(n: int) -> torch.Tensor:
    """Position IDs in token order: the global token index."""
    return torch.arange(n, dtype=torch.int64)
