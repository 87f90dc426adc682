"""Shared helpers for the GPU parity tests: tolerances, comparisons and skip logic."""
from __future__ import annotations

import numpy as np
import pytest
import torch

# Tolerances against the fp64 oracle on the identical (already rounded) inputs.
F32_O_ABS = 1e-4          # float32 inputs: O max-abs
F32_LSE_ABS = 1e-4        # float32 inputs: LSE max-abs
BF16_O_ABS = 2e-2         # bf16 inputs: O max-abs
BF16_O_RELFRO = 1e-2      # bf16 inputs: ||O - O_ref||_F / ||O_ref||_F
BF16_LSE_ABS = 1e-3       # bf16 inputs: LSE max-abs


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import striped_blockwise_amd as ra
    ra.lib()                                 # raises if libra.so is missing: no silent fallback


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def compare(o_gpu, lse_gpu, o_ref, lse_ref, kind: str, label: str = ""):
    """Element-wise comparison; rows with reference LSE = -inf must be exactly (0, -inf)."""
    o = np64(o_gpu) if isinstance(o_gpu, torch.Tensor) else np.asarray(o_gpu, np.float64)
    lse = np64(lse_gpu) if isinstance(lse_gpu, torch.Tensor) else np.asarray(lse_gpu, np.float64)
    o_ref = np.asarray(o_ref, np.float64)
    lse_ref = np.asarray(lse_ref, np.float64)
    assert o.shape == o_ref.shape, (label, o.shape, o_ref.shape)
    assert lse.shape == lse_ref.shape, (label, lse.shape, lse_ref.shape)
    empty = ~np.isfinite(lse_ref)
    assert np.all(lse[empty] == -np.inf), f"{label}: empty rows must have LSE = -inf"
    assert np.all(o[empty] == 0.0), f"{label}: empty rows must have O = 0"
    live = ~empty
    assert np.all(np.isfinite(lse[live])) and np.all(np.isfinite(o[live])), f"{label}: non-finite output"
    err_o = float(np.abs(o[live] - o_ref[live]).max()) if live.any() else 0.0
    err_l = float(np.abs(lse[live] - lse_ref[live]).max()) if live.any() else 0.0
    if kind == "f32":
        assert err_o <= F32_O_ABS, f"{label}: O max-abs {err_o:.3e} > {F32_O_ABS}"
        assert err_l <= F32_LSE_ABS, f"{label}: LSE max-abs {err_l:.3e} > {F32_LSE_ABS}"
    else:
        num = float(np.linalg.norm((o - o_ref)[live]))
        den = float(np.linalg.norm(o_ref[live])) or 1.0
        assert err_o <= BF16_O_ABS, f"{label}: O max-abs {err_o:.3e} > {BF16_O_ABS}"
        assert num / den <= BF16_O_RELFRO, f"{label}: O rel-Frobenius {num / den:.3e} > {BF16_O_RELFRO}"
        assert err_l <= BF16_LSE_ABS, f"{label}: LSE max-abs {err_l:.3e} > {BF16_LSE_ABS}"
    return err_o, err_l


# Gradients (backward pass) against the fp64 oracle.  float32: same bound as the forward.
# bf16: the kernels round P and dS to bf16 before the fp32-accumulated MFMA sums (relative error
# <= 2^-9 each, RMS 2^-9/sqrt(3) ~ 1.1e-3 for round-to-nearest, independent from term to term),
# and P is formed from the bf16 forward's LSE (within 1e-3 absolute, so P within ~1e-3
# relative, the same for every key of a row).  Adding the two in quadrature gives ~1.5e-3 for a
# gradient tensor's relative Frobenius error; measured 1.6-1.8e-3.  The bound, 5e-3, is ~3x
# that.  Max-abs is taken relative to the tensor's largest reference entry.
F32_GRAD_ABS = 1e-4
BF16_GRAD_RELFRO = 5e-3
BF16_GRAD_MAXREL = 2e-2


def compare_grad(got, ref, kind: str, label: str = ""):
    g = np64(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert g.shape == ref.shape, (label, g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{label}: non-finite gradient"
    err = float(np.abs(g - ref).max()) if g.size else 0.0
    if kind == "f32":
        assert err <= F32_GRAD_ABS, f"{label}: max-abs {err:.3e} > {F32_GRAD_ABS}"
        return err
    top = float(np.abs(ref).max()) if ref.size else 0.0
    num = float(np.linalg.norm(g - ref))
    den = float(np.linalg.norm(ref))
    if den == 0.0:
        assert err == 0.0, f"{label}: reference is zero, got max-abs {err:.3e}"
        return 0.0
    assert num / den <= BF16_GRAD_RELFRO, f"{label}: rel-Frobenius {num / den:.3e} > {BF16_GRAD_RELFRO}"
    assert err <= BF16_GRAD_MAXREL * top, f"{label}: max-abs {err:.3e} > {BF16_GRAD_MAXREL} x {top:.3e}"
    return num / den
