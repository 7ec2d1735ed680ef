"""Shared helpers of the test suite (comparisons and conversions only)."""

import sys

import numpy as np
import torch

# Attention tolerance for bf16 inputs with fp32 accumulation.
ATTN_MAX_ABS = 2e-2
ATTN_REL_FRO = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_attn_close(got: np.ndarray, want: np.ndarray, what: str = ""):
    err = np.abs(got - want)
    fro = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert err.max() <= ATTN_MAX_ABS, f"{what}: max-abs {err.max():.3e}"
    assert fro <= ATTN_REL_FRO, f"{what}: rel-Frobenius {fro:.3e}"
    return err.max(), fro


def assert_energy_close(got: np.ndarray, want: np.ndarray, what: str = ""):
    """Per element |dE| <= 1e-4 E + 1e-7 and per row sum |dE| <= 1e-4."""
    d = np.abs(got - want)
    bad = d > 1e-4 * np.abs(want) + 1e-7
    assert not bad.any(), f"{what}: {bad.sum()} entries off, worst {d.max():.3e}"
    assert d.sum(axis=-1).max() <= 1e-4, f"{what}: row L1 {d.sum(axis=-1).max():.3e}"
