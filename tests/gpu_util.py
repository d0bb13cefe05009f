"""Helpers shared by the GPU parity tests (no attention arithmetic here)."""

from __future__ import annotations

import numpy as np
import torch

# Tolerances: bf16 -> max|gpu - oracle| / max|oracle| per tensor; fp32 -> max abs.
TOL_BF16_O = 2e-2
TOL_BF16_GRAD = 5e-2
TOL_F32_ABS = 1e-5


def device():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible MI355X")
    return torch.device("cuda:0")


def f64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().float().cpu().numpy().astype(np.float64)
    return np.asarray(t, dtype=np.float64)


def rel_err(gpu, ref) -> float:
    gpu, ref = f64(gpu), f64(ref)
    scale = np.abs(ref).max()
    return float(np.abs(gpu - ref).max() / (scale if scale > 0 else 1.0))


def abs_err(gpu, ref) -> float:
    return float(np.abs(f64(gpu) - f64(ref)).max())


def assert_rel(gpu, ref, tol, name):
    err = rel_err(gpu, ref)
    assert err <= tol, f"{name}: max|gpu-oracle|/max|oracle| = {err:.3e} > {tol}"
    return err


def assert_abs(gpu, ref, tol, name):
    err = abs_err(gpu, ref)
    assert err <= tol, f"{name}: max|gpu-oracle| = {err:.3e} > {tol}"
    return err


def say(*args):
    print("[case]", *args, flush=True)
