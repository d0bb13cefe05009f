"""Helpers shared by the GPU parity tests (no attention arithmetic here)."""

from __future__ import annotations

import numpy as np
import torch

# Tolerances: bf16 -> max|gpu - oracle| / max|oracle| per tensor; fp32 -> max abs.
TOL_BF16_O = 2e-2
TOL_BF16_GRAD = 5e-2
TOL_F32_ABS = 1e-5
# Per-row bars (see row_rel_err): bf16 rows of O within 1% of their own size,
# rows of dQ, dK, dV within 1.5% (the GPU measures at most 0.64% and 0.73% on
# every workload). A row of O or dQ missing one 64-key tile is off by at
# least about 2% of its size at the long workload's length, and far more
# earlier in the sequence (tests/test_row_diagnostic_cpu.py).
ROW_TOL_O = 1e-2
ROW_TOL_GRAD = 1.5e-2


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


# Per-row diagnostic. A row is one token of one head (the last axis holds its
# d values): err_i = max_c |gpu_ic - oracle_ic| / max_c |oracle_ic|. With the
# long workload's 0.5-scaled inputs |O_i| shrinks like 0.5 / sqrt(i), so the
# per-tensor bar (relative to the tensor's max, set by the first rows) would
# let a wrong late row through; this bar is relative to each row's own size.
#
# Gradient rows get one allowance on top. The backward forms D_i = rowsum(dO_i
# * O_i) from the forward's stored O, which the O bar lets differ from the
# exact O_i by ROW_TOL_O * |O_i|_inf per element, so D_i may be off by
# delta_i <= ROW_TOL_O * |O_i|_inf * |dO_i|_1. That moves dS_ij by -P_ij delta_i,
# hence dQ_i by -scale delta_i kbar_i (kbar_i = sum_j P_ij k_j, the P-weighted
# mean key) and dK_j by -scale sum_i P_ij delta_i q_i, whatever the exact
# gradient's own size: where it cancels to nearly zero (the first queries of a
# document) only that allowance is a meaningful bar. It is negligible on late
# rows, which keep the full relative bar.
ROW_FLOOR = 1e-4


def row_max(x) -> np.ndarray:
    x = f64(x)
    return np.abs(x.reshape(-1, x.shape[-1])).max(axis=1)


def delta_bound(O, dO) -> np.ndarray:
    """Per row: the most D_i can be off when O_i is off by ROW_TOL_O * |O_i|_inf."""
    dO = f64(dO)
    return ROW_TOL_O * row_max(O) * np.abs(dO.reshape(-1, dO.shape[-1])).sum(axis=1)


def dq_allowance(scale, kbar, O, dO) -> np.ndarray:
    """Per query row: scale * delta_i * |kbar_i|_inf (see above)."""
    return scale * delta_bound(O, dO) * row_max(kbar)


def dk_weights(O, dO, q) -> np.ndarray:
    """w_i = delta_i * |q_i|_inf; the dK allowance of key j is scale * sum_i P_ij w_i."""
    return delta_bound(O, dO) * row_max(q)


def row_rel_err(gpu, ref, allowance=None, tol=1.0) -> np.ndarray:
    """max_c |gpu_ic - ref_ic| / den_i with den_i = max(|ref_i|_inf, allowance_i / tol,
    ROW_FLOOR * |ref|_inf): the error in units of the row's own size, or of its
    allowance where that is larger."""
    g, r = f64(gpu), f64(ref)
    g = g.reshape(-1, g.shape[-1])
    r = r.reshape(-1, r.shape[-1])
    num = np.abs(g - r).max(axis=1)
    den = np.maximum(np.abs(r).max(axis=1), ROW_FLOOR * max(float(np.abs(r).max()), 1e-300))
    if allowance is not None:
        den = np.maximum(den, np.asarray(allowance, dtype=np.float64).reshape(-1) / tol)
    return num / den


def assert_rows(gpu, ref, tol, name, allowance=None):
    e = row_rel_err(gpu, ref, allowance, tol)
    worst = int(np.argmax(e)) if e.size else 0
    err = float(e.max()) if e.size else 0.0
    assert err <= tol, f"{name}: worst row {worst}: max|gpu-oracle| / row scale = {err:.3e} > {tol}"
    return err
