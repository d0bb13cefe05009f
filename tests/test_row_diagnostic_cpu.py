"""What the per-row bars of the GPU parity tests can see (CPU only).

At the long workload's length (131072 keys per row, inputs N(0, 0.5^2) in
bf16) with q = 0, where O and dQ have closed forms, this computes rows of O
and dQ with one 64-key tile left out and checks that the per-row diagnostic
(tests/gpu_util.py, with the dQ allowance applied) flags every such row,
while the exact values rounded to bf16 pass. So a kernel that skipped a key
tile of a late row, or zeroed late rows, fails the GPU tests even though the
per-tensor bar (relative to the tensor's largest row) could not see it.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from tests.gpu_util import ROW_TOL_GRAD, ROW_TOL_O, dq_allowance, row_rel_err

N, D = 131072, 128


@pytest.fixture(scope="module")
def head():
    g = torch.Generator().manual_seed(9)
    k, v, do = (torch.randn(N, D, generator=g) * 0.5 for _ in range(3))
    return tuple(x.to(torch.bfloat16).double().numpy() for x in (k, v, do))


def _row(k, v, do, i, keep):
    """O_i and dQ_i of query i when q = 0 and only the keys in keep are visible:
    P uniform over them (hand-derived, as in tests/closed_forms.py)."""
    Kp, Vp = k[:i + 1][keep], v[:i + 1][keep]
    O = Vp.mean(axis=0)
    Di = do[i] @ O
    dq = (Vp @ do[i] - Di) @ Kp / len(Vp) / math.sqrt(D)
    return O, dq, Kp.mean(axis=0)


def _tiles(i):
    """First, middle and last full 64-key tiles of query i's keys."""
    full = (i + 1) // 64
    return sorted({0, full // 2, full - 1})


@pytest.mark.parametrize("i", [N - 1, N // 2 + 17, 4096 + 5, 300])
def test_missing_key_tile_is_flagged(head, i):
    k, v, do = head
    allk = np.ones(i + 1, dtype=bool)
    O, dq, kbar = _row(k, v, do, i, allk)
    allow = dq_allowance(1 / math.sqrt(D), kbar[None], O[None], do[i][None])
    for t in _tiles(i):
        keep = allk.copy()
        keep[64 * t:64 * t + 64] = False
        O_m, dq_m, _ = _row(k, v, do, i, keep)
        e_o = float(row_rel_err(O_m[None], O[None])[0])
        e_q = float(row_rel_err(dq_m[None], dq[None], allow, ROW_TOL_GRAD)[0])
        assert e_o > ROW_TOL_O, (i, t, e_o)
        assert e_q > ROW_TOL_GRAD, (i, t, e_q)


def test_zeroed_late_rows_are_flagged(head):
    k, v, do = head
    rows = [N - 1, N - 1000, N // 2]
    for i in rows:
        O, dq, kbar = _row(k, v, do, i, np.ones(i + 1, dtype=bool))
        allow = dq_allowance(1 / math.sqrt(D), kbar[None], O[None], do[i][None])
        assert row_rel_err(np.zeros((1, D)), O[None])[0] == pytest.approx(1.0)
        assert row_rel_err(np.zeros((1, D)), dq[None], allow, ROW_TOL_GRAD)[0] > 0.9


def test_bf16_rounding_of_exact_rows_passes(head):
    k, v, do = head
    for i in (0, 1, 63, 64, 4095, N // 2, N - 1):
        O, dq, kbar = _row(k, v, do, i, np.ones(i + 1, dtype=bool))
        allow = dq_allowance(1 / math.sqrt(D), kbar[None], O[None], do[i][None])
        rb = lambda x: torch.from_numpy(x).to(torch.bfloat16).double().numpy()  # noqa: E731
        assert row_rel_err(rb(O)[None], O[None])[0] <= 2.0 ** -8 < ROW_TOL_O / 2
        assert row_rel_err(rb(dq)[None], dq[None], allow, ROW_TOL_GRAD)[0] <= 2.0 ** -8 < ROW_TOL_GRAD / 2
