"""Pins of the sequence-parallel loss aggregation oracle (CPU only).

What the page fixes: the weighted aggregate equals the mean over every counted
token of the whole batch; ranks without counted tokens drop out; counts are
those of labels different from -100. Checked against scalar loops, the global
mean, and special cases."""

from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from oracle import loss as L


def _case(sp, B, Ns, seed, p_ignore=0.3):
    rng = np.random.default_rng(seed)
    tl = rng.exponential(2.0, (sp, B, Ns)).astype(np.float32)
    lab = rng.integers(0, 32000, (sp, B, Ns)).astype(np.int64)
    lab[rng.random((sp, B, Ns)) < p_ignore] = -100
    return tl, lab


@pytest.mark.parametrize("sp,B,Ns,seed", [(2, 1, 7, 0), (4, 2, 33, 1), (8, 1, 128, 2), (1, 3, 5, 3)])
def test_aggregate_equals_global_mean_of_counted_tokens(sp, B, Ns, seed):
    tl, lab = _case(sp, B, Ns, seed)
    loss, _, good = oracle.sp_loss(tl, lab)
    keep = lab != -100
    assert good.sum() == keep.sum()
    assert abs(loss - tl.astype(np.float64)[keep].mean()) < 1e-12


def test_scalar_loops():
    tl, lab = _case(3, 2, 9, 5)
    loss, loss_r, good_r = oracle.sp_loss(tl, lab)
    num, den = 0.0, 0
    for r in range(3):
        s, n = 0.0, 0
        for b in range(2):
            for t in range(9):
                if lab[r, b, t] != -100:
                    s += float(tl[r, b, t])
                    n += 1
        assert good_r[r] == n
        assert math.isclose(loss_r[r], s / n if n else 0.0, rel_tol=1e-14)
        num += s
        den += n
    assert math.isclose(loss, num / den, rel_tol=1e-14)


def test_rank_without_counted_tokens_drops_out():
    tl, lab = _case(4, 1, 16, 7)
    lab[2] = -100                      # a slice made only of prompt tokens
    tl[2, 0, 3] = np.nan               # whatever its losses hold
    tl[2, 0, 4] = np.inf
    loss, loss_r, good_r = oracle.sp_loss(tl, lab)
    assert good_r[2] == 0 and loss_r[2] == 0.0 and np.isfinite(loss)
    rest = [0, 1, 3]
    want, _, _ = oracle.sp_loss(tl[rest], lab[rest])
    assert abs(loss - want) < 1e-13


def test_ignored_positions_do_not_leak():
    tl, lab = _case(2, 1, 10, 8)
    tl2 = tl.copy()
    tl2[lab == -100] = np.nan
    assert oracle.sp_loss(tl, lab)[0] == oracle.sp_loss(tl2, lab)[0]


def test_equal_counts_reduce_to_plain_mean_and_unequal_counts_do_not():
    rng = np.random.default_rng(9)
    tl = rng.random((4, 1, 8))
    lab = np.zeros((4, 1, 8), dtype=np.int64)
    loss, loss_r, _ = oracle.sp_loss(tl, lab)
    assert abs(loss - loss_r.mean()) < 1e-14
    lab[0, 0, :6] = -100               # rank 0 keeps 2 tokens, the others 8
    loss, loss_r, good = oracle.sp_loss(tl, lab)
    assert list(good) == [2, 8, 8, 8]
    assert abs(loss - (loss_r * good).sum() / good.sum()) < 1e-14
    assert abs(loss - loss_r.mean()) > 1e-3


def test_no_counted_token_anywhere():
    tl = np.ones((2, 1, 4), dtype=np.float32)
    lab = np.full((2, 1, 4), -100, dtype=np.int64)
    loss, loss_r, good = oracle.sp_loss(tl, lab)
    assert loss == 0.0 and not loss_r.any() and not good.any()


def test_aggregate_of_gathered_values():
    assert L.aggregate([2.0, 4.0, 7.0], [1, 3, 0]) == pytest.approx((2.0 + 12.0) / 4)
    assert L.aggregate([np.nan, 1.0], [0, 5]) == 1.0
