"""GPU parity of the SP loss aggregation against the float64 oracle: counts
bit-exact, losses to fp32 rounding, on masks of several shapes (prompt
prefixes masked, a rank with no counted token, none anywhere, NaN in ignored
positions), aligned and unaligned slices, and the long and million workloads'
token counts."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import ulysses_sequence_parallelism_seq_amd as uly
from tests.gpu_util import device, say

pytestmark = pytest.mark.gpu

REL = 1e-6  # fp64 sums on the GPU; outputs rounded to fp32 once


def _inputs(sp, B, Ns, seed, mode):
    rng = np.random.default_rng(seed)
    tl = rng.exponential(2.0, (sp, B, Ns)).astype(np.float32)
    lab = rng.integers(0, 32000, (sp, B, Ns)).astype(np.int64)
    if mode == "random":
        lab[rng.random((sp, B, Ns)) < 0.3] = -100
    elif mode == "prompt":  # each row's first part is prompt: not counted; rank 0 entirely prompt
        for r in range(sp):
            for b in range(B):
                cut = Ns if r == 0 else int(rng.integers(0, Ns))
                lab[r, b, :cut] = -100
    elif mode == "none":
        lab[:] = -100
    tl[lab == -100] = np.where(rng.random(int((lab == -100).sum())) < 0.5, np.nan, np.inf)
    return tl, lab


def _check(tl, lab):
    dev = device()
    loss, rank_loss, good = uly.ulysses_sp_loss(torch.from_numpy(tl).to(dev), torch.from_numpy(lab).to(dev))
    torch.cuda.synchronize()
    w_loss, w_rank, w_good = oracle.sp_loss(tl, lab)
    assert np.array_equal(good.cpu().numpy(), w_good)
    got_rank = rank_loss.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got_rank))
    assert np.abs(got_rank - w_rank).max() <= REL * max(1.0, np.abs(w_rank).max())
    got = float(loss.cpu()[0])
    assert abs(got - w_loss) <= REL * max(1.0, abs(w_loss)), (got, w_loss)
    return got, w_loss


@pytest.mark.parametrize("sp,B,Ns,mode", [
    (8, 1, 16384, "random"),   # the long workload's 8 ranks
    (16, 1, 32768, "prompt"),  # the million workload's 16 ranks, rank 0 only prompt
    (4, 2, 1024, "random"),    # the llama7b workload's 4 ranks
    (3, 1, 7, "random"),       # slices not 16-byte aligned
    (5, 3, 4097, "prompt"),
    (2, 1, 64, "none"),        # no counted token anywhere
    (1, 1, 1, "random"),
])
def test_sp_loss_against_oracle(sp, B, Ns, mode):
    say("sp loss", sp, B, Ns, mode)
    tl, lab = _inputs(sp, B, Ns, 50 + sp + Ns, mode)
    got, want = _check(tl, lab)
    say(f"loss {got:.8f} oracle {want:.8f}")


def test_sp_loss_is_bit_reproducible():
    dev = device()
    tl, lab = _inputs(8, 1, 16384, 3, "random")
    a = torch.from_numpy(tl).to(dev)
    b = torch.from_numpy(lab).to(dev)
    first = [t.clone() for t in uly.ulysses_sp_loss(a, b)]
    for _ in range(3):
        again = uly.ulysses_sp_loss(a, b)
        assert all(torch.equal(x, y) for x, y in zip(first, again))
