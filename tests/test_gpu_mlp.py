"""The tiled MLP on the GPU against the float64 oracle: small shapes with
ragged token counts and tiles (every output), tiled == one tile on the GPU,
and the long workload's per-rank shape (16384 tokens, hidden 4096, inter
11008) on sampled tokens and sampled intermediate units."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
import ulysses_sequence_parallelism_seq_amd as uly
from tests.gpu_util import TOL_BF16_GRAD, TOL_BF16_O, assert_rel, assert_rows, device, f64, say

pytestmark = pytest.mark.gpu

# Per-row bars: each token's row of y and dx, each row of a weight gradient,
# against its own size. The operands are bf16; the intermediates A, dG, dU
# and the backward's factors U * silu'(G), silu(G) are stored in bf16 between
# the products; accumulation is fp32. Measured worst rows: 0.50% (y), 0.63%
# (dx and the weight gradients), against 2^-8 = 0.39% for the rounding of
# one bf16 output alone.
ROW_TOL_Y = 1e-2
ROW_TOL_G = 1.5e-2


def _run(x, wg, wu, wd, dy, tile):
    dev = device()
    xd, gd, ud, dd, dyd = (t.to(dev) for t in (x, wg, wu, wd, dy))
    y = uly.ulysses_tiled_mlp_fwd(xd, gd, ud, dd, tile)
    grads = uly.ulysses_tiled_mlp_bwd(xd, gd, ud, dd, dyd, tile)
    torch.cuda.synchronize()
    return (y.cpu(),) + tuple(t.cpu() for t in grads)


@pytest.mark.parametrize("tokens,hidden,inter,tile", [
    (700, 256, 512, 256),    # ragged last tile (188 tokens), ragged M tile
    (700, 256, 512, 1000),   # one tile larger than the tokens
    (300, 512, 256, 64),     # many small tiles
    (1, 256, 256, 256),      # a single token
    (513, 256, 768, 300),    # tile not a multiple of the 64-token K step
])
def test_mlp_parity(tokens, hidden, inter, tile):
    say("tiled mlp", tokens, hidden, inter, tile)
    x, wg, wu, wd, dy = workloads.mlp_inputs(tokens, hidden, inter, 11 + tokens)
    y, dx, dwg, dwu, dwd = _run(x, wg, wu, wd, dy, tile)
    Y = oracle.mlp_fwd(x, wg, wu, wd)
    G = oracle.mlp_bwd(x, wg, wu, wd, dy)
    errs = {"y": assert_rel(y, Y, TOL_BF16_O, "y")}
    for name, got, want in zip(("dx", "dWg", "dWu", "dWd"), (dx, dwg, dwu, dwd), G):
        errs[name] = assert_rel(got, want, TOL_BF16_GRAD, name)
    rows = {"y": assert_rows(y, Y, ROW_TOL_Y, "y")}
    for name, got, want in zip(("dx", "dWg", "dWu", "dWd"), (dx, dwg, dwu, dwd), G):
        rows[name] = assert_rows(got, want, ROW_TOL_G, name)
    say("per tensor", errs, "worst row", rows)


def test_mlp_tiles_equal_one_tile():
    """Tiling changes nothing but the order of the weight-gradient sums: y and
    dx are bit-identical, the weight gradients agree to fp32 rounding."""
    say("tiled mlp: tiles == one tile")
    x, wg, wu, wd, dy = workloads.mlp_inputs(1000, 256, 512, 5)
    one = _run(x, wg, wu, wd, dy, 1000)
    tiled = _run(x, wg, wu, wd, dy, 128)
    assert torch.equal(one[0], tiled[0]) and torch.equal(one[1], tiled[1])
    for a, b in zip(one[2:], tiled[2:]):
        assert float((a - b).abs().max()) <= 1e-5 * float(a.abs().max())


def test_mlp_long_shape_sampled():
    """One rank's shard of the long workload (16384 tokens) through the Llama-7B
    FFN (hidden 4096, inter 11008) in tiles of 4096: sampled token rows of y
    and dx, and sampled intermediate units of the weight gradients (their sums
    run over every token), against the oracle."""
    tokens, hidden, inter, tile = 16384, workloads.MLP_HIDDEN, workloads.MLP_INTER, 4096
    say("tiled mlp long shape", tokens, hidden, inter, tile)
    x, wg, wu, wd, dy = workloads.mlp_inputs(tokens, hidden, inter, 4)
    y, dx, dwg, dwu, dwd = _run(x, wg, wu, wd, dy, tile)
    rng = np.random.default_rng(4)
    rows = sorted(set([0, 1, 4095, 4096, 8191, 12288, tokens - 1]) | set(rng.integers(0, tokens, 25).tolist()))
    units = sorted(set([0, 127, 128, inter - 1]) | set(rng.integers(0, inter, 8).tolist()))
    Y = oracle.mlp_fwd(x[rows], wg, wu, wd)
    dX = oracle.mlp_bwd(x[rows], wg, wu, wd, dy[rows])[0]
    dWg, dWu, dWd = oracle.mlp_bwd_weight_units(x, wg, wu, wd, dy, units)
    got = {"y": f64(y)[rows], "dx": f64(dx)[rows], "dWg": f64(dwg)[units], "dWu": f64(dwu)[units],
           "dWd": f64(dwd)[:, units].T}
    want = {"y": Y, "dx": dX, "dWg": dWg, "dWu": dWu, "dWd": dWd.T}
    for name in got:
        tol = TOL_BF16_O if name == "y" else TOL_BF16_GRAD
        e = assert_rel(got[name], want[name], tol, name)
        r = assert_rows(got[name], want[name], ROW_TOL_Y if name == "y" else ROW_TOL_G, name)
        say(f"{name} rel err {e:.3e}, worst row {r:.3e}")
