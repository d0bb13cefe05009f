"""Oracle of the tiled MLP of ALST (TiledMLP), forward and backward (test infrastructure only).

What is computed (float64 throughout):

  * HF Transformers docs, "Ulysses sequence parallelism" (deepspeed_alst),
    the paragraph after the layout diagram, and the jianying88 page's section
    on the boundary of what Transformers integrates: Arctic Long Sequence
    Training pairs Ulysses with TiledMLP and activation-checkpoint offloading.
    The jianying88 page's account of the layout adds that after the second
    all-to-all the rest of the layer (the FFN, LayerNorm, ...) runs locally on
    each rank's own token shard. The pages name TiledMLP and say no more.
  * Reading (the plainest the rest supports): the FFN of the Llama-style
    model the workloads are shaped like (32 heads of width 128, so hidden
    h = 4096), the SwiGLU MLP
        G = X Wg^T,  U = X Wu^T,  A = silu(G) * U,  Y = A Wd^T,
    with silu(z) = z / (1 + exp(-z)), X [T, h], Wg and Wu [I, h], Wd [h, I].
    It acts on every token alone, so computing it over the rank's tokens in
    tiles of `tile` tokens, holding one tile's [tile, I] intermediates at a
    time and recomputing them in the backward, gives the same Y and dX; the
    weight gradients are sums over tokens, accumulated tile after tile.
  * Backward (analytic, with s = sigmoid(G), silu'(G) = s (1 + G (1 - s))):
        dA = dY Wd,  dWd = dY^T A,
        dG = dA * U * silu'(G),  dU = dA * silu(G),
        dX = dG Wg + dU Wu,  dWg = dG^T X,  dWu = dU^T X.

mlp_fwd / mlp_bwd are the whole-shard definition; tiled_mlp_fwd /
tiled_mlp_bwd take the tiles in order. Arrays are [tokens, features].
"""

from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().float().numpy()
    return np.asarray(x, dtype=np.float64)


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def mlp_fwd(x, wg, wu, wd):
    """Y [T, h] of the SwiGLU MLP over all tokens at once."""
    X, Wg, Wu, Wd = (_f64(a) for a in (x, wg, wu, wd))
    G = X @ Wg.T
    U = X @ Wu.T
    A = G * _sigmoid(G) * U
    return A @ Wd.T


def mlp_bwd(x, wg, wu, wd, dy):
    """(dX, dWg, dWu, dWd) of L = sum(Y * dY) over all tokens at once."""
    X, Wg, Wu, Wd, dY = (_f64(a) for a in (x, wg, wu, wd, dy))
    G = X @ Wg.T
    U = X @ Wu.T
    s = _sigmoid(G)
    silu = G * s
    A = silu * U
    dA = dY @ Wd
    dWd = dY.T @ A
    dG = dA * U * (s * (1.0 + G * (1.0 - s)))
    dU = dA * silu
    dX = dG @ Wg + dU @ Wu
    return dX, dG.T @ X, dU.T @ X, dWd


def _tiles(T: int, tile: int):
    if tile <= 0:
        raise ValueError("tile must be positive")
    return [(t0, min(T, t0 + tile)) for t0 in range(0, T, tile)]


def tiled_mlp_fwd(x, wg, wu, wd, tile: int):
    """Y computed tile by tile (each tile's intermediates exist only while it runs)."""
    X = _f64(x)
    Y = np.zeros((X.shape[0], _f64(wd).shape[0]))
    for t0, t1 in _tiles(X.shape[0], tile):
        Y[t0:t1] = mlp_fwd(X[t0:t1], wg, wu, wd)
    return Y


def tiled_mlp_bwd(x, wg, wu, wd, dy, tile: int):
    """(dX, dWg, dWu, dWd): each tile's intermediates recomputed from its X, the
    weight gradients accumulated over the tiles in order."""
    X, dY = _f64(x), _f64(dy)
    Wg, Wu, Wd = _f64(wg), _f64(wu), _f64(wd)
    dX = np.zeros_like(X)
    dWg, dWu, dWd = np.zeros_like(Wg), np.zeros_like(Wu), np.zeros_like(Wd)
    for t0, t1 in _tiles(X.shape[0], tile):
        gx, gg, gu, gd = mlp_bwd(X[t0:t1], Wg, Wu, Wd, dY[t0:t1])
        dX[t0:t1] = gx
        dWg += gg
        dWu += gu
        dWd += gd
    return dX, dWg, dWu, dWd


# ---- sampled outputs, for sizes where the whole oracle is too slow ----
# Each token's Y and dX depend on that token alone, so rows of Y and dX are
# the definition applied to those tokens (mlp_fwd / mlp_bwd on a subset). A
# weight gradient is a sum over every token: the rows below take all tokens
# but only the requested intermediate units i.


def mlp_bwd_weight_units(x, wg, wu, wd, dy, units):
    """dWg[units], dWu[units] ([len(units), h]) and dWd[:, units] ([h, len(units)])
    summed over every token, from the same definitions as mlp_bwd restricted
    to the columns i in units of G, U, A, dA, dG and dU."""
    X, dY = _f64(x), _f64(dy)
    Wg, Wu, Wd = _f64(wg), _f64(wu), _f64(wd)
    idx = np.asarray(units, dtype=np.int64)
    G = X @ Wg[idx].T
    U = X @ Wu[idx].T
    s = _sigmoid(G)
    silu = G * s
    A = silu * U
    dA = dY @ Wd[:, idx]
    dG = dA * U * (s * (1.0 + G * (1.0 - s)))
    dU = dA * silu
    return dG.T @ X, dU.T @ X, dY.T @ A
