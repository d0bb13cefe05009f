"""Pins of the tiled-MLP oracle (CPU only): pure-Python loops, finite
differences, torch's float64 autograd, closed forms with a zero weight,
token independence, and tiled == whole-shard for every tile size. Planted
mistakes (each a plausible slip) must fail some pin."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle.mlp as om


def _rand(rng, *shape, s=1.0):
    return rng.standard_normal(shape) * s


def _inputs(seed, T=7, h=5, I=6):
    rng = np.random.default_rng(seed)
    return (_rand(rng, T, h), _rand(rng, I, h, s=0.5), _rand(rng, I, h, s=0.5), _rand(rng, h, I, s=0.5),
            _rand(rng, T, h))


def check_forward_loops():
    x, wg, wu, wd, _ = _inputs(1)
    T, h = x.shape
    I = wg.shape[0]
    Y = om.mlp_fwd(x, wg, wu, wd)
    for t in range(T):
        a = []
        for i in range(I):
            g = sum(x[t][c] * wg[i][c] for c in range(h))
            u = sum(x[t][c] * wu[i][c] for c in range(h))
            a.append(g / (1.0 + math.exp(-g)) * u)
        for c in range(h):
            assert abs(Y[t][c] - sum(a[i] * wd[c][i] for i in range(I))) < 1e-12


def check_backward_finite_differences():
    x, wg, wu, wd, dy = _inputs(2)
    grads = om.mlp_bwd(x, wg, wu, wd, dy)
    eps = 1e-6

    def loss(args):
        return float((om.mlp_fwd(*args) * dy).sum())

    base = [x, wg, wu, wd]
    for which, g in zip((0, 1, 2, 3), grads):
        num = np.zeros_like(g)
        for idx in np.ndindex(*g.shape):
            up = [a.copy() for a in base]
            dn = [a.copy() for a in base]
            up[which][idx] += eps
            dn[which][idx] -= eps
            num[idx] = (loss(up) - loss(dn)) / (2 * eps)
        err = np.abs(num - g).max() / max(np.abs(g).max(), 1e-30)
        assert err <= 1e-6, (which, err)


def check_vs_torch_autograd():
    x, wg, wu, wd, dy = _inputs(3, T=11, h=8, I=12)
    tx, tg, tu, td = (torch.tensor(a, requires_grad=True) for a in (x, wg, wu, wd))
    ty = (torch.nn.functional.silu(tx @ tg.T) * (tx @ tu.T)) @ td.T
    ty.backward(torch.tensor(dy))
    np.testing.assert_allclose(om.mlp_fwd(x, wg, wu, wd), ty.detach().numpy(), rtol=1e-12, atol=1e-13)
    for mine, t in zip(om.mlp_bwd(x, wg, wu, wd, dy), (tx, tg, tu, td)):
        np.testing.assert_allclose(mine, t.grad.numpy(), rtol=1e-11, atol=1e-12)


def check_zero_weight_closed_forms():
    x, wg, wu, wd, dy = _inputs(4)
    # Wg = 0: G = 0, silu(0) = 0 and silu'(0) = 1/2, so A = 0 and Y = 0;
    # dA = dY Wd, dG = dA * U / 2, dU = 0: dX = dG Wg = 0, dWg = dG^T X, dWu = dWd = 0
    z = np.zeros_like(wg)
    assert np.abs(om.mlp_fwd(x, z, wu, wd)).max() == 0
    dx, dwg, dwu, dwd = om.mlp_bwd(x, z, wu, wd, dy)
    assert np.abs(dx).max() == 0 and np.abs(dwu).max() == 0 and np.abs(dwd).max() == 0
    dG = (dy @ wd) * (x @ wu.T) / 2
    np.testing.assert_allclose(dwg, dG.T @ x, rtol=1e-13, atol=1e-14)
    # Wu = 0: U = 0, A = 0, Y = 0; dG = 0 and dU = dA * silu(G): dWu = dU^T X, the rest 0
    dx, dwg, dwu, dwd = om.mlp_bwd(x, wg, z, wd, dy)
    G = x @ wg.T
    dU = (dy @ wd) * G / (1 + np.exp(-G))
    assert np.abs(dx).max() == 0 and np.abs(dwg).max() == 0 and np.abs(dwd).max() == 0
    np.testing.assert_allclose(dwu, dU.T @ x, rtol=1e-13, atol=1e-14)
    # Wd = 0: Y = 0, dA = 0, every gradient but dWd vanishes; dWd = dY^T A
    dx, dwg, dwu, dwd = om.mlp_bwd(x, wg, wu, np.zeros_like(wd), dy)
    A = G / (1 + np.exp(-G)) * (x @ wu.T)
    assert np.abs(dx).max() == 0 and np.abs(dwg).max() == 0 and np.abs(dwu).max() == 0
    np.testing.assert_allclose(dwd, dy.T @ A, rtol=1e-13, atol=1e-14)


def check_tiled_equals_whole():
    x, wg, wu, wd, dy = _inputs(5, T=23, h=6, I=9)
    Y = om.mlp_fwd(x, wg, wu, wd)
    G = om.mlp_bwd(x, wg, wu, wd, dy)
    for tile in (1, 4, 7, 22, 23, 64):  # ragged last tiles, one tile, tile > tokens
        np.testing.assert_allclose(om.tiled_mlp_fwd(x, wg, wu, wd, tile), Y, rtol=1e-13, atol=1e-13)
        for a, b in zip(om.tiled_mlp_bwd(x, wg, wu, wd, dy, tile), G):
            np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def check_token_independence():
    x, wg, wu, wd, dy = _inputs(6, T=9)
    perm = np.random.default_rng(0).permutation(9)
    np.testing.assert_allclose(om.mlp_fwd(x[perm], wg, wu, wd), om.mlp_fwd(x, wg, wu, wd)[perm], rtol=1e-13)
    a = om.mlp_bwd(x[perm], wg, wu, wd, dy[perm])
    b = om.mlp_bwd(x, wg, wu, wd, dy)
    np.testing.assert_allclose(a[0], b[0][perm], rtol=1e-12, atol=1e-13)
    for u, v in zip(a[1:], b[1:]):
        np.testing.assert_allclose(u, v, rtol=1e-12, atol=1e-13)


PINS = [check_forward_loops, check_backward_finite_differences, check_vs_torch_autograd,
        check_zero_weight_closed_forms, check_tiled_equals_whole, check_token_independence]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_weight_units_match_whole():
    x, wg, wu, wd, dy = _inputs(8, T=13, h=6, I=10)
    _, dwg, dwu, dwd = om.mlp_bwd(x, wg, wu, wd, dy)
    units = [0, 3, 9, 4]
    a, b, c = om.mlp_bwd_weight_units(x, wg, wu, wd, dy, units)
    np.testing.assert_allclose(a, dwg[units], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(b, dwu[units], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(c, dwd[:, units], rtol=1e-12, atol=1e-13)


def test_rejects_bad_tile():
    x, wg, wu, wd, dy = _inputs(7)
    with pytest.raises(ValueError):
        om.tiled_mlp_fwd(x, wg, wu, wd, 0)


def _mutants():
    orig_bwd = om.mlp_bwd

    def silu_grad_as_sigmoid(x, wg, wu, wd, dy):
        X, Wg, Wu, Wd, dY = (np.asarray(a, dtype=np.float64) for a in (x, wg, wu, wd, dy))
        G, U = X @ Wg.T, X @ Wu.T
        s = 1 / (1 + np.exp(-G))
        A = G * s * U
        dA = dY @ Wd
        dG = dA * U * s  # drops the G (1 - s) term of silu'
        dU = dA * G * s
        return dG @ Wg + dU @ Wu, dG.T @ X, dU.T @ X, dY.T @ A

    def gate_and_up_swapped(x, wg, wu, wd, dy):
        dx, dwg, dwu, dwd = orig_bwd(x, wg, wu, wd, dy)
        return dx, dwu, dwg, dwd

    def fwd_gelu_tanh(x, wg, wu, wd):
        X = np.asarray(x, dtype=np.float64)
        G = X @ np.asarray(wg).T
        gel = 0.5 * G * (1 + np.tanh(math.sqrt(2 / math.pi) * (G + 0.044715 * G ** 3)))
        return (gel * (X @ np.asarray(wu).T)) @ np.asarray(wd).T

    def tiled_bwd_last_tile_dropped(x, wg, wu, wd, dy, tile):
        X = np.asarray(x, dtype=np.float64)
        keep = (X.shape[0] // tile) * tile or X.shape[0]
        out = list(orig_bwd(X[:keep], wg, wu, wd, np.asarray(dy)[:keep]))
        dx = np.zeros_like(X)
        dx[:keep] = out[0]
        return (dx, *out[1:])

    def tiled_bwd_overwrites(x, wg, wu, wd, dy, tile):
        X, dY = np.asarray(x, dtype=np.float64), np.asarray(dy, dtype=np.float64)
        dX = np.zeros_like(X)
        res = None
        for t0 in range(0, X.shape[0], tile):
            res = orig_bwd(X[t0:t0 + tile], wg, wu, wd, dY[t0:t0 + tile])
            dX[t0:t0 + tile] = res[0]
        return (dX, *res[1:])

    return {
        "silu' without its G(1 - s) term": ("mlp_bwd", silu_grad_as_sigmoid),
        "dWg and dWu swapped": ("mlp_bwd", gate_and_up_swapped),
        "gelu instead of silu": ("mlp_fwd", fwd_gelu_tanh),
        "ragged last tile dropped": ("tiled_mlp_bwd", tiled_bwd_last_tile_dropped),
        "weight gradients overwritten per tile": ("tiled_mlp_bwd", tiled_bwd_overwrites),
    }


@pytest.mark.parametrize("name", list(_mutants().keys()))
def test_pins_catch_planted_mistakes(name, monkeypatch):
    attr, fn = _mutants()[name]
    monkeypatch.setattr(om, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake: {name}"
