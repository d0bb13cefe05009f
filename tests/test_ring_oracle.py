"""Pins of the ring-attention oracle (CPU only).

The pages print no worked example for ring attention, so the oracle is pinned
to what the mathematics fixes: after all ring steps it must equal exact
attention over the stitched sequence (the independently pinned attention
oracle); the log-sum-exp merge must equal a softmax over the union of two
key sets (scalar loops); the running state after each step must equal
attention over exactly the keys visited so far (scalar loops); the backward's
per-step sums must add up to the analytic gradient.
"""

from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from oracle import ring



def _inputs(sp, B, Ns, H, d, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((sp, B, Ns, H, d)) for _ in range(4)]


@pytest.mark.parametrize("sp", [1, 2, 3, 4])
@pytest.mark.parametrize("causal", [True, False])
def test_ring_forward_equals_full_attention(sp, causal):
    q, k, v, _ = _inputs(sp, 2, 5, 2, 8, 10 + sp)
    o, lse = ring.ring_fwd(q, k, v, causal)
    O, L = oracle.attn_fwd(ring.stitch(q), ring.stitch(k), ring.stitch(v), None, causal)
    assert np.abs(ring.stitch(o) - O).max() < 1e-12
    assert np.abs(ring.stitch_lse(lse) - L).max() < 1e-12


@pytest.mark.parametrize("sp", [1, 2, 3, 4])
@pytest.mark.parametrize("causal", [True, False])
def test_ring_backward_equals_full_gradient(sp, causal):
    q, k, v, do = _inputs(sp, 2, 5, 2, 8, 20 + sp)
    o, lse = ring.ring_fwd(q, k, v, causal)
    dq, dk, dv = ring.ring_bwd(q, k, v, do, o, lse, causal)
    G = oracle.attn_bwd(ring.stitch(q), ring.stitch(k), ring.stitch(v), ring.stitch(do), None, causal)
    for got, want in zip((dq, dk, dv), G):
        assert np.abs(ring.stitch(got) - want).max() < 1e-11


def _softmax_loops(qrow, keys, vals, scale):
    """Softmax attention of one query row over the given key/value rows, scalar loops."""
    s = [scale * sum(qrow[c] * kr[c] for c in range(len(qrow))) for kr in keys]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    tot = sum(w)
    out = [sum(w[n] * vals[n][c] for n in range(len(keys))) / tot for c in range(len(vals[0]))]
    return out, m + math.log(tot)


def test_merge_equals_softmax_over_union():
    rng = np.random.default_rng(3)
    d, na, nb = 6, 4, 7
    q = rng.standard_normal((1, d))
    ka, va = rng.standard_normal((na, d)) * 2, rng.standard_normal((na, d))
    kb, vb = rng.standard_normal((nb, d)) * 2, rng.standard_normal((nb, d))
    Oa, La = ring.block_attn(q, ka, va, "full")
    Ob, Lb = ring.block_attn(q, kb, vb, "full")
    O, L = ring.merge(Oa, La, Ob, Lb)
    want, want_l = _softmax_loops(q[0], list(ka) + list(kb), list(va) + list(vb), 1 / math.sqrt(d))
    assert np.abs(O[0] - np.array(want)).max() < 1e-13
    assert abs(L[0] - want_l) < 1e-13


def test_merge_with_empty_partial_is_identity():
    rng = np.random.default_rng(4)
    O = rng.standard_normal((3, 5))
    L = rng.standard_normal(3)
    Om, Lm = ring.merge(O, L, np.zeros((3, 5)), np.full(3, -np.inf))
    assert np.array_equal(Lm, L) and np.abs(Om - O).max() < 1e-15


def test_block_modes_and_rotation():
    sp = 4
    # step i: rank r holds chunk r - i (mod sp); over sp steps every rank sees every chunk once
    for r in range(sp):
        assert sorted(ring.ring_chunk(r, i, sp) for i in range(sp)) == list(range(sp))
        assert ring.ring_chunk(r, 0, sp) == r
        assert ring.ring_chunk(r, 1, sp) == (r - 1) % sp
    # at every step each chunk sits on exactly one rank
    for i in range(sp):
        assert sorted(ring.ring_chunk(r, i, sp) for r in range(sp)) == list(range(sp))
    assert [ring.block_mode(2, j, True) for j in range(4)] == ["full", "full", "diag", "none"]
    assert [ring.block_mode(2, j, False) for j in range(4)] == ["full"] * 4


@pytest.mark.parametrize("causal", [True, False])
def test_running_state_after_each_step(causal):
    """After step i, rank r's (o, lse) is attention over exactly the allowed keys of
    the chunks it has held so far, chunk r - i' (mod sp) for i' <= i (scalar loops)."""
    sp, B, Ns, H, d = 3, 1, 3, 2, 4
    q, k, v, _ = _inputs(sp, B, Ns, H, d, 5)
    scale = 1 / math.sqrt(d)
    for steps in range(1, sp + 1):
        o, lse = ring.ring_fwd(q, k, v, causal, steps=steps)
        for r in range(sp):
            for h in range(H):
                for t in range(Ns):
                    gi = r * Ns + t
                    keys, vals = [], []
                    for i in range(steps):
                        j = (r - i) % sp
                        for u in range(Ns):
                            if not causal or j * Ns + u <= gi:
                                keys.append(k[j, 0, u, h])
                                vals.append(v[j, 0, u, h])
                    if not keys:
                        assert np.isneginf(lse[r, 0, h, t]) and not np.any(o[r, 0, t, h])
                        continue
                    want, want_l = _softmax_loops(q[r, 0, t, h], keys, vals, scale)
                    assert np.abs(o[r, 0, t, h] - np.array(want)).max() < 1e-12
                    assert abs(lse[r, 0, h, t] - want_l) < 1e-12


@pytest.mark.parametrize("causal", [True, False])
def test_backward_partial_sums_after_each_step(causal):
    """After step i, dq[r] sums the terms of keys in chunks rank r has held and
    dk[j], dv[j] those of queries of ranks chunk j has visited (scalar loops,
    P from the final lse, D = rowsum(dO * O))."""
    sp, B, Ns, H, d = 3, 1, 2, 1, 3
    q, k, v, do = _inputs(sp, B, Ns, H, d, 6)
    scale = 1 / math.sqrt(d)
    o, lse = ring.ring_fwd(q, k, v, causal)
    for steps in range(1, sp + 1):
        dq, dk, dv = ring.ring_bwd(q, k, v, do, o, lse, causal, steps=steps)
        wq, wk, wv = np.zeros_like(dq), np.zeros_like(dk), np.zeros_like(dv)
        for i in range(steps):
            for r in range(sp):
                j = (r - i) % sp
                for t in range(Ns):
                    Dt = sum(do[r, 0, t, 0, c] * o[r, 0, t, 0, c] for c in range(d))
                    for u in range(Ns):
                        if causal and j * Ns + u > r * Ns + t:
                            continue
                        sc = scale * sum(q[r, 0, t, 0, c] * k[j, 0, u, 0, c] for c in range(d))
                        p = math.exp(sc - lse[r, 0, 0, t])
                        dp = sum(do[r, 0, t, 0, c] * v[j, 0, u, 0, c] for c in range(d))
                        ds = p * (dp - Dt)
                        for c in range(d):
                            wq[r, 0, t, 0, c] += scale * ds * k[j, 0, u, 0, c]
                            wk[j, 0, u, 0, c] += scale * ds * q[r, 0, t, 0, c]
                            wv[j, 0, u, 0, c] += p * do[r, 0, t, 0, c]
        for got, want in ((dq, wq), (dk, wk), (dv, wv)):
            assert np.abs(got - want).max() < 1e-12


def test_chunk_rows_split_matches_whole_block(monkeypatch):
    """Evaluating a block in row chunks changes nothing (the diagonal mask uses block-local rows)."""
    rng = np.random.default_rng(7)
    Qc, Kc, Vc = (rng.standard_normal((10, 4)) for _ in range(3))
    whole = ring.block_attn(Qc, Kc, Vc, "diag")
    monkeypatch.setattr(ring, "_CHUNK_ROWS", 3)
    split = ring.block_attn(Qc, Kc, Vc, "diag")
    assert np.abs(whole[0] - split[0]).max() < 1e-15 and np.abs(whole[1] - split[1]).max() < 1e-15
