"""Pins of the float64 oracle against things other than itself (CPU only).

Each check compares the oracle with an independent fact: a worked example
read off the pages' layout diagram, a pure-Python brute force, closed forms,
finite differences, torch's own float64 attention, or an invariant the pages
state (heads are independent; packed samples do not see each other; the
second all-to-all undoes the first). The last test plants mistakes in the
oracle and checks that some pin catches each one.
"""

from __future__ import annotations

import math
import os

import numpy as np
import pytest
import torch

import oracle
import oracle.attention as oatt
import oracle.permute as operm
from tests import closed_forms as cf
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG_SEED = 1234


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _lengths_to_cu(lengths):
    return workloads.cu_seqlens_from_lengths(lengths)


# ---------------------------------------------------------------- permute pins


def check_permute_golden_diagram():
    rows = {}
    with open(os.path.join(GOLDEN, "permute_diagram_2gpu.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            head, vals = line.split(":")
            kind, rank = head.split()
            rows[(kind, int(rank))] = [int(x) for x in vals.split()]
    seq = np.stack([np.array(rows[("seq", r)]).reshape(1, 2, 2, 1) for r in range(2)])
    head = np.stack([np.array(rows[("head", r)]).reshape(1, 4, 1, 1) for r in range(2)])
    assert np.array_equal(operm.seq_to_head(seq), head)
    assert np.array_equal(operm.head_to_seq(head), seq)


def check_permute_index_formula():
    """Element by element: out[r][b][s*Ns+t][h'] = in[s][b][t][r*Hl+h'] (pure Python loops)."""
    sp, B, Ns, H, d = 3, 2, 2, 6, 2
    Hl = H // sp
    x = np.arange(sp * B * Ns * H * d, dtype=np.int64).reshape(sp, B, Ns, H, d)
    y = operm.seq_to_head(x)
    assert y.shape == (sp, B, sp * Ns, Hl, d)
    for r in range(sp):
        for b in range(B):
            for s in range(sp):
                for t in range(Ns):
                    for hh in range(Hl):
                        for c in range(d):
                            assert y[r, b, s * Ns + t, hh, c] == x[s, b, t, r * Hl + hh, c]
    z = operm.head_to_seq(y)
    for s in range(sp):
        for b in range(B):
            for t in range(Ns):
                for h in range(H):
                    for c in range(d):
                        assert z[s, b, t, h, c] == y[h // Hl, b, s * Ns + t, h % Hl, c]


def test_permute_golden_diagram():
    check_permute_golden_diagram()


def test_permute_index_formula():
    check_permute_index_formula()


@pytest.mark.parametrize("sp,B,Ns,H,d", [(2, 1, 128, 4, 64), (4, 2, 8, 32, 16), (1, 3, 5, 2, 8), (8, 1, 3, 8, 4)])
def test_permute_roundtrip_bits(sp, B, Ns, H, d):
    x = workloads.random_bits((sp, B, Ns, H, d), seed=sp * 100 + H, dtype="bf16").view(torch.int16).numpy()
    y = operm.seq_to_head(x)
    assert np.array_equal(operm.head_to_seq(y), x)
    h = workloads.random_bits((sp, B, Ns * sp, H // sp, d), seed=7, dtype="fp32").view(torch.int32).numpy()
    assert np.array_equal(operm.seq_to_head(operm.head_to_seq(h)), h)


def test_permute_single_rank_is_copy():
    x = np.arange(2 * 5 * 4 * 3).reshape(1, 2, 5, 4, 3)
    assert np.array_equal(operm.seq_to_head(x), x)
    assert np.array_equal(operm.head_to_seq(x), x)


def test_permute_rejects_bad_shapes():
    with pytest.raises(ValueError):
        operm.seq_to_head(np.zeros((3, 1, 2, 4, 1)))


# -------------------------------------------------------------- forward pins


def brute_forward(q, k, v, doc, causal):
    """Pure-Python attention of one head: loops over tokens, a doc-id mask, math.exp."""
    N, d = len(q), len(q[0])
    sc = 1.0 / math.sqrt(d)
    O, LSE = [], []
    for i in range(N):
        keys = [j for j in range(N) if doc[j] == doc[i] and (not causal or j <= i)]
        s = {j: sc * sum(q[i][c] * k[j][c] for c in range(d)) for j in keys}
        m = max(s.values())
        z = sum(math.exp(x - m) for x in s.values())
        O.append([sum(math.exp(s[j] - m) * v[j][c] for j in keys) / z for c in range(d)])
        LSE.append(m + math.log(z))
    return np.array(O), np.array(LSE)


def check_forward_bruteforce():
    rng = np.random.default_rng(RNG_SEED)
    N, H, d = 7, 2, 3
    for causal in (True, False):
        for lengths in ([7], [3, 4], [1, 5, 1], [2, 0, 5]):
            cu = _lengths_to_cu(lengths)
            q, k, v = (_rand(rng, 2, N, H, d) for _ in range(3))
            O, LSE = oracle.attn_fwd(q, k, v, cu, causal)
            doc = oatt.doc_ids(N, cu)
            for b in range(2):
                for h in range(H):
                    Ob, Lb = brute_forward(q[b, :, h].tolist(), k[b, :, h].tolist(), v[b, :, h].tolist(), doc, causal)
                    np.testing.assert_allclose(O[b, :, h], Ob, rtol=1e-12, atol=1e-13)
                    np.testing.assert_allclose(LSE[b, h], Lb, rtol=1e-12, atol=1e-13)


def check_forward_q0_closed_form():
    rng = np.random.default_rng(RNG_SEED + 1)
    N, H, d = 200, 2, 8
    cu = _lengths_to_cu([37, 1, 90, 0, 72])
    for causal in (True, False):
        for c in (None, cu):
            q = np.zeros((N, H, d))
            k, v = _rand(rng, N, H, d), _rand(rng, N, H, d)
            O, LSE = oracle.attn_fwd(q, k, v, c, causal)
            for h in range(H):
                Oc, Lc = cf.q0_forward(v[:, h], c, causal)
                np.testing.assert_allclose(O[:, h], Oc, rtol=1e-12, atol=1e-12)
                np.testing.assert_allclose(LSE[h], Lc, rtol=1e-12, atol=1e-12)


def check_forward_single_token_docs():
    rng = np.random.default_rng(RNG_SEED + 2)
    N, H, d = 9, 3, 5
    cu = _lengths_to_cu([1] * N)
    q, k, v = (_rand(rng, N, H, d) for _ in range(3))
    O, LSE = oracle.attn_fwd(q, k, v, cu, causal=False)
    np.testing.assert_allclose(O, v, rtol=0, atol=1e-14)
    np.testing.assert_allclose(LSE, (q * k).sum(-1).T / math.sqrt(d), rtol=1e-13, atol=1e-14)


def check_forward_vs_torch():
    rng = np.random.default_rng(RNG_SEED + 3)
    N, H, d = 48, 2, 16
    lengths = [20, 28]
    cu = _lengths_to_cu(lengths)
    q, k, v, do = (_rand(rng, N, H, d) for _ in range(4))
    for causal in (True, False):
        O, LSE = oracle.attn_fwd(q, k, v, cu, causal)
        dq, dk, dv = oracle.attn_bwd(q, k, v, do, cu, causal)
        for s, e in zip(cu[:-1], cu[1:]):
            tq, tk, tv = (torch.tensor(x[s:e]).permute(1, 0, 2).contiguous().requires_grad_(True) for x in (q, k, v))
            to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal)
            to.backward(torch.tensor(do[s:e]).permute(1, 0, 2))
            np.testing.assert_allclose(O[s:e], to.detach().permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-12)
            for mine, t in ((dq, tq), (dk, tk), (dv, tv)):
                np.testing.assert_allclose(mine[s:e], t.grad.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-11)
            # torch's logsumexp of the masked scaled scores
            S = torch.einsum("hid,hjd->hij", tq.detach(), tk.detach()) / math.sqrt(d)
            if causal:
                S = S.masked_fill(torch.ones(e - s, e - s, dtype=torch.bool).triu(1), float("-inf"))
            np.testing.assert_allclose(LSE[:, s:e], torch.logsumexp(S, dim=-1).numpy(), rtol=1e-12, atol=1e-12)


def test_forward_bruteforce():
    check_forward_bruteforce()


def test_forward_q0_closed_form():
    check_forward_q0_closed_form()


def test_forward_single_token_docs():
    check_forward_single_token_docs()


def test_forward_and_backward_vs_torch_float64():
    check_forward_vs_torch()


def test_forward_constant_v():
    rng = np.random.default_rng(RNG_SEED + 4)
    N, H, d = 64, 2, 8
    q, k = _rand(rng, N, H, d), _rand(rng, N, H, d)
    c = _rand(rng, H, d)
    v = np.broadcast_to(c[None], (N, H, d)).copy()
    for causal in (True, False):
        O, _ = oracle.attn_fwd(q, k, v, _lengths_to_cu([10, 54]), causal)
        np.testing.assert_allclose(O, v, rtol=1e-13, atol=1e-13)


def test_forward_key_shift():
    """Adding c to every key leaves O alone and moves lse_i by q_i . c / sqrt(d)."""
    rng = np.random.default_rng(RNG_SEED + 5)
    N, H, d = 40, 2, 8
    q, k, v = (_rand(rng, N, H, d) for _ in range(3))
    c = _rand(rng, H, d)
    O1, L1 = oracle.attn_fwd(q, k, v)
    O2, L2 = oracle.attn_fwd(q, k + c[None], v)
    np.testing.assert_allclose(O2, O1, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(L2 - L1, (q * c[None]).sum(-1).T / math.sqrt(d), rtol=1e-11, atol=1e-11)


def test_packed_equals_separate():
    """Guide, sp_attn_implementation paragraph: packed samples must not see each other."""
    rng = np.random.default_rng(RNG_SEED + 6)
    N, H, d = 90, 2, 8
    lengths = [25, 1, 0, 40, 24]
    cu = _lengths_to_cu(lengths)
    q, k, v, do = (_rand(rng, 2, N, H, d) for _ in range(4))
    for causal in (True, False):
        O, LSE = oracle.attn_fwd(q, k, v, cu, causal)
        grads = oracle.attn_bwd(q, k, v, do, cu, causal)
        for s, e in zip(cu[:-1], cu[1:]):
            if s == e:
                continue
            Os, Ls = oracle.attn_fwd(q[:, s:e], k[:, s:e], v[:, s:e], None, causal)
            gs = oracle.attn_bwd(q[:, s:e], k[:, s:e], v[:, s:e], do[:, s:e], None, causal)
            np.testing.assert_allclose(O[:, s:e], Os, rtol=1e-13, atol=1e-14)
            np.testing.assert_allclose(LSE[..., s:e], Ls, rtol=1e-13, atol=1e-14)
            for g, g1 in zip(grads, gs):
                np.testing.assert_allclose(g[:, s:e], g1, rtol=1e-13, atol=1e-14)


def test_packed_differs_from_unpacked():
    """The mask matters: dropping it (one document) changes rows after the first boundary."""
    rng = np.random.default_rng(RNG_SEED + 7)
    N, H, d = 32, 1, 4
    q, k, v = (_rand(rng, N, H, d) for _ in range(3))
    O_packed, _ = oracle.attn_fwd(q, k, v, _lengths_to_cu([16, 16]))
    O_one, _ = oracle.attn_fwd(q, k, v)
    np.testing.assert_allclose(O_packed[:16], O_one[:16], rtol=1e-13)
    assert np.abs(O_packed[16:] - O_one[16:]).max() > 1e-3


def test_head_independence():
    """congresoia365 article, "Cómo Funciona Ulysses": heads are independent."""
    rng = np.random.default_rng(RNG_SEED + 8)
    N, H, d = 33, 4, 8
    q, k, v, do = (_rand(rng, N, H, d) for _ in range(4))
    O, LSE = oracle.attn_fwd(q, k, v)
    g = oracle.attn_bwd(q, k, v, do)
    for h in range(H):
        Oh, Lh = oracle.attn_fwd(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1])
        np.testing.assert_array_equal(Oh[:, 0], O[:, h])
        np.testing.assert_array_equal(Lh[0], LSE[h])
    q2 = q.copy()
    q2[:, 1] += 1.0
    O2, _ = oracle.attn_fwd(q2, k, v)
    g2 = oracle.attn_bwd(q2, k, v, do)
    for h in (0, 2, 3):
        np.testing.assert_array_equal(O2[:, h], O[:, h])
        for a, b in zip(g, g2):
            np.testing.assert_array_equal(a[:, h], b[:, h])
    assert np.abs(O2[:, 1] - O[:, 1]).max() > 1e-3


def test_stitched_virtual_ranks_equal_unsharded():
    """Guide, layout diagram: all-to-all, per-rank attention over H/sp heads, all-to-all back
    gives the same result as attention over all H heads of the unsharded sequence."""
    rng = np.random.default_rng(RNG_SEED + 9)
    for sp, B, N, H, d, lengths in ((2, 1, 32, 4, 8, None), (4, 2, 24, 8, 4, [5, 11, 8])):
        cu = None if lengths is None else _lengths_to_cu(lengths)
        full = [_rand(rng, B, N, H, d) for _ in range(4)]  # q, k, v, dO, seq-major
        Ns = N // sp
        shards = [np.stack([x[:, s * Ns:(s + 1) * Ns] for s in range(sp)]) for x in full]
        heads = [operm.seq_to_head(x) for x in shards]  # [sp, B, N, Hl, d]
        o_h, _ = oracle.attn_fwd(heads[0], heads[1], heads[2], cu)
        grads_h = oracle.attn_bwd(*heads, cu)
        o_seq = operm.head_to_seq(o_h)
        O, _ = oracle.attn_fwd(full[0], full[1], full[2], cu)
        grads = oracle.attn_bwd(*full, cu)
        np.testing.assert_allclose(np.concatenate(list(o_seq), axis=1), O, rtol=1e-13, atol=1e-14)
        for gh, g in zip(grads_h, grads):
            np.testing.assert_allclose(np.concatenate(list(operm.head_to_seq(gh)), axis=1), g, rtol=1e-13, atol=1e-14)


def test_causal_prefix():
    rng = np.random.default_rng(RNG_SEED + 10)
    N, H, d, M = 50, 2, 8, 21
    q, k, v, do = (_rand(rng, N, H, d) for _ in range(4))
    O, LSE = oracle.attn_fwd(q, k, v)
    Om, Lm = oracle.attn_fwd(q[:M], k[:M], v[:M])
    np.testing.assert_allclose(O[:M], Om, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(LSE[:, :M], Lm, rtol=1e-13, atol=1e-14)
    dq, _, _ = oracle.attn_bwd(q, k, v, do)
    dqm, _, _ = oracle.attn_bwd(q[:M], k[:M], v[:M], do[:M])
    np.testing.assert_allclose(dq[:M], dqm, rtol=1e-12, atol=1e-13)


# -------------------------------------------------------------- backward pins


def check_backward_finite_differences():
    rng = np.random.default_rng(RNG_SEED + 11)
    N, H, d = 7, 2, 4
    cu = _lengths_to_cu([3, 4])
    h = 1e-6
    for causal in (True, False):
        q, k, v, do = (_rand(rng, N, H, d) for _ in range(4))
        grads = oracle.attn_bwd(q, k, v, do, cu, causal)

        def loss(q_, k_, v_):
            return float((oracle.attn_fwd(q_, k_, v_, cu, causal)[0] * do).sum())

        for which, g in enumerate(grads):
            num = np.zeros_like(g)
            for idx in np.ndindex(*g.shape):
                args = [q.copy(), k.copy(), v.copy()]
                args[which][idx] += h
                up = loss(*args)
                args[which][idx] -= 2 * h
                dn = loss(*args)
                num[idx] = (up - dn) / (2 * h)
            err = np.abs(num - g).max() / max(np.abs(g).max(), 1e-30)
            assert err <= 1e-6, (causal, which, err)


def check_backward_q0_closed_form():
    rng = np.random.default_rng(RNG_SEED + 12)
    N, H, d = 150, 2, 8
    for causal in (True, False):
        for lengths in (None, [40, 1, 0, 109]):
            cu = None if lengths is None else _lengths_to_cu(lengths)
            q = np.zeros((N, H, d))
            k, v, do = (_rand(rng, N, H, d) for _ in range(3))
            dq, dk, dv = oracle.attn_bwd(q, k, v, do, cu, causal)
            for hh in range(H):
                cq, ck, cv = cf.q0_backward(k[:, hh], v[:, hh], do[:, hh], cu, causal, block=16)
                np.testing.assert_allclose(dq[:, hh], cq, rtol=1e-10, atol=1e-12)
                np.testing.assert_allclose(dk[:, hh], ck, rtol=0, atol=1e-13)
                np.testing.assert_allclose(dv[:, hh], cv, rtol=1e-12, atol=1e-13)


def check_uniform_rows_closed_form():
    """Queries orthogonal to the varying part of the keys: equal scores along
    each row, so O, lse, dQ, dK and dV have the closed forms of
    tests/closed_forms.py (dK non-zero, unlike q = 0)."""
    N, H, d = 160, 2, 8
    for causal in (True, False):
        for lengths in (None, [33, 1, 0, 90, 36]):
            cu = None if lengths is None else _lengths_to_cu(lengths)
            ins = [np.zeros((N, H, d)) for _ in range(4)]
            for hh in range(H):
                for dst, x in zip(ins, cf.uniform_inputs(N, d, 17 + hh)):
                    dst[:, hh] = x.numpy()
            q, k, v, do = ins
            O, LSE = oracle.attn_fwd(q, k, v, cu, causal)
            grads = oracle.attn_bwd(q, k, v, do, cu, causal)
            for hh in range(H):
                Oc, Lc = cf.uniform_forward(q[:, hh], k[:, hh], v[:, hh], cu, causal)
                np.testing.assert_allclose(O[:, hh], Oc, rtol=1e-12, atol=1e-12)
                np.testing.assert_allclose(LSE[hh], Lc, rtol=1e-12, atol=1e-12)
                gc = cf.uniform_backward(q[:, hh], k[:, hh], v[:, hh], do[:, hh], cu, causal, block=16)
                for g, c in zip(grads, gc):
                    assert np.abs(c).max() > 1e-2  # none of the three is trivially zero here
                    np.testing.assert_allclose(g[:, hh], c, rtol=1e-10, atol=1e-12)


def test_backward_finite_differences():
    check_backward_finite_differences()


def test_uniform_rows_closed_form():
    check_uniform_rows_closed_form()


def test_backward_q0_closed_form():
    check_backward_q0_closed_form()


def test_backward_constant_v():
    rng = np.random.default_rng(RNG_SEED + 13)
    N, H, d = 40, 2, 8
    q, k, do = (_rand(rng, N, H, d) for _ in range(3))
    v = np.broadcast_to(_rand(rng, H, d)[None], (N, H, d)).copy()
    dq, dk, dv = oracle.attn_bwd(q, k, v, do)
    assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13
    # dV = P^T dO with P from torch's softmax of the masked scores
    for h in range(H):
        S = torch.tensor(q[:, h] @ k[:, h].T / math.sqrt(d))
        S = S.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
        P = torch.softmax(S, dim=-1).numpy()
        np.testing.assert_allclose(dv[:, h], P.T @ do[:, h], rtol=1e-12, atol=1e-13)


def test_rowsum_identity():
    """D_i = rowsum(dO * O) equals rowsum(P * dP)."""
    rng = np.random.default_rng(RNG_SEED + 14)
    N, d = 30, 8
    q, k, v, do = (_rand(rng, N, 1, d) for _ in range(4))
    O, _ = oracle.attn_fwd(q, k, v)
    S = torch.tensor(q[:, 0] @ k[:, 0].T / math.sqrt(d))
    S = S.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    P = torch.softmax(S, dim=-1).numpy()
    dP = do[:, 0] @ v[:, 0].T
    np.testing.assert_allclose((do[:, 0] * O[:, 0]).sum(-1), (P * dP).sum(-1), rtol=1e-12, atol=1e-13)


def test_sampled_oracle_matches_full():
    rng = np.random.default_rng(RNG_SEED + 15)
    N, d = 120, 8
    cu = _lengths_to_cu([50, 0, 3, 67])
    q, k, v, do = (_rand(rng, N, 1, d) for _ in range(4))
    for causal in (True, False):
        O, LSE = oracle.attn_fwd(q, k, v, cu, causal)
        dq, dk, dv = oracle.attn_bwd(q, k, v, do, cu, causal)
        rows = [0, 1, 49, 50, 51, 52, 53, 100, 119]
        o_r, l_r = oracle.attn_fwd_rows(q[:, 0], k[:, 0], v[:, 0], rows, cu, causal)
        np.testing.assert_allclose(o_r, O[rows, 0], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(l_r, LSE[0, rows], rtol=1e-13, atol=1e-14)
        dq_r = oracle.attn_bwd_dq_rows(q[:, 0], k[:, 0], v[:, 0], do[:, 0], rows, cu, causal)
        np.testing.assert_allclose(dq_r, dq[rows, 0], rtol=1e-12, atol=1e-13)
        dk_c, dv_c = oracle.attn_bwd_dkdv_cols(q[:, 0], k[:, 0], v[:, 0], do[:, 0], rows, cu, causal)
        np.testing.assert_allclose(dk_c, dk[rows, 0], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(dv_c, dv[rows, 0], rtol=1e-12, atol=1e-13)


def test_oracle_rejects_bad_cu_seqlens():
    q = np.zeros((8, 1, 2))
    for bad in ([0, 9], [1, 8], [0, 5, 3, 8], [0]):
        with pytest.raises(ValueError):
            oracle.attn_fwd(q, q, q, np.array(bad))


# ------------------------------------------------------------ planted mistakes

PINS = [
    check_permute_golden_diagram,
    check_permute_index_formula,
    check_forward_bruteforce,
    check_forward_q0_closed_form,
    check_forward_single_token_docs,
    check_forward_vs_torch,
    check_backward_finite_differences,
    check_backward_q0_closed_form,
    check_uniform_rows_closed_form,
]


def _mutants():
    def scores_no_scale(Qr, qpos, Kd, kpos, causal, scale):
        return oatt.__dict__["_orig_scores"](Qr, qpos, Kd, kpos, causal, 1.0)

    def scores_anticausal(Qr, qpos, Kd, kpos, causal, scale):
        S = scale * (Qr @ Kd.T)
        return np.where(kpos[None, :] >= qpos[:, None], S, -np.inf) if causal else S

    def softmax_dropped_max(S):
        m = S.max(axis=1, keepdims=True)
        lse = np.log(np.exp(S - m).sum(axis=1))
        return np.exp(S - m - lse[:, None]), lse

    def seq_to_head_swapped(x_seq):
        sp, B, Ns, H, d = x_seq.shape
        Hl = H // sp
        full = np.concatenate([x_seq[s] for s in range(sp)], axis=1)
        return np.stack([full[:, :, r::sp, :][:, :, :Hl] for r in range(sp)])

    def bwd_dropped_rowsum(q, k, v, do, cu_seqlens=None, causal=True):
        lead = tuple(q.shape)[:-3]
        Q, K, V, DO = (oatt._flatten(x) for x in (q, k, v, do))
        G, N, H, d = Q.shape
        sc = 1 / math.sqrt(d)
        dQ, dK, dV = np.zeros_like(Q), np.zeros_like(Q), np.zeros_like(Q)
        pos = np.arange(N)
        for g in range(G):
            for h in range(H):
                for s, e in oatt.doc_bounds(N, cu_seqlens):
                    if e == s:
                        continue
                    P, _ = oatt._softmax_rows(oatt._scores(Q[g, s:e, h], pos[s:e], K[g, s:e, h], pos[s:e], causal, sc))
                    dP = DO[g, s:e, h] @ V[g, s:e, h].T
                    dS = P * dP
                    dQ[g, s:e, h] = sc * dS @ K[g, s:e, h]
                    dK[g, s:e, h] = sc * dS.T @ Q[g, s:e, h]
                    dV[g, s:e, h] = P.T @ DO[g, s:e, h]
        shape = lead + (N, H, d)
        return dQ.reshape(shape), dK.reshape(shape), dV.reshape(shape)

    def bwd_dk_transposed_operand(q, k, v, do, cu_seqlens=None, causal=True):
        dq, dk, dv = oatt.__dict__["_orig_bwd"](q, k, v, do, cu_seqlens, causal)
        return dq, dv, dk

    return {
        "scores without 1/sqrt(d)": (oatt, "_scores", scores_no_scale),
        "causal mask reversed": (oatt, "_scores", scores_anticausal),
        "lse without the row max": (oatt, "_softmax_rows", softmax_dropped_max),
        "heads dealt round-robin": (operm, "seq_to_head", seq_to_head_swapped),
        "dS without the rowsum term": (oatt, "attn_bwd", bwd_dropped_rowsum),
        "dK and dV swapped": (oatt, "attn_bwd", bwd_dk_transposed_operand),
    }


@pytest.mark.parametrize("name", list(_mutants().keys()))
def test_pins_catch_planted_mistakes(name, monkeypatch):
    module, attr, fn = _mutants()[name]
    monkeypatch.setitem(oatt.__dict__, "_orig_scores", oatt._scores)
    monkeypatch.setitem(oatt.__dict__, "_orig_bwd", oatt.attn_bwd)
    monkeypatch.setattr(module, attr, fn)
    if attr in ("attn_bwd", "seq_to_head"):
        monkeypatch.setattr(oracle, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, FloatingPointError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake: {name}"
