"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times: sampled outputs the oracle computes one by one, the q = 0
and uniform-row closed forms over every row and key, and bit-exact permutes
checked on sampled tokens plus a full round trip. Besides the per-tensor
bars, every compared row is held to a bar relative to its own size
(row_rel_err), so late rows of long sequences, whose values are hundreds of
times smaller than the first rows', are checked too."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
import ulysses_sequence_parallelism_seq_amd as uly
from tests import closed_forms as cf
from tests.gpu_util import (ROW_TOL_GRAD, ROW_TOL_O, TOL_BF16_GRAD, TOL_BF16_O, assert_rel, assert_rows, device,
                            dk_weights, dq_allowance, f64, rel_err, row_rel_err, say)

pytestmark = pytest.mark.gpu


def _docs(w):
    cu = workloads.workload_cu_seqlens(w)
    bounds = [(0, w.N)] if cu is None else list(zip(cu[:-1].tolist(), cu[1:].tolist()))
    return cu, bounds


def _sample_rows(bounds, rng, n_random):
    rows = set()
    for s, e in bounds:
        for r in (s, s + 1, s + 63, s + 64, s + 127, s + 128, s + 129, (s + e) // 2, e - 129, e - 128, e - 2, e - 1):
            if s <= r < e:
                rows.add(r)
    N = bounds[-1][1]
    rows.update(int(x) for x in rng.integers(0, N, n_random))
    return sorted(rows)


def _end_cols(bounds, per_doc):
    cols = []
    for s, e in bounds:
        cols.extend(range(max(s, e - per_doc), e))
    return cols


def _gpu_fwd_bwd(q, k, v, do, cu):
    dev = device()
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    packing = None if cu is None else uly.DocPacking(cu, q.shape[2], dev)
    o, lse = uly.ulysses_attn_fwd(qd, kd, vd, packing, True)
    dq, dk, dv = uly.ulysses_attn_bwd(qd, kd, vd, o, dod, lse, packing, True)
    torch.cuda.synchronize()
    out = tuple(t.cpu() for t in (o, lse, dq, dk, dv))
    del qd, kd, vd, dod, o, lse, dq, dk, dv
    torch.cuda.empty_cache()
    return out


def _sampled(q1, k1, v1, do1, rows, cols, cu):
    """Oracle values of sampled rows (O, lse, dQ) and key columns (dK, dV) of one
    head, with the per-row allowances for dQ and dK (tests/gpu_util.py)."""
    scale = 1.0 / np.sqrt(q1.shape[-1])
    O_r, L_r = oracle.attn_fwd_rows(q1, k1, v1, rows, cu)
    kbar, _ = oracle.attn_fwd_rows(q1, k1, k1, rows, cu)  # sum_j P_ij k_j
    dq_r = oracle.attn_bwd_dq_rows(q1, k1, v1, do1, rows, cu)
    dk_c, dv_c = oracle.attn_bwd_dkdv_cols(q1, k1, v1, do1, cols, cu)
    # the allowance of key j sums over the queries that see it: the rows from the
    # sampled columns to their document's end (causal)
    cols_a = np.asarray(cols)
    seen = []
    for s, e in _bounds_of(cu, q1.shape[0]):
        mine = cols_a[(cols_a >= s) & (cols_a < e)]
        if mine.size:
            seen.extend(range(int(mine.min()), e))
    O_seen, _ = oracle.attn_fwd_rows(q1, k1, v1, seen, cu)
    W = np.zeros(tuple(q1.shape), dtype=np.float64)
    W[seen] = dk_weights(O_seen, f64(do1)[seen], f64(q1)[seen])[:, None]
    _, ptw = oracle.attn_bwd_dkdv_cols(q1, k1, v1, W, cols, cu)  # sum_i P_ij w_i
    return {"O": O_r, "dQ": dq_r, "dK": dk_c, "dV": dv_c, "lse": L_r,
            "allow_dQ": dq_allowance(scale, kbar, O_r, f64(do1)[rows]), "allow_dK": scale * ptw[:, 0]}


def _bounds_of(cu, N):
    return [(0, N)] if cu is None else list(zip(np.asarray(cu)[:-1].tolist(), np.asarray(cu)[1:].tolist()))


def _check_sampled(tag, got, want, allow, lse_err):
    for n in got:
        tol = TOL_BF16_O if n == "O" else TOL_BF16_GRAD
        err = assert_rel(np.stack(got[n]), np.stack(want[n]), tol, f"{tag} {n}")
        rtol = ROW_TOL_O if n == "O" else ROW_TOL_GRAD
        a = np.concatenate(allow[n]) if n in allow else None
        rerr = float(row_rel_err(np.stack(got[n]), np.stack(want[n]), a, rtol).max())
        say(f"{tag} {n} rel err {err:.3e}, worst row {rerr:.3e}")
    for n in got:
        a = np.concatenate(allow[n]) if n in allow else None
        assert_rows(np.stack(got[n]), np.stack(want[n]), ROW_TOL_O if n == "O" else ROW_TOL_GRAD, f"{tag} {n}", a)
    say(f"{tag} lse max abs err {lse_err:.3e}")
    assert lse_err < 1e-3


@pytest.mark.parametrize("name", ["llama7b", "packed", "long", "million"])
def test_fullsize_sampled_oracle(name):
    w = workloads.WORKLOADS[name]
    say("full-size sampled", w)
    cu, bounds = _docs(w)
    q, k, v, do = workloads.qkv_do((1, w.B, w.N, w.Hl, w.d), w.seed, w.dtype, w.scale)
    o, lse, dq, dk, dv = _gpu_fwd_bwd(q, k, v, do, cu)
    rng = np.random.default_rng(w.seed)
    rows = _sample_rows(bounds, rng, 24)
    cols = _end_cols(bounds, 48 if w.N > 40000 else 256)
    got = {n: [] for n in ("O", "dQ", "dK", "dV")}
    want = {n: [] for n in got}
    allow = {"dQ": [], "dK": []}
    lse_err = 0.0
    for b in range(w.B):
        for h in range(w.Hl):
            sl = lambda t: t[0, b, :, h]  # noqa: E731
            ref = _sampled(sl(q), sl(k), sl(v), sl(do), rows, cols, cu)
            lse_err = max(lse_err, float(np.abs(f64(lse)[0, b, h, rows] - ref["lse"]).max()))
            for n, t, idx in (("O", o, rows), ("dQ", dq, rows), ("dK", dk, cols), ("dV", dv, cols)):
                got[n].append(f64(sl(t))[idx])
                want[n].append(ref[n])
            allow["dQ"].append(ref["allow_dQ"])
            allow["dK"].append(ref["allow_dK"])
    _check_sampled(name, got, want, allow, lse_err)


@pytest.mark.parametrize("name", ["llama7b", "packed"])
def test_fullsize_full_oracle_one_unit(name):
    """Every output of one (batch row, head) against the full oracle."""
    w = workloads.WORKLOADS[name]
    say("full-size full oracle, one unit", w)
    cu, _ = _docs(w)
    q, k, v, do = workloads.qkv_do((1, w.B, w.N, w.Hl, w.d), w.seed, w.dtype, w.scale)
    o, lse, dq, dk, dv = _gpu_fwd_bwd(q, k, v, do, cu)
    b, h = w.B - 1, w.Hl - 1
    one = lambda t: t[:, b:b + 1, :, h:h + 1]  # noqa: E731
    O, L = oracle.attn_fwd(one(q), one(k), one(v), cu)
    G = oracle.attn_bwd(one(q), one(k), one(v), one(do), cu)
    scale = 1.0 / np.sqrt(w.d)
    kbar, _ = oracle.attn_fwd(one(q), one(k), one(k), cu)  # sum_j P_ij k_j
    W = np.broadcast_to(dk_weights(O, one(do), one(q)).reshape(O.shape[:-1])[..., None], O.shape)
    ptw = oracle.attn_bwd(one(q), one(k), one(v), W, cu)[2][..., 0]  # sum_i P_ij w_i
    allow = {"dQ": dq_allowance(scale, kbar, O, one(do)), "dK": scale * ptw, "dV": None}
    assert_rel(one(o), O, TOL_BF16_O, "O")
    say(f"{name} O worst row {assert_rows(one(o), O, ROW_TOL_O, 'O'):.3e}")
    assert float(np.abs(f64(lse)[:, b:b + 1, h:h + 1] - L).max()) < 1e-3
    for n, got, want in zip(("dQ", "dK", "dV"), (one(dq), one(dk), one(dv)), G):
        err = assert_rel(got, want, TOL_BF16_GRAD, n)
        rerr = assert_rows(got, want, ROW_TOL_GRAD, n, allow[n])
        say(f"{name} {n} rel err {err:.3e}, worst row {rerr:.3e}")


@pytest.mark.parametrize("name", ["packed", "long", "million"])
def test_fullsize_q0_closed_form(name):
    """q = 0 at full size: every row of O, lse, dQ, dK, dV against the closed forms."""
    w = workloads.WORKLOADS[name]
    say("full-size q=0 closed form", w)
    cu, _ = _docs(w)
    _, k, v, do = workloads.qkv_do((1, w.B, w.N, w.Hl, w.d), w.seed + 100, w.dtype, w.scale)
    q = torch.zeros_like(k)
    o, lse, dq, dk, dv = _gpu_fwd_bwd(q, k, v, do, cu)
    assert torch.count_nonzero(dk) == 0
    worst = {"O": 0.0, "dQ": 0.0, "dV": 0.0, "lse": 0.0}
    rows = {"O": 0.0, "dQ": 0.0, "dV": 0.0}
    for b in range(w.B):
        for h in range(w.Hl):
            sl = lambda t: f64(t[0, b, :, h])  # noqa: E731
            O_c, L_c = cf.q0_forward(sl(v), cu)
            dq_c, _, dv_c = cf.q0_backward(sl(k), sl(v), sl(do), cu, block=512)
            kbar, _ = cf.q0_forward(sl(k), cu)  # uniform P: the mean of the keys a query sees
            allow = {"O": None, "dQ": dq_allowance(1.0 / np.sqrt(w.d), kbar, O_c, sl(do)), "dV": None}
            for n, got, want in (("O", sl(o), O_c), ("dQ", sl(dq), dq_c), ("dV", sl(dv), dv_c)):
                worst[n] = max(worst[n], rel_err(got, want))
                rows[n] = max(rows[n], float(row_rel_err(got, want, allow[n], ROW_TOL_O if n == "O"
                                                         else ROW_TOL_GRAD).max()))
            worst["lse"] = max(worst["lse"], float(np.abs(f64(lse)[0, b, h] - L_c).max()))
    say(name, "per tensor", worst, "worst row", rows)
    assert worst["O"] <= TOL_BF16_O and worst["dQ"] <= TOL_BF16_GRAD and worst["dV"] <= TOL_BF16_GRAD
    assert worst["lse"] < 1e-3
    assert rows["O"] <= ROW_TOL_O and rows["dQ"] <= ROW_TOL_GRAD and rows["dV"] <= ROW_TOL_GRAD, rows


def uniform_allowances(q1, k1, v1, do1, O, cu, causal=True):
    """dQ and dK row allowances (tests/gpu_util.py) when P is uniform over each
    row: kbar_i is the mean of the keys query i sees, and sum_i P_ij w_i is the
    dV closed form with dO replaced by w."""
    scale = 1.0 / np.sqrt(q1.shape[-1])
    kbar, _ = cf.q0_forward(k1, cu, causal)
    W = np.broadcast_to(dk_weights(O, do1, q1)[:, None], q1.shape)
    ptw = cf.q0_backward(k1, v1, W, cu, causal, block=512)[2][:, 0]
    return {"dQ": dq_allowance(scale, kbar, O, do1), "dK": scale * ptw}


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", ["packed", "long", "million"])
def test_fullsize_uniform_rows_closed_form(name):
    """Queries orthogonal to the varying part of the keys (q_i = [a_i, 0], k_j =
    [c, u_j]) give equal scores along each row, so every output has a closed
    form: every row of O, lse and dQ and every key of dK and dV at full size,
    with the dK/dV kernel's longest walks (every query tile of the document)
    accumulating non-zero dS-weighted queries."""
    w = workloads.WORKLOADS[name]
    say("full-size uniform-row closed form", w)
    cu, _ = _docs(w)
    shape = (1, w.B, w.N, w.Hl, w.d)
    ins = [torch.empty(shape, dtype=workloads.torch_dtype(w.dtype)) for _ in range(4)]
    for b in range(w.B):
        for h in range(w.Hl):
            one = cf.uniform_inputs(w.N, w.d, 1000 * w.seed + 10 * b + h, w.scale)
            for dst, x in zip(ins, one):
                dst[0, b, :, h] = x.to(dst.dtype)
    q, k, v, do = ins
    o, lse, dq, dk, dv = _gpu_fwd_bwd(q, k, v, do, cu)
    worst = {"O": 0.0, "dQ": 0.0, "dK": 0.0, "dV": 0.0, "lse": 0.0}
    rows = {"O": 0.0, "dQ": 0.0, "dK": 0.0, "dV": 0.0}
    for b in range(w.B):
        for h in range(w.Hl):
            sl = lambda t: f64(t[0, b, :, h])  # noqa: E731
            O_c, L_c = cf.uniform_forward(sl(q), sl(k), sl(v), cu)
            dq_c, dk_c, dv_c = cf.uniform_backward(sl(q), sl(k), sl(v), sl(do), cu, block=512)
            allow = uniform_allowances(sl(q), sl(k), sl(v), sl(do), O_c, cu)
            for n, got, want in (("O", sl(o), O_c), ("dQ", sl(dq), dq_c), ("dK", sl(dk), dk_c),
                                 ("dV", sl(dv), dv_c)):
                worst[n] = max(worst[n], rel_err(got, want))
                rows[n] = max(rows[n], float(row_rel_err(got, want, allow.get(n), ROW_TOL_O if n == "O"
                                                         else ROW_TOL_GRAD).max()))
            worst["lse"] = max(worst["lse"], float(np.abs(f64(lse)[0, b, h] - L_c).max()))
    say(name, "per tensor", worst, "worst row", rows)
    assert worst["O"] <= TOL_BF16_O and worst["lse"] < 1e-3
    assert max(worst["dQ"], worst["dK"], worst["dV"]) <= TOL_BF16_GRAD
    assert rows["O"] <= ROW_TOL_O, rows
    assert max(rows["dQ"], rows["dK"], rows["dV"]) <= ROW_TOL_GRAD, rows


@pytest.mark.parametrize("name", ["long", "million"])
def test_fullsize_permute(name):
    """The workload's sp shards of [N/sp, 32, 128] bf16: sampled tokens against the
    oracle, and seq -> head -> seq restores every bit."""
    w = workloads.WORKLOADS[name]
    say("full-size permute", w)
    dev = device()
    g = torch.Generator(device=dev).manual_seed(w.seed)
    x = torch.randint(-(1 << 15), 1 << 15, workloads.seq_shard_shape(w), generator=g, dtype=torch.int16,
                      device=dev).view(torch.bfloat16)
    head = uly.ulysses_seq_to_head(x)
    back = uly.ulysses_head_to_seq(head)
    torch.cuda.synchronize()
    assert torch.equal(back.view(torch.int16), x.view(torch.int16))
    del back
    idx = np.sort(np.random.default_rng(w.seed).choice(w.Ns, 96, replace=False))
    idx_t = torch.from_numpy(idx).to(dev)
    sub = x.view(torch.int16).index_select(2, idx_t).cpu().numpy()
    want = oracle.seq_to_head(sub)  # rows ordered (shard s, sample j) -> token s*Ns + idx[j]
    rows = torch.from_numpy((np.arange(w.sp)[:, None] * w.Ns + idx[None, :]).reshape(-1)).to(dev)
    got = head.view(torch.int16).index_select(2, rows).cpu().numpy()
    assert np.array_equal(got, want)


def test_bench_step_long_sampled():
    """The exact step bench.py times on the long workload (q, k, v through
    seq_to_head, one attention call over all 8 stacked virtual-rank shares,
    head_to_seq back, the backward likewise), checked on sampled outputs of
    three heads held by different virtual ranks against the oracle run on the
    unsharded full-H tensors."""
    import bench

    w = workloads.WORKLOADS["long"]
    say("bench step, sampled", w)
    dev = device()
    bufs = bench.make_buffers(w, dev)
    bench.step(w, bufs, None)
    torch.cuda.synchronize()
    q, k, v, do = bufs["seq_in"]
    outs = dict(zip(("O", "dQ", "dK", "dV"), bufs["seq_out"]))
    lse = bufs["head_out"][1]

    def full_head(x, h):  # [sp][B][Ns][H][d] -> the whole sequence of batch row 0, head h: [N][d]
        return x[:, 0, :, h].reshape(w.N, w.d).cpu()

    rng = np.random.default_rng(w.seed)
    rows = _sample_rows([(0, w.N)], rng, 12)
    cols = _end_cols([(0, w.N)], 32)
    got = {n: [] for n in outs}
    want = {n: [] for n in outs}
    allow = {"dQ": [], "dK": []}
    lse_err = 0.0
    for h in (0, 13, 31):  # virtual ranks 0, 3 and 7
        qh, kh, vh, doh = (full_head(x, h) for x in (q, k, v, do))
        ref = _sampled(qh, kh, vh, doh, rows, cols, None)
        lse_err = max(lse_err, float(np.abs(f64(lse[h // w.Hl, 0, h % w.Hl].cpu())[rows] - ref["lse"]).max()))
        for n, idx in (("O", rows), ("dQ", rows), ("dK", cols), ("dV", cols)):
            got[n].append(f64(full_head(outs[n], h))[idx])
            want[n].append(ref[n])
        allow["dQ"].append(ref["allow_dQ"])
        allow["dK"].append(ref["allow_dK"])
    del bufs
    torch.cuda.empty_cache()
    _check_sampled("bench step", got, want, allow, lse_err)
