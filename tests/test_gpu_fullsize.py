"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times: sampled outputs the oracle computes one by one, the q = 0
closed forms over every row, and bit-exact permutes checked on sampled tokens
plus a full round trip."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
import ulysses_sequence_parallelism_seq_amd as uly
from tests import closed_forms as cf
from tests.gpu_util import TOL_BF16_GRAD, TOL_BF16_O, assert_rel, device, f64, rel_err, say

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
    lse_err = 0.0
    for b in range(w.B):
        for h in range(w.Hl):
            sl = lambda t: t[0, b, :, h]  # noqa: E731
            O_r, L_r = oracle.attn_fwd_rows(sl(q), sl(k), sl(v), rows, cu)
            got["O"].append(f64(sl(o))[rows])
            want["O"].append(O_r)
            lse_err = max(lse_err, float(np.abs(f64(lse)[0, b, h, rows] - L_r).max()))
            got["dQ"].append(f64(sl(dq))[rows])
            want["dQ"].append(oracle.attn_bwd_dq_rows(sl(q), sl(k), sl(v), sl(do), rows, cu))
            dk_c, dv_c = oracle.attn_bwd_dkdv_cols(sl(q), sl(k), sl(v), sl(do), cols, cu)
            got["dK"].append(f64(sl(dk))[cols])
            want["dK"].append(dk_c)
            got["dV"].append(f64(sl(dv))[cols])
            want["dV"].append(dv_c)
    for n in got:
        tol = TOL_BF16_O if n == "O" else TOL_BF16_GRAD
        err = assert_rel(np.stack(got[n]), np.stack(want[n]), tol, f"{name} {n}")
        say(f"{name} {n} rel err {err:.3e}")
    say(f"{name} lse max abs err {lse_err:.3e}")
    assert lse_err < 1e-3


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
    assert_rel(one(o), O, TOL_BF16_O, "O")
    assert float(np.abs(f64(lse)[:, b:b + 1, h:h + 1] - L).max()) < 1e-3
    for n, got, want in zip(("dQ", "dK", "dV"), (one(dq), one(dk), one(dv)), G):
        err = assert_rel(got, want, TOL_BF16_GRAD, n)
        say(f"{name} {n} rel err {err:.3e}")


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
    for b in range(w.B):
        for h in range(w.Hl):
            sl = lambda t: f64(t[0, b, :, h])  # noqa: E731
            O_c, L_c = cf.q0_forward(sl(v), cu)
            dq_c, _, dv_c = cf.q0_backward(sl(k), sl(v), sl(do), cu, block=512)
            worst["O"] = max(worst["O"], rel_err(sl(o), O_c))
            worst["dQ"] = max(worst["dQ"], rel_err(sl(dq), dq_c))
            worst["dV"] = max(worst["dV"], rel_err(sl(dv), dv_c))
            worst["lse"] = max(worst["lse"], float(np.abs(f64(lse)[0, b, h] - L_c).max()))
    say(name, worst)
    assert worst["O"] <= TOL_BF16_O and worst["dQ"] <= TOL_BF16_GRAD and worst["dV"] <= TOL_BF16_GRAD
    assert worst["lse"] < 1e-3


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
    lse_err = 0.0
    for h in (0, 13, 31):  # virtual ranks 0, 3 and 7
        qh, kh, vh, doh = (full_head(x, h) for x in (q, k, v, do))
        O_r, L_r = oracle.attn_fwd_rows(qh, kh, vh, rows)
        got["O"].append(f64(full_head(outs["O"], h))[rows])
        want["O"].append(O_r)
        lse_err = max(lse_err, float(np.abs(f64(lse[h // w.Hl, 0, h % w.Hl].cpu())[rows] - L_r).max()))
        got["dQ"].append(f64(full_head(outs["dQ"], h))[rows])
        want["dQ"].append(oracle.attn_bwd_dq_rows(qh, kh, vh, doh, rows))
        dk_c, dv_c = oracle.attn_bwd_dkdv_cols(qh, kh, vh, doh, cols)
        got["dK"].append(f64(full_head(outs["dK"], h))[cols])
        want["dK"].append(dk_c)
        got["dV"].append(f64(full_head(outs["dV"], h))[cols])
        want["dV"].append(dv_c)
    del bufs
    torch.cuda.empty_cache()
    for n in outs:
        tol = TOL_BF16_O if n == "O" else TOL_BF16_GRAD
        err = assert_rel(np.stack(got[n]), np.stack(want[n]), tol, f"bench step {n}")
        say(f"bench step {n} rel err {err:.3e}")
    say(f"bench step lse max abs err {lse_err:.3e}")
    assert lse_err < 1e-3
