"""GPU parity of the ring-attention steps against the float64 ring oracle:
the running state after every step (o_acc, lse; dq_acc, dk_acc, dv_acc),
the bf16 outputs written at each chunk's last step, several query and key
tiles with ragged tails, both head widths, causal and not; and the long
workload's shape as a ring of 8 chunks, on sampled outputs."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import ring
import ulysses_sequence_parallelism_seq_amd as uly
from tests import closed_forms as cf
from tests.gpu_util import TOL_BF16_GRAD, TOL_BF16_O, assert_rel, device, f64, rel_err, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("sp,B,Ns,H,d,causal", [
    (2, 1, 300, 2, 128, True),   # two query tiles (second ragged), five key tiles (last ragged)
    (4, 2, 130, 2, 64, True),    # idle ranks at late steps, d = 64
    (3, 1, 257, 1, 128, False),  # every block full
    (1, 1, 200, 2, 128, True),   # a ring of one: plain causal attention
])
def test_ring_steps_against_oracle(sp, B, Ns, H, d, causal):
    say("ring steps", sp, B, Ns, H, d, causal)
    dev = device()
    q, k, v, do = workloads.qkv_do((sp, B, Ns, H, d), 40 + sp, "bf16")
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o = o_acc = lse = None
    for step in range(sp):
        o, o_acc, lse = uly.ulysses_ring_attn_fwd_step(qd, kd, vd, step, causal, o, o_acc, lse)
        torch.cuda.synchronize()
        O_s, L_s = ring.ring_fwd(q, k, v, causal, steps=step + 1)
        err = assert_rel(o_acc.cpu(), O_s, TOL_BF16_O, f"o_acc after step {step}")
        lerr = float(np.abs(f64(lse.cpu()) - L_s).max())
        say(f"step {step}: o_acc rel err {err:.3e}, lse abs err {lerr:.3e}")
        assert lerr < 1e-3
    O, L = ring.ring_fwd(q, k, v, causal)
    assert_rel(o.cpu(), O, TOL_BF16_O, "o")
    # the bf16 output equals the fp32 running state rounded to bf16
    assert torch.equal(o.cpu(), o_acc.cpu().to(torch.bfloat16))

    ws = uly.ulysses_ring_attn_bwd_prepare(o, dod, lse)
    bufs = [None] * 6
    for step in range(sp):
        out = uly.ulysses_ring_attn_bwd_step(qd, kd, vd, dod, lse, ws, step, causal, bufs[3], bufs[4], bufs[5],
                                             bufs[0], bufs[1], bufs[2])
        bufs = list(out)
        torch.cuda.synchronize()
        want = ring.ring_bwd(q, k, v, do, O, L, causal, steps=step + 1)
        for name, got, w in zip(("dq_acc", "dk_acc", "dv_acc"), bufs[3:], want):
            err = assert_rel(got.cpu(), w, TOL_BF16_GRAD, f"{name} after step {step}")
            say(f"step {step}: {name} rel err {err:.3e}")
    G = ring.ring_bwd(q, k, v, do, O, L, causal)
    for name, got, acc, w in zip(("dq", "dk", "dv"), bufs[:3], bufs[3:], G):
        assert_rel(got.cpu(), w, TOL_BF16_GRAD, name)
        assert torch.equal(got.cpu(), acc.cpu().to(torch.bfloat16))
    # the ring's result is attention over the whole sequence
    O_full, _ = oracle.attn_fwd(ring.stitch(f64(q)), ring.stitch(f64(k)), ring.stitch(f64(v)), None, causal)
    assert_rel(ring.stitch(f64(o.cpu())), O_full, TOL_BF16_O, "o vs whole-sequence attention")


@pytest.mark.parametrize("sp,B,Ns,H,d,causal", [
    (2, 1, 300, 2, 128, True),
    (4, 2, 130, 2, 64, True),
    (3, 1, 257, 1, 128, False),
])
def test_ring_fwd_persistent_equals_one_tile_per_workgroup(sp, B, Ns, H, d, causal):
    """The forward steps' persistent launch (ulysses_ring_attn_fwd_step_ws) computes
    every tile whole in one workgroup: the same bits as one workgroup per tile,
    whatever the workspace held on entry, with one workspace serving every step."""
    say("ring fwd persistent", sp, B, Ns, H, d, causal)
    dev = device()
    q, k, v, _ = (t.to(dev) for t in workloads.qkv_do((sp, B, Ns, H, d), 50 + sp, "bf16"))
    o1, l1 = uly.ring_attn_fwd(q, k, v, causal)
    fws = torch.full((uly.ulysses_attn_fwd_workspace_bytes(),), 0xFF, dtype=torch.uint8, device=dev)
    o2, l2 = uly.ring_attn_fwd(q, k, v, causal, workspace=fws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_ring_long_workload_sampled():
    """The long workload's sequence (131072 tokens, 32 heads, d = 128, inputs
    scaled by 0.5) as a ring of 8 chunks, all steps: sampled query rows and
    late key columns of three heads against the whole-sequence oracle."""
    w = workloads.WORKLOADS["long"]
    say("ring, long workload", w)
    dev = device()
    shape = (w.sp, w.B, w.Ns, w.H, w.d)
    g = torch.Generator(device=dev).manual_seed(w.seed)
    q, k, v, do = ((torch.randn(shape, generator=g, device=dev) * w.scale).bfloat16() for _ in range(4))
    o, lse = uly.ring_attn_fwd(q, k, v, True)
    dq, dk, dv = uly.ring_attn_bwd(q, k, v, o, do, lse, True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.seed)
    rows = sorted({0, 1, 63, 64, w.Ns - 1, w.Ns, w.Ns + 1, 3 * w.Ns + 7, w.N - 2, w.N - 1}
                  | {int(x) for x in rng.integers(0, w.N, 10)})
    cols = list(range(w.N - 32, w.N))
    got = {n: [] for n in ("O", "dQ", "dK", "dV")}
    want = {n: [] for n in got}
    lse_err = 0.0

    def full(x, h):  # [sp, 1, Ns, H, d] -> [N, d] of head h
        return x[:, 0, :, h].reshape(w.N, w.d).cpu()

    for h in (0, 17, 31):
        qh, kh, vh, doh = (full(x, h) for x in (q, k, v, do))
        O_r, L_r = oracle.attn_fwd_rows(qh, kh, vh, rows)
        got["O"].append(f64(full(o, h))[rows])
        want["O"].append(O_r)
        lse_h = lse[:, 0, h].reshape(w.N).cpu()
        lse_err = max(lse_err, float(np.abs(f64(lse_h)[rows] - L_r).max()))
        got["dQ"].append(f64(full(dq, h))[rows])
        want["dQ"].append(oracle.attn_bwd_dq_rows(qh, kh, vh, doh, rows))
        dk_c, dv_c = oracle.attn_bwd_dkdv_cols(qh, kh, vh, doh, cols)
        got["dK"].append(f64(full(dk, h))[cols])
        want["dK"].append(dk_c)
        got["dV"].append(f64(full(dv, h))[cols])
        want["dV"].append(dv_c)
    del q, k, v, do, o, dq, dk, dv
    torch.cuda.empty_cache()
    for n in got:
        tol = TOL_BF16_O if n == "O" else TOL_BF16_GRAD
        err = assert_rel(np.stack(got[n]), np.stack(want[n]), tol, f"ring long {n}")
        say(f"ring long {n} rel err {err:.3e}")
    say(f"ring long lse max abs err {lse_err:.3e}")
    assert lse_err < 1e-3


def test_ring_long_workload_q0_closed_form():
    """q = 0 on the long workload's ring of 8 chunks: every row of O, lse, dQ,
    dV of four heads against the closed forms, and dK = 0 everywhere. Every
    key/value chunk's sums collect terms over several ring steps here."""
    w = workloads.WORKLOADS["long"]
    say("ring, long workload, q = 0", w)
    dev = device()
    shape = (w.sp, w.B, w.Ns, w.H, w.d)
    g = torch.Generator(device=dev).manual_seed(w.seed + 100)
    k, v, do = ((torch.randn(shape, generator=g, device=dev) * w.scale).bfloat16() for _ in range(3))
    q = torch.zeros_like(k)
    o, lse = uly.ring_attn_fwd(q, k, v, True)
    dq, dk, dv = uly.ring_attn_bwd(q, k, v, o, do, lse, True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dk) == 0

    def full(x, h):
        return f64(x[:, 0, :, h].reshape(w.N, w.d).cpu())

    worst = {"O": 0.0, "dQ": 0.0, "dV": 0.0, "lse": 0.0}
    for h in (0, 9, 22, 31):
        O_c, L_c = cf.q0_forward(full(v, h))
        dq_c, _, dv_c = cf.q0_backward(full(k, h), full(v, h), full(do, h), block=512)
        worst["O"] = max(worst["O"], rel_err(full(o, h), O_c))
        worst["dQ"] = max(worst["dQ"], rel_err(full(dq, h), dq_c))
        worst["dV"] = max(worst["dV"], rel_err(full(dv, h), dv_c))
        worst["lse"] = max(worst["lse"], float(np.abs(f64(lse[:, 0, h].reshape(w.N).cpu()) - L_c).max()))
    say("ring long q=0", worst)
    assert worst["O"] <= TOL_BF16_O and worst["dQ"] <= TOL_BF16_GRAD and worst["dV"] <= TOL_BF16_GRAD
    assert worst["lse"] < 1e-3
