"""GPU parity against the float64 oracle, element by element, at sizes the
oracle finishes in seconds: several tiles, ragged tails, packed documents
(including empty and one-token ones), both head widths, causal and not."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
import ulysses_sequence_parallelism_seq_amd as uly
from tests import closed_forms as cf
from tests.gpu_util import (ROW_TOL_GRAD, ROW_TOL_O, TOL_BF16_GRAD, TOL_BF16_O, TOL_F32_ABS, assert_abs, assert_rel,
                            assert_rows, device, dk_weights, dq_allowance, f64, say)

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ permute


@pytest.mark.parametrize("sp,B,Ns,H,d,dtype", [
    (2, 1, 128, 4, 64, "fp32"),     # tiny workload's shards
    (4, 2, 1024, 32, 128, "bf16"),  # llama7b workload's shards (full size)
    (3, 2, 7, 6, 64, "bf16"),
    (1, 1, 5, 2, 128, "fp32"),
    (8, 1, 33, 16, 128, "bf16"),
    (2, 1, 10, 6, 64, "bf16"),      # 3 heads per rank: 24-chunk runs (not a power of two)
    (3, 1, 9, 9, 64, "fp32"),       # 3 ranks, 3 heads each: neither sp nor the run a power of two
])
def test_permute_bit_exact(sp, B, Ns, H, d, dtype):
    say("permute", sp, B, Ns, H, d, dtype)
    dev = device()
    x = workloads.random_bits((sp, B, Ns, H, d), seed=11 + sp, dtype=dtype)
    ibits = torch.int16 if dtype == "bf16" else torch.int32
    head = uly.ulysses_seq_to_head(x.to(dev))
    torch.cuda.synchronize()
    want = oracle.seq_to_head(x.view(ibits).numpy())
    assert np.array_equal(head.cpu().view(ibits).numpy(), want)
    back = uly.ulysses_head_to_seq(head)
    torch.cuda.synchronize()
    assert np.array_equal(back.cpu().view(ibits).numpy(), x.view(ibits).numpy())
    y = workloads.random_bits((sp, B, Ns * sp, H // sp, d), seed=5, dtype=dtype)
    seq = uly.ulysses_head_to_seq(y.to(dev))
    torch.cuda.synchronize()
    assert np.array_equal(seq.cpu().view(ibits).numpy(), oracle.head_to_seq(y.view(ibits).numpy()))


@pytest.mark.parametrize("n,sp,B,Ns,H,d,dtype", [
    (3, 4, 2, 1024, 32, 128, "bf16"),  # q, k, v of the llama7b workload (full size)
    (4, 3, 1, 9, 9, 64, "fp32"),       # neither sp nor the run a power of two
    (2, 2, 1, 10, 6, 64, "bf16"),
    (1, 8, 1, 33, 16, 128, "bf16"),
])
def test_batched_permute_bit_exact(n, sp, B, Ns, H, d, dtype):
    """n tensors in one launch: each output equals the oracle's layout change of its input."""
    say("batched permute", n, sp, B, Ns, H, d, dtype)
    dev = device()
    ibits = torch.int16 if dtype == "bf16" else torch.int32
    xs = [workloads.random_bits((sp, B, Ns, H, d), seed=40 + i, dtype=dtype) for i in range(n)]
    heads = uly.ulysses_seq_to_head_n([x.to(dev) for x in xs])
    torch.cuda.synchronize()
    for x, h in zip(xs, heads):
        assert np.array_equal(h.cpu().view(ibits).numpy(), oracle.seq_to_head(x.view(ibits).numpy()))
    ys = [workloads.random_bits((sp, B, Ns * sp, H // sp, d), seed=50 + i, dtype=dtype) for i in range(n)]
    seqs = uly.ulysses_head_to_seq_n([y.to(dev) for y in ys])
    torch.cuda.synchronize()
    for y, q in zip(ys, seqs):
        assert np.array_equal(q.cpu().view(ibits).numpy(), oracle.head_to_seq(y.view(ibits).numpy()))


# ------------------------------------------------------------ fp32 exactness


def _run_gpu(q, k, v, do, cu, causal):
    dev = device()
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = uly.ulysses_attn_fwd(qd, kd, vd, cu, causal)
    dq, dk, dv = uly.ulysses_attn_bwd(qd, kd, vd, o, dod, lse, cu, causal)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu(), dq.cpu(), dk.cpu(), dv.cpu()


def test_tiny_fp32_exact():
    """The tiny workload: B=1, N=256, 2 local heads of width 64, fp32, causal."""
    w = workloads.WORKLOADS["tiny"]
    say("tiny fp32", w)
    q, k, v, do = workloads.qkv_do((1, w.B, w.N, w.Hl, w.d), w.seed, "fp32")
    o, lse, dq, dk, dv = _run_gpu(q, k, v, do, None, True)
    O, L = oracle.attn_fwd(q, k, v)
    G = oracle.attn_bwd(q, k, v, do)
    assert_abs(o, O, TOL_F32_ABS, "O")
    assert_abs(lse, L, TOL_F32_ABS, "lse")
    for name, got, want in zip(("dQ", "dK", "dV"), (dq, dk, dv), G):
        assert_abs(got, want, TOL_F32_ABS, name)


@pytest.mark.parametrize("N,Hl,d,causal,lengths", [
    (300, 2, 128, False, [1, 150, 0, 149]),
    (200, 1, 64, True, [70, 130]),
    (65, 3, 64, False, None),
])
def test_fp32_shapes(N, Hl, d, causal, lengths):
    say("fp32", N, Hl, d, causal, lengths)
    cu = None if lengths is None else workloads.cu_seqlens_from_lengths(lengths)
    q, k, v, do = workloads.qkv_do((2, 1, N, Hl, d), 21, "fp32")
    o, lse, dq, dk, dv = _run_gpu(q, k, v, do, cu, causal)
    O, L = oracle.attn_fwd(q, k, v, cu, causal)
    G = oracle.attn_bwd(q, k, v, do, cu, causal)
    assert_abs(o, O, TOL_F32_ABS, "O")
    assert_abs(lse, L, TOL_F32_ABS, "lse")
    for name, got, want in zip(("dQ", "dK", "dV"), (dq, dk, dv), G):
        assert_abs(got, want, TOL_F32_ABS, name)


def test_tiny_stitched_virtual_ranks():
    """Full-H sequence shards -> seq_to_head -> per-rank attention -> head_to_seq on
    the GPU equals the oracle's attention over all heads of the unsharded sequence."""
    w = workloads.WORKLOADS["tiny"]
    say("tiny stitched", w)
    dev = device()
    full = workloads.qkv_do((w.B, w.N, w.H, w.d), w.seed, "fp32")  # [B, N, H, d]
    shards = [x.view(w.B, w.sp, w.Ns, w.H, w.d).permute(1, 0, 2, 3, 4).contiguous() for x in full]
    heads = [uly.ulysses_seq_to_head(s.to(dev)) for s in shards]
    o, lse = uly.ulysses_attn_fwd(heads[0], heads[1], heads[2])
    dq, dk, dv = uly.ulysses_attn_bwd(heads[0], heads[1], heads[2], o, heads[3], lse)
    outs = [uly.ulysses_head_to_seq(t) for t in (o, dq, dk, dv)]
    torch.cuda.synchronize()
    O, _ = oracle.attn_fwd(*full[:3])
    G = oracle.attn_bwd(*full)
    for name, got, want in zip(("O", "dQ", "dK", "dV"), outs, (O,) + G):
        got_full = got.cpu().permute(1, 0, 2, 3, 4).reshape(w.B, w.N, w.H, w.d)
        assert_abs(got_full, want, TOL_F32_ABS, name)


# -------------------------------------------------------------- bf16 MFMA


BF16_CASES = [
    # (sp, B, N, Hl, d, causal, lengths)
    (1, 2, 1000, 2, 128, True, None),
    (1, 1, 1000, 2, 64, True, [300, 0, 1, 699]),
    (1, 1, 777, 3, 128, False, [129, 128, 520]),
    (2, 1, 640, 2, 128, True, [5, 200, 435]),
    (1, 1, 97, 1, 128, True, None),
    (1, 1, 1, 1, 128, True, None),
    (1, 1, 513, 2, 64, False, None),
    (1, 1, 384, 4, 128, True, [128, 128, 128]),
    (1, 1, 1200, 1, 128, True, [1] * 50 + [1150]),
]


@pytest.mark.parametrize("sp,B,N,Hl,d,causal,lengths", BF16_CASES)
def test_bf16_parity(sp, B, N, Hl, d, causal, lengths):
    say("bf16", sp, B, N, Hl, d, causal, lengths)
    cu = None if lengths is None else workloads.cu_seqlens_from_lengths(lengths)
    q, k, v, do = workloads.qkv_do((sp, B, N, Hl, d), 31 + N, "bf16")
    o, lse, dq, dk, dv = _run_gpu(q, k, v, do, cu, causal)
    O, L = oracle.attn_fwd(q, k, v, cu, causal)
    G = oracle.attn_bwd(q, k, v, do, cu, causal)
    assert_rel(o, O, TOL_BF16_O, "O")
    assert_abs(lse, L, 1e-3, "lse")
    for name, got, want in zip(("dQ", "dK", "dV"), (dq, dk, dv), G):
        assert_rel(got, want, TOL_BF16_GRAD, name)
    # every row (token of one head) against its own size as well, with the
    # allowances for dQ and dK that the stored O's rounding leaves (gpu_util)
    rows = {"O": assert_rows(o, O, ROW_TOL_O, "O")}
    for name, got, want, allow in zip(("dQ", "dK", "dV"), (dq, dk, dv), G, _grad_allowances(q, k, v, do, O, cu, causal)):
        rows[name] = assert_rows(got, want, ROW_TOL_GRAD, name, allow)
    say("worst rows", rows)


def _grad_allowances(q, k, v, do, O, cu, causal):
    """Per-row allowances of dQ (scale delta_i |kbar_i|) and dK (scale sum_i P_ij w_i)
    from the oracle: the forward with v := k gives kbar_i = sum_j P_ij k_j, the
    backward with dO := w gives sum_i P_ij w_i in its dV slot."""
    scale = 1.0 / np.sqrt(q.shape[-1])
    kbar, _ = oracle.attn_fwd(q, k, k, cu, causal)
    W = np.broadcast_to(dk_weights(O, do, q).reshape(O.shape[:-1])[..., None], O.shape)
    ptw = oracle.attn_bwd(q, k, v, W, cu, causal)[2][..., 0]
    return dq_allowance(scale, kbar, O, do), scale * ptw, None


@pytest.mark.parametrize("N,causal,lengths", [
    (1000, True, None),
    (777, False, [129, 128, 520]),
    (900, True, [300, 0, 1, 64, 535]),
])
def test_bf16_uniform_rows(N, causal, lengths):
    """Equal scores along each row (q_i = [a_i, 0], k_j = [c, u_j]): the GPU
    against the hand-derived closed forms (pinned to the oracle on the CPU),
    every row and key."""
    say("bf16 uniform rows", N, causal, lengths)
    cu = None if lengths is None else workloads.cu_seqlens_from_lengths(lengths)
    ins = [torch.empty((1, 1, N, 2, 128), dtype=torch.bfloat16) for _ in range(4)]
    for h in range(2):
        for dst, x in zip(ins, cf.uniform_inputs(N, 128, 50 + h)):
            dst[0, 0, :, h] = x.to(torch.bfloat16)
    q, k, v, do = ins
    o, lse, dq, dk, dv = _run_gpu(q, k, v, do, cu, causal)
    for h in range(2):
        sl = lambda t: f64(t[0, 0, :, h])  # noqa: E731
        O_c, L_c = cf.uniform_forward(sl(q), sl(k), sl(v), cu, causal)
        G_c = cf.uniform_backward(sl(q), sl(k), sl(v), sl(do), cu, causal, block=64)
        assert_rel(sl(o), O_c, TOL_BF16_O, "O")
        assert_rows(sl(o), O_c, ROW_TOL_O, "O")
        assert_abs(f64(lse)[0, 0, h], L_c, 1e-3, "lse")
        # uniform P: kbar_i is the mean of the keys query i sees; sum_i P_ij w_i the dV form with dO := w
        scale = 1.0 / np.sqrt(128)
        kbar, _ = cf.q0_forward(sl(k), cu, causal)
        W = np.broadcast_to(dk_weights(O_c, sl(do), sl(q))[:, None], O_c.shape)
        ptw = cf.q0_backward(sl(k), sl(v), W, cu, causal, block=64)[2][:, 0]
        allow = (dq_allowance(scale, kbar, O_c, sl(do)), scale * ptw, None)
        for name, got, want, a in zip(("dQ", "dK", "dV"), (dq, dk, dv), G_c, allow):
            assert_rel(sl(got), want, TOL_BF16_GRAD, name)
            assert_rows(sl(got), want, ROW_TOL_GRAD, name, a)


def test_bf16_packed_equals_separate():
    """Guide, sp_attn_implementation: packed documents give the same result as each run alone."""
    say("bf16 packed == separate")
    lengths = [200, 1, 311, 0, 88]
    cu = workloads.cu_seqlens_from_lengths(lengths)
    N = sum(lengths)
    q, k, v, do = workloads.qkv_do((1, 1, N, 2, 128), 77, "bf16")
    packed = _run_gpu(q, k, v, do, cu, True)
    for s, e in zip(cu[:-1], cu[1:]):
        if s == e:
            continue
        alone = _run_gpu(*(t[:, :, s:e].contiguous() for t in (q, k, v, do)), None, True)
        for name, a, b in zip(("O", "dQ", "dK", "dV"), (packed[0], *packed[2:]), (alone[0], *alone[2:])):
            assert torch.equal(a[:, :, s:e], b), name
        assert torch.equal(packed[1][..., s:e], alone[1]), "lse"


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp32", 64)])
def test_backward_in_two_calls_equals_one(dtype, d):
    """ulysses_attn_bwd_prepare then ulysses_attn_bwd_prepared (the split the
    benchmark times) give ulysses_attn_bwd's results bit for bit."""
    say("backward in two calls", dtype, d)
    dev = device()
    lengths = [300, 0, 1, 211]
    packing = uly.DocPacking(workloads.cu_seqlens_from_lengths(lengths), sum(lengths), dev)
    q, k, v, do = (t.to(dev) for t in workloads.qkv_do((2, 1, sum(lengths), 2, d), 41, dtype))
    o, lse = uly.ulysses_attn_fwd(q, k, v, packing, True)
    one = uly.ulysses_attn_bwd(q, k, v, o, do, lse, packing, True)
    ws = uly.ulysses_attn_bwd_prepare(o, do, lse)
    two = uly.ulysses_attn_bwd_prepared(q, k, v, do, lse, ws, packing, True)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), one, two):
        assert torch.equal(a, b), name


@pytest.mark.parametrize("shape,lengths,causal", [
    ((4, 2, 4096, 8, 128), None, True),                     # the llama7b workload's shares (full size)
    ((1, 1, 3000, 8, 128), [900, 0, 1, 1200, 899], True),   # empty and one-token documents
    ((3, 1, 1000, 3, 64), [1, 999], False),
])
def test_persistent_launch_equals_one_tile_per_workgroup(shape, lengths, causal):
    """The persistent launches (ulysses_attn_fwd_ws; the backward's dK/dV and dQ
    kernels) compute every tile whole in one workgroup: the same bits as the
    one-tile-per-workgroup forward, whatever the workspace held on entry, and
    one prepare serves several prepared calls (each kernel leaves its queue
    counters cleared)."""
    say("persistent == one tile per workgroup", shape, lengths, causal)
    dev = device()
    sp, B, N, Hl, d = shape
    packing = None if lengths is None else uly.DocPacking(workloads.cu_seqlens_from_lengths(lengths), N, dev)
    q, k, v, do = (t.to(dev) for t in workloads.qkv_do(shape, 43, "bf16"))
    o1, lse1 = uly.ulysses_attn_fwd(q, k, v, packing, causal, persistent=False)
    fws = torch.full((uly.ulysses_attn_fwd_workspace_bytes(),), 0xFF, dtype=torch.uint8, device=dev)
    o2, lse2 = uly.ulysses_attn_fwd(q, k, v, packing, causal, workspace=fws)
    o3, lse3 = uly.ulysses_attn_fwd(q, k, v, packing, causal, workspace=fws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(lse1, lse2), "forward, dirty workspace"
    assert torch.equal(o1, o3) and torch.equal(lse1, lse3), "forward, workspace reused"
    # the queue counters (nine ints, 128 bytes apart) are left cleared; the rest is untouched
    words = fws.view(torch.int32)
    ctr = torch.zeros_like(words, dtype=torch.bool)
    ctr[0::32] = True
    assert int(ctr.sum()) == 9
    assert torch.count_nonzero(words[ctr]).item() == 0, "the forward leaves its counters cleared"
    assert torch.all(words[~ctr] == -1).item(), "the forward writes only its counters"
    ws = torch.full((uly.ulysses_attn_bwd_workspace_bytes(*shape, torch.bfloat16),), 0xFF, dtype=torch.uint8,
                    device=dev)
    g1 = uly.ulysses_attn_bwd(q, k, v, o1, do, lse1, packing, causal, workspace=ws)
    uly.ulysses_attn_bwd_prepare(o1, do, lse1, ws)
    g2 = uly.ulysses_attn_bwd_prepared(q, k, v, do, lse1, ws, packing, causal)
    g3 = uly.ulysses_attn_bwd_prepared(q, k, v, do, lse1, ws, packing, causal)
    torch.cuda.synchronize()
    for name, a, b, c in zip(("dq", "dk", "dv"), g1, g2, g3):
        assert torch.equal(a, b) and torch.equal(a, c), name


def test_bf16_bitwise_reproducible():
    say("bf16 reproducible")
    q, k, v, do = workloads.qkv_do((1, 1, 1500, 2, 128), 5, "bf16")
    r1 = _run_gpu(q, k, v, do, None, True)
    r2 = _run_gpu(q, k, v, do, None, True)
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)


def test_bf16_constant_v_and_zero_q():
    """Closed forms: constant v gives O = v and dQ = dK = 0 (up to rounding);
    q = 0 gives O_i = mean of v over keys 0..i and lse_i = ln(i + 1)."""
    say("bf16 closed forms small")
    N, d = 700, 128
    dev = device()
    q, k, v, do = workloads.qkv_do((1, 1, N, 1, d), 8, "bf16")
    vc = v[:, :, :1].expand(1, 1, N, 1, d).contiguous()
    o, lse, dq, dk, dv = _run_gpu(q, k, vc, do, None, True)
    assert_rel(o, vc, 1e-2, "O const v")
    assert np.abs(f64(dq)).max() < 1e-2 * np.abs(f64(do)).max()
    z = torch.zeros_like(q)
    o, lse, dq, dk, dv = _run_gpu(z, k, v, do, None, True)
    want = np.cumsum(f64(v)[0, 0, :, 0], axis=0) / np.arange(1, N + 1)[:, None]
    assert_rel(o[0, 0, :, 0], want, TOL_BF16_O, "O q=0")
    np.testing.assert_allclose(f64(lse)[0, 0, 0], np.log(np.arange(1, N + 1)), atol=1e-4)
    assert torch.count_nonzero(dk) == 0


@pytest.mark.parametrize("causal", [True, False])
def test_bf16_rising_scores(causal):
    """Scores that climb by about 25 log2 units per 64-key tile along every
    row (keys scaled by a ramp): the forward's running max falls far behind
    and is moved many times by the overflow check of a tile's row sum, with
    weights up to 2^64 before each move. Same softmax as the oracle's."""
    say("bf16 rising scores", causal)
    N, d = 1024, 128
    base = workloads.qkv_do((1, 1, N, 2, d), 91, "fp32")
    ramp = (50.0 * torch.arange(N, dtype=torch.float32) / N).view(1, 1, N, 1, 1)
    q = (0.5 + 0.1 * base[0]).to(torch.bfloat16)
    k = (ramp * (1.0 + 0.1 * base[1])).to(torch.bfloat16)
    v = base[2].to(torch.bfloat16)
    do = base[3].to(torch.bfloat16)
    o, lse, dq, dk, dv = _run_gpu(q, k, v, do, None, causal)
    O, L = oracle.attn_fwd(q, k, v, None, causal)
    G = oracle.attn_bwd(q, k, v, do, None, causal)
    assert_rel(o, O, TOL_BF16_O, "O")
    assert_abs(lse, L, 1e-3, "lse")
    for name, got, want in zip(("dQ", "dK", "dV"), (dq, dk, dv), G):
        assert_rel(got, want, TOL_BF16_GRAD, name)
