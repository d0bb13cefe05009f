"""ulysses_attn_bwd_noalloc (the backward without a workspace, on the
library's fixed per-GPU scratch) called through the C ABI gives bit for bit
what ulysses_attn_bwd gives with a workspace: on consecutive calls whose
second is smaller than the first (the scratch keeps the first call's
contents), and on a call that needs the whole scratch."""

from __future__ import annotations

import ctypes

import pytest
import torch

import workloads
import ulysses_sequence_parallelism_seq_amd as uly
from tests.gpu_util import device, say

pytestmark = pytest.mark.gpu


def _noalloc_via_abi(q, k, v, o, dout, lse, packing, causal, dq, dk, dv):
    sp, B, N, Hl, d = q.shape
    cu_dev, ndoc, maxlen = (None, 1, N) if packing is None else (packing.device_tensor, packing.ndoc,
                                                               packing.max_doc_len)
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    stream = ctypes.c_void_p(torch.cuda.current_stream(q.device).cuda_stream)
    dtype = uly.ULY_BF16 if q.dtype == torch.bfloat16 else uly.ULY_F32
    return uly.library().ulysses_attn_bwd_noalloc(p(q), p(k), p(v), p(o), p(dout), p(lse), p(dq), p(dk), p(dv),
                                                  p(cu_dev), ndoc, maxlen, sp, B, N, Hl, d, int(causal), dtype,
                                                  stream)


def _inputs(shape, dtype, seed, dev, on_device):
    if not on_device:
        return [t.to(dev) for t in workloads.qkv_do(shape, seed, dtype)]
    g = torch.Generator(device=dev).manual_seed(seed)  # large cases: drawn on the device
    return [torch.randn(shape, generator=g, device=dev).to(workloads.torch_dtype(dtype)) for _ in range(4)]


def _case(shape, dtype, lengths, causal, seed, on_device=False):
    sp, B, N, Hl, d = shape
    say("noalloc", shape, dtype, lengths, causal)
    dev = device()
    packing = None if lengths is None else uly.DocPacking(workloads.cu_seqlens_from_lengths(lengths), N, dev)
    q, k, v, do = _inputs(shape, dtype, seed, dev, on_device)
    o, lse = uly.ulysses_attn_fwd(q, k, v, packing, causal)
    want = uly.ulysses_attn_bwd(q, k, v, o, do, lse, packing, causal)
    got = tuple(torch.full_like(q, float("nan")) for _ in range(3))
    rc = _noalloc_via_abi(q, k, v, o, do, lse, packing, causal, *got)
    assert rc == 0, uly.ulysses_status_string(rc)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, want):
        assert torch.equal(a, b), name
    return uly.ulysses_attn_bwd_workspace_bytes(sp, B, N, Hl, d, q.dtype)


def test_noalloc_matches_workspace_call_twice():
    big = _case((8, 1, 8192, 4, 128), "bf16", None, True, 3)
    small = _case((1, 1, 1000, 2, 64), "bf16", [300, 0, 1, 699], True, 4)
    assert small < big <= uly.ULY_NOALLOC_SCRATCH_BYTES
    _case((1, 1, 300, 2, 64), "fp32", [100, 200], False, 5)


def test_noalloc_whole_scratch_and_over_limit():
    # sp * B * Hl * N = 8388608 rows: exactly the scratch
    need = _case((1, 2048, 1024, 4, 64), "bf16", None, True, 6, on_device=True)
    assert need == uly.ULY_NOALLOC_SCRATCH_BYTES
    # one row more than fits is refused before anything is enqueued
    dev = device()
    t = torch.empty(16, dtype=torch.bfloat16, device=dev)
    p = ctypes.c_void_p(t.data_ptr())
    lib = uly.library()
    rc = lib.ulysses_attn_bwd_noalloc(p, p, p, p, p, p, p, p, p, None, 1, 1, 1, 1, 8388609, 1, 64, 1, uly.ULY_BF16,
                                      None)
    assert rc == 4  # ULY_EWORKSPACE
