"""One Ulysses layer (layout changes, forward, backward) captured in a HIP
graph and replayed: every replay gives the eager call's bits. The persistent
launches clear their tile-queue counters with kernels (the forward's clear
kernel, the backward's D pre-pass), never with a memset, so that the calls can
be captured; each replay here follows eager work on the same buffers and a
device synchronisation, and is checked on its own."""

from __future__ import annotations

import pytest
import torch

import workloads
import ulysses_sequence_parallelism_seq_amd as uly
from tests.gpu_util import device, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("sp,B,N,H,d,docs", [
    (2, 1, 1024, 8, 128, None),                      # two virtual ranks, one causal sequence
    (1, 1, 2048, 4, 64, [0, 300, 301, 1500, 2048]),  # packed documents, a one-token one among them
])
def test_captured_layer_replays_bit_exact(sp, B, N, H, d, docs):
    say("graph capture", sp, B, N, H, d, docs)
    dev = device()
    g = torch.Generator(device=dev).manual_seed(21)
    seq_shape = (sp, B, N // sp, H, d)
    qs, ks, vs, dos = (torch.randn(seq_shape, generator=g, device=dev).bfloat16() for _ in range(4))
    packing = None if docs is None else uly.DocPacking(docs, N, dev)
    head_shape = (sp, B, N, H // sp, d)
    qh, kh, vh, doh, o, dq, dk, dv = (torch.empty(head_shape, dtype=torch.bfloat16, device=dev) for _ in range(8))
    lse = torch.empty((sp, B, H // sp, N), dtype=torch.float32, device=dev)
    os_, dqs, dks, dvs = (torch.empty(seq_shape, dtype=torch.bfloat16, device=dev) for _ in range(4))
    fws = torch.empty(uly.ulysses_attn_fwd_workspace_bytes(), dtype=torch.uint8, device=dev)
    ws = torch.empty(uly.ulysses_attn_bwd_workspace_bytes(sp, B, N, H // sp, d, torch.bfloat16),
                     dtype=torch.uint8, device=dev)
    outs = (o, lse, dq, dk, dv, os_, dqs, dks, dvs)

    def layer():
        uly.ulysses_seq_to_head_n([qs, ks, vs], [qh, kh, vh])
        uly.ulysses_attn_fwd(qh, kh, vh, packing, True, out=o, lse=lse, workspace=fws)
        uly.ulysses_head_to_seq(o, out=os_)
        uly.ulysses_seq_to_head(dos, out=doh)
        uly.ulysses_attn_bwd_prepare(o, doh, lse, ws)
        uly.ulysses_attn_bwd_prepared(qh, kh, vh, doh, lse, ws, packing, True, dq=dq, dk=dk, dv=dv)
        uly.ulysses_head_to_seq_n([dq, dk, dv], [dqs, dks, dvs])

    layer()
    torch.cuda.synchronize()
    want = [t.clone() for t in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer()  # warm-up on the capture's stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer()
    torch.cuda.synchronize()

    for rep in range(3):
        for t in outs:
            t.fill_(7)  # eager work on the graph's buffers between the replays
        if rep == 1:
            layer()  # and, once, the eager layer itself
        for t in outs:
            t.fill_(-3)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("o", "lse", "dq", "dk", "dv", "o_seq", "dq_seq", "dk_seq", "dv_seq"), outs, want):
            assert torch.equal(got, ref), f"replay {rep}: {name}"
