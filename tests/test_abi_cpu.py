"""The C-ABI library loads, exports every declared call, and rejects bad
arguments on the host before enqueuing anything (CPU only: no call here
reaches a kernel launch)."""

from __future__ import annotations

import ctypes
import os
import re

import pytest

import ulysses_sequence_parallelism_seq_amd as uly

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ulysses.h")
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first
OK, EINVAL, ESHAPE, EUNSUP, EWS = 0, 1, 2, 3, 4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ulysses_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = uly.library()
    names = declared_functions()
    assert set(names) == {
        "ulysses_seq_to_head", "ulysses_head_to_seq", "ulysses_seq_to_head_n", "ulysses_head_to_seq_n",
        "ulysses_attn_fwd", "ulysses_attn_bwd",
        "ulysses_attn_fwd_ws", "ulysses_attn_fwd_workspace_bytes",
        "ulysses_attn_bwd_workspace_bytes", "ulysses_status_string", "ulysses_attn_bwd_noalloc",
        "ulysses_attn_bwd_prepare", "ulysses_attn_bwd_prepared",
        "ulysses_ring_attn_fwd_step", "ulysses_ring_attn_fwd_step_ws",
        "ulysses_ring_attn_bwd_workspace_bytes", "ulysses_ring_attn_bwd_prepare",
        "ulysses_ring_attn_bwd_step", "ulysses_sp_loss_workspace_bytes", "ulysses_sp_loss",
        "ulysses_tiled_mlp_workspace_bytes", "ulysses_tiled_mlp_fwd", "ulysses_tiled_mlp_bwd",
    }
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for code in range(6):
        assert uly.ulysses_status_string(code)
    assert uly.ulysses_status_string(99) == "unknown status"


def test_permute_argument_errors():
    lib = uly.library()
    f = lib.ulysses_seq_to_head
    assert f(None, FAKE, 1, 8, 4, 64, 2, 1, None) == EINVAL
    assert f(FAKE, FAKE, 0, 8, 4, 64, 2, 1, None) == EINVAL
    assert f(FAKE, ctypes.c_void_p(0x100000), 1, 9, 4, 64, 2, 1, None) == ESHAPE  # N % sp
    assert f(FAKE, ctypes.c_void_p(0x100000), 1, 8, 5, 64, 2, 1, None) == ESHAPE  # H % sp
    assert f(FAKE, ctypes.c_void_p(0x100000), 1, 8, 4, 96, 2, 1, None) == EUNSUP  # d
    assert f(FAKE, ctypes.c_void_p(0x100000), 1, 8, 4, 64, 2, 7, None) == EUNSUP  # dtype
    # overlapping buffers
    assert f(FAKE, ctypes.c_void_p(0x1000 + 64), 1, 8, 4, 64, 2, 1, None) == EINVAL
    g = lib.ulysses_head_to_seq
    assert g(FAKE, ctypes.c_void_p(0x100000), 1, 6, 4, 64, 4, 1, None) == ESHAPE
    # 16-byte accesses: misaligned buffers are rejected
    assert f(ctypes.c_void_p(0x1002), ctypes.c_void_p(0x100000), 1, 8, 4, 64, 2, 1, None) == EINVAL
    assert g(FAKE, ctypes.c_void_p(0x100008), 1, 8, 4, 64, 2, 1, None) == EINVAL


def test_batched_permute_argument_errors():
    """ulysses_seq_to_head_n / ulysses_head_to_seq_n reject what the header lists before any launch."""
    lib = uly.library()

    def arr(*ps):
        return (ctypes.c_void_p * len(ps))(*ps)

    a, b, c, d_ = 0x100000, 0x200000, 0x300000, 0x400000  # 4 KiB tensors (1, 8, 4, 64, bf16)
    for f in (lib.ulysses_seq_to_head_n, lib.ulysses_head_to_seq_n):
        assert f(arr(a, b), arr(c, d_), 0, 1, 8, 4, 64, 2, 1, None) == EINVAL  # n < 1
        assert f(arr(a, b, a, b, a), arr(c, d_, c, d_, c), 5, 1, 8, 4, 64, 2, 1, None) == EINVAL  # n > 4
        assert f(None, arr(c, d_), 2, 1, 8, 4, 64, 2, 1, None) == EINVAL
        assert f(arr(a, b), None, 2, 1, 8, 4, 64, 2, 1, None) == EINVAL
        assert f(arr(a, None), arr(c, d_), 2, 1, 8, 4, 64, 2, 1, None) == EINVAL
        assert f(arr(a, b), arr(c, c + 64), 2, 1, 8, 4, 64, 2, 1, None) == EINVAL  # outputs overlap
        assert f(arr(a, b), arr(c, a + 64), 2, 1, 8, 4, 64, 2, 1, None) == EINVAL  # output on an input
        assert f(arr(a, b), arr(c + 8, d_), 2, 1, 8, 4, 64, 2, 1, None) == EINVAL  # misaligned
        assert f(arr(a, b), arr(c, d_), 2, 1, 9, 4, 64, 2, 1, None) == ESHAPE  # N % sp
        assert f(arr(a, b), arr(c, d_), 2, 1, 8, 4, 96, 2, 1, None) == EUNSUP  # d
        # n * sp beyond the grid's z (tensors 1 TiB apart, one token per shard)
        t = 1 << 40
        assert f(arr(t, 2 * t), arr(3 * t, 4 * t), 2, 1, 32768, 32768, 64, 32768, 1, None) == ESHAPE


def test_attention_argument_errors():
    lib = uly.library()
    fwd = lib.ulysses_attn_fwd
    args = dict(cu=None, ndoc=1, maxlen=8, sp=1, B=1, N=8, Hl=2, d=64, causal=1, dtype=1)

    def call(**kw):
        a = {**args, **kw}
        return fwd(FAKE, FAKE, FAKE, FAKE, FAKE, a["cu"], a["ndoc"], a["maxlen"], a["sp"], a["B"], a["N"],
                   a["Hl"], a["d"], a["causal"], a["dtype"], None)

    assert fwd(None, FAKE, FAKE, FAKE, FAKE, None, 1, 8, 1, 1, 8, 2, 64, 1, 1, None) == EINVAL
    # the persistent forward: 1152 bytes of queue counters (nine on 128-byte lines), else
    # ULY_EWORKSPACE; then the same checks
    fws = lib.ulysses_attn_fwd_ws
    assert lib.ulysses_attn_fwd_workspace_bytes() == 1152
    assert fws(FAKE, FAKE, FAKE, FAKE, FAKE, None, 1152, None, 1, 8, 1, 1, 8, 2, 64, 1, 1, None) == EWS
    assert fws(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1151, None, 1, 8, 1, 1, 8, 2, 64, 1, 1, None) == EWS
    assert fws(None, FAKE, FAKE, FAKE, FAKE, FAKE, 1152, None, 1, 8, 1, 1, 8, 2, 64, 1, 1, None) == EINVAL
    assert fws(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1152, None, 1, 8, 1, 1, 8, 2, 48, 1, 1, None) == EUNSUP
    assert fws(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1152, FAKE, 1, 9, 1, 1, 8, 2, 64, 1, 1, None) == ESHAPE
    assert call(N=0) == EINVAL
    assert call(d=32) == EUNSUP
    assert call(dtype=3) == EUNSUP
    assert call(cu=FAKE, ndoc=0) == EINVAL
    assert call(cu=FAKE, maxlen=9) == ESHAPE

    bwd = lib.ulysses_attn_bwd
    need = lib.ulysses_attn_bwd_workspace_bytes(1, 1, 8, 2, 64, 1)
    # D and lse in log2 units, one float each per (unit, token), rounded up to 256 bytes,
    # then 2304 bytes of tile-queue counters (two queues)
    assert need == (2 * 1 * 1 * 2 * 8 * 4 + 255) // 256 * 256 + 2304
    assert lib.ulysses_attn_bwd_workspace_bytes(1, 1, 8, 2, 48, 1) == 0
    ptrs = [FAKE] * 9
    assert bwd(*ptrs, FAKE, need - 1, None, 1, 8, 1, 1, 8, 2, 64, 1, 1, None) == EWS
    assert bwd(*ptrs, None, need, None, 1, 8, 1, 1, 8, 2, 64, 1, 1, None) == EWS
    assert bwd(*ptrs[:8], None, FAKE, need, None, 1, 8, 1, 1, 8, 2, 64, 1, 1, None) == EINVAL
    assert bwd(*ptrs, FAKE, need, None, 1, 8, 1, 1, 8, 2, 64, 1, 9, None) == EUNSUP


def test_noalloc_argument_errors():
    """Refusals happen on the host, before the scratch's address is looked up."""
    lib = uly.library()
    f = lib.ulysses_attn_bwd_noalloc
    ptrs = [FAKE] * 9
    assert f(*ptrs[:8], None, None, 1, 8, 1, 1, 8, 2, 64, 1, 1, None) == EINVAL
    assert f(*ptrs, None, 1, 8, 1, 1, 8, 2, 48, 1, 1, None) == EUNSUP
    assert f(*ptrs, FAKE, 1, 9, 1, 1, 8, 2, 64, 1, 1, None) == ESHAPE  # max_doc_len > N
    # sp * B * Hl * N = 8388609 rows: one more than the scratch holds
    assert f(*ptrs, None, 1, 1, 1, 1, 8388609, 1, 64, 1, 1, None) == EWS
    assert f(*ptrs, None, 1, 1, 4, 2, 1048577, 1, 64, 1, 1, None) == EWS


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define ULY_NOALLOC_SCRATCH_BYTES \(\(\(size_t\)(\d+) << (\d+)\) \+ (\d+)\)", text)
    assert m, "ULY_NOALLOC_SCRATCH_BYTES not found in the header"
    assert (int(m.group(1)) << int(m.group(2))) + int(m.group(3)) == uly.ULY_NOALLOC_SCRATCH_BYTES
    # the limit in rows stated in the header: two floats per (token, head) row, plus the
    # 2304 bytes of tile-queue counters
    assert (uly.ULY_NOALLOC_SCRATCH_BYTES - 2304) // 8 == 8388608
    lib = uly.library()
    assert lib.ulysses_attn_bwd_workspace_bytes(1, 1, 8388608, 1, 64, 1) == uly.ULY_NOALLOC_SCRATCH_BYTES


def test_workspace_is_linear_in_n():
    """O(N) workspace: two floats per (unit, token) plus a fixed 2304 bytes of queue counters."""
    lib = uly.library()
    w1 = lib.ulysses_attn_bwd_workspace_bytes(1, 1, 131072, 4, 128, 1) - 2304
    w2 = lib.ulysses_attn_bwd_workspace_bytes(1, 1, 262144, 4, 128, 1) - 2304
    assert w2 == 2 * w1 == 2 * 2 * 131072 * 4 * 4


def test_binding_rejects_host_tensors():
    import torch

    with pytest.raises(ValueError):
        uly.ulysses_seq_to_head(torch.zeros(2, 1, 4, 4, 64, dtype=torch.bfloat16),
                                out=torch.zeros(2, 1, 8, 2, 64, dtype=torch.bfloat16))


def test_binding_validates_cu_seqlens():
    for bad in ([0, 5], [1, 8], [0, 6, 3, 8]):
        with pytest.raises(ValueError):
            uly.DocPacking(bad, 8, "cpu")
    p = uly.DocPacking([0, 3, 3, 8], 8, "cpu")
    assert (p.ndoc, p.max_doc_len) == (3, 5)


def test_ring_argument_errors():
    lib = uly.library()
    f = lib.ulysses_ring_attn_fwd_step
    ok = dict(step=0, sp=4, B=1, Ns=8, H=2, d=64, causal=1, dtype=1)

    def call(**kw):
        a = {**ok, **kw}
        return f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, a["step"], a["sp"], a["B"], a["Ns"], a["H"], a["d"],
                 a["causal"], a["dtype"], None)

    assert f(FAKE, FAKE, FAKE, FAKE, None, FAKE, 0, 4, 1, 8, 2, 64, 1, 1, None) == EINVAL  # o_acc
    fws = lib.ulysses_ring_attn_fwd_step_ws
    fneed = lib.ulysses_attn_fwd_workspace_bytes()
    assert fws(*([FAKE] * 6), None, fneed, 0, 4, 1, 8, 2, 64, 1, 1, None) == EWS
    assert fws(*([FAKE] * 6), FAKE, fneed - 1, 0, 4, 1, 8, 2, 64, 1, 1, None) == EWS
    assert fws(*([FAKE] * 6), FAKE, fneed, 4, 4, 1, 8, 2, 64, 1, 1, None) == EINVAL  # step
    assert fws(*([FAKE] * 5), None, FAKE, fneed, 0, 4, 1, 8, 2, 64, 1, 1, None) == EINVAL  # lse
    assert call(step=-1) == EINVAL
    assert call(step=4) == EINVAL  # steps are 0 .. sp-1
    assert call(Ns=0) == EINVAL
    assert call(dtype=0) == EUNSUP  # bf16 only
    assert call(d=96) == EUNSUP

    need = lib.ulysses_ring_attn_bwd_workspace_bytes(4, 1, 8, 2, 64, 1)
    assert need == 2 * 4 * 1 * 2 * 8 * 4 + 2304  # two floats per row (256-byte aligned), then the queue counters
    assert lib.ulysses_ring_attn_bwd_workspace_bytes(4, 1, 8, 2, 64, 0) == 0
    prep = lib.ulysses_ring_attn_bwd_prepare
    assert prep(FAKE, FAKE, FAKE, FAKE, need - 1, 4, 1, 8, 2, 64, 1, None) == EWS
    assert prep(FAKE, FAKE, None, FAKE, need, 4, 1, 8, 2, 64, 1, None) == EINVAL
    step = lib.ulysses_ring_attn_bwd_step
    ptrs = [FAKE] * 5
    assert step(*ptrs, FAKE, need, *([FAKE] * 6), 4, 4, 1, 8, 2, 64, 1, 1, None) == EINVAL  # step
    assert step(*ptrs, None, need, *([FAKE] * 6), 0, 4, 1, 8, 2, 64, 1, 1, None) == EWS
    assert step(*ptrs, FAKE, need, *([FAKE] * 5), None, 0, 4, 1, 8, 2, 64, 1, 1, None) == EINVAL


def test_sp_loss_argument_errors():
    lib = uly.library()
    need = lib.ulysses_sp_loss_workspace_bytes(8, 1, 16384)
    assert need == 8 * 4 * 16  # 4 partials of 4096 tokens per rank, fp64 sum + int64 count each
    assert lib.ulysses_sp_loss_workspace_bytes(0, 1, 8) == 0
    assert lib.ulysses_sp_loss_workspace_bytes(4097, 1, 8) == 0
    f = lib.ulysses_sp_loss
    assert f(None, FAKE, FAKE, FAKE, FAKE, FAKE, need, 8, 1, 16384, -100, None) == EINVAL
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, 8, 0, 16384, -100, None) == EINVAL
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, 5000, 1, 8, -100, None) == ESHAPE
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, 8, 1, 16384, -100, None) == EWS
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, None, need, 8, 1, 16384, -100, None) == EWS


def test_ring_binding_needs_running_state_after_step_0():
    import torch

    q = torch.zeros(2, 1, 8, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        uly.ulysses_ring_attn_fwd_step(q, q, q, 1, True)
    with pytest.raises(ValueError):
        uly.ulysses_ring_attn_bwd_step(q, q, q, q, torch.zeros(2, 1, 2, 8), torch.zeros(8, dtype=torch.uint8), 1)


def test_tiled_mlp_argument_errors():
    lib = uly.library()
    ws = lib.ulysses_tiled_mlp_workspace_bytes
    assert ws(16384, 4096, 11008, 4096) == 3 * 4096 * 11008 * 2  # three [tile][inter] bf16 arrays of one tile
    assert ws(100, 256, 512, 4096) == 3 * 100 * 512 * 2  # a tile larger than the tokens holds only them
    assert ws(100, 100, 512, 64) == 0 and ws(0, 256, 256, 64) == 0 and ws(8, 256, 256, 0) == 0
    need = ws(300, 256, 512, 128)
    fwd = lib.ulysses_tiled_mlp_fwd
    assert fwd(None, FAKE, FAKE, FAKE, FAKE, FAKE, need, 300, 256, 512, 128, None) == EINVAL
    assert fwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, 300, 250, 512, 128, None) == ESHAPE  # hidden % 256
    assert fwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, 300, 256, 500, 128, None) == ESHAPE  # inter % 256
    assert fwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, 300, 256, 512, 0, None) == EINVAL
    assert fwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, 300, 256, 512, 128, None) == EWS
    assert fwd(FAKE, FAKE, FAKE, FAKE, FAKE, None, need, 300, 256, 512, 128, None) == EWS
    assert fwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, 300, 1 << 22, 512, 128, None) == ESHAPE  # 2 GiB tiles
    bwd = lib.ulysses_tiled_mlp_bwd
    assert bwd(*([FAKE] * 8), None, FAKE, need, 300, 256, 512, 128, None) == EINVAL  # dw_down
    assert bwd(*([FAKE] * 9), FAKE, need - 1, 300, 256, 512, 128, None) == EWS
    assert bwd(*([FAKE] * 9), FAKE, need, -1, 256, 512, 128, None) == EINVAL
    # every pointer must be 16-byte aligned (the kernels' 16-byte loads and stores)
    odd = ctypes.c_void_p(FAKE.value + 8)
    assert fwd(FAKE, FAKE, FAKE, FAKE, odd, FAKE, need, 300, 256, 512, 128, None) == EINVAL  # y
    assert fwd(FAKE, FAKE, FAKE, FAKE, FAKE, odd, need, 300, 256, 512, 128, None) == EINVAL  # workspace
    assert bwd(*([FAKE] * 8), odd, FAKE, need, 300, 256, 512, 128, None) == EINVAL  # dw_down
    assert bwd(FAKE, FAKE, FAKE, FAKE, FAKE, odd, FAKE, FAKE, FAKE, FAKE, need, 300, 256, 512, 128, None) == EINVAL


FAR = ctypes.c_void_p(1 << 52)  # a second fake buffer far from FAKE: no overlap at these sizes


def test_every_size_limit_in_the_header_is_enforced():
    """Each ULY_ESHAPE (and size EINVAL) condition ulysses.h lists, triggered on
    the host before anything is enqueued (fake pointers are never touched)."""
    lib = uly.library()
    p2h, h2p = lib.ulysses_seq_to_head, lib.ulysses_head_to_seq
    assert p2h(FAKE, FAR, 1, 65536 * 2, 65536, 64, 65536, 1, None) == ESHAPE  # sp > 65535
    assert p2h(FAKE, FAR, 1, 1 << 20, 256, 128, 1, 1, None) == ESHAPE  # seq->head slab: 2^20 * 4096 chunks
    assert h2p(FAKE, FAR, 1, 1 << 20, 512, 128, 2, 1, None) == ESHAPE  # head->seq slab: 2^20 * 4096 chunks
    fwd = lib.ulysses_attn_fwd

    def f(cu=None, ndoc=1, maxlen=8, sp=1, B=1, N=8, Hl=2, d=64, dtype=1):
        return fwd(FAKE, FAKE, FAKE, FAKE, FAKE, cu, ndoc, maxlen, sp, B, N, Hl, d, 1, dtype, None)

    assert f(cu=FAKE, maxlen=9) == ESHAPE  # max_doc_len > N
    assert f(sp=1, B=1 << 24, Hl=2) == ESHAPE  # sp * B * Hl > 2^24
    assert f(N=1 << 22, maxlen=1 << 22, Hl=4, d=128) == ESHAPE  # one (row, head) spans 2 GiB
    assert f(cu=FAKE, ndoc=1 << 20, N=1 << 16, maxlen=1 << 16, B=1 << 11, Hl=2) == ESHAPE  # tile index
    bwd = lib.ulysses_attn_bwd
    need = lib.ulysses_attn_bwd_workspace_bytes(1, 1 << 11, 1 << 16, 2, 64, 1)
    assert need > 0
    # 128-token backward tiles: ceil(2^16 / 128) * 2^19 * 2^12 > 2^31 - 1 although the forward's
    # 256-token tiles give exactly 2^31: the backward refuses, the forward does not (its launch
    # would be huge, so only the refusal is checked here)
    assert bwd(*([FAKE] * 9), FAKE, need, FAKE, 1 << 19, 1 << 16, 1, 1 << 11, 1 << 16, 2, 64, 1, 1, None) == ESHAPE
    prep, prepd = lib.ulysses_attn_bwd_prepare, lib.ulysses_attn_bwd_prepared
    assert prepd(*([FAKE] * 8), FAKE, need, FAKE, 1 << 19, 1 << 16, 1, 1 << 11, 1 << 16, 2, 64, 1, 1, None) == ESHAPE
    assert prep(FAKE, FAKE, FAKE, FAKE, 7, 1, 1, 8, 2, 64, 1, None) == EWS
    assert prep(None, FAKE, FAKE, FAKE, 1 << 20, 1, 1, 8, 2, 64, 1, None) == EINVAL
    assert prepd(*([FAKE] * 8), None, 1 << 20, None, 1, 8, 1, 1, 8, 2, 64, 1, 1, None) == EWS
    ring = lib.ulysses_ring_attn_fwd_step
    assert ring(*([FAKE] * 6), 0, 16, 1 << 20, 1 << 20, 1, 64, 1, 1, None) == ESHAPE  # ceil(Ns/256) * units
    assert ring(*([FAKE] * 6), 0, 2, 1 << 23, 8, 2, 64, 1, 1, None) == ESHAPE  # sp * B * H = 2^25 > 2^24
    loss = lib.ulysses_sp_loss
    assert loss(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, 2, 1 << 20, 1 << 20, -100, None) == EINVAL  # B*Ns
