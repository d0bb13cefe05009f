"""Ulysses sequence parallelism, per-rank hot path on MI355X (gfx950).

A thin Python binding over the C-ABI library ``libulysses.so`` (declared in
``include/ulysses.h``). It only marshals arguments: torch tensors become
device pointers, torch's current HIP stream becomes the launch stream, and
output tensors are allocated with torch. Every step of the computation runs
in the library's HIP kernels; there is no CPU or eager fallback, and a
missing library is an error.

Functions carry the C names:
  ulysses_seq_to_head(x_seq, sp)          [sp,B,N/sp,H,d] -> [sp,B,N,H/sp,d]
  ulysses_head_to_seq(x_head, sp)         [sp,B,N,H/sp,d] -> [sp,B,N/sp,H,d]
  ulysses_seq_to_head_n(xs), ulysses_head_to_seq_n(xs)  the same for up to four
                                          tensors of one shape in one launch
  ulysses_attn_fwd(q, k, v, ...)          -> (o, lse)  (bf16: the persistent launch of
                                          ulysses_attn_fwd_ws unless persistent=False)
  ulysses_attn_fwd_workspace_bytes()
  ulysses_attn_bwd(q, k, v, o, dout, lse, ...) -> (dq, dk, dv)
  ulysses_attn_bwd_workspace_bytes(...), ulysses_status_string(code)
  ulysses_attn_bwd_prepare(o, dout, lse, workspace)  the D pre-pass alone
  ulysses_attn_bwd_prepared(q, k, v, dout, lse, workspace, ...)  the rest of the backward
  ulysses_attn_bwd_noalloc(q, k, v, o, dout, lse, ..., dq=, dk=, dv=)
                                          the backward without a workspace (the
                                          library's fixed per-GPU scratch)
  ulysses_ring_attn_fwd_step(q, k, v, step, ...) one ring step (running o_acc, lse)
  ulysses_ring_attn_bwd_prepare(o, dout, lse)     D and lse*log2(e) into a workspace
  ulysses_ring_attn_bwd_step(q, k, v, dout, lse, workspace, step, ...)
  ulysses_ring_attn_bwd_workspace_bytes(...)
and two loops over the ring steps, ring_attn_fwd and ring_attn_bwd.
  ulysses_sp_loss(token_loss, labels)      -> (loss, rank_loss, good_tokens)
  ulysses_tiled_mlp_fwd(x, wg, wu, wd, tile) -> y           ALST's tiled SwiGLU MLP
  ulysses_tiled_mlp_bwd(x, wg, wu, wd, dy, tile) -> (dx, dwg, dwu, dwd)
  ulysses_tiled_mlp_workspace_bytes(tokens, hidden, inter, tile)
"""

from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libulysses.so")

ULY_F32, ULY_BF16 = 0, 1
_DTYPES = {torch.float32: ULY_F32, torch.bfloat16: ULY_BF16}

_lib = None


class UlyssesError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__(f"{fn} failed with status {code}: {ulysses_status_string(code)}")


def library() -> ctypes.CDLL:
    """The loaded C-ABI library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m ulysses_sequence_parallelism_seq_amd.build`"
            )
        lib = ctypes.CDLL(LIB_PATH)
        vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        lib.ulysses_seq_to_head.argtypes = [vp, vp, i, i, i, i, i, i, vp]
        lib.ulysses_head_to_seq.argtypes = [vp, vp, i, i, i, i, i, i, vp]
        lib.ulysses_seq_to_head_n.argtypes = [vp, vp] + [i] * 7 + [vp]
        lib.ulysses_head_to_seq_n.argtypes = [vp, vp] + [i] * 7 + [vp]
        lib.ulysses_attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, vp]
        lib.ulysses_attn_fwd_workspace_bytes.argtypes = []
        lib.ulysses_attn_fwd_workspace_bytes.restype = sz
        lib.ulysses_attn_fwd_ws.argtypes = [vp] * 6 + [sz, vp] + [i] * 9 + [vp]
        lib.ulysses_attn_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i]
        lib.ulysses_attn_bwd_workspace_bytes.restype = sz
        lib.ulysses_attn_bwd.argtypes = [vp] * 10 + [sz, vp] + [i] * 9 + [vp]
        lib.ulysses_attn_bwd_noalloc.argtypes = [vp] * 10 + [i] * 9 + [vp]
        lib.ulysses_attn_bwd_prepare.argtypes = [vp] * 4 + [sz] + [i] * 6 + [vp]
        lib.ulysses_attn_bwd_prepared.argtypes = [vp] * 9 + [sz, vp] + [i] * 9 + [vp]
        lib.ulysses_ring_attn_fwd_step.argtypes = [vp] * 6 + [i] * 8 + [vp]
        lib.ulysses_ring_attn_fwd_step_ws.argtypes = [vp] * 7 + [sz] + [i] * 8 + [vp]
        lib.ulysses_ring_attn_bwd_workspace_bytes.argtypes = [i] * 6
        lib.ulysses_ring_attn_bwd_workspace_bytes.restype = sz
        lib.ulysses_ring_attn_bwd_prepare.argtypes = [vp] * 4 + [sz] + [i] * 6 + [vp]
        lib.ulysses_ring_attn_bwd_step.argtypes = [vp] * 6 + [sz] + [vp] * 6 + [i] * 8 + [vp]
        lib.ulysses_sp_loss_workspace_bytes.argtypes = [i, i, i]
        lib.ulysses_sp_loss_workspace_bytes.restype = sz
        lib.ulysses_sp_loss.argtypes = [vp] * 6 + [sz] + [i] * 4 + [vp]
        lib.ulysses_tiled_mlp_workspace_bytes.argtypes = [i] * 4
        lib.ulysses_tiled_mlp_workspace_bytes.restype = sz
        lib.ulysses_tiled_mlp_fwd.argtypes = [vp] * 6 + [sz] + [i] * 4 + [vp]
        lib.ulysses_tiled_mlp_bwd.argtypes = [vp] * 10 + [sz] + [i] * 4 + [vp]
        lib.ulysses_status_string.argtypes = [i]
        lib.ulysses_status_string.restype = ctypes.c_char_p
        for name in ("ulysses_seq_to_head", "ulysses_head_to_seq", "ulysses_seq_to_head_n",
                     "ulysses_head_to_seq_n", "ulysses_attn_fwd", "ulysses_attn_fwd_ws",
                     "ulysses_attn_bwd",
                     "ulysses_attn_bwd_noalloc", "ulysses_attn_bwd_prepare", "ulysses_attn_bwd_prepared",
                     "ulysses_ring_attn_fwd_step", "ulysses_ring_attn_fwd_step_ws",
                     "ulysses_ring_attn_bwd_prepare", "ulysses_ring_attn_bwd_step",
                     "ulysses_sp_loss", "ulysses_tiled_mlp_fwd", "ulysses_tiled_mlp_bwd"):
            getattr(lib, name).restype = i
        _lib = lib
    return _lib


def ulysses_status_string(code: int) -> str:
    return library().ulysses_status_string(int(code)).decode()


def _check(fn: str, code: int):
    if code != 0:
        raise UlyssesError(fn, code)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")
    return _DTYPES[t.dtype]


def _require_device(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU (the HIP path has no CPU fallback)")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _expect(t: torch.Tensor, shape, dtype, name: str):
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {tuple(shape)} {dtype}, got {tuple(t.shape)} {t.dtype}")


def ulysses_seq_to_head(x_seq: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """[sp, B, N/sp, H, d] sequence shards -> [sp, B, N, H/sp, d] head shards (bit-exact)."""
    sp, B, Ns, H, d = x_seq.shape
    if H % sp:
        raise ValueError("H must be divisible by sp")
    if out is None:
        out = torch.empty((sp, B, Ns * sp, H // sp, d), dtype=x_seq.dtype, device=x_seq.device)
    _expect(out, (sp, B, Ns * sp, H // sp, d), x_seq.dtype, "out")
    _require_device(x_seq, out)
    _check("ulysses_seq_to_head", library().ulysses_seq_to_head(
        _ptr(x_seq), _ptr(out), B, Ns * sp, H, d, sp, _dtype_code(x_seq), _stream(x_seq)))
    return out


def ulysses_head_to_seq(x_head: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """[sp, B, N, H/sp, d] head shards -> [sp, B, N/sp, H, d] sequence shards (bit-exact)."""
    sp, B, N, Hl, d = x_head.shape
    if N % sp:
        raise ValueError("N must be divisible by sp")
    if out is None:
        out = torch.empty((sp, B, N // sp, Hl * sp, d), dtype=x_head.dtype, device=x_head.device)
    _expect(out, (sp, B, N // sp, Hl * sp, d), x_head.dtype, "out")
    _require_device(x_head, out)
    _check("ulysses_head_to_seq", library().ulysses_head_to_seq(
        _ptr(x_head), _ptr(out), B, N, Hl * sp, d, sp, _dtype_code(x_head), _stream(x_head)))
    return out


def _ptr_array(ts):
    return (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])


def ulysses_seq_to_head_n(xs_seq, outs=None):
    """ulysses_seq_to_head of up to four tensors of one shape in one launch (bit-exact)."""
    xs_seq = list(xs_seq)
    if not 1 <= len(xs_seq) <= 4:
        raise ValueError("one to four tensors")
    sp, B, Ns, H, d = xs_seq[0].shape
    if H % sp:
        raise ValueError("H must be divisible by sp")
    shape = (sp, B, Ns * sp, H // sp, d)
    if outs is None:
        outs = [torch.empty(shape, dtype=x.dtype, device=x.device) for x in xs_seq]
    outs = list(outs)
    if len(outs) != len(xs_seq):
        raise ValueError("as many outputs as inputs")
    for x, o in zip(xs_seq, outs):
        _expect(x, xs_seq[0].shape, xs_seq[0].dtype, "inputs")
        _expect(o, shape, xs_seq[0].dtype, "outs")
        _require_device(x, o)
    _check("ulysses_seq_to_head_n", library().ulysses_seq_to_head_n(
        _ptr_array(xs_seq), _ptr_array(outs), len(xs_seq), B, Ns * sp, H, d, sp, _dtype_code(xs_seq[0]),
        _stream(xs_seq[0])))
    return outs


def ulysses_head_to_seq_n(xs_head, outs=None):
    """ulysses_head_to_seq of up to four tensors of one shape in one launch (bit-exact)."""
    xs_head = list(xs_head)
    if not 1 <= len(xs_head) <= 4:
        raise ValueError("one to four tensors")
    sp, B, N, Hl, d = xs_head[0].shape
    if N % sp:
        raise ValueError("N must be divisible by sp")
    shape = (sp, B, N // sp, Hl * sp, d)
    if outs is None:
        outs = [torch.empty(shape, dtype=x.dtype, device=x.device) for x in xs_head]
    outs = list(outs)
    if len(outs) != len(xs_head):
        raise ValueError("as many outputs as inputs")
    for x, o in zip(xs_head, outs):
        _expect(x, xs_head[0].shape, xs_head[0].dtype, "inputs")
        _expect(o, shape, xs_head[0].dtype, "outs")
        _require_device(x, o)
    _check("ulysses_head_to_seq_n", library().ulysses_head_to_seq_n(
        _ptr_array(xs_head), _ptr_array(outs), len(xs_head), B, N, Hl * sp, d, sp, _dtype_code(xs_head[0]),
        _stream(xs_head[0])))
    return outs


class DocPacking:
    """Document boundaries (cu_seqlens) checked on the host and held on the device."""

    def __init__(self, cu_seqlens, N: int, device):
        cu = np.asarray(cu_seqlens.cpu() if isinstance(cu_seqlens, torch.Tensor) else cu_seqlens).reshape(-1)
        cu = cu.astype(np.int64)
        if len(cu) < 2 or cu[0] != 0 or cu[-1] != N or np.any(np.diff(cu) < 0):
            raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at N")
        self.ndoc = len(cu) - 1
        self.max_doc_len = int(np.diff(cu).max())
        self.host = cu.astype(np.int32)
        self.device_tensor = torch.from_numpy(self.host).to(device)


def _packing(cu_seqlens, N, device):
    if cu_seqlens is None:
        return None, 1, N
    p = cu_seqlens if isinstance(cu_seqlens, DocPacking) else DocPacking(cu_seqlens, N, device)
    return p.device_tensor, p.ndoc, p.max_doc_len


def _share_shape(q: torch.Tensor):
    if q.dim() == 4:  # one rank: [B, N, Hl, d]
        return (1,) + tuple(q.shape)
    if q.dim() == 5:  # stacked virtual ranks: [sp, B, N, Hl, d]
        return tuple(q.shape)
    raise ValueError("q must be [B, N, Hl, d] or [sp, B, N, Hl, d]")


def ulysses_attn_fwd(q, k, v, cu_seqlens=None, causal: bool = True, out=None, lse=None, workspace=None,
                     persistent: bool = True):
    """Attention forward over head-sharded shares; returns (o, lse).

    q, k, v: [sp, B, N, Hl, d] or [B, N, Hl, d]; lse is [..., Hl, N] float32.
    cu_seqlens: None, host int sequence / tensor, or a DocPacking.
    persistent (bf16): the persistent launch of ulysses_attn_fwd_ws, with
    `workspace` (>= ulysses_attn_fwd_workspace_bytes() bytes on the device;
    allocated here when None); False: ulysses_attn_fwd, one tile per
    workgroup. Both give the same bits.
    """
    sp, B, N, Hl, d = _share_shape(q)
    for t in (k, v):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("q, k, v must share shape and dtype")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(tuple(q.shape[:-3]) + (Hl, N), dtype=torch.float32, device=q.device)
    _expect(out, q.shape, q.dtype, "out")
    _expect(lse, tuple(q.shape[:-3]) + (Hl, N), torch.float32, "lse")
    _require_device(q, k, v, out, lse)
    cu_dev, ndoc, maxlen = _packing(cu_seqlens, N, q.device)
    lib = library()
    if persistent:
        need = int(lib.ulysses_attn_fwd_workspace_bytes())
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        _require_device(workspace)
        _check("ulysses_attn_fwd_ws", lib.ulysses_attn_fwd_ws(
            _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _ptr(cu_dev), ndoc, maxlen,
            sp, B, N, Hl, d, int(bool(causal)), _dtype_code(q), _stream(q)))
    else:
        _check("ulysses_attn_fwd", lib.ulysses_attn_fwd(
            _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_dev), ndoc, maxlen,
            sp, B, N, Hl, d, int(bool(causal)), _dtype_code(q), _stream(q)))
    return out, lse


def ulysses_attn_fwd_workspace_bytes() -> int:
    return int(library().ulysses_attn_fwd_workspace_bytes())


def ulysses_attn_bwd_workspace_bytes(sp: int, B: int, N: int, Hl: int, d: int, dtype: torch.dtype) -> int:
    return int(library().ulysses_attn_bwd_workspace_bytes(sp, B, N, Hl, d, _DTYPES[dtype]))


def ulysses_attn_bwd(q, k, v, o, dout, lse, cu_seqlens=None, causal: bool = True, workspace=None,
                     dq=None, dk=None, dv=None):
    """Attention backward; returns (dq, dk, dv) with q's shape and dtype."""
    sp, B, N, Hl, d = _share_shape(q)
    for t in (k, v, o, dout):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("q, k, v, o, dout must share shape and dtype")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    need = ulysses_attn_bwd_workspace_bytes(sp, B, N, Hl, d, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _expect(lse, tuple(q.shape[:-3]) + (Hl, N), torch.float32, "lse")
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _expect(t, q.shape, q.dtype, name)
    _require_device(q, k, v, o, dout, lse, dq, dk, dv, workspace)
    cu_dev, ndoc, maxlen = _packing(cu_seqlens, N, q.device)
    _check("ulysses_attn_bwd", library().ulysses_attn_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(cu_dev), ndoc, maxlen,
        sp, B, N, Hl, d, int(bool(causal)), _dtype_code(q), _stream(q)))
    return dq, dk, dv


def ulysses_attn_bwd_prepare(o, dout, lse, workspace=None):
    """The backward's D pre-pass alone (into the returned workspace)."""
    sp, B, N, Hl, d = _share_shape(o)
    if dout.shape != o.shape or dout.dtype != o.dtype:
        raise ValueError("o and dout must share shape and dtype")
    need = ulysses_attn_bwd_workspace_bytes(sp, B, N, Hl, d, o.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=o.device)
    _expect(lse, tuple(o.shape[:-3]) + (Hl, N), torch.float32, "lse")
    _require_device(o, dout, lse, workspace)
    _check("ulysses_attn_bwd_prepare", library().ulysses_attn_bwd_prepare(
        _ptr(o), _ptr(dout), _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(),
        sp, B, N, Hl, d, _dtype_code(o), _stream(o)))
    return workspace


def ulysses_attn_bwd_prepared(q, k, v, dout, lse, workspace, cu_seqlens=None, causal: bool = True, dq=None,
                              dk=None, dv=None):
    """The backward's dK/dV and dQ kernels from a workspace ulysses_attn_bwd_prepare filled."""
    sp, B, N, Hl, d = _share_shape(q)
    for t in (k, v, dout):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("q, k, v, dout must share shape and dtype")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    _expect(lse, tuple(q.shape[:-3]) + (Hl, N), torch.float32, "lse")
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _expect(t, q.shape, q.dtype, name)
    _require_device(q, k, v, dout, lse, workspace, dq, dk, dv)
    cu_dev, ndoc, maxlen = _packing(cu_seqlens, N, q.device)
    _check("ulysses_attn_bwd_prepared", library().ulysses_attn_bwd_prepared(
        _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(cu_dev), ndoc, maxlen, sp, B, N, Hl, d,
        int(bool(causal)), _dtype_code(q), _stream(q)))
    return dq, dk, dv


# The fixed per-GPU scratch of ulysses_attn_bwd_noalloc (ULY_NOALLOC_SCRATCH_BYTES in ulysses.h).
ULY_NOALLOC_SCRATCH_BYTES = (64 << 20) + 2304


def ulysses_attn_bwd_noalloc(q, k, v, o, dout, lse, cu_seqlens=None, causal: bool = True, dq=None, dk=None,
                             dv=None):
    """Attention backward without a workspace; returns (dq, dk, dv).

    The library's own scratch replaces the workspace, so a caller that passes
    dq, dk, dv and a DocPacking (or None) makes the call allocate nothing.
    Calls that overlap on one GPU share that scratch and race.
    """
    sp, B, N, Hl, d = _share_shape(q)
    for t in (k, v, o, dout):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("q, k, v, o, dout must share shape and dtype")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    _expect(lse, tuple(q.shape[:-3]) + (Hl, N), torch.float32, "lse")
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _expect(t, q.shape, q.dtype, name)
    _require_device(q, k, v, o, dout, lse, dq, dk, dv)
    cu_dev, ndoc, maxlen = _packing(cu_seqlens, N, q.device)
    with torch.cuda.device(q.device):  # the scratch used is the current device's
        _check("ulysses_attn_bwd_noalloc", library().ulysses_attn_bwd_noalloc(
            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
            _ptr(cu_dev), ndoc, maxlen, sp, B, N, Hl, d, int(bool(causal)), _dtype_code(q), _stream(q)))
    return dq, dk, dv


# ---------------------------------------------------------------- ring attention
# q, k, v, dout, o: [sp, B, Ns, H, d] bf16 chunks (rank r holds tokens r*Ns ..);
# lse: [sp, B, H, Ns] float32.


def _ring_shape(q):
    if q.dim() != 5:
        raise ValueError("ring attention takes [sp, B, Ns, H, d] chunks")
    if q.dtype != torch.bfloat16:
        raise TypeError("ring attention runs in bfloat16")
    return tuple(q.shape)


def ulysses_ring_attn_fwd_step(q, k, v, step: int, causal: bool = True, o=None, o_acc=None, lse=None,
                               workspace=None):
    """One forward ring step; returns (o, o_acc, lse). Pass the previous step's o_acc and lse back in.
    With a workspace (ulysses_attn_fwd_workspace_bytes() bytes) the step runs as the
    persistent launch of ulysses_ring_attn_fwd_step_ws (same bits)."""
    sp, B, Ns, H, d = _ring_shape(q)
    for t in (k, v):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("q, k, v must share shape and dtype")
    if step > 0 and (o is None or o_acc is None or lse is None):
        raise ValueError("steps after the first continue from the previous step's o, o_acc and lse")
    o = torch.empty_like(q) if o is None else o
    o_acc = torch.empty(q.shape, dtype=torch.float32, device=q.device) if o_acc is None else o_acc
    lse = torch.empty((sp, B, H, Ns), dtype=torch.float32, device=q.device) if lse is None else lse
    _expect(o, q.shape, q.dtype, "o")
    _expect(o_acc, q.shape, torch.float32, "o_acc")
    _expect(lse, (sp, B, H, Ns), torch.float32, "lse")
    _require_device(q, k, v, o, o_acc, lse)
    if workspace is None:
        _check("ulysses_ring_attn_fwd_step", library().ulysses_ring_attn_fwd_step(
            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(o_acc), _ptr(lse), int(step), sp, B, Ns, H, d,
            int(bool(causal)), ULY_BF16, _stream(q)))
    else:
        _require_device(q, workspace)
        _check("ulysses_ring_attn_fwd_step_ws", library().ulysses_ring_attn_fwd_step_ws(
            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(o_acc), _ptr(lse), _ptr(workspace),
            workspace.numel() * workspace.element_size(), int(step), sp, B, Ns, H, d,
            int(bool(causal)), ULY_BF16, _stream(q)))
    return o, o_acc, lse


def ring_attn_fwd(q, k, v, causal: bool = True, o=None, o_acc=None, lse=None, workspace=None):
    """All sp forward ring steps in order; returns (o, lse)."""
    for step in range(q.shape[0]):
        o, o_acc, lse = ulysses_ring_attn_fwd_step(q, k, v, step, causal, o, o_acc, lse, workspace)
    return o, lse


def ulysses_ring_attn_bwd_workspace_bytes(sp: int, B: int, Ns: int, H: int, d: int) -> int:
    return int(library().ulysses_ring_attn_bwd_workspace_bytes(sp, B, Ns, H, d, ULY_BF16))


def ulysses_ring_attn_bwd_prepare(o, dout, lse, workspace=None):
    """-D = -rowsum(dO * O) and lse * log2(e) into the (returned) workspace."""
    sp, B, Ns, H, d = _ring_shape(o)
    if dout.shape != o.shape or dout.dtype != o.dtype:
        raise ValueError("o and dout must share shape and dtype")
    need = ulysses_ring_attn_bwd_workspace_bytes(sp, B, Ns, H, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=o.device)
    _expect(lse, (sp, B, H, Ns), torch.float32, "lse")
    _require_device(o, dout, lse, workspace)
    _check("ulysses_ring_attn_bwd_prepare", library().ulysses_ring_attn_bwd_prepare(
        _ptr(o), _ptr(dout), _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(),
        sp, B, Ns, H, d, ULY_BF16, _stream(o)))
    return workspace


def ulysses_ring_attn_bwd_step(q, k, v, dout, lse, workspace, step: int, causal: bool = True,
                               dq_acc=None, dk_acc=None, dv_acc=None, dq=None, dk=None, dv=None):
    """One backward ring step; returns (dq, dk, dv, dq_acc, dk_acc, dv_acc)."""
    sp, B, Ns, H, d = _ring_shape(q)
    for t in (k, v, dout):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("q, k, v, dout must share shape and dtype")
    if step > 0 and any(t is None for t in (dq_acc, dk_acc, dv_acc, dq, dk, dv)):
        raise ValueError("steps after the first continue from the previous step's sums and outputs")
    f32 = lambda: torch.empty(q.shape, dtype=torch.float32, device=q.device)  # noqa: E731
    dq_acc = f32() if dq_acc is None else dq_acc
    dk_acc = f32() if dk_acc is None else dk_acc
    dv_acc = f32() if dv_acc is None else dv_acc
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for name, t in (("dq_acc", dq_acc), ("dk_acc", dk_acc), ("dv_acc", dv_acc)):
        _expect(t, q.shape, torch.float32, name)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _expect(t, q.shape, q.dtype, name)
    _expect(lse, (sp, B, H, Ns), torch.float32, "lse")
    _require_device(q, k, v, dout, lse, workspace, dq_acc, dk_acc, dv_acc, dq, dk, dv)
    _check("ulysses_ring_attn_bwd_step", library().ulysses_ring_attn_bwd_step(
        _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(dq_acc), _ptr(dk_acc), _ptr(dv_acc),
        _ptr(dq), _ptr(dk), _ptr(dv), int(step), sp, B, Ns, H, d, int(bool(causal)), ULY_BF16, _stream(q)))
    return dq, dk, dv, dq_acc, dk_acc, dv_acc


def ring_attn_bwd(q, k, v, o, dout, lse, causal: bool = True, workspace=None):
    """Prepare plus all sp backward ring steps in order; returns (dq, dk, dv)."""
    workspace = ulysses_ring_attn_bwd_prepare(o, dout, lse, workspace)
    bufs = (None,) * 6
    for step in range(q.shape[0]):
        dq, dk, dv, dqa, dka, dva = ulysses_ring_attn_bwd_step(q, k, v, dout, lse, workspace, step, causal,
                                                               bufs[3], bufs[4], bufs[5], *bufs[:3])
        bufs = (dq, dk, dv, dqa, dka, dva)
    return bufs[0], bufs[1], bufs[2]


# ------------------------------------------------------- SP loss aggregation


def ulysses_sp_loss(token_loss, labels, ignore_index: int = -100, workspace=None, loss=None, rank_loss=None,
                    good_tokens=None):
    """Count-weighted loss of sp ranks; returns (loss [1] f32, rank_loss [sp] f32, good_tokens [sp] int64).

    token_loss: [sp, B, Ns] float32 per-token losses; labels: [sp, B, Ns] int64.
    """
    if token_loss.dim() != 3 or token_loss.dtype != torch.float32:
        raise ValueError("token_loss must be [sp, B, Ns] float32")
    if labels.shape != token_loss.shape or labels.dtype != torch.int64:
        raise ValueError("labels must be int64 with token_loss's shape")
    sp, B, Ns = token_loss.shape
    dev = token_loss.device
    need = int(library().ulysses_sp_loss_workspace_bytes(sp, B, Ns))
    if workspace is None:
        workspace = torch.empty(max(need, 8), dtype=torch.uint8, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev) if loss is None else loss
    rank_loss = torch.empty(sp, dtype=torch.float32, device=dev) if rank_loss is None else rank_loss
    good_tokens = torch.empty(sp, dtype=torch.int64, device=dev) if good_tokens is None else good_tokens
    _expect(loss, (1,), torch.float32, "loss")
    _expect(rank_loss, (sp,), torch.float32, "rank_loss")
    _expect(good_tokens, (sp,), torch.int64, "good_tokens")
    _require_device(token_loss, labels, workspace, loss, rank_loss, good_tokens)
    _check("ulysses_sp_loss", library().ulysses_sp_loss(
        _ptr(token_loss), _ptr(labels), _ptr(rank_loss), _ptr(good_tokens), _ptr(loss), _ptr(workspace),
        workspace.numel() * workspace.element_size(), sp, B, Ns, int(ignore_index), _stream(token_loss)))
    return loss, rank_loss, good_tokens


# ------------------------------------------------------------------ tiled MLP
# x, y, dy, dx: [tokens, hidden] bf16; wg, wu: [inter, hidden] bf16; wd: [hidden, inter] bf16;
# weight gradients fp32, same shapes as the weights.


def ulysses_tiled_mlp_workspace_bytes(tokens: int, hidden: int, inter: int, tile: int) -> int:
    return int(library().ulysses_tiled_mlp_workspace_bytes(tokens, hidden, inter, tile))


def _mlp_shapes(x, wg, wu, wd):
    if x.dim() != 2 or x.dtype != torch.bfloat16:
        raise ValueError("x must be [tokens, hidden] bfloat16")
    tokens, hidden = x.shape
    inter = wg.shape[0]
    _expect(wg, (inter, hidden), torch.bfloat16, "w_gate")
    _expect(wu, (inter, hidden), torch.bfloat16, "w_up")
    _expect(wd, (hidden, inter), torch.bfloat16, "w_down")
    return tokens, hidden, inter


def _mlp_workspace(tokens, hidden, inter, tile, workspace, device):
    need = ulysses_tiled_mlp_workspace_bytes(tokens, hidden, inter, tile)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    return workspace


def ulysses_tiled_mlp_fwd(x, w_gate, w_up, w_down, tile: int, workspace=None, y=None):
    """Y = (silu(x Wg^T) * (x Wu^T)) Wd^T over tiles of `tile` tokens; returns y."""
    tokens, hidden, inter = _mlp_shapes(x, w_gate, w_up, w_down)
    workspace = _mlp_workspace(tokens, hidden, inter, tile, workspace, x.device)
    y = torch.empty_like(x) if y is None else y
    _expect(y, x.shape, x.dtype, "y")
    _require_device(x, w_gate, w_up, w_down, y, workspace)
    _check("ulysses_tiled_mlp_fwd", library().ulysses_tiled_mlp_fwd(
        _ptr(x), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(y), _ptr(workspace),
        workspace.numel() * workspace.element_size(), tokens, hidden, inter, int(tile), _stream(x)))
    return y


def ulysses_tiled_mlp_bwd(x, w_gate, w_up, w_down, dy, tile: int, workspace=None, dx=None, dw_gate=None,
                          dw_up=None, dw_down=None):
    """Gradients of the tiled MLP; returns (dx, dw_gate, dw_up, dw_down), weight gradients in fp32."""
    tokens, hidden, inter = _mlp_shapes(x, w_gate, w_up, w_down)
    _expect(dy, x.shape, x.dtype, "dy")
    workspace = _mlp_workspace(tokens, hidden, inter, tile, workspace, x.device)
    f32 = lambda t: torch.empty(t.shape, dtype=torch.float32, device=x.device)  # noqa: E731
    dx = torch.empty_like(x) if dx is None else dx
    dw_gate = f32(w_gate) if dw_gate is None else dw_gate
    dw_up = f32(w_up) if dw_up is None else dw_up
    dw_down = f32(w_down) if dw_down is None else dw_down
    _expect(dx, x.shape, x.dtype, "dx")
    for name, t, wt in (("dw_gate", dw_gate, w_gate), ("dw_up", dw_up, w_up), ("dw_down", dw_down, w_down)):
        _expect(t, wt.shape, torch.float32, name)
    _require_device(x, w_gate, w_up, w_down, dy, dx, dw_gate, dw_up, dw_down, workspace)
    _check("ulysses_tiled_mlp_bwd", library().ulysses_tiled_mlp_bwd(
        _ptr(x), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(dy), _ptr(dx), _ptr(dw_gate), _ptr(dw_up),
        _ptr(dw_down), _ptr(workspace), workspace.numel() * workspace.element_size(), tokens, hidden, inter,
        int(tile), _stream(x)))
    return dx, dw_gate, dw_up, dw_down


__all__ = [
    "DocPacking",
    "UlyssesError",
    "library",
    "ulysses_seq_to_head",
    "ulysses_head_to_seq",
    "ulysses_seq_to_head_n",
    "ulysses_head_to_seq_n",
    "ulysses_attn_fwd",
    "ulysses_attn_fwd_workspace_bytes",
    "ulysses_attn_bwd",
    "ulysses_attn_bwd_workspace_bytes",
    "ulysses_attn_bwd_noalloc",
    "ulysses_attn_bwd_prepare",
    "ulysses_attn_bwd_prepared",
    "ULY_NOALLOC_SCRATCH_BYTES",
    "ulysses_status_string",
    "ulysses_ring_attn_fwd_step",
    "ulysses_ring_attn_bwd_prepare",
    "ulysses_ring_attn_bwd_step",
    "ulysses_ring_attn_bwd_workspace_bytes",
    "ring_attn_fwd",
    "ring_attn_bwd",
    "ulysses_sp_loss",
    "ulysses_tiled_mlp_workspace_bytes",
    "ulysses_tiled_mlp_fwd",
    "ulysses_tiled_mlp_bwd",
]
