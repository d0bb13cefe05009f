"""Oracle for the seq-sharded <-> head-sharded layout change (test infrastructure only).

Source: HF Transformers docs, "Ulysses sequence parallelism" (deepspeed_alst),
opening paragraph and layout diagram: before attention each of the sp ranks
holds a contiguous block of N/sp tokens with all H heads (rank 0 the first
block); an all-to-all turns that into each rank holding all N tokens for a
contiguous block of H/sp heads (rank 0 the first heads); a second all-to-all
turns it back. The congresoia365 article "Nuevo método Ulysses ..." (section
"Cómo Funciona Ulysses", steps 1, 3 and 5) describes the same two exchanges.

Readings taken where the pages are silent:
  * inside a shard the layout is [B, tokens, heads, d], row-major;
  * the sp shards of all virtual ranks on one device are stacked along a
    leading axis, shard r at index r (as an all-to-all buffer with chunk r for
    rank r).

The oracle is the definition by slicing: glue the sequence shards back into
the full [B, N, H, d] tensor, then cut out each rank's head block (and the
reverse). It works on any dtype, so integer views compare bit for bit.
"""

from __future__ import annotations

import numpy as np


def seq_to_head(x_seq: np.ndarray) -> np.ndarray:
    """[sp, B, N/sp, H, d] sequence shards -> [sp, B, N, H/sp, d] head shards."""
    sp, B, Ns, H, d = x_seq.shape
    if H % sp:
        raise ValueError("H must be divisible by sp")
    Hl = H // sp
    full = np.concatenate([x_seq[s] for s in range(sp)], axis=1)  # [B, N, H, d]
    return np.stack([full[:, :, r * Hl:(r + 1) * Hl, :] for r in range(sp)])


def head_to_seq(x_head: np.ndarray) -> np.ndarray:
    """[sp, B, N, H/sp, d] head shards -> [sp, B, N/sp, H, d] sequence shards."""
    sp, B, N, Hl, d = x_head.shape
    if N % sp:
        raise ValueError("N must be divisible by sp")
    Ns = N // sp
    full = np.concatenate([x_head[r] for r in range(sp)], axis=2)  # [B, N, H, d]
    return np.stack([full[:, s * Ns:(s + 1) * Ns] for s in range(sp)])
