"""Seeded synthetic inputs for the Ulysses per-rank attention path.

This module only draws numbers and describes shapes. It holds none of the
attention or layout arithmetic, so both the float64 oracle's tests and the
GPU path's tests and benchmark can take their inputs from it without sharing
any computation.

Workloads (shapes of the pages' setting: Llama-style 32 heads of width 128,
sequences from 4k to a million tokens split over ``sp`` sequence-parallel
ranks; see the HF Transformers "Ulysses sequence parallelism" guide, section
on configuration, where a 32-head model allows sp in {1, 2, 4, 8, 16, 32}):

  tiny      B=1 N=256    H=4  sp=2  d=64  fp32, one causal document
  llama7b   B=2 N=4096   H=32 sp=4  d=128 bf16, one causal document per row
  packed    B=1 N=32768  H=8  sp=1  d=128 bf16, documents log-uniform in
            [512, 8192] tokens (last one truncated to fit), causal
  long      B=1 N=131072 H=32 sp=8  d=128 bf16 (values scaled by 0.5)
  million   B=1 N=524288 H=32 sp=16 d=128 bf16, 4 documents of 131072

Random draws: a CPU ``torch.Generator`` seeded with the workload's seed draws
q, k, v, dO in that order as float32 N(0,1) (times the workload's scale), and
bf16 workloads round them to bf16 with round-to-nearest-even. Document lengths
come from ``numpy.random.default_rng(seed)``.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    N: int
    H: int
    sp: int
    d: int
    dtype: str  # "fp32" or "bf16"
    seed: int
    scale: float = 1.0
    causal: bool = True
    docs: str = "single"  # "single", "loguniform", or "equal4"

    @property
    def Hl(self) -> int:
        return self.H // self.sp

    @property
    def Ns(self) -> int:
        return self.N // self.sp


WORKLOADS = {
    "tiny": Workload("tiny", B=1, N=256, H=4, sp=2, d=64, dtype="fp32", seed=1),
    "llama7b": Workload("llama7b", B=2, N=4096, H=32, sp=4, d=128, dtype="bf16", seed=2),
    "packed": Workload("packed", B=1, N=32768, H=8, sp=1, d=128, dtype="bf16", seed=3,
                       docs="loguniform"),
    "long": Workload("long", B=1, N=131072, H=32, sp=8, d=128, dtype="bf16", seed=4, scale=0.5),
    "million": Workload("million", B=1, N=524288, H=32, sp=16, d=128, dtype="bf16", seed=5,
                        docs="equal4"),
}


def torch_dtype(name: str) -> torch.dtype:
    return {"fp32": torch.float32, "bf16": torch.bfloat16}[name]


def loguniform_doc_lengths(seed: int, N: int, lo: int = 512, hi: int = 8192) -> list[int]:
    """Document lengths L = floor(exp(U[ln lo, ln hi))) drawn until they cover N.

    The last length is cut so the lengths sum to exactly N (it may end up below
    ``lo``, which is kept as an edge case).
    """
    rng = np.random.default_rng(seed)
    lens: list[int] = []
    total = 0
    while total < N:
        L = int(math.floor(math.exp(rng.uniform(math.log(lo), math.log(hi)))))
        L = min(L, N - total)
        lens.append(L)
        total += L
    return lens


def cu_seqlens_from_lengths(lengths) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


def workload_cu_seqlens(w: Workload) -> np.ndarray | None:
    """cu_seqlens (int32, [ndoc+1]) of a workload, or None for one document per row."""
    if w.docs == "single":
        return None
    if w.docs == "loguniform":
        return cu_seqlens_from_lengths(loguniform_doc_lengths(w.seed, w.N))
    if w.docs == "equal4":
        return cu_seqlens_from_lengths([w.N // 4] * 4)
    raise ValueError(w.docs)


def random_lengths(rng: np.random.Generator, N: int, ndoc: int, allow_empty: bool = False) -> list[int]:
    """Split N into ndoc lengths at random cut points (small test cases)."""
    if ndoc == 1:
        return [N]
    lo = 0 if allow_empty else 1
    cuts = np.sort(rng.choice(np.arange(lo, N + 1 - lo), size=ndoc - 1, replace=allow_empty))
    bounds = np.concatenate([[0], cuts, [N]])
    return [int(x) for x in np.diff(bounds)]


def randn(shape, generator: torch.Generator, dtype: str, scale: float = 1.0) -> torch.Tensor:
    x = torch.randn(*shape, generator=generator, dtype=torch.float32)
    if scale != 1.0:
        x = x * scale
    return x.to(torch_dtype(dtype))


def qkv_do(shape, seed: int, dtype: str, scale: float = 1.0):
    """q, k, v, dO of the given shape, drawn in that order from one seeded CPU generator."""
    g = torch.Generator().manual_seed(seed)
    return tuple(randn(shape, g, dtype, scale) for _ in range(4))


def share_shape(w: Workload, n_ranks: int = 1) -> tuple:
    """Stacked per-rank head-sharded shares: [n_ranks, B, N, Hl, d]."""
    return (n_ranks, w.B, w.N, w.Hl, w.d)


def seq_shard_shape(w: Workload) -> tuple:
    """All sp sequence shards stacked: [sp, B, N/sp, H, d]."""
    return (w.sp, w.B, w.Ns, w.H, w.d)


def random_bits(shape, seed: int, dtype: str) -> torch.Tensor:
    """Arbitrary bit patterns (NaN payloads, -0, infinities included) viewed as ``dtype``."""
    g = torch.Generator().manual_seed(seed)
    if dtype == "bf16":
        raw = torch.randint(-(1 << 15), 1 << 15, shape, generator=g, dtype=torch.int16)
        return raw.view(torch.bfloat16)
    raw = torch.randint(-(1 << 31), (1 << 31) - 1, shape, generator=g, dtype=torch.int32)
    return raw.view(torch.float32)


# ------------------------------------------------------------- tiled MLP inputs
# The FFN of the Llama-style model the workloads are shaped like: hidden =
# H * d = 4096 and the Llama-7B intermediate width 11008; its tokens are one
# rank's sequence shard (N / sp of them). Weights are drawn like a standard
# initialisation, N(0, 1/fan_in), activations and their gradients N(0, 1).
MLP_HIDDEN, MLP_INTER = 4096, 11008


def mlp_inputs(tokens: int, hidden: int, inter: int, seed: int, dtype: str = "bf16"):
    """x [tokens, hidden], w_gate, w_up [inter, hidden], w_down [hidden, inter],
    dy [tokens, hidden], drawn in that order from one seeded CPU generator."""
    g = torch.Generator().manual_seed(seed)
    x = randn((tokens, hidden), g, dtype)
    wg = randn((inter, hidden), g, dtype, hidden ** -0.5)
    wu = randn((inter, hidden), g, dtype, hidden ** -0.5)
    wd = randn((hidden, inter), g, dtype, inter ** -0.5)
    dy = randn((tokens, hidden), g, dtype)
    return x, wg, wu, wd, dy
