"""Float64 CPU oracle for the Ulysses per-rank attention path.

TEST INFRASTRUCTURE ONLY. This package is the slow, plain definition that the
GPU path is checked against. Only the test suite, the package smoke check and
the benchmark's CPU-baseline leg may import it; the product path never does,
and this package imports nothing from the product package.

Contents:
  permute    seq-sharded <-> head-sharded layout change of sp virtual ranks
             (the data movement of Ulysses' all-to-alls), by slicing.
  attention  exact softmax attention (causal or not, packed documents kept
             apart) forward with its log-sum-exp, and the analytic backward,
             in float64 with whole-row normalisation.
  ring       the ring-attention variant: blockwise attention of each rank's
             query chunk against key/value chunks passed around a ring,
             partial results merged by their log-sum-exp; its backward.
  loss       the sequence-parallel loss aggregation: per-rank mean loss and
             counted-token count, combined as a count-weighted mean.
  mlp        ALST's tiled MLP: the SwiGLU FFN over a rank's tokens, whole or
             tile by tile (intermediates recomputed in the backward, weight
             gradients accumulated over the tiles).

Every function here is pinned by tests that do not call it twice: closed
forms, finite differences, brute-force loops, an independent library
(torch float64 SDPA) and the invariants the pages state.
"""

from .permute import seq_to_head, head_to_seq  # noqa: F401
from .attention import (  # noqa: F401
    attn_fwd,
    attn_bwd,
    attn_fwd_rows,
    attn_bwd_dq_rows,
    attn_bwd_dkdv_cols,
    doc_ids,
)
from .loss import sp_loss, rank_losses, aggregate  # noqa: F401
from .mlp import mlp_fwd, mlp_bwd, tiled_mlp_fwd, tiled_mlp_bwd, mlp_bwd_weight_units  # noqa: F401
from .ring import ring_fwd, ring_bwd, ring_chunk, block_mode, block_attn, merge, stitch, stitch_lse  # noqa: F401
