"""Oracle for the sequence-parallel loss aggregation (test infrastructure only).

Source: the jianying88 guide to DeepSpeed Ulysses in Transformers (the
gitcode page), section on the work Trainer does by itself, item 3 (weighted
loss aggregation across ranks). Each SP rank holds a different slice of the
sequence, so it has its own loss (the mean over its own counted tokens) and
its own count of counted tokens, good_tokens = the number of shift_labels
that are not -100. Both are all-gathered over the SP group and combined as

    loss = sum_r (loss_r * good_r) / sum_r good_r,

leaving out ranks whose good_r is 0 (for example a slice made only of
prompt tokens, all labelled -100). The page notes that this equals the mean
over every counted token of the whole batch, which a plain mean of the rank
losses would not.

Readings where the page is silent:
  * Per-token losses are given (the model's cross-entropy per position) as
    float; labels are int64 with -100 marking a position that does not count.
    A position that does not count contributes nothing, whatever its loss
    value holds (NaN or inf included).
  * A rank with no counted token has loss_r = 0 (a mean over nothing) and
    weight 0. If no rank has a counted token, the aggregated loss is 0.

Layouts: token_loss, labels [sp][B][Ns] (rank r's own B rows of Ns tokens).
Float64 throughout.
"""

from __future__ import annotations

import numpy as np

IGNORE_INDEX = -100


def rank_losses(token_loss, labels, ignore_index: int = IGNORE_INDEX):
    """Per rank: (loss_r as the mean over its counted tokens, good_r as int64)."""
    tl = np.asarray(token_loss, dtype=np.float64)
    lab = np.asarray(labels)
    sp = tl.shape[0]
    loss = np.zeros(sp)
    good = np.zeros(sp, dtype=np.int64)
    for r in range(sp):
        keep = lab[r] != ignore_index
        good[r] = int(keep.sum())
        if good[r] > 0:
            loss[r] = tl[r][keep].sum() / good[r]
    return loss, good


def aggregate(loss, good):
    """The all-gathered (loss_r, good_r) of every rank -> the weighted mean, zero-count ranks left out."""
    loss = np.asarray(loss, dtype=np.float64)
    good = np.asarray(good, dtype=np.int64)
    use = good > 0
    total = int(good[use].sum())
    if total == 0:
        return 0.0
    return float((loss[use] * good[use]).sum() / total)


def sp_loss(token_loss, labels, ignore_index: int = IGNORE_INDEX):
    """(loss, loss_r [sp], good_r [sp]) of sp ranks."""
    loss_r, good_r = rank_losses(token_loss, labels, ignore_index)
    return aggregate(loss_r, good_r), loss_r, good_r
