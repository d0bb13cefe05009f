"""Property tests of the oracle over random small shapes and document splits (CPU only)."""

from __future__ import annotations

import numpy as np
from hypothesis import given, settings, strategies as st

import oracle
import workloads


@st.composite
def _layouts(draw):
    sp = draw(st.sampled_from([1, 2, 3, 4]))
    Hl = draw(st.integers(1, 3))
    Ns = draw(st.integers(1, 5))
    B = draw(st.integers(1, 2))
    d = draw(st.sampled_from([1, 2, 8]))
    return sp, B, Ns, sp * Hl, d


@settings(max_examples=40, deadline=None)
@given(_layouts(), st.integers(0, 2**31 - 1))
def test_permute_roundtrips(shape, seed):
    x = np.random.default_rng(seed).integers(0, 2**16, size=shape, dtype=np.uint16)
    h = oracle.seq_to_head(x)
    sp, B, Ns, H, d = shape
    assert h.shape == (sp, B, Ns * sp, H // sp, d)
    assert np.array_equal(oracle.head_to_seq(h), x)


@settings(max_examples=25, deadline=None)
@given(st.integers(2, 40), st.integers(1, 5), st.booleans(), st.booleans(), st.integers(0, 2**31 - 1))
def test_packed_equals_separate_random_splits(N, ndoc, causal, allow_empty, seed):
    rng = np.random.default_rng(seed)
    ndoc = min(ndoc, N)
    lengths = workloads.random_lengths(rng, N, ndoc, allow_empty=allow_empty)
    cu = workloads.cu_seqlens_from_lengths(lengths)
    q, k, v, do = (rng.standard_normal((N, 2, 4)) for _ in range(4))
    O, L = oracle.attn_fwd(q, k, v, cu, causal)
    G = oracle.attn_bwd(q, k, v, do, cu, causal)
    for s, e in zip(cu[:-1], cu[1:]):
        if s == e:
            continue
        Os, Ls = oracle.attn_fwd(q[s:e], k[s:e], v[s:e], None, causal)
        Gs = oracle.attn_bwd(q[s:e], k[s:e], v[s:e], do[s:e], None, causal)
        np.testing.assert_allclose(O[s:e], Os, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(L[:, s:e], Ls, rtol=1e-12, atol=1e-13)
        for g, gs in zip(G, Gs):
            np.testing.assert_allclose(g[s:e], gs, rtol=1e-12, atol=1e-13)


def test_loguniform_lengths_cover_n():
    for seed in range(1, 6):
        lens = workloads.loguniform_doc_lengths(seed, 32768)
        assert sum(lens) == 32768
        assert all(1 <= L <= 8192 for L in lens)
        assert all(L >= 512 for L in lens[:-1])
