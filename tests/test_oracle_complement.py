"""Pins of the oracle's complement-partition reading of the enrichment (CPU only).

Under this reading a query's entries are the fine tokens of its kept level-1 blocks plus, at every level l,
the pooled tokens of the candidates its level-l unit scored and did not keep (bias l ln B).  Pins that do not
restate the construction:
  * coverage: the entry weights (1 per raw token, B^l per level-l pooled token) add up to n for every query
    when L_e = L -- each raw key is represented exactly once -- while the selected-token reading does not;
  * K, V constant on every B^L span (so every pooled token equals each token it pools): the attention equals
    full dense attention exactly (torch fp64 SDPA), for any selection -- and the selected-token reading does
    not;
  * every candidate kept at every level: no pooled entry is left, the attention is full dense attention.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

CASES = [(64, 4, 2, 2, 8), (256, 4, 3, 2, 8), (1024, 16, 1, 8, 16), (4096, 16, 2, 4, 16)]


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _dense(q, k, v, scale):
    qt, kt, vt = (torch.from_numpy(a) for a in (q, k, v))
    return F.scaled_dot_product_attention(qt, kt, vt, scale=scale).numpy()


def _piecewise(shape, span, seed):
    bh, n, D = shape
    return np.repeat(_rand((bh, n // span, D), seed), span, axis=1)


@pytest.mark.parametrize("n,B,L,K,D", CASES)
def test_entry_weights_cover_every_key_once(n, B, L, K, D):
    q, k, v = _rand((1, n, D), 1), _rand((1, n, D), 2), _rand((1, n, D), 3)
    r = oracle.run(q, k, v, B, K, levels=L)
    idx = r["idx"][0]
    ne_sel = None
    for t in range(0, n, max(1, n // 97)):
        ne, w = oracle.entry_weight(idx, n, B, L, K, L, t, complement=True)
        assert w == n, (t, w)
        ne_sel, w_sel = oracle.entry_weight(idx, n, B, L, K, L, t, complement=False)
        assert w_sel != n  # the selected-token reading covers keys a different number of times
    assert ne_sel is not None


@pytest.mark.parametrize("n,B,L,K,D", CASES)
def test_constant_spans_give_dense_attention(n, B, L, K, D):
    q = _rand((2, n, D), 4)
    k, v = _piecewise((2, n, D), B ** L, 5), _piecewise((2, n, D), B ** L, 6)
    scale = 1.0 / np.sqrt(D)
    pk, pv = oracle.pool(k, B, L), oracle.pool(v, B, L)
    idx, _ = oracle.select(oracle.pool(q, B, L), pk, n, B, L, K)
    dense = _dense(q, k, v, scale)
    o, _ = oracle.attn_fwd(q, k, v, pk, pv, idx, B, L, K, L, scale, complement=True)
    np.testing.assert_allclose(o, dense, rtol=0, atol=1e-12)
    o_sel, _ = oracle.attn_fwd(q, k, v, pk, pv, idx, B, L, K, L, scale, complement=False)
    assert np.abs(o_sel - dense).max() > 1e-6


@pytest.mark.parametrize("n,B,L", [(64, 4, 2), (256, 4, 3)])
def test_everything_kept_is_dense_attention(n, B, L):
    D = 8
    K = n // B  # every level-1 block kept, hence every candidate of every level
    q, k, v = _rand((2, n, D), 7), _rand((2, n, D), 8), _rand((2, n, D), 9)
    scale = 1.0 / np.sqrt(D)
    pk, pv = oracle.pool(k, B, L), oracle.pool(v, B, L)
    idx, _ = oracle.select(oracle.pool(q, B, L), pk, n, B, L, K)
    o, _ = oracle.attn_fwd(q, k, v, pk, pv, idx, B, L, K, L, scale, complement=True)
    np.testing.assert_allclose(o, _dense(q, k, v, scale), rtol=0, atol=1e-12)
