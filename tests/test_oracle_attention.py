"""Pins of the oracle's enriched sparse attention forward (CPU only).

* dense masked attention on the augmented sequence via torch SDPA (library routine);
* special cases where the method reduces to full attention exactly (K covers every block);
* the multiplicity identity that pins the enrichment weight W^(l) = B^l under the nearest-upsample
  assumption, with a negative control (W = 1) that must fail;
* softmax normalisation and shift equivariance.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from dense_ref import bias_matrix, dense_forward

PARTIAL = [(8, 2, 2, 1, 4), (64, 4, 2, 2, 8), (256, 4, 3, 2, 8), (4096, 16, 2, 8, 16)]


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _full_sdpa(q, k, v, scale, log_mult=None):
    qt, kt, vt = (torch.from_numpy(a) for a in (q, k, v))
    mask = None if log_mult is None else torch.from_numpy(log_mult)
    return F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale).numpy()


@pytest.mark.parametrize("n,B,L,K,D", PARTIAL)
def test_forward_matches_dense_masked_sdpa(n, B, L, K, D):
    q, k, v = _rand((2, n, D), 10), _rand((2, n, D), 11), _rand((2, n, D), 12)
    r = oracle.run(q, k, v, B, K, levels=L)
    o, lse = dense_forward(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), r["idx"], B, L, L,
                           r["scale"])
    np.testing.assert_allclose(r["o"], o.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["lse"], lse.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("n,B,L,K,D", [(64, 4, 2, 16, 8), (256, 4, 1, 64, 8), (256, 4, 3, 64, 8)])
def test_no_enrichment_full_coverage_is_full_attention(n, B, L, K, D):
    q, k, v = _rand((2, n, D), 13), _rand((2, n, D), 14), _rand((2, n, D), 15)
    r = oracle.run(q, k, v, B, K, levels=L, enrich_levels=0)
    np.testing.assert_allclose(r["o"], _full_sdpa(q, k, v, r["scale"]), rtol=0, atol=1e-12)


def _piecewise(shape, span, seed):
    bh, n, D = shape
    base = _rand((bh, n // span, D), seed)
    return np.repeat(base, span, axis=1)


@pytest.mark.parametrize("n,B,L,K,D", [(64, 4, 2, 16, 8), (256, 4, 3, 64, 8), (256, 4, 1, 64, 8)])
def test_enriched_full_coverage_constant_spans_is_full_attention(n, B, L, K, D):
    """Every block kept at every level and K, V constant on each B^L span: each raw token gains the
    same multiplicity 1 + L, which cancels in the softmax."""
    q = _rand((2, n, D), 16)
    k, v = _piecewise((2, n, D), B ** L, 17), _piecewise((2, n, D), B ** L, 18)
    r = oracle.run(q, k, v, B, K, levels=L)
    np.testing.assert_allclose(r["o"], _full_sdpa(q, k, v, r["scale"]), rtol=0, atol=1e-12)


def _multiplicity_logbias(idx, n, B, L, Le, weights):
    """log mu_n(m): raw token m counted once if its block is fine-selected, plus weights[l]/B^l per
    level l whose kept set (for the query's level-l ancestor) contains m's level-l unit."""
    bh = idx.shape[0]
    offs = [oracle.level_offset(n, B, l) for l in range(1, L + 1)]
    out = np.full((bh, n, n), -np.inf)
    for s in range(bh):
        for qi in range(n):
            i = qi // B
            mu = np.zeros(n)
            fine = set(int(c) for c in idx[s, offs[0] + i] if c >= 0)
            mu += np.array([1.0 if (m // B) in fine else 0.0 for m in range(n)])
            for l in range(1, Le + 1):
                kept = set(int(j) for j in idx[s, offs[l - 1] + i // B ** (l - 1)] if j >= 0)
                mu += np.array([weights[l - 1] / B ** l if (m // B ** l) in kept else 0.0 for m in range(n)])
            with np.errstate(divide="ignore"):
                out[s, qi] = np.log(mu)
    return out


@pytest.mark.parametrize("n,B,L,K,D", [(64, 4, 2, 2, 8), (256, 4, 3, 2, 8), (256, 4, 2, 3, 4)])
def test_multiplicity_identity_pins_weights(n, B, L, K, D):
    """K, V constant on each B^L span: a kept level-l token with weight B^l is exactly B^l copies of
    the raw tokens it pools, so the output equals dense attention over raw tokens with integer
    multiplicities.  With weight 1 instead of B^l (negative control) the identity must break."""
    q = _rand((2, n, D), 19)
    k, v = _piecewise((2, n, D), B ** L, 20), _piecewise((2, n, D), B ** L, 21)
    r = oracle.run(q, k, v, B, K, levels=L)
    good = _multiplicity_logbias(r["idx"], n, B, L, L, [B ** l for l in range(1, L + 1)])
    np.testing.assert_allclose(r["o"], _full_sdpa(q, k, v, r["scale"], good), rtol=0, atol=1e-12)
    bad = _multiplicity_logbias(r["idx"], n, B, L, L, [1.0] * L)
    assert np.abs(r["o"] - _full_sdpa(q, k, v, r["scale"], bad)).max() > 1e-3


@pytest.mark.parametrize("n,B,L,K,D", PARTIAL)
def test_softmax_rows_sum_to_one(n, B, L, K, D):
    q, k, v = _rand((1, n, D), 22), _rand((1, n, D), 23), _rand((1, n, D), 24)
    r = oracle.run(q, k, v, B, K, levels=L)
    kk = np.concatenate([k[0], r["pk"][0]], 0)
    logits = r["scale"] * q[0] @ kk.T + bias_matrix(r["idx"][0], n, B, L, L)
    p = np.exp(logits - r["lse"][0][:, None])
    np.testing.assert_allclose(p.sum(1), 1.0, rtol=0, atol=1e-12)
    # entry count per query: k_1 * B fine tokens + sum_l k_l coarse tokens
    cnt = np.isfinite(logits).sum(1)
    assert np.all(cnt == min(K, n // B) * B + sum(min(K, n // B ** l) for l in range(1, L + 1)))


@pytest.mark.parametrize("n,B,L,K,D", PARTIAL[1:])
def test_shift_equivariance(n, B, L, K, D):
    q, k, v = _rand((1, n, D), 25), _rand((1, n, D), 26), _rand((1, n, D), 27)
    c = _rand((1, 1, D), 28)
    base = oracle.run(q, k, v, B, K, levels=L)
    shifted_k = oracle.run(q, k + c, v, B, K, levels=L)
    shifted_v = oracle.run(q, k, v + c, B, K, levels=L)
    assert np.array_equal(base["idx"], shifted_k["idx"])
    np.testing.assert_allclose(shifted_k["o"], base["o"], rtol=0, atol=1e-10)
    np.testing.assert_allclose(shifted_v["o"], base["o"] + c, rtol=0, atol=1e-12)


def test_partial_enrichment_levels():
    """Le < L appends levels 1..Le only (finest first)."""
    n, B, L, K, D = 256, 4, 3, 2, 8
    q, k, v = _rand((1, n, D), 29), _rand((1, n, D), 30), _rand((1, n, D), 31)
    for Le in (0, 1, 2):
        r = oracle.run(q, k, v, B, K, levels=L, enrich_levels=Le)
        o, _ = dense_forward(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), r["idx"], B, L, Le,
                             r["scale"])
        np.testing.assert_allclose(r["o"], o.numpy(), rtol=0, atol=1e-12)
