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


def _dense_grads(q, k, v, dout, scale):
    qt, kt, vt = (torch.from_numpy(a).requires_grad_(True) for a in (q, k, v))
    o = F.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    o.backward(torch.from_numpy(dout))
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("n,B,L,K,D", CASES)
def test_backward_constant_spans_give_dense_gradients(n, B, L, K, D):
    """K, V constant on every B^L span: every query sees each key once (itself or one pooled ancestor whose
    logit carries + l ln B), so dQ, dK, dV equal dense attention's gradients (torch autograd, fp64) -- the
    pooled token's gradient, spread B^-l over its span, is each key's dense gradient.  The selected-token
    reading's gradients differ."""
    q, dout = _rand((2, n, D), 14), _rand((2, n, D), 17)
    k, v = _piecewise((2, n, D), B ** L, 15), _piecewise((2, n, D), B ** L, 16)
    scale = 1.0 / np.sqrt(D)
    pk, pv = oracle.pool(k, B, L), oracle.pool(v, B, L)
    idx, _ = oracle.select(oracle.pool(q, B, L), pk, n, B, L, K)
    ref = _dense_grads(q, k, v, dout, scale)
    o, lse = oracle.attn_fwd(q, k, v, pk, pv, idx, B, L, K, L, scale, complement=True)
    got = oracle.attn_bwd(q, k, v, o, lse, dout, pk, pv, idx, B, L, K, L, scale, complement=True)
    for g, r in zip(got, ref):
        np.testing.assert_allclose(g, r, rtol=0, atol=1e-10)
    o1, lse1 = oracle.attn_fwd(q, k, v, pk, pv, idx, B, L, K, L, scale)
    sel = oracle.attn_bwd(q, k, v, o1, lse1, dout, pk, pv, idx, B, L, K, L, scale)
    assert max(np.abs(g - r).max() for g, r in zip(sel, ref)) > 1e-6


@pytest.mark.parametrize("n,B,L,K,Le", [(256, 4, 3, 2, 3), (256, 4, 3, 3, 2), (512, 16, 1, 3, 1)])
def test_backward_matches_finite_differences(n, B, L, K, Le):
    """Central differences of sum(dO * O) through the oracle's complement forward, with the pyramid re-pooled
    from the perturbed K and V and the selection held fixed (no gradient through Top-K), on sampled elements
    of Q, K and V."""
    D = 8
    q, k, v, dout = (_rand((1, n, D), s) for s in (21, 22, 23, 24))
    scale = 1.0 / np.sqrt(D)
    idx, _ = oracle.select(oracle.pool(q, B, L), oracle.pool(k, B, L), n, B, L, K)

    def loss(qq, kk, vv):
        o, _ = oracle.attn_fwd(qq, kk, vv, oracle.pool(kk, B, L), oracle.pool(vv, B, L), idx, B, L, K, Le, scale,
                               complement=True)
        return float((o * dout).sum())

    pk, pv = oracle.pool(k, B, L), oracle.pool(v, B, L)
    o, lse = oracle.attn_fwd(q, k, v, pk, pv, idx, B, L, K, Le, scale, complement=True)
    grads = oracle.attn_bwd(q, k, v, o, lse, dout, pk, pv, idx, B, L, K, Le, scale, complement=True)
    rng = np.random.default_rng(25)
    h = 1e-5
    for which in range(3):
        for _ in range(12):
            t, c = int(rng.integers(n)), int(rng.integers(D))
            args = [q.copy(), k.copy(), v.copy()]
            args[which][0, t, c] += h
            up = loss(*args)
            args[which][0, t, c] -= 2 * h
            dn = loss(*args)
            fd = (up - dn) / (2 * h)
            assert abs(fd - grads[which][0, t, c]) <= 1e-7 * max(1.0, abs(fd)), (which, t, c, fd,
                                                                              grads[which][0, t, c])
