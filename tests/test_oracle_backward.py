"""Pins of the oracle's backward (CPU only): torch autograd through the dense augmented formulation
(pooling as a reshape-mean so the B^-l chain is explicit), central finite differences of the oracle's
own forward with the selection held fixed, and the shift invariants sum_m dK[m] = 0 and
sum_m dV[m] = sum_n dO[n]."""
import numpy as np
import pytest
import torch

import oracle
from dense_ref import dense_forward

SHAPES = [(8, 2, 2, 1, 4), (64, 4, 2, 2, 8), (256, 4, 3, 2, 8), (1024, 16, 1, 4, 16), (4096, 16, 2, 8, 16)]


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("n,B,L,K,D", SHAPES)
@pytest.mark.parametrize("Le", [None, 1])
def test_backward_matches_autograd(n, B, L, K, D, Le):
    Le = L if Le is None else min(Le, L)
    q, k, v, do = (_rand((2, n, D), 50 + i) for i in range(4))
    r = oracle.run(q, k, v, B, K, levels=L, enrich_levels=Le, dout=do)
    qt, kt, vt = (torch.from_numpy(a).requires_grad_(True) for a in (q, k, v))
    o, _ = dense_forward(qt, kt, vt, r["idx"], B, L, Le, r["scale"])
    (o * torch.from_numpy(do)).sum().backward()
    for name, t in (("dq", qt), ("dk", kt), ("dv", vt)):
        np.testing.assert_allclose(r[name], t.grad.numpy(), rtol=0, atol=1e-10, err_msg=name)


@pytest.mark.parametrize("n,B,L,K,D", SHAPES[:3])
def test_backward_matches_finite_differences(n, B, L, K, D):
    q, k, v, do = (_rand((1, n, D), 60 + i) for i in range(4))
    r = oracle.run(q, k, v, B, K, levels=L, dout=do)
    idx, sigma = r["idx"], r["scale"]

    def loss(qq, kk, vv):
        o, _ = oracle.attn_fwd(qq, kk, vv, oracle.pool(kk, B, L), oracle.pool(vv, B, L), idx, B, L, K, L, sigma)
        return float((o * do).sum())

    h = 1e-6
    g = np.random.default_rng(61)
    for name, arr, pos in (("dq", q, 0), ("dk", k, 1), ("dv", v, 2)):
        picks = [(int(g.integers(n)), int(g.integers(D))) for _ in range(12)]
        for (m, c) in picks:
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[pos][0, m, c] += h
            args_m[pos][0, m, c] -= h
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - r[name][0, m, c]) < 1e-6 * max(1.0, abs(fd)), (name, m, c, fd, r[name][0, m, c])


@pytest.mark.parametrize("n,B,L,K,D", SHAPES)
def test_backward_shift_invariants(n, B, L, K, D):
    q, k, v, do = (_rand((2, n, D), 70 + i) for i in range(4))
    r = oracle.run(q, k, v, B, K, levels=L, dout=do)
    np.testing.assert_allclose(r["dk"].sum(1), 0.0, rtol=0, atol=1e-10)
    np.testing.assert_allclose(r["dv"].sum(1), do.sum(1), rtol=0, atol=1e-10)
