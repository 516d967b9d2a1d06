"""Pins of the oracle's CSR -> CSC sparse-index transpose (CPU only): scipy's csr->csc conversion
(library routine), dense 0/1 reconstruction, structural invariants and the round trip."""
import numpy as np
import pytest
import scipy.sparse as sp

import oracle

SHAPES = [(8, 2, 2, 1, 4), (64, 4, 2, 2, 8), (256, 4, 3, 2, 8), (4096, 16, 2, 8, 16), (64, 4, 2, 16, 8)]


def _sel(n, B, L, K, D, seed):
    g = np.random.default_rng(seed)
    x, y = g.standard_normal((2, n, D)), g.standard_normal((2, n, D))
    idx, _ = oracle.select(oracle.pool(x, B, L), oracle.pool(y, B, L), n, B, L, K)
    return idx


@pytest.mark.parametrize("n,B,L,K,D", SHAPES)
@pytest.mark.parametrize("Le", [None, 0, 1])
def test_transpose_matches_scipy_and_roundtrips(n, B, L, K, D, Le):
    Le = L if Le is None else Le
    idx = _sel(n, B, L, K, D, 40)
    cp, pm = oracle.index_transpose(idx, n, B, L, K, Le)
    T = max(1, min(Le, L))
    assert cp.shape[1] == sum(n // B ** l + 1 for l in range(1, T + 1))
    for s in range(idx.shape[0]):
        cpo = pmo = 0
        for l in range(1, T + 1):
            nl, off, kl = n // B ** l, oracle.level_offset(n, B, l), min(K, n // B ** l)
            rows = idx[s, off:off + nl]
            c, p = cp[s, cpo:cpo + nl + 1], pm[s, pmo:pmo + nl * K]
            # scipy: store position+1 as data so the CSC carries the CSR positions
            u, kk = np.nonzero(rows >= 0)
            csr = sp.csr_matrix(((u * K + kk + 1).astype(np.int64), (u, rows[u, kk])), shape=(nl, nl))
            csc = csr.tocsc()
            csc.sort_indices()
            assert np.array_equal(c, csc.indptr)
            assert np.array_equal(p[:c[-1]], csc.data - 1)
            # invariants
            assert c[0] == 0 and np.all(np.diff(c) >= 0) and c[-1] == nl * kl
            for j in range(nl):
                col = p[c[j]:c[j + 1]]
                assert np.all(np.diff(col) > 0)
                assert np.all(rows.reshape(-1)[col] == j)
            # dense reconstruction: transpose back gives the CSR
            dense_csr = np.zeros((nl, nl), np.int8)
            dense_csr[u, rows[u, kk]] = 1
            dense_csc = np.zeros((nl, nl), np.int8)
            for j in range(nl):
                dense_csc[p[c[j]:c[j + 1]] // K, j] = 1
            assert np.array_equal(dense_csr, dense_csc)
            cpo += nl + 1
            pmo += nl * K
