"""Pins of the oracle's pooling and hierarchical Top-K (CPU only).

Pyramid: direct mean over the B^l raw tokens of each level-l unit (a closed form that is not the
oracle's recursive pooling) and the mass invariant.  Selection: exhaustive sort of every candidate set,
the structure of each row, the single-level special case L = 1 (plain exhaustive Top-K over all N/B
blocks), and the exact count of scored pairs from the complexity argument of the LLSA review page
(Sec. 4.2 / Eq. 6 as relayed in "Circularity Check").
"""
import numpy as np
import pytest

import oracle
from dense_ref import exhaustive_topk

PARTIAL = [(8, 2, 2, 1, 4), (64, 4, 2, 2, 8), (256, 4, 3, 2, 8), (4096, 16, 2, 8, 16)]
FULL = [(64, 4, 2, 16, 8), (256, 4, 1, 64, 8)]


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("n,B,L,K,D", PARTIAL + FULL)
def test_pool_direct_mean_and_mass(n, B, L, K, D):
    x = _rand((3, n, D), 1)
    pyr = oracle.pool(x, B, L)
    for l in range(1, L + 1):
        off, rows, span = oracle.level_offset(n, B, l), n // B ** l, B ** l
        direct = x.reshape(3, rows, span, D).mean(axis=2)
        np.testing.assert_allclose(pyr[:, off:off + rows], direct, rtol=0, atol=1e-13)
        # mass invariant: sum_j B^l X^(l)[j] = sum_m X[m]
        np.testing.assert_allclose(span * pyr[:, off:off + rows].sum(1), x.sum(1), rtol=1e-12, atol=1e-12)


def test_default_levels_formula():
    # L = floor(log_B N - 1) for the workloads' sequence lengths and the Figure 1 toy
    assert oracle.default_levels(4096, 16) == 2
    assert oracle.default_levels(16384, 16) == 2
    assert oracle.default_levels(65536, 16) == 3
    assert oracle.default_levels(262144, 16) == 3
    assert oracle.default_levels(8, 2) == 2
    # boundary: exactly a power of B
    assert oracle.default_levels(16 ** 5, 16) == 4
    assert oracle.default_levels(16 ** 5 - 16, 16) == 3


def _check_selection(pq, pk, idx, n, B, L, K):
    """Brute-force every level: full sort of the candidate set implied by the parent row."""
    bh = pq.shape[0]
    for s in range(bh):
        nL, offL = n // B ** L, oracle.level_offset(n, B, L)
        kL = min(K, nL)
        for u in range(nL):
            cand = np.arange(nL)
            sc = pk[s, offL:offL + nL] @ pq[s, offL + u]
            ref = exhaustive_topk(sc, cand, kL)
            row = idx[s, offL + u]
            assert list(row[:kL]) == list(ref)
            assert all(row[kL:] == -1)
        for l in range(L - 1, 0, -1):
            nl, off, offp = n // B ** l, oracle.level_offset(n, B, l), oracle.level_offset(n, B, l + 1)
            kp, kl = min(K, n // B ** (l + 1)), min(K, nl)
            for u in range(nl):
                parent = idx[s, offp + u // B, :kp]
                cand = (parent[:, None] * B + np.arange(B)[None]).reshape(-1)
                sc = pk[s, off + cand] @ pq[s, off + u]
                ref = exhaustive_topk(sc, cand, kl)
                row = idx[s, off + u]
                assert list(row[:kl]) == list(ref), (s, l, u)
                assert len(set(row[:kl])) == kl and np.all(np.diff(row[:kl]) > 0)
                assert set(row[:kl]) <= set(cand)


@pytest.mark.parametrize("n,B,L,K,D", PARTIAL + FULL)
def test_select_matches_exhaustive_sort(n, B, L, K, D):
    x = _rand((2, n, D), 2)
    y = _rand((2, n, D), 3)
    pq, pk = oracle.pool(x, B, L), oracle.pool(y, B, L)
    idx, pairs = oracle.select(pq, pk, n, B, L, K)
    _check_selection(pq, pk, idx, n, B, L, K)
    # exact number of scored (unit, block) pairs: n_L^2 + sum_{l<L} n_l * k_{l+1} * B, per slice
    expect = (n // B ** L) ** 2 + sum((n // B ** l) * min(K, n // B ** (l + 1)) * B for l in range(1, L))
    assert pairs == 2 * expect


@pytest.mark.parametrize("n,B,K", [(64, 4, 3), (256, 16, 4), (4096, 16, 8)])
def test_single_level_is_exhaustive_topk(n, B, K):
    """L = 1: the hierarchy degenerates to single-level Top-K over all N/B blocks (Figure 1, left)."""
    x, y = _rand((1, n, 8), 4), _rand((1, n, 8), 5)
    q1 = x.reshape(1, n // B, B, 8).mean(2)
    k1 = y.reshape(1, n // B, B, 8).mean(2)
    idx, _ = oracle.select(oracle.pool(x, B, 1), oracle.pool(y, B, 1), n, B, 1, K)
    for u in range(n // B):
        ref = exhaustive_topk(k1[0] @ q1[0, u], np.arange(n // B), K)
        assert list(idx[0, u]) == list(ref)


@pytest.mark.parametrize("n,B,L,K,D", FULL)
def test_full_coverage_selects_everything(n, B, L, K, D):
    x, y = _rand((1, n, D), 6), _rand((1, n, D), 7)
    idx, _ = oracle.select(oracle.pool(x, B, L), oracle.pool(y, B, L), n, B, L, K)
    for l in range(1, L + 1):
        nl, off = n // B ** l, oracle.level_offset(n, B, l)
        for u in range(nl):
            assert list(idx[0, off + u, :nl]) == list(range(nl))


def test_tie_rule_lower_index_wins():
    """All pooled keys equal: every score ties, so each unit keeps the K lowest block indices."""
    n, B, L, K = 256, 4, 3, 2
    x = _rand((1, n, 4), 8)
    y = np.ones((1, n, 4))
    idx, _ = oracle.select(oracle.pool(x, B, L), oracle.pool(y, B, L), n, B, L, K)
    off3 = oracle.level_offset(n, B, 3)
    assert list(idx[0, off3]) == [0, 1]
    # level 2 candidates are children of {0, 1} -> {0..7}; ties keep 0, 1
    off2 = oracle.level_offset(n, B, 2)
    assert all(list(idx[0, off2 + u]) == [0, 1] for u in range(n // 16))


@pytest.mark.parametrize("where", ["q", "k", "v", "dout"])
@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_oracle_rejects_non_finite_inputs(where, bad):
    """Non-finite inputs lie outside the method's definition: every oracle step refuses them."""
    rng = np.random.default_rng(3)
    x = {nm: rng.standard_normal((1, 64, 4)) for nm in ("q", "k", "v", "dout")}
    x[where][0, 17, 2] = bad
    with pytest.raises(ValueError, match="non-finite"):
        oracle.run(x["q"], x["k"], x["v"], 4, 2, levels=2, dout=x["dout"])
    if where != "dout":
        with pytest.raises(ValueError, match="non-finite"):
            oracle.pool(x[where], 4, 2)
