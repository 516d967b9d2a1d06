"""GPU selection under exact ties, bit for bit against the oracle on every row.

Q and K take integer values in {-1, 0, 1}.  Pooling divides by B = 16 (exact in binary).  A level-l pooled value
is a multiple of 2^-4l in [-1, 1].  With L <= 2, every score is a multiple of 2^-16 of magnitude at most 64: 22
significant bits at most, exact in the GPU's fp32 (in any summation order) as in the oracle's fp64.  Scores then
repeat a great deal, and the K-th and (K+1)-th often tie.  The selection must realise the tie rule (equal
scores go to the lower block index) exactly, at every level, with no parity band.  The cases cover each Top-K
path of the selection kernel:
  * sorted-list merges of 8 keys per lane (K <= 8, at most 128 candidates);
  * merges of 16 keys per lane (K <= 16, at most 256 candidates);
  * the bitwise threshold search (K = 32).
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

B, D = 16, 64
CASES = [  # (n, K, L)
    (512, 3, 1),
    (4096, 8, 2),
    (4096, 16, 2),
    (16384, 5, 2),
    (65536, 16, 2),
    (65536, 32, 2),
]


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from hierarchical_sparse_attention_mean_amd import llsa
    return llsa


@pytest.mark.parametrize("n,K,levels", CASES, ids=[f"n{c[0]}_K{c[1]}_L{c[2]}" for c in CASES])
def test_selection_ties_exact(L, n, K, levels):
    rng = np.random.default_rng(1000 + n + K + levels)
    q, k, v = (rng.integers(-1, 2, size=(1, n, D)).astype(np.float64) for _ in range(3))
    idx_ref, _ = oracle.select(oracle.pool(q, B, levels), oracle.pool(k, B, levels), n, B, levels, K)
    b = L.Buffers(L.problem(1, 1, n, D, B, K, levels), backward=False)
    dev = lambda a: torch.from_numpy(a.astype(np.float32)).cuda().to(torch.bfloat16)  # exact: small integers
    b.pyramid(dev(q), dev(k), dev(v))
    L.select(b.prob, b.pq, b.pk, b.idx)
    torch.cuda.synchronize()
    got = b.idx.cpu().numpy()
    assert got.shape == idx_ref.shape
    bad = np.nonzero(np.any(got != idx_ref, axis=-1))
    assert bad[0].size == 0, f"{bad[0].size} rows differ; first row {bad[1][0]}: gpu {got[bad[0][0], bad[1][0]]} " \
                             f"oracle {idx_ref[bad[0][0], bad[1][0]]}"
