"""GPU parity of the 2-D-local index reordering (llsa_reorder): a permutation of rows, so bit-exact against
the oracle's reordering, in both directions, for bf16 and fp32, square and rectangular grids, and the round
trip restores the input."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import dev, flat
from hierarchical_sparse_attention_mean_amd import inputs

pytestmark = pytest.mark.gpu

CASES = [
    ("bf16_256x256_L3", 256, 256, 3, "bf16", 2),
    ("f32_64x64_L2", 64, 64, 2, "f32", 3),
    ("bf16_512x512_L3", 512, 512, 3, "bf16", 1),
    ("bf16_48x32_L1", 48, 32, 1, "bf16", 2),
    ("f32_64x256_L2", 64, 256, 2, "f32", 1),
]


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from hierarchical_sparse_attention_mean_amd import llsa
    return llsa


@pytest.mark.parametrize("name,H,W,levels,dtype,heads", CASES, ids=[c[0] for c in CASES])
def test_reorder_bit_exact(L, name, H, W, levels, dtype, heads):
    n = H * W
    w = inputs.custom(1, heads, n, 64, dtype, seed=51, levels=levels)
    x = inputs.make_inputs(w)
    p = L.problem(1, heads, n, 64, 16, 1, levels, -1, L.BF16 if dtype == "bf16" else L.F32)
    src = dev(x["q"])
    y = torch.empty_like(src)
    back = torch.empty_like(src)
    L.reorder(p, H, W, True, src, y)
    L.reorder(p, H, W, False, y, back)
    torch.cuda.synchronize()
    lo = oracle.reorder_index(H, W, 16, levels)
    ref = oracle.reorder(flat(x["q"].exact), lo, True)
    got = flat(y.float().cpu().numpy().astype(np.float64))
    assert np.array_equal(got, ref)
    assert torch.equal(back, src)
