"""llsa_index_transpose_noalloc (workspace in the library's static device scratch) against
llsa_index_transpose (caller workspace): identical col_ptr and perm, bit for bit, over calls in a row on
one GPU, each later call on a smaller problem than the one before (the scratch keeps the previous call's
contents).  The problems take the code paths of the transpose: counters in global memory (n_1 + 1 > 16384),
counters in LDS, and the scatter/order path (L_e < L)."""
import sys

import pytest
import torch

from hierarchical_sparse_attention_mean_amd import inputs, llsa

pytestmark = pytest.mark.gpu

# (batch, heads, n, topk, levels, enrich_levels), largest transpose workspace first
CASES = [
    (1, 1, 1 << 20, 8, 4, -1),   # global counters + hierarchical fill
    (1, 2, 262144, 16, 3, -1),   # global counters, K = 16
    (1, 4, 65536, 8, 3, 1),      # LDS counters, then scatter + order (T = 1 < L)
    (1, 2, 4096, 8, 2, -1),      # LDS counters + hierarchical fill, small
]


def _selection(prob, seed):
    """A selection made by the library's own pyramid and hierarchical Top-K on seeded N(0, 1) inputs."""
    w = inputs.custom(prob.batch, prob.heads, prob.n, 64, "bf16", seed=seed, topk=prob.topk, levels=prob.levels)
    x = inputs.make_inputs(w)
    q, k, v = (torch.from_numpy(x[nm].store.view("int16")).cuda().view(torch.bfloat16) for nm in ("q", "k", "v"))
    b = llsa.Buffers(prob, device="cuda", backward=False)
    b.pyramid(q, k, v)
    llsa.select(prob, b.pq, b.pk, b.idx)
    return b.idx


def test_noalloc_transpose_matches_workspace_transpose():
    assert torch.cuda.is_available()
    for seed, (batch, heads, n, topk, levels, le) in enumerate(CASES):
        prob = llsa.resolve(llsa.problem(batch, heads, n, topk=topk, levels=levels, enrich_levels=le))
        need = llsa.workspace_bytes(prob, llsa.OP_INDEX_TRANSPOSE)
        assert 0 < need <= llsa.NOALLOC_SCRATCH_BYTES
        print(f"no-alloc transpose: bh={batch * heads} n={n} K={topk} L={levels} Le={prob.enrich_levels} "
              f"workspace {need} B", flush=True)
        sys.stdout.flush()
        idx = _selection(prob, 100 + seed)
        bh = batch * heads
        cpl, pml = llsa.colptr_len(prob), llsa.perm_len(prob)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        cp_ref = torch.full((bh, cpl), -7, dtype=torch.int32, device="cuda")
        pm_ref = torch.full((bh, pml), -7, dtype=torch.int32, device="cuda")
        llsa.index_transpose(prob, idx, cp_ref, pm_ref, ws)
        cp, pm = torch.full_like(cp_ref, -9), torch.full_like(pm_ref, -9)
        llsa.index_transpose_noalloc(prob, idx, cp, pm)
        torch.cuda.synchronize()
        assert torch.equal(cp, cp_ref), f"col_ptr differs (n={n})"
        assert torch.equal(pm, pm_ref), f"perm differs (n={n})"
        # the CSC is complete: every column entry was written and the last col_ptr of each level is n_l K
        assert int(pm.min()) >= 0
        del ws, cp_ref, pm_ref, cp, pm, idx
