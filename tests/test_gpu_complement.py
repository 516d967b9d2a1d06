"""GPU parity of the complement-partition forward and backward (llsa_attn_fwd_complement,
llsa_attn_bwd_complement) with the oracle's complement reading, both fed the oracle's selection: O, LSE, dQ, dK,
dV element by element (bf16: per slice max abs <= 2e-2 x max |ref|, LSE 2e-2), at sizes that span several tiles
with ragged tails, L = 1, L_e < L, K = 16 (empty level-2 lists), hub inputs (split dK/dV groups), and at the
N = 65536 benchmark size on sampled slices.  A negative control checks that the two readings of the enrichment
differ on these inputs by far more than the tolerance, so the comparison can tell them apart.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import check_close, dev, flat, host, selection_parity
from hierarchical_sparse_attention_mean_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from hierarchical_sparse_attention_mean_amd import llsa
    return llsa


# (name, workload, levels, enrich_levels); entries per fine block in the comment
CASES = [
    ("n4096_h2_K8", inputs.custom(1, 2, 4096, 64, "bf16", seed=31, topk=8, levels=2), 2, -1),       # 120 + 8
    ("ragged_n592_L1_K3", inputs.custom(1, 3, 592, 64, "bf16", seed=32, topk=3, levels=1), 1, -1),  # 34
    ("ragged_n5120_K5_b2", inputs.custom(2, 1, 5120, 64, "bf16", seed=33, topk=5, levels=2), 2, -1),  # 75 + 15
    ("n4096_Le1", inputs.custom(1, 2, 4096, 64, "bf16", seed=34, topk=8, levels=2), 2, 1),          # 120
    ("n4096_Le0", inputs.custom(1, 1, 4096, 64, "bf16", seed=35, topk=8, levels=2), 2, 0),          # 0
    ("n4096_K16", inputs.custom(1, 1, 4096, 64, "bf16", seed=36, topk=16, levels=2), 2, -1),        # 240 + 0
    ("field_n65536_L3", inputs.custom(1, 1, 65536, 64, "bf16", seed=37, kind="field", topk=8, levels=3),
     3, -1),                                                                                            # 248
    ("n65536_L2_K4", inputs.custom(1, 1, 65536, 64, "bf16", seed=38, topk=4, levels=2), 2, -1),      # 60 + 252
]


def _ws(L, prob):
    return torch.empty(max(1, L.workspace_bytes(prob, L.OP_ATTN_FWD_COMPLEMENT)), dtype=torch.uint8,
                       device="cuda")


@pytest.mark.parametrize("name,w,levels,Le", CASES, ids=[c[0] for c in CASES])
def test_complement_forward_with_oracle_selection(L, name, w, levels, Le):
    x = inputs.make_inputs(w)
    ex = {k_: flat(t.exact) for k_, t in x.items()}
    Le_ref = levels if Le == -1 else Le
    ref = oracle.run(ex["q"], ex["k"], ex["v"], w.block, w.topk, levels=levels, enrich_levels=Le_ref)
    o_ref, lse_ref = oracle.attn_fwd(ex["q"], ex["k"], ex["v"], ref["pk"], ref["pv"], ref["idx"], w.block, levels,
                                     w.topk, Le_ref, ref["scale"], complement=True)
    prob = L.problem(w.batch, w.heads, w.n, w.d, w.block, w.topk, levels, Le, L.BF16)
    b = L.Buffers(prob, backward=False)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    b.pyramid(q, k, v)
    idx = torch.from_numpy(ref["idx"]).cuda()
    ws = _ws(L, b.prob)
    L.attn_fwd_complement(b.prob, q, k, v, b.pka, b.pva, idx, b.o, b.lse, ws)
    torch.cuda.synchronize()
    worst = check_close("O", flat(host(b.o)), o_ref, "bf16")
    lse_err = np.abs(host(b.lse) - lse_ref).max()
    assert lse_err <= 2e-2, lse_err
    # a second call (the lists rewritten in the same workspace) gives the same bits
    o1 = b.o.clone()
    L.attn_fwd_complement(b.prob, q, k, v, b.pka, b.pva, idx, b.o, b.lse, ws)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), b.o.view(torch.int16))
    # negative control: where the enrichment is not empty the selected-token reading is far from this one
    if Le_ref > 0:
        sep = np.abs(ref["o"] - o_ref).max() / np.abs(o_ref).max()
        assert sep > 5 * 2e-2, sep
    print(f"{name}: O worst {worst:.2e}, lse max err {lse_err:.2e}")


@pytest.mark.parametrize("wname,samples", [("fwd_bf16_n65536", (3,)), ("fwdbwd_bf16_n262144", (6,))])
def test_complement_fullsize_sampled(L, wname, samples):
    """N = 65536, 16 heads, K = 8, L = 3 (248 entries per fine block) and N = 262144, 8 heads, K = 16, L = 3
    (528): the GPU's own selection on every slice, the oracle's on the sampled slices, which then compare
    element by element."""
    w = inputs.WORKLOADS[wname]
    x = inputs.make_inputs(w)
    q, k, v = (dev(x[nm]) for nm in ("q", "k", "v"))
    b = L.Buffers(L.problem(w.batch, w.heads, w.n, w.d, w.block, w.topk, w.levels), backward=False)
    b.pyramid(q, k, v)
    L.select(b.prob, b.pq, b.pk, b.idx)
    ws = _ws(L, b.prob)
    torch.cuda.synchronize()
    for s in samples:
        ex = {nm: x[nm].exact.reshape(w.bh, w.n, w.d)[s:s + 1] for nm in ("q", "k", "v")}
        ref = oracle.run(ex["q"], ex["k"], ex["v"], w.block, w.topk, levels=w.levels)
        compared, total = selection_parity(b.idx[s:s + 1].cpu().numpy(), ref["idx"], ref["pq"], ref["pk"], w.n,
                                           w.block, w.levels, w.topk)
        assert compared >= 0.9 * total
        o_ref, lse_ref = oracle.attn_fwd(ex["q"], ex["k"], ex["v"], ref["pk"], ref["pv"], ref["idx"], w.block,
                                         w.levels, w.topk, w.levels, ref["scale"], complement=True)
        b.idx[s] = torch.from_numpy(ref["idx"][0]).cuda()
        L.attn_fwd_complement(b.prob, q, k, v, b.pka, b.pva, b.idx, b.o, b.lse, ws)
        torch.cuda.synchronize()
        assert torch.isfinite(b.o.float()).all() and torch.isfinite(b.lse).all()
        g = host(b.o).reshape(w.bh, w.n, w.d)[s:s + 1]
        worst = check_close("O", g.reshape(1, -1), o_ref.reshape(1, -1), "bf16")
        lse_err = np.abs(host(b.lse).reshape(w.bh, w.n)[s] - lse_ref[0]).max()
        assert lse_err <= 2e-2, lse_err
        print(f"{w.name} slice {s}: complement O worst {worst:.2e}, lse {lse_err:.2e}")


def test_complement_empty_batch(L):
    p = L.problem(0, 4, 4096)
    L.attn_fwd_complement(p, None, None, None, None, None, None, None, None, None)


BWD_CASES = [
    ("n4096_h2_K8", inputs.custom(1, 2, 4096, 64, "bf16", seed=41, topk=8, levels=2, backward=True), 2, -1),
    ("ragged_n592_L1_K3", inputs.custom(1, 3, 592, 64, "bf16", seed=42, topk=3, levels=1, backward=True), 1, -1),
    ("ragged_n5120_K5_b2", inputs.custom(2, 1, 5120, 64, "bf16", seed=43, topk=5, levels=2, backward=True), 2, -1),
    ("n4096_Le1", inputs.custom(1, 2, 4096, 64, "bf16", seed=44, topk=8, levels=2, backward=True), 2, 1),
    ("n4096_Le0", inputs.custom(1, 1, 4096, 64, "bf16", seed=45, topk=8, levels=2, backward=True), 2, 0),
    ("n4096_K16", inputs.custom(1, 1, 4096, 64, "bf16", seed=46, topk=16, levels=2, backward=True), 2, -1),
    ("hub_n4096_split", inputs.custom(1, 2, 4096, 64, "bf16", seed=47, kind="hub", topk=8, levels=2,
                                      backward=True), 2, -1),
    ("field_n65536_L3", inputs.custom(1, 1, 65536, 64, "bf16", seed=48, kind="field", topk=8, levels=3,
                                      backward=True), 3, -1),
    ("n65536_L3_Le2", inputs.custom(1, 1, 65536, 64, "bf16", seed=49, topk=4, levels=3, backward=True), 3, 2),
    # 504 entries per fine block: all but K of the 512 coarsest blocks
    ("n8192_L1_nL512", inputs.custom(1, 2, 8192, 64, "bf16", seed=50, topk=8, levels=1, backward=True), 1, -1),
]


def _bwd_run(L, prob, x, idx_np, b=None):
    b = b or L.Buffers(prob, backward=False)
    q, k, v, do = (dev(x[nm]) for nm in ("q", "k", "v", "dout"))
    b.pyramid(q, k, v)
    idx = torch.from_numpy(idx_np).cuda()
    L.attn_fwd_complement(b.prob, q, k, v, b.pka, b.pva, idx, b.o, b.lse, _ws(L, b.prob))
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    wsb = torch.empty(max(1, L.workspace_bytes(b.prob, L.OP_ATTN_BWD_COMPLEMENT)), dtype=torch.uint8, device="cuda")
    L.attn_bwd_complement(b.prob, q, k, v, b.o, b.lse, do, b.pka, b.pva, idx, dq, dk, dv, wsb)
    torch.cuda.synchronize()
    return dq, dk, dv


@pytest.mark.parametrize("name,w,levels,Le", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_complement_backward_with_oracle_selection(L, name, w, levels, Le):
    x = inputs.make_inputs(w, with_dout=True)
    ex = {k_: flat(t.exact) for k_, t in x.items()}
    Le_ref = levels if Le == -1 else Le
    ref = oracle.run(ex["q"], ex["k"], ex["v"], w.block, w.topk, levels=levels, enrich_levels=Le_ref)
    o_ref, lse_ref = oracle.attn_fwd(ex["q"], ex["k"], ex["v"], ref["pk"], ref["pv"], ref["idx"], w.block, levels,
                                     w.topk, Le_ref, ref["scale"], complement=True)
    grads = oracle.attn_bwd(ex["q"], ex["k"], ex["v"], o_ref, lse_ref, ex["dout"], ref["pk"], ref["pv"], ref["idx"],
                            w.block, levels, w.topk, Le_ref, ref["scale"], complement=True)
    prob = L.problem(w.batch, w.heads, w.n, w.d, w.block, w.topk, levels, Le, L.BF16)
    got = _bwd_run(L, prob, x, ref["idx"])
    msg = []
    for nm, g_, r_ in zip(("dq", "dk", "dv"), got, grads):
        worst = check_close(nm, flat(host(g_)), r_, "bf16")
        msg.append(f"{nm} {worst:.2e}")
    # a second run gives the same bits (fixed-order sums only)
    again = _bwd_run(L, prob, x, ref["idx"])
    for a_, b_ in zip(got, again):
        assert torch.equal(a_.view(torch.int16), b_.view(torch.int16))
    if Le_ref > 0:  # negative control: the selected-token reading's gradients are far from these
        sel = oracle.attn_bwd(ex["q"], ex["k"], ex["v"], ref["o"], ref["lse"], ex["dout"], ref["pk"], ref["pv"],
                              ref["idx"], w.block, levels, w.topk, Le_ref, ref["scale"])
        sep = max(np.abs(a_ - b_).max() / np.abs(b_).max() for a_, b_ in zip(sel, grads))
        assert sep > 5 * 2e-2, sep
    print(f"{name}: " + ", ".join(msg))


def test_complement_backward_fullsize_sampled(L):
    """N = 65536, 16 heads, K = 8, L = 3: the GPU's own selection on every slice, the oracle's on a sampled
    slice, whose dQ, dK, dV then compare element by element."""
    w = inputs.WORKLOADS["fwdbwd_bf16_n65536"]
    x = inputs.make_inputs(w, with_dout=True)
    q = dev(x["q"])
    b = L.Buffers(L.problem(w.batch, w.heads, w.n, w.d, w.block, w.topk, w.levels), backward=False)
    b.pyramid(q, dev(x["k"]), dev(x["v"]))
    L.select(b.prob, b.pq, b.pk, b.idx)
    torch.cuda.synchronize()
    s = 9
    ex = {nm: x[nm].exact.reshape(w.bh, w.n, w.d)[s:s + 1] for nm in ("q", "k", "v", "dout")}
    ref = oracle.run(ex["q"], ex["k"], ex["v"], w.block, w.topk, levels=w.levels)
    idx = b.idx.cpu().numpy()
    idx[s] = ref["idx"][0]
    o_ref, lse_ref = oracle.attn_fwd(ex["q"], ex["k"], ex["v"], ref["pk"], ref["pv"], ref["idx"], w.block, w.levels,
                                     w.topk, w.levels, ref["scale"], complement=True)
    grads = oracle.attn_bwd(ex["q"], ex["k"], ex["v"], o_ref, lse_ref, ex["dout"], ref["pk"], ref["pv"], ref["idx"],
                            w.block, w.levels, w.topk, w.levels, ref["scale"], complement=True)
    got = _bwd_run(L, b.prob, x, idx, b)
    msg = []
    for nm, g_, r_ in zip(("dq", "dk", "dv"), got, grads):
        assert torch.isfinite(g_.float()).all()
        gs = host(g_).reshape(w.bh, w.n, w.d)[s:s + 1]
        worst = check_close(nm, gs.reshape(1, -1), r_.reshape(1, -1), "bf16")
        msg.append(f"{nm} {worst:.2e}")
    print(f"{w.name} slice {s}: complement " + ", ".join(msg))


def test_complement_grid_hint_changes_no_output(L):
    """The complement reading with and without the grid hint (grid_w): the forward's sweep order and the dK/dV
    work-list order change, the outputs keep their bits (field inputs on a 64 x 256 grid, two heads)."""
    H, W = 64, 256
    w = inputs.custom(1, 2, H * W, 64, "bf16", seed=41, kind="field", grid=(H, W), topk=8, levels=2, backward=True)
    x = inputs.make_inputs(w, with_dout=True)
    q, k, v, do = (dev(x[nm]) for nm in ("q", "k", "v", "dout"))
    outs = []
    for gw in (0, W):
        b = L.Buffers(L.problem(1, 2, H * W, topk=8, levels=2, grid_w=gw))
        assert b.prob.grid_w == gw
        b.pyramid(q, k, v)
        L.select(b.prob, b.pq, b.pk, b.idx)
        wf = torch.empty(max(1, L.workspace_bytes(b.prob, L.OP_ATTN_FWD_COMPLEMENT)), dtype=torch.uint8, device="cuda")
        wb = torch.empty(max(1, L.workspace_bytes(b.prob, L.OP_ATTN_BWD_COMPLEMENT)), dtype=torch.uint8, device="cuda")
        L.attn_fwd_complement(b.prob, q, k, v, b.pka, b.pva, b.idx, b.o, b.lse, wf)
        L.attn_bwd_complement(b.prob, q, k, v, b.o, b.lse, do, b.pka, b.pva, b.idx, b.dq, b.dk, b.dv, wb)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (b.idx, b.o, b.lse, b.dq, b.dk, b.dv)])
    for nm, a, c in zip(("idx", "o", "lse", "dq", "dk", "dv"), *outs):
        assert torch.equal(a, c), nm
