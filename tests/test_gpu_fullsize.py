"""GPU parity at the full workload sizes (the benchmark one in the launch configuration bench.py times), on
sampled slices.

The whole chain runs on every (batch, head) slice of the N = 65536 forward+backward workload (16 heads, K = 8,
L = 3) and of the N = 262144 one (8 heads, K = 16, L = 3 -- the backward's two-tile path for the level >= 2
partials).  The fp64 oracle runs on a few sampled slices only:
  * selection of the sampled slices under the selection-parity rule (see test_gpu_parity);
  * then the sampled slices' selection rows are replaced by the oracle's (the others keep the GPU's) and the
    forward, transpose and backward run again on all slices, so that O, LSE, dQ, dK, dV of the sampled slices
    compare element by element with the oracle (bf16: per slice max abs <= 2e-2 x max |ref|), col_ptr and
    perm bit-exactly;
  * every slice's outputs are finite.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import check_close, host, selection_parity
from hierarchical_sparse_attention_mean_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from hierarchical_sparse_attention_mean_amd import llsa
    return llsa


def _dev(t):
    return torch.from_numpy(t.store.view(np.int16)).cuda().view(torch.bfloat16)


def _run_sampled(L, w, samples):
    x = inputs.make_inputs(w, with_dout=True)
    q, k, v, do = (_dev(x[nm]) for nm in ("q", "k", "v", "dout"))
    # in the launch configuration bench.py times: the token grid as the scheduling hint
    b = L.Buffers(L.problem(w.batch, w.heads, w.n, w.d, w.block, w.topk, w.levels, grid_w=w.grid[1]))
    b.forward(q, k, v)
    b.backward(q, k, v, do)
    torch.cuda.synchronize()
    for t in (b.o, b.lse, b.dq, b.dk, b.dv):
        assert torch.isfinite(t.float()).all()
    idx = b.idx.clone()
    for s in samples:
        ex = {nm: x[nm].exact.reshape(w.bh, w.n, w.d)[s:s + 1] for nm in ("q", "k", "v", "dout")}
        ref = oracle.run(ex["q"], ex["k"], ex["v"], w.block, w.topk, levels=w.levels, dout=ex["dout"])
        # the pyramid at this size's launch shape (levels 1 and 2 in one launch, then level 3, at N = 262144):
        # fp32 means of bf16 inputs, so within fp32 rounding of the oracle's
        for nm, got in (("pq", b.pq), ("pk", b.pk), ("pv", b.pv)):
            g = host(got).reshape(w.bh, -1)[s]
            err = np.abs(g - ref[nm].reshape(-1)).max()
            assert err <= 1e-5 * max(1.0, np.abs(ref[nm]).max()), (nm, s, err)
        compared, total = selection_parity(idx[s:s + 1].cpu().numpy(), ref["idx"], ref["pq"], ref["pk"], w.n,
                                           w.block, w.levels, w.topk)
        print(f"{w.name} slice {s}: selection rows compared {compared}/{total}")
        assert compared >= 0.9 * total
        # the oracle's selection for this slice, everything after it on the GPU again (all slices)
        idx2 = idx.clone()
        idx2[s] = torch.from_numpy(ref["idx"][0]).cuda()
        b.idx.copy_(idx2)
        L.attn_fwd(b.prob, q, k, v, b.pka, b.pva, b.idx, b.o, b.lse)
        b.backward(q, k, v, do)
        torch.cuda.synchronize()
        assert np.array_equal(b.col_ptr[s].cpu().numpy(), ref["col_ptr"][0])
        assert np.array_equal(b.perm[s].cpu().numpy(), ref["perm"][0])
        msg = []
        for nm, got in (("O", b.o), ("dq", b.dq), ("dk", b.dk), ("dv", b.dv)):
            g = host(got).reshape(w.bh, w.n, w.d)[s:s + 1]
            worst = check_close(nm, g.reshape(1, -1), ref[nm.lower()].reshape(1, -1), w.dtype)
            msg.append(f"{nm} {worst:.2e}")
        lse_err = np.abs(host(b.lse).reshape(w.bh, w.n)[s] - ref["lse"][0]).max()
        assert lse_err <= 2e-2, lse_err
        print(f"{w.name} slice {s}: " + ", ".join(msg) + f", lse {lse_err:.2e}")


def test_fullsize_n65536_16_heads(L):
    _run_sampled(L, inputs.WORKLOADS["fwdbwd_bf16_n65536"], samples=(0, 11))


def test_fullsize_n262144_K16(L):
    _run_sampled(L, inputs.WORKLOADS["fwdbwd_bf16_n262144"], samples=(5,))


def test_fullsize_fwd_n16384_8_heads(L):
    """The N = 16384 forward workload (8 heads, i.i.d. inputs, K = 8, L = 2): the GPU chain on every slice,
    selection parity on sampled slices, then O and LSE element by element on them with the oracle's selection."""
    w = inputs.WORKLOADS["fwd_bf16_n16384"]
    x = inputs.make_inputs(w)
    q, k, v = (_dev(x[nm]) for nm in ("q", "k", "v"))
    b = L.Buffers(L.problem(w.batch, w.heads, w.n, w.d, w.block, w.topk, w.levels, grid_w=w.grid[1]), backward=False)
    b.forward(q, k, v)
    torch.cuda.synchronize()
    assert torch.isfinite(b.o.float()).all()
    idx = b.idx.clone()
    for s in (2, 7):
        ex = {nm: x[nm].exact.reshape(w.bh, w.n, w.d)[s:s + 1] for nm in ("q", "k", "v")}
        ref = oracle.run(ex["q"], ex["k"], ex["v"], w.block, w.topk, levels=w.levels)
        compared, total = selection_parity(idx[s:s + 1].cpu().numpy(), ref["idx"], ref["pq"], ref["pk"], w.n,
                                           w.block, w.levels, w.topk)
        assert compared >= 0.9 * total
        idx2 = idx.clone()
        idx2[s] = torch.from_numpy(ref["idx"][0]).cuda()
        L.attn_fwd(b.prob, q, k, v, b.pka, b.pva, idx2, b.o, b.lse)
        torch.cuda.synchronize()
        g = host(b.o).reshape(w.bh, w.n, w.d)[s:s + 1]
        worst = check_close("O", g.reshape(1, -1), ref["o"].reshape(1, -1), w.dtype)
        lse_err = np.abs(host(b.lse).reshape(w.bh, w.n)[s] - ref["lse"][0]).max()
        assert lse_err <= 2e-2, lse_err
        print(f"{w.name} slice {s}: selection rows compared {compared}/{total}, O {worst:.2e}, lse {lse_err:.2e}")


def test_two_stream_chain_matches_one_stream(L):
    """The chain as bench.py times it -- the index transpose on a second stream, beside the forward
    (Buffers.forward_backward) -- gives bit for bit what the one-stream chain gives, over back-to-back steps on
    alternating inputs with no synchronisation between them (each step's outputs are copied on the main stream
    before the next step starts), so that a step that overtook its predecessor's reads would show."""
    import dataclasses
    w = inputs.WORKLOADS["fwdbwd_bf16_n65536"]
    sets = []
    for seed in (w.seed, w.seed + 1):
        x = inputs.make_inputs(dataclasses.replace(w, seed=seed), with_dout=True)
        sets.append([_dev(x[nm]) for nm in ("q", "k", "v", "dout")])
    b = L.Buffers(L.problem(w.batch, w.heads, w.n, w.d, w.block, w.topk, w.levels, grid_w=w.grid[1]))
    outs = lambda: [t.clone() for t in (b.idx, b.o, b.lse, b.dq, b.dk, b.dv)]
    ref = []
    for q, k, v, do in sets:
        b.forward(q, k, v)
        b.backward(q, k, v, do)
        ref.append(outs())
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    got = []
    for s in (0, 1, 0, 1):
        b.forward_backward(*sets[s], stream, side)
        got.append((s, outs()))
    torch.cuda.synchronize()
    for s, g in got:
        for nm, a, r in zip(("idx", "O", "lse", "dq", "dk", "dv"), g, ref[s]):
            assert torch.equal(a, r), (s, nm)


def test_two_stream_chain_replays_as_graph(L):
    """The two-stream chain captured once as a HIP graph (its fork and join are device-scope event waits, and
    no call in it issues a memset) replays bit for bit what the eager one-stream chain gives: four replays on
    alternating inputs copied into the captured input buffers, with an eager step on the other inputs and a
    synchronisation between replays."""
    import dataclasses
    w = inputs.WORKLOADS["fwdbwd_bf16_n65536"]
    sets = []
    for seed in (w.seed, w.seed + 1):
        x = inputs.make_inputs(dataclasses.replace(w, seed=seed), with_dout=True)
        sets.append([_dev(x[nm]) for nm in ("q", "k", "v", "dout")])
    b = L.Buffers(L.problem(w.batch, w.heads, w.n, w.d, w.block, w.topk, w.levels, grid_w=w.grid[1]))
    outs = lambda: [t.clone() for t in (b.idx, b.o, b.lse, b.dq, b.dk, b.dv)]
    ref = []
    for q, k, v, do in sets:
        b.forward(q, k, v)
        b.backward(q, k, v, do)
        ref.append(outs())
    static = [t.clone() for t in sets[0]]
    main, side = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(main):
        b.forward_backward(*static, main, side)          # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=main):
        b.forward_backward(*static, main, side)
    torch.cuda.synchronize()
    for s in (0, 1, 0, 1):
        for dst, src in zip(static, sets[s]):
            dst.copy_(src)
        for t in (b.o, b.dq, b.dk, b.dv):
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for nm, a, r in zip(("idx", "O", "lse", "dq", "dk", "dv"), outs(), ref[s]):
            assert torch.equal(a, r), (s, nm)
        with torch.cuda.stream(main):
            b.forward_backward(*sets[1 - s], main, side)  # eager work between replays
        torch.cuda.synchronize()
        for nm, a, r in zip(("idx", "O", "lse", "dq", "dk", "dv"), outs(), ref[1 - s]):
            assert torch.equal(a, r), (s, "eager", nm)
