"""GPU parity of every hot-path step against the fp64 oracle, through the C ABI.

Stage-wise: pyramid vs oracle pyramid; selection vs oracle selection under the selection-parity rule
(rows compared where the parent matched and the K-th / (K+1)-th oracle scores differ by > 1e-3
relative; ties toward the lower block index); forward, transpose and backward fed the *oracle's*
selection so that they are compared element by element (fp32: 1e-4 max abs; bf16: per slice
2e-2 x max |ref|; integer outputs bit-exact).  End-to-end: the GPU's own chain, outputs compared on
query blocks whose whole selection chain matched.  Shapes span several tiles and ragged tails.
"""
import math

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


# (name, workload, levels, enrich_levels)
CASES = [
    ("tiny_f32_n4096", inputs.WORKLOADS["tiny_fwd_f32_n4096"], 2, -1),
    ("bf16_n4096_h2", inputs.custom(1, 2, 4096, 64, "bf16", seed=11, topk=8, levels=2, backward=True), 2, -1),
    ("bf16_ragged_n592_L1_K3", inputs.custom(1, 3, 592, 64, "bf16", seed=12, topk=3, levels=1, backward=True), 1, -1),
    ("f32_ragged_n592_L1_K3", inputs.custom(1, 3, 592, 64, "f32", seed=13, topk=3, levels=1), 1, -1),
    ("bf16_ragged_n5120_K5_b2", inputs.custom(2, 1, 5120, 64, "bf16", seed=14, topk=5, levels=2, backward=True), 2, -1),
    ("bf16_n4096_Le0", inputs.custom(1, 2, 4096, 64, "bf16", seed=15, topk=8, levels=2, backward=True), 2, 0),
    ("bf16_n4096_Le1", inputs.custom(1, 2, 4096, 64, "bf16", seed=16, topk=8, levels=2, backward=True), 2, 1),
    ("bf16_n4096_fullK16", inputs.custom(1, 1, 4096, 64, "bf16", seed=17, topk=16, levels=2, backward=True), 2, -1),
    ("f32_n4096_K7_Le1", inputs.custom(1, 2, 4096, 64, "f32", seed=18, topk=7, levels=2), 2, 1),
    ("bf16_field_n65536_L3_h1", inputs.custom(1, 1, 65536, 64, "bf16", seed=19, kind="field", topk=8, levels=3,
                                              backward=True), 3, -1),
    # the largest coarsest level (n_L = 512 candidates per unit), the largest K, the deepest pyramid (L = 4)
    ("bf16_n8192_L1_nL512", inputs.custom(1, 1, 8192, 64, "bf16", seed=23, topk=8, levels=1, backward=True), 1, -1),
    ("bf16_n65536_L2_K32", inputs.custom(1, 1, 65536, 64, "bf16", seed=24, topk=32, levels=2, backward=True), 2, -1),
    ("bf16_n1048576_L4", inputs.custom(1, 1, 1 << 20, 64, "bf16", seed=25, topk=8, levels=4, backward=True), 4, -1),
    # the bf16 forward's pair kernel at its edges: K = 2 with no enrichment gives pairs whose union is a single stage;
    # K * L_e = 66 > 64 runs the one-block-per-wave forward (forward only: K (L_e - 1) > 32 is past the backward)
    ("bf16_n4096_K2_Le0", inputs.custom(1, 2, 4096, 64, "bf16", seed=26, topk=2, levels=2, backward=True), 2, 0),
    ("bf16_n98304_K22_L3_fwd", inputs.custom(1, 1, 98304, 64, "bf16", seed=27, topk=22, levels=3), 3, -1),
    # hub inputs: a few key blocks kept by every query block, so the dK/dV kernel splits their groups
    ("bf16_hub_n4096_split", inputs.custom(1, 2, 4096, 64, "bf16", seed=21, kind="hub", topk=8, levels=2,
                                           backward=True), 2, -1),
    ("bf16_hub_n4096_K5_Le1", inputs.custom(1, 1, 4096, 64, "bf16", seed=22, kind="hub", topk=5, levels=2,
                                            backward=True), 2, 1),
]
_cache = {}


def _prepare(name, w, levels, Le):
    if name in _cache:
        return _cache[name]
    x = inputs.make_inputs(w)
    ex = {k_: flat(t.exact) for k_, t in x.items()}
    Le_ref = levels if Le == -1 else Le
    ref = oracle.run(ex["q"], ex["k"], ex["v"], w.block, w.topk, levels=levels, enrich_levels=Le_ref,
                     dout=ex.get("dout"))
    _cache[name] = (x, ex, ref)
    return _cache[name]


def _prob(L, w, levels, Le, grid_w=None):
    """The problem of a case, with the workload's token grid as the scheduling hint when it has one (as bench.py
    runs it: on 2-D fields the bf16 forward then pairs fine blocks one grid row apart)."""
    gw = w.grid[1] if grid_w is None else grid_w
    return L.problem(w.batch, w.heads, w.n, w.d, w.block, w.topk, levels, Le, L.BF16 if w.dtype == "bf16" else L.F32,
                     grid_w=gw)


@pytest.mark.parametrize("name,w,levels,Le", CASES, ids=[c[0] for c in CASES])
def test_pyramid(L, name, w, levels, Le):
    x, ex, ref = _prepare(name, w, levels, Le)
    b = L.Buffers(_prob(L, w, levels, Le), backward=False)
    b.pyramid(dev(x["q"]), dev(x["k"]), dev(x["v"]))
    torch.cuda.synchronize()
    for nm, got in (("pq", b.pq), ("pk", b.pk), ("pv", b.pv)):
        err = np.abs(host(got) - ref[nm]).max()
        assert err <= 1e-5 * max(1.0, np.abs(ref[nm]).max()), (nm, err)
    if w.dtype == "bf16":
        # the bf16 copies are the oracle's means to within one bf16 rounding (8-bit significand: relative 2^-8)
        # plus the fp32 error
        for nm, got in (("pk", b.pkb), ("pv", b.pvb)):
            r = ref[nm].reshape(got.shape)
            err = np.abs(got.float().cpu().numpy() - r) - (2.0 ** -8 * np.abs(r) + 1e-6 * max(1.0, np.abs(r).max()))
            assert err.max() <= 0, (nm, err.max())


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_pyramid_many_slices(L, dtype):
    """384 slices of N = 4096 (L = 2): 384 x 16 chunks x 3 tensors = 18432 pooling workgroups, several rounds of
    them on the device; every slice's whole pyramid against the oracle's."""
    w = inputs.custom(2, 192, 4096, 64, dtype, seed=31, topk=8, levels=2)
    x = inputs.make_inputs(w)
    b = L.Buffers(_prob(L, w, 2, -1), backward=False)
    b.pyramid(dev(x["q"]), dev(x["k"]), dev(x["v"]))
    torch.cuda.synchronize()
    for nm, got in (("pq", b.pq), ("pk", b.pk), ("pv", b.pv)):
        ref = oracle.pool(flat(x["q" if nm == "pq" else "k" if nm == "pk" else "v"].exact), w.block, 2)
        err = np.abs(host(got) - ref).max()
        assert err <= 1e-5 * max(1.0, np.abs(ref).max()), (nm, err)
    if dtype == "bf16":
        for nm, got, src in (("pk", b.pkb, "k"), ("pv", b.pvb, "v")):
            r = oracle.pool(flat(x[src].exact), w.block, 2).reshape(got.shape)
            err = np.abs(got.float().cpu().numpy() - r) - (2.0 ** -8 * np.abs(r) + 1e-6 * max(1.0, np.abs(r).max()))
            assert err.max() <= 0, (nm, err.max())


@pytest.mark.parametrize("name,w,levels,Le", CASES, ids=[c[0] for c in CASES])
def test_select(L, name, w, levels, Le):
    x, ex, ref = _prepare(name, w, levels, Le)
    b = L.Buffers(_prob(L, w, levels, Le), backward=False)
    b.pyramid(dev(x["q"]), dev(x["k"]), dev(x["v"]))
    L.select(b.prob, b.pq, b.pk, b.idx)
    torch.cuda.synchronize()
    idx = b.idx.cpu().numpy()
    compared, total = selection_parity(idx, ref["idx"], ref["pq"], ref["pk"], w.n, w.block, levels, w.topk)
    print(f"{name}: selection rows compared {compared}/{total}")
    assert compared >= 0.9 * total
    # structure of every GPU row: distinct, ascending, in range
    for l in range(1, levels + 1):
        nl, off = w.n // w.block ** l, oracle.level_offset(w.n, w.block, l)
        rows = idx[:, off:off + nl]
        assert np.all(np.diff(rows, axis=2) > 0) and rows.min() >= 0 and rows.max() < nl


@pytest.mark.parametrize("name,w,levels,Le", CASES, ids=[c[0] for c in CASES])
def test_forward_with_oracle_selection(L, name, w, levels, Le):
    x, ex, ref = _prepare(name, w, levels, Le)
    b = L.Buffers(_prob(L, w, levels, Le), backward=False)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    b.pyramid(q, k, v)
    idx = torch.from_numpy(ref["idx"]).cuda()
    L.attn_fwd(b.prob, q, k, v, b.pka, b.pva, idx, b.o, b.lse)
    torch.cuda.synchronize()
    worst = check_close("O", flat(host(b.o)), ref["o"], w.dtype)
    lse_err = np.abs(host(b.lse) - ref["lse"]).max()
    assert lse_err <= (1e-4 if w.dtype == "f32" else 2e-2), lse_err
    print(f"{name}: O worst {worst:.2e}, lse max err {lse_err:.2e}")


# A row length for a synthetic grid hint: 64 tokens (four key blocks per grid row) when it tiles n into an even number
# of rows, so that the bf16 forward pairs every fine block with the one four blocks later (vertical pairs).
def _vertical_hint(n):
    return 64 if n % 64 == 0 and (n // 64) % 2 == 0 else 0


@pytest.mark.parametrize("name,w,levels,Le", [c for c in CASES if c[1].dtype == "bf16" and _vertical_hint(c[1].n)],
                         ids=[c[0] for c in CASES if c[1].dtype == "bf16" and _vertical_hint(c[1].n)])
def test_forward_vertical_pairs_with_oracle_selection(L, name, w, levels, Le):
    """The bf16 forward with fine blocks paired four blocks apart (a grid hint of 64 tokens per row, whatever the
    inputs' own layout): each wave walks the union of two blocks' entry lists, so every case of the table -- odd K,
    L_e = 0 and 1, K = 16 and 32, L = 4, hub selections -- runs with shared, one-sided and padding slots."""
    x, ex, ref = _prepare(name, w, levels, Le)
    b = L.Buffers(_prob(L, w, levels, Le, grid_w=_vertical_hint(w.n)), backward=False)
    assert L.resolve(b.prob).grid_w == _vertical_hint(w.n)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    b.pyramid(q, k, v)
    idx = torch.from_numpy(ref["idx"]).cuda()
    L.attn_fwd(b.prob, q, k, v, b.pka, b.pva, idx, b.o, b.lse)
    torch.cuda.synchronize()
    worst = check_close("O", flat(host(b.o)), ref["o"], w.dtype)
    lse_err = np.abs(host(b.lse) - ref["lse"]).max()
    assert lse_err <= 2e-2, lse_err
    print(f"{name} (vertical pairs): O worst {worst:.2e}, lse max err {lse_err:.2e}")


def _backward_cases():
    return [c for c in CASES if c[1].backward]


@pytest.mark.parametrize("name,w,levels,Le", _backward_cases(), ids=[c[0] for c in _backward_cases()])
def test_transpose_bit_exact(L, name, w, levels, Le):
    x, ex, ref = _prepare(name, w, levels, Le)
    b = L.Buffers(_prob(L, w, levels, Le))
    idx = torch.from_numpy(ref["idx"]).cuda()
    L.index_transpose(b.prob, idx, b.col_ptr, b.perm, b.ws_t)
    torch.cuda.synchronize()
    assert np.array_equal(b.col_ptr.cpu().numpy(), ref["col_ptr"])
    assert np.array_equal(b.perm.cpu().numpy(), ref["perm"])


def test_transpose_partitioned_counts(L):
    """n_1 = 16384 (N = 262144, K = 16, L = 3): the column counts come from per-part LDS histograms summed per
    column (one counter too many for the one-workgroup LDS count); the oracle's own selection of two slices, CSC
    bit for bit."""
    w = inputs.custom(1, 2, 262144, 64, "bf16", seed=29, topk=16, levels=3)
    x = inputs.make_inputs(w)
    ex = {nm: flat(t.exact) for nm, t in x.items()}
    pq, pk = oracle.pool(ex["q"], 16, 3), oracle.pool(ex["k"], 16, 3)
    idx, _ = oracle.select(pq, pk, w.n, 16, 3, 16)
    cp_ref, pm_ref = oracle.index_transpose(idx, w.n, 16, 3, 16, 3)
    b = L.Buffers(L.problem(1, 2, w.n, topk=16, levels=3))
    L.index_transpose(b.prob, torch.from_numpy(idx.astype(np.int32)).cuda(), b.col_ptr, b.perm, b.ws_t)
    torch.cuda.synchronize()
    assert np.array_equal(b.col_ptr.cpu().numpy(), cp_ref)
    assert np.array_equal(b.perm.cpu().numpy(), pm_ref)


@pytest.mark.parametrize("n,K,levels,Le", [(4096, 8, 2, 2), (65536, 8, 3, 3), (4096, 5, 2, 1), (262144, 16, 3, 3)])
def test_transpose_non_hierarchical(L, n, K, levels, Le):
    """Rows that are not children of their parent's picks (random ascending rows at every level): the
    hierarchical fill misses entries, raises its flag and the general path must give the oracle's CSC."""
    rng = np.random.default_rng(7 + n + K)
    bh = 2
    R = oracle.pyramid_rows(n, 16, levels)
    idx = np.empty((bh, R, K), dtype=np.int32)
    for l in range(1, levels + 1):
        nl, off = n // 16 ** l, oracle.level_offset(n, 16, l)
        for b in range(bh):
            for u in range(nl):
                idx[b, off + u] = np.sort(rng.choice(nl, size=K, replace=False))
    cp_ref, pm_ref = oracle.index_transpose(idx, n, 16, levels, K, Le)
    b = L.Buffers(L.problem(1, bh, n, topk=K, levels=levels, enrich_levels=Le))
    L.index_transpose(b.prob, torch.from_numpy(idx).cuda(), b.col_ptr, b.perm, b.ws_t)
    torch.cuda.synchronize()
    assert np.array_equal(b.col_ptr.cpu().numpy(), cp_ref)
    assert np.array_equal(b.perm.cpu().numpy(), pm_ref)


@pytest.mark.parametrize("name,w,levels,Le", _backward_cases(), ids=[c[0] for c in _backward_cases()])
def test_backward_with_oracle_selection(L, name, w, levels, Le):
    x, ex, ref = _prepare(name, w, levels, Le)
    b = L.Buffers(_prob(L, w, levels, Le))
    q, k, v, do = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["dout"])
    b.pyramid(q, k, v)
    b.idx.copy_(torch.from_numpy(ref["idx"]))
    L.attn_fwd(b.prob, q, k, v, b.pka, b.pva, b.idx, b.o, b.lse)
    b.backward(q, k, v, do)
    torch.cuda.synchronize()
    msg = []
    for nm, got in (("dq", b.dq), ("dk", b.dk), ("dv", b.dv)):
        worst = check_close(nm, flat(host(got)), ref[nm], w.dtype)
        msg.append(f"{nm} {worst:.2e}")
    print(f"{name}: " + ", ".join(msg))


@pytest.mark.parametrize("name,w,levels,Le", CASES, ids=[c[0] for c in CASES])
def test_end_to_end_chain(L, name, w, levels, Le):
    """The GPU's own selection feeds the forward; O is compared on every fine query block whose
    selection rows (at all levels) equal the oracle's."""
    x, ex, ref = _prepare(name, w, levels, Le)
    b = L.Buffers(_prob(L, w, levels, Le), backward=False)
    b.forward(dev(x["q"]), dev(x["k"]), dev(x["v"]))
    torch.cuda.synchronize()
    idx = b.idx.cpu().numpy()
    n1 = w.n // w.block
    clean = np.ones((w.bh, n1), bool)
    for l in range(1, levels + 1):
        off, nl = oracle.level_offset(w.n, w.block, l), w.n // w.block ** l
        same = np.all(idx[:, off:off + nl] == ref["idx"][:, off:off + nl], axis=2)
        clean &= same[:, np.arange(n1) // w.block ** (l - 1)]
    assert clean.mean() >= 0.9
    o = flat(host(b.o)).reshape(w.bh, n1, w.block, w.d)
    r = ref["o"].reshape(w.bh, n1, w.block, w.d)
    tol = 1e-4 if w.dtype == "f32" else 2e-2
    for s in range(w.bh):
        err = np.abs(o[s][clean[s]] - r[s][clean[s]]).max()
        lim = tol if w.dtype == "f32" else tol * np.abs(r[s]).max()
        assert err <= lim, (s, err, lim)


@pytest.mark.parametrize("name,w,levels,Le", _backward_cases()[:3], ids=[c[0] for c in _backward_cases()[:3]])
def test_deterministic(L, name, w, levels, Le):
    """Two runs of the whole chain are bitwise identical (no floating-point atomics anywhere)."""
    x, ex, ref = _prepare(name, w, levels, Le)
    q, k, v, do = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["dout"])
    outs = []
    for _ in range(2):
        b = L.Buffers(_prob(L, w, levels, Le))
        b.forward(q, k, v)
        b.backward(q, k, v, do)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (b.idx, b.o, b.lse, b.col_ptr, b.perm, b.dq, b.dk, b.dv)])
    for a, c in zip(*outs):
        assert torch.equal(a, c)


def test_split_groups_deterministic(L):
    """Hub inputs: the oracle's level-1 columns put more than 4x the mean group length (4 K stages) into one
    group of 4 key blocks, so its stages run as several chunks whose partial sums dkdv_combine adds; two runs
    give identical bits."""
    name, w, levels, Le = next(c for c in CASES if c[0] == "bf16_hub_n4096_split")
    x, ex, ref = _prepare(name, w, levels, Le)
    n1 = w.n // w.block
    cp1 = ref["col_ptr"][:, :n1 + 1]
    groups = cp1[:, np.minimum(np.arange(0, n1, 4) + 4, n1)] - cp1[:, np.arange(0, n1, 4)]
    assert groups.max() > 4 * 4 * w.topk, groups.max()
    q, k, v, do = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["dout"])
    outs = []
    for _ in range(2):
        b = L.Buffers(_prob(L, w, levels, Le))
        b.pyramid(q, k, v)
        b.idx.copy_(torch.from_numpy(ref["idx"]))
        L.attn_fwd(b.prob, q, k, v, b.pka, b.pva, b.idx, b.o, b.lse)
        b.backward(q, k, v, do)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (b.dq, b.dk, b.dv)])
    for a, c in zip(*outs):
        assert torch.equal(a.view(torch.int16), c.view(torch.int16))


@pytest.mark.parametrize("kind,grid,levels", [("hub", (32, 128), 2), ("field", (18, 256), 2), ("field", (256, 256), 3)],
                         ids=["hub_n4096_split_groups", "field_n4608_partial_band", "field_n65536"])
def test_grid_hint_keeps_selection_and_backward_bits(L, kind, grid, levels):
    """grid_w changes no selection, and the backward from the same forward outputs gives the same bits with and
    without it (it only reorders the dK/dV work list: groups of four consecutive grid rows next to each other) --
    on hub inputs whose long groups run as chunks, with a last band of only two grid rows, and on a three-level
    field.  The forward pairs fine blocks one grid row apart with the hint and side by side without it: the same
    sums in another order, so O and LSE agree to the bf16 tolerance and each meets the oracle (n <= 4608 here)."""
    H, W = grid
    n = H * W
    w = inputs.custom(1, 2, n, 64, "bf16", seed=37, kind=kind, grid=grid, topk=8, levels=levels, backward=True)
    x = inputs.make_inputs(w, with_dout=True)
    q, k, v, do = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["dout"])
    bufs = []
    for gw in (0, W):
        p = L.problem(1, 2, n, topk=8, levels=levels, grid_w=gw)
        assert L.resolve(p).grid_w == gw
        b = L.Buffers(p)
        b.forward(q, k, v)
        torch.cuda.synchronize()
        bufs.append(b)
    b0, b1 = bufs
    assert torch.equal(b0.idx, b1.idx)
    check_close("O", host(b1.o).reshape(2, -1), host(b0.o).reshape(2, -1), "bf16")
    assert np.abs(host(b1.lse) - host(b0.lse)).max() <= 2e-2
    if n <= 4608:
        ex = {nm: flat(x[nm].exact) for nm in ("q", "k", "v")}
        ref = oracle.run(ex["q"], ex["k"], ex["v"], 16, 8, levels=levels)
        if np.array_equal(host(b0.idx).astype(np.int64), ref["idx"].astype(np.int64)):
            for b in bufs:
                check_close("O", flat(host(b.o)), ref["o"], "bf16")
                assert np.abs(host(b.lse) - ref["lse"]).max() <= 2e-2
    # the backward from the same O and LSE
    b1.o.copy_(b0.o)
    b1.lse.copy_(b0.lse)
    outs = []
    for b in bufs:
        b.backward(q, k, v, do)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (b.dq, b.dk, b.dv)])
    for nm, a, c in zip(("dq", "dk", "dv"), *outs):
        assert torch.equal(a, c), nm


def test_tie_rule_on_gpu(L):
    """Every pooled key equal: all scores tie exactly, every unit keeps the lowest block indices."""
    n, K = 4096, 8
    w = inputs.custom(1, 1, n, 64, "bf16", seed=20, topk=K, levels=2)
    x = inputs.make_inputs(w)
    kconst = np.broadcast_to(x["k"].store[:, :, :1, :], x["k"].store.shape).copy()
    b = L.Buffers(L.problem(1, 1, n, topk=K, levels=2), backward=False)
    kt = torch.from_numpy(kconst.view(np.int16)).cuda().view(torch.bfloat16)
    b.forward(dev(x["q"]), kt, dev(x["v"]))
    torch.cuda.synchronize()
    idx = b.idx.cpu().numpy()[0]
    assert np.all(idx[256:272] == np.arange(K))     # level 2: blocks 0..7
    assert np.all(idx[:256] == np.arange(K))         # level 1: children 0..7 of block 0


def test_empty_batch(L):
    p = L.problem(0, 2, 4096)
    e = torch.empty(0, device="cuda")
    L.build_pyramid(p, e, e, e, e, e, e)
    L.attn_fwd(p, e, e, e, e, e, e.int(), e, e)
