"""Oracle vs the hand-worked Figure 1-shaped toy (tests/golden/fig1_toy.txt): every pooled value,
selected index, scored-pair count, entry set, output, log-sum-exp and CSC entry was derived by hand."""
import math
import os

import numpy as np

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _fixture():
    vals, entries = {}, {}
    for line in open(os.path.join(HERE, "golden", "fig1_toy.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        key, *rest = line.split()
        if key == "entry":
            entries[int(rest[0])] = [tuple(float(t) for t in e.split(":")) for e in rest[1:]]
        else:
            vals[key] = [float(t) for t in rest]
    return vals, entries


def test_fig1_toy():
    f, entries = _fixture()
    n, B, K, L, D = (int(f[k][0]) for k in ("n", "B", "K", "L", "D"))
    q, k, v = (np.array(f[name]).reshape(1, n, D) for name in ("q", "k", "v"))
    assert oracle.default_levels(n, B) == L
    r = oracle.run(q, k, v, B, K, dout=np.ones((1, n, D)))
    assert r["scale"] == 1.0
    for name in ("q", "k", "v"):
        np.testing.assert_array_equal(r["p" + name].reshape(-1), np.array(f["pool_" + name]))
    assert list(r["idx"].reshape(-1)) == [int(x) for x in f["idx"]]
    assert r["pairs"] == int(f["pairs"][0])
    for qi, ent in entries.items():
        w = np.array([e[1] for e in ent]); z = np.array([e[0] for e in ent]); vv = np.array([e[2] for e in ent])
        o = (w * np.exp(z) * vv).sum() / (w * np.exp(z)).sum()
        assert abs(r["o"][0, qi, 0] - o) < 1e-13
        assert abs(r["lse"][0, qi] - math.log((w * np.exp(z)).sum())) < 1e-13
    assert abs(r["o"][0, 7, 0] - f["o7"][0]) < 1e-15
    assert abs(r["lse"][0, 7] - math.log(8.0)) < 1e-15
    assert list(r["col_ptr"].reshape(-1)) == [int(x) for x in f["col_ptr"]]
    assert list(r["perm"].reshape(-1)) == [int(x) for x in f["perm"]]


def _fixture2():
    vals, exprs = {}, []
    for line in open(os.path.join(HERE, "golden", "ancestor_toy.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        key, *rest = line.split()
        if key == "expr":
            exprs.append((rest[0], int(rest[1]), " ".join(rest[2:])))
        else:
            vals[key] = [float(t) for t in rest]
    return vals, exprs


def _closed_form(expr: str) -> float:
    """A hand-derived closed form in e and E = e^2 (the fixture's notation), evaluated in double precision."""
    return float(eval(expr, {"__builtins__": {}}, {"e": math.e, "E": math.e ** 2, "log": math.log}))


def test_ancestor_toy_forward_and_backward():
    """Oracle vs the hand-worked toy in which the level-2 units keep different blocks (tests/golden/
    ancestor_toy.txt): pyramid, selection, scored pairs, CSC, O, LSE, dQ, dK, dV and the pooled-token gradients
    against values and closed forms derived by hand.  Pins the fine-block -> level-l ancestor map i / B^(l-1) and
    the backward's B^-l distribution of pooled-token gradients."""
    f, exprs = _fixture2()
    n, B, K, L, D = (int(f[k][0]) for k in ("n", "B", "K", "L", "D"))
    q, k, v = (np.array(f[name]).reshape(1, n, D) for name in ("q", "k", "v"))
    r = oracle.run(q, k, v, B, K, levels=L, dout=np.ones((1, n, D)))
    assert r["scale"] == 1.0
    for name in ("q", "k", "v"):
        np.testing.assert_array_equal(r["p" + name].reshape(-1), np.array(f["pool_" + name]))
    assert list(r["idx"].reshape(-1)) == [int(x) for x in f["idx"]]
    assert r["pairs"] == int(f["pairs"][0])
    assert list(r["col_ptr"].reshape(-1)) == [int(x) for x in f["col_ptr"]]
    assert list(r["perm"].reshape(-1)) == [int(x) for x in f["perm"]]
    n1 = n // B
    got = {"o": r["o"][0, :, 0], "lse": r["lse"][0], "dq": r["dq"][0, :, 0], "dk": r["dk"][0, :, 0],
           "dv": r["dv"][0, :, 0], "dpk1": r["dpk"][0, :n1, 0], "dpk2": r["dpk"][0, n1:, 0],
           "dpv2": r["dpv"][0, n1:, 0]}
    assert len(exprs) > 60
    for name, i, expr in exprs:
        want = _closed_form(expr)
        assert abs(got[name][i] - want) <= 1e-12 * max(1.0, abs(want)), (name, i, got[name][i], want, expr)
    # the invariants the derivation was checked against
    assert abs(r["dk"].sum()) < 1e-12
    assert abs(r["dv"].sum() - n) < 1e-12


def test_ancestor_toy_negative_control():
    """A mistake planted in a copy of the inputs must break the pins: with query 8's q flipped, unit 2's level-2
    pick moves and the entry sets of fine blocks 4 and 5 change, so their outputs leave the hand values."""
    f, exprs = _fixture2()
    n, B, K, L, D = (int(f[k][0]) for k in ("n", "B", "K", "L", "D"))
    q, k, v = (np.array(f[name]).reshape(1, n, D) for name in ("q", "k", "v"))
    q = q.copy()
    q[0, 8:10, 0] = 1.0      # level-2 unit 2 now pools to +1 and keeps block 0
    r = oracle.run(q, k, v, B, K, levels=L, dout=np.ones((1, n, D)))
    assert int(r["idx"][0, n // B + 2, 0]) == 0
    want = _closed_form("1/(2*e+2)")
    assert abs(r["o"][0, 8, 0] - want) > 1e-3
