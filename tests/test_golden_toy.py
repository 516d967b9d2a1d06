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
