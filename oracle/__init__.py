"""fp64 CPU oracle of Log-linear Sparse Attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import
this package.  It loads ``oracle/liboracle.so`` (plain C99 + OpenMP, built from ``llsa_oracle.c`` with
gcc) through ctypes.  It shares no code with the HIP library.

Arrays are numpy float64 (int32 for indices), laid out ``[bh, rows, d]`` with ``bh = batch * heads``.
Every function follows one step of the method as the LLSA review page (pith.science review of arXiv
2512.16615) relays it; the C source cites the section for each step.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "llsa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_i64 = ctypes.c_int64
_i32 = ctypes.c_int
_dbl = ctypes.c_double
_pd = ctypes.POINTER(ctypes.c_double)
_pi = ctypes.POINTER(ctypes.c_int32)


def build(verbose: bool = False) -> str:
    """Compile liboracle.so with gcc (-O2, OpenMP, fp64).  Returns the library path."""
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-o", _LIB_PATH, _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.llsa_ref_default_levels.restype = _i32
    lib.llsa_ref_default_levels.argtypes = [_i64, _i32]
    lib.llsa_ref_pyramid_rows.restype = _i64
    lib.llsa_ref_pyramid_rows.argtypes = [_i64, _i32, _i32]
    lib.llsa_ref_pool.restype = None
    lib.llsa_ref_pool.argtypes = [_i64, _i64, _i32, _i32, _i32, _pd, _pd]
    lib.llsa_ref_select.restype = _i64
    lib.llsa_ref_select.argtypes = [_i64, _i64, _i32, _i32, _i32, _i32, _pd, _pd, _pi]
    lib.llsa_ref_attn_fwd.restype = None
    lib.llsa_ref_attn_fwd.argtypes = [_i64, _i64, _i32, _i32, _i32, _i32, _i32, _dbl,
                                      _pd, _pd, _pd, _pd, _pd, _pi, _pd, _pd]
    lib.llsa_ref_attn_fwd_complement.restype = None
    lib.llsa_ref_attn_fwd_complement.argtypes = lib.llsa_ref_attn_fwd.argtypes
    lib.llsa_ref_entry_weight.restype = _i32
    lib.llsa_ref_entry_weight.argtypes = [_i64, _i32, _i32, _i32, _i32, _pi, _i64, _i32, ctypes.POINTER(ctypes.c_double)]
    lib.llsa_ref_index_transpose.restype = None
    lib.llsa_ref_index_transpose.argtypes = [_i64, _i64, _i32, _i32, _i32, _i32, _pi, _pi, _pi]
    lib.llsa_ref_attn_bwd.restype = None
    lib.llsa_ref_attn_bwd.argtypes = [_i64, _i64, _i32, _i32, _i32, _i32, _i32, _dbl,
                                      _pd, _pd, _pd, _pd, _pd, _pd, _pd, _pd, _pi,
                                      _pd, _pd, _pd, _pd, _pd]
    lib.llsa_ref_attn_bwd_complement.restype = None
    lib.llsa_ref_attn_bwd_complement.argtypes = lib.llsa_ref_attn_bwd.argtypes
    lib.llsa_ref_reorder_index.restype = _i32
    lib.llsa_ref_reorder_index.argtypes = [_i64, _i64, _i32, _i32, ctypes.POINTER(ctypes.c_int64)]
    lib.llsa_ref_reorder.restype = None
    lib.llsa_ref_reorder.argtypes = [_i64, _i64, _i32, ctypes.POINTER(ctypes.c_int64), _i32, _pd, _pd]
    lib.llsa_ref_num_threads.restype = _i32
    lib.llsa_ref_num_threads.argtypes = []
    _lib = lib
    return lib


def _finite(name: str, *arrays):
    """Non-finite inputs are outside the method's definition: the oracle refuses them instead of returning
    whatever the arithmetic makes of them."""
    for a in arrays:
        if a is not None and not np.all(np.isfinite(a)):
            raise ValueError(f"oracle.{name}: input holds a non-finite value")


def _d(a: np.ndarray):
    assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"], (a.dtype, a.flags)
    return a.ctypes.data_as(_pd)


def _i(a: np.ndarray):
    assert a.dtype == np.int32 and a.flags["C_CONTIGUOUS"], (a.dtype, a.flags)
    return a.ctypes.data_as(_pi)


def num_threads() -> int:
    return int(_load().llsa_ref_num_threads())


def default_levels(n: int, block: int) -> int:
    """L = floor(log_B n - 1), computed with integers."""
    return int(_load().llsa_ref_default_levels(n, block))


def pyramid_rows(n: int, block: int, levels: int) -> int:
    return int(_load().llsa_ref_pyramid_rows(n, block, levels))


def level_rows(n: int, block: int, level: int) -> int:
    return n // block ** level


def level_offset(n: int, block: int, level: int) -> int:
    return sum(n // block ** j for j in range(1, level))


def pool(x: np.ndarray, block: int, levels: int) -> np.ndarray:
    """Mean-pooled pyramid of x [bh, n, d] -> [bh, R, d]."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    _finite("pool", x)
    bh, n, d = x.shape
    out = np.empty((bh, pyramid_rows(n, block, levels), d), np.float64)
    _load().llsa_ref_pool(bh, n, d, block, levels, _d(x), _d(out))
    return out


def select(pq: np.ndarray, pk: np.ndarray, n: int, block: int, levels: int, topk: int):
    """Hierarchical Top-K.  Returns (idx [bh, R, K] int32, scored_pairs)."""
    pq = np.ascontiguousarray(pq, dtype=np.float64)
    pk = np.ascontiguousarray(pk, dtype=np.float64)
    _finite("select", pq, pk)
    bh, R, d = pq.shape
    idx = np.empty((bh, R, topk), np.int32)
    pairs = _load().llsa_ref_select(bh, n, d, block, levels, topk, _d(pq), _d(pk), _i(idx))
    return idx, int(pairs)


def attn_fwd(q, k, v, pk, pv, idx, block, levels, topk, enrich_levels, scale, complement: bool = False):
    """Enriched sparse attention forward.  Returns (o [bh, n, d], lse [bh, n]).  complement=True takes the
    complement-partition reading of the enrichment (the unkept candidates of every level)."""
    q, k, v, pk, pv = (np.ascontiguousarray(a, dtype=np.float64) for a in (q, k, v, pk, pv))
    _finite("attn_fwd", q, k, v, pk, pv)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    bh, n, d = q.shape
    o = np.empty_like(q)
    lse = np.empty((bh, n), np.float64)
    fn = _load().llsa_ref_attn_fwd_complement if complement else _load().llsa_ref_attn_fwd
    fn(bh, n, d, block, levels, topk, enrich_levels, scale,
       _d(q), _d(k), _d(v), _d(pk), _d(pv), _i(idx), _d(o), _d(lse))
    return o, lse


def entry_weight(idx_slice, n, block, levels, topk, enrich_levels, query, complement):
    """(number of entries, sum of their weights B^level) of one query of one slice's selection."""
    idx_slice = np.ascontiguousarray(idx_slice, dtype=np.int32)
    w = ctypes.c_double()
    ne = _load().llsa_ref_entry_weight(n, block, levels, topk, enrich_levels, _i(idx_slice), query,
                                       int(bool(complement)), ctypes.byref(w))
    return int(ne), w.value


def transposed_levels(levels: int, enrich_levels: int) -> int:
    return max(1, min(enrich_levels, levels))


def colptr_len(n: int, block: int, levels: int, enrich_levels: int) -> int:
    return sum(level_rows(n, block, l) + 1 for l in range(1, transposed_levels(levels, enrich_levels) + 1))


def perm_len(n: int, block: int, levels: int, enrich_levels: int, topk: int) -> int:
    return sum(level_rows(n, block, l) * topk for l in range(1, transposed_levels(levels, enrich_levels) + 1))


def index_transpose(idx, n, block, levels, topk, enrich_levels):
    """CSR -> CSC of levels 1..max(1, Le).  Returns (col_ptr [bh, C], perm [bh, P])."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    bh = idx.shape[0]
    cp = np.empty((bh, colptr_len(n, block, levels, enrich_levels)), np.int32)
    pm = np.empty((bh, perm_len(n, block, levels, enrich_levels, topk)), np.int32)
    _load().llsa_ref_index_transpose(bh, n, block, levels, topk, enrich_levels, _i(idx), _i(cp), _i(pm))
    return cp, pm


def attn_bwd(q, k, v, o, lse, dout, pk, pv, idx, block, levels, topk, enrich_levels, scale,
             want_pooled: bool = False, complement: bool = False):
    """Backward.  Returns (dq, dk, dv) or (dq, dk, dv, dpk, dpv) with pooled-token gradients.
    complement=True takes the complement-partition reading of the enrichment."""
    q, k, v, o, dout, pk, pv = (np.ascontiguousarray(a, dtype=np.float64) for a in (q, k, v, o, dout, pk, pv))
    lse = np.ascontiguousarray(lse, dtype=np.float64)
    _finite("attn_bwd", q, k, v, o, lse, dout, pk, pv)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    bh, n, d = q.shape
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    if want_pooled:
        dpk, dpv = np.empty_like(pk), np.empty_like(pv)
        pdpk, pdpv = _d(dpk), _d(dpv)
    else:
        dpk = dpv = None
        pdpk = pdpv = ctypes.cast(None, _pd)
    fn = _load().llsa_ref_attn_bwd_complement if complement else _load().llsa_ref_attn_bwd
    fn(bh, n, d, block, levels, topk, enrich_levels, scale,
       _d(q), _d(k), _d(v), _d(o), _d(lse), _d(dout), _d(pk), _d(pv), _i(idx),
       _d(dq), _d(dk), _d(dv), pdpk, pdpv)
    if want_pooled:
        return dq, dk, dv, dpk, dpv
    return dq, dk, dv


def run(q, k, v, block, topk, levels=None, enrich_levels=None, scale=None, dout=None):
    """The whole chain pool -> select -> forward (-> transpose -> backward when dout is given).

    q, k, v (and dout): float64 [bh, n, d].  Returns a dict of every intermediate.
    """
    _finite("run", q, k, v, dout)
    bh, n, d = q.shape
    L = default_levels(n, block) if not levels else levels
    Le = L if enrich_levels is None or enrich_levels < 0 else enrich_levels
    sigma = 1.0 / math.sqrt(d) if not scale else scale
    pq, pk, pv = pool(q, block, L), pool(k, block, L), pool(v, block, L)
    idx, pairs = select(pq, pk, n, block, L, topk)
    o, lse = attn_fwd(q, k, v, pk, pv, idx, block, L, topk, Le, sigma)
    out = dict(levels=L, enrich_levels=Le, scale=sigma, pq=pq, pk=pk, pv=pv, idx=idx, pairs=pairs,
               o=o, lse=lse)
    if dout is not None:
        cp, pm = index_transpose(idx, n, block, L, topk, Le)
        dq, dk, dv, dpk, dpv = attn_bwd(q, k, v, o, lse, dout, pk, pv, idx, block, L, topk, Le, sigma,
                                        want_pooled=True)
        out.update(col_ptr=cp, perm=pm, dq=dq, dk=dk, dv=dv, dpk=dpk, dpv=dpv)
    return out


def reorder_index(H: int, W: int, block: int, levels: int) -> np.ndarray:
    """local_of[t]: position in the 2-D-local order of row-major pixel t (recursive sqrt(B) x sqrt(B) tiles)."""
    out = np.empty(H * W, np.int64)
    rc = _load().llsa_ref_reorder_index(H, W, block, levels, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
    if rc != 0:
        raise ValueError("block must be a square and sqrt(block)^levels must divide the grid")
    return out


def reorder(x: np.ndarray, local_of: np.ndarray, to_local: bool) -> np.ndarray:
    """Rows of x [bh, n, d] moved to the 2-D-local order (to_local) or back to row-major."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    bh, n, d = x.shape
    lo = np.ascontiguousarray(local_of, dtype=np.int64)
    y = np.empty_like(x)
    _load().llsa_ref_reorder(bh, n, d, lo.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), int(to_local), _d(x),
                             _d(y))
    return y
