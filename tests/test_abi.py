"""CPU-only checks of the C ABI: the library loads, exports every entry point declared in
include/llsa.h, and its host-side validation returns the documented status codes before any GPU call
(no compute is issued here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    from hierarchical_sparse_attention_mean_amd import llsa
    return llsa


def _declared():
    src = open(os.path.join(ROOT, "include", "llsa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(llsa_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert {"llsa_build_pyramid", "llsa_select", "llsa_attn_fwd", "llsa_index_transpose", "llsa_attn_bwd",
            "llsa_select_exhaustive", "llsa_reorder", "llsa_attn_fwd_complement",
            "llsa_attn_bwd_complement"} <= set(names)
    for n in names:
        assert hasattr(L.lib(), n), n


def test_resolve_defaults(L):
    r = L.resolve(L.problem(1, 16, 65536))
    assert (r.levels, r.enrich_levels, r.topk) == (3, 3, 8)
    assert abs(r.scale - 0.125) < 1e-9
    assert L.pyramid_rows(r) == 4096 + 256 + 16
    assert L.colptr_len(r) == (4096 + 1) + (256 + 1) + (16 + 1)
    assert L.perm_len(r) == (4096 + 256 + 16) * 8
    r = L.resolve(L.problem(1, 2, 4096, dtype=L.F32))
    assert (r.levels, r.enrich_levels) == (2, 2)
    r = L.resolve(L.problem(1, 8, 262144, topk=16))
    assert r.levels == 3 and L.pyramid_rows(r) == 16384 + 1024 + 64


def test_grid_hint_kept_only_where_it_applies(L):
    """grid_w (a dK/dV scheduling hint) survives resolution only when a grid row holds whole groups of four key
    blocks (a multiple of 4B = 64 tokens) and the rows tile n; otherwise it resolves to 0 (no grid)."""
    assert L.resolve(L.problem(1, 2, 65536, grid_w=256)).grid_w == 256
    assert L.resolve(L.problem(1, 2, 65536, grid_w=0)).grid_w == 0
    assert L.resolve(L.problem(1, 2, 65536, grid_w=96)).grid_w == 0      # not a multiple of 64
    assert L.resolve(L.problem(1, 2, 4608, grid_w=256, levels=2)).grid_w == 256   # 18 rows
    assert L.resolve(L.problem(1, 2, 4096, grid_w=192)).grid_w == 0      # 192 does not divide 4096


@pytest.mark.parametrize("kw,code", [
    (dict(n=4096 + 16), "ERR_SHAPE"),          # n mod B^L != 0 at the default L = 2
    (dict(n=4096, levels=3), "ERR_SHAPE"),     # L above floor(log_B n - 1)
    (dict(n=200), "ERR_SHAPE"),                # n < B^2: no pooled level
    (dict(n=4096, topk=17), "ERR_SHAPE"),      # K > n_L = 16
    (dict(n=4096, topk=0), "ERR_SHAPE"),
    (dict(n=4096, enrich_levels=3), "ERR_SHAPE"),
    (dict(n=4096, enrich_levels=-2), "ERR_SHAPE"),
    (dict(n=4096, d=32), "ERR_UNSUPPORTED"),
    (dict(n=4096, block=8), "ERR_UNSUPPORTED"),
    (dict(n=1 << 20, levels=1, topk=8), "ERR_UNSUPPORTED"),  # n_L = 65536 > 512
    (dict(n=4096, dtype=7), "ERR_DTYPE"),
    (dict(n=4096, scale=float("inf")), "ERR_PARAM"),
    (dict(n=4096, grid_w=-64), "ERR_SHAPE"),
])
def test_validation_codes(L, kw, code):
    base = dict(batch=1, heads=2)
    base.update(kw)
    p = L.problem(**base)
    assert L.lib().llsa_resolve(ctypes.byref(p), None) == getattr(L, code)
    # the entry points return the same status and launch nothing
    assert L.lib().llsa_build_pyramid(ctypes.byref(p), None, None, None, None, None, None, None, None,
                                      None) == getattr(L, code)
    assert L.workspace_bytes(p, L.OP_ATTN_BWD) == 0


def test_null_and_alignment_checked_before_the_device(L):
    p = L.problem(1, 2, 4096)
    f = L.lib()
    assert f.llsa_attn_fwd(ctypes.byref(p), None, None, None, None, None, None, None, None, None) == L.ERR_NULL
    assert f.llsa_build_pyramid(ctypes.byref(p), 16, 32, 48, 64, 80, 88, 96, 112, None) == L.ERR_ALIGN
    # bf16 problems need the bf16 copies of the pooled K, V pyramids
    assert f.llsa_build_pyramid(ctypes.byref(p), 16, 32, 48, 64, 80, 96, None, 112, None) == L.ERR_NULL
    assert f.llsa_build_pyramid(ctypes.byref(p), 16, 32, 48, 64, 80, 96, 112, 8, None) == L.ERR_ALIGN
    assert f.llsa_select(None, 16, 16, 16, None) == L.ERR_NULL


def test_workspace_checked_before_the_device(L):
    p = L.problem(1, 2, 4096)
    need = L.workspace_bytes(p, L.OP_INDEX_TRANSPOSE)
    assert need > 0
    f = L.lib()
    assert f.llsa_index_transpose(ctypes.byref(p), 16, 32, 48, 64, need - 1, None) == L.ERR_WORKSPACE
    assert f.llsa_index_transpose(ctypes.byref(p), 16, 32, 48, None, need, None) == L.ERR_WORKSPACE
    nb = L.workspace_bytes(p, L.OP_ATTN_BWD)
    args = [16] * 14
    assert f.llsa_attn_bwd(ctypes.byref(p), *args, 64, nb - 1, None) == L.ERR_WORKSPACE
    pf = L.problem(1, 2, 4096, dtype=L.F32)
    assert f.llsa_attn_bwd(ctypes.byref(pf), *args, 64, nb, None) == L.ERR_DTYPE


def test_complement_forward_host_checks(L):
    f = L.lib()
    p = L.problem(1, 2, 65536)  # K = 8, L = 3: 120 + 120 + 8 = 248 entries per fine block
    need = L.workspace_bytes(p, L.OP_ATTN_FWD_COMPLEMENT)
    ints = 4096 * 120 + 256 * 120 + 16 * 8
    assert need == -(-2 * ints * 4 // 256) * 256
    args = [16] * 8
    assert f.llsa_attn_fwd_complement(ctypes.byref(p), *args, 64, need - 1, None) == L.ERR_WORKSPACE
    assert f.llsa_attn_fwd_complement(ctypes.byref(p), *args, None, need, None) == L.ERR_WORKSPACE
    assert f.llsa_attn_fwd_complement(ctypes.byref(p), *([None] * 8), 64, need, None) == L.ERR_NULL
    pf = L.problem(1, 2, 65536, dtype=L.F32)
    assert f.llsa_attn_fwd_complement(ctypes.byref(pf), *args, 64, need, None) == L.ERR_DTYPE
    big = L.problem(1, 1, 65536, topk=32, levels=2)  # 480 + 224 = 704 > 576
    assert f.llsa_attn_fwd_complement(ctypes.byref(big), *args, 64, 1 << 30, None) == L.ERR_UNSUPPORTED
    empty = L.problem(0, 4, 65536)
    assert f.llsa_attn_fwd_complement(ctypes.byref(empty), *([None] * 8), None, 0, None) == L.OK
    # backward: 13 pointers, then the workspace
    nb = L.workspace_bytes(p, L.OP_ATTN_BWD_COMPLEMENT)
    assert nb > need
    bargs = [16] * 12
    assert f.llsa_attn_bwd_complement(ctypes.byref(p), *bargs, 64, nb - 1, None) == L.ERR_WORKSPACE
    assert f.llsa_attn_bwd_complement(ctypes.byref(p), *([None] * 12), 64, nb, None) == L.ERR_NULL
    assert f.llsa_attn_bwd_complement(ctypes.byref(pf), *bargs, 64, nb, None) == L.ERR_DTYPE
    assert f.llsa_attn_bwd_complement(ctypes.byref(big), *bargs, 64, 1 << 30, None) == L.ERR_UNSUPPORTED
    assert f.llsa_attn_bwd_complement(ctypes.byref(empty), *([None] * 12), None, 0, None) == L.OK


def test_empty_batch_is_a_no_op(L):
    p = L.problem(0, 4, 4096)
    f = L.lib()
    assert f.llsa_build_pyramid(ctypes.byref(p), None, None, None, None, None, None, None, None, None) == L.OK
    assert f.llsa_attn_fwd(ctypes.byref(p), None, None, None, None, None, None, None, None, None) == L.OK


def test_workspace_is_linear_in_n(L):
    """No dense N x N structure anywhere: workspaces grow linearly with the sequence length."""
    a = L.problem(1, 1, 65536, topk=8)
    b = L.problem(1, 1, 16 * 65536, topk=8, levels=3)
    for op in (L.OP_INDEX_TRANSPOSE, L.OP_ATTN_BWD):
        wa, wb = L.workspace_bytes(a, op), L.workspace_bytes(b, op)
        assert wb <= 16 * wa * 1.01 + 4096, (op, wa, wb)


def test_status_strings(L):
    for s in range(0, -11, -1):
        assert L.status_string(s) != "unknown status"
    assert L.status_string(-99) == "unknown status"


def test_timing_api_without_launches(L):
    L.timing_enable(True)
    rec = L.timing_read()
    assert set(rec) == set(L.KERNELS) and all(v == (0.0, 0) for v in rec.values())
    L.timing_enable(False)
    t, c = ctypes.c_double(), ctypes.c_int64()
    assert L.lib().llsa_timing_read(99, ctypes.byref(t), ctypes.byref(c)) == L.ERR_PARAM
    assert L.lib().llsa_timing_read(0, None, None) == L.ERR_NULL


def test_reorder_validation(L):
    p = L.problem(1, 2, 65536)  # L = 3: the grid sides must be multiples of 4^3 = 64
    f = L.lib()
    assert f.llsa_reorder(ctypes.byref(p), 256, 256, 1, None, None, None) == L.ERR_NULL
    assert f.llsa_reorder(ctypes.byref(p), 256, 128, 1, 16, 32, None) == L.ERR_SHAPE   # 256 * 128 != n
    assert f.llsa_reorder(ctypes.byref(p), 32, 2048, 1, 16, 32, None) == L.ERR_SHAPE   # 64 does not divide 32
    assert f.llsa_reorder(ctypes.byref(p), 256, 256, 1, 16, 16, None) == L.ERR_PARAM   # in place
    assert f.llsa_reorder(ctypes.byref(p), 256, 256, 1, 16, 40, None) == L.ERR_ALIGN


def test_noalloc_transpose_host_checks(L):
    """The no-alloc transpose rejects a problem whose workspace exceeds the static scratch before touching the
    device, and otherwise validates like llsa_index_transpose."""
    f = L.lib()
    fits = L.problem(1, 8, 262144, topk=16)                 # 9.5 MB of workspace
    assert L.workspace_bytes(fits, L.OP_INDEX_TRANSPOSE) <= L.NOALLOC_SCRATCH_BYTES
    big = L.problem(1, 16, 262144, topk=16)                 # 19 MB > 16 MiB
    assert L.workspace_bytes(big, L.OP_INDEX_TRANSPOSE) > L.NOALLOC_SCRATCH_BYTES
    assert f.llsa_index_transpose_noalloc(ctypes.byref(big), 16, 32, 48, None) == L.ERR_SCRATCH
    assert f.llsa_index_transpose_noalloc(ctypes.byref(fits), None, 32, 48, None) == L.ERR_NULL
    assert f.llsa_index_transpose_noalloc(ctypes.byref(fits), 16, 32, 40, None) == L.ERR_ALIGN
    assert f.llsa_index_transpose_noalloc(ctypes.byref(L.problem(1, 2, 4096 + 16)), 16, 32, 48, None) == L.ERR_SHAPE
    assert f.llsa_index_transpose_noalloc(ctypes.byref(L.problem(0, 2, 4096)), None, None, None, None) == L.OK
    assert L.status_string(L.ERR_SCRATCH) != "unknown status"


# The five calls of the contract, parameter types in order (names dropped).  CONTRACT is the problem-level
# statement (fp32 pyramids into the attention calls); AMENDED lists the one documented difference: bf16 problems
# pass the bf16 copies of the pooled K, V pyramids, which llsa_build_pyramid writes as two more outputs.
CONTRACT = {
    "llsa_build_pyramid": ["const llsa_problem*", "const void*", "const void*", "const void*", "float*", "float*",
                           "float*", "hipStream_t"],
    "llsa_select": ["const llsa_problem*", "const float*", "const float*", "int32_t*", "hipStream_t"],
    "llsa_attn_fwd": ["const llsa_problem*", "const void*", "const void*", "const void*", "const float*",
                      "const float*", "const int32_t*", "void*", "float*", "hipStream_t"],
    "llsa_index_transpose": ["const llsa_problem*", "const int32_t*", "int32_t*", "int32_t*", "void*", "size_t",
                             "hipStream_t"],
    "llsa_attn_bwd": ["const llsa_problem*", "const void*", "const void*", "const void*", "const void*",
                      "const float*", "const void*", "const float*", "const float*", "const int32_t*",
                      "const int32_t*", "const int32_t*", "void*", "void*", "void*", "void*", "size_t",
                      "hipStream_t"],
}
AMENDED = {
    "llsa_build_pyramid": lambda t: t[:7] + ["void*", "void*"] + t[7:],
    "llsa_attn_fwd": lambda t: t[:4] + ["const void*", "const void*"] + t[6:],
    "llsa_attn_bwd": lambda t: t[:7] + ["const void*", "const void*"] + t[9:],
}


def _param_types(name):
    src = open(os.path.join(ROOT, "include", "llsa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    m = re.search(r"\bint\s+" + name + r"\s*\((.*?)\)\s*;", src, flags=re.S)
    assert m, name
    out = []
    for p in m.group(1).split(","):
        p = " ".join(p.split())
        out.append(re.sub(r"\s*\b\w+$", "", p).replace(" *", "*"))
    return out


@pytest.mark.parametrize("name", sorted(CONTRACT))
def test_hot_path_signatures(name):
    want = AMENDED.get(name, lambda t: t)(CONTRACT[name])
    assert _param_types(name) == want
