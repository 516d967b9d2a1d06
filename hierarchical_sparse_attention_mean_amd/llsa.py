"""Thin ctypes binding of libllsa.so (the gfx950 HIP library declared in include/llsa.h).

Argument marshalling only: every step runs in the library's kernels.  Tensors are torch tensors on
the GPU (used for device memory); the stream defaults to torch's current stream.  Loading fails
loudly (ImportError) when the library has not been built -- there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libllsa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libllsa.so is not built ({LIB_PATH}); run __graft_entry__.build() or "
                      "python hierarchical_sparse_attention_mean_amd/build.py")

_lib = ctypes.CDLL(LIB_PATH)

F32, BF16 = 0, 1
OK = 0
ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_DTYPE, ERR_ALIGN, ERR_WORKSPACE, ERR_LAUNCH, ERR_PARAM, ERR_DEVICE = \
    -1, -2, -3, -4, -5, -6, -7, -8, -9
ERR_SCRATCH = -10
NOALLOC_SCRATCH_BYTES = 16 << 20   # LLSA_NOALLOC_SCRATCH_BYTES
OP_INDEX_TRANSPOSE, OP_ATTN_BWD, OP_ATTN_FWD_COMPLEMENT, OP_ATTN_BWD_COMPLEMENT = 1, 2, 3, 4
KERNELS = ("pool", "select", "attn_fwd", "transpose", "bwd_dq", "bwd_reduce", "bwd_dkdv",
           "select_exhaustive", "reorder", "complement")  # LLSA_KERNEL_* order


class Problem(ctypes.Structure):
    """Mirror of llsa_problem."""
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("n", ctypes.c_int32),
                ("d", ctypes.c_int32), ("block", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("levels", ctypes.c_int32), ("enrich_levels", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("scale", ctypes.c_float), ("grid_w", ctypes.c_int32)]

    def __repr__(self):
        return ("Problem(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")")


def problem(batch, heads, n, d=64, block=16, topk=8, levels=0, enrich_levels=-1, dtype=BF16, scale=0.0, grid_w=0):
    """grid_w: tokens per row of a row-major 2-D token grid (a scheduling hint; 0 = none)."""
    return Problem(batch, heads, n, d, block, topk, levels, enrich_levels, dtype, scale, grid_w)


class LlsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_P = ctypes.POINTER(Problem)
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t

_lib.llsa_build_pyramid.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.llsa_select.argtypes = [_P, _vp, _vp, _vp, _vp]
_lib.llsa_select_exhaustive.argtypes = [_P, _vp, _vp, _vp, _vp]
_lib.llsa_reorder.argtypes = [_P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _vp, _vp, _vp]
_lib.llsa_attn_fwd.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.llsa_attn_fwd_complement.argtypes = [_P] + [_vp] * 9 + [_sz, _vp]
_lib.llsa_attn_bwd_complement.argtypes = [_P] + [_vp] * 13 + [_sz, _vp]
_lib.llsa_index_transpose.argtypes = [_P, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.llsa_index_transpose_noalloc.argtypes = [_P, _vp, _vp, _vp, _vp]
_lib.llsa_attn_bwd.argtypes = [_P] + [_vp] * 15 + [_sz, _vp]
for _f in ("llsa_build_pyramid", "llsa_select", "llsa_select_exhaustive", "llsa_reorder", "llsa_attn_fwd",
           "llsa_attn_fwd_complement", "llsa_attn_bwd_complement", "llsa_index_transpose", "llsa_index_transpose_noalloc",
           "llsa_attn_bwd"):
    getattr(_lib, _f).restype = ctypes.c_int
_lib.llsa_resolve.argtypes = [_P, _P]
_lib.llsa_resolve.restype = ctypes.c_int
for _f in ("llsa_pyramid_rows", "llsa_colptr_len", "llsa_perm_len"):
    getattr(_lib, _f).argtypes = [_P]
    getattr(_lib, _f).restype = ctypes.c_int64
_lib.llsa_workspace_bytes.argtypes = [_P, ctypes.c_int]
_lib.llsa_workspace_bytes.restype = ctypes.c_size_t
_lib.llsa_stream_wait.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
_lib.llsa_stream_wait.restype = ctypes.c_int
_lib.llsa_timing_enable.argtypes = [ctypes.c_int]
_lib.llsa_timing_enable.restype = ctypes.c_int
_lib.llsa_timing_read.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
_lib.llsa_timing_read.restype = ctypes.c_int
_lib.llsa_status_string.argtypes = [ctypes.c_int]
_lib.llsa_status_string.restype = ctypes.c_char_p


def lib():
    return _lib


def status_string(status: int) -> str:
    return _lib.llsa_status_string(status).decode()


def _check(status: int, where: str):
    if status != OK:
        raise LlsaError(status, where)


def resolve(prob: Problem) -> Problem:
    out = Problem()
    _check(_lib.llsa_resolve(ctypes.byref(prob), ctypes.byref(out)), "llsa_resolve")
    return out


def pyramid_rows(prob: Problem) -> int:
    return int(_lib.llsa_pyramid_rows(ctypes.byref(prob)))


def colptr_len(prob: Problem) -> int:
    return int(_lib.llsa_colptr_len(ctypes.byref(prob)))


def perm_len(prob: Problem) -> int:
    return int(_lib.llsa_perm_len(ctypes.byref(prob)))


def workspace_bytes(prob: Problem, op: int) -> int:
    return int(_lib.llsa_workspace_bytes(ctypes.byref(prob), op))


def stream_wait(waiter, signaler):
    """`waiter` waits, on the device, for the work enqueued on `signaler` so far (device-scope event)."""
    _check(_lib.llsa_stream_wait(_stream(waiter), _stream(signaler)), "llsa_stream_wait")


def timing_enable(on: bool = True):
    """Bracket every library kernel launch with hipEvents on its stream (clears earlier records)."""
    _check(_lib.llsa_timing_enable(1 if on else 0), "llsa_timing_enable")


def timing_read() -> dict:
    """{kernel family: (total ms, launches)} of the launches recorded since timing_enable."""
    out = {}
    for i, name in enumerate(KERNELS):
        t, c = ctypes.c_double(), ctypes.c_int64()
        _check(_lib.llsa_timing_read(i, ctypes.byref(t), ctypes.byref(c)), "llsa_timing_read")
        out[name] = (t.value, c.value)
    return out


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def build_pyramid(prob, q, k, v, pq, pk, pv, pk_bf16=None, pv_bf16=None, stream=None):
    """fp32 pyramids pq, pk, pv; for bf16 problems also the bf16 copies of pk, pv (the attention operands)."""
    _check(_lib.llsa_build_pyramid(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(pq), _ptr(pk), _ptr(pv),
                                   _ptr(pk_bf16), _ptr(pv_bf16), _stream(stream)), "llsa_build_pyramid")


def select(prob, pq, pk, idx, stream=None):
    _check(_lib.llsa_select(ctypes.byref(prob), _ptr(pq), _ptr(pk), _ptr(idx), _stream(stream)), "llsa_select")


def select_exhaustive(prob, pq, pk, idx1, stream=None):
    """Single-level exhaustive Top-K over all level-1 blocks (idx1: int32 [batch*heads, n_1, K])."""
    _check(_lib.llsa_select_exhaustive(ctypes.byref(prob), _ptr(pq), _ptr(pk), _ptr(idx1), _stream(stream)),
           "llsa_select_exhaustive")


def reorder(prob, grid_h, grid_w, to_local, x, y, stream=None):
    """Rows of x moved to the 2-D-local order (to_local) or back to row-major, into y."""
    _check(_lib.llsa_reorder(ctypes.byref(prob), grid_h, grid_w, int(bool(to_local)), _ptr(x), _ptr(y),
                             _stream(stream)), "llsa_reorder")


def attn_fwd(prob, q, k, v, pk, pv, idx, o, lse, stream=None):
    _check(_lib.llsa_attn_fwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(pk), _ptr(pv), _ptr(idx), _ptr(o),
                              _ptr(lse), _stream(stream)), "llsa_attn_fwd")


def attn_fwd_complement(prob, q, k, v, pk, pv, idx, o, lse, ws, stream=None):
    """Forward under the complement-partition reading of the enrichment (ws: OP_ATTN_FWD_COMPLEMENT bytes)."""
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.llsa_attn_fwd_complement(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(pk), _ptr(pv),
                                         _ptr(idx), _ptr(o), _ptr(lse), _ptr(ws), nbytes, _stream(stream)),
           "llsa_attn_fwd_complement")


def attn_bwd_complement(prob, q, k, v, o, lse, dout, pk, pv, idx, dq, dk, dv, ws, stream=None):
    """Backward under the complement-partition reading (ws: OP_ATTN_BWD_COMPLEMENT bytes)."""
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.llsa_attn_bwd_complement(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                         _ptr(dout), _ptr(pk), _ptr(pv), _ptr(idx), _ptr(dq), _ptr(dk), _ptr(dv),
                                         _ptr(ws), nbytes, _stream(stream)),
           "llsa_attn_bwd_complement")


def index_transpose(prob, idx, col_ptr, perm, ws, stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.llsa_index_transpose(ctypes.byref(prob), _ptr(idx), _ptr(col_ptr), _ptr(perm), _ptr(ws), nbytes,
                                     _stream(stream)), "llsa_index_transpose")


def index_transpose_noalloc(prob, idx, col_ptr, perm, stream=None):
    """llsa_index_transpose with its workspace in the library's static device scratch (allocates nothing)."""
    _check(_lib.llsa_index_transpose_noalloc(ctypes.byref(prob), _ptr(idx), _ptr(col_ptr), _ptr(perm),
                                             _stream(stream)), "llsa_index_transpose_noalloc")


def attn_bwd(prob, q, k, v, o, lse, dout, pk, pv, idx, col_ptr, perm, dq, dk, dv, ws, stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.llsa_attn_bwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                              _ptr(pk), _ptr(pv), _ptr(idx), _ptr(col_ptr), _ptr(perm), _ptr(dq), _ptr(dk), _ptr(dv),
                              _ptr(ws), nbytes, _stream(stream)), "llsa_attn_bwd")


class Buffers:
    """Device buffers for one problem (allocation through torch; compute through the library)."""

    def __init__(self, prob: Problem, device="cuda", backward=True):
        import torch
        r = resolve(prob)
        self.prob = r
        bh = r.batch * r.heads
        tdt = torch.bfloat16 if r.dtype == BF16 else torch.float32
        R = pyramid_rows(r)
        shape = (r.batch, r.heads, r.n, r.d)
        self.pq, self.pk, self.pv = (torch.empty((bh, R, r.d), dtype=torch.float32, device=device) for _ in range(3))
        # pooled K, V in the raw dtype, read by the attention calls (the fp32 pyramids themselves for fp32)
        if r.dtype == BF16:
            self.pkb, self.pvb = (torch.empty((bh, R, r.d), dtype=torch.bfloat16, device=device) for _ in range(2))
            self.pka, self.pva = self.pkb, self.pvb
        else:
            self.pkb = self.pvb = None
            self.pka, self.pva = self.pk, self.pv
        self.idx = torch.empty((bh, R, r.topk), dtype=torch.int32, device=device)
        self.o = torch.empty(shape, dtype=tdt, device=device)
        self.lse = torch.empty((bh, r.n), dtype=torch.float32, device=device)
        if backward:
            self.col_ptr = torch.empty((bh, colptr_len(r)), dtype=torch.int32, device=device)
            self.perm = torch.empty((bh, perm_len(r)), dtype=torch.int32, device=device)
            self.ws_t = torch.empty(max(1, workspace_bytes(r, OP_INDEX_TRANSPOSE)), dtype=torch.uint8, device=device)
            self.ws_b = torch.empty(max(1, workspace_bytes(r, OP_ATTN_BWD)), dtype=torch.uint8, device=device)
            self.dq, self.dk, self.dv = (torch.empty(shape, dtype=tdt, device=device) for _ in range(3))

    def pyramid(self, q, k, v, stream=None):
        build_pyramid(self.prob, q, k, v, self.pq, self.pk, self.pv, self.pkb, self.pvb, stream)

    def forward(self, q, k, v, stream=None):
        p = self.prob
        self.pyramid(q, k, v, stream)
        select(p, self.pq, self.pk, self.idx, stream)
        attn_fwd(p, q, k, v, self.pka, self.pva, self.idx, self.o, self.lse, stream)

    def backward(self, q, k, v, dout, stream=None):
        p = self.prob
        index_transpose(p, self.idx, self.col_ptr, self.perm, self.ws_t, stream)
        attn_bwd(p, q, k, v, self.o, self.lse, dout, self.pka, self.pva, self.idx, self.col_ptr, self.perm,
                 self.dq, self.dk, self.dv, self.ws_b, stream)

    def forward_backward(self, q, k, v, dout, stream, side):
        """The whole chain with the index transpose on the second stream `side`, beside the forward: it needs
        only the selection, and the backward waits for it (device-scope events through stream_wait; both
        streams at default priority)."""
        p = self.prob
        self.pyramid(q, k, v, stream)
        select(p, self.pq, self.pk, self.idx, stream)
        stream_wait(side, stream)
        index_transpose(p, self.idx, self.col_ptr, self.perm, self.ws_t, side)
        attn_fwd(p, q, k, v, self.pka, self.pva, self.idx, self.o, self.lse, stream)
        stream_wait(stream, side)
        attn_bwd(p, q, k, v, self.o, self.lse, dout, self.pka, self.pva, self.idx, self.col_ptr, self.perm,
                 self.dq, self.dk, self.dv, self.ws_b, stream)
