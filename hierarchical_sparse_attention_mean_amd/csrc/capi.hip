// capi.hip -- the C ABI of libllsa.so: host-side validation, workspace carving and kernel launches.
//
// Every entry point validates the problem and its pointers before launching anything, enqueues its
// kernels on the caller's stream and returns without synchronising (contract in include/llsa.h).
#include <math.h>
#include <string.h>

#include <algorithm>
#include <atomic>

#include "entries.hpp"
#include "launch.hpp"
#include "llsa.h"

namespace {

using llsa::CscGeom;
using llsa::Geom;

struct Resolved {
  llsa_problem p;
  Geom g;
  CscGeom cg;
  int64_t bh;
};

// largest m with B^m <= n
int floor_log(int64_t n, int B) {
  int m = 0;
  int64_t p = 1;
  while (p <= n / B) {
    p *= B;
    ++m;
  }
  return m;
}

int resolve(const llsa_problem* in, Resolved* r) {
  if (!in) return LLSA_ERR_NULL;
  llsa_problem p = *in;
  if (p.dtype != LLSA_F32 && p.dtype != LLSA_BF16) return LLSA_ERR_DTYPE;
  if (p.batch < 0 || p.heads < 0 || p.n < 1 || p.d < 1 || p.block < 2 || p.topk < 1) return LLSA_ERR_SHAPE;
  // pooled levels: L = floor(log_B n - 1) by default, and 1 <= L <= that maximum
  const int lmax = floor_log(p.n, p.block) - 1;
  if (lmax < 1) return LLSA_ERR_SHAPE;
  const int L = p.levels == 0 ? lmax : p.levels;
  if (L < 1 || L > lmax || L > llsa::kMaxLevels) return LLSA_ERR_SHAPE;
  int64_t span = 1;
  for (int l = 0; l < L; ++l) span *= p.block;
  if (p.n % span != 0) return LLSA_ERR_SHAPE;
  const int64_t nL = p.n / span;
  if (p.topk > nL) return LLSA_ERR_SHAPE;
  const int Le = p.enrich_levels == -1 ? L : p.enrich_levels;
  if (Le < 0 || Le > L) return LLSA_ERR_SHAPE;
  float scale = p.scale == 0.0f ? 1.0f / sqrtf((float)p.d) : p.scale;
  if (!isfinite(scale)) return LLSA_ERR_PARAM;
  if (p.grid_w < 0) return LLSA_ERR_SHAPE;
  // limits of the gfx950 kernels
  if (p.d != llsa::kD || p.block != llsa::kB) return LLSA_ERR_UNSUPPORTED;
  if (p.topk > 32 || nL > 512 || (int64_t)p.topk * Le > 128) return LLSA_ERR_UNSUPPORTED;
  const int64_t bh = (int64_t)p.batch * p.heads;
  if (bh * p.n * p.d >= ((int64_t)1 << 31)) return LLSA_ERR_UNSUPPORTED;
  p.levels = L;
  p.enrich_levels = Le;
  p.scale = scale;
  // the grid hint applies when a grid row holds whole dK/dV key-block groups (4 blocks of B tokens)
  const int64_t group_tokens = 4 * (int64_t)p.block;
  if (p.grid_w > 0 && (p.grid_w % group_tokens != 0 || p.n % p.grid_w != 0)) p.grid_w = 0;
  if (r) {
    r->p = p;
    r->bh = bh;
    Geom& g = r->g;
    memset(&g, 0, sizeof(g));
    g.bh = (int)bh;
    g.n = p.n;
    g.K = p.topk;
    g.L = L;
    g.Le = Le;
    g.rows[0] = p.n;
    int off = 0;
    for (int l = 1; l <= L; ++l) {
      g.rows[l] = g.rows[l - 1] / p.block;
      g.off[l] = off;
      off += g.rows[l];
    }
    g.off[L + 1] = off;
    g.R = off;
    g.scale = scale;
    g.scale_log2 = scale * llsa::kLog2e;
    g.gpr = (int)(p.grid_w / group_tokens);
    CscGeom& cg = r->cg;
    memset(&cg, 0, sizeof(cg));
    cg.T = Le < 1 ? 1 : Le;
    int cpo = 0, pmo = 0;
    for (int l = 1; l <= cg.T; ++l) {
      cg.cp_off[l] = cpo;
      cg.pm_off[l] = pmo;
      cpo += g.rows[l] + 1;
      pmo += g.rows[l] * p.topk;
    }
    cg.cp_len = cpo;
    cg.pm_len = pmo;
  }
  return LLSA_OK;
}

// The kernels are built for gfx950 only; check the current device once per device (the cached answer is an
// atomic: concurrent first calls may both query, and store the same value).
int check_device() {
  static std::atomic<int> state[64];  // 0 unknown, 1 gfx950, -1 other
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LLSA_ERR_DEVICE;
  if (dev < 0 || dev >= 64) return LLSA_ERR_DEVICE;
  int st = state[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return LLSA_ERR_DEVICE;
    st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    state[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? LLSA_OK : LLSA_ERR_DEVICE;
}

int check_ptrs(std::initializer_list<const void*> ptrs) {
  for (const void* x : ptrs)
    if (!x) return LLSA_ERR_NULL;
  for (const void* x : ptrs)
    if (reinterpret_cast<uintptr_t>(x) & 15u) return LLSA_ERR_ALIGN;
  return LLSA_OK;
}

int launched(hipError_t e) { return e == hipSuccess ? LLSA_OK : LLSA_ERR_LAUNCH; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// transpose workspace: per-column counters (cursors) of every slice and level, then the unordered CSC staging
size_t transpose_cnt_bytes(const Resolved& r) {
  return align256((size_t)r.bh * r.cg.cp_len * sizeof(int32_t));
}
size_t transpose_ws(const Resolved& r) {
  return transpose_cnt_bytes(r) + align256((size_t)r.bh * r.cg.pm_len * sizeof(int32_t));
}

// Complement lists: level l = 1..L_e, m_l = (B-1) K candidates scored and not kept per unit (n_L - K at the
// coarsest level), n_l units.
llsa::CompGeom comp_geom(const Resolved& r) {
  llsa::CompGeom cm;
  memset(&cm, 0, sizeof(cm));
  const llsa::Geom& g = r.g;
  int off = 0;
  for (int l = 1; l <= g.Le; ++l) {
    cm.m[l] = l == g.L ? g.rows[l] - g.K : (llsa::kB - 1) * g.K;
    cm.off[l] = off;
    off += g.rows[l] * cm.m[l];
    cm.total += cm.m[l];
  }
  cm.slice = off;
  return cm;
}
size_t complement_ws(const Resolved& r) { return align256((size_t)r.bh * comp_geom(r).slice * sizeof(int32_t)); }

// CSC of levels 1..T (the layout llsa_index_transpose produces for T = max(1, L_e)).
llsa::CscGeom csc_geom(const Resolved& r, int T) {
  llsa::CscGeom cg;
  memset(&cg, 0, sizeof(cg));
  cg.T = T;
  int cpo = 0, pmo = 0;
  for (int l = 1; l <= T; ++l) {
    cg.cp_off[l] = cpo;
    cg.pm_off[l] = pmo;
    cpo += r.g.rows[l] + 1;
    pmo += r.g.rows[l] * r.g.K;
  }
  cg.cp_len = cpo;
  cg.pm_len = pmo;
  return cg;
}

// Backward of the complement reading: its pooled-gradient reduction reads the CSC of level l + 1 for every
// l <= L_e below the coarsest level, so it builds the CSC of levels 1..min(L_e + 1, L) itself.
llsa::CscGeom comp_csc_geom(const Resolved& r) { return csc_geom(r, std::max(1, std::min(r.g.Le + 1, r.g.L))); }
llsa::PartGeom part_geom(const Resolved& r) {
  llsa::PartGeom pg;
  memset(&pg, 0, sizeof(pg));
  pg.n2u = (r.g.rows[1] + 15) / 16;
  for (int l = 1; l <= r.g.Le; ++l) {
    pg.ncand[l] = l == r.g.L ? r.g.rows[l] : llsa::kB * r.g.K;
    pg.xoff[l] = pg.nc;
    pg.nc += pg.ncand[l];
  }
  return pg;
}
// [complement lists | col_ptr | perm | transpose counters | transpose staging | backward workspace]
struct CompBwdParts {
  size_t lists, cp, pm, cnt, tmp, bwd;
};
CompBwdParts comp_bwd_parts(const Resolved& r) {
  const llsa::CscGeom cg = comp_csc_geom(r);
  CompBwdParts z;
  z.lists = complement_ws(r);
  z.cp = align256((size_t)r.bh * cg.cp_len * sizeof(int32_t));
  z.pm = align256((size_t)r.bh * cg.pm_len * sizeof(int32_t));
  z.cnt = z.cp;
  z.tmp = z.pm;
  z.bwd = llsa::bwd_comp_ws_layout(r.g, part_geom(r), nullptr, nullptr);
  return z;
}
size_t comp_bwd_ws(const Resolved& r) {
  const CompBwdParts z = comp_bwd_parts(r);
  return z.lists + z.cp + z.pm + z.cnt + z.tmp + z.bwd;
}

#define LLSA_TRY(x)          \
  do {                       \
    const int _s = (x);      \
    if (_s != LLSA_OK) return _s; \
  } while (0)

}  // namespace

namespace llsa {
// For llsa_index_transpose_noalloc (noalloc.hip): the validated geometry of a transpose and the bytes of its
// workspace (column counters first, then the staging array).
int resolve_transpose(const llsa_problem* prob, Geom* g, CscGeom* cg, size_t* cnt_bytes, size_t* ws_bytes) {
  Resolved r;
  LLSA_TRY(resolve(prob, &r));
  *g = r.g;
  *cg = r.cg;
  *cnt_bytes = transpose_cnt_bytes(r);
  *ws_bytes = transpose_ws(r);
  return LLSA_OK;
}
int check_device_gfx950() { return check_device(); }
}  // namespace llsa

extern "C" {

int llsa_resolve(const llsa_problem* prob, llsa_problem* out) {
  Resolved r;
  LLSA_TRY(resolve(prob, &r));
  if (out) *out = r.p;
  return LLSA_OK;
}

int64_t llsa_pyramid_rows(const llsa_problem* prob) {
  Resolved r;
  const int s = resolve(prob, &r);
  return s == LLSA_OK ? (int64_t)r.g.R : (int64_t)s;
}

int64_t llsa_colptr_len(const llsa_problem* prob) {
  Resolved r;
  const int s = resolve(prob, &r);
  return s == LLSA_OK ? (int64_t)r.cg.cp_len : (int64_t)s;
}

int64_t llsa_perm_len(const llsa_problem* prob) {
  Resolved r;
  const int s = resolve(prob, &r);
  return s == LLSA_OK ? (int64_t)r.cg.pm_len : (int64_t)s;
}

size_t llsa_workspace_bytes(const llsa_problem* prob, int op) {
  Resolved r;
  if (resolve(prob, &r) != LLSA_OK) return 0;
  if (op == LLSA_OP_INDEX_TRANSPOSE) return transpose_ws(r);
  if (op == LLSA_OP_ATTN_BWD) return llsa::bwd_ws_layout(r.g, nullptr, nullptr);
  if (op == LLSA_OP_ATTN_FWD_COMPLEMENT) return complement_ws(r);
  if (op == LLSA_OP_ATTN_BWD_COMPLEMENT) return comp_bwd_ws(r);
  return 0;
}

const char* llsa_status_string(int status) {
  switch (status) {
    case LLSA_OK: return "ok";
    case LLSA_ERR_NULL: return "a required pointer is NULL";
    case LLSA_ERR_SHAPE: return "invalid shape: need n mod B^L == 0, 1 <= L <= floor(log_B n - 1), 1 <= K <= n/B^L, 0 <= L_e <= L";
    case LLSA_ERR_UNSUPPORTED: return "outside the limits of the gfx950 kernels (d = 64, B = 16, K <= 32, n/B^L <= 512, K*L_e <= 128, K*(L_e-1) <= 32, size < 2^31)";
    case LLSA_ERR_DTYPE: return "unsupported dtype for this entry point";
    case LLSA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case LLSA_ERR_WORKSPACE: return "workspace missing or too small";
    case LLSA_ERR_LAUNCH: return "kernel launch failed";
    case LLSA_ERR_PARAM: return "scale is not finite";
    case LLSA_ERR_DEVICE: return "the current device is not gfx950";
    case LLSA_ERR_SCRATCH: return "the transpose workspace exceeds the static scratch of llsa_index_transpose_noalloc (16 MiB)";
    default: return "unknown status";
  }
}

int llsa_build_pyramid(const llsa_problem* prob, const void* q, const void* k, const void* v, float* pq, float* pk,
                       float* pv, void* pk_bf16, void* pv_bf16, hipStream_t stream) {
  Resolved r;
  LLSA_TRY(resolve(prob, &r));
  if (r.bh == 0) return LLSA_OK;
  const bool bf16 = r.p.dtype == LLSA_BF16;
  LLSA_TRY(check_ptrs({q, k, v, pq, pk, pv}));
  if (bf16) LLSA_TRY(check_ptrs({pk_bf16, pv_bf16}));
  LLSA_TRY(check_device());
  return launched(llsa::launch_pyramid(r.g, bf16, q, k, v, pq, pk, pv, bf16 ? pk_bf16 : nullptr,
                                       bf16 ? pv_bf16 : nullptr, stream));
}

int llsa_select(const llsa_problem* prob, const float* pq, const float* pk, int32_t* idx, hipStream_t stream) {
  Resolved r;
  LLSA_TRY(resolve(prob, &r));
  if (r.bh == 0) return LLSA_OK;
  LLSA_TRY(check_ptrs({pq, pk, idx}));
  LLSA_TRY(check_device());
  return launched(llsa::launch_select(r.g, pq, pk, idx, stream));
}

int llsa_select_exhaustive(const llsa_problem* prob, const float* pq, const float* pk, int32_t* idx1, hipStream_t stream) {
  Resolved r;
  LLSA_TRY(resolve(prob, &r));
  if (r.bh == 0) return LLSA_OK;
  LLSA_TRY(check_ptrs({pq, pk, idx1}));
  LLSA_TRY(check_device());
  return launched(llsa::launch_select_exhaustive(r.g, pq, pk, idx1, stream));
}

int llsa_reorder(const llsa_problem* prob, int32_t grid_h, int32_t grid_w, int32_t to_local, const void* x, void* y,
                 hipStream_t stream) {
  Resolved r;
  LLSA_TRY(resolve(prob, &r));
  const int64_t S = (int64_t)1 << (2 * r.g.L);  // 4^L
  if (grid_h < 1 || grid_w < 1 || (int64_t)grid_h * grid_w != r.p.n || grid_h % S != 0 || grid_w % S != 0)
    return LLSA_ERR_SHAPE;
  if (r.bh == 0) return LLSA_OK;
  LLSA_TRY(check_ptrs({x, y}));
  if (x == y) return LLSA_ERR_PARAM;
  LLSA_TRY(check_device());
  return launched(llsa::launch_reorder(r.g, r.p.dtype == LLSA_BF16 ? 2 : 4, grid_w, to_local != 0, x, y,
                                       stream));
}

int llsa_attn_fwd(const llsa_problem* prob, const void* q, const void* k, const void* v, const void* pk,
                  const void* pv, const int32_t* idx, void* o, float* lse, hipStream_t stream) {
  Resolved r;
  LLSA_TRY(resolve(prob, &r));
  if (r.bh == 0) return LLSA_OK;
  LLSA_TRY(check_ptrs({q, k, v, pk, pv, idx, o, lse}));
  LLSA_TRY(check_device());
  return launched(
      llsa::launch_attn_fwd(r.g, r.p.dtype == LLSA_BF16, q, k, v, pk, pv, idx, o, lse, stream));
}

int llsa_attn_fwd_complement(const llsa_problem* prob, const void* q, const void* k, const void* v, const void* pk,
                             const void* pv, const int32_t* idx, void* o, float* lse, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  Resolved r;
  LLSA_TRY(resolve(prob, &r));
  if (r.p.dtype != LLSA_BF16) return LLSA_ERR_DTYPE;
  const llsa::CompGeom cm = comp_geom(r);
  if (cm.total > llsa::kMaxComplement) return LLSA_ERR_UNSUPPORTED;
  if (r.bh == 0) return LLSA_OK;
  LLSA_TRY(check_ptrs({q, k, v, pk, pv, idx, o, lse}));
  const size_t need = complement_ws(r);
  if (need > 0 && (!ws || ws_bytes < need)) return LLSA_ERR_WORKSPACE;
  if (need > 0) LLSA_TRY(check_ptrs({ws}));
  LLSA_TRY(check_device());
  int32_t* comp = static_cast<int32_t*>(ws);
  hipError_t e = llsa::launch_complement_lists(r.g, cm, idx, comp, stream);
  if (e != hipSuccess) return LLSA_ERR_LAUNCH;
  return launched(llsa::launch_attn_fwd_complement(r.g, cm, q, k, v, pk, pv, idx, comp ? comp : idx, o, lse,
                                                   stream));
}

int llsa_index_transpose(const llsa_problem* prob, const int32_t* idx, int32_t* col_ptr, int32_t* perm, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  Resolved r;
  LLSA_TRY(resolve(prob, &r));
  if (r.bh == 0) return LLSA_OK;
  LLSA_TRY(check_ptrs({idx, col_ptr, perm}));
  const size_t need = transpose_ws(r);
  if (!ws || ws_bytes < need) return LLSA_ERR_WORKSPACE;
  LLSA_TRY(check_ptrs({ws}));
  LLSA_TRY(check_device());
  int32_t* cnt = static_cast<int32_t*>(ws);
  int32_t* tmp = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + transpose_cnt_bytes(r));
  return launched(llsa::launch_index_transpose(r.g, r.cg, idx, col_ptr, perm, cnt, tmp, stream));
}

int llsa_attn_bwd(const llsa_problem* prob, const void* q, const void* k, const void* v, const void* o,
                  const float* lse, const void* dout, const void* pk, const void* pv, const int32_t* idx,
                  const int32_t* col_ptr, const int32_t* perm, void* dq, void* dk, void* dv, void* ws,
                  size_t ws_bytes, hipStream_t stream) {
  Resolved r;
  LLSA_TRY(resolve(prob, &r));
  if (r.p.dtype != LLSA_BF16) return LLSA_ERR_DTYPE;
  if (r.g.Le >= 2 && r.g.K * (r.g.Le - 1) > 32) return LLSA_ERR_UNSUPPORTED;
  if (r.bh == 0) return LLSA_OK;
  LLSA_TRY(check_ptrs({q, k, v, o, lse, dout, pk, pv, idx, col_ptr, perm, dq, dk, dv}));
  const size_t need = llsa::bwd_ws_layout(r.g, nullptr, nullptr);
  if (!ws || ws_bytes < need) return LLSA_ERR_WORKSPACE;
  LLSA_TRY(check_ptrs({ws}));
  LLSA_TRY(check_device());
  llsa::BwdWs w;
  llsa::bwd_ws_layout(r.g, &w, ws);
  return launched(llsa::launch_attn_bwd(r.g, r.cg, q, k, v, o, lse, dout, pk, pv, idx, col_ptr, perm, dq, dk, dv, w,
                                        stream));
}

int llsa_attn_bwd_complement(const llsa_problem* prob, const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout, const void* pk, const void* pv, const int32_t* idx,
                             void* dq, void* dk, void* dv, void* ws, size_t ws_bytes, hipStream_t stream) {
  Resolved r;
  LLSA_TRY(resolve(prob, &r));
  if (r.p.dtype != LLSA_BF16) return LLSA_ERR_DTYPE;
  const llsa::CompGeom cm = comp_geom(r);
  if (cm.total > llsa::kMaxComplement) return LLSA_ERR_UNSUPPORTED;
  if (r.bh == 0) return LLSA_OK;
  LLSA_TRY(check_ptrs({q, k, v, o, lse, dout, pk, pv, idx, dq, dk, dv}));
  if (!ws || ws_bytes < comp_bwd_ws(r)) return LLSA_ERR_WORKSPACE;
  LLSA_TRY(check_ptrs({ws}));
  LLSA_TRY(check_device());
  const CompBwdParts z = comp_bwd_parts(r);
  char* p = static_cast<char*>(ws);
  int32_t* comp = reinterpret_cast<int32_t*>(p);
  int32_t* col_ptr = reinterpret_cast<int32_t*>(p + z.lists);
  int32_t* perm = reinterpret_cast<int32_t*>(p + z.lists + z.cp);
  int32_t* cnt = reinterpret_cast<int32_t*>(p + z.lists + z.cp + z.pm);
  int32_t* tmp = reinterpret_cast<int32_t*>(p + z.lists + z.cp + z.pm + z.cnt);
  llsa::BwdWs w;
  const llsa::PartGeom pg = part_geom(r);
  llsa::bwd_comp_ws_layout(r.g, pg, &w, p + z.lists + z.cp + z.pm + z.cnt + z.tmp);
  const llsa::CscGeom cg = comp_csc_geom(r);
  const hipStream_t st = stream;
  hipError_t e = llsa::launch_complement_lists(r.g, cm, idx, comp, st);
  if (e == hipSuccess) e = llsa::launch_index_transpose(r.g, cg, idx, col_ptr, perm, cnt, tmp, st);
  if (e != hipSuccess) return LLSA_ERR_LAUNCH;
  return launched(llsa::launch_attn_bwd_complement(r.g, cg, cm, pg, q, k, v, o, lse, dout, pk, pv, idx, comp, col_ptr,
                                                   perm, dq, dk, dv, w, st));
}

int llsa_stream_wait(hipStream_t waiter, hipStream_t signaler) {
  // an event without the system-scope fence: kernels of one device see each other's results through the
  // device-scope release at kernel end; the host- and peer-visible fence only delays the waiting stream
  hipEvent_t ev;
  if (hipEventCreateWithFlags(&ev, hipEventDisableTiming | hipEventDisableSystemFence) != hipSuccess)
    return LLSA_ERR_LAUNCH;
  hipError_t e = hipEventRecord(ev, signaler);
  if (e == hipSuccess) e = hipStreamWaitEvent(waiter, ev, 0);
  const hipError_t d = hipEventDestroy(ev);  // released once the recorded point completes
  return e == hipSuccess && d == hipSuccess ? LLSA_OK : LLSA_ERR_LAUNCH;
}

}  // extern "C"
