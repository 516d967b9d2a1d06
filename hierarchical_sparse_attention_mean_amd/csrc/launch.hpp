// launch.hpp -- host-side launchers of the gfx950 kernels (internal to libllsa.so).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.hpp"

namespace llsa {

// Kernel-family ids (same values as LLSA_KERNEL_* in llsa.h).
enum KernelFamily { kPool = 0, kSelect, kAttnFwd, kTranspose, kBwdDq, kBwdReduce, kBwdDkdv, kSelectExhaustive, kReorder,
                    kComplement, kFamilies };

// Brackets one kernel launch with hipEvents on its stream while timing is enabled (llsa_timing_enable).
class LaunchTimer {
 public:
  LaunchTimer(int family, hipStream_t stream);
  ~LaunchTimer();
  LaunchTimer(const LaunchTimer&) = delete;
  LaunchTimer& operator=(const LaunchTimer&) = delete;

 private:
  int family_;
  hipStream_t stream_;
  hipEvent_t start_ = nullptr, stop_ = nullptr;
};

// Per-level offsets of the concatenated CSC arrays (levels 1..T).
struct CscGeom {
  int T;                        // transposed levels
  int cp_len, pm_len;           // per-slice lengths of col_ptr and perm
  int cp_off[kMaxLevels + 1];   // cp_off[l]: first col_ptr entry of level l
  int pm_off[kMaxLevels + 1];   // pm_off[l]: first perm entry of level l
};

// Workgroups of `kernel` (at `threads` per workgroup, static LDS only) that the current device holds at
// once; 0 if the runtime cannot tell.  Cached per device and kernel.
int resident_workgroups(const void* kernel, int threads);
// Grid of a persistent kernel that wants `wanted` workgroups of work: at most one resident wave of
// workgroups, rounded up to a multiple of 8 (one per XCD), at least 8.
int persistent_grid(const void* kernel, int threads, int64_t wanted);
int resident_workgroups(const void* kernel, int threads);

hipError_t launch_pyramid(const Geom& g, int dtype_bf16, const void* q, const void* k, const void* v, float* pq,
                          float* pk, float* pv, void* pk_bf16, void* pv_bf16, hipStream_t stream);
hipError_t launch_select(const Geom& g, const float* pq, const float* pk, int32_t* idx, hipStream_t stream);
hipError_t launch_reorder(const Geom& g, int elem_bytes, int grid_w, int to_local, const void* x, void* y,
                          hipStream_t stream);
hipError_t launch_select_exhaustive(const Geom& g, const float* pq, const float* pk, int32_t* idx1,
                                    hipStream_t stream);
hipError_t launch_attn_fwd(const Geom& g, int dtype_bf16, const void* q, const void* k, const void* v,
                           const void* pk, const void* pv, const int32_t* idx, void* o, float* lse,
                           hipStream_t stream);
struct CompGeom;
// Candidate layout of the complement reading's pooled-gradient partials: per slice, n2u units of 16 fine
// blocks, each with nc partial rows (levels 1..L_e: ncand[l] candidates from row xoff[l]; 16 K below the
// coarsest level, n_L there), a row = d K values then d V values (fp32).
struct PartGeom {
  int n2u, nc;
  int ncand[kMaxLevels + 1], xoff[kMaxLevels + 1];
};
hipError_t launch_comp_grads(const Geom& g, const CscGeom& cg, const PartGeom& pg, const void* q, const void* dout,
                             const float* lse, const float* delta, const void* pk, const void* pv,
                             const int32_t* idx, const int32_t* col_ptr, const int32_t* perm, float* part,
                             float* gk, float* gv, hipStream_t stream);
hipError_t launch_complement_lists(const Geom& g, const CompGeom& cm, const int32_t* idx, int32_t* comp,
                                   hipStream_t stream);
hipError_t launch_attn_fwd_complement(const Geom& g, const CompGeom& cm, const void* q, const void* k,
                                      const void* v, const void* pk, const void* pv, const int32_t* idx,
                                      const int32_t* comp, void* o, float* lse, hipStream_t stream);
hipError_t launch_index_transpose(const Geom& g, const CscGeom& cg, const int32_t* idx, int32_t* col_ptr,
                                  int32_t* perm, int32_t* ws_cnt, int32_t* ws_tmp, hipStream_t stream);

// Backward workspace carve-up: fp32 delta [bh][n]; partials of pooled-token gradients for levels >= 2
// [bh][n_2][K*(Le-1)][d] (K and V); reduced pooled gradients of levels >= 2 [bh][R - n_1][d] (K, V); int32
// dK/dV work order [bh][ceil(n_1 / 4)].
struct BwdWs {
  float* delta;
  float* part_k;
  float* part_v;
  float* gk;
  float* gv;
  int4* items;       // [bh][DkdvBounds::items]: dK/dV work items, an end marker (group -1) after the last
  int4* splits;      // [bh][DkdvBounds::splits]: split groups (group, first slot, chunks, stages)
  int32_t* split_done;  // [bh][DkdvBounds::splits]: chunks of each split group finished
  float* dkdv_part;  // [bh][DkdvBounds::slots][4 blocks][K, V][16 keys][d]: partial sums of split groups
};
struct DkdvBounds {
  int items, slots, splits;  // per-slice capacities
};
DkdvBounds dkdv_bounds(const Geom& g);
size_t bwd_ws_layout(const Geom& g, BwdWs* out, void* base);
struct PartGeom;
struct CompGeom;
// The complement reading's backward workspace: delta, pooled gradients of every level (gk, gv: [bh][R][d]),
// the pooled-gradient partials (in part_k) and the dK/dV work lists.
size_t bwd_comp_ws_layout(const Geom& g, const PartGeom& pg, BwdWs* out, void* base);
hipError_t launch_attn_bwd_complement(const Geom& g, const CscGeom& cg, const CompGeom& cm, const PartGeom& pg,
                                      const void* q, const void* k, const void* v, const void* o, const float* lse,
                                      const void* dout, const void* pk, const void* pv, const int32_t* idx,
                                      const int32_t* comp, const int32_t* col_ptr, const int32_t* perm, void* dq,
                                      void* dk, void* dv, const BwdWs& ws, hipStream_t stream);
hipError_t launch_attn_bwd(const Geom& g, const CscGeom& cg, const void* q, const void* k, const void* v,
                           const void* o, const float* lse, const void* dout, const void* pk, const void* pv,
                           const int32_t* idx, const int32_t* col_ptr, const int32_t* perm, void* dq, void* dk,
                           void* dv, const BwdWs& ws, hipStream_t stream);

}  // namespace llsa
