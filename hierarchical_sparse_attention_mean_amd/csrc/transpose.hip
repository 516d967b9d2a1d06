// transpose.hip -- CSR -> CSC transpose of the per-level block selection.
//
// Method [LLSA review (pith.science, arXiv 2512.16615), "What carries the argument": a CSR-to-CSC scan
// gives every key block the list of query blocks that selected it, so the backward pass needs no
// dense N x N mask; Gustavson's permuted transposition is the cited prior art]: column j of level l
// lists the CSR positions p = u*K + k with idx[u][k] = j, in ascending p.
//
// Design (all levels 1..T of all slices in each launch, integer work only):
//   1. zero the per-column counters;
//   2. count: one thread per CSR entry, integer atomic add on its column's counter;
//   3. scan: one 1024-thread workgroup per (slice, level) turns counts into col_ptr with wavefront
//      prefix sums (__shfl_up inside each wave, then a scan of the 16 wave totals) and seeds the
//      per-column cursors;
//   4. scatter: one thread per entry claims a slot in its column with an atomic on the cursor;
//   5. order: one thread per entry counts the entries of its column with a smaller CSR position and
//      writes itself to that rank, which makes every column ascending (Gustavson order) and the whole
//      result independent of the order in which the atomics of step 4 landed.
#include "common.hpp"
#include "launch.hpp"

namespace llsa {

namespace {

// Flat entry id x in [0, pm_len) of one slice -> level and position p within that level.
__device__ __forceinline__ int entry_level(const CscGeom& cg, int x, int* p) {
  int l = 1;
  while (l < cg.T && x >= cg.pm_off[l + 1]) ++l;
  *p = x - cg.pm_off[l];
  return l;
}

__global__ void zero_i32(int32_t* __restrict__ a, int64_t n) {
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n; t += (int64_t)gridDim.x * blockDim.x)
    a[t] = 0;
}

// grid.x * blockDim.x >= pm_len, grid.y = slice.  cnt[slice][cp_off[l] + j + 1] += 1.
__global__ __launch_bounds__(256) void csc_count(const int32_t* __restrict__ idx, int32_t* __restrict__ cnt, Geom g,
                                                 CscGeom cg) {
  const int x = blockIdx.x * blockDim.x + threadIdx.x;
  if (x >= cg.pm_len) return;
  const int slice = blockIdx.y;
  int p;
  const int l = entry_level(cg, x, &p);
  const int j = idx[(size_t)slice * g.R * g.K + (size_t)g.off[l] * g.K + p];
  atomicAdd(&cnt[(size_t)slice * cg.cp_len + cg.cp_off[l] + j + 1], 1);
}

__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
    const int u = __shfl_up(v, s, 64);
    if (lane >= s) v += u;
  }
  return v;
}

// grid.x = T levels, grid.y = slice; 256 threads, 4 consecutive counters per thread (a small workgroup, so
// that it can run beside a resident attention kernel).  cnt[cp_off + 0 .. n_l] (entry 0 is zero, entry j+1
// the count of column j) is scanned inclusively into col_ptr, and the cursor of column j (= col_ptr[j]) is
// left in cnt[cp_off + j].
constexpr int kScanThreads = 256, kScanPer = 4;
__global__ __launch_bounds__(kScanThreads) void csc_scan(int32_t* __restrict__ cnt, int32_t* __restrict__ col_ptr,
                                                         Geom g, CscGeom cg) {
  constexpr int kWaves = kScanThreads / 64, kChunk = kScanThreads * kScanPer;
  __shared__ int wave_tot[kWaves];
  __shared__ int carry_s;
  const int l = blockIdx.x + 1, slice = blockIdx.y;
  const int len = g.rows[l] + 1;
  int32_t* a = cnt + (size_t)slice * cg.cp_len + cg.cp_off[l];
  int32_t* cp = col_ptr + (size_t)slice * cg.cp_len + cg.cp_off[l];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  if (t == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base < len; base += kChunk) {
    const int x0 = base + kScanPer * t;
    int v[kScanPer], run = 0;
#pragma unroll
    for (int i = 0; i < kScanPer; ++i) {
      v[i] = x0 + i < len ? a[x0 + i] : 0;
      run += v[i];
      v[i] = run;  // inclusive within the thread
    }
    const int inc = wave_inclusive_scan(run, lane);
    if (lane == 63) wave_tot[w] = inc;
    __syncthreads();
    if (w == 0) {
      const int tv = lane < kWaves ? wave_tot[lane] : 0;
      const int ti = wave_inclusive_scan(tv, lane);
      if (lane < kWaves) wave_tot[lane] = ti - tv;  // exclusive prefix of wave totals
    }
    __syncthreads();
    const int before = carry_s + wave_tot[w] + inc - run;  // exclusive prefix of this thread's first counter
#pragma unroll
    for (int i = 0; i < kScanPer; ++i) {
      const int x = x0 + i, out = before + v[i];
      if (x < len) cp[x] = out;
      if (x < len - 1) a[x] = out;  // cursor of column x = col_ptr[x]; a[x] was already read
    }
    __syncthreads();
    if (t == kScanThreads - 1) carry_s = before + run;
    __syncthreads();
  }
}

// tmp[slice][pm_off[l] + slot] = p, slot claimed from the column cursor.
__global__ __launch_bounds__(256) void csc_scatter(const int32_t* __restrict__ idx, int32_t* __restrict__ cursor,
                                                   int32_t* __restrict__ tmp, Geom g, CscGeom cg) {
  const int x = blockIdx.x * blockDim.x + threadIdx.x;
  if (x >= cg.pm_len) return;
  const int slice = blockIdx.y;
  int p;
  const int l = entry_level(cg, x, &p);
  const int j = idx[(size_t)slice * g.R * g.K + (size_t)g.off[l] * g.K + p];
  const int slot = atomicAdd(&cursor[(size_t)slice * cg.cp_len + cg.cp_off[l] + j], 1);
  tmp[(size_t)slice * cg.pm_len + cg.pm_off[l] + slot] = p;
}

// perm[col_ptr[j] + rank(p)] = p with rank = number of entries of column j below p.
__global__ __launch_bounds__(256) void csc_order(const int32_t* __restrict__ idx, const int32_t* __restrict__ col_ptr,
                                                 const int32_t* __restrict__ tmp, int32_t* __restrict__ perm, Geom g,
                                                 CscGeom cg) {
  const int x = blockIdx.x * blockDim.x + threadIdx.x;
  if (x >= cg.pm_len) return;
  const int slice = blockIdx.y;
  int p;
  const int l = entry_level(cg, x, &p);
  const int j = idx[(size_t)slice * g.R * g.K + (size_t)g.off[l] * g.K + p];
  const int32_t* cp = col_ptr + (size_t)slice * cg.cp_len + cg.cp_off[l];
  const int32_t* col = tmp + (size_t)slice * cg.pm_len + cg.pm_off[l];
  const int b = cp[j], e = cp[j + 1];
  int rank = 0;
  for (int y = b; y < e; ++y) rank += col[y] < p;
  perm[(size_t)slice * cg.pm_len + cg.pm_off[l] + b + rank] = p;
}

}  // namespace

hipError_t launch_index_transpose(const Geom& g, const CscGeom& cg, const int32_t* idx, int32_t* col_ptr,
                                  int32_t* perm, int32_t* ws_cnt, int32_t* ws_tmp, hipStream_t stream) {
  const int64_t ncnt = (int64_t)g.bh * cg.cp_len;
  {
    LaunchTimer timer(kTranspose, stream);
    zero_i32<<<(int)((ncnt + 255) / 256 < 4096 ? (ncnt + 255) / 256 : 4096), 256, 0, stream>>>(ws_cnt, ncnt);
  }
  const dim3 egrid((cg.pm_len + 255) / 256, g.bh);
  {
    LaunchTimer timer(kTranspose, stream);
    csc_count<<<egrid, 256, 0, stream>>>(idx, ws_cnt, g, cg);
  }
  {
    LaunchTimer timer(kTranspose, stream);
    csc_scan<<<dim3(cg.T, g.bh), kScanThreads, 0, stream>>>(ws_cnt, col_ptr, g, cg);
  }
  {
    LaunchTimer timer(kTranspose, stream);
    csc_scatter<<<egrid, 256, 0, stream>>>(idx, ws_cnt, ws_tmp, g, cg);
  }
  {
    LaunchTimer timer(kTranspose, stream);
    csc_order<<<egrid, 256, 0, stream>>>(idx, col_ptr, ws_tmp, perm, g, cg);
  }
  return hipGetLastError();
}

}  // namespace llsa
