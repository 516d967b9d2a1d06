// transpose.hip -- CSR -> CSC transpose of the per-level block selection.
//
// Method [LLSA review (pith.science, arXiv 2512.16615), "What carries the argument": a CSR-to-CSC scan
// gives every key block the list of query blocks that selected it, so the backward pass needs no
// dense N x N mask; Gustavson's permuted transposition is the cited prior art]: column j of level l
// lists the CSR positions p = u*K + k with idx[u][k] = j, in ascending p.
//
// Design (integer work only; all levels of all slices in each launch unless stated):
//   Column counts and col_ptr (with the per-column cursors), in one of three ways:
//   a. n_1 + 1 <= 16384: csc_count_scan -- counters in LDS, one workgroup per slice and level, counted and scanned
//      in one kernel;
//   b. else, when K >= 4 and every level is transposed: csc_count_part -- partial histograms in LDS over 4, 8 or
//      16 (<= K) parts of each level's entries and ranges of 4096 columns, small enough to run beside the forward
//      -- then csc_sum_parts (the parts of each column summed in part order) and csc_scan; no global atomics;
//   c. else: zero the counters; csc_count, one thread per CSR entry, an integer atomic add on its column's
//      counter; csc_scan, one 1024-thread workgroup per (slice, level), wavefront prefix sums.
//   Then the entries:
//   - fill, when every level is transposed (T = L), level by level from the coarsest: the selection is
//     hierarchical -- a unit's picks at level l < L are children of its parent's picks at level l+1 -- so
//     the units that can have picked key block j of level l are the children of the level-(l+1) units in
//     column j/B of level l+1.  One wavefront per (slice, group of B = 16 columns) walks those candidate
//     units in ascending order (at the coarsest level: all units) and writes each found entry at its
//     column's start plus its rank, from ballot prefix counts: ascending order directly, no atomics.  A
//     column with fewer entries found than counted (an input that is not hierarchical) is redone by a scan of
//     all its level's rows;
//   - otherwise (T < L): scatter, one thread per entry claiming a slot in its column with an atomic on the
//     cursor, then order, one thread per entry writing itself at its rank among the column's entries, which
//     makes every column ascending and the result independent of the order in which the atomics landed.
#include <type_traits>

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
  // an index outside [0, n_l) (not a selection) is skipped below 0 and clamped above, as in every transpose
  // kernel, so that no write leaves the arrays; the result is then unspecified
  if (j >= 0) atomicAdd(&cnt[(size_t)slice * cg.cp_len + cg.cp_off[l] + min(j, g.rows[l] - 1) + 1], 1);
}

__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
    const int u = __shfl_up(v, s, 64);
    if (lane >= s) v += u;
  }
  return v;
}

// grid.x = T levels, grid.y = slice; 1024 threads, 4 consecutive counters per thread.  cnt[cp_off + 0 .. n_l]
// (entry 0 is zero, entry j+1 the count of column j) is scanned inclusively into col_ptr, and the cursor of
// column j (= col_ptr[j]) is left in cnt[cp_off + j].
constexpr int kScanThreads = 1024, kScanPer = 4;
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

// Steps 1-3 in one kernel when a level's counters fit in LDS: grid.x = T levels, grid.y = slice, 1024
// threads, dynamic LDS of max_l (n_l + 1) ints.  The counts are LDS atomics (their sum does not depend on the
// order), then the same scan as csc_scan runs on the LDS copy; col_ptr and the cursors go to memory.
constexpr int kFusedCountMax = 16384;  // counters per level held in LDS (64 KB)
__global__ __launch_bounds__(kScanThreads) void csc_count_scan(const int32_t* __restrict__ idx,
                                                               int32_t* __restrict__ cursor,
                                                               int32_t* __restrict__ col_ptr, Geom g, CscGeom cg) {
  extern __shared__ int cnt_s[];
  constexpr int kWaves = kScanThreads / 64, kChunk = kScanThreads * kScanPer;
  __shared__ int wave_tot[kWaves];
  __shared__ int carry_s;
  const int l = blockIdx.x + 1, slice = blockIdx.y;
  const int nl = g.rows[l], len = nl + 1;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  for (int x = t; x < len; x += kScanThreads) cnt_s[x] = 0;
  if (t == 0) carry_s = 0;
  __syncthreads();
  const int32_t* I = idx + (size_t)slice * g.R * g.K + (size_t)g.off[l] * g.K;
  const int ne = nl * g.K;
  // 8 loads in flight per thread before their (clamped, in-LDS) atomic increments
  for (int x0 = 0; x0 < ne; x0 += 8 * kScanThreads) {
    int v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int x = x0 + i * kScanThreads + t;
      v[i] = x < ne ? I[x] : -1;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (v[i] >= 0) atomicAdd(&cnt_s[min(v[i], nl - 1) + 1], 1);
  }
  __syncthreads();
  int32_t* cur = cursor + (size_t)slice * cg.cp_len + cg.cp_off[l];
  int32_t* cp = col_ptr + (size_t)slice * cg.cp_len + cg.cp_off[l];
  for (int base = 0; base < len; base += kChunk) {
    const int x0 = base + kScanPer * t;
    int v[kScanPer], run = 0;
#pragma unroll
    for (int i = 0; i < kScanPer; ++i) {
      run += x0 + i < len ? cnt_s[x0 + i] : 0;
      v[i] = run;  // inclusive within the thread
    }
    const int inc = wave_inclusive_scan(run, lane);
    if (lane == 63) wave_tot[w] = inc;
    __syncthreads();
    if (w == 0) {
      const int tv = lane < kWaves ? wave_tot[lane] : 0;
      const int ti = wave_inclusive_scan(tv, lane);
      if (lane < kWaves) wave_tot[lane] = ti - tv;
    }
    __syncthreads();
    const int before = carry_s + wave_tot[w] + inc - run;
#pragma unroll
    for (int i = 0; i < kScanPer; ++i) {
      const int x = x0 + i, out = before + v[i];
      if (x < len) cp[x] = out;
      if (x < len - 1) cur[x] = out;
    }
    __syncthreads();
    if (t == kScanThreads - 1) carry_s = before + run;
    __syncthreads();
  }
}

// Counts without global atomics when a level's entries are too many for one workgroup (csc_count_scan):
// grid.x = P parts x ranges of kPartCols columns, grid.y = T levels, grid.z = slice; 1024 threads, LDS of
// kPartCols ints (16 KB: these workgroups fit on a CU beside the forward's, which the transpose runs beside).
// Part p counts the entries [p ne / P, (p+1) ne / P) of its level whose column lies in its range, with LDS
// atomics, and writes its range of the histogram to part[p][j] at tmp[slice][pm_off[l] + p n_l + j] (the
// level's staging area holds n_l K >= n_l P ints); csc_sum_parts then sums the P histograms of each column in
// part order, and csc_scan scans the counts.  Integer counts: the result does not depend on the order of the
// atomics.  (Global atomics for the counts slowed the forward running beside them by about 8 %.)
constexpr int kPartCols = 4096;
template <int P>
__global__ __launch_bounds__(kScanThreads) void csc_count_part(const int32_t* __restrict__ idx,
                                                               int32_t* __restrict__ tmp, Geom g, CscGeom cg) {
  __shared__ int cnt_s[kPartCols];
  const int part = blockIdx.x % P, c0 = kPartCols * (blockIdx.x / P), l = blockIdx.y + 1, slice = blockIdx.z;
  const int nl = g.rows[l], t = threadIdx.x;
  if (c0 >= nl) return;  // a column range past this level's columns (no barrier is used before this point)
  const int nc = min(kPartCols, nl - c0);
  for (int x = t; x < nc; x += kScanThreads) cnt_s[x] = 0;
  __syncthreads();
  const int32_t* I = idx + (size_t)slice * g.R * g.K + (size_t)g.off[l] * g.K;
  const int ne = nl * g.K;
  const int e0 = (int)((int64_t)part * ne / P), e1 = (int)((int64_t)(part + 1) * ne / P);
  for (int x0 = e0; x0 < e1; x0 += 8 * kScanThreads) {
    int v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int x = x0 + i * kScanThreads + t;
      v[i] = x < e1 ? I[x] : -1;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = min(v[i], nl - 1) - c0;  // below 0 (skipped) for a negative index
      if (v[i] >= 0 && j >= 0 && j < nc) atomicAdd(&cnt_s[j], 1);
    }
  }
  __syncthreads();
  int32_t* out = tmp + (size_t)slice * cg.pm_len + cg.pm_off[l] + (size_t)part * nl + c0;
  for (int x = t; x < nc; x += kScanThreads) out[x] = cnt_s[x];
}

// grid.x = column groups of 256, grid.y = T levels, grid.z = slice; 256 threads, one column each.  Column j's
// count is the sum of the P part histograms (in part order), written as csc_count leaves it
// (cnt[cp_off + j + 1], entry 0 zero) for csc_scan.  Few registers and no LDS, so that it runs beside the forward.
template <int P>
__global__ __launch_bounds__(256) void csc_sum_parts(const int32_t* __restrict__ tmp, int32_t* __restrict__ cnt,
                                                     Geom g, CscGeom cg) {
  const int l = blockIdx.y + 1, slice = blockIdx.z, nl = g.rows[l];
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= nl) return;
  const int32_t* parts = tmp + (size_t)slice * cg.pm_len + cg.pm_off[l] + j;
  int pc[P];
#pragma unroll
  for (int q = 0; q < P; ++q) pc[q] = parts[(size_t)q * nl];
  int c = 0;
#pragma unroll
  for (int q = 0; q < P; ++q) c += pc[q];
  int32_t* a = cnt + (size_t)slice * cg.cp_len + cg.cp_off[l];
  a[j + 1] = c;
  if (j == 0) a[0] = 0;
}

constexpr int kMaxTopK = 32;  // K limit of the GPU path

// Level-l fill (see the design notes).  grid.x = ceil(n_l / 16) column groups, grid.y = slice; one wavefront
// each, so that all of them are resident at once.  Candidates go in rounds of 64 kFillPer (4 kFillPer parents):
// the parents' positions are read by the first lanes, then every lane issues the row loads of its kFillPer
// candidates of the round at once (a long column would otherwise pay one memory round trip per 64 candidates);
// the kFillPer sub-chunks of 64 candidates are then ranked in candidate order with one ballot per column, the
// running per-column counts wave-uniform.
// KM: the smallest of 8, 16, 32 that holds K (registers per candidate row).  kFillPer: candidates per lane and
// round; 2 for KM = 16 (62 VGPRs), so that two of these waves fit on a SIMD beside the forward's two, which the
// transpose runs beside (with 8: 168 VGPRs, one wave, and the N = 262144 transpose outlasted the forward).
template <int KM, int kFillPer>
__global__ __launch_bounds__(64) void csc_fill(const int32_t* __restrict__ idx, const int32_t* __restrict__ col_ptr,
                                               int32_t* __restrict__ perm, Geom g, CscGeom cg, int l) {
  constexpr int kFillRound = 64 * kFillPer;
  const int J = blockIdx.x, slice = blockIdx.y, lane = threadIdx.x;
  const int nl = g.rows[l], K = g.K;
  const int32_t* I = idx + (size_t)slice * g.R * K + (size_t)g.off[l] * K;  // level-l rows
  const int32_t* cp = col_ptr + (size_t)slice * cg.cp_len + cg.cp_off[l];
  int32_t* pm = perm + (size_t)slice * cg.pm_len + cg.pm_off[l];
  const int cpl = cp[min(16 * J + lane, nl)];  // lanes 0..16: starts of the group's columns and the end
  // candidate units: all units at the coarsest level, else the 16 children of each unit of column J at l+1
  const bool top = l == g.L;
  int ncand = nl, pbeg = 0, nparent = 1;
  const int32_t* ppm = nullptr;
  if (!top) {
    const int32_t* cp1 = col_ptr + (size_t)slice * cg.cp_len + cg.cp_off[l + 1];
    pbeg = cp1[J];
    ncand = 16 * (cp1[J + 1] - pbeg);
    ppm = perm + (size_t)slice * cg.pm_len + cg.pm_off[l + 1];
    nparent = g.rows[l + 1];
  }
  int done[16];
#pragma unroll
  for (int cc = 0; cc < 16; ++cc) done[cc] = 0;
  for (int r0 = 0; r0 < ncand; r0 += kFillRound) {
    int par = 0;  // lanes 0..31: parent unit r0/16 + lane (clamped: reads stay in bounds)
    if (!top && lane < kFillRound / 16 && r0 / 16 + lane < ncand / 16)
      par = min(max(ppm[pbeg + r0 / 16 + lane] / K, 0), nparent - 1);
    // this lane's candidates r0 + 64 i + lane: the rows' entries, all loads issued before any is used
    int vals[kFillPer][KM];
    int unit[kFillPer];
    const int nsub = min(kFillPer, (ncand - r0 + 63) / 64);  // sub-chunks of this round that hold candidates
#pragma unroll
    for (int i = 0; i < kFillPer; ++i) {
      if (i >= nsub) break;  // uniform
      const int cl = min(r0 + 64 * i + lane, ncand - 1) - r0;  // in-bounds duplicate past the end, never used
      unit[i] = top ? r0 + cl : 16 * __shfl(par, cl >> 4, 64) + (cl & 15);
      const int32_t* row = I + (size_t)unit[i] * K;
      if ((K & 3) == 0) {
#pragma unroll
        for (int q4 = 0; q4 < KM / 4; ++q4) {
          if (4 * q4 < K) {
            const int4 x = *reinterpret_cast<const int4*>(row + 4 * q4);
            vals[i][4 * q4] = x.x; vals[i][4 * q4 + 1] = x.y; vals[i][4 * q4 + 2] = x.z; vals[i][4 * q4 + 3] = x.w;
          }
        }
      } else {
#pragma unroll
        for (int k = 0; k < KM; ++k)
          if (k < K) vals[i][k] = row[k];
      }
    }
#pragma unroll
    for (int i = 0; i < kFillPer; ++i) {
      if (i >= nsub) break;  // uniform
      uint32_t mask = 0;  // columns 16J + c this candidate picked (at most one entry each; a row ascends)
      int k0 = 0;
      if (r0 + 64 * i + lane < ncand) {
#pragma unroll
        for (int k = KM - 1; k >= 0; --k) {
          if (k < K && (vals[i][k] >> 4) == J) {
            mask |= 1u << (vals[i][k] & 15);
            k0 = k;  // ends at the first (lowest) slot in the group
          }
        }
      }
      // an entry's rank: the column's entries of earlier sub-chunks, then the lanes below with the same column
#pragma unroll
      for (int cc = 0; cc < 16; ++cc) {
        const bool has = (mask >> cc) & 1u;
        const uint64_t b = __ballot(has);
        const int pos = __builtin_amdgcn_readlane(cpl, cc) + done[cc] +
                        __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0));
        if (has && pos < __builtin_amdgcn_readlane(cpl, cc + 1))
          pm[pos] = unit[i] * K + k0 + __popc(mask & ((1u << cc) - 1u));
        done[cc] += __popcll(b);
      }
    }
  }
  // A column with fewer entries found than counted (the input was not hierarchical) is redone by a scan of all
  // level-l rows in ascending order: slow, but only such inputs take it.
  for (int cc = 0; cc < 16; ++cc) {
    const int j = 16 * J + cc;
    const int b0 = __builtin_amdgcn_readlane(cpl, cc), b1 = __builtin_amdgcn_readlane(cpl, cc + 1);
    if (j >= nl || done[cc] == b1 - b0) continue;  // uniform
    int rank = 0;
    for (int u0 = 0; u0 < nl; u0 += 64) {
      const int u = u0 + lane;
      int kf = -1;
      if (u < nl)
        for (int k = 0; k < K; ++k)
          if (I[(size_t)u * K + k] == j) kf = k;
      const uint64_t b = __ballot(kf >= 0);
      const int pos = b0 + rank + __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0));
      if (kf >= 0 && pos < b1) pm[pos] = u * K + kf;
      rank += __popcll(b);
    }
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
  if (j < 0) return;
  const int slot = atomicAdd(&cursor[(size_t)slice * cg.cp_len + cg.cp_off[l] + min(j, g.rows[l] - 1)], 1);
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
  const int jr = idx[(size_t)slice * g.R * g.K + (size_t)g.off[l] * g.K + p];
  if (jr < 0) return;
  const int j = min(jr, g.rows[l] - 1);
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
  const dim3 egrid((cg.pm_len + 255) / 256, g.bh);
  const bool fused = g.rows[1] + 1 <= kFusedCountMax;
  if (fused) {
    LaunchTimer timer(kTranspose, stream);
    csc_count_scan<<<dim3(cg.T, g.bh), kScanThreads, (g.rows[1] + 1) * sizeof(int32_t), stream>>>(idx, ws_cnt,
                                                                                              col_ptr, g, cg);
  } else if (cg.T == g.L && g.K >= 4) {
    // partial histograms in the staging area, which the fills below do not use (P <= K parts fit it)
    auto run = [&](auto kp) {
      constexpr int P = decltype(kp)::value;
      {
        LaunchTimer timer(kTranspose, stream);
        const int ranges = (g.rows[1] + kPartCols - 1) / kPartCols;
        csc_count_part<P><<<dim3(P * ranges, cg.T, g.bh), kScanThreads, 0, stream>>>(idx, ws_tmp, g, cg);
      }
      {
        LaunchTimer timer(kTranspose, stream);
        csc_sum_parts<P><<<dim3((g.rows[1] + 255) / 256, cg.T, g.bh), 256, 0, stream>>>(ws_tmp, ws_cnt, g, cg);
      }
      {
        LaunchTimer timer(kTranspose, stream);
        csc_scan<<<dim3(cg.T, g.bh), kScanThreads, 0, stream>>>(ws_cnt, col_ptr, g, cg);
      }
    };
    if (g.K >= 16)
      run(std::integral_constant<int, 16>{});
    else if (g.K >= 8)
      run(std::integral_constant<int, 8>{});
    else
      run(std::integral_constant<int, 4>{});
  } else {
    const int64_t ncnt = (int64_t)g.bh * cg.cp_len;
    {
      LaunchTimer timer(kTranspose, stream);
      zero_i32<<<(int)((ncnt + 255) / 256 < 4096 ? (ncnt + 255) / 256 : 4096), 256, 0, stream>>>(ws_cnt, ncnt);
    }
    {
      LaunchTimer timer(kTranspose, stream);
      csc_count<<<egrid, 256, 0, stream>>>(idx, ws_cnt, g, cg);
    }
    {
      LaunchTimer timer(kTranspose, stream);
      csc_scan<<<dim3(cg.T, g.bh), kScanThreads, 0, stream>>>(ws_cnt, col_ptr, g, cg);
    }
  }
  if (cg.T == g.L) {
    for (int l = g.L; l >= 1; --l) {
      LaunchTimer timer(kTranspose, stream);
      auto kernel = g.K <= 8 ? csc_fill<8, 8> : g.K <= 16 ? csc_fill<16, 2> : csc_fill<kMaxTopK, 8>;
      kernel<<<dim3((g.rows[l] + 15) / 16, g.bh), 64, 0, stream>>>(idx, col_ptr, perm, g, cg, l);
    }
  } else {
    {
      LaunchTimer timer(kTranspose, stream);
      csc_scatter<<<egrid, 256, 0, stream>>>(idx, ws_cnt, ws_tmp, g, cg);
    }
    {
      LaunchTimer timer(kTranspose, stream);
      csc_order<<<egrid, 256, 0, stream>>>(idx, col_ptr, ws_tmp, perm, g, cg);
    }
  }
  return hipGetLastError();
}

}  // namespace llsa
