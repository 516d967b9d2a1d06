// select.hip -- hierarchical Top-K block selection.
//
// Method [LLSA review (pith.science, arXiv 2512.16615), "Core claim", "What carries the argument",
// referee major comment 1 on Algorithm 1]: the coarsest level L scores every pooled key block for each
// pooled query unit and keeps the best K; each finer level l scores only the B children of each block
// kept by the unit's parent (u / B) at level l+1 and keeps the best K.  Score = pooled query . pooled
// key (unscaled); ties go to the lower block index; each index row is stored ascending.
//
// Design:
//   * One 256-thread workgroup per (slice, parent unit at level l+1): its B = 16 child units share the
//     same K*16 candidate rows, so the scores are a 16 x (16K) x 64 fp32 product, run on
//     v_mfma_f32_16x16x4_f32 (fp32 keeps the ranking faithful to the exact scores).  The coarsest
//     level uses the same products and Top-K with "all n_L blocks" as the candidate list: for L = 1 in a
//     launch of its own (16 query units per workgroup), else inside the first descent launch, whose
//     workgroup selects its parent's coarsest row before the parent's children.
//   * Top-K per query row without sorting: a 32-step bitwise search for the K-th largest
//     order-preserving score key (one compare + one ballot per slot group and step, the group count a
//     compile-time constant), then ties at the threshold are
//     taken in ascending slot order and the kept slots are compacted in ascending order with ballot
//     prefix counts -- candidate slots ascend with block index, so this realises the tie rule and the
//     ascending row order directly.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace llsa {

namespace {

constexpr int kMaxSlotsPerLane = 8;  // up to 512 candidates per query row
// Top-K modes (a template parameter of select_level, so that each instance holds only its own registers):
// sorted-list merges of 8 keys per lane (K <= 8, at most 128 candidates), of 16 keys per lane (K <= 16, at most
// 256 candidates), else the bitwise threshold search.
enum TopkMode { kMerge8 = 0, kMerge16 = 1, kBitwise = 2 };

// Order-preserving map of an fp32 score to uint32 (+0 and -0 compare equal).
__device__ __forceinline__ uint32_t ord_key(float s) {
  uint32_t u = __float_as_uint(s + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }

// Number of set bits of `m` below this lane.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

// Top-K of each of the workgroup's query rows from the scores in LDS (16 rows x ldc floats, slot order =
// candidate order): a 32-step bitwise search for the K-th largest order-preserving key (one compare and one
// ballot per slot group and step), ties at the threshold taken in ascending slot order, kept slots compacted in
// ascending order with ballot prefix counts.  Candidate slots ascend with block index, so this realises the
// tie rule and the ascending row order directly.  Wave w handles rows 4w .. 4w+3, their four searches
// interleaved step by step (independent compare -> count -> select chains that hide each other's latency).
// kM = ceil(ncand / 64) slot groups per lane, a compile-time constant so that the 32 search steps carry no
// per-group branches.
template <int kM>
__device__ __forceinline__ void topk_rows(const float* sc, int ldc, int ncand, int nq, int K, int w, int lane,
                                          int32_t* out_rows, const int32_t* picks, int coarsest) {
  constexpr int kR = 4;
  uint32_t key[kR][kM];
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    const int row = 4 * w + r;
#pragma unroll
    for (int m = 0; m < kM; ++m) {
      const int s = lane + 64 * m;
      // invalid slots (beyond the candidate count or past the last level-L block) and rows past nq get key
      // 0, below every real score's key (the smallest, -inf, maps to 0x007FFFFF)
      key[r][m] = (row < nq && s < ncand) ? ord_key(sc[row * ldc + s]) : 0u;
    }
  }
  // K-th largest key of each row by bitwise search: largest T with #{key >= T} >= K
  uint32_t T[kR];
#pragma unroll
  for (int r = 0; r < kR; ++r) T[r] = 0;
#pragma unroll 2
  for (int bit = 31; bit >= 0; --bit) {
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      const uint32_t cand = T[r] | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int m = 0; m < kM; ++m) cnt += popc64(__ballot(key[r][m] >= cand));
      T[r] = cnt >= K ? cand : T[r];
    }
  }
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    const int row = 4 * w + r;
    if (row >= nq) break;
    int greater = 0;
#pragma unroll
    for (int m = 0; m < kM; ++m) greater += popc64(__ballot(key[r][m] > T[r]));
    const int need = K - greater;  // ties at T to take, lowest slots first
    int eq_before = 0, sel_before = 0;
    int32_t* out = out_rows + (size_t)row * K;
#pragma unroll
    for (int m = 0; m < kM; ++m) {
      const uint64_t eqm = __ballot(key[r][m] == T[r]);
      const bool sel_eq = (key[r][m] == T[r]) && (eq_before + lanes_below(eqm) < need);
      const bool sel = (key[r][m] > T[r]) || sel_eq;
      const uint64_t selm = __ballot(sel);
      if (sel) {
        const int s = lane + 64 * m;
        const int blk = coarsest ? s : picks[s >> 4] * kB + (s & 15);
        out[sel_before + lanes_below(selm)] = blk;
      }
      eq_before += popc64(eqm);
      sel_before += popc64(selm);
    }
  }
}

// Compare-exchange of two keys, the larger first.
__device__ __forceinline__ void cx(uint32_t& a, uint32_t& b) {
  const uint32_t hi = max(a, b), lo = min(a, b);
  a = hi;
  b = lo;
}

// Sorts a lane's kL keys, largest first: the 19-comparator network for 8 keys, a bitonic network for 16.
template <int kL>
__device__ __forceinline__ void sort_desc(uint32_t t[kL]) {
  if constexpr (kL == 8) {
    cx(t[0], t[2]); cx(t[1], t[3]); cx(t[4], t[6]); cx(t[5], t[7]);
    cx(t[0], t[4]); cx(t[1], t[5]); cx(t[2], t[6]); cx(t[3], t[7]);
    cx(t[0], t[1]); cx(t[2], t[3]); cx(t[4], t[5]); cx(t[6], t[7]);
    cx(t[2], t[4]); cx(t[3], t[5]);
    cx(t[1], t[4]); cx(t[3], t[6]);
    cx(t[1], t[2]); cx(t[3], t[4]); cx(t[5], t[6]);
  } else {
#pragma unroll
    for (int k = 2; k <= kL; k <<= 1)
#pragma unroll
      for (int j = k >> 1; j >= 1; j >>= 1)
#pragma unroll
        for (int i = 0; i < kL; ++i)
          if ((i ^ j) > i) {
            if ((i & k) == 0)
              cx(t[i], t[i ^ j]);
            else
              cx(t[i ^ j], t[i]);
          }
  }
}

// One merge step of the per-lane sorted (descending) kL-key lists: the partner lane's list comes over DPP
// (`kCtrl`), the element-wise maxima of this list and the partner's reversed list are the kL largest keys of
// the two (a bitonic sequence), and a half-cleaner network sorts them again.
template <int kL, int kCtrl>
__device__ __forceinline__ void merge_lists(uint32_t t[kL]) {
  uint32_t c[kL];
#pragma unroll
  for (int i = 0; i < kL; ++i)
    c[i] = max(t[i], (uint32_t)__builtin_amdgcn_mov_dpp((int)t[kL - 1 - i], kCtrl, 0xf, 0xf, false));
#pragma unroll
  for (int d = kL / 2; d >= 1; d >>= 1)
#pragma unroll
    for (int i = 0; i < kL; ++i)
      if ((i & d) == 0) cx(c[i], c[i + d]);
#pragma unroll
  for (int i = 0; i < kL; ++i) t[i] = c[i];
}

// Top-K for K <= kL and at most 16 kL candidates.  Row 4w + r of the workgroup goes to quarter-wave r (lanes
// 16r .. 16r+15); lane l16 holds the kL slots l16 + 16i.
//   1. Each lane sorts its keys (sort_desc).
//   2. Four merge steps with the lanes 1 and 2 apart (quad swaps), then 4 and 8 apart (row rotations): every
//      lane of the quarter ends up with the row's kL largest keys, sorted.  The K-th of them is the threshold T.
//   3. The kept slots are taken as in topk_rows: keys above T, then keys equal to T in ascending slot order,
//      compacted in ascending slot order with ballot prefix counts restricted to the quarter.
// So the result equals the exact Top-K with ties to the lower slot (the lower block index).
template <int kL>
__device__ __forceinline__ void topk_rows_merge(const float* sc, int ldc, int ncand, int nq, int K, int w, int lane,
                                                int32_t* out_rows, const int32_t* picks, int coarsest) {
  const int r = lane >> 4, l16 = lane & 15, row = 4 * w + r;
  const bool live = row < nq;
  uint32_t key[kL], t[kL];
#pragma unroll
  for (int i = 0; i < kL; ++i) {
    const int s = l16 + 16 * i;
    // invalid slots and rows past nq get key 0, below every real score's key (-inf maps to 0x007FFFFF)
    key[i] = (live && s < ncand) ? ord_key(sc[row * ldc + s]) : 0u;
    t[i] = key[i];
  }
  sort_desc<kL>(t);
  merge_lists<kL, 0xB1 /* quad_perm [1,0,3,2] */>(t);
  merge_lists<kL, 0x4E /* quad_perm [2,3,0,1] */>(t);
  merge_lists<kL, 0x124 /* row_ror:4 */>(t);
  merge_lists<kL, 0x128 /* row_ror:8 */>(t);
  uint32_t T = t[0];
#pragma unroll
  for (int i = 1; i < kL; ++i) T = i == K - 1 ? t[i] : T;
  const uint64_t qmask = 0xFFFFull << (16 * r);
  int greater = 0;
#pragma unroll
  for (int i = 0; i < kL; ++i) greater += popc64(__ballot(key[i] > T) & qmask);
  const int need = K - greater;  // ties at T to take, lowest slots first
  int eq_before = 0, sel_before = 0;
  int32_t* out = out_rows + (size_t)row * K;
#pragma unroll
  for (int i = 0; i < kL; ++i) {
    const uint64_t eqm = __ballot(key[i] == T) & qmask;
    const bool sel = key[i] > T || (key[i] == T && eq_before + lanes_below(eqm) < need);
    const uint64_t selm = __ballot(sel) & qmask;
    if (sel && live) {
      const int s = l16 + 16 * i;
      const int blk = coarsest ? s : picks[s >> 4] * kB + (s & 15);
      out[sel_before + lanes_below(selm)] = blk;
    }
    eq_before += popc64(eqm);
    sel_before += popc64(selm);
  }
}

__host__ __device__ constexpr int topk_mode(int K, int ncand) {
  return (K <= 8 && ncand <= 128) ? kMerge8 : (K <= 16 && ncand <= 256) ? kMerge16 : kBitwise;
}

template <int kMode>
__device__ __forceinline__ void topk_dispatch(const float* sc, int ldc, int ncand, int nq, int K, int w, int lane,
                                              int32_t* out_rows, const int32_t* picks, int coarsest) {
  if constexpr (kMode == kMerge8) {
    topk_rows_merge<8>(sc, ldc, ncand, nq, K, w, lane, out_rows, picks, coarsest);
  } else if constexpr (kMode == kMerge16) {
    topk_rows_merge<16>(sc, ldc, ncand, nq, K, w, lane, out_rows, picks, coarsest);
  } else {
    const int M = (ncand + 63) / 64;
    if (M <= 1)
      topk_rows<1>(sc, ldc, ncand, nq, K, w, lane, out_rows, picks, coarsest);
    else if (M == 2)
      topk_rows<2>(sc, ldc, ncand, nq, K, w, lane, out_rows, picks, coarsest);
    else if (M <= 4)
      topk_rows<4>(sc, ldc, ncand, nq, K, w, lane, out_rows, picks, coarsest);
    else
      topk_rows<kMaxSlotsPerLane>(sc, ldc, ncand, nq, K, w, lane, out_rows, picks, coarsest);
  }
}

// Scores and Top-K of the query rows q0 .. q0+nq-1 of `level` (nq <= 16), written to `out` (nq rows of K).
// coarsest: the candidates are all n_L blocks; else the B children of each pick of the parent, read from
// `cand_picks` (the parent's selection row, in memory or LDS), with `lds_picks` the same picks in LDS for the
// block numbers of the kept slots.  Dynamic LDS `sc`: 16 rows x ldc floats of scores.  Ends after the Top-K
// (the caller orders any reuse of sc).
template <int kMode>
__device__ __forceinline__ void select_rows(const float* __restrict__ PQ, const float* __restrict__ PK,
                                            const Geom& g, int level, int coarsest, int q0, int nq,
                                            const int32_t* cand_picks, const int32_t* lds_picks, int ncand, int ldc,
                                            float* sc, int32_t* out) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, c = lane & 15, gg = lane >> 4;
  const int nl = g.rows[level];
  const int ntiles = (ncand + 15) / 16;
  // A operand: this lane's query row (q0 + c); step s = 4m + e uses dim 16m + 4gg + e, so that the four lanes
  // of a row read 64 contiguous bytes per load (the same dim order for both operands).
  float qf[16];
  {
    const bool ok = c < nq;
    const float4* src = reinterpret_cast<const float4*>(PQ + (size_t)(g.off[level] + q0 + (ok ? c : 0)) * kD + 4 * gg);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float4 x = ok ? src[4 * m] : make_float4(0, 0, 0, 0);
      qf[4 * m] = x.x; qf[4 * m + 1] = x.y; qf[4 * m + 2] = x.z; qf[4 * m + 3] = x.w;
    }
  }
  // candidate row of tile t for this lane's column c (row 0 where the slot is empty), scores -inf there
  auto cand_row = [&](int t, bool* valid) {
    int j;
    if (coarsest) {
      j = 16 * t + c;
      *valid = j < nl;
    } else {
      j = cand_picks[t] * kB + c;
      *valid = true;
    }
    return g.off[level] + (*valid ? j : 0);
  };
  auto load_row = [&](int row, float kf[16]) {
    const float4* src = reinterpret_cast<const float4*>(PK + (size_t)row * kD + 4 * gg);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const float4 x = src[4 * m];
      kf[4 * m] = x.x; kf[4 * m + 1] = x.y; kf[4 * m + 2] = x.z; kf[4 * m + 3] = x.w;
    }
  };
  // tiles two at a time (t and t + 4): both tiles' rows in flight together, their MFMA chains interleaved
  for (int t = w; t < ntiles; t += 8) {
    const bool two = t + 4 < ntiles;
    bool v0, v1 = false;
    const int r0 = cand_row(t, &v0);
    const int r1 = two ? cand_row(t + 4, &v1) : r0;
    float k0[16], k1[16];
    load_row(r0, k0);
    load_row(r1, k1);
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      a0 = mfma_f32_k4(qf[s], k0[s], a0);
      a1 = mfma_f32_k4(qf[s], k1[s], a1);
    }
    // a*[r] = score(query row 4*gg + r, candidate slot 16*t + c)
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[(4 * gg + r) * ldc + 16 * t + c] = v0 ? a0[r] : -INFINITY;
    if (two) {
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[(4 * gg + r) * ldc + 16 * (t + 4) + c] = v1 ? a1[r] : -INFINITY;
    }
  }
  __syncthreads();

  topk_dispatch<kMode>(sc, ldc, ncand, nq, g.K, w, lane, out, lds_picks, coarsest);
}

// Coarsest: grid.x = 16-row query tiles, grid.y = slice.  Descent: 1-D grid over (slice, parent unit at
// level+1), remapped so that consecutive parents run on one XCD and its L2 holds their slices' pooled keys.
// kTop >= 0 (the descent from the coarsest level only): the workgroup first selects its parent's own row of the
// coarsest level (Top-K mode kTop; the same products and Top-K as the coarsest launch, so the same picks) and
// keeps it in LDS, which saves the coarsest level its own launch.  Dynamic LDS: 16 rows x ldc floats of scores
// (ldc covers the coarsest level's candidates too when kTop >= 0).
template <int kMode, int kTop>
__global__ __launch_bounds__(256) void select_level(const float* __restrict__ pq, const float* __restrict__ pk,
                                                    int32_t* __restrict__ idx, Geom g, int level, int coarsest,
                                                    int ncand, int ldc) {
  extern __shared__ float sc[];
  int slice = blockIdx.y, bx = blockIdx.x;
  if (!coarsest) {
    const int np = g.rows[level + 1];
    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    slice = wg / np; bx = wg - slice * np;
  }
  const float* PQ = pq + (size_t)slice * g.R * kD;
  const float* PK = pk + (size_t)slice * g.R * kD;
  int32_t* I = idx + (size_t)slice * g.R * g.K;
  const int nl = g.rows[level];
  const int q0 = 16 * bx;
  const int nq = coarsest ? min(16, nl - q0) : 16;
  // the parent's picks also in LDS, for the block numbers of the kept slots (a global read there would wait
  // behind the row's stores, which may alias it)
  __shared__ int pks[32];
  const int32_t* picks = nullptr;
  if constexpr (kTop >= 0) {
    const int nL = g.rows[level + 1];
    select_rows<kTop>(PQ, PK, g, level + 1, 1, bx, 1, nullptr, nullptr, nL, ldc, sc, pks);
    __syncthreads();  // the row is in pks, and the scores are read
    if (threadIdx.x < g.K) I[(size_t)(g.off[level + 1] + bx) * g.K + threadIdx.x] = pks[threadIdx.x];
    picks = pks;
  } else {
    picks = coarsest ? nullptr : I + (size_t)(g.off[level + 1] + bx) * g.K;
    if (!coarsest && threadIdx.x < g.K) pks[threadIdx.x] = picks[threadIdx.x];
  }
  select_rows<kMode>(PQ, PK, g, level, coarsest, q0, nq, picks, pks, ncand, ldc, sc,
                     I + (size_t)(g.off[level] + q0) * g.K);
}

// ------------------------------------------------------------------------------------------------
// Exhaustive single-level Top-K (the quadratic baseline of the hierarchy; "general Top-K" of Figure 1):
// every level-1 unit scores all n_1 level-1 key blocks.  grid.x = slices x 16-unit tiles (remapped),
// 256 threads.  Candidates stream by in chunks of 64 (one 16x16 fp32 MFMA tile per wave); each row keeps a
// buffer of at most kBuf (score, block) pairs in LDS: a candidate enters only if its score beats the row's
// current K-th best (candidates arrive in ascending block order, so an equal score loses the tie), and the
// buffer is cut back to its best K whenever it passes kBuf - 64 entries.
// ------------------------------------------------------------------------------------------------
constexpr int kBuf = 128;

// Best K of the first `cnt` entries of one row buffer, ties to the lower slot (= lower block), moved to slots
// 0..K-1 in slot order; returns the order-preserving key of the K-th best.
__device__ __forceinline__ uint32_t row_cut(float* bs, int* bi, int cnt, int K, int lane) {
  uint32_t key[2];
  float sv[2];
  int iv[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int s = lane + 64 * m;
    sv[m] = s < cnt ? bs[s] : 0.f;
    iv[m] = s < cnt ? bi[s] : 0;
    key[m] = s < cnt ? ord_key(sv[m]) : 0u;
  }
  uint32_t T = 0;
#pragma unroll 4
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    const int c = popc64(__ballot(key[0] >= cand)) + popc64(__ballot(key[1] >= cand));
    T = c >= K ? cand : T;
  }
  const int need = K - popc64(__ballot(key[0] > T)) - popc64(__ballot(key[1] > T));
  int eq_before = 0, sel_before = 0;
  int dst[2];
  bool sel[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const uint64_t eqm = __ballot(key[m] == T);
    sel[m] = key[m] > T || (key[m] == T && eq_before + lanes_below(eqm) < need);
    const uint64_t selm = __ballot(sel[m]);
    dst[m] = sel_before + lanes_below(selm);
    eq_before += popc64(eqm);
    sel_before += popc64(selm);
  }
  // every read above is done before any slot is overwritten (values are held in registers)
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    if (sel[m]) {
      bs[dst[m]] = sv[m];
      bi[dst[m]] = iv[m];
    }
  }
  return T;
}

__global__ __launch_bounds__(256) void select_exhaustive(const float* __restrict__ pq, const float* __restrict__ pk,
                                                         int32_t* __restrict__ out, Geom g) {
  __shared__ float sc[16][64 + 4];
  __shared__ float bs[16][kBuf];
  __shared__ int bi[16][kBuf];
  __shared__ uint32_t thr[16];
  __shared__ int bcnt[16];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, c = lane & 15, gg = lane >> 4;
  const int n1 = g.rows[1];
  const int tiles = (n1 + 15) / 16;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int slice = wg / tiles, q0 = 16 * (wg - slice * tiles);
  const int nq = min(16, n1 - q0);
  const float* PQ = pq + ((size_t)slice * g.R + g.off[1]) * kD;
  const float* PK = pk + ((size_t)slice * g.R + g.off[1]) * kD;
  float qf[16];
  {
    const float4* src = reinterpret_cast<const float4*>(PQ + (size_t)(q0 + min(c, nq - 1)) * kD + 16 * gg);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const float4 x = src[m];
      qf[4 * m] = x.x; qf[4 * m + 1] = x.y; qf[4 * m + 2] = x.z; qf[4 * m + 3] = x.w;
    }
  }
  if (threadIdx.x < 16) {
    thr[threadIdx.x] = 0u;
    bcnt[threadIdx.x] = 0;
  }
  __syncthreads();
  for (int c0 = 0; c0 < n1; c0 += 64) {
    {
      const int j = c0 + 16 * w + c;
      const bool valid = j < n1;
      const float4* src = reinterpret_cast<const float4*>(PK + (size_t)(valid ? j : 0) * kD + 16 * gg);
      float kf[16];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float4 x = src[m];
        kf[4 * m] = x.x; kf[4 * m + 1] = x.y; kf[4 * m + 2] = x.z; kf[4 * m + 3] = x.w;
      }
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s2 = 0; s2 < 16; ++s2) acc = mfma_f32_k4(qf[s2], kf[s2], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[4 * gg + r][16 * w + c] = valid ? acc[r] : -INFINITY;
    }
    __syncthreads();
    for (int rr = 0; rr < 4; ++rr) {
      const int row = 4 * w + rr;
      if (row >= nq) break;
      const float s = sc[row][lane];
      const bool take = c0 + lane < n1 && ord_key(s) > thr[row];
      const uint64_t mask = __ballot(take);
      int cnt = bcnt[row];
      if (take) {
        const int pos = cnt + lanes_below(mask);
        bs[row][pos] = s;
        bi[row][pos] = c0 + lane;
      }
      cnt += popc64(mask);
      if (cnt > kBuf - 64) {
        const uint32_t T = row_cut(bs[row], bi[row], cnt, g.K, lane);
        cnt = g.K;
        if (lane == 0) thr[row] = T;
      }
      if (lane == 0) bcnt[row] = cnt;
    }
    __syncthreads();
  }
  for (int rr = 0; rr < 4; ++rr) {
    const int row = 4 * w + rr;
    if (row >= nq) break;
    const int cnt = bcnt[row];
    if (cnt > g.K) row_cut(bs[row], bi[row], cnt, g.K, lane);
    if (lane < g.K) out[((size_t)slice * n1 + q0 + row) * g.K + lane] = bi[row][lane];
  }
}

}  // namespace

// select_level's instance for the level's Top-K mode (and, top >= 0, the fused coarsest row's)
template <int kTop>
static void launch_select_level_t(dim3 grid, int ldc, hipStream_t stream, const float* pq, const float* pk,
                                  int32_t* idx, const Geom& g, int level, int coarsest, int ncand) {
  const size_t lds = 16 * ldc * sizeof(float);
  switch (topk_mode(g.K, ncand)) {
    case kMerge8:
      select_level<kMerge8, kTop><<<grid, 256, lds, stream>>>(pq, pk, idx, g, level, coarsest, ncand, ldc);
      break;
    case kMerge16:
      select_level<kMerge16, kTop><<<grid, 256, lds, stream>>>(pq, pk, idx, g, level, coarsest, ncand, ldc);
      break;
    default:
      select_level<kBitwise, kTop><<<grid, 256, lds, stream>>>(pq, pk, idx, g, level, coarsest, ncand, ldc);
  }
}

hipError_t launch_select(const Geom& g, const float* pq, const float* pk, int32_t* idx, hipStream_t stream) {
  const int nL = g.rows[g.L];
  const int ncandL = ((nL + 15) / 16) * 16;
  if (g.L == 1) {  // the coarsest level alone: all n_L blocks are candidates
    LaunchTimer timer(kSelect, stream);
    launch_select_level_t<-1>(dim3((nL + 15) / 16, g.bh), ncandL + 4, stream, pq, pk, idx, g, g.L, 1, nL);
    return hipGetLastError();
  }
  for (int l = g.L - 1; l >= 1; --l) {
    const int ncand = g.K * kB;
    // one workgroup per (slice, parent), on a 1-D grid remapped so that an XCD takes consecutive parents; the
    // first descent also selects its parent's coarsest row
    const int grid = g.rows[l + 1] * g.bh;
    LaunchTimer timer(kSelect, stream);
    if (l == g.L - 1) {
      const int ldc = std::max(ncand, ncandL) + 4;
      switch (topk_mode(g.K, nL)) {
        case kMerge8:
          launch_select_level_t<kMerge8>(dim3(grid), ldc, stream, pq, pk, idx, g, l, 0, ncand);
          break;
        case kMerge16:
          launch_select_level_t<kMerge16>(dim3(grid), ldc, stream, pq, pk, idx, g, l, 0, ncand);
          break;
        default:
          launch_select_level_t<kBitwise>(dim3(grid), ldc, stream, pq, pk, idx, g, l, 0, ncand);
      }
    } else {
      launch_select_level_t<-1>(dim3(grid), ncand + 4, stream, pq, pk, idx, g, l, 0, ncand);
    }
  }
  return hipGetLastError();
}

hipError_t launch_select_exhaustive(const Geom& g, const float* pq, const float* pk, int32_t* idx1,
                                    hipStream_t stream) {
  const int grid = ((g.rows[1] + 15) / 16) * g.bh;
  LaunchTimer timer(kSelectExhaustive, stream);
  select_exhaustive<<<grid, 256, 0, stream>>>(pq, pk, idx1, g);
  return hipGetLastError();
}

}  // namespace llsa
