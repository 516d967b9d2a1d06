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
//     level uses the same kernel with "all n_L blocks" as the candidate list, 16 query units per
//     workgroup.
//   * Top-K per query row without sorting: a 32-step bitwise search for the K-th largest
//     order-preserving score key (one compare + one ballot per slot group and step, the group count a
//     compile-time constant), then ties at the threshold are
//     taken in ascending slot order and the kept slots are compacted in ascending order with ballot
//     prefix counts -- candidate slots ascend with block index, so this realises the tie rule and the
//     ascending row order directly.
#include "common.hpp"
#include "launch.hpp"

namespace llsa {

namespace {

constexpr int kMaxSlotsPerLane = 8;  // up to 512 candidates per query row

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
// ballot per step), ties at the threshold taken in ascending slot order, kept slots compacted in ascending
// order with ballot prefix counts.  Candidate slots ascend with block index, so this realises the tie rule
// and the ascending row order directly.  Wave w handles rows 4w .. 4w+3.
// kM = ceil(ncand / 64) slot groups per lane, a compile-time constant so that the 32 search steps carry no
// per-group branches.
template <int kM>
__device__ __forceinline__ void topk_rows(const float* sc, int ldc, int ncand, int nq, int K, int w, int lane,
                                          int32_t* out_rows, const int32_t* picks, int coarsest) {
  for (int rr = 0; rr < 4; ++rr) {
    const int row = 4 * w + rr;
    if (row >= nq) break;
    uint32_t key[kM];
#pragma unroll
    for (int m = 0; m < kM; ++m) {
      const int s = lane + 64 * m;
      // invalid slots (beyond the candidate count or past the last level-L block) get key 0, below
      // every real score's key (the smallest, -inf, maps to 0x007FFFFF)
      key[m] = s < ncand ? ord_key(sc[row * ldc + s]) : 0u;
    }
    // K-th largest key by bitwise search: largest T with #{key >= T} >= K
    uint32_t T = 0;
#pragma unroll 4
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = T | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int m = 0; m < kM; ++m) cnt += popc64(__ballot(key[m] >= cand));
      T = cnt >= K ? cand : T;
    }
    int greater = 0;
#pragma unroll
    for (int m = 0; m < kM; ++m) greater += popc64(__ballot(key[m] > T));
    const int need = K - greater;  // ties at T to take, lowest slots first
    int eq_before = 0, sel_before = 0;
    int32_t* out = out_rows + (size_t)row * K;
#pragma unroll
    for (int m = 0; m < kM; ++m) {
      {
        const uint64_t eqm = __ballot(key[m] == T);
        const bool sel_eq = (key[m] == T) && (eq_before + lanes_below(eqm) < need);
        const bool sel = (key[m] > T) || sel_eq;
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
}

__device__ __forceinline__ void topk_dispatch(const float* sc, int ldc, int ncand, int nq, int K, int w, int lane,
                                              int32_t* out_rows, const int32_t* picks, int coarsest) {
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

// Coarsest: grid.x = 16-row query tiles, grid.y = slice.  Descent: 1-D grid over (slice, parent unit at
// level+1), remapped so that consecutive parents run on one XCD and its L2 holds their slices' pooled keys.
// Dynamic LDS: 16 rows x ldc floats of scores.
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
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, c = lane & 15, gg = lane >> 4;
  const float* PQ = pq + (size_t)slice * g.R * kD;
  const float* PK = pk + (size_t)slice * g.R * kD;
  int32_t* I = idx + (size_t)slice * g.R * g.K;
  const int nl = g.rows[level];
  const int q0 = 16 * bx;
  const int nq = coarsest ? min(16, nl - q0) : 16;
  const int32_t* picks = coarsest ? nullptr : I + (size_t)(g.off[level + 1] + bx) * g.K;
  const int ntiles = (ncand + 15) / 16;

  // A operand: this lane's query row (q0 + c), dims 16*gg .. 16*gg+15 (step s uses dim 16*gg + s).
  float qf[16];
  {
    const bool ok = c < nq;
    const float4* src = reinterpret_cast<const float4*>(PQ + (size_t)(g.off[level] + q0 + (ok ? c : 0)) * kD + 16 * gg);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float4 x = ok ? src[m] : make_float4(0, 0, 0, 0);
      qf[4 * m] = x.x; qf[4 * m + 1] = x.y; qf[4 * m + 2] = x.z; qf[4 * m + 3] = x.w;
    }
  }
  for (int t = w; t < ntiles; t += 4) {
    int j;  // candidate block index (row within the level) for this lane's column c
    bool valid;
    if (coarsest) {
      j = 16 * t + c;
      valid = j < nl;
    } else {
      j = picks[t] * kB + c;
      valid = true;
    }
    float kf[16];
    const float4* src = reinterpret_cast<const float4*>(PK + (size_t)(g.off[level] + (valid ? j : 0)) * kD + 16 * gg);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float4 x = src[m];
      kf[4 * m] = x.x; kf[4 * m + 1] = x.y; kf[4 * m + 2] = x.z; kf[4 * m + 3] = x.w;
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 16; ++s) acc = mfma_f32_k4(qf[s], kf[s], acc);
    // acc[r] = score(query row 4*gg + r, candidate slot 16*t + c)
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[(4 * gg + r) * ldc + 16 * t + c] = valid ? acc[r] : -INFINITY;
  }
  __syncthreads();

  topk_dispatch(sc, ldc, ncand, nq, g.K, w, lane, I + (size_t)(g.off[level] + q0) * g.K, picks, coarsest);
}

}  // namespace

hipError_t launch_select(const Geom& g, const float* pq, const float* pk, int32_t* idx, hipStream_t stream) {
  // coarsest level: all n_L blocks are candidates
  {
    const int nL = g.rows[g.L];
    const int ncand = ((nL + 15) / 16) * 16;
    const int ldc = ncand + 4;
    dim3 grid((nL + 15) / 16, g.bh);
    LaunchTimer timer(kSelect, stream);
    select_level<<<grid, 256, 16 * ldc * sizeof(float), stream>>>(pq, pk, idx, g, g.L, 1, nL, ldc);
  }
  for (int l = g.L - 1; l >= 1; --l) {
    const int ncand = g.K * kB;
    const int ldc = ncand + 4;
    // one workgroup per (slice, parent), on a 1-D grid remapped so that an XCD takes consecutive parents
    const int grid = g.rows[l + 1] * g.bh;
    LaunchTimer timer(kSelect, stream);
    select_level<<<grid, 256, 16 * ldc * sizeof(float), stream>>>(pq, pk, idx, g, l, 0, ncand, ldc);
  }
  return hipGetLastError();
}

}  // namespace llsa
