// complement.hip -- the candidates each unit scored and did not keep, per level (the complement-partition
// reading of the enrichment).
//
// Method [LLSA review (pith.science, arXiv 2512.16615), "Core claim" (KV enrichment, weights B^l) and
// "What carries the argument" (hierarchical Top-K: the coarsest level scores every block, a finer unit
// scores the B children of each block its parent kept)]: under this reading a fine query block attends, at
// every level l = 1..L_e, the level-l blocks its level-l ancestor unit scored but did not keep.  Listed here
// in scoring order (the parent's picks ascending, each block's children ascending; every block at the
// coarsest level), the kept ones left out.
//
// Design: one wavefront per (level-l unit, slice).  The unit's K picks and its parent's K picks sit in lanes
// 0..K-1; candidates go 64 at a time, one per lane, each compared with the K picks (scalar reads of the pick
// lanes), and the unkept ones are compacted in order with ballot prefix counts.  A list that comes out short
// (a selection that is not hierarchical) is padded with block 0, so the forward's reads stay in bounds.
#include "common.hpp"
#include "entries.hpp"
#include "launch.hpp"

namespace llsa {

namespace {

// grid.x = n_l units, grid.y = slice; 64 threads.
__global__ __launch_bounds__(64) void complement_lists(const int32_t* __restrict__ idx, int32_t* __restrict__ comp,
                                                       Geom g, CompGeom cm, int l) {
  const int a = blockIdx.x, slice = blockIdx.y, lane = threadIdx.x;
  const int K = g.K;
  const int32_t* I = idx + (size_t)slice * g.R * K;
  const int pick = lane < K ? I[(size_t)(g.off[l] + a) * K + lane] : -1;
  const bool top = l == g.L;
  const int par = (!top && lane < K) ? I[(size_t)(g.off[l + 1] + a / 16) * K + lane] : 0;
  const int ncand = top ? g.rows[l] : 16 * K;
  const int m = cm.m[l];
  int32_t* out = comp + (size_t)slice * cm.slice + cm.off[l] + (size_t)a * m;
  int written = 0;
  for (int x0 = 0; x0 < ncand; x0 += 64) {
    const int x = x0 + lane;
    const int cand = top ? x : 16 * __shfl(par, min(x, ncand - 1) >> 4, 64) + (x & 15);
    bool kept = false;
    for (int kk = 0; kk < K; ++kk) kept |= __builtin_amdgcn_readlane(pick, kk) == cand;
    const bool take = x < ncand && !kept;
    const uint64_t b = __ballot(take);
    const int pos = written + __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0));
    if (take && pos < m) out[pos] = cand;
    written += __popcll(b);
  }
  for (int x = written + lane; x < m; x += 64) out[x] = 0;
}

}  // namespace

hipError_t launch_complement_lists(const Geom& g, const CompGeom& cm, const int32_t* idx, int32_t* comp,
                                   hipStream_t stream) {
  for (int l = 1; l <= g.Le; ++l) {
    LaunchTimer timer(kComplement, stream);
    complement_lists<<<dim3(g.rows[l], g.bh), 64, 0, stream>>>(idx, comp, g, cm, l);
  }
  return hipGetLastError();
}

}  // namespace llsa
