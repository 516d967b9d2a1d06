// entries.hpp -- the entry list of one fine query block, and its staged gather (device side).
//
// Entry set [LLSA review (pith.science, arXiv 2512.16615), "Core claim", "What carries the argument"]:
// fine query block i attends the B raw tokens of each of the K level-1 blocks in idx row i, and for
// l = 1..L_e the K level-l pooled tokens kept by its level-l ancestor unit i / B^(l-1), with logit bias
// l*ln B.  Enrichment entry e (0 <= e < K*L_e) is ordered levels 2..L_e first, then level 1.
//
// The kernels walk this list in *stages* of 32 bf16 key rows (K and V, 8 x 16 bytes per lane):
//   fine stage s   : raw key blocks I1[2s], I1[2s+1];
//   coarse stage s : enrichment entries 32s .. 32s+31 (rows of the bf16 copy of the pooled pyramid).
// Stage s+1's loads are issued before stage s is consumed, so one stage of loads is always in flight.
#pragma once
#include "common.hpp"

namespace llsa {

__device__ __forceinline__ void coarse_entry(const Geom& g, int e, int* level, int* slot) {
  const int nhigh = g.Le >= 2 ? g.K * (g.Le - 1) : 0;
  if (e < nhigh) {
    *level = 2 + e / g.K;
    *slot = e % g.K;
  } else {
    *level = 1;
    *slot = e - nhigh;
  }
}

__device__ __forceinline__ int coarse_level(const Geom& g, int e) {
  int l, s;
  coarse_entry(g, e, &l, &s);
  return l;
}

// First pyramid row of level l (1 <= l <= L) for a per-lane l, computed as sum_{m<l} n / 16^m: indexing the
// offset array with a per-lane value would read the kernel arguments from memory inside the loop.
__device__ __forceinline__ int level_off(const Geom& g, int l) {
  int o = 0;
#pragma unroll
  for (int m = 1; m < kMaxLevels; ++m) o += m < l ? (g.n >> (4 * m)) : 0;
  return o;
}

// Pyramid row (within the slice) of enrichment entry e for fine block i.
__device__ __forceinline__ int coarse_row(const Geom& g, const int32_t* I, int i, int e) {
  int l, s;
  coarse_entry(g, e, &l, &s);
  const int unit = i >> (4 * (l - 1));  // i / B^(l-1), B = 16
  const int off = level_off(g, l);
  return off + I[(size_t)(off + unit) * g.K + s];
}

// One stage of gathered rows: 8 x 16 bytes per lane.
struct Stage {
  uint4 r[8];
};

// Per-wave plan of a fine block's stages.
struct Plan {
  int nfine;     // ceil(K / 2) stages of raw key blocks
  int ncoarse;   // enrichment entries K * L_e
  int nstages;   // nfine + ceil(ncoarse / 32)
};

__device__ __forceinline__ Plan make_plan(const Geom& g) {
  Plan p;
  p.nfine = (g.K + 1) / 2;
  p.ncoarse = g.K * g.Le;
  p.nstages = p.nfine + (p.ncoarse + 31) / 32;
  return p;
}

constexpr int kMaxCoarse = 128;  // K * L_e enrichment entries per fine block (a limit of the GPU path)

// Per-entry constants of the enrichment list -- the same for every fine block, so a workgroup computes them
// once (fill_entry_tab) and the stage loop reads them from LDS instead of re-deriving level and offsets:
//   row0[e]  first pyramid row of entry e's level;
//   pos0[e], shift[e]  the entry's position in the slice's selection array for fine block i is
//            pos0[e] + (i >> shift[e]) * K  (its ancestor unit of level l is i / B^(l-1));
//   bias[e]  the logit bias l * log2(B) = 4l in the log2 domain, -inf past the end of the list (up to 31
//            padding entries), so that the padded rows of a stage get probability exactly 0.
// Entries past the end repeat the last entry's row and position (in-bounds duplicates).
struct EntryTab {
  int row0[kMaxCoarse];
  int pos0[kMaxCoarse];
  int shift[kMaxCoarse];
  float bias[kMaxCoarse];
};

// All threads of the workgroup take part; ends with a workgroup barrier.
__device__ __forceinline__ void fill_entry_tab(const Geom& g, EntryTab& t) {
  const int ncoarse = g.K * g.Le;
  for (int e = threadIdx.x; e < kMaxCoarse; e += blockDim.x) {
    const int ec = min(e, max(ncoarse - 1, 0));
    int l, slot;
    coarse_entry(g, ec, &l, &slot);
    const int off = level_off(g, l);
    t.row0[e] = off;
    t.pos0[e] = off * g.K + slot;
    t.shift[e] = 4 * (l - 1);
    t.bias[e] = e < ncoarse ? 4.0f * (float)l : -INFINITY;
  }
  __syncthreads();
}

}  // namespace llsa
