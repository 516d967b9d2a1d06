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

__device__ __forceinline__ Plan make_plan(const Geom& g, int ncoarse) {
  Plan p;
  p.nfine = (g.K + 1) / 2;
  p.ncoarse = ncoarse;
  p.nstages = p.nfine + (p.ncoarse + 31) / 32;
  return p;
}
__device__ __forceinline__ Plan make_plan(const Geom& g) { return make_plan(g, g.K * g.Le); }

constexpr int kMaxCoarse = 128;      // K * L_e selected enrichment entries per fine block (a GPU-path limit)
constexpr int kMaxComplement = 576;  // entries of the complement reading per fine block (a GPU-path limit)

// Per-entry constants of the enrichment list -- the same for every fine block, so a workgroup computes them
// once (fill_entry_tab*) and the stage loop reads them from LDS instead of re-deriving level and offsets:
//   row0[e]  first pyramid row of entry e's level;
//   pos0[e], shift[e], stride[e]  the position of the entry's block index in its source array (the
//            selection, or the complement lists) for fine block i is pos0[e] + (i >> shift[e]) * stride[e]
//            (its ancestor unit of level l is i / B^(l-1));
//   bias[e]  the logit bias l * log2(B) = 4l in the log2 domain, -inf past the end of the list (up to 31
//            padding entries), so that the padded rows of a stage get probability exactly 0.
// Entries past the end repeat the last entry's row and position (in-bounds duplicates).
template <int kN>
struct EntryTabT {
  int row0[kN];
  int pos0[kN];
  int shift[kN];
  int stride[kN];
  float bias[kN];
};
using EntryTab = EntryTabT<kMaxCoarse>;

// Selected-token reading: entry e is slot s of level l's row of the ancestor (levels 2..L_e first, then level
// 1).  All threads of the workgroup take part; ends with a workgroup barrier.
template <int kN>
__device__ __forceinline__ void fill_entry_tab(const Geom& g, EntryTabT<kN>& t) {
  const int ncoarse = g.K * g.Le;
  for (int e = threadIdx.x; e < kN; e += blockDim.x) {
    const int ec = min(e, max(ncoarse - 1, 0));
    int l, slot;
    coarse_entry(g, ec, &l, &slot);
    const int off = level_off(g, l);
    t.row0[e] = off;
    t.pos0[e] = off * g.K + slot;
    t.shift[e] = 4 * (l - 1);
    t.stride[e] = g.K;
    t.bias[e] = e < ncoarse ? 4.0f * (float)l : -INFINITY;
  }
  __syncthreads();
}

// Layout of the complement lists (one slice): level l = 1..L_e holds, for each of its n_l units, the m_l
// candidates the unit scored and did not keep, at off[l] + unit * m_l.
struct CompGeom {
  int total;                 // sum_l m_l: entries per fine block
  int slice;                 // ints per slice
  int m[kMaxLevels + 1];     // m_l
  int off[kMaxLevels + 1];   // first int of level l
};

// Complement reading: entry e is item x of level l's list of the ancestor, levels 1..L_e in order.
template <int kN>
__device__ __forceinline__ void fill_entry_tab_complement(const Geom& g, const CompGeom& cm, EntryTabT<kN>& t) {
  for (int e = threadIdx.x; e < kN; e += blockDim.x) {
    const int ec = min(e, max(cm.total - 1, 0));
    int l = 1, start = 0;
    while (l < g.Le && ec >= start + cm.m[l]) start += cm.m[l++];
    t.row0[e] = level_off(g, l);
    t.pos0[e] = cm.off[l] + (ec - start);
    t.shift[e] = 4 * (l - 1);
    t.stride[e] = cm.m[l];
    t.bias[e] = e < cm.total ? 4.0f * (float)l : -INFINITY;
  }
  __syncthreads();
}

}  // namespace llsa
