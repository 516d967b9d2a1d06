// entries.hpp -- the entry list of one fine query block, and its staged gather (device side).
//
// Entry set [LLSA review (pith.science, arXiv 2512.16615), "Core claim", "What carries the argument"]:
// fine query block i attends the B raw tokens of each of the K level-1 blocks in idx row i, and for
// l = 1..L_e the K level-l pooled tokens kept by its level-l ancestor unit i / B^(l-1), with logit bias
// l*ln B.  Enrichment entry e (0 <= e < K*L_e) is ordered levels 2..L_e first, then level 1.
//
// The kernels walk this list in *stages* of equal register cost (8 x 16 bytes per lane):
//   fine stage s   : raw key blocks I1[2s], I1[2s+1] (32 keys);
//   coarse stage s : 16 enrichment tokens (fp32 pyramid rows).
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

// Position within the slice's selection array of the entry behind enrichment entry e of fine block i, and
// the level offset to add to that entry: split so that a caller can copy the entry early and add the offset
// when it is used.
__device__ __forceinline__ int coarse_sel_pos(const Geom& g, int i, int e) {
  int l, s;
  coarse_entry(g, e, &l, &s);
  const int unit = i >> (4 * (l - 1));
  return (level_off(g, l) + unit) * g.K + s;
}
__device__ __forceinline__ int coarse_off(const Geom& g, int e) { return level_off(g, coarse_level(g, e)); }

// One stage of gathered rows: 8 x 16 bytes per lane.
struct Stage {
  uint4 r[8];
};

// Per-wave plan of a fine block's stages.
struct Plan {
  int nfine;     // ceil(K / 2) stages of raw key blocks
  int ncoarse;   // enrichment entries K * L_e
  int nstages;   // nfine + ceil(ncoarse / 16)
};

__device__ __forceinline__ Plan make_plan(const Geom& g) {
  Plan p;
  p.nfine = (g.K + 1) / 2;
  p.ncoarse = g.K * g.Le;
  p.nstages = p.nfine + (p.ncoarse + 15) / 16;
  return p;
}

// Fill `erow` (wave-private LDS, >= ncoarse ints) with the pyramid row of every enrichment entry of fine
// block i, so that later stages index it with an LDS read instead of a dependent global load.
__device__ __forceinline__ void stage_entry_rows(const Geom& g, const int32_t* I, int i, int ncoarse, int lane,
                                                 int* erow) {
  for (int e = lane; e < ncoarse; e += 64) erow[e] = coarse_row(g, I, i, e);
}

// Operand mappings (the k order of a dot product is free, so it is chosen for coalescing):
//   raw bf16 rows ("natural"): lane (c, g) holds dims 8g..8g+7 (MFMA step 0) and 32+8g..32+8g+7 (step 1) of
//     row c -- each 16-byte load instruction reads one contiguous 64-byte line per row;
//   fp32 pyramid rows ("coarse"): lane (c, g) holds dims 16m+4g..16m+4g+3, m = 0..3; step 0 uses m = 0, 1 and
//     step 1 uses m = 2, 3 -- again one contiguous 64-byte line per row and instruction.
// The matching B operand of a query block therefore exists in two copies (natural and coarse order).

// Natural-order operand of bf16 row `row` (elements) for this lane.
__device__ __forceinline__ void load_natural(const bf16_t* __restrict__ base, uint32_t row, int lane, uint4& s0,
                                             uint4& s1) {
  const uint32_t o = row * kD + 8u * (uint32_t)(lane >> 4);
  s0 = ld16(base + o);
  s1 = ld16(base + o + 32);
}

// Coarse-order operand of a bf16 row (four 8-byte pieces) -- used for the query-side B operand.
__device__ __forceinline__ void load_coarse_bf16(const bf16_t* __restrict__ base, uint32_t row, int lane, bf16x8& s0,
                                                 bf16x8& s1) {
  const uint32_t o = row * kD + 4u * (uint32_t)(lane >> 4);
  uint2 p[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) p[m] = *reinterpret_cast<const uint2*>(base + o + 16 * m);
  uint4 a = make_uint4(p[0].x, p[0].y, p[1].x, p[1].y), b = make_uint4(p[2].x, p[2].y, p[3].x, p[3].y);
  s0 = as_bf16x8(a);
  s1 = as_bf16x8(b);
}

// Loads of one fine stage (raw key blocks b0, b1), 32-bit lane offsets from uniform bases.
//   r[0..1], r[2..3]: natural-order K operands of rows 16*b0 + c and 16*b1 + c.
//   r[4..7], kVTile (forward; V goes to an LDS tile): instruction m reads the 1 KB of V rows 8m..8m+7 of the
//            32 keys (rows 0..15 of block b0, 16..31 of block b1): lane l gets row 8m + l/8, bytes 16*(l%8)...
//   r[4..7], !kVTile (backward; V is an A operand like K): natural-order V operands of the two blocks.
template <bool kVTile>
__device__ __forceinline__ void issue_fine(int b0, int b1, const bf16_t* __restrict__ Kraw,
                                           const bf16_t* __restrict__ Vraw, int lane, Stage& st) {
  const uint32_t c = lane & 15;
  load_natural(Kraw, 16u * b0 + c, lane, st.r[0], st.r[1]);
  load_natural(Kraw, 16u * b1 + c, lane, st.r[2], st.r[3]);
  if (kVTile) {
    const uint32_t sub = (uint32_t)lane >> 3, col = 8u * (lane & 7);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t blk = m < 2 ? b0 : b1;
      st.r[4 + m] = ld16(Vraw + (16u * blk + 8u * (m & 1) + sub) * kD + col);
    }
  } else {
    load_natural(Vraw, 16u * b0 + c, lane, st.r[4], st.r[5]);
    load_natural(Vraw, 16u * b1 + c, lane, st.r[6], st.r[7]);
  }
}

// Loads of one coarse stage (enrichment entries e0 .. e0+15; rows past the end are read in bounds and
// masked by the consumer).
//   r[0..3]: coarse-order fp32 K operand of the pyramid row of entry e0 + c (instruction m: dims 16m+4g..+3).
//   r[4..7], kVTile: instruction m reads pyramid V row of entry e0 + 4m + l/16, dims 4*(l%16)..+3.
//   r[4..7], !kVTile: coarse-order fp32 V operand of the pyramid row of entry e0 + c.
template <bool kVTile>
__device__ __forceinline__ void issue_coarse(int e0, int ncoarse, const float* __restrict__ PK,
                                             const float* __restrict__ PV, const int* erow, int lane, Stage& st) {
  const uint32_t c = lane & 15, gq = (uint32_t)lane >> 4;
  const uint32_t ko = (uint32_t)erow[min(e0 + (int)c, ncoarse - 1)] * kD + 4u * gq;
#pragma unroll
  for (int m = 0; m < 4; ++m) st.r[m] = ld16(PK + ko + 16 * m);
  if (kVTile) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int ent = min(e0 + 4 * m + (lane >> 4), ncoarse - 1);
      st.r[4 + m] = ld16(PV + (uint32_t)erow[ent] * kD + 4u * (lane & 15));
    }
  } else {
#pragma unroll
    for (int m = 0; m < 4; ++m) st.r[4 + m] = ld16(PV + ko + 16 * m);
  }
}

// Loads of stage s of the plan (fine stages first, then 16-entry coarse stages).  Both branches issue the
// same number of loads, so callers can issue unconditionally and keep exact wait counts.
template <bool kVTile>
__device__ __forceinline__ void issue_stage(const Plan& p, int s, const int32_t* I1, int K,
                                            const bf16_t* __restrict__ Kraw, const bf16_t* __restrict__ Vraw,
                                            const float* __restrict__ PK, const float* __restrict__ PV,
                                            const int* erow, int lane, Stage& st) {
  if (s < p.nfine) {
    const int b0 = I1[2 * s];
    const int b1 = (2 * s + 1 < K) ? I1[2 * s + 1] : b0;
    issue_fine<kVTile>(b0, b1, Kraw, Vraw, lane, st);
  } else {
    issue_coarse<kVTile>(16 * (s - p.nfine), p.ncoarse, PK, PV, erow, lane, st);
  }
}

// Loads of one enrichment stage in natural order (forward): 16 tokens, lane (c, g) reading token c's pyramid
// rows `prow` (rows past the end of the list duplicate a valid row and are masked by the consumer):
//   r[0..3]: K dims 8g..8g+3, 8g+4..8g+7, 32+8g..32+8g+3, 32+8g+4..32+8g+7;   r[4..7]: the same of V.
// Per instruction this touches one 128-byte line per row, as the raw bf16 loads do.
__device__ __forceinline__ void issue_coarse_nat(int prow, const float* __restrict__ PK, const float* __restrict__ PV,
                                                 int lane, Stage& st) {
  const uint32_t o = (uint32_t)prow * kD + 8u * (uint32_t)(lane >> 4);
  st.r[0] = ld16(PK + o);
  st.r[1] = ld16(PK + o + 4);
  st.r[2] = ld16(PK + o + 32);
  st.r[3] = ld16(PK + o + 36);
  st.r[4] = ld16(PV + o);
  st.r[5] = ld16(PV + o + 4);
  st.r[6] = ld16(PV + o + 32);
  st.r[7] = ld16(PV + o + 36);
}

// Natural-order fp32 operand (dims 8g..8g+7 in r[0..1], 32+8g..32+8g+7 in r[2..3]) -> two bf16x8 operands.
__device__ __forceinline__ void nat_ops(const uint4* r, bf16x8& a0, bf16x8& a1) {
  float4 f[4];
  __builtin_memcpy(f, r, 64);
  a0 = f32x8_to_bf16x8(f[0], f[1]);
  a1 = f32x8_to_bf16x8(f[2], f[3]);
}

// Coarse-order fp32 operand (4 x 16 B, dims 16m+4g..+3) -> two bf16x8 MFMA operands (steps 0 and 1).
__device__ __forceinline__ void coarse_ops(const uint4* r, bf16x8& a0, bf16x8& a1) {
  float4 f[4];
  __builtin_memcpy(f, r, 64);
  a0 = f32x8_to_bf16x8(f[0], f[1]);
  a1 = f32x8_to_bf16x8(f[2], f[3]);
}

}  // namespace llsa
