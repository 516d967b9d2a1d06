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
//
// Backward of the pooled tokens under this reading (comp_partial, comp_reduce).  A level-l pooled token c is an
// entry of every query whose level-l unit scored c and did not keep it.  Group the queries by "units" u of 16
// fine blocks (256 queries; the level-2 units when L >= 2): for l < L all of u's level-l units score the same
// candidates -- the B children of each block kept by u's level-(l+1) ancestor p -- and at the coarsest level
// every unit scores all n_L blocks.  comp_partial runs u's 256 queries against those candidates densely (MFMA,
// 16 candidates per wave), with P = 0 where the query's level-l unit kept the candidate, and writes each
// candidate's partial dK, dV (fp32) for u.  comp_reduce then sums, for every pooled token c, the partials of
// the units whose candidates hold it, in a fixed order: for l < L those under the level-(l+1) units that kept
// c's parent (the level-(l+1) CSC column of c / B), at the coarsest level all units.
#include "common.hpp"
#include "entries.hpp"
#include "launch.hpp"
#include "persist.hpp"

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

// Partials of unit u (grid.x) of slice grid.y; 256 threads.  Wave w takes candidates 16 w .. 16 w + 15 of each
// 64-candidate tile; lane (c, g): candidate c of the wave, MFMA row group g.
__global__ __launch_bounds__(256, 2) void comp_partial(const bf16_t* __restrict__ q, const bf16_t* __restrict__ dout,
                                                       const float* __restrict__ lse, const float* __restrict__ delta,
                                                       const bf16_t* __restrict__ pk, const bf16_t* __restrict__ pv,
                                                       const int32_t* __restrict__ idx, float* __restrict__ part,
                                                       Geom g, PartGeom pg) {
  __shared__ __attribute__((aligned(16))) bf16_t qs[16][16 * kD];  // Q rows of the unit's 16 fine blocks (swizzled)
  __shared__ __attribute__((aligned(16))) bf16_t dos[16][16 * kD]; // dO rows (swizzled)
  __shared__ __attribute__((aligned(16))) float ls[256];           // LSE * log2(e)
  __shared__ __attribute__((aligned(16))) float dl[256];           // Delta
  __shared__ int pick1[16][32];                                      // level-1 picks of each fine block
  const int u = blockIdx.x, slice = blockIdx.y;
  const int lane = threadIdx.x & 63, c = lane & 15, gq = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n1 = g.rows[1], K = g.K;
  const int nb = min(16, n1 - 16 * u);  // fine blocks of this unit (fewer only in a ragged last unit, L = 1)
  const size_t qbase = ((size_t)slice * g.n + (size_t)256 * u) * kD;
  for (int j = w; j < nb; j += 4) {
    const size_t r = qbase + (size_t)16 * j * kD + swz_dma_src(lane);
    lds_dma16(q + r, &qs[j][0]);
    lds_dma16(q + r + 8 * kD, &qs[j][8 * kD]);
    lds_dma16(dout + r, &dos[j][0]);
    lds_dma16(dout + r + 8 * kD, &dos[j][8 * kD]);
  }
  const int t = threadIdx.x;
  if (t < 16 * nb) {
    ls[t] = lse[(size_t)slice * g.n + 256 * u + t] * kLog2e;
    dl[t] = delta[(size_t)slice * g.n + 256 * u + t];
  }
  const int32_t* I = idx + (size_t)slice * g.R * K;
  for (int x = t; x < nb * K; x += 256) pick1[x / K][x % K] = I[(size_t)(g.off[1] + 16 * u + x / K) * K + x % K];
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  const int c7 = c & 7;
  const int a0 = c * kD + ((gq ^ c7) << 3), a1 = c * kD + (((4 + gq) ^ c7) << 3);
  const int trr = 4 * gq + (c >> 2);
  const float sl2 = g.scale_log2;
  float* P0 = part + ((size_t)slice * pg.n2u + u) * pg.nc * (2 * kD);
  for (int l = 1; l <= g.Le; ++l) {
    const bool top = l == g.L;
    const int ncand = pg.ncand[l];
    const float bias = 4.0f * (float)l;  // l * log2(B) in the log2 domain
    const int p = (16 * u) >> (4 * l);                  // level-(l+1) unit holding u (l < L)
    const int a = l >= 2 ? (16 * u) >> (4 * (l - 1)) : 0;  // level-l unit of all of u's queries (l >= 2)
    for (int x0 = 0; x0 < ncand; x0 += 64) {
      const int x = x0 + 16 * w + c;
      const bool xv = x < ncand;
      int cb = 0;  // candidate block (row within level l)
      if (xv) cb = top ? x : kB * I[(size_t)(g.off[l + 1] + p) * K + (x >> 4)] + (x & 15);
      // B operands: the candidate's pooled K, V rows (bf16 copies), dims 8g .. 8g+7 and 32 + 8g ..
      const size_t rowp = ((size_t)slice * g.R + g.off[l] + cb) * kD + 8 * gq;
      const bf16x8 kb0 = as_bf16x8(ld16(pk + rowp)), kb1 = as_bf16x8(ld16(pk + rowp + 32));
      const bf16x8 vb0 = as_bf16x8(ld16(pv + rowp)), vb1 = as_bf16x8(ld16(pv + rowp + 32));
      // kept[j]: the query block's level-l unit kept the candidate (no entry); invalid slots likewise
      uint32_t kept = xv ? 0u : 0xFFFFu;
      if (xv) {
        if (l == 1) {
          for (int j = 0; j < nb; ++j)
            for (int k = 0; k < K; ++k) kept |= (uint32_t)(pick1[j][k] == cb) << j;
        } else {
          bool kk = false;
          for (int k = 0; k < K; ++k) kk |= I[(size_t)(g.off[l] + a) * K + k] == cb;
          kept = kk ? 0xFFFFu : 0u;
        }
      }
      f32x4 dk_acc[4], dv_acc[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) dk_acc[tt] = dv_acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int j = 0; j < nb; ++j) {
        const bf16_t* qt = qs[j];
        const bf16_t* dt = dos[j];
        const bf16x8 qa0 = *reinterpret_cast<const bf16x8*>(qt + a0), qa1 = *reinterpret_cast<const bf16x8*>(qt + a1);
        const bf16x8 da0 = *reinterpret_cast<const bf16x8*>(dt + a0), da1 = *reinterpret_cast<const bf16x8*>(dt + a1);
        f32x4 sx = {0.f, 0.f, 0.f, 0.f}, dpv = {0.f, 0.f, 0.f, 0.f};
        sx = mfma_bf16_k32(qa0, kb0, sx);
        sx = mfma_bf16_k32(qa1, kb1, sx);
        dpv = mfma_bf16_k32(da0, vb0, dpv);
        dpv = mfma_bf16_k32(da1, vb1, dpv);
        // sx[r] = S[query 4g + r of block j][candidate c]
        const float4 l4 = *reinterpret_cast<const float4*>(&ls[16 * j + 4 * gq]);
        const float4 d4 = *reinterpret_cast<const float4*>(&dl[16 * j + 4 * gq]);
        const float lq[4] = {l4.x, l4.y, l4.z, l4.w}, dq4[4] = {d4.x, d4.y, d4.z, d4.w};
        const bool off = (kept >> j) & 1u;
        float pr[4], ds[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pr[r] = off ? 0.f : fast_exp2(sx[r] * sl2 + bias - lq[r]);
          ds[r] = pr[r] * (dpv[r] - dq4[r]);
        }
        bf16x4 pb, db;
        {
          const uint2 up = make_uint2(pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]));
          const uint2 ud = make_uint2(pack_bf16x2(ds[0], ds[1]), pack_bf16x2(ds[2], ds[3]));
          __builtin_memcpy(&pb, &up, 8);
          __builtin_memcpy(&db, &ud, 8);
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const int xo = swz(trr, 16 * tt + 4 * (c & 3));
          dv_acc[tt] = mfma_bf16_k16(lds_read_tr16(dt + xo), pb, dv_acc[tt]);
          dk_acc[tt] = mfma_bf16_k16(lds_read_tr16(qt + xo), db, dk_acc[tt]);
        }
      }
      // lane holds d = 16 tt + 4 g + r of candidate c: partial row [K dims | V dims]
      if (xv) {
        float* P = P0 + (size_t)(pg.xoff[l] + x) * (2 * kD);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          *reinterpret_cast<f32x4*>(P + 16 * tt + 4 * gq) = dk_acc[tt] * g.scale;
          *reinterpret_cast<f32x4*>(P + kD + 16 * tt + 4 * gq) = dv_acc[tt];
        }
      }
    }
  }
}

// Pooled-token gradient of token grid.x (levels 1..L_e concatenated) of slice grid.y; 64 threads, thread = dim.
__global__ __launch_bounds__(64) void comp_reduce(const int32_t* __restrict__ col_ptr, const int32_t* __restrict__ perm,
                                                  const float* __restrict__ part, float* __restrict__ gk,
                                                  float* __restrict__ gv, Geom g, CscGeom cg, PartGeom pg) {
  const int slice = blockIdx.y, d = threadIdx.x;
  int l = 1, cb = blockIdx.x;
  while (l < g.Le && cb >= g.rows[l]) cb -= g.rows[l++];
  const float* Pb = part + (size_t)slice * pg.n2u * pg.nc * (2 * kD) + (size_t)pg.xoff[l] * (2 * kD) + d;
  const size_t ustride = (size_t)pg.nc * (2 * kD);
  float sk = 0.f, sv = 0.f;
  if (l == g.L) {
    for (int u = 0; u < pg.n2u; ++u) {
      const float* P = Pb + u * ustride + (size_t)cb * (2 * kD);
      sk += P[0];
      sv += P[kD];
    }
  } else {
    const int par = cb >> 4, x = cb & 15;
    const int32_t* cp = col_ptr + (size_t)slice * cg.cp_len + cg.cp_off[l + 1];
    const int32_t* pm = perm + (size_t)slice * cg.pm_len + cg.pm_off[l + 1];
    const int span = 1 << (4 * (l - 1));  // units u under one level-(l+1) unit
    for (int e = cp[par]; e < cp[par + 1]; ++e) {
      const int pos = pm[e], p = pos / g.K, k = pos - p * g.K;
      const int u1 = min((p + 1) * span, pg.n2u);
      for (int u = p * span; u < u1; ++u) {
        const float* P = Pb + u * ustride + (size_t)(16 * k + x) * (2 * kD);
        sk += P[0];
        sv += P[kD];
      }
    }
  }
  const size_t o = ((size_t)slice * g.R + g.off[l] + cb) * kD + d;
  gk[o] = sk;
  gv[o] = sv;
}

}  // namespace

hipError_t launch_comp_grads(const Geom& g, const CscGeom& cg, const PartGeom& pg, const void* q, const void* dout,
                             const float* lse, const float* delta, const void* pk, const void* pv,
                             const int32_t* idx, const int32_t* col_ptr, const int32_t* perm, float* part,
                             float* gk, float* gv, hipStream_t stream) {
  if (g.Le < 1) return hipGetLastError();
  LaunchTimer timer(kBwdReduce, stream);
  comp_partial<<<dim3(pg.n2u, g.bh), 256, 0, stream>>>((const bf16_t*)q, (const bf16_t*)dout, lse, delta,
                                                       (const bf16_t*)pk, (const bf16_t*)pv, idx, part, g, pg);
  int tokens = 0;
  for (int l = 1; l <= g.Le; ++l) tokens += g.rows[l];
  comp_reduce<<<dim3(tokens, g.bh), 64, 0, stream>>>(col_ptr, perm, part, gk, gv, g, cg, pg);
  return hipGetLastError();
}

hipError_t launch_complement_lists(const Geom& g, const CompGeom& cm, const int32_t* idx, int32_t* comp,
                                   hipStream_t stream) {
  for (int l = 1; l <= g.Le; ++l) {
    LaunchTimer timer(kComplement, stream);
    complement_lists<<<dim3(g.rows[l], g.bh), 64, 0, stream>>>(idx, comp, g, cm, l);
  }
  return hipGetLastError();
}

}  // namespace llsa
