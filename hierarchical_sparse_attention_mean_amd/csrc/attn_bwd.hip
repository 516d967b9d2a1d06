// attn_bwd.hip -- backward of the enriched sparse block attention (bf16, MFMA).
//
// Method [LLSA review (pith.science, arXiv 2512.16615), "If this is right" (the backward pass uses only
// the sparse indices), "What carries the argument" (CSR-to-CSC transpose gives each key block its
// query blocks), "Core claim" (enrichment tokens are mean-pooled, weight B^l)]:
//   Delta_t = dO_t . O_t;  for every entry e of query t with P = exp(z_e - lse_t):
//   dV_e += P dO_t,  dS = P (dO_t . v_e - Delta_t),  dQ_t += sigma dS k_e,  dK_e += sigma dS q_t.
//   Pooled level-l tokens pass their gradient to the B^l raw tokens they average with factor B^-l.
//
// Kernels, in stream order:
//   1. bwd_dq (Q-major, each wavefront owning whole level-2 units and running their 16 fine blocks in
//      turn): recomputes P over fine and enrichment entries, writes dQ and Delta, and -- because all 256
//      queries of a level-2 unit share the enrichment tokens of levels >= 2 -- accumulates their dK^(l),
//      dV^(l) contributions for the unit in registers and stores them at the unit's end (partials per
//      level-2 unit and slot).
//   2. reduce_and_order: for each pooled token of levels >= 2, sums the partials of the (unit, slot) pairs
//      that kept it, found through that level's CSC column (no atomics); beside it, in the same launch, the
//      dK/dV work lists (dkdv_order's job, which needs only the CSC).
//   3. bwd_dkdv (K-major, one wavefront per work item: a group of four key blocks, or a
//      chunk of a long group's stages): walks the key blocks' CSC columns of level 1 -- the query blocks that
//      kept them -- and accumulates dK, dV for their keys.  The same query blocks are exactly those that
//      attend a block's level-1 pooled token, so that token's gradient (scaled by B^-1) is folded into the
//      same products, and the B^-l share of the level >= 2 tokens is added before the bf16 store.  Chunks of
//      a split group write fp32 partials; the last chunk to finish adds them in chunk order.
// The complement reading of the enrichment (launch_attn_bwd_complement) runs bwd_dq over the complement
// lists, its pooled-token gradients in complement.hip, and bwd_dkdv without the level-1 fold.
// Every gradient element is summed in a fixed order: no floating-point atomics, bitwise reproducible (the
// only atomic is the integer count of a split group's finished chunks).
#include "common.hpp"
#include "entries.hpp"
#include "launch.hpp"
#include "persist.hpp"

namespace llsa {

namespace {

constexpr int kLd = kD + 8;   // bf16 row stride of K / Q / dO tiles in LDS

__device__ __forceinline__ float dot16_bf16(uint4 a0, uint4 a1, uint4 b0, uint4 b1) {
  const uint32_t x[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
  const uint32_t y[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    s += __uint_as_float(x[e] << 16) * __uint_as_float(y[e] << 16);
    s += __uint_as_float(x[e] & 0xFFFF0000u) * __uint_as_float(y[e] & 0xFFFF0000u);
  }
  return s;
}

__device__ __forceinline__ bf16x4 pack4(float a, float b, float c, float d) {
  const uint2 u = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
  bf16x4 r;
  __builtin_memcpy(&r, &u, 8);
  return r;
}

// ------------------------------------------------------------------------------------------------
// 1. dQ, Delta and the level >= 2 pooled-token partials.
// Persistent: grid = 8 * (workgroups resident per XCD), 256 threads.  Each wave takes level-2 units (16 fine
// blocks each) from its XCD's sweep (wave slot 4 * (b / 8) + w) and runs their blocks in order (ragged units
// run clamped dummy blocks whose results are dropped); its stage list is the concatenation of those blocks'
// stages, the next block's first stage in flight while the current one finishes.  A unit's pooled-token
// partials stay in the wave's registers and are stored when its last block ends: the waves of a workgroup never
// wait for each other (four waves sharing a unit and summing their partials through LDS made the step 13.5 us
// slower at N = 65536, most of it waves waiting at the unit ends).  A block's
// Q, dO, O rows, LSE and indices are copied to LDS a whole block ahead (LDS DMA).  Gathered K / V / pyramid
// rows are loaded coalesced (issue_stage_coalesced) and reordered through swizzled LDS tiles.
// ------------------------------------------------------------------------------------------------
constexpr int kSt = 16 + 8;      // bf16 row stride of the dS^T / P^T tiles (entry rows x 16 queries)

// kT: 16-entry tiles of level >= 2 enrichment entries whose partials are held in registers (K*(L_e-1) <= 16 kT).
// kMaxC, kComp: as in the forward -- the complement reading takes its enrichment entries from the complement
// lists `esrc` (laid out by `cm`) and leaves the pooled-token gradients to comp_partial.
template <int kT, int kMaxC, bool kComp>
__global__ __launch_bounds__(256, 2) void bwd_dq_bf16(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                      const bf16_t* __restrict__ v, const bf16_t* __restrict__ o,
                                                      const float* __restrict__ lse, const bf16_t* __restrict__ dout,
                                                      const bf16_t* __restrict__ pk, const bf16_t* __restrict__ pv,
                                                      const int32_t* __restrict__ idx, bf16_t* __restrict__ dq,
                                                      float* __restrict__ delta, float* __restrict__ part_k,
                                                      float* __restrict__ part_v, const int32_t* __restrict__ esrc,
                                                      Geom g, CompGeom cm) {
  __shared__ __attribute__((aligned(16))) bf16_t kvts[2][4][32 * kD];  // K tiles, then V tiles (swizzled)
  __shared__ __attribute__((aligned(16))) bf16_t qsl[4][2][16 * kD];   // Q rows, two slots (swizzled)
  __shared__ __attribute__((aligned(16))) bf16_t dsl[4][2][16 * kD];   // dO rows, two slots (swizzled)
  __shared__ __attribute__((aligned(16))) bf16_t osl[4][16 * kD];      // O rows of the next block (swizzled)
  __shared__ __attribute__((aligned(16))) float lsl[4][2][16];         // LSE of the block's queries
  __shared__ __attribute__((aligned(16))) int is1[4][2][32];           // level-1 selection row
  __shared__ __attribute__((aligned(16))) int es[4][2][kMaxC];         // enrichment entries' block indices
  __shared__ __attribute__((aligned(16))) EntryTabT<kMaxC> tab;        // per-entry constants (shared)
  const int lane = threadIdx.x & 63, c = lane & 15, gq = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (kComp)
    fill_entry_tab_complement(g, cm, tab);
  else
    fill_entry_tab(g, tab);
  const int n1 = g.rows[1];
  const int gps = (n1 + 15) / 16;
  const Sweep su = xcd_sweep(g.bh * gps, 4 * (blockIdx.x / 8) + w, 4 * (gridDim.x / 8));  // units of this wave
  if (su.count == 0) return;  // no workgroup barrier is used below
  const int nblk = 16 * su.count;
  bf16_t* kt = kvts[0][w];
  bf16_t* vt = kvts[1][w];
  const Plan plan = make_plan(g, kComp ? cm.total : g.K * g.Le);
  const int nst = plan.nstages;
  const int nhigh = (!kComp && g.Le >= 2) ? g.K * (g.Le - 1) : 0;
  const size_t slice_elems = (size_t)g.n * kD, slice_rows = (size_t)g.R * kD;
  const size_t esrc_slice = kComp ? (size_t)cm.slice : (size_t)g.R * g.K;
  const float sl2 = g.scale_log2;

  struct Blk {
    int slice, u2, i;
    bool valid;
  };
  // the wave's j-th block (clamped to the last)
  auto blk = [&](int j) {
    const int jc = min(j, nblk - 1);
    const int U = su.first + su.stride * (jc >> 4);
    Blk b;
    b.slice = uniform(U / gps);
    b.u2 = U - b.slice * gps;
    const int i = 16 * b.u2 + (jc & 15);
    b.valid = i < n1;
    b.i = min(i, n1 - 1);
    return b;
  };
  // copy the inputs of the wave's j-th block into slot p (O: the single O slot)
  auto prefetch = [&](int j, int p) {
    const Blk b = blk(j);
    const size_t rb = b.slice * slice_elems + (size_t)16 * b.i * kD + swz_dma_src(lane);
    lds_dma16_nt(q + rb, &qsl[w][p][0]);
    lds_dma16_nt(q + rb + 8 * kD, &qsl[w][p][8 * kD]);
    lds_dma16_nt(dout + rb, &dsl[w][p][0]);
    lds_dma16_nt(dout + rb + 8 * kD, &dsl[w][p][8 * kD]);
    lds_dma16_nt(o + rb, &osl[w][0]);
    lds_dma16_nt(o + rb + 8 * kD, &osl[w][8 * kD]);
    if (lane < 16) lds_dma4(lse + (size_t)b.slice * g.n + 16 * b.i + lane, &lsl[w][p][0]);
    const int32_t* I = idx + (size_t)b.slice * g.R * g.K;
    if (lane < g.K) lds_dma4(I + (size_t)(g.off[1] + b.i) * g.K + lane, &is1[w][p][0]);
    const int32_t* E = esrc + b.slice * esrc_slice;
#pragma unroll
    for (int jj = 0; jj < kMaxC / 64; ++jj) {
      if (64 * jj < plan.ncoarse) {
        const int e = min(lane + 64 * jj, plan.ncoarse - 1);
        lds_dma4(E + tab.pos0[e] + (b.i >> tab.shift[e]) * tab.stride[e], &es[w][p][64 * jj]);
      }
    }
  };
  auto issue = [&](int p, int slice, int s, Stage& st) {
    issue_stage_coalesced(plan, s, g.K, is1[w][p], es[w][p], tab.row0, k + slice * slice_elems,
                          v + slice * slice_elems, pk + slice * slice_rows, pv + slice * slice_rows, lane, st);
  };

  int par = 0;   // slot of the block being consumed
  int cj = 0, cs = 0;
  int ij = 0, is = 0;
  Blk cur = blk(0), nxt = blk(1);
  float dlt = 0.f, lse2 = 0.f;
  // B operands (natural order) of the current block's Q and dO rows, read from their slots at block start
  bf16x8 qa0, qa1, da0, da1;
  f32x4 dq_acc[4], gk_acc[kT][4], gv_acc[kT][4];
#pragma unroll
  for (int T = 0; T < kT; ++T)
#pragma unroll
    for (int t = 0; t < 4; ++t) gk_acc[T][t] = gv_acc[T][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // start of block cj (inputs in slot par): B operands, Delta, LSE; then the next block's copies
  auto begin_block = [&]() {
    const int c7 = c & 7;
    const bf16_t* qr = &qsl[w][par][c * kD];
    const bf16_t* dr = &dsl[w][par][c * kD];
    const bf16_t* orr = &osl[w][c * kD];
    const uint4 d0 = *reinterpret_cast<const uint4*>(dr + ((gq ^ c7) << 3));
    const uint4 d1 = *reinterpret_cast<const uint4*>(dr + (((4 + gq) ^ c7) << 3));
    const uint4 o0 = *reinterpret_cast<const uint4*>(orr + ((gq ^ c7) << 3));
    const uint4 o1 = *reinterpret_cast<const uint4*>(orr + (((4 + gq) ^ c7) << 3));
    qa0 = *reinterpret_cast<const bf16x8*>(qr + ((gq ^ c7) << 3));
    qa1 = *reinterpret_cast<const bf16x8*>(qr + (((4 + gq) ^ c7) << 3));
    da0 = as_bf16x8(d0);
    da1 = as_bf16x8(d1);
    lse2 = lsl[w][par][c] * kLog2e;
    wait_lds();  // the O slot is refilled below
    dlt = group_sum(dot16_bf16(d0, d1, o0, o1));
    if (cur.valid && gq == 0) delta[(size_t)cur.slice * g.n + 16 * cur.i + c] = dlt;
    prefetch(cj + 1, par ^ 1);
#pragma unroll
    for (int t = 0; t < 4; ++t) dq_acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  auto issue_next = [&](Stage& st) {
    if (++is == nst) {
      is = 0;
      ++ij;
    }
    if (ij >= nblk) {
      issue(par, cur.slice, nst - 1, st);  // past the end: an in-bounds reload that is never consumed
    } else if (is == 0) {
      // first stage of the next block: its indices were copied at the start of the current block, and every
      // stage issued since (nst - 1 of them) is newer
      if (nst >= 2)
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      issue(par ^ 1, nxt.slice, 0, st);
    } else {
      issue(par, cur.slice, is, st);
    }
  };

  // dQ^T += K^T dS^T over the stage's 32 keys (key order of the S tiles), K^T read transposed
  auto dq_32 = [&](const float ds[8]) {
    uint4 u;
    u.x = pack_bf16x2(ds[0], ds[1]);
    u.y = pack_bf16x2(ds[2], ds[3]);
    u.z = pack_bf16x2(ds[4], ds[5]);
    u.w = pack_bf16x2(ds[6], ds[7]);
    const bf16x8 db = as_bf16x8(u);
    const int r = 4 * gq + (c >> 2);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int col = 16 * t + 4 * (c & 3);
      const bf16x8 ka = cat4(lds_read_tr16(kt + swz(r, col)), lds_read_tr16(kt + swz(r + 16, col)));
      dq_acc[t] = mfma_bf16_k32(ka, db, dq_acc[t]);
    }
  };

  // One stage of 32 keys (two fine blocks, or 32 enrichment entries): K and V rows into the swizzled tiles,
  // S^T = K Q^T and dP^T = V dO^T per 16-key half, P = 2^(S sigma log2e + bias - LSE) with the stage's bias (fine:
  // 0, or -inf for a missing second block; enrichment: 4l per entry, -inf past the end of the list),
  // dS = P (dP - Delta), then dQ.  The first enrichment stage also holds the level >= 2 entries (at most 32).
  auto consume_stage = [&](const Stage& st) {
    {
      const int r = lane >> 3, ch = lane & 7;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int o2 = (8 * m + r) * kD + ((ch ^ r) << 3);
        *reinterpret_cast<uint4*>(kt + o2) = st.r[m];
        *reinterpret_cast<uint4*>(vt + o2) = st.r[4 + m];
      }
    }
    const bool coarse = cs >= plan.nfine;
    float bb[8];
    if (!coarse) {
      const float h1 = 2 * cs + 1 < g.K ? -lse2 : -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        bb[r] = -lse2;
        bb[4 + r] = h1;
      }
    } else {
      const int e0 = 32 * (cs - plan.nfine) + 4 * gq;
      const float4 b0 = *reinterpret_cast<const float4*>(&tab.bias[e0]);
      const float4 b1 = *reinterpret_cast<const float4*>(&tab.bias[e0 + 16]);
      bb[0] = b0.x - lse2; bb[1] = b0.y - lse2; bb[2] = b0.z - lse2; bb[3] = b0.w - lse2;
      bb[4] = b1.x - lse2; bb[5] = b1.y - lse2; bb[6] = b1.z - lse2; bb[7] = b1.w - lse2;
    }
    const int c7 = c & 7;
    const int a0 = c * kD + ((gq ^ c7) << 3), a1 = c * kD + (((4 + gq) ^ c7) << 3);
    float ds[8], pr[8];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const int ro = 16 * kD * t2;
      const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(kt + ro + a0), k1 = *reinterpret_cast<const bf16x8*>(kt + ro + a1);
      const bf16x8 v0 = *reinterpret_cast<const bf16x8*>(vt + ro + a0), v1 = *reinterpret_cast<const bf16x8*>(vt + ro + a1);
      f32x4 sx = {0.f, 0.f, 0.f, 0.f}, dpv = {0.f, 0.f, 0.f, 0.f};
      sx = mfma_bf16_k32(k0, qa0, sx);
      sx = mfma_bf16_k32(k1, qa1, sx);
      dpv = mfma_bf16_k32(v0, da0, dpv);
      dpv = mfma_bf16_k32(v1, da1, dpv);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2(fmaf(sx[r], sl2, bb[4 * t2 + r]));
        pr[4 * t2 + r] = p;
        ds[4 * t2 + r] = p * (dpv[r] - dlt);
      }
    }
    dq_32(ds);
    if (coarse && cs == plan.nfine && nhigh > 0 && cur.valid) {
      // entries of levels >= 2 (shared by the unit's 256 queries), 16-entry tile T = entries 16T .. 16T+15:
      // dK^(l)[e] += sum_q dS^T[e][q] q and dV^(l)[e] += sum_q P^T[e][q] dO over this block's 16 queries
      // (16x16x16, k = query); dS^T and P^T go through a small tile in the V tile's space, whose operand reads
      // are complete
      bf16_t* sttile = vt;
      bf16_t* pttile = vt + 16 * kSt;
      const bf16_t* qtile = qsl[w][par];
      const bf16_t* dtile = dsl[w][par];
      const int r = 4 * gq + (c >> 2);
#pragma unroll
      for (int T = 0; T < kT; ++T) {
        if (16 * T < nhigh) {
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            sttile[(4 * gq + rr) * kSt + c] = f32_to_bf16(ds[4 * T + rr]);
            pttile[(4 * gq + rr) * kSt + c] = f32_to_bf16(pr[4 * T + rr]);
          }
          const bf16x4 as = *reinterpret_cast<const bf16x4*>(sttile + c * kSt + 4 * gq);
          const bf16x4 ap = *reinterpret_cast<const bf16x4*>(pttile + c * kSt + 4 * gq);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int x = swz(r, 16 * t + 4 * (c & 3));
            gk_acc[T][t] = mfma_bf16_k16(as, lds_read_tr16(qtile + x), gk_acc[T][t]);
            gv_acc[T][t] = mfma_bf16_k16(ap, lds_read_tr16(dtile + x), gv_acc[T][t]);
          }
        }
      }
    }
  };

  // dQ = sigma * dQ^T (lane holds d = 16t + 4g + r of query c) -> bf16 rows through the K tile, then whole-row
  // coalesced stores
  auto finish_block = [&]() {
    if (!cur.valid) return;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint2 u = make_uint2(pack_bf16x2(dq_acc[t][0] * g.scale, dq_acc[t][1] * g.scale),
                                 pack_bf16x2(dq_acc[t][2] * g.scale, dq_acc[t][3] * g.scale));
      *reinterpret_cast<uint2*>(kt + swz(c, 16 * t + 4 * gq)) = u;
    }
    const int r = lane >> 3, ch = lane & 7;
    const uint4 x0 = *reinterpret_cast<const uint4*>(kt + r * kD + ((ch ^ r) << 3));
    const uint4 x1 = *reinterpret_cast<const uint4*>(kt + (8 + r) * kD + ((ch ^ r) << 3));
    bf16_t* ob = dq + cur.slice * slice_elems + (size_t)16 * cur.i * kD + r * kD + 8 * ch;
    st16_nt(ob, x0);
    st16_nt(ob + 8 * kD, x1);
  };

  // End of the wave's ju-th unit: the pooled-token partials it accumulated in registers over the unit's 16
  // blocks are stored to the unit's slot (K partials with the softmax scale), and the accumulators cleared.
  auto unit_end = [&](int ju) {
    if (nhigh == 0) return;
    const int U = su.first + su.stride * ju;
    const int slice = uniform(U / gps), u2 = U - slice * gps;
    float* outk = part_k + ((size_t)slice * gps + u2) * nhigh * kD;
    float* outv = part_v + ((size_t)slice * gps + u2) * nhigh * kD;
#pragma unroll
    for (int T = 0; T < kT; ++T)
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = 16 * T + 4 * gq + r, d = 16 * t + c;
          if (e < nhigh) {
            outk[e * kD + d] = gk_acc[T][t][r] * g.scale;
            outv[e * kD + d] = gv_acc[T][t][r];
          }
        }
#pragma unroll
    for (int T = 0; T < kT; ++T)
#pragma unroll
      for (int t = 0; t < 4; ++t) gk_acc[T][t] = gv_acc[T][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  auto consume = [&](const Stage& st) {
    consume_stage(st);
    if (++cs == nst) {
      finish_block();
      cs = 0;
      if ((cj & 15) == 15) unit_end(cj >> 4);
      if (++cj < nblk) {
        par ^= 1;
        cur = nxt;
        nxt = blk(cj + 1);
        begin_block();
      }
    }
  };

  prefetch(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  begin_block();
  const int T = nblk * nst;
  Stage A, B;
  issue(0, cur.slice, 0, A);
  for (int t = 0; t < T; t += 2) {
    issue_next(B);
    consume(A);
    issue_next(A);
    if (t + 1 < T) consume(B);
  }
}

// ------------------------------------------------------------------------------------------------
// 2. Pooled-token gradients of levels 2..Le from the per-(level-2 unit, slot) partials via the CSC.
// One 256-thread workgroup per (slice, token) of levels 2..Le.  Token j of level l sums, over the CSR positions
// p = u*K + s of its column, the partials of entry (l, s) of the B^(l-2) level-2 units under unit u.  Those
// (position, unit) items go four to a wave instruction -- lane l takes item 4 i + l / 16 of its wave's share
// and dims 4 (l % 16) .. +3 of its K and V rows (16-byte loads), eight items of a wave in flight -- and are
// summed in a fixed order: per lane in item order, then the four item lanes of a wave, then the four waves.
// ------------------------------------------------------------------------------------------------
__device__ __forceinline__ void coarse_reduce_block(const int32_t* __restrict__ col_ptr,
                                                    const int32_t* __restrict__ perm,
                                                    const float* __restrict__ part_k,
                                                    const float* __restrict__ part_v, float* __restrict__ gk,
                                                    float* __restrict__ gv, const Geom& g, const CscGeom& cg,
                                                    int slice, int token) {
  __shared__ float4 red[2][4][16];
  const int lane = threadIdx.x & 63, q4 = lane >> 4, d4 = 4 * (lane & 15);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int x = token, l = 2;
  while (x >= g.rows[l]) {
    x -= g.rows[l];
    ++l;
  }
  const int j = x;
  const int nhigh = g.K * (g.Le - 1);
  const int n2 = g.rows[2];
  const int32_t* cp = col_ptr + (size_t)slice * cg.cp_len + cg.cp_off[l];
  const int32_t* pm = perm + (size_t)slice * cg.pm_len + cg.pm_off[l];
  const int sh = 4 * (l - 2);  // level-2 units per level-l unit: 1 << sh
  const int y0 = cp[j];
  const int items = (cp[j + 1] - y0) << sh;
  const float* PKs = part_k + (size_t)slice * n2 * nhigh * kD + d4;
  const float* PVs = part_v + (size_t)slice * n2 * nhigh * kD + d4;
  float4 ak = make_float4(0.f, 0.f, 0.f, 0.f), av = ak;
  // wave w takes items 16 r + 4 w + q4 (r = 0, 1, ...), summed per lane in r order; the items of pair m are
  // 32 m + 4 w + q4 and that + 16 (the second zero past the end), and a pair counts while its first item exists.
  // Four pairs are loaded per trip (a level-3 token's 8 items per lane at once), then added in pair order.
  for (int m0 = 0; 32 * m0 + 4 * w + q4 < items; m0 += 4) {
    float4 xk[8], xv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = 32 * m0 + 4 * w + q4 + 16 * i;
      xk[i] = xv[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (q < items) {
        const int p = pm[y0 + (q >> sh)];
        const int u = p / g.K, slot = p - u * g.K;
        const int u2 = (u << sh) + (q & ((1 << sh) - 1));
        const size_t off = ((size_t)u2 * nhigh + (l - 2) * g.K + slot) * kD;
        // partials are read once: non-temporal loads
        const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(PKs + off));
        const u32x4 b = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(PVs + off));
        xk[i] = make_float4(__uint_as_float(a.x), __uint_as_float(a.y), __uint_as_float(a.z), __uint_as_float(a.w));
        xv[i] = make_float4(__uint_as_float(b.x), __uint_as_float(b.y), __uint_as_float(b.z), __uint_as_float(b.w));
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (32 * (m0 + i / 2) + 4 * w + q4 < items) {
        ak.x += xk[i].x; ak.y += xk[i].y; ak.z += xk[i].z; ak.w += xk[i].w;
        av.x += xv[i].x; av.y += xv[i].y; av.z += xv[i].z; av.w += xv[i].w;
      }
    }
  }
  // the four item lanes of each dim group (lanes d, d + 16, d + 32, d + 48), the same order in every lane
  float4 sk, sv;
  sk.x = group_sum(ak.x); sk.y = group_sum(ak.y); sk.z = group_sum(ak.z); sk.w = group_sum(ak.w);
  sv.x = group_sum(av.x); sv.y = group_sum(av.y); sv.z = group_sum(av.z); sv.w = group_sum(av.w);
  if (q4 == 0) {
    red[0][w][lane] = sk;
    red[1][w][lane] = sv;
  }
  __syncthreads();
  if (w == 0 && q4 < 2) {
    const int dl = lane & 15;
    float4 r = red[q4][0][dl];
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) {
      const float4 z = red[q4][ww][dl];
      r.x += z.x; r.y += z.y; r.z += z.z; r.w += z.w;
    }
    const size_t o = ((size_t)slice * (g.R - g.rows[1]) + g.off[l] - g.rows[1] + j) * kD + d4;
    *reinterpret_cast<float4*>((q4 == 0 ? gk : gv) + o) = r;
  }
}

constexpr int kGroup = 4;       // key blocks per wavefront
constexpr int kSplitMul = 4;    // groups longer than kSplitMul x the mean group length are split into chunks
constexpr int kMaxShares = 4;   // levels 2..L_e with L_e <= 5 (implied by the size limit n * d < 2^31)

}  // namespace

// Per-slice capacities of the dK/dV work lists (see dkdv_order).
DkdvBounds dkdv_bounds(const Geom& g) {
  const int n1 = g.rows[1];
  DkdvBounds b;
  b.items = (n1 + kGroup - 1) / kGroup + n1 / 8 + 1;
  b.slots = n1 / 8 + 1;
  b.splits = n1 / 16 + 1;
  return b;
}

namespace {

// ------------------------------------------------------------------------------------------------
// 3a. Work items of the dK/dV kernel.  A group is 4 consecutive key blocks; its stages are the query blocks of
// their level-1 CSC columns, concatenated (T_g of them).  A group with more than S stages is split into
// ceil(T_g / S) chunks of near-equal size: on smooth or reordered inputs single columns reach 30x the mean, and
// one wavefront walking such a group would end the kernel long after the others.  S (>= kSplitMul x the mean
// group length 4 K) is set by the host to twice the stages per resident wavefront, so only groups that would
// outlast the rest are split.  Each chunk writes fp32 partial dK, dV of the key blocks it touches to a slot of
// its own; the chunk that finishes last (an integer counter per split group) sums all of them in chunk order,
// so the result does not depend on which chunk that is.
// Items: an unsplit group is (group, 0, T_g, -1); chunk c of split group i is (group, c, i, first slot + c),
// the split record (group, first slot, chunks, T_g).  Item order per slice: groups with more than twice the
// mean length first (each expanded into its chunks), then the rest, each part in list order (stable
// partitions by block-wide prefix sums), so the longest work starts first.  List order is group order, or
// with a token grid, groups of four consecutive grid rows at the same column next to each other.  Bounds per
// slice (n_1 K stages in all), for the smallest S: items <= groups + n_1 / 8, slots <= n_1 / 8, split groups
// <= n_1 / 16 (each split group has T_g > S and at most 2 T_g / S chunks).
// grid.x = slices, 1024 threads.
// ------------------------------------------------------------------------------------------------
// kT threads (a multiple of 64, at most 1024) build slice `slice`'s list.
template <int kT>
__device__ __forceinline__ void dkdv_order_block(const int32_t* __restrict__ col_ptr, int4* __restrict__ items,
                                                 int4* __restrict__ splits, int32_t* __restrict__ counters,
                                                 const Geom& g, const CscGeom& cg, const DkdvBounds& bd, int S,
                                                 int walk, int slice) {
  __shared__ long long wave_tot[kT / 64];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int n1 = g.rows[1], gps = (n1 + kGroup - 1) / kGroup;
  const int32_t* cp = col_ptr + (size_t)slice * cg.cp_len + cg.cp_off[1];
  int4* it_out = items + (size_t)slice * bd.items;
  int4* sp_out = splits + (size_t)slice * bd.splits;
  const int thresh = 2 * kGroup * g.K;  // twice the mean group length
  auto glen = [&](int gi) { return cp[min(kGroup * gi + kGroup, n1)] - cp[kGroup * gi]; };
  auto chunks = [&](int T) { return T > S ? (T + S - 1) / S : 1; };
  // block-wide exclusive prefix of two counts at once (low and high 32 bits), with the totals
  auto scan = [&](int lo, int hi, int* elo, int* ehi, int* tlo, int* thi) {
    const long long f = ((long long)hi << 32) + lo;
    long long inc = f;
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
      const long long u = __shfl_up(inc, s, 64);
      if (lane >= s) inc += u;
    }
    if (lane == 63) wave_tot[w] = inc;
    __syncthreads();
    long long before = 0, tot = 0;
    for (int i = 0; i < kT / 64; ++i) {
      before += i < w ? wave_tot[i] : 0;
      tot += wave_tot[i];
    }
    const long long e = before + inc - f;
    *elo = (int)(e & 0xFFFFFFFFll);
    *ehi = (int)(e >> 32);
    *tlo = (int)(tot & 0xFFFFFFFFll);
    *thi = (int)(tot >> 32);
    __syncthreads();
  };
  // List order of the groups: with a token grid (g.gpr groups per grid row), bands of four grid rows taken
  // column by column, so that the four consecutive items a workgroup takes come from four consecutive rows --
  // groups one row apart share query blocks, which the workgroup's waves then find in the CU's L1 -- and rows
  // past the last whole band in group order; without a grid, group order.
  const int band = 4 * g.gpr, banded = g.gpr > 0 ? gps / band * band : 0;
  auto list_group = [&](int pp) {
    if (pp >= banded) return pp;
    const int b0 = pp / band * band, within = pp - b0;
    return b0 + (within & 3) * g.gpr + (within >> 2);
  };
  // Thread t owns the contiguous run [g0, g1) of that order: it counts its items, one scan places every run,
  // and the thread then writes its run's items in that order.
  const int m = (gps + kT - 1) / kT;
  const int g0 = min(gps, t * m), g1 = min(gps, g0 + m);
  int c_long = 0, c_short = 0, c_slot = 0, c_split = 0;
  for (int pp = g0; pp < g1; ++pp) {
    const int gi = list_group(pp);
    const int T = glen(gi);
    const bool lng = T > thresh, split = lng && T > S;
    const int nch = split ? chunks(T) : 1;
    c_long += lng ? nch : 0;
    c_short += lng ? 0 : 1;
    c_slot += split ? nch : 0;
    c_split += split ? 1 : 0;
  }
  int p_long, p_short, p_slot, p_split, nlong, nshort, t2, t3;
  scan(c_long, c_short, &p_long, &p_short, &nlong, &nshort);  // item positions: long groups, then the others
  scan(c_slot, c_split, &p_slot, &p_split, &t2, &t3);          // partial slots, split-group index
  for (int pp = g0; pp < g1; ++pp) {
    const int gi = list_group(pp);
    const int T = glen(gi);
    const bool lng = T > thresh, split = lng && T > S;
    if (split) {
      const int nch = chunks(T);
      for (int c = 0; c < nch; ++c) it_out[p_long + c] = make_int4(gi, c, p_split, p_slot + c);
      sp_out[p_split] = make_int4(gi, p_slot, nch, T);
      counters[(size_t)slice * bd.splits + p_split] = 0;
      p_long += nch;
      p_slot += nch;
      ++p_split;
    } else if (lng) {
      it_out[p_long++] = make_int4(gi, 0, T, -1);
    } else {
      it_out[nlong + p_short++] = make_int4(gi, 0, T, -1);
    }
  }
  // the positions the dK/dV grid walks past the last item hold an end marker (group -1)
  for (int p = nlong + nshort + t; p < walk; p += kT) it_out[p] = make_int4(-1, 0, 0, -1);
}

// grid.x = slices, 1024 threads.
__global__ __launch_bounds__(1024) void dkdv_order(const int32_t* __restrict__ col_ptr, int4* __restrict__ items,
                                                   int4* __restrict__ splits, int32_t* __restrict__ counters,
                                                   Geom g, CscGeom cg, DkdvBounds bd, int S, int walk) {
  dkdv_order_block<1024>(col_ptr, items, splits, counters, g, cg, bd, S, walk, blockIdx.x);
}

// The pooled-token reduction (step 2) and the dK/dV work lists (step 3a) in one launch: they are independent --
// the lists need only the CSC, the reduction the dQ kernel's partials.  Blocks 0 .. slices-1 build the lists
// (256 threads each); block slices + slice * tokens_hi + j reduces token j of the slice's levels 3..Le, and the
// blocks after those the level-2 tokens, slice by slice: the longest chains (the work lists, the level >= 3
// columns) start first.
__global__ __launch_bounds__(256) void reduce_and_order(const int32_t* __restrict__ col_ptr,
                                                        const int32_t* __restrict__ perm,
                                                        const float* __restrict__ part_k,
                                                        const float* __restrict__ part_v, float* __restrict__ gk,
                                                        float* __restrict__ gv, int4* __restrict__ items,
                                                        int4* __restrict__ splits, int32_t* __restrict__ counters,
                                                        Geom g, CscGeom cg, DkdvBounds bd, int S, int walk,
                                                        int tokens_hi) {
  const int b = blockIdx.x;
  if (b < g.bh) {
    dkdv_order_block<256>(col_ptr, items, splits, counters, g, cg, bd, S, walk, b);
    return;
  }
  int r = b - g.bh;
  if (r < g.bh * tokens_hi) {  // tokens of levels 3..Le (the longest columns, dispatched first)
    const int slice = r / tokens_hi;
    coarse_reduce_block(col_ptr, perm, part_k, part_v, gk, gv, g, cg, slice, g.rows[2] + r - slice * tokens_hi);
    return;
  }
  r -= g.bh * tokens_hi;  // level-2 tokens
  const int slice = r / g.rows[2];
  coarse_reduce_block(col_ptr, perm, part_k, part_v, gk, gv, g, cg, slice, r - slice * g.rows[2]);
}

// ------------------------------------------------------------------------------------------------
// 3. dK, dV over the level-1 CSC, four consecutive key blocks per wavefront.
// grid.x = ceil(bh * walk / 4) (remapped; walk = the items-per-slice bound for the split length in use),
// 256 threads; wave w takes work item 4 * id + w: a
// key-block group (key blocks 4*gi .. 4*gi+3 of one slice) or a chunk of a split group's stages.  The group's columns are consecutive in perm, so the wave walks
// one list of query blocks (its stages) across its key blocks, the next stage's loads in flight while a stage
// is consumed.  A key block's own rows (K, V and its level-1 pooled token) are copied to LDS (DMA) while the
// previous block is consumed; the levels >= 2 shares -- the same for the four blocks, whose ancestors coincide
// -- are copied once.  One wavefront per group (not persistent) keeps the hardware's dynamic scheduling over
// the very uneven column lengths.
// ------------------------------------------------------------------------------------------------

// LDS of the dK/dV kernel (per wave w: index [w]).
struct DkdvLds {
  bf16_t qs[4][16 * kD];               // Q rows of the query block (swizzled)
  bf16_t dos[4][16 * kD];              // dO rows (swizzled)
  float lds_ld[4][64];                 // LSE (0..15) and Delta (16..31)
  bf16_t kvs[4][2][16 * kD];           // K, V rows of the next key block
  bf16_t p1s[4][2][kD];                // its level-1 pooled K, V rows (bf16)
  float shs[4][kMaxShares][2][kD];     // ancestors' pooled K, V gradients
};

// One work item of wave w.  split: a chunk of a split group (partial sums; the last chunk combines).
// Pooled-gradient shares of a key-block group: share s is level s + 2, whose ancestor j >> 4(l-1) is the same for
// the group's four blocks; row of the level's gradient array (levels >= 2 only, or every level for the
// complement reading).
__device__ __forceinline__ int share_level(int s) { return s + 2; }
__device__ __forceinline__ int share_count(const Geom& g) { return max(0, min(g.Le, kMaxShares + 1) - 1); }
template <bool kComp>
__device__ __forceinline__ size_t share_row(const Geom& g, int slice, int l, int j) {
  const int a = j >> (4 * (l - 1));
  return kComp ? (size_t)slice * g.R + g.off[l] + a : (size_t)slice * (g.R - g.rows[1]) + g.off[l] - g.rows[1] + a;
}

// kComp: the complement reading -- the query blocks of a key block's column do not attend its level-1 pooled
// token (they kept the block), so nothing is folded into the products; instead each key block adds B^-1 of its
// own level-1 pooled token's gradient, and the group the shares of levels >= 2 (gk, gv: [slice][R][d]).
template <bool split, bool kComp>
__device__ __forceinline__ void dkdv_item(DkdvLds& sm, const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                          const bf16_t* __restrict__ v, const bf16_t* __restrict__ dout,
                                          const float* __restrict__ lse, const float* __restrict__ delta,
                                          const bf16_t* __restrict__ pk, const bf16_t* __restrict__ pv,
                                          const int32_t* __restrict__ col_ptr, const int32_t* __restrict__ perm,
                                          const float* __restrict__ gk, const float* __restrict__ gv,
                                          const int4* __restrict__ splits, int32_t* __restrict__ counters,
                                          float* __restrict__ part, bf16_t* __restrict__ dk, bf16_t* __restrict__ dv,
                                          const Geom& g, const CscGeom& cg, const DkdvBounds& bd, int slice,
                                          int4 item, int w) {
  const int lane = threadIdx.x & 63, c = lane & 15, gq = lane >> 4;
  const int n1 = g.rows[1];
  const int j0 = kGroup * item.x;
  const int slot = item.w;
  int4 sp = make_int4(0, 0, 1, 0);
  if (split) sp = splits[(size_t)slice * bd.splits + item.z];  // group, first slot, chunks, stages
  const int s0 = split ? (int)((int64_t)item.y * sp.w / sp.z) : 0;
  const int s1 = split ? (int)((int64_t)(item.y + 1) * sp.w / sp.z) : item.z;
  const int nkb = min(kGroup, n1 - j0);
  const size_t base = (size_t)slice * g.n * kD;
  const bf16_t* Q = q + base;
  const bf16_t* DO = dout + base;
  const float* LS = lse + (size_t)slice * g.n;
  const float* DL = delta + (size_t)slice * g.n;
  const int32_t* cp = col_ptr + (size_t)slice * cg.cp_len + cg.cp_off[1];
  const int32_t* pm = perm + (size_t)slice * cg.pm_len + cg.pm_off[1];
  bf16_t* qt = sm.qs[w];
  bf16_t* dt = sm.dos[w];
  float* ldt = sm.lds_ld[w];
  const int c7 = c & 7;
  const int a0 = c * kD + ((gq ^ c7) << 3), a1 = c * kD + (((4 + gq) ^ c7) << 3);
  const int trr = 4 * gq + (c >> 2);
  const bool enrich1 = !kComp && g.Le >= 1;
  const int nsh = split ? 0 : share_count(g);  // chunks leave the shares to the combine

  // column starts of the group's key blocks (lane t: column j0 + t; lane nkb: the end of the last one), as stage
  // numbers of the item (clipped to its stages [s0, s1) of the group)
  const int cpr = cp[j0 + min(lane, nkb)];
  const int yg = __builtin_amdgcn_readfirstlane(cpr);
  const int cpl = min(max(cpr - yg, s0), s1) - s0;
  const int y0 = yg + s0;  // perm position of the item's first stage
  const int total = __builtin_amdgcn_readlane(cpl, nkb);
  auto col_len = [&](int b) { return __builtin_amdgcn_readlane(cpl, b + 1) - __builtin_amdgcn_readlane(cpl, b); };
  auto next_nonempty = [&](int b) {  // first block after b with a non-empty column, nkb if none
    int nb = b + 1;
    while (nb < nkb && col_len(nb) == 0) ++nb;
    return nb;
  };

  // copies of one key block's rows into the (single) block slot, and of the shares.  The block's K, V and
  // level-1 pooled rows are read by this item alone: non-temporal, so that they leave the L2 to the Q and dO
  // rows that the stages of other items gather again
  auto dma_block = [&](int b) {
    const size_t r = base + (size_t)16 * (j0 + b) * kD + swz_dma_src(lane);
    lds_dma16_nt(k + r, &sm.kvs[w][0][0]);
    lds_dma16_nt(k + r + 8 * kD, &sm.kvs[w][0][8 * kD]);
    lds_dma16_nt(v + r, &sm.kvs[w][1][0]);
    lds_dma16_nt(v + r + 8 * kD, &sm.kvs[w][1][8 * kD]);
    if (lane < 16)
      lds_dma16_nt((lane < 8 ? pk : pv) + ((size_t)slice * g.R + g.off[1] + j0 + b) * kD + 8 * (lane & 7), &sm.p1s[w][0][0]);
  };
  if (lane < 32) {
    for (int s = 0; s < nsh; ++s) {
      const size_t gr = share_row<kComp>(g, slice, share_level(s), j0) * kD + 4 * (lane & 15);
      lds_dma16((lane < 16 ? gk : gv) + gr, &sm.shs[w][s][0][0]);
    }
  }

  // B operands (natural order) of the current key block: its K and V rows, and its level-1 pooled token (bf16,
  // as in the forward products) as a broadcast operand (every column holds it)
  bf16x8 kb0, kb1, vb0, vb1, k1b0, k1b1, v1b0, v1b1;
  auto read_block = [&]() {
    kb0 = *reinterpret_cast<const bf16x8*>(&sm.kvs[w][0][a0]);
    kb1 = *reinterpret_cast<const bf16x8*>(&sm.kvs[w][0][a1]);
    vb0 = *reinterpret_cast<const bf16x8*>(&sm.kvs[w][1][a0]);
    vb1 = *reinterpret_cast<const bf16x8*>(&sm.kvs[w][1][a1]);
    k1b0 = *reinterpret_cast<const bf16x8*>(&sm.p1s[w][0][8 * gq]);
    k1b1 = *reinterpret_cast<const bf16x8*>(&sm.p1s[w][0][8 * gq + 32]);
    v1b0 = *reinterpret_cast<const bf16x8*>(&sm.p1s[w][1][8 * gq]);
    v1b1 = *reinterpret_cast<const bf16x8*>(&sm.p1s[w][1][8 * gq + 32]);
    wait_lds();  // the slot is refilled next
  };

  f32x4 dk_acc[4], dv_acc[4];
  auto zero_acc = [&]() {
#pragma unroll
    for (int t = 0; t < 4; ++t) dk_acc[t] = dv_acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  // dK = sigma dK^T + shares, dV = dV^T + shares (lane holds d = 16t + 4g + r of key c; with_acc false for a key
  // block no query block kept) -> bf16 rows through the Q / dO tiles, then whole-row coalesced stores
  auto finish = [&](int b, bool with_acc) {
    if (split) {  // fp32 partial of a touched block to the item's slot: [block][K, V][key][dim]
      if (with_acc) {
        float* P = part + (((size_t)slice * bd.slots + slot) * kGroup + b) * (2 * 16 * kD) + c * kD + 4 * gq;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          *reinterpret_cast<f32x4*>(P + 16 * t) = dk_acc[t];
          *reinterpret_cast<f32x4*>(P + 16 * kD + 16 * t) = dv_acc[t];
        }
      }
      return;
    }
    float kx[4][4], vx[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        kx[t][r] = with_acc ? dk_acc[t][r] * g.scale : 0.f;
        vx[t][r] = with_acc ? dv_acc[t][r] : 0.f;
      }
    if (kComp && g.Le >= 1) {  // the block's own level-1 pooled token
      const size_t r1 = share_row<true>(g, slice, 1, j0 + b) * kD + 4 * gq;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float4 gk4 = *reinterpret_cast<const float4*>(gk + r1 + 16 * t);
        const float4 gv4 = *reinterpret_cast<const float4*>(gv + r1 + 16 * t);
        const float wgt = 1.0f / (float)kB;
        kx[t][0] += gk4.x * wgt; kx[t][1] += gk4.y * wgt; kx[t][2] += gk4.z * wgt; kx[t][3] += gk4.w * wgt;
        vx[t][0] += gv4.x * wgt; vx[t][1] += gv4.y * wgt; vx[t][2] += gv4.z * wgt; vx[t][3] += gv4.w * wgt;
      }
    }
    for (int s = 0; s < nsh; ++s) {
      const float wgt = 1.0f / (float)(1 << (4 * share_level(s)));
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float4 gk4 = *reinterpret_cast<const float4*>(&sm.shs[w][s][0][16 * t + 4 * gq]);
        const float4 gv4 = *reinterpret_cast<const float4*>(&sm.shs[w][s][1][16 * t + 4 * gq]);
        kx[t][0] += gk4.x * wgt; kx[t][1] += gk4.y * wgt; kx[t][2] += gk4.z * wgt; kx[t][3] += gk4.w * wgt;
        vx[t][0] += gv4.x * wgt; vx[t][1] += gv4.y * wgt; vx[t][2] += gv4.z * wgt; vx[t][3] += gv4.w * wgt;
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      *reinterpret_cast<uint2*>(qt + swz(c, 16 * t + 4 * gq)) =
          make_uint2(pack_bf16x2(kx[t][0], kx[t][1]), pack_bf16x2(kx[t][2], kx[t][3]));
      *reinterpret_cast<uint2*>(dt + swz(c, 16 * t + 4 * gq)) =
          make_uint2(pack_bf16x2(vx[t][0], vx[t][1]), pack_bf16x2(vx[t][2], vx[t][3]));
    }
    const int r = lane >> 3, ch = lane & 7;
    const int o0 = r * kD + ((ch ^ r) << 3);
    const size_t go = base + ((size_t)16 * (j0 + b) + r) * kD + 8 * ch;
    st16_nt(dk + go, *reinterpret_cast<const uint4*>(qt + o0));
    st16_nt(dk + go + 8 * kD, *reinterpret_cast<const uint4*>(qt + o0 + 8 * kD));
    st16_nt(dv + go, *reinterpret_cast<const uint4*>(dt + o0));
    st16_nt(dv + go + 8 * kD, *reinterpret_cast<const uint4*>(dt + o0 + 8 * kD));
  };

  int cb = next_nonempty(-1);  // key block being consumed
  if (cb < nkb) dma_block(cb);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  for (int b = 0; b < cb; ++b) finish(b, false);  // leading key blocks nobody kept
  if (cb >= nkb) return;
  read_block();
  int nb = next_nonempty(cb);  // the block whose rows sit in the slot next
  if (nb < nkb) dma_block(nb);
  zero_acc();

  // query blocks of the group's stages, 64 at a time in lanes (read with readlane)
  int chunk = 0;
  int qb_lane = pm[y0 + min(lane, total - 1)] / g.K;
  auto stage_qb = [&](int s) {
    if (s >= chunk + 64) {
      chunk += 64;
      qb_lane = pm[y0 + min(chunk + lane, total - 1)] / g.K;
    }
    return __builtin_amdgcn_readlane(qb_lane, s - chunk);
  };

  // One stage = one query block, loaded coalesced: Q and dO rows (lane l: rows l/8 and 8 + l/8, bytes
  // 16 (l%8)), then LSE (lanes 0..15) and Delta (lanes 16..31) of its 16 queries.
  struct QStage {
    uint4 q0, q1, d0, d1;
    float ld;
  };
  const int ro = (lane >> 3) * kD + 8 * (lane & 7);
  auto issue = [&](int i, QStage& st) {
    const bf16_t* qr = Q + (size_t)16 * i * kD + ro;
    const bf16_t* dr = DO + (size_t)16 * i * kD + ro;
    st.q0 = ld16(qr);
    st.q1 = ld16(qr + 8 * kD);
    st.d0 = ld16(dr);
    st.d1 = ld16(dr + 8 * kD);
    st.ld = (lane < 16 ? LS : DL)[16 * i + (lane & 15)];
  };
  int gi = 0;  // last issued stage
  auto issue_next = [&](QStage& st) {
    gi = min(gi + 1, total - 1);  // past the end: an in-bounds reload that is never consumed
    issue(stage_qb(gi), st);
  };

  auto compute = [&](const QStage& st) {
    {
      const int r = lane >> 3, ch = lane & 7;
      const int o0 = r * kD + ((ch ^ r) << 3), o1 = o0 + 8 * kD;
      *reinterpret_cast<uint4*>(qt + o0) = st.q0;
      *reinterpret_cast<uint4*>(qt + o1) = st.q1;
      *reinterpret_cast<uint4*>(dt + o0) = st.d0;
      *reinterpret_cast<uint4*>(dt + o1) = st.d1;
      ldt[lane] = st.ld;  // every lane writes (lanes 32..63 a duplicate): no divergent store before the reads
    }
    const bf16x8 qa0 = *reinterpret_cast<const bf16x8*>(qt + a0), qa1 = *reinterpret_cast<const bf16x8*>(qt + a1);
    const bf16x8 da0 = *reinterpret_cast<const bf16x8*>(dt + a0), da1 = *reinterpret_cast<const bf16x8*>(dt + a1);
    f32x4 s = {0.f, 0.f, 0.f, 0.f}, dpv = {0.f, 0.f, 0.f, 0.f};
    s = mfma_bf16_k32(qa0, kb0, s);
    s = mfma_bf16_k32(qa1, kb1, s);
    dpv = mfma_bf16_k32(da0, vb0, dpv);
    dpv = mfma_bf16_k32(da1, vb1, dpv);
    // s[r] = S[query 4g + r][key c]
    const float4 ls4 = *reinterpret_cast<const float4*>(ldt + 4 * gq);
    const float4 dl4 = *reinterpret_cast<const float4*>(ldt + 16 + 4 * gq);
    const float ls[4] = {ls4.x, ls4.y, ls4.z, ls4.w};
    const float dl[4] = {dl4.x, dl4.y, dl4.z, dl4.w};
    float p[4], ds[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float lse2 = ls[r] * kLog2e;
      p[r] = fast_exp2(s[r] * g.scale_log2 - lse2);
      ds[r] = p[r] * (dpv[r] - dl[r]);
    }
    if (enrich1) {
      // the query block also attends this block's level-1 pooled token (logit + ln B); each raw key of
      // the block receives B^-1 of that token's gradient, folded into the same products
      f32x4 sc = {0.f, 0.f, 0.f, 0.f}, dpc = {0.f, 0.f, 0.f, 0.f};
      sc = mfma_bf16_k32(qa0, k1b0, sc);
      sc = mfma_bf16_k32(qa1, k1b1, sc);
      dpc = mfma_bf16_k32(da0, v1b0, dpc);
      dpc = mfma_bf16_k32(da1, v1b1, dpc);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pc = fast_exp2(sc[r] * g.scale_log2 + 4.0f - ls[r] * kLog2e);
        p[r] += pc * (1.0f / (float)kB);
        ds[r] += pc * (dpc[r] - dl[r]) * (1.0f / (float)kB);
      }
    }
    const bf16x4 pb = pack4(p[0], p[1], p[2], p[3]);
    const bf16x4 db = pack4(ds[0], ds[1], ds[2], ds[3]);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int x = swz(trr, 16 * t + 4 * (c & 3));
      dv_acc[t] = mfma_bf16_k16(lds_read_tr16(dt + x), pb, dv_acc[t]);
      dk_acc[t] = mfma_bf16_k16(lds_read_tr16(qt + x), db, dk_acc[t]);
    }
  };

  int gc = 0;  // stages consumed
  int cend = __builtin_amdgcn_readlane(cpl, cb + 1);
  auto consume = [&](const QStage& st) {
    compute(st);
    if (++gc == cend) {
      // key block cb is complete.  The next non-empty block's rows were copied while cb was consumed: that
      // copy is older than the one stage (5 loads) issued since, so vmcnt(5) covers it.  Its operands are
      // read before cb's results are stored, so the stores never sit between the copy and this wait.
      const int prev = cb;
      if (nb < nkb) {
        asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
        read_block();
        cb = nb;
        nb = next_nonempty(cb);
        if (nb < nkb) dma_block(nb);
        cend = __builtin_amdgcn_readlane(cpl, cb + 1);
      }
      finish(prev, true);
      for (int b = prev + 1; b < (cb > prev ? cb : nkb); ++b) finish(b, false);  // blocks nobody kept
      zero_acc();
    }
  };

  QStage A, B;
  issue(stage_qb(0), A);
  for (int t = 0; t < total; t += 2) {
    issue_next(B);
    consume(A);
    issue_next(A);
    if (t + 1 < total) consume(B);
  }
  if (!split) return;

  // Split group: count this chunk done (its partial stores made visible first); the last one to finish sums
  // every chunk's partials of each key block in chunk order (a chunk's partial of block b exists iff its
  // stages meet b's column), then scale and shares as in finish.  Lane: key lane / 4, dims 16 (lane % 4) + 0..15.
  __threadfence();
  int done = 0;
  if (lane == 0) done = atomicAdd(&counters[(size_t)slice * bd.splits + item.z], 1);
  done = __shfl(done, 0, 64);
  if (done != sp.z - 1) return;
  __threadfence();
  const int key = lane >> 2, d0 = 16 * (lane & 3);
  const int nshc = share_count(g);
  for (int b = 0; b < nkb; ++b) {
    const int cs = __builtin_amdgcn_readlane(cpr, b) - yg, ce = __builtin_amdgcn_readlane(cpr, b + 1) - yg;
    float kx[16], vx[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) kx[e] = vx[e] = 0.f;
    for (int ch = 0; ch < sp.z; ++ch) {
      const int c0 = (int)((int64_t)ch * sp.w / sp.z), c1 = (int)((int64_t)(ch + 1) * sp.w / sp.z);
      if (max(cs, c0) >= min(ce, c1)) continue;
      const float* P = part + (((size_t)slice * bd.slots + sp.y + ch) * kGroup + b) * (2 * 16 * kD) + key * kD + d0;
#pragma unroll
      for (int e = 0; e < 16; e += 4) {
        const float4 a = *reinterpret_cast<const float4*>(P + e);
        const float4 z = *reinterpret_cast<const float4*>(P + 16 * kD + e);
        kx[e] += a.x; kx[e + 1] += a.y; kx[e + 2] += a.z; kx[e + 3] += a.w;
        vx[e] += z.x; vx[e + 1] += z.y; vx[e + 2] += z.z; vx[e + 3] += z.w;
      }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) kx[e] *= g.scale;
    if (kComp && g.Le >= 1) {  // the block's own level-1 pooled token
      const size_t r1 = share_row<true>(g, slice, 1, j0 + b) * kD + d0;
#pragma unroll
      for (int e = 0; e < 16; e += 4) {
        const float4 a4 = *reinterpret_cast<const float4*>(gk + r1 + e);
        const float4 z4 = *reinterpret_cast<const float4*>(gv + r1 + e);
        const float wgt = 1.0f / (float)kB;
        kx[e] += a4.x * wgt; kx[e + 1] += a4.y * wgt; kx[e + 2] += a4.z * wgt; kx[e + 3] += a4.w * wgt;
        vx[e] += z4.x * wgt; vx[e + 1] += z4.y * wgt; vx[e + 2] += z4.z * wgt; vx[e + 3] += z4.w * wgt;
      }
    }
    for (int sh = 0; sh < nshc; ++sh) {
      const int l = share_level(sh);
      const float wgt = 1.0f / (float)(1 << (4 * l));
      const size_t gr = share_row<kComp>(g, slice, l, j0) * kD + d0;
#pragma unroll
      for (int e = 0; e < 16; e += 4) {
        const float4 a4 = *reinterpret_cast<const float4*>(gk + gr + e);
        const float4 z4 = *reinterpret_cast<const float4*>(gv + gr + e);
        kx[e] += a4.x * wgt; kx[e + 1] += a4.y * wgt; kx[e + 2] += a4.z * wgt; kx[e + 3] += a4.w * wgt;
        vx[e] += z4.x * wgt; vx[e + 1] += z4.y * wgt; vx[e + 2] += z4.z * wgt; vx[e + 3] += z4.w * wgt;
      }
    }
    const size_t go = base + ((size_t)16 * (j0 + b) + key) * kD + d0;
    st16_nt(dk + go, make_uint4(pack_bf16x2(kx[0], kx[1]), pack_bf16x2(kx[2], kx[3]), pack_bf16x2(kx[4], kx[5]),
                             pack_bf16x2(kx[6], kx[7])));
    st16_nt(dk + go + 8, make_uint4(pack_bf16x2(kx[8], kx[9]), pack_bf16x2(kx[10], kx[11]),
                                 pack_bf16x2(kx[12], kx[13]), pack_bf16x2(kx[14], kx[15])));
    st16_nt(dv + go, make_uint4(pack_bf16x2(vx[0], vx[1]), pack_bf16x2(vx[2], vx[3]), pack_bf16x2(vx[4], vx[5]),
                             pack_bf16x2(vx[6], vx[7])));
    st16_nt(dv + go + 8, make_uint4(pack_bf16x2(vx[8], vx[9]), pack_bf16x2(vx[10], vx[11]),
                                 pack_bf16x2(vx[12], vx[13]), pack_bf16x2(vx[14], vx[15])));
  }
}

template <bool kComp>
__global__ __launch_bounds__(256, 3) void bwd_dkdv_bf16(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                     const bf16_t* __restrict__ v, const bf16_t* __restrict__ dout,
                                                     const float* __restrict__ lse, const float* __restrict__ delta,
                                                     const bf16_t* __restrict__ pk, const bf16_t* __restrict__ pv,
                                                     const int32_t* __restrict__ col_ptr,
                                                     const int32_t* __restrict__ perm, const float* __restrict__ gk,
                                                     const float* __restrict__ gv,
                                                     const int4* __restrict__ items,
                                                     const int4* __restrict__ splits, int32_t* __restrict__ counters,
                                                     float* __restrict__ part, bf16_t* __restrict__ dk,
                                                     bf16_t* __restrict__ dv, Geom g, CscGeom cg, DkdvBounds bd,
                                                     int walk) {
  __shared__ __attribute__((aligned(16))) DkdvLds sm;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Work item: the item list puts each slice's long groups first.  With bh a multiple of 8, XCD x (= block % 8,
  // round-robin dispatch) owns slices [x bh/8, (x+1) bh/8) and walks their lists position-major (four positions
  // of one slice per workgroup), so every XCD starts on its longest groups and keeps its slices in its L2;
  // otherwise all slices go position-major the same way.
  // A workgroup's four waves take four consecutive positions of one slice's list (neighbouring groups, which
  // share query blocks in the CU's L1); consecutive workgroups alternate between the slices.
  int slice, pos;
  if (g.bh % 8 == 0) {
    const int nsl = g.bh / 8, quad = blockIdx.x / 8;
    slice = (blockIdx.x % 8) * nsl + quad % nsl;
    pos = 4 * (quad / nsl) + w;
  } else {
    const int quad = blockIdx.x;
    slice = quad % g.bh;
    pos = 4 * (quad / g.bh) + w;
  }
  if (pos >= walk) return;  // no workgroup barrier below
  int4 item = items[(size_t)slice * bd.items + pos];  // pos < walk <= capacity; group -1 past the last item
  item = make_int4(uniform(item.x), uniform(item.y), uniform(item.z), uniform(item.w));
  if (item.x < 0) return;
  // two copies of the item code: the one for unsplit groups carries none of the split path
  if (item.w >= 0)
    dkdv_item<true, kComp>(sm, q, k, v, dout, lse, delta, pk, pv, col_ptr, perm, gk, gv, splits, counters, part, dk, dv, g,
                    cg, bd, slice, item, w);
  else
    dkdv_item<false, kComp>(sm, q, k, v, dout, lse, delta, pk, pv, col_ptr, perm, gk, gv, splits, counters, part, dk, dv,
                     g, cg, bd, slice, item, w);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Split length and list length of the dK/dV work lists.
struct DkdvPlan {
  int S;     // groups longer than S stages are split
  int walk;  // item positions per slice the kernel walks
};
template <bool kComp>
DkdvPlan dkdv_plan(const Geom& g) {
  const int n1 = g.rows[1];
  const DkdvBounds bd = dkdv_bounds(g);
  // split length: twice the stages per resident wavefront (all slices' n_1 K stages spread over the waves
  // the device holds), at least kSplitMul x the mean group length
  const int64_t waves = 4 * (int64_t)std::max(1, resident_workgroups((const void*)bwd_dkdv_bf16<kComp>, 256));
  const int64_t per_wave = ((int64_t)g.bh * n1 * g.K + waves - 1) / waves;
  DkdvPlan pl;
  pl.S = (int)std::min<int64_t>(std::max<int64_t>(kSplitMul * kGroup * g.K, 2 * per_wave), 1 << 30);
  // items per slice with this S: groups + at most 2 n_1 K / S chunks beyond one per split group
  pl.walk = (int)std::min<int64_t>(bd.items, (n1 + kGroup - 1) / kGroup + 2 * (int64_t)n1 * g.K / pl.S + 1);
  return pl;
}

// The work lists (unless lists_ready: built already, with the same plan), then the dK/dV kernel.
template <bool kComp>
void launch_dkdv(const Geom& g, const CscGeom& cg, const void* q, const void* k, const void* v, const float* lse,
                 const void* dout, const void* pk, const void* pv, const int32_t* col_ptr, const int32_t* perm,
                 void* dk, void* dv, const BwdWs& ws, const DkdvPlan& pl, bool lists_ready, hipStream_t stream) {
  const DkdvBounds bd = dkdv_bounds(g);
  const int walk = pl.walk;
  const int quads = (walk + 3) / 4;  // workgroups per slice: four list positions each
  const int grid = g.bh % 8 == 0 ? 8 * (g.bh / 8) * quads : g.bh * quads;
  if (!lists_ready)
    dkdv_order<<<g.bh, 1024, 0, stream>>>(col_ptr, ws.items, ws.splits, ws.split_done, g, cg, bd, pl.S, walk);
  bwd_dkdv_bf16<kComp><<<grid, 256, 0, stream>>>((const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v,
                                                 (const bf16_t*)dout, lse, ws.delta, (const bf16_t*)pk,
                                                 (const bf16_t*)pv, col_ptr, perm, ws.gk, ws.gv, ws.items, ws.splits,
                                                 ws.split_done, ws.dkdv_part, (bf16_t*)dk, (bf16_t*)dv, g, cg, bd,
                                                 walk);
}

// Work-list part of a backward workspace, from `p` (null: sizes only); adds its bytes.
void dkdv_ws(const Geom& g, BwdWs* out, char* p, size_t* bytes) {
  const DkdvBounds bd = dkdv_bounds(g);
  const size_t n_items = align256((size_t)g.bh * bd.items * sizeof(int4));
  const size_t n_splits = align256((size_t)g.bh * bd.splits * sizeof(int4));
  const size_t n_ctr = align256((size_t)g.bh * bd.splits * sizeof(int32_t));
  const size_t n_dkdv = align256((size_t)g.bh * bd.slots * kGroup * 2 * 16 * kD * sizeof(float));
  if (out) {
    out->items = reinterpret_cast<int4*>(p);
    out->splits = reinterpret_cast<int4*>(p + n_items);
    out->split_done = reinterpret_cast<int32_t*>(p + n_items + n_splits);
    out->dkdv_part = reinterpret_cast<float*>(p + n_items + n_splits + n_ctr);
  }
  *bytes += n_items + n_splits + n_ctr + n_dkdv;
}

}  // namespace

size_t bwd_ws_layout(const Geom& g, BwdWs* out, void* base) {
  const int nhigh = g.Le >= 2 ? g.K * (g.Le - 1) : 0;
  const size_t n_delta = align256((size_t)g.bh * g.n * sizeof(float));
  const size_t n_part = nhigh ? align256((size_t)g.bh * g.rows[2] * nhigh * kD * sizeof(float)) : 0;
  const size_t n_g = nhigh ? align256((size_t)g.bh * (g.R - g.rows[1]) * kD * sizeof(float)) : 0;
  size_t bytes = n_delta + 2 * n_part + 2 * n_g;
  if (out) {
    char* p = static_cast<char*>(base);
    out->delta = reinterpret_cast<float*>(p);
    p += n_delta;
    out->part_k = nhigh ? reinterpret_cast<float*>(p) : nullptr;
    p += n_part;
    out->part_v = nhigh ? reinterpret_cast<float*>(p) : nullptr;
    p += n_part;
    out->gk = nhigh ? reinterpret_cast<float*>(p) : nullptr;
    p += n_g;
    out->gv = nhigh ? reinterpret_cast<float*>(p) : nullptr;
    p += n_g;
  }
  dkdv_ws(g, out, out ? static_cast<char*>(base) + bytes : nullptr, &bytes);
  return bytes;
}

size_t bwd_comp_ws_layout(const Geom& g, const PartGeom& pg, BwdWs* out, void* base) {
  const size_t n_delta = align256((size_t)g.bh * g.n * sizeof(float));
  const size_t n_g = align256((size_t)g.bh * g.R * kD * sizeof(float));
  const size_t n_part = align256((size_t)g.bh * pg.n2u * pg.nc * 2 * kD * sizeof(float));
  size_t bytes = n_delta + 2 * n_g + n_part;
  if (out) {
    char* p = static_cast<char*>(base);
    out->delta = reinterpret_cast<float*>(p);
    out->gk = reinterpret_cast<float*>(p + n_delta);
    out->gv = reinterpret_cast<float*>(p + n_delta + n_g);
    out->part_k = reinterpret_cast<float*>(p + n_delta + 2 * n_g);  // the pooled-gradient partials
    out->part_v = nullptr;
  }
  dkdv_ws(g, out, out ? static_cast<char*>(base) + bytes : nullptr, &bytes);
  return bytes;
}

hipError_t launch_attn_bwd(const Geom& g, const CscGeom& cg, const void* q, const void* k, const void* v,
                           const void* o, const float* lse, const void* dout, const void* pk, const void* pv,
                           const int32_t* idx, const int32_t* col_ptr, const int32_t* perm, void* dq, void* dk,
                           void* dv, const BwdWs& ws, hipStream_t stream) {
  const int n1 = g.rows[1];
  const int groups = g.bh * ((n1 + 15) / 16);
  {
    LaunchTimer timer(kBwdDq, stream);
    const int nhigh = g.Le >= 2 ? g.K * (g.Le - 1) : 0;
    auto kernel = nhigh <= 16 ? bwd_dq_bf16<1, kMaxCoarse, false> : bwd_dq_bf16<2, kMaxCoarse, false>;
    kernel<<<persistent_grid((const void*)kernel, 256, groups), 256, 0, stream>>>(
        (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, (const bf16_t*)o, lse, (const bf16_t*)dout,
        (const bf16_t*)pk, (const bf16_t*)pv,
        idx, (bf16_t*)dq, ws.delta, ws.part_k, ws.part_v, idx, g, CompGeom{});
  }
  const DkdvPlan pl = dkdv_plan<false>(g);
  if (g.Le >= 2) {
    // the pooled-token reduction, with the dK/dV work lists built beside it
    int tokens_hi = 0;
    for (int l = 3; l <= g.Le; ++l) tokens_hi += g.rows[l];
    LaunchTimer timer(kBwdReduce, stream);
    reduce_and_order<<<g.bh + (g.rows[2] + tokens_hi) * g.bh, 256, 0, stream>>>(
        col_ptr, perm, ws.part_k, ws.part_v, ws.gk, ws.gv, ws.items, ws.splits, ws.split_done, g, cg, dkdv_bounds(g),
        pl.S, pl.walk, tokens_hi);
  }
  {
    LaunchTimer timer(kBwdDkdv, stream);
    launch_dkdv<false>(g, cg, q, k, v, lse, dout, pk, pv, col_ptr, perm, dk, dv, ws, pl, g.Le >= 2, stream);
  }
  return hipGetLastError();
}

hipError_t launch_attn_bwd_complement(const Geom& g, const CscGeom& cg, const CompGeom& cm, const PartGeom& pg,
                                      const void* q, const void* k, const void* v, const void* o, const float* lse,
                                      const void* dout, const void* pk, const void* pv, const int32_t* idx,
                                      const int32_t* comp, const int32_t* col_ptr, const int32_t* perm, void* dq,
                                      void* dk, void* dv, const BwdWs& ws, hipStream_t stream) {
  const int groups = g.bh * ((g.rows[1] + 15) / 16);
  {
    LaunchTimer timer(kBwdDq, stream);
    auto kernel = bwd_dq_bf16<1, kMaxComplement, true>;
    kernel<<<persistent_grid((const void*)kernel, 256, groups), 256, 0, stream>>>(
        (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, (const bf16_t*)o, lse, (const bf16_t*)dout,
        (const bf16_t*)pk, (const bf16_t*)pv, idx, (bf16_t*)dq, ws.delta, nullptr, nullptr, comp, g, cm);
  }
  hipError_t e = launch_comp_grads(g, cg, pg, q, dout, lse, ws.delta, pk, pv, idx, col_ptr, perm, ws.part_k, ws.gk,
                                   ws.gv, stream);
  if (e != hipSuccess) return e;
  {
    LaunchTimer timer(kBwdDkdv, stream);
    launch_dkdv<true>(g, cg, q, k, v, lse, dout, pk, pv, col_ptr, perm, dk, dv, ws, dkdv_plan<true>(g), false,
                      stream);
  }
  return hipGetLastError();
}

}  // namespace llsa
