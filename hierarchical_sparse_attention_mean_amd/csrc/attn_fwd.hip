// attn_fwd.hip -- sparse block attention with hierarchical KV enrichment, forward.
//
// Method [LLSA review (pith.science, arXiv 2512.16615), "Core claim", "What carries the argument",
// abstract]: a raw query in fine block i attends (a) the B raw tokens of each of the K level-1 blocks
// in idx row i and (b) for l = 1..L_e, the K level-l pooled tokens kept by its level-l ancestor unit
// i / B^(l-1), whose logits carry + l*ln B (weight B^l).  Only sparse indices are read.
//
// bf16 design (one wavefront = one fine query block of 16 queries at a time, persistent):
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 with K rows as the A operand and Q rows as the B operand.
//     Its result leaves every lane holding 4 keys x 1 query, which is exactly the B-operand layout of
//     O^T = V^T P^T, so probabilities never leave registers.
//   * Gathered K and V rows are loaded with coalesced instructions (each quarter-wave reads whole 128-byte
//     lines) and put into operand order through wave-private LDS tiles: K read back as the MFMA A operand,
//     V^T read with ds_read_b64_tr_b16 (transposed 4x16 reads).  Loading the operands directly in MFMA
//     order would make each quarter-wave touch 16 rows, and the vector L1 is bound by such accesses.
//   * Keys go 32 per stage: two fine blocks, or 32 enrichment tokens (rows of the bf16 copy of the pooled
//     pyramid) with a per-entry logit bias that is -inf past the end of the list.
//   * Online softmax in the log2 domain with fp32 running max / sum; O rounded to bf16 at the end,
//     natural-log LSE stored for the backward pass.
//   * Persistent waves: each XCD sweeps a contiguous range of fine blocks with all its resident waves (for a
//     row-major token grid, in bands of four grid rows, so that a workgroup's waves run blocks one row apart,
//     whose selections overlap), and each wave pipelines its blocks' stages back to back (the next block's
//     first stage is in flight while the current block finishes; its Q rows and indices are copied to LDS a
//     whole block ahead).
//   * The complement reading of the enrichment (launch_attn_fwd_complement) is the same kernel with its
//     entry table pointing into the complement lists (up to 576 entries per fine block).
// bf16 pair design (attn_fwd_pair_bf16, the selected-token reading when n_1 is even, K <= 32 and K L_e <= 64):
// one wavefront = two fine blocks, each its own 16-query tile and online softmax, walking the union of the two
// blocks' entry lists once -- the gathered K and V rows of a stage, their LDS tiles and the transposed V reads
// serve both tiles, and an entry a block does not attend gets bias -inf in its tile.  With a token grid the two
// blocks are one grid row apart, where selections overlap most, and the union has about 40 % fewer rows than the
// two lists.
// fp32 design: same wavefront-per-block mapping on the VALU (lane = query x 16-dim quarter), for the
// small fp32 workloads that need 1e-4 agreement.
#include "common.hpp"
#include "entries.hpp"
#include "launch.hpp"
#include "persist.hpp"

namespace llsa {

namespace {

constexpr int kLd = kD + 8;  // LDS row stride (bf16 elements): 144 bytes, 16-byte aligned rows

struct Softmax {
  float m = -INFINITY;  // reference max (log2 domain), identical in the 4 lanes of a query
  float l = 0.f;        // this lane's partial running sum of 2^(x - m)
  bool first = true;    // wave-uniform: no logits folded in yet
  f32x4 acc[4];         // O^T[d = 16t + 4g + r][query c]

  __device__ void init() {
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Folds a new block of N logits of this lane's query into the running state and returns their
  // probabilities (relative to the running reference max) in p.  The reference max only moves when some
  // query of the wave has grown by more than 2^8 (log2 domain), so the accumulator rescale -- a round trip
  // of the MFMA accumulators through the VALU -- is rare; unnormalised probabilities stay below 2^8.
  template <int N>
  __device__ void update(const float* x, float* p) {
    float mx = x[0];
#pragma unroll
    for (int e = 1; e < N; ++e) mx = fmaxf(mx, x[e]);
    mx = group_max(mx);
    if (first) {
      m = mx;
      first = false;
    } else if (__ballot(mx > m + 8.0f)) {
      const float m_new = fmaxf(m, mx);
      const float alpha = fast_exp2(m - m_new);
      l *= alpha;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[t][r] *= alpha;
      m = m_new;
    }
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < N; ++e) {
      p[e] = fast_exp2(x[e] - m);
      ps += p[e];
    }
    l += ps;
  }

  // 32 keys: x[r] = key 4g+r of tile 0, x[4+r] = key 4g+r of tile 1; V rows 0..31 in the LDS tile.
  __device__ void step32(const float x[8], const bf16_t* vt, int c, int gq) {
    float p[8];
    update<8>(x, p);
    uint4 pu;
    pu.x = pack_bf16x2(p[0], p[1]);
    pu.y = pack_bf16x2(p[2], p[3]);
    pu.z = pack_bf16x2(p[4], p[5]);
    pu.w = pack_bf16x2(p[6], p[7]);
    const bf16x8 pb = as_bf16x8(pu);
    const bf16_t* r0 = vt + (4 * gq + (c >> 2)) * kLd + 4 * (c & 3);
    const bf16_t* r1 = r0 + 16 * kLd;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const bf16x8 va = cat4(lds_read_tr16(r0 + 16 * t), lds_read_tr16(r1 + 16 * t));
      acc[t] = mfma_bf16_k32(va, pb, acc[t]);
    }
  }
};

// Persistent kernel: grid = 8 * (workgroups resident per XCD), 256 threads; each wave runs the fine blocks
// of its xcd_sweep() back to back (wave slot 4 * (b / 8) + w of its XCD).  Its stage list is the concatenation of the blocks' stages, and the loads
// of stage t+1 (possibly the next block's first stage) are in flight while stage t is consumed.  The next
// block's Q rows, selection row and enrichment entries are copied into a second set of LDS buffers a whole
// block ahead, with DMA loads that hold no registers.  So the latency chain index -> gather -> product of
// one block hides behind the work of the previous one.
// kMaxC: enrichment entries per fine block the LDS holds; kComp: the complement reading (entries from the
// complement lists `esrc`, laid out by `cm`) instead of the selected tokens (entries from the selection `idx`).
template <int kMaxC, bool kComp>
__global__ __launch_bounds__(256, 3) void attn_fwd_bf16(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                     const bf16_t* __restrict__ v, const bf16_t* __restrict__ pk,
                                                     const bf16_t* __restrict__ pv, const int32_t* __restrict__ idx,
                                                     const int32_t* __restrict__ esrc, bf16_t* __restrict__ o,
                                                     float* __restrict__ lse, Geom g, CompGeom cm) {
  __shared__ __attribute__((aligned(16))) bf16_t vs[4][32 * kLd];      // V tile (read transposed)
  __shared__ __attribute__((aligned(16))) bf16_t ks[4][32 * kLd];      // K tile (read as MFMA A operand)
  __shared__ __attribute__((aligned(16))) bf16_t qs[4][16 * kD];       // Q rows of the next block
  __shared__ __attribute__((aligned(16))) int is1[4][2][32];           // level-1 selection row, two slots
  __shared__ __attribute__((aligned(16))) int es[4][2][kMaxC];         // enrichment entries' block indices
  __shared__ __attribute__((aligned(16))) EntryTabT<kMaxC> tab;        // per-entry constants (shared)
  const int lane = threadIdx.x & 63, c = lane & 15, gq = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (kComp)
    fill_entry_tab_complement(g, cm, tab);
  else
    fill_entry_tab(g, tab);
  const Sweep wb = xcd_sweep(g.bh * g.rows[1], 4 * (blockIdx.x / 8) + w, 4 * (gridDim.x / 8));
  if (wb.count == 0) return;  // no workgroup barrier is used below
  bf16_t* vt = vs[w];
  bf16_t* kt = ks[w];
  const Plan plan = make_plan(g, kComp ? cm.total : g.K * g.Le);
  const int nst = plan.nstages;
  const size_t slice_elems = (size_t)g.n * kD, slice_rows = (size_t)g.R * kD;
  const size_t esrc_slice = kComp ? (size_t)cm.slice : (size_t)g.R * g.K;
  const float sl2 = g.scale_log2;

  // Fine block of sweep position ip within a slice: with a token grid (g.gpr key-block groups, 4 g.gpr fine
  // blocks per grid row), bands of four grid rows taken column by column, so that a workgroup's four waves,
  // which take consecutive positions, run fine blocks one grid row apart -- their selections overlap, and the
  // shared key rows hit in the CU's L1; rows past the last whole band, and problems without a grid, in order.
  const int brow = 4 * g.gpr, bband = 4 * brow, bbanded = g.gpr > 0 ? g.rows[1] / bband * bband : 0;
  auto sweep_block = [&](int ip) {
    if (ip >= bbanded) return ip;
    const int b0 = ip / bband * bband, within = ip - b0;
    return b0 + (within & 3) * brow + (within >> 2);
  };
  // copy the inputs of the wave's j-th block (clamped to the last) into slot p (Q: the single Q slot)
  auto prefetch = [&](int j, int p) {
    const int gb = wb.first + wb.stride * min(j, wb.count - 1);
    const int slice = uniform(gb / g.rows[1]), i = sweep_block(gb - slice * g.rows[1]);
    const bf16_t* qrows = q + slice * slice_elems + (size_t)16 * i * kD;  // 2 KB, contiguous
    lds_dma16_nt(qrows + 8 * lane, &qs[w][0]);
    lds_dma16_nt(qrows + 512 + 8 * lane, &qs[w][512]);
    const int32_t* I = idx + (size_t)slice * g.R * g.K;
    if (lane < g.K) lds_dma4(I + (size_t)(g.off[1] + i) * g.K + lane, &is1[w][p][0]);
    const int32_t* E = esrc + slice * esrc_slice;
#pragma unroll
    for (int jj = 0; jj < kMaxC / 64; ++jj) {
      if (64 * jj < plan.ncoarse) {
        const int e = min(lane + 64 * jj, plan.ncoarse - 1);
        lds_dma4(E + tab.pos0[e] + (i >> tab.shift[e]) * tab.stride[e], &es[w][p][64 * jj]);
      }
    }
  };
  auto block_slice = [&](int j) { return uniform((wb.first + wb.stride * j) / g.rows[1]); };

  // stage s of the block in slot p (slice `slice`), coalesced (see issue_stage_coalesced)
  auto issue = [&](int p, int slice, int s, Stage& st) {
    issue_stage_coalesced(plan, s, g.K, is1[w][p], es[w][p], tab.row0, k + slice * slice_elems,
                          v + slice * slice_elems, pk + slice * slice_rows, pv + slice * slice_rows, lane, st);
  };

  int par = 0;                       // slot of the block being consumed
  int cj = 0, cs = 0;                // block / stage being consumed
  int ij = 0, is = 0;                // block / stage last issued
  int cslice = block_slice(0), nslice = block_slice(min(1, wb.count - 1));
  uint4 q0, q1;
  // Q operands of the block whose rows sit in the Q slot; the slot is refilled right after, so the reads
  // must have completed before the next DMA is issued
  auto read_q = [&]() {
    const bf16_t* qr = &qs[w][c * kD + 8 * gq];
    q0 = *reinterpret_cast<const uint4*>(qr);
    q1 = *reinterpret_cast<const uint4*>(qr + 32);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };
  prefetch(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  read_q();
  prefetch(1, 1);

  Softmax sm;
  sm.init();

  auto issue_next = [&](Stage& st) {
    if (++is == nst) {
      is = 0;
      ++ij;
    }
    if (ij >= wb.count)
      issue(par, cslice, nst - 1, st);  // past the end: an in-bounds reload that is never consumed
    else if (is == 0) {
      // first stage of the next block (the current one is in its last stage): its selection row was copied at
      // the start of the current block, and every stage issued since (nst - 1 of them) is newer
      if (nst >= 2)
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      issue(par ^ 1, nslice, 0, st);
    }
    else
      issue(par, cslice, is, st);
  };

  auto finish_block = [&]() {
    const int gb = wb.first + wb.stride * cj;
    const int i = sweep_block(gb - cslice * g.rows[1]);
    const float lt = group_sum(sm.l);
    const float inv = 1.0f / lt;
    // O^T[d][query c] -> bf16 rows of the K tile (query c, dims 16t + 4g .. +3), then coalesced 16-byte stores
    // of whole rows (lane l: query l/8 and 8 + l/8, bytes 16 (l%8))
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint2 u;
      u.x = pack_bf16x2(sm.acc[t][0] * inv, sm.acc[t][1] * inv);
      u.y = pack_bf16x2(sm.acc[t][2] * inv, sm.acc[t][3] * inv);
      *reinterpret_cast<uint2*>(kt + c * kLd + 16 * t + 4 * gq) = u;
    }
    bf16_t* ob = o + cslice * slice_elems + (size_t)16 * i * kD;
    const int ro = (lane >> 3) * kLd + 8 * (lane & 7), go = (lane >> 3) * kD + 8 * (lane & 7);
    const uint4 o0 = *reinterpret_cast<const uint4*>(kt + ro);
    const uint4 o1 = *reinterpret_cast<const uint4*>(kt + ro + 8 * kLd);
    st16_nt(ob + go, o0);
    st16_nt(ob + go + 8 * kD, o1);
    if (gq == 0) lse[(size_t)cslice * g.n + 16 * i + c] = (sm.m + log2f(lt)) * kLn2;
  };

  // One stage: the 32 key rows go to the K and V tiles; S^T = K Q^T for keys 0..15 (s0) and 16..31 (s1); the
  // logits take the stage's bias (fine stages: 0, or -inf for a missing second block when K is odd; enrichment
  // stages: 4l per entry -- level-l weight B^l = 16^l in the log2 domain -- and -inf past the end of the list).
  auto consume = [&](const Stage& st) {
    {
      // key rows 8m + lane/8 of the 32 keys, 16 bytes at column 8*(lane%8), into the K and V tiles
      const int o = (lane >> 3) * kLd + 8 * (lane & 7);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        *reinterpret_cast<uint4*>(kt + o + 8 * m * kLd) = st.r[m];
        *reinterpret_cast<uint4*>(vt + o + 8 * m * kLd) = st.r[4 + m];
      }
    }
    float4 b0, b1;
    if (cs < plan.nfine) {
      b0 = make_float4(0.f, 0.f, 0.f, 0.f);
      const float h1 = 2 * cs + 1 < g.K ? 0.f : -INFINITY;
      b1 = make_float4(h1, h1, h1, h1);
    } else {
      const int e0 = 32 * (cs - plan.nfine) + 4 * gq;
      b0 = *reinterpret_cast<const float4*>(&tab.bias[e0]);
      b1 = *reinterpret_cast<const float4*>(&tab.bias[e0 + 16]);
    }
    // A operands: key row c and 16 + c, dims 8g..8g+7 and 32+8g..32+8g+7
    const bf16_t* kr = kt + c * kLd + 8 * gq;
    const bf16x8 k00 = *reinterpret_cast<const bf16x8*>(kr), k01 = *reinterpret_cast<const bf16x8*>(kr + 32);
    const bf16x8 k10 = *reinterpret_cast<const bf16x8*>(kr + 16 * kLd);
    const bf16x8 k11 = *reinterpret_cast<const bf16x8*>(kr + 16 * kLd + 32);
    const bf16x8 qa0 = as_bf16x8(q0), qa1 = as_bf16x8(q1);
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    s0 = mfma_bf16_k32(k00, qa0, s0);
    s0 = mfma_bf16_k32(k01, qa1, s0);
    s1 = mfma_bf16_k32(k10, qa0, s1);
    s1 = mfma_bf16_k32(k11, qa1, s1);
    const float x[8] = {fmaf(s0[0], sl2, b0.x), fmaf(s0[1], sl2, b0.y), fmaf(s0[2], sl2, b0.z), fmaf(s0[3], sl2, b0.w),
                        fmaf(s1[0], sl2, b1.x), fmaf(s1[1], sl2, b1.y), fmaf(s1[2], sl2, b1.z), fmaf(s1[3], sl2, b1.w)};
    sm.step32(x, vt, c, gq);
    if (++cs == nst) {
      finish_block();
      cs = 0;
      if (++cj < wb.count) {
        par ^= 1;
        cslice = nslice;
        nslice = block_slice(min(cj + 1, wb.count - 1));
        read_q();
        prefetch(cj + 1, par ^ 1);
        sm = Softmax();
        sm.init();
      }
    }
  };

  const int T = uniform(wb.count * nst);
  Stage A, B;
  issue(0, cslice, 0, A);
  for (int t = 0; t < T; t += 2) {
    issue_next(B);
    consume(A);
    issue_next(A);
    if (t + 1 < T) consume(B);
  }
}

// Two fine blocks per wavefront.  With a token grid the pair is vertical -- blocks i and i + (blocks per grid row),
// whose selections overlap most (two fine blocks one grid row apart keep about 6.8 of 8 key blocks in common on
// 2-D fields) -- else blocks 2p and 2p + 1.  The wave walks the union of the two blocks' entry lists once: every
// stage's 32 K and V rows go through the LDS tiles once and serve both 16-query tiles, each with its own online
// softmax; an entry the tile's block does not attend carries logit bias -inf there (probability exactly 0), so
// each tile computes the same sums as its block alone, in another order.
//   * Raw stages (two key blocks each): the blocks both keep, two per stage, then one block only A keeps beside one
//     only B keeps (there are as many of each), then the odd shared block beside a padding slot.  The first stage
//     thus holds entries of both blocks, so both running maxima start finite.
//   * Enrichment stages: per level l >= 2 the K tokens of A's ancestor unit, and B's that A's unit does not keep
//     (nothing more when the two share the unit); then the level-1 tokens of the union of the picks; 32 per stage,
//     bias 4l where the tile's block attends the entry, -inf elsewhere and past the end.
// The union of pair j + 1 is built from its selection rows and entry indices (copied to LDS a pair ahead) just
// before its first stage is issued, into the second of two union slots, while pair j's last stage is consumed.
constexpr int kPairCoarse = 64;  // enrichment entries per block (K * L_e) the pair kernel takes
// A union entry: row (key block, or pyramid row) in bits 0..23, level in bits 24..29, and in bits 30 and 31 the
// tiles (A: 1, B: 2) whose block attends it.
__device__ __forceinline__ int tagged(int row, int level, int tiles) {
  return (int)((uint32_t)row | ((uint32_t)level << 24) | ((uint32_t)tiles << 30));
}

template <int kMaxPC>
__global__ __launch_bounds__(256, 2) void attn_fwd_pair_bf16(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                          const bf16_t* __restrict__ v, const bf16_t* __restrict__ pk,
                                                          const bf16_t* __restrict__ pv, const int32_t* __restrict__ idx,
                                                          bf16_t* __restrict__ o, float* __restrict__ lse, Geom g) {
  __shared__ __attribute__((aligned(16))) bf16_t vs[4][32 * kLd];      // V tile (read transposed)
  __shared__ __attribute__((aligned(16))) bf16_t ks[4][32 * kLd];      // K tile (read as MFMA A operand)
  __shared__ __attribute__((aligned(16))) bf16_t qs[4][32 * kD];       // Q rows of the next pair: A 0..15, B 16..31
  __shared__ __attribute__((aligned(16))) int is1[4][64];              // next pair's selection rows: A at 0, B at 32
  __shared__ __attribute__((aligned(16))) int es[4][2][kMaxPC];        // next pair's enrichment block indices (A, B)
  __shared__ __attribute__((aligned(16))) int ub[4][2][64];            // union slots: key block | tiles << 30
  __shared__ __attribute__((aligned(16))) int ue[4][2][2 * kMaxPC];    // union entries: row | level << 24 | tiles << 30
  __shared__ __attribute__((aligned(16))) EntryTabT<kMaxPC> tab;       // per-entry constants (shared)
  const int lane = threadIdx.x & 63, c = lane & 15, gq = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  fill_entry_tab(g, tab);
  // Sweep: XCD x (= block % 8, round-robin dispatch) owns the contiguous position range [plo, phi) of all slices'
  // pairs, and its per_xcd waves take it round by round: in round j, wave r runs position
  // plo + j per_xcd + (r + 148 j) mod per_xcd.  Each round covers one window of neighbouring pairs (kept in the
  // XCD's L2), a workgroup's four waves take four consecutive positions (their pairs share key rows in L1), and
  // the rotation by a multiple of four moves each wave to another column of the window every round: the pairs'
  // stage counts differ with the image (the unions differ), and a wave always on the same column would collect
  // one strip's.
  const int npairs = g.rows[1] / 2;
  const int per_xcd = 4 * (gridDim.x / 8), wr = 4 * (blockIdx.x / 8) + w, xcd = blockIdx.x % 8;
  const int plo = (int)((int64_t)xcd * g.bh * npairs / 8), phi = (int)((int64_t)(xcd + 1) * g.bh * npairs / 8);
  auto sweep_pos = [&](int j) { return plo + j * per_xcd + (wr + 148 * j) % per_xcd; };
  const int jfull = (phi - plo) / per_xcd;
  const int count = uniform(jfull + (sweep_pos(jfull) < phi ? 1 : 0));
  if (count == 0) return;  // no workgroup barrier is used below
  bf16_t* vt = vs[w];
  bf16_t* kt = ks[w];
  const int K = g.K, ncA = g.K * g.Le;
  const size_t slice_elems = (size_t)g.n * kD, slice_rows = (size_t)g.R * kD;
  const float sl2 = g.scale_log2;

  // Pair of sweep position ip within a slice.  Vertical pairs need an even number of grid rows; pair rows are then
  // taken in bands of four, column by column, so that a workgroup's four waves run pairs one pair row apart.
  const int R = 4 * g.gpr;
  const bool vert = g.gpr > 0 && (g.rows[1] / R) % 2 == 0;
  const int dB = vert ? R : 1;
  const int pband = 4 * R, pbanded = vert ? npairs / pband * pband : 0;
  auto pair_a = [&](int ip) {
    if (!vert) return 2 * ip;
    int prow, col;
    if (ip < pbanded) {
      const int b0 = ip / pband * pband, within = ip - b0;
      prow = b0 / R + (within & 3);
      col = within >> 2;
    } else {
      prow = ip / R;
      col = ip - prow * R;
    }
    return 2 * prow * R + col;
  };
  // slice and first block of the wave's j-th pair (clamped to the last), from a table of 64 pairs at a time held in
  // lanes (pair pchunk + lane): the divisions run once per 64 pairs, in parallel
  int pchunk = -64, lslice = 0, lia = 0;
  auto pair_of = [&](int j, int* slice, int* ia) {
    j = min(j, count - 1);
    if (j < pchunk || j >= pchunk + 64) {
      pchunk = j & ~63;
      const int pos = sweep_pos(min(pchunk + lane, count - 1));
      lslice = pos / npairs;
      lia = pair_a(pos - lslice * npairs);
    }
    *slice = __builtin_amdgcn_readlane(lslice, j - pchunk);
    *ia = __builtin_amdgcn_readlane(lia, j - pchunk);
  };
  // copy the inputs of the wave's j-th pair (clamped to the last) into the single set of next-pair buffers
  auto prefetch = [&](int j) {
    int slice, ia;
    pair_of(j, &slice, &ia);
    const int ib = ia + dB;
    const bf16_t* qa = q + slice * slice_elems + (size_t)16 * ia * kD;  // 2 KB each, contiguous
    const bf16_t* qb = q + slice * slice_elems + (size_t)16 * ib * kD;
    lds_dma16_nt(qa + 8 * lane, &qs[w][0]);
    lds_dma16_nt(qa + 512 + 8 * lane, &qs[w][512]);
    lds_dma16_nt(qb + 8 * lane, &qs[w][1024]);
    lds_dma16_nt(qb + 512 + 8 * lane, &qs[w][1536]);
    const int32_t* I = idx + (size_t)slice * g.R * g.K;
    if ((lane & 31) < K) lds_dma4(I + (size_t)(g.off[1] + (lane < 32 ? ia : ib)) * K + (lane & 31), &is1[w][0]);
    if (ncA > 0) {
      const int e = min(lane, ncA - 1);
      lds_dma4(I + tab.pos0[e] + (ia >> tab.shift[e]) * tab.stride[e], &es[w][0][0]);
      lds_dma4(I + tab.pos0[e] + (ib >> tab.shift[e]) * tab.stride[e], &es[w][1][0]);
    }
  };

  // Union of the pair whose inputs sit in the next-pair buffers, into union slot u; returns its raw stages and
  // enrichment entries.  Lane s < K holds A's value s, lane 32 + s B's value s.
  // Membership compares all K x K pairs at once: with Kp = K rounded up to a power of two, pair (i, j) is bit
  // i Kp + j of a wave ballot (one ballot per 64 pairs); A's value i is in B's list if row i has a bit set, B's value
  // j in A's list if column j has.
  const int lgK = K <= 1 ? 0 : 32 - __builtin_clz(K - 1), Kp = 1 << lgK;
  const int rounds = max(1, (Kp * Kp) >> 6);
  uint64_t colpat = 0;  // bit j of every row
  for (int t = 0; t < 64; t += Kp) colpat |= 1ull << t;
  const uint64_t rowpat = Kp >= 64 ? ~0ull : (1ull << Kp) - 1;
  auto member = [&](int val, bool act) {  // whether the other block's list holds val
    bool hit = false;
    const int rowbit = (lane & 31) * Kp;  // first bit of row i = lane (A's lanes)
    for (int r = 0; r < rounds; ++r) {
      const int pp = 64 * r + lane, i = pp >> lgK, j = pp & (Kp - 1);
      const int a = __shfl(val, min(i, 31), 64), b = __shfl(val, 32 + min(j, 31), 64);
      const uint64_t m = __ballot(i < K && j < K && a == b);
      if (lane < 32)
        hit |= (rowbit >> 6) == r && ((m >> (rowbit & 63)) & rowpat) != 0;
      else
        hit |= (m & (colpat << (lane & 31))) != 0;
    }
    return act && hit;
  };
  auto below = [&](uint64_t m) {  // set bits of m below this lane
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
  };
  auto build_union = [&](int u, int ia, int ib, int* nraw, int* nc) {
    const bool act = (lane & 31) < K, sideA = lane < 32;
    // raw key blocks
    const int val = act ? is1[w][lane] : -1;
    const bool hit = member(val, act);
    const uint64_t msh = __ballot(act && sideA && hit), mao = __ballot(act && sideA && !hit);
    const uint64_t mbo = __ballot(act && !sideA && !hit);
    const int ns = __popcll(msh), no = K - ns, hs = ns >> 1, odd = ns & 1;
    if (act && sideA && hit) {
      const int r = below(msh);
      const int slot = r < 2 * hs ? r : 2 * hs + 2 * no;
      ub[w][u][slot] = tagged(val, 0, 3);
      if (r >= 2 * hs) ub[w][u][slot + 1] = val;  // padding slot: attended by neither tile
    } else if (act && sideA) {
      ub[w][u][2 * hs + 2 * below(mao)] = tagged(val, 0, 1);
    } else if (act) {
      ub[w][u][2 * hs + 2 * below(mbo) + 1] = tagged(val, 0, 2);
    }
    *nraw = hs + no + odd;
    // enrichment entries: levels 2..L_e, then level 1 (the raw union's tokens)
    int base = 0;
    for (int l = 2; l <= g.Le; ++l) {
      const int off = level_off(g, l), sh = 4 * (l - 1);
      const int ev = act ? es[w][sideA ? 0 : 1][(l - 2) * K + (lane & 31)] : -1;
      if ((ia >> sh) == (ib >> sh)) {  // one ancestor unit: the same K tokens
        if (act && sideA) ue[w][u][base + lane] = tagged(off + ev, l, 3);
        base += K;
      } else {
        const bool eh = member(ev, act);
        const uint64_t meo = __ballot(act && !sideA && !eh);
        if (act && sideA) ue[w][u][base + lane] = tagged(off + ev, l, eh ? 3 : 1);
        else if (act && !eh) ue[w][u][base + K + below(meo)] = tagged(off + ev, l, 2);
        base += K + __popcll(meo);
      }
    }
    if (g.Le >= 1) {
      const int off = level_off(g, 1);
      if (act && sideA) ue[w][u][base + lane] = tagged(off + val, 1, hit ? 3 : 1);
      else if (act && !hit) ue[w][u][base + K + below(mbo)] = tagged(off + val, 1, 2);
      base += K + no;
    }
    *nc = base;
  };

  // stage s of the pair in union slot u (slice `slice`), coalesced: instruction m reads rows 8m .. 8m+7 of the
  // stage's 32 keys (lane l: row 8m + l/8, bytes 16 (l%8)) -- K into r[m], V into r[4+m]
  auto issue = [&](int u, int slice, int nraw, int nc, int s, Stage& st) {
    const char* kb;
    const char* vb;
    uint32_t off[4];
    const uint32_t sub = (uint32_t)lane >> 3, col = 16u * (lane & 7);
    if (s < nraw) {
      const int b0 = __builtin_amdgcn_readfirstlane(ub[w][u][2 * s]) & 0x3fffffff;
      const int b1 = __builtin_amdgcn_readfirstlane(ub[w][u][2 * s + 1]) & 0x3fffffff;
      kb = reinterpret_cast<const char*>(k + slice * slice_elems);
      vb = reinterpret_cast<const char*>(v + slice * slice_elems);
#pragma unroll
      for (int m = 0; m < 4; ++m) off[m] = (16u * (m < 2 ? b0 : b1) + 8u * (m & 1) + sub) * (2 * kD) + col;
    } else {
      const int e0 = 32 * (s - nraw) + (int)sub;
      kb = reinterpret_cast<const char*>(pk + slice * slice_rows);
      vb = reinterpret_cast<const char*>(pv + slice * slice_rows);
#pragma unroll
      for (int m = 0; m < 4; ++m) off[m] = (uint32_t)(ue[w][u][min(e0 + 8 * m, nc - 1)] & 0xffffff) * (2 * kD) + col;
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) st.r[m] = ld16(kb + off[m]);
#pragma unroll
    for (int m = 0; m < 4; ++m) st.r[4 + m] = ld16(vb + off[m]);
  };

  int par = 0;            // union slot of the pair being consumed
  int cj = 0, cs = 0;     // pair / stage being consumed
  int ij = 0, is = 0;     // pair / stage last issued
  int cslice, cia, nslice, nia;
  pair_of(0, &cslice, &cia);
  pair_of(1, &nslice, &nia);
  int craw, cnc, nraw_n = 0, nnc = 0;
  uint4 q0, q1, q2, q3;
  // Q operands of the pair whose rows sit in the Q slot; the slot is refilled right after, so the reads must have
  // completed before the next DMA is issued
  auto read_q = [&]() {
    const bf16_t* qr = &qs[w][c * kD + 8 * gq];
    q0 = *reinterpret_cast<const uint4*>(qr);
    q1 = *reinterpret_cast<const uint4*>(qr + 32);
    q2 = *reinterpret_cast<const uint4*>(qr + 16 * kD);
    q3 = *reinterpret_cast<const uint4*>(qr + 16 * kD + 32);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };
  prefetch(0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  read_q();
  build_union(0, cia, cia + dB, &craw, &cnc);
  wait_lds();  // the union is read (and the next-pair buffers refilled) next
  prefetch(1);
  int cnst = craw + (cnc + 31) / 32, nnst = 0;

  Softmax sa, sb;
  sa.init();
  sb.init();

  auto issue_next = [&](Stage& st) {
    if (++is == (ij == cj ? cnst : nnst)) {
      is = 0;
      ++ij;
      if (ij < count) {
        // first stage of the next pair (the current one is in its last stage): its inputs were copied at the
        // start of the current pair, and every stage issued since (cnst - 1 of them) is newer
        if (cnst >= 2)
          __builtin_amdgcn_s_waitcnt(0xf78);  // vmcnt(8), as a builtin so that the compiler's own waits see it
        else
          __builtin_amdgcn_s_waitcnt(0xf70);  // vmcnt(0)
        build_union(par ^ 1, nia, nia + dB, &nraw_n, &nnc);
        nnst = nraw_n + (nnc + 31) / 32;
      }
    }
    // past the end: an in-bounds reload (the current pair's first stage) that is never consumed
    const bool cur = ij >= count || ij == cj;
    issue(cur ? par : par ^ 1, cur ? cslice : nslice, cur ? craw : nraw_n, cur ? cnc : nnc,
          ij >= count ? 0 : is, st);
  };

  auto store_o = [&](const Softmax& sm, bf16_t* tile, int i) {
    const float lt = group_sum(sm.l);
    const float inv = 1.0f / lt;
    // O^T[d][query c] -> bf16 rows of the tile (query c, dims 16t + 4g .. +3), then coalesced 16-byte stores of
    // whole rows (lane l: query l/8 and 8 + l/8, bytes 16 (l%8))
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint2 x;
      x.x = pack_bf16x2(sm.acc[t][0] * inv, sm.acc[t][1] * inv);
      x.y = pack_bf16x2(sm.acc[t][2] * inv, sm.acc[t][3] * inv);
      *reinterpret_cast<uint2*>(tile + c * kLd + 16 * t + 4 * gq) = x;
    }
    bf16_t* ob = o + cslice * slice_elems + (size_t)16 * i * kD;
    const int ro = (lane >> 3) * kLd + 8 * (lane & 7), go = (lane >> 3) * kD + 8 * (lane & 7);
    const uint4 o0 = *reinterpret_cast<const uint4*>(tile + ro);
    const uint4 o1 = *reinterpret_cast<const uint4*>(tile + ro + 8 * kLd);
    st16_nt(ob + go, o0);
    st16_nt(ob + go + 8 * kD, o1);
    if (gq == 0) lse[(size_t)cslice * g.n + 16 * i + c] = (sm.m + log2f(lt)) * kLn2;
  };

  // One stage: the 32 key rows go to the K and V tiles; S^T = K Q^T for both tiles; each tile's logits take its
  // own bias; P^T of both tiles against the one transposed V read.  Returns true once the last pair is done; a
  // stage past the end (an in-bounds reload) only goes to the tiles.
  auto consume = [&](const Stage& st) {
    {
      const int o = (lane >> 3) * kLd + 8 * (lane & 7);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        *reinterpret_cast<uint4*>(kt + o + 8 * m * kLd) = st.r[m];
        *reinterpret_cast<uint4*>(vt + o + 8 * m * kLd) = st.r[4 + m];
      }
    }
    if (cj >= count) return true;
    float ba[8], bb[8];
    if (cs < craw) {
      const uint32_t t0 = (uint32_t)ub[w][par][2 * cs] >> 30, t1 = (uint32_t)ub[w][par][2 * cs + 1] >> 30;
      const float a0 = (t0 & 1) ? 0.f : -INFINITY, a1 = (t1 & 1) ? 0.f : -INFINITY;
      const float b0 = (t0 & 2) ? 0.f : -INFINITY, b1 = (t1 & 2) ? 0.f : -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ba[r] = a0; ba[4 + r] = a1;
        bb[r] = b0; bb[4 + r] = b1;
      }
    } else {
      const int e0 = 32 * (cs - craw) + 4 * gq;
      const int4 w0 = *reinterpret_cast<const int4*>(&ue[w][par][e0]);
      const int4 w1 = *reinterpret_cast<const int4*>(&ue[w][par][e0 + 16]);
      const int wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int e = e0 + (r & 3) + 16 * (r >> 2);
        const uint32_t x = (uint32_t)wv[r];
        const float bias = 4.0f * (float)((x >> 24) & 63);
        ba[r] = e < cnc && (x >> 30) & 1 ? bias : -INFINITY;
        bb[r] = e < cnc && (x >> 30) & 2 ? bias : -INFINITY;
      }
    }
    // A operands: key row c and 16 + c, dims 8g..8g+7 and 32+8g..32+8g+7
    const bf16_t* kr = kt + c * kLd + 8 * gq;
    const bf16x8 k00 = *reinterpret_cast<const bf16x8*>(kr), k01 = *reinterpret_cast<const bf16x8*>(kr + 32);
    const bf16x8 k10 = *reinterpret_cast<const bf16x8*>(kr + 16 * kLd);
    const bf16x8 k11 = *reinterpret_cast<const bf16x8*>(kr + 16 * kLd + 32);
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    f32x4 u0 = {0.f, 0.f, 0.f, 0.f}, u1 = {0.f, 0.f, 0.f, 0.f};
    s0 = mfma_bf16_k32(k00, as_bf16x8(q0), s0);
    s0 = mfma_bf16_k32(k01, as_bf16x8(q1), s0);
    s1 = mfma_bf16_k32(k10, as_bf16x8(q0), s1);
    s1 = mfma_bf16_k32(k11, as_bf16x8(q1), s1);
    u0 = mfma_bf16_k32(k00, as_bf16x8(q2), u0);
    u0 = mfma_bf16_k32(k01, as_bf16x8(q3), u0);
    u1 = mfma_bf16_k32(k10, as_bf16x8(q2), u1);
    u1 = mfma_bf16_k32(k11, as_bf16x8(q3), u1);
    float xa[8], xb[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      xa[r] = fmaf(s0[r], sl2, ba[r]);
      xa[4 + r] = fmaf(s1[r], sl2, ba[4 + r]);
      xb[r] = fmaf(u0[r], sl2, bb[r]);
      xb[4 + r] = fmaf(u1[r], sl2, bb[4 + r]);
    }
    float pa[8], pb[8];
    sa.update<8>(xa, pa);
    sb.update<8>(xb, pb);
    uint4 wa, wb2;
    wa.x = pack_bf16x2(pa[0], pa[1]);
    wa.y = pack_bf16x2(pa[2], pa[3]);
    wa.z = pack_bf16x2(pa[4], pa[5]);
    wa.w = pack_bf16x2(pa[6], pa[7]);
    wb2.x = pack_bf16x2(pb[0], pb[1]);
    wb2.y = pack_bf16x2(pb[2], pb[3]);
    wb2.z = pack_bf16x2(pb[4], pb[5]);
    wb2.w = pack_bf16x2(pb[6], pb[7]);
    const bf16x8 pva = as_bf16x8(wa), pvb = as_bf16x8(wb2);
    const bf16_t* r0 = vt + (4 * gq + (c >> 2)) * kLd + 4 * (c & 3);
    const bf16_t* r1 = r0 + 16 * kLd;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const bf16x8 va = cat4(lds_read_tr16(r0 + 16 * t), lds_read_tr16(r1 + 16 * t));
      sa.acc[t] = mfma_bf16_k32(va, pva, sa.acc[t]);
      sb.acc[t] = mfma_bf16_k32(va, pvb, sb.acc[t]);
    }
    if (++cs == cnst) {
      store_o(sa, kt, cia);
      store_o(sb, vt, cia + dB);
      cs = 0;
      if (++cj >= count) return true;
      par ^= 1;
      cslice = nslice;
      cia = nia;
      craw = nraw_n;
      cnc = nnc;
      cnst = nnst;
      pair_of(cj + 1, &nslice, &nia);
      read_q();
      prefetch(cj + 1);
      sa = Softmax();
      sa.init();
      sb = Softmax();
      sb.init();
    }
    return false;
  };

  // Every trip runs both halves and the loop exits only at its end, so that each path into the loop header has the
  // same loads in flight (A's); a consume after the last pair only drains its stage (see consume).  An exit from
  // the middle would reach the header in the compiler's control flow with B's loads in flight, and its waits would
  // then treat B's registers as loading on every trip.
  Stage A, B;
  issue(par, cslice, craw, cnc, 0, A);
  for (;;) {
    issue_next(B);
    const bool d1 = consume(A);
    issue_next(A);
    const bool d2 = consume(B);
    if (d1 || d2) break;
  }
}

// fp32 path: wave per fine block, lane = (query c, dims 16g .. 16g+15), entries one at a time on the VALU.
__global__ __launch_bounds__(256) void attn_fwd_f32(const float* __restrict__ q, const float* __restrict__ k,
                                                    const float* __restrict__ v, const float* __restrict__ pk,
                                                    const float* __restrict__ pv, const int32_t* __restrict__ idx,
                                                    float* __restrict__ o, float* __restrict__ lse, Geom g) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, c = lane & 15, gq = lane >> 4;
  const int nb = g.bh * g.rows[1];
  const int gb = xcd_remap(blockIdx.x, gridDim.x) * 4 + w;
  if (gb >= nb) return;
  const int slice = gb / g.rows[1], i = gb - slice * g.rows[1];
  const size_t base = (size_t)slice * g.n * kD;
  const float* PK = pk + (size_t)slice * g.R * kD;
  const float* PV = pv + (size_t)slice * g.R * kD;
  const int32_t* I = idx + (size_t)slice * g.R * g.K;
  float qv[16];
  {
    const float4* p = reinterpret_cast<const float4*>(q + base + (size_t)(16 * i + c) * kD + 16 * gq);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const float4 x = p[m];
      qv[4 * m] = x.x; qv[4 * m + 1] = x.y; qv[4 * m + 2] = x.z; qv[4 * m + 3] = x.w;
    }
  }
  float mrun = -INFINITY, lrun = 0.f, acc[16];
#pragma unroll
  for (int d = 0; d < 16; ++d) acc[d] = 0.f;

  auto visit = [&](const float* krow, const float* vrow, float bias) {
    const float4* kp = reinterpret_cast<const float4*>(krow + 16 * gq);
    float dot = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const float4 x = kp[m];
      dot += qv[4 * m] * x.x + qv[4 * m + 1] * x.y + qv[4 * m + 2] * x.z + qv[4 * m + 3] * x.w;
    }
    const float z = group_sum(dot) * g.scale_log2 + bias;
    const float m_new = fmaxf(mrun, z);
    const float alpha = exp2f(mrun - m_new);
    const float p = exp2f(z - m_new);
    lrun = lrun * alpha + p;
    mrun = m_new;
    const float4* vp = reinterpret_cast<const float4*>(vrow + 16 * gq);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const float4 x = vp[m];
      acc[4 * m] = acc[4 * m] * alpha + p * x.x;
      acc[4 * m + 1] = acc[4 * m + 1] * alpha + p * x.y;
      acc[4 * m + 2] = acc[4 * m + 2] * alpha + p * x.z;
      acc[4 * m + 3] = acc[4 * m + 3] * alpha + p * x.w;
    }
  };

  const int32_t* I1 = I + (size_t)(g.off[1] + i) * g.K;
  for (int kk = 0; kk < g.K; ++kk) {
    const int b = I1[kk];
    for (int t = 0; t < kB; ++t) {
      const size_t row = base + (size_t)(16 * b + t) * kD;
      visit(k + row, v + row, 0.f);
    }
  }
  const int ncoarse = g.K * g.Le;
  for (int e = 0; e < ncoarse; ++e) {
    const int row = coarse_row(g, I, i, e);
    visit(PK + (size_t)row * kD, PV + (size_t)row * kD, 4.0f * (float)coarse_level(g, e));
  }
  const float inv = 1.0f / lrun;
  float4* op = reinterpret_cast<float4*>(o + base + (size_t)(16 * i + c) * kD + 16 * gq);
#pragma unroll
  for (int m = 0; m < 4; ++m)
    op[m] = make_float4(acc[4 * m] * inv, acc[4 * m + 1] * inv, acc[4 * m + 2] * inv, acc[4 * m + 3] * inv);
  if (gq == 0) lse[(size_t)slice * g.n + 16 * i + c] = (mrun + log2f(lrun)) * kLn2;
}

}  // namespace

hipError_t launch_attn_fwd(const Geom& g, int dtype_bf16, const void* q, const void* k, const void* v,
                           const void* pk, const void* pv, const int32_t* idx, void* o, float* lse,
                           hipStream_t stream) {
  const int nb = g.bh * g.rows[1];
  const int grid = (nb + 3) / 4;
  LaunchTimer timer(kAttnFwd, stream);
  if (dtype_bf16) {
    if (g.rows[1] % 2 == 0 && g.K <= 32 && g.K * g.Le <= kPairCoarse) {
      // two fine blocks per wave; two workgroups per CU (their LDS), which leaves room for the index transpose
      auto kernel = attn_fwd_pair_bf16<kPairCoarse>;
      kernel<<<max(8, persistent_grid((const void*)kernel, 256, (nb / 2 + 3) / 4) / 8 * 8), 256, 0, stream>>>(
          (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, (const bf16_t*)pk, (const bf16_t*)pv, idx,
          (bf16_t*)o, lse, g);
      return hipGetLastError();
    }
    // two thirds of the resident workgroups: as fast as a full load (the gathers are bound by the CU's vector
    // memory path, not by the number of waves), and it leaves room for a kernel on another stream -- the index
    // transpose, which needs only the selection, can run beside the forward
    auto kernel = attn_fwd_bf16<kMaxCoarse, false>;
    kernel<<<max(8, persistent_grid((const void*)kernel, 256, grid) * 2 / 3 / 8 * 8), 256, 0, stream>>>(
        (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, (const bf16_t*)pk, (const bf16_t*)pv, idx, idx,
        (bf16_t*)o, lse, g, CompGeom{});
  } else {
    attn_fwd_f32<<<grid, 256, 0, stream>>>((const float*)q, (const float*)k, (const float*)v, (const float*)pk,
                                           (const float*)pv, idx, (float*)o, lse, g);
  }
  return hipGetLastError();
}

hipError_t launch_attn_fwd_complement(const Geom& g, const CompGeom& cm, const void* q, const void* k,
                                      const void* v, const void* pk, const void* pv, const int32_t* idx,
                                      const int32_t* comp, void* o, float* lse, hipStream_t stream) {
  const int nb = g.bh * g.rows[1];
  LaunchTimer timer(kAttnFwd, stream);
  auto kernel = attn_fwd_bf16<kMaxComplement, true>;
  kernel<<<persistent_grid((const void*)kernel, 256, (nb + 3) / 4), 256, 0, stream>>>(
      (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, (const bf16_t*)pk, (const bf16_t*)pv, idx, comp,
      (bf16_t*)o, lse, g, cm);
  return hipGetLastError();
}

}  // namespace llsa
