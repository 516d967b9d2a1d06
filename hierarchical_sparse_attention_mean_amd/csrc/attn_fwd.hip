// attn_fwd.hip -- sparse block attention with hierarchical KV enrichment, forward.
//
// Method [LLSA review (pith.science, arXiv 2512.16615), "Core claim", "What carries the argument",
// abstract]: a raw query in fine block i attends (a) the B raw tokens of each of the K level-1 blocks
// in idx row i and (b) for l = 1..L_e, the K level-l pooled tokens kept by its level-l ancestor unit
// i / B^(l-1), whose logits carry + l*ln B (weight B^l).  Only sparse indices are read.
//
// bf16 design (one wavefront = one fine query block of 16 queries):
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 with K rows as the A operand and Q rows as the B operand,
//     both loaded straight from HBM/L2 into registers (each lane reads a 32-byte run of one row).  Its
//     result leaves every lane holding 4 keys x 1 query, which is exactly the B-operand layout of
//     O^T = V^T P^T, so probabilities never leave registers.
//   * V^T comes from a wave-private LDS tile read with ds_read_b64_tr_b16 (transposed 4x16 reads).
//   * Keys go two fine blocks (32 keys) per step; enrichment tokens (fp32 pyramid rows, rounded to
//     bf16 for the products) go 32 per step with a per-entry logit bias and a validity mask.
//   * Online softmax in the log2 domain with fp32 running max / sum; O rounded to bf16 at the end,
//     natural-log LSE stored for the backward pass.
//   * Four waves per workgroup take four consecutive fine blocks (siblings share candidate key blocks);
//     workgroup ids are remapped so that neighbouring workgroups run on the same XCD and share its L2.
// fp32 design: same wavefront-per-block mapping on the VALU (lane = query x 16-dim quarter), for the
// small fp32 workloads that need 1e-4 agreement.
#include "common.hpp"
#include "entries.hpp"
#include "launch.hpp"

namespace llsa {

namespace {

constexpr int kLd = kD + 8;  // LDS row stride (bf16 elements): 144 bytes, 16-byte aligned rows
constexpr int kMaxCoarse = 256;  // K * L_e enrichment entries per fine block (K <= 32, L_e <= 8)

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

  // 16 keys: x[r] = key 4g+r; V rows 0..15 in the LDS tile (16x16x16 product over the keys).
  __device__ void step16(const float x[4], const bf16_t* vt, int c, int gq) {
    float p[4];
    update<4>(x, p);
    const uint2 pu = make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
    bf16x4 pb;
    __builtin_memcpy(&pb, &pu, 8);
    const bf16_t* r0 = vt + (4 * gq + (c >> 2)) * kLd + 4 * (c & 3);
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = mfma_bf16_k16(lds_read_tr16(r0 + 16 * t), pb, acc[t]);
  }
};

// grid.x = ceil(bh * n_1 / 4); 256 threads; wave w handles fine block 4 * (remapped block id) + w.
__global__ __launch_bounds__(256, 3) void attn_fwd_bf16(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                     const bf16_t* __restrict__ v, const float* __restrict__ pk,
                                                     const float* __restrict__ pv, const int32_t* __restrict__ idx,
                                                     bf16_t* __restrict__ o, float* __restrict__ lse, Geom g) {
  __shared__ __attribute__((aligned(16))) bf16_t vs[4][32 * kLd];
  __shared__ int erows[4][kMaxCoarse];
  const int lane = threadIdx.x & 63, c = lane & 15, gq = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nb = g.bh * g.rows[1];
  const int gb = xcd_remap(blockIdx.x, gridDim.x) * 4 + w;
  if (gb >= nb) return;  // no workgroup barrier is used below
  const int slice = gb / g.rows[1], i = gb - slice * g.rows[1];
  const size_t base = (size_t)slice * g.n * kD;
  const float* PK = pk + (size_t)slice * g.R * kD;
  const float* PV = pv + (size_t)slice * g.R * kD;
  const int32_t* I = idx + (size_t)slice * g.R * g.K;
  const int32_t* I1 = I + (size_t)(g.off[1] + i) * g.K;
  bf16_t* vt = vs[w];
  int* erow = erows[w];
  const Plan plan = make_plan(g);

  // prologue: enrichment rows (to LDS), Q, and the first stage in flight
  stage_entry_rows(g, I, i, plan.ncoarse, lane, erow);
  // query-side B operands in both orders (natural for raw keys, coarse for pyramid rows)
  bf16x8 qa0, qa1, qc0, qc1;
  {
    uint4 u0, u1;
    load_natural(q + base, 16u * i + c, lane, u0, u1);
    qa0 = as_bf16x8(u0);
    qa1 = as_bf16x8(u1);
    load_coarse_bf16(q + base, 16u * i + c, lane, qc0, qc1);
  }
  const bf16_t* Kraw = k + base;
  const bf16_t* Vraw = v + base;

  Softmax sm;
  sm.init();

  auto consume_fine = [&](int s, const Stage& st) {
    const bool has1 = 2 * s + 1 < g.K;
    {
      // V rows 8m + lane/8 of the 32 keys, 16 bytes at column 8*(lane%8)
      bf16_t* dst = vt + (lane >> 3) * kLd + 8 * (lane & 7);
#pragma unroll
      for (int m = 0; m < 4; ++m) *reinterpret_cast<uint4*>(dst + 8 * m * kLd) = st.r[4 + m];
    }
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    s0 = mfma_bf16_k32(as_bf16x8(st.r[0]), qa0, s0);
    s0 = mfma_bf16_k32(as_bf16x8(st.r[1]), qa1, s0);
    s1 = mfma_bf16_k32(as_bf16x8(st.r[2]), qa0, s1);
    s1 = mfma_bf16_k32(as_bf16x8(st.r[3]), qa1, s1);
    float x[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = s0[r] * g.scale_log2;
      x[4 + r] = has1 ? s1[r] * g.scale_log2 : -INFINITY;
    }
    sm.step32(x, vt, c, gq);
  };
  auto consume_coarse = [&](int e0, const Stage& st) {
    {
      // V rows (fp32) -> bf16 LDS tile: instruction m brought entry 4m + lane/16, dims 4*(lane%16)..+3
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int row = 4 * m + (lane >> 4);
        float4 f;
        __builtin_memcpy(&f, &st.r[4 + m], 16);
        const uint2 u = e0 + row < plan.ncoarse ? make_uint2(pack_bf16x2(f.x, f.y), pack_bf16x2(f.z, f.w))
                                                : make_uint2(0u, 0u);
        *reinterpret_cast<uint2*>(vt + row * kLd + 4 * (lane & 15)) = u;
      }
    }
    bf16x8 a0, a1;
    coarse_ops(&st.r[0], a0, a1);
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f};
    s0 = mfma_bf16_k32(a0, qc0, s0);
    s0 = mfma_bf16_k32(a1, qc1, s0);
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = e0 + 4 * gq + r;
      // level-l weight B^l = 16^l -> + 4l in the log2 domain
      x[r] = e < plan.ncoarse ? s0[r] * g.scale_log2 + 4.0f * (float)coarse_level(g, e) : -INFINITY;
    }
    sm.step16(x, vt, c, gq);
  };

  // Stage s+1 is always issued (clamped to the last stage) before stage s is consumed, so that both
  // branches of every iteration leave the same loads in flight and the waits stay exact.
  auto consume = [&](int s, const Stage& st) {
    if (s < plan.nfine)
      consume_fine(s, st);
    else
      consume_coarse(16 * (s - plan.nfine), st);
  };
  const int last = plan.nstages - 1;
  Stage A, B;
  issue_stage<true>(plan, 0, I1, g.K, Kraw, Vraw, PK, PV, erow, lane, A);
  for (int s = 0; s < plan.nstages; s += 2) {
    issue_stage<true>(plan, min(s + 1, last), I1, g.K, Kraw, Vraw, PK, PV, erow, lane, B);
    consume(s, A);
    issue_stage<true>(plan, min(s + 2, last), I1, g.K, Kraw, Vraw, PK, PV, erow, lane, A);
    if (s + 1 < plan.nstages) consume(s + 1, B);
  }

  const float lt = group_sum(sm.l);
  const float inv = 1.0f / lt;
  bf16_t* orow = o + base + (size_t)(16 * i + c) * kD + 4 * gq;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    uint2 u;
    u.x = pack_bf16x2(sm.acc[t][0] * inv, sm.acc[t][1] * inv);
    u.y = pack_bf16x2(sm.acc[t][2] * inv, sm.acc[t][3] * inv);
    *reinterpret_cast<uint2*>(orow + 16 * t) = u;
  }
  if (gq == 0) lse[(size_t)slice * g.n + 16 * i + c] = (sm.m + log2f(lt)) * kLn2;
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
                           const float* pk, const float* pv, const int32_t* idx, void* o, float* lse,
                           hipStream_t stream) {
  const int nb = g.bh * g.rows[1];
  const int grid = (nb + 3) / 4;
  LaunchTimer timer(kAttnFwd, stream);
  if (dtype_bf16)
    attn_fwd_bf16<<<grid, 256, 0, stream>>>((const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, pk, pv, idx,
                                            (bf16_t*)o, lse, g);
  else
    attn_fwd_f32<<<grid, 256, 0, stream>>>((const float*)q, (const float*)k, (const float*)v, pk, pv, idx,
                                           (float*)o, lse, g);
  return hipGetLastError();
}

}  // namespace llsa
