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
#include "launch.hpp"

namespace llsa {

namespace {

constexpr int kLd = kD + 8;  // LDS row stride (bf16 elements): 144 bytes, 16-byte aligned rows

// Enrichment entry e (0 <= e < K*Le) -> (level, slot): levels 2..Le first, then level 1.
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

// Pyramid row (within the slice) of enrichment entry e for fine block i.
__device__ __forceinline__ int coarse_row(const Geom& g, const int32_t* I, int i, int e, int* level) {
  int l, s;
  coarse_entry(g, e, &l, &s);
  *level = l;
  const int unit = i >> (4 * (l - 1));  // i / B^(l-1), B = 16
  return g.off[l] + I[(size_t)(g.off[l] + unit) * g.K + s];
}

struct Softmax {
  float m = -INFINITY;  // running max (log2 domain), identical in the 4 lanes of a query
  float l = 0.f;        // this lane's partial running sum
  f32x4 acc[4];         // O^T[d = 16t + 4g + r][query c]

  __device__ void init() {
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // x: 8 logits (log2 domain) of this lane's query for keys {4g+r} of the two 16-key tiles; vt: LDS tile
  // of 32 value rows (row = 16*tile + key).
  __device__ void step(const float x[8], const bf16_t* vt, int c, int gq) {
    float mx = x[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, x[e]);
    mx = group_max(mx);
    const float m_new = fmaxf(m, mx);
    const float alpha = exp2f(m - m_new);
    float p[8], ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = exp2f(x[e] - m_new);
      ps += p[e];
    }
    l = l * alpha + ps;
    m = m_new;
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
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[t][r] *= alpha;
      const bf16x8 va = cat4(lds_read_tr16(r0 + 16 * t), lds_read_tr16(r1 + 16 * t));
      acc[t] = mfma_bf16_k32(va, pb, acc[t]);
    }
  }
};

// grid.x = ceil(bh * n_1 / 4); 256 threads; wave w handles fine block 4 * (remapped block id) + w.
__global__ __launch_bounds__(256) void attn_fwd_bf16(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                     const bf16_t* __restrict__ v, const float* __restrict__ pk,
                                                     const float* __restrict__ pv, const int32_t* __restrict__ idx,
                                                     bf16_t* __restrict__ o, float* __restrict__ lse, Geom g) {
  __shared__ __attribute__((aligned(16))) bf16_t vs[4][32 * kLd];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, c = lane & 15, gq = lane >> 4;
  const int nb = g.bh * g.rows[1];
  const int gb = xcd_remap(blockIdx.x, gridDim.x) * 4 + w;
  if (gb >= nb) return;  // no workgroup barrier is used below
  const int slice = gb / g.rows[1], i = gb - slice * g.rows[1];
  const size_t base = (size_t)slice * g.n * kD;
  const bf16_t* Qs = q + base;
  const bf16_t* Ks = k + base;
  const bf16_t* Vs = v + base;
  const float* PK = pk + (size_t)slice * g.R * kD;
  const float* PV = pv + (size_t)slice * g.R * kD;
  const int32_t* I = idx + (size_t)slice * g.R * g.K;
  bf16_t* vt = vs[w];

  // B operand of S^T: Q[16i + c][16g .. 16g+15]
  const uint4* qp = reinterpret_cast<const uint4*>(Qs + (size_t)(16 * i + c) * kD + 16 * gq);
  const bf16x8 qa0 = as_bf16x8(qp[0]), qa1 = as_bf16x8(qp[1]);

  Softmax sm;
  sm.init();
  const int32_t* I1 = I + (size_t)(g.off[1] + i) * g.K;
  const int kr = lane >> 1, half = lane & 1;  // LDS fill: row kr (0..31), dims 32*half .. +31

  for (int kk = 0; kk < g.K; kk += 2) {
    const int b0 = I1[kk];
    const bool has1 = kk + 1 < g.K;
    const int b1 = has1 ? I1[kk + 1] : b0;
    const uint4* k0 = reinterpret_cast<const uint4*>(Ks + (size_t)(16 * b0 + c) * kD + 16 * gq);
    const uint4* k1 = reinterpret_cast<const uint4*>(Ks + (size_t)(16 * b1 + c) * kD + 16 * gq);
    const bf16x8 a00 = as_bf16x8(k0[0]), a01 = as_bf16x8(k0[1]);
    const bf16x8 a10 = as_bf16x8(k1[0]), a11 = as_bf16x8(k1[1]);
    {
      const int blk = kr < 16 ? b0 : b1;
      const uint4* vp = reinterpret_cast<const uint4*>(Vs + (size_t)(16 * blk + (kr & 15)) * kD + 32 * half);
      const uint4 x0 = vp[0], x1 = vp[1], x2 = vp[2], x3 = vp[3];
      uint4* dst = reinterpret_cast<uint4*>(vt + kr * kLd + 32 * half);
      dst[0] = x0; dst[1] = x1; dst[2] = x2; dst[3] = x3;
    }
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    s0 = mfma_bf16_k32(a00, qa0, s0);
    s0 = mfma_bf16_k32(a01, qa1, s0);
    s1 = mfma_bf16_k32(a10, qa0, s1);
    s1 = mfma_bf16_k32(a11, qa1, s1);
    float x[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = s0[r] * g.scale_log2;
      x[4 + r] = has1 ? s1[r] * g.scale_log2 : -INFINITY;
    }
    sm.step(x, vt, c, gq);
  }

  // Enrichment tokens, 32 per step.
  const int ncoarse = g.K * g.Le;
  for (int e0 = 0; e0 < ncoarse; e0 += 32) {
    bf16x8 a[2][2];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const int e = e0 + 16 * t2 + c;
      int lvl;
      const int row = e < ncoarse ? coarse_row(g, I, i, e, &lvl) : g.off[1];
      const float4* src = reinterpret_cast<const float4*>(PK + (size_t)row * kD + 16 * gq);
      a[t2][0] = f32x8_to_bf16x8(src[0], src[1]);
      a[t2][1] = f32x8_to_bf16x8(src[2], src[3]);
    }
    {
      const int e = e0 + kr;
      uint4* dst = reinterpret_cast<uint4*>(vt + kr * kLd + 32 * half);
      if (e < ncoarse) {
        int lvl;
        const int row = coarse_row(g, I, i, e, &lvl);
        const float4* src = reinterpret_cast<const float4*>(PV + (size_t)row * kD + 32 * half);
        float4 f[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) f[m] = src[m];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          uint4 u;
          u.x = pack_bf16x2(f[2 * m].x, f[2 * m].y);
          u.y = pack_bf16x2(f[2 * m].z, f[2 * m].w);
          u.z = pack_bf16x2(f[2 * m + 1].x, f[2 * m + 1].y);
          u.w = pack_bf16x2(f[2 * m + 1].z, f[2 * m + 1].w);
          dst[m] = u;
        }
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) dst[m] = make_uint4(0, 0, 0, 0);
      }
    }
    f32x4 s[2];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      s[t2] = f32x4{0.f, 0.f, 0.f, 0.f};
      s[t2] = mfma_bf16_k32(a[t2][0], qa0, s[t2]);
      s[t2] = mfma_bf16_k32(a[t2][1], qa1, s[t2]);
    }
    float x[8];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = e0 + 16 * t2 + 4 * gq + r;
        int lvl, slot;
        coarse_entry(g, e, &lvl, &slot);
        // level-l weight B^l = 16^l -> + 4l in the log2 domain
        x[4 * t2 + r] = e < ncoarse ? s[t2][r] * g.scale_log2 + 4.0f * (float)lvl : -INFINITY;
      }
    }
    sm.step(x, vt, c, gq);
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
    int lvl;
    const int row = coarse_row(g, I, i, e, &lvl);
    visit(PK + (size_t)row * kD, PV + (size_t)row * kD, 4.0f * (float)lvl);
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
