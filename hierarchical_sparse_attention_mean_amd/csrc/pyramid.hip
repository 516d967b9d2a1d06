// pyramid.hip -- hierarchical compression: mean pooling of Q, K, V into L fp32 levels.
//
// Method: X^(l)[j] = (1/B) * sum_{t<B} X^(l-1)[jB + t], X^(0) = X, l = 1..L
// [LLSA review (pith.science, arXiv 2512.16615), "Core claim" and "What carries the argument"].
//
// Design (HBM-bound streaming reduction, read once, all levels in one pass):
//   * One 256-thread workgroup owns one level-3 unit (16 chunks of 256 raw tokens) of one tensor of
//     one slice when L >= 3, else one level-2 unit (or one 256-token chunk when L = 1).
//   * Per chunk each thread sums 8 rows x 8 dims (16-byte loads), pairs with its partner lane for the
//     16-row level-1 mean, writes it, and the level-2 mean is formed from LDS; level 3 accumulates
//     in registers across the 16 chunks.  The next chunk is loaded before the current one is reduced.
//   * Levels >= 4 (n >= B^5) are pooled by a small follow-up kernel from level 3.
#include "common.hpp"
#include "launch.hpp"

namespace llsa {

namespace {

template <typename T>
struct ChunkRegs;

// bf16: 8 rows x 8 dims = 8 x 16 bytes per thread.
template <>
struct ChunkRegs<bf16_t> {
  uint4 r[8];
  __device__ void load(const bf16_t* base, int valid) {
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = valid ? ld16(base + j * kD) : make_uint4(0, 0, 0, 0);
  }
  __device__ void sum(float s[8]) const {
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t w[4] = {r[j].x, r[j].y, r[j].z, r[j].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[2 * e] += __uint_as_float(w[e] << 16);
        s[2 * e + 1] += __uint_as_float(w[e] & 0xFFFF0000u);
      }
    }
  }
};

// fp32: 8 rows x 8 dims = 16 x 16 bytes per thread.
template <>
struct ChunkRegs<float> {
  float4 r[16];
  __device__ void load(const float* base, int valid) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      r[2 * j] = valid ? *reinterpret_cast<const float4*>(base + j * kD) : make_float4(0, 0, 0, 0);
      r[2 * j + 1] = valid ? *reinterpret_cast<const float4*>(base + j * kD + 4) : make_float4(0, 0, 0, 0);
    }
  }
  __device__ void sum(float s[8]) const {
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      s[0] += r[2 * j].x; s[1] += r[2 * j].y; s[2] += r[2 * j].z; s[3] += r[2 * j].w;
      s[4] += r[2 * j + 1].x; s[5] += r[2 * j + 1].y; s[6] += r[2 * j + 1].z; s[7] += r[2 * j + 1].w;
    }
  }
};

// grid.x = units per slice, grid.y = slice, grid.z = tensor (0 = Q, 1 = K, 2 = V)
template <typename T>
__global__ __launch_bounds__(256) void pool_levels123(const T* __restrict__ q, const T* __restrict__ k,
                                                      const T* __restrict__ v, float* __restrict__ pq,
                                                      float* __restrict__ pk, float* __restrict__ pv, Geom g,
                                                      int chunks_per_wg) {
  __shared__ float l1s[16][kD];
  const int tensor = blockIdx.z, slice = blockIdx.y, wg = blockIdx.x;
  const T* src = (tensor == 0 ? q : tensor == 1 ? k : v) + (size_t)slice * g.n * kD;
  float* dst = (tensor == 0 ? pq : tensor == 1 ? pk : pv) + (size_t)slice * g.R * kD;
  const int t = threadIdx.x;
  const int dim0 = 8 * (t & 7), half = (t >> 3) & 1, u1 = t >> 4;
  const int n1 = g.rows[1];
  const float inv = 1.0f / (float)kB;

  float acc3 = 0.f;
  ChunkRegs<T> cur, nxt;
  {
    const int gc = wg * chunks_per_wg;
    const int valid = (16 * gc + u1) < n1;
    cur.load(src + ((size_t)256 * gc + u1 * 16 + half * 8) * kD + dim0, valid);
  }
  for (int c = 0; c < chunks_per_wg; ++c) {
    const int gc = wg * chunks_per_wg + c;
    const int row1 = 16 * gc + u1;
    if (c + 1 < chunks_per_wg) {
      const int valid = (row1 + 16) < n1;
      nxt.load(src + ((size_t)256 * (gc + 1) + u1 * 16 + half * 8) * kD + dim0, valid);
    }
    float s[8];
    cur.sum(s);
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] += shfl_xor_f(s[e], 8);
    float m[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) m[e] = s[4 * half + e] * inv;
    if (row1 < n1)
      *reinterpret_cast<float4*>(dst + (size_t)(g.off[1] + row1) * kD + dim0 + 4 * half) =
          make_float4(m[0], m[1], m[2], m[3]);
    if (g.L >= 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) l1s[u1][dim0 + 4 * half + e] = m[e];
      __syncthreads();
      if (t < kD) {
        float x = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) x += l1s[r][t];
        x *= inv;
        dst[(size_t)(g.off[2] + gc) * kD + t] = x;
        acc3 += x;
      }
      __syncthreads();
    }
    if (c + 1 < chunks_per_wg) cur = nxt;
  }
  if (g.L >= 3 && t < kD) dst[(size_t)(g.off[3] + wg) * kD + t] = acc3 * inv;
}

// Level l >= 4 from level l-1: grid.x = rows of level l, grid.y = slice, grid.z = tensor; 64 threads.
__global__ __launch_bounds__(64) void pool_up(float* __restrict__ pq, float* __restrict__ pk,
                                              float* __restrict__ pv, Geom g, int level) {
  const int tensor = blockIdx.z, slice = blockIdx.y, j = blockIdx.x, t = threadIdx.x;
  float* base = (tensor == 0 ? pq : tensor == 1 ? pk : pv) + (size_t)slice * g.R * kD;
  const float* src = base + (size_t)(g.off[level - 1] + j * kB) * kD + t;
  float x = 0.f;
#pragma unroll
  for (int r = 0; r < kB; ++r) x += src[r * kD];
  base[(size_t)(g.off[level] + j) * kD + t] = x * (1.0f / (float)kB);
}

}  // namespace

hipError_t launch_pyramid(const Geom& g, int dtype_bf16, const void* q, const void* k, const void* v, float* pq,
                          float* pk, float* pv, hipStream_t stream) {
  int chunks, units;
  if (g.L >= 3) {
    chunks = 16;
    units = g.rows[3];
  } else if (g.L == 2) {
    chunks = 1;
    units = g.rows[2];
  } else {
    chunks = 1;
    units = (g.rows[1] + 15) / 16;
  }
  dim3 grid(units, g.bh, 3);
  {
    LaunchTimer timer(kPool, stream);
    if (dtype_bf16)
      pool_levels123<bf16_t><<<grid, 256, 0, stream>>>((const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, pq,
                                                        pk, pv, g, chunks);
    else
      pool_levels123<float><<<grid, 256, 0, stream>>>((const float*)q, (const float*)k, (const float*)v, pq, pk,
                                                       pv, g, chunks);
  }
  for (int l = 4; l <= g.L; ++l) {
    LaunchTimer timer(kPool, stream);
    pool_up<<<dim3(g.rows[l], g.bh, 3), 64, 0, stream>>>(pq, pk, pv, g, l);
  }
  return hipGetLastError();
}

}  // namespace llsa
