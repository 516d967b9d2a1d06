// pyramid.hip -- hierarchical compression: mean pooling of Q, K, V into L fp32 levels.
//
// Method: X^(l)[j] = (1/B) * sum_{t<B} X^(l-1)[jB + t], X^(0) = X, l = 1..L
// [LLSA review (pith.science, arXiv 2512.16615), "Core claim" and "What carries the argument"].
//
// Design (HBM-bound streaming reduction, raw tensors read once):
//   * pool_levels12: one 256-thread workgroup per 256-token chunk (one level-2 unit) of one tensor of one
//     slice -- bh * n / 256 * 3 independent workgroups, enough to keep every CU's loads in flight.  Each
//     thread loads 8 rows x 8 dims (8 x 16 bytes, all issued at once), pairs with its partner lane for the
//     16-row level-1 mean, and the level-2 mean is formed from LDS.
//   * pool_levels123 (L >= 3, when its workgroups fit on the device at once): one workgroup per level-3 unit
//     walks the unit's 16 chunks as pool_levels12 does, the next chunk's loads in flight, and forms the level-3
//     row from its chunks' level-2 rows -- one launch fewer on the way to the selection.
//   * pool_up: level l >= 3 (>= 4 after pool_levels123) from level l - 1 (1/256 of the raw bytes and less).
//   * For bf16 problems the pooled K and V rows are also stored rounded to bf16 (the attention kernels'
//     operands -- their products round pooled tokens to bf16 anyway), so that the attention gathers read
//     128 bytes per pooled row instead of 256.
#include "common.hpp"
#include "launch.hpp"

namespace llsa {

namespace {

template <typename T>
struct ChunkRegs;

// bf16: 8 rows x 8 dims = 8 x 16 bytes per thread, non-temporal loads: the raw tensors are read once here, and
// the attention kernels then gather K and V from HBM with the caches left to their gathers (two-stream step at
// N = 65536: 0.906 -> 0.897 ms with Q non-temporal, then -> 0.864 ms for all three once the attention kernels'
// own once-read rows and outputs were non-temporal too).
template <>
struct ChunkRegs<bf16_t> {
  uint4 r[8];
  __device__ void load(const bf16_t* base, int valid) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (valid) {
        const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + j * kD));
        r[j] = make_uint4(x.x, x.y, x.z, x.w);
      } else {
        r[j] = make_uint4(0, 0, 0, 0);
      }
    }
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

// grid.x = 256-token chunks per slice, grid.y = slice, grid.z = tensor (0 = Q, 1 = K, 2 = V)
template <typename T>
__global__ __launch_bounds__(256) void pool_levels12(const T* __restrict__ q, const T* __restrict__ k,
                                                     const T* __restrict__ v, float* __restrict__ pq,
                                                     float* __restrict__ pk, float* __restrict__ pv,
                                                     bf16_t* __restrict__ pkh, bf16_t* __restrict__ pvh, Geom g) {
  __shared__ float l1s[16][kD];
  const int tensor = blockIdx.z, slice = blockIdx.y, gc = blockIdx.x;
  const T* src = (tensor == 0 ? q : tensor == 1 ? k : v) + (size_t)slice * g.n * kD;
  const size_t pbase = (size_t)slice * g.R * kD;
  float* dst = (tensor == 0 ? pq : tensor == 1 ? pk : pv) + pbase;
  bf16_t* dsth = tensor == 0 ? nullptr : (tensor == 1 ? pkh : pvh);
  if (dsth) dsth += pbase;
  const int t = threadIdx.x;
  const int dim0 = 8 * (t & 7), half = (t >> 3) & 1, u1 = t >> 4;
  const int row1 = 16 * gc + u1;
  const float inv = 1.0f / (float)kB;

  ChunkRegs<T> cur;
  cur.load(src + ((size_t)256 * gc + u1 * 16 + half * 8) * kD + dim0, row1 < g.rows[1]);
  float s[8];
  cur.sum(s);
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] += xor8_f(s[e]);
  float m[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) m[e] = s[4 * half + e] * inv;
  const int col = dim0 + 4 * half;
  if (row1 < g.rows[1]) {
    const size_t o = (size_t)(g.off[1] + row1) * kD + col;
    if (tensor == 2) {
      // the fp32 V pyramid: an output that no later step of a bf16 pass reads (the attention kernels read the
      // bf16 copy), stored non-temporally
      const u32x4 x = {__float_as_uint(m[0]), __float_as_uint(m[1]), __float_as_uint(m[2]), __float_as_uint(m[3])};
      __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(dst + o));
    } else {
      *reinterpret_cast<float4*>(dst + o) = make_float4(m[0], m[1], m[2], m[3]);
    }
    if (dsth) *reinterpret_cast<uint2*>(dsth + o) = make_uint2(pack_bf16x2(m[0], m[1]), pack_bf16x2(m[2], m[3]));
  }
  if (g.L >= 2) {
#pragma unroll
    for (int e = 0; e < 4; ++e) l1s[u1][col + e] = m[e];
    __syncthreads();
    if (t < kD / 2) {
      // two dims per thread, so that the bf16 copy is one 4-byte store
      float x0 = 0.f, x1 = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        x0 += l1s[r][2 * t];
        x1 += l1s[r][2 * t + 1];
      }
      x0 *= inv;
      x1 *= inv;
      const size_t o = (size_t)(g.off[2] + gc) * kD + 2 * t;
      *reinterpret_cast<float2*>(dst + o) = make_float2(x0, x1);
      if (dsth) *reinterpret_cast<uint32_t*>(dsth + o) = pack_bf16x2(x0, x1);
    }
  }
}

// Levels 1, 2 and 3 in one pass when L >= 3: one 256-thread workgroup per level-3 unit (4096 tokens, 16 chunks of
// 256) of one tensor of one slice walks its chunks in order, each exactly as pool_levels12 does, with the next
// chunk's loads in flight while the current one is reduced; the chunk's level-2 row also stays in LDS, and the
// level-3 row is their mean at the end, summed in the order pool_up uses (so the values are the same bits).
// grid.x = level-3 units per slice, grid.y = slice, grid.z = tensor.
template <typename T>
__global__ __launch_bounds__(256) void pool_levels123(const T* __restrict__ q, const T* __restrict__ k,
                                                      const T* __restrict__ v, float* __restrict__ pq,
                                                      float* __restrict__ pk, float* __restrict__ pv,
                                                      bf16_t* __restrict__ pkh, bf16_t* __restrict__ pvh, Geom g) {
  __shared__ float l1s[16][kD];
  __shared__ float l2s[kB][kD];
  const int tensor = blockIdx.z, slice = blockIdx.y, u3 = blockIdx.x;
  const T* src = (tensor == 0 ? q : tensor == 1 ? k : v) + (size_t)slice * g.n * kD;
  const size_t pbase = (size_t)slice * g.R * kD;
  float* dst = (tensor == 0 ? pq : tensor == 1 ? pk : pv) + pbase;
  bf16_t* dsth = tensor == 0 ? nullptr : (tensor == 1 ? pkh : pvh);
  if (dsth) dsth += pbase;
  const int t = threadIdx.x;
  const int dim0 = 8 * (t & 7), half = (t >> 3) & 1, u1 = t >> 4;
  const int col = dim0 + 4 * half;
  const float inv = 1.0f / (float)kB;
  auto chunk_src = [&](int gc) { return src + ((size_t)256 * gc + u1 * 16 + half * 8) * kD + dim0; };

  ChunkRegs<T> bufA, bufB;
  bufA.load(chunk_src(kB * u3), 1);
  auto one_chunk = [&](int c, ChunkRegs<T>& cur, ChunkRegs<T>& nxt) {
    const int gc = kB * u3 + c;
    if (c + 1 < kB) nxt.load(chunk_src(gc + 1), 1);
    float s[8];
    cur.sum(s);
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] += xor8_f(s[e]);
    float m[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) m[e] = s[4 * half + e] * inv;
    const int row1 = 16 * gc + u1;
    const size_t o = (size_t)(g.off[1] + row1) * kD + col;
    if (tensor == 2) {
      const u32x4 x = {__float_as_uint(m[0]), __float_as_uint(m[1]), __float_as_uint(m[2]), __float_as_uint(m[3])};
      __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(dst + o));
    } else {
      *reinterpret_cast<float4*>(dst + o) = make_float4(m[0], m[1], m[2], m[3]);
    }
    if (dsth) *reinterpret_cast<uint2*>(dsth + o) = make_uint2(pack_bf16x2(m[0], m[1]), pack_bf16x2(m[2], m[3]));
    __syncthreads();  // the previous chunk's level-2 reads of l1s are done
#pragma unroll
    for (int e = 0; e < 4; ++e) l1s[u1][col + e] = m[e];
    __syncthreads();
    if (t < kD / 2) {
      float x0 = 0.f, x1 = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        x0 += l1s[r][2 * t];
        x1 += l1s[r][2 * t + 1];
      }
      x0 *= inv;
      x1 *= inv;
      const size_t o2 = (size_t)(g.off[2] + gc) * kD + 2 * t;
      *reinterpret_cast<float2*>(dst + o2) = make_float2(x0, x1);
      if (dsth) *reinterpret_cast<uint32_t*>(dsth + o2) = pack_bf16x2(x0, x1);
      l2s[c][2 * t] = x0;
      l2s[c][2 * t + 1] = x1;
    }
  };
  for (int c = 0; c < kB; c += 2) {
    one_chunk(c, bufA, bufB);
    one_chunk(c + 1, bufB, bufA);
  }
  __syncthreads();
  if (t < kD) {
    float x = 0.f;
#pragma unroll
    for (int r = 0; r < kB; ++r) x += l2s[r][t];
    x *= inv;
    const size_t o3 = (size_t)(g.off[3] + u3) * kD + t;
    dst[o3] = x;
    if (dsth) dsth[o3] = f32_to_bf16(x);
  }
}

// Level l >= 3 from level l-1: grid.x = rows of level l, grid.y = slice, grid.z = tensor; 64 threads.
__global__ __launch_bounds__(64) void pool_up(float* __restrict__ pq, float* __restrict__ pk,
                                              float* __restrict__ pv, bf16_t* __restrict__ pkh,
                                              bf16_t* __restrict__ pvh, Geom g, int level) {
  const int tensor = blockIdx.z, slice = blockIdx.y, j = blockIdx.x, t = threadIdx.x;
  const size_t pbase = (size_t)slice * g.R * kD;
  float* base = (tensor == 0 ? pq : tensor == 1 ? pk : pv) + pbase;
  bf16_t* baseh = tensor == 0 ? nullptr : (tensor == 1 ? pkh : pvh);
  const float* src = base + (size_t)(g.off[level - 1] + j * kB) * kD + t;
  float x = 0.f;
#pragma unroll
  for (int r = 0; r < kB; ++r) x += src[r * kD];
  x *= 1.0f / (float)kB;
  const size_t o = (size_t)(g.off[level] + j) * kD + t;
  base[o] = x;
  if (baseh) baseh[pbase + o] = f32_to_bf16(x);
}

}  // namespace

hipError_t launch_pyramid(const Geom& g, int dtype_bf16, const void* q, const void* k, const void* v, float* pq,
                          float* pk, float* pv, void* pkh, void* pvh, hipStream_t stream) {
  bf16_t* kh = dtype_bf16 ? static_cast<bf16_t*>(pkh) : nullptr;
  bf16_t* vh = dtype_bf16 ? static_cast<bf16_t*>(pvh) : nullptr;
  // levels 1..3 in one launch (a level-3 unit per workgroup) when those workgroups all fit on the device at once
  // (one unit walks 16 chunks in turn, so a second round of them would double the time); else levels 1, 2 and
  // then one launch per level
  const void* k3 = dtype_bf16 ? (const void*)pool_levels123<bf16_t> : (const void*)pool_levels123<float>;
  const bool fused = g.L >= 3 && (int64_t)g.rows[3] * g.bh * 3 <= resident_workgroups(k3, 256);
  if (fused) {
    const dim3 grid3(g.rows[3], g.bh, 3);
    LaunchTimer timer(kPool, stream);
    if (dtype_bf16)
      pool_levels123<bf16_t><<<grid3, 256, 0, stream>>>((const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, pq,
                                                         pk, pv, kh, vh, g);
    else
      pool_levels123<float><<<grid3, 256, 0, stream>>>((const float*)q, (const float*)k, (const float*)v, pq, pk,
                                                        pv, kh, vh, g);
  } else {
    const dim3 grid((g.rows[1] + 15) / 16, g.bh, 3);
    LaunchTimer timer(kPool, stream);
    if (dtype_bf16)
      pool_levels12<bf16_t><<<grid, 256, 0, stream>>>((const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, pq,
                                                       pk, pv, kh, vh, g);
    else
      pool_levels12<float><<<grid, 256, 0, stream>>>((const float*)q, (const float*)k, (const float*)v, pq, pk,
                                                      pv, kh, vh, g);
  }
  for (int l = fused ? 4 : 3; l <= g.L; ++l) {
    LaunchTimer timer(kPool, stream);
    pool_up<<<dim3(g.rows[l], g.bh, 3), 64, 0, stream>>>(pq, pk, pv, kh, vh, g, l);
  }
  return hipGetLastError();
}

}  // namespace llsa
