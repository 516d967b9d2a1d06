// common.hpp -- device-side building blocks shared by the gfx950 kernels of the LLSA hot path.
//
// Lane layouts used throughout (64-lane wavefront, lane = 16*g + c, g = lane >> 4, c = lane & 15):
//   v_mfma_f32_16x16x32_bf16: A lane holds A[row c][k = 8g..8g+7], B lane holds B[k = 8g..8g+7][col c],
//                             D lane holds D[row 4g+r][col c], r = 0..3.
//   v_mfma_f32_16x16x16_bf16: same with k = 4g..4g+3.
//   v_mfma_f32_16x16x4_f32:   A lane holds A[row c][k = g], B lane holds B[k = g][col c], same D.
//   ds_read_b64_tr_b16:        inside each 16-lane group, output lane j element e is element (j % 4) of
//                             the 8-byte load addressed by lane 4e + j/4.  With lane i addressing
//                             &M[r0 + i/4][c0 + 4*(i%4)] of a row-major bf16 matrix M, lane j receives
//                             M[r0 + e][c0 + j], e = 0..3 -- a transposed 4x16 sub-block.
// Because a dot product may visit its k index in any order, A and B operands are always loaded with
// the same (permuted) k order, which lets every lane read contiguous 32-byte runs of a row.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace llsa {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef uint16_t bf16_t;

constexpr int kD = 64;      // head dim handled by the GPU kernels
constexpr int kB = 16;      // block / pooling factor handled by the GPU kernels
constexpr int kMaxLevels = 8;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Per-problem geometry passed by value to kernels.
struct Geom {
  int bh;                       // batch * heads
  int n;                        // raw tokens per slice
  int K;                        // top-k
  int L;                        // pooled levels
  int Le;                       // enrichment levels
  int R;                        // pyramid rows per slice
  int rows[kMaxLevels + 1];     // rows[l] = n / B^l (rows[0] = n)
  int off[kMaxLevels + 2];      // off[l] = first pyramid row of level l (l >= 1)
  float scale_log2;             // sigma * log2(e)
  float scale;                  // sigma
  int gpr;                      // dK/dV key-block groups per row of the token grid (0: no grid)
};

typedef __bf16 hbf16x2 __attribute__((ext_vector_type(2)));
typedef float hf32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair, round-to-nearest-even (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const hf32x2 x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, hbf16x2));
}

__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return (bf16_t)(pack_bf16x2(f, 0.f) & 0xFFFFu); }

// 2^x on the transcendental unit (v_exp_f32): no range reduction; exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x4 mfma_bf16_k32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_bf16_k16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32_k4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Transposed 4x16 bf16 read from LDS (see the layout note above).
__device__ __forceinline__ bf16x4 lds_read_tr16(const bf16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) bf16x4*)(p));
}

__device__ __forceinline__ bf16x8 cat4(bf16x4 a, bf16x4 b) {
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

// v of lane l ^ 8 (within each 16-lane row): a DPP row rotation by 8 on the VALU.
__device__ __forceinline__ float xor8_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128 /* row_ror:8 */, 0xf, 0xf, false));
}

// Reduce over the four 16-lane groups (lanes c, c+16, c+32, c+48); every lane gets the same result.
// gfx950's lane swaps stay on the VALU (a shuffle would go through the LDS unit and wait for it):
// v_permlane32_swap(v, v) returns (v of lanes 0..31, v of lanes 32..63) in both halves, and
// v_permlane16_swap(v, v) returns the even and the odd 16-lane rows of each half -- so combining the two
// results combines lane l with lane l^32, then with lane l^16, in the same order in every lane.
__device__ __forceinline__ void swap32(float v, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap16(float v, float& even, float& odd) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  even = __uint_as_float(r[0]);
  odd = __uint_as_float(r[1]);
}
__device__ __forceinline__ float group_sum(float v) {
  float a, b;
  swap32(v, a, b);
  swap16(a + b, a, b);
  return a + b;
}
__device__ __forceinline__ float group_max(float v) {
  float a, b;
  swap32(v, a, b);
  swap16(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}

// Workgroup ids are dispatched round-robin over the 8 XCDs; remap so that consecutive logical ids
// land on the same XCD (and share its L2).  A bijection on [0, G).
__device__ __forceinline__ int xcd_remap(int b, int G) {
  const int full = (G / 8) * 8;
  if (b >= full) return b;
  return (b % 8) * (G / 8) + b / 8;
}

// 16-byte global loads / stores.
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // for the non-temporal builtins
// Non-temporal 16-byte store, for the attention outputs (O, dQ, dK, dV), which nothing in the same pass reads
// back soon: written through, they leave the caches to the K, V, Q and dO rows the kernels still gather.
__device__ __forceinline__ void st16_nt(void* p, uint4 v) {
  const u32x4 x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(p));
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

}  // namespace llsa
