// persist.hpp -- device helpers of the persistent gfx950 kernels: asynchronous global -> LDS copies,
// the XCD-contiguous work mapping, swizzled LDS row tiles and the coalesced stage gather.
#pragma once
#include "common.hpp"
#include "entries.hpp"

namespace llsa {

// Asynchronous global -> LDS copies that hold no registers: lane l's 16 (4) bytes land at dst + 16 l (4 l).
// They are written as inline assembly so that the compiler does not see them: it models an LDS DMA as a
// flat access of unknown order and would then drain all outstanding loads (vmcnt(0)) at every later wait.
// The hardware counts them on vmcnt in issue order with the other vector loads, so a kernel waits for
// them itself at the point where their data is first read; the compiler's own waits, which do not count
// them, only get stricter by their presence.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void lds_dma16(const void* src, const void* dst) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds_addr(dst)) : "memory");
}
// The same copy with the non-temporal hint, for rows a kernel reads once (a block's Q, dO, O rows): they then
// leave the caches to the gathered K and V rows.
__device__ __forceinline__ void lds_dma16_nt(const void* src, const void* dst) {
  asm volatile("global_load_lds_dwordx4 %0, off nt" ::"v"(src), "{m0}"(lds_addr(dst)) : "memory");
}
__device__ __forceinline__ void lds_dma4(const void* src, const void* dst) {
  asm volatile("global_load_lds_dword %0, off" ::"v"(src), "{m0}"(lds_addr(dst)) : "memory");
}
// Waits (LDS traffic only) and a workgroup barrier that does not drain outstanding global loads.
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Items of one worker.  Workgroup b runs on XCD b % 8 (round-robin dispatch); XCD x owns the contiguous
// item range [x*n/8, (x+1)*n/8), and its `per_xcd` workers sweep that range together: worker r takes items
// lo + r, lo + r + per_xcd, ...  At any moment one XCD thus works on a window of consecutive items, whose
// selections overlap, so their key blocks stay in that XCD's L2.
struct Sweep {
  int first, stride, count;
};
// Wave-uniform value in a scalar register.  Integer divisions are expanded on the vector unit, and the
// compiler then treats their results -- and every loop bound or index derived from them -- as divergent:
// loops turn into exec-masked loops and per-stage address arithmetic runs on the VALU.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ Sweep xcd_sweep(int n, int r, int per_xcd) {
  const int x = blockIdx.x % 8;
  const int lo = (int)(((int64_t)x * n) / 8), hi = (int)(((int64_t)(x + 1) * n) / 8);
  Sweep sw;
  sw.first = uniform(lo + r);
  sw.stride = uniform(per_xcd);
  sw.count = uniform(r < hi - lo ? (hi - lo - r + per_xcd - 1) / per_xcd : 0);
  return sw;
}

// Unpadded bf16 tile of 64-element rows with an XOR swizzle of the 16-byte chunks: element (row, col) sits at
// row*64 + 8*((col/8) ^ (row%8)) + col%8.  Row-wise writes stay contiguous per chunk, and column-wise reads
// (MFMA operands, transposed reads) spread over the banks.
__device__ __forceinline__ int swz(int row, int col) { return row * kD + ((((col >> 3) ^ row) & 7) << 3) + (col & 7); }

// Source offset (elements, within 8 consecutive rows) of lane l for an LDS DMA that fills a swizzled tile:
// lane l's 16 bytes land in chunk l%8 of row l/8, which holds logical chunk (l%8) ^ (l/8).
__device__ __forceinline__ int swz_dma_src(int lane) { return (lane >> 3) * kD + (((lane & 7) ^ (lane >> 3)) << 3); }

// Loads of stage s of a block's plan, coalesced: a quarter-wave (16 lanes) reads whole 128-byte lines (two
// bf16 rows), and the consumer puts rows into MFMA operand order through LDS tiles.  Instruction m reads
// rows 8m .. 8m+7 of the stage's 32 keys (lane l: row 8m + l/8, bytes 16 (l%8)) -- K into r[m], V into
// r[4+m]:
//   fine:   rows 0..15 are key block b0 = sel[2s], rows 16..31 block b1 = sel[2s+1] (raw K, V);
//   coarse: row j is enrichment entry 32(s - nfine) + j (clamped to the list) of the bf16 pooled pyramid.
// The branch only forms two uniform base pointers and four per-lane byte offsets; the eight loads then
// follow on one straight path, so every stage leaves the same loads in flight in the same registers and
// the compiler's waits stay exact.
// sel: the block's level-1 selection row; esel: its enrichment entries' selection values; row0: the first
// pyramid row of each entry's level (EntryTab::row0) -- all in LDS.
__device__ __forceinline__ void issue_stage_coalesced(const Plan& plan, int s, int K, const int* sel,
                                                      const int* esel, const int* row0, const bf16_t* kslice,
                                                      const bf16_t* vslice, const bf16_t* pkslice,
                                                      const bf16_t* pvslice, int lane, Stage& st) {
  const char* kb;
  const char* vb;
  uint32_t off[4];
  const uint32_t sub = (uint32_t)lane >> 3, col = 16u * (lane & 7);
  if (s < plan.nfine) {
    const int b0 = __builtin_amdgcn_readfirstlane(sel[2 * s]);
    const int b1 = __builtin_amdgcn_readfirstlane(sel[min(2 * s + 1, K - 1)]);
    kb = reinterpret_cast<const char*>(kslice);
    vb = reinterpret_cast<const char*>(vslice);
#pragma unroll
    for (int m = 0; m < 4; ++m) off[m] = (16u * (m < 2 ? b0 : b1) + 8u * (m & 1) + sub) * (2 * kD) + col;
  } else {
    const int e0 = 32 * (s - plan.nfine) + (int)sub;
    kb = reinterpret_cast<const char*>(pkslice);
    vb = reinterpret_cast<const char*>(pvslice);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int e = min(e0 + 8 * m, plan.ncoarse - 1);
      off[m] = (uint32_t)(esel[e] + row0[e]) * (2 * kD) + col;
    }
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) st.r[m] = ld16(kb + off[m]);
#pragma unroll
  for (int m = 0; m < 4; ++m) st.r[4 + m] = ld16(vb + off[m]);
}

}  // namespace llsa
