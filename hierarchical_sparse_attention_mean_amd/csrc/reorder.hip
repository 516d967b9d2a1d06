// reorder.hip -- 2-D-local index reordering of the token rows.
//
// Method [LLSA review (pith.science, arXiv 2512.16615), domain-assumption ledger: after index reordering,
// spatially adjacent pixels are adjacent in the flattened sequence (paper Sec. 5.1, ablation Table 5d);
// Figure 2 caption (truncated)].  The page does not give the order; the one built here takes recursive 4 x 4
// tiles (B = 16), so that every level-l unit is a 4^l x 4^l square patch for l <= L: pixel (y, x) of an H x W
// grid goes to (row-major index of its 4^L x 4^L top tile) * 16^L + sum_{k<L} (4 * digit_k(y) + digit_k(x)) *
// 16^k, digit_k the k-th base-4 digit of the coordinate inside the top tile.
//
// Both directions are gathers, one thread per 16-byte piece of a destination row: to the local order, row j
// takes the row-major row of the pixel at local position j; back, row t takes the local row of pixel t.  Writes
// are contiguous; reads come in runs of four consecutive pixels of a grid row.
#include "common.hpp"
#include "launch.hpp"

namespace llsa {

namespace {

__device__ __forceinline__ int local_of(int y, int x, int W, int L) {
  const int S = 1 << (2 * L);
  const int tile = (y >> (2 * L)) * (W >> (2 * L)) + (x >> (2 * L));
  const int yy = y & (S - 1), xx = x & (S - 1);
  int inner = 0;
  for (int k = 0; k < L; ++k) inner |= ((((yy >> (2 * k)) & 3) << 2) | ((xx >> (2 * k)) & 3)) << (4 * k);
  return (tile << (4 * L)) | inner;
}

__device__ __forceinline__ int rowmajor_of(int j, int W, int L) {
  const int tile = j >> (4 * L), inner = j & ((1 << (4 * L)) - 1);
  const int tiles_x = W >> (2 * L);
  const int ty = tile / tiles_x, tx = tile - ty * tiles_x;
  int yy = 0, xx = 0;
  for (int k = 0; k < L; ++k) {
    const int dgt = (inner >> (4 * k)) & 15;
    yy |= (dgt >> 2) << (2 * k);
    xx |= (dgt & 3) << (2 * k);
  }
  return ((ty << (2 * L)) + yy) * W + (tx << (2 * L)) + xx;
}

// grid: ceil(rows * pieces / 256) x 256 threads; rows = bh * n, pieces = 16-byte pieces per row.
__global__ __launch_bounds__(256) void reorder_rows(const uint4* __restrict__ x, uint4* __restrict__ y, int64_t rows,
                                                    int n, int W, int L, int pieces, int to_local) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = g / pieces;
  if (row >= rows) return;
  const int piece = (int)(g - row * pieces);
  const int64_t slice = row / n;
  const int j = (int)(row - slice * n);
  const int src = to_local ? rowmajor_of(j, W, L) : local_of(j / W, j % W, W, L);
  y[row * pieces + piece] = x[(slice * n + src) * pieces + piece];
}

}  // namespace

hipError_t launch_reorder(const Geom& g, int elem_bytes, int grid_w, int to_local, const void* x, void* y,
                          hipStream_t stream) {
  const int pieces = kD * elem_bytes / 16;
  const int64_t rows = (int64_t)g.bh * g.n;
  const int64_t threads = rows * pieces;
  LaunchTimer timer(kReorder, stream);
  reorder_rows<<<(unsigned)((threads + 255) / 256), 256, 0, stream>>>((const uint4*)x, (uint4*)y, rows, g.n, grid_w,
                                                                      g.L, pieces, to_local);
  return hipGetLastError();
}

}  // namespace llsa
