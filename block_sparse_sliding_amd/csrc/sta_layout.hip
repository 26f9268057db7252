// Layout kernels: tile-major gather / scatter of token rows (the public
// sta_tile_gather / sta_tile_scatter) and the Hilbert-order gather / scatter.
// The attention kernels apply the tile map themselves when they read q, k and
// v and write their outputs.
//
// Tile-major order (each (6,8,8) tile becomes 384 contiguous rows) follows the
// tile definition of the STA README "Usage" section; it turns every dense
// (query tile, key tile) block of the attention map into contiguous slabs.
#include "sta_internal.h"

namespace sta {
namespace {

constexpr int kThreads = 256;

// One workgroup per 64-row block of the tile-major sequence (S_t rows), one
// grid row per (batch, head) slab. Copies whole rows in 16-byte chunks; both
// sides coalesce (a 64-row tile-major block of a full tile is the 8x8 (h, w)
// patch of one frame: 8 raster runs of 8 rows). Padding rows of partial tiles
// are written as zeros by the gather and not read by the scatter.
template <int D>
__global__ __launch_bounds__(kThreads) void rows_permute_kernel(Geom g, const uint4* __restrict__ src,
                                                                uint4* __restrict__ dst, int to_tiled) {
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  const size_t slab_r = size_t(blockIdx.y) * g.S * CPR;    // raster rows
  const size_t slab_t = size_t(blockIdx.y) * g.S_t * CPR;  // tile-major rows
  const int r0 = blockIdx.x * kKeyBlock;
#pragma unroll
  for (int c = threadIdx.x; c < kKeyBlock * CPR; c += kThreads) {
    const int rt = r0 + c / CPR;
    const int col = c % CPR;
    const int rr = tiled_to_raster(rt, g);  // -1: padding
    if (to_tiled)
      dst[slab_t + size_t(rt) * CPR + col] = rr >= 0 ? src[slab_r + size_t(rr) * CPR + col] : make_uint4(0, 0, 0, 0);
    else if (rr >= 0)
      dst[slab_r + size_t(rr) * CPR + col] = src[slab_t + size_t(rt) * CPR + col];
  }
}

// Raster <-> Hilbert order of a 2D image's rows (one frame, side 8 * 2^hil_m):
// Hilbert row d holds the token at position d of the order hil_m + 3 curve
// ("Boosting 2D Local Attention Efficiency with Hilbert-Guided Sparsity",
// "The Hilbert Curve Advantage"); text rows keep their place. grid (S / 64,
// B * heads): one workgroup per 64 Hilbert rows (one 8x8 tile).
template <int D>
__global__ __launch_bounds__(kThreads) void rows_hilbert_kernel(Geom g, const uint4* __restrict__ src,
                                                                uint4* __restrict__ dst, int to_hilbert) {
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  const size_t slab = size_t(blockIdx.y) * g.S * CPR;
  const int r0 = blockIdx.x * kKeyBlock;
  const int k = g.hil_m + 3;
  for (int c = threadIdx.x; c < kKeyBlock * CPR; c += kThreads) {
    const int rh = r0 + c / CPR;
    const int col = c % CPR;
    int rr = rh;  // text rows
    if (rh < g.n_video) {
      int x, y;
      hilbert_d2xy(k, rh, x, y);
      rr = y * g.W + x;
    }
    if (to_hilbert)
      dst[slab + size_t(rh) * CPR + col] = src[slab + size_t(rr) * CPR + col];
    else
      dst[slab + size_t(rr) * CPR + col] = src[slab + size_t(rh) * CPR + col];
  }
}

}  // namespace

hipError_t launch_rows_permute(const Geom& g, const void* src, void* dst, bool to_tiled,
                               hipStream_t stream) {
  dim3 grid(g.S_t / kKeyBlock, g.B * g.heads);
  if (g.D == 128)
    rows_permute_kernel<128><<<grid, kThreads, 0, stream>>>(g, (const uint4*)src, (uint4*)dst, to_tiled);
  else
    rows_permute_kernel<64><<<grid, kThreads, 0, stream>>>(g, (const uint4*)src, (uint4*)dst, to_tiled);
  return hipGetLastError();
}

hipError_t launch_rows_hilbert(const Geom& g, const void* src, void* dst, bool to_hilbert,
                               hipStream_t stream) {
  dim3 grid(g.S / kKeyBlock, g.B * g.heads);
  if (g.D == 128)
    rows_hilbert_kernel<128><<<grid, kThreads, 0, stream>>>(g, (const uint4*)src, (uint4*)dst, to_hilbert);
  else
    rows_hilbert_kernel<64><<<grid, kThreads, 0, stream>>>(g, (const uint4*)src, (uint4*)dst, to_hilbert);
  return hipGetLastError();
}

}  // namespace sta
