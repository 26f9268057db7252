// Layout kernels: tile-major gather / scatter of token rows (the public
// sta_tile_gather / sta_tile_scatter), and the V^T fragment pack the fused
// attention kernel streams. The attention kernel applies the same tile map
// itself when it reads q and k and writes out / lse.
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

// Pack v for the PV product of the attention kernel, tile-major. Block b (64
// tile-major rows) becomes 2 x (D/16) fragments of 1 KB; in fragment
// (h, dt) lane l (group gq = l/16, column i = l%16) holds, for e = 0..7,
// V[64b + 32h + 16(e/4) + 4gq + e%4][16dt + i]. That is the A operand of a
// 16x16x32 MFMA computing O^T += V^T P^T, with the keys in the order in which
// an S^T = K Q^T accumulator leaves them in the lanes (lane l holds keys
// 4(l/16) .. +3 of each 16-key group), so P^T is used where it is produced.
// Rows at or after valid_end (for V: the valid text length) are written as
// zeros, so padded text slots (whatever they hold) contribute exactly nothing.
// The backward packs K, Q and dout the same way.
template <int D>
__global__ __launch_bounds__(kThreads) void pack_v_kernel(Geom g, const uint4* __restrict__ v,
                                                          uint4* __restrict__ vt, int valid_end) {
  constexpr int CPR = D / 8;     // 16-byte chunks per row
  constexpr int DT = D / 16;     // column groups
  constexpr int PITCH = D + 2;   // LDS row pitch in bf16 (odd word count: no bank aliasing)
  __shared__ uint16_t rows[kKeyBlock * PITCH];
  const size_t slab_in = size_t(blockIdx.y) * g.S * CPR;     // raster rows
  const size_t slab_out = size_t(blockIdx.y) * g.S_t * CPR;  // tile-major rows
  const int r0 = blockIdx.x * kKeyBlock;
#pragma unroll
  for (int c = threadIdx.x; c < kKeyBlock * CPR; c += kThreads) {
    const int r = c / CPR, col = c % CPR;
    uint4 x = make_uint4(0, 0, 0, 0);
    const int rr = r0 + r < valid_end ? tiled_to_raster(r0 + r, g) : -1;
    if (rr >= 0) x = v[slab_in + size_t(rr) * CPR + col];
    uint32_t* dst = reinterpret_cast<uint32_t*>(&rows[r * PITCH]) + col * 4;
    dst[0] = x.x;
    dst[1] = x.y;
    dst[2] = x.z;
    dst[3] = x.w;
  }
  __syncthreads();
  uint4* out = vt + slab_out + size_t(r0) * CPR;
#pragma unroll
  for (int o = threadIdx.x; o < kKeyBlock * CPR; o += kThreads) {
    const int frag = o >> 6, l = o & 63;
    const int h = frag / DT, dt = frag % DT;
    const int col = 16 * dt + (l & 15);
    const int key = 32 * h + 4 * (l >> 4);
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int r = key + 16 * (e >> 2) + (e & 3);
      w[e >> 1] = uint32_t(rows[r * PITCH + col]) | (uint32_t(rows[(r + 1) * PITCH + col]) << 16);
    }
    out[o] = make_uint4(w[0], w[1], w[2], w[3]);
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

hipError_t launch_pack_rows(const Geom& g, const void* src, void* dst, int valid_end,
                            hipStream_t stream) {
  dim3 grid(g.S_t / kKeyBlock, g.B * g.heads);
  if (g.D == 128)
    pack_v_kernel<128><<<grid, kThreads, 0, stream>>>(g, (const uint4*)src, (uint4*)dst, valid_end);
  else
    pack_v_kernel<64><<<grid, kThreads, 0, stream>>>(g, (const uint4*)src, (uint4*)dst, valid_end);
  return hipGetLastError();
}

hipError_t launch_pack_v(const Geom& g, const void* v, void* vt, hipStream_t stream) {
  return launch_pack_rows(g, v, vt, g.n_vt + (g.has_text ? g.text_length : 0), stream);
}

}  // namespace sta
