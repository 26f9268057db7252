// Layout kernels: tile-major gather / scatter of token rows, and the packing of
// k and v into the forms the fused attention kernel streams (the attention
// kernel reads q and writes out / lse in raster order itself).
//
// Tile-major order (each (6,8,8) tile becomes 384 contiguous rows) follows the
// tile definition of the STA README "Usage" section; it turns every dense
// (query tile, key tile) block of the attention map into contiguous slabs.
#include "sta_internal.h"

namespace sta {
namespace {

constexpr int kThreads = 256;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

// One workgroup per 64-row block of the tile-major sequence, one grid row per
// (batch, head) slab. Copies whole rows in 16-byte chunks; both sides coalesce
// (a 64-row tile-major block is the 8x8 (h, w) patch of one frame: 8 raster
// runs of 8 rows).
template <int D>
__global__ __launch_bounds__(kThreads) void rows_permute_kernel(Geom g, const uint4* __restrict__ src,
                                                                uint4* __restrict__ dst, int to_tiled) {
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  const size_t slab = size_t(blockIdx.y) * g.S * CPR;
  const int r0 = blockIdx.x * kKeyBlock;
#pragma unroll
  for (int c = threadIdx.x; c < kKeyBlock * CPR; c += kThreads) {
    const int rt = r0 + c / CPR;
    const int col = c % CPR;
    const int rr = tiled_to_raster(rt, g);
    if (to_tiled)
      dst[slab + size_t(rt) * CPR + col] = src[slab + size_t(rr) * CPR + col];
    else
      dst[slab + size_t(rr) * CPR + col] = src[slab + size_t(rt) * CPR + col];
  }
}

// Pack k and v for the attention kernel (grid.z: 0 = k, 1 = v), tile-major.
//
// k: scaled by k_scale = log2(e)/sqrt(D) and rounded to bf16 (so the MFMA
//    yields scores in the log2 domain; rounding the scaled keys rather than
//    the queries keeps the rounding error independent from key to key), then
//    each 64-key block is stored as (4 key groups) x (D/32 k-steps) fragments
//    of 1 KB; in fragment (kt, ks) lane l's 16 bytes are
//    K[16*kt + l%16][32*ks + 8*(l/16) .. +8], the A operand of a 16x16x32
//    MFMA that computes S^T = K Q^T.
// v: each 64-key block is stored as (2 k-steps) x (D/16 d-groups) fragments;
//    in fragment (ks, dt) lane l (g = l/16, i = l%16) holds, for j = 0..7,
//    V[32*ks + 16*(j/4) + 4*g + j%4][16*dt + i]: the A operand of the MFMA
//    that computes O^T = V^T P^T, with keys ordered to match how S^T leaves
//    the accumulator registers (so P^T needs no cross-lane movement).
// Text rows at or after text_length are written as zeros in k and v, so that
// nothing stored there (even non-finite values) can reach the output.
template <int D>
__global__ __launch_bounds__(kThreads) void pack_kv_kernel(Geom g, const uint4* __restrict__ k,
                                                           const uint4* __restrict__ v,
                                                           uint4* __restrict__ kp,
                                                           uint4* __restrict__ vp, float k_scale) {
  constexpr int CPR = D / 8;
  constexpr int ROWH = D + 4;  // padded LDS row (in bf16) for the V transpose
  __shared__ uint16_t tile[kKeyBlock * ROWH];
  const size_t slab = size_t(blockIdx.y) * g.S * CPR;
  const int r0 = blockIdx.x * kKeyBlock;
  const int which = blockIdx.z;
  const int valid_end = g.n_video + (g.has_text ? g.text_length : 0);

  if (which == 0) {
    uint4* dst = kp + slab + size_t(r0) * CPR;
#pragma unroll
    for (int c = threadIdx.x; c < kKeyBlock * CPR; c += kThreads) {
      const int j = c / CPR, col = c % CPR;
      const int rt = r0 + j;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (rt < valid_end) {
        x = k[slab + size_t(tiled_to_raster(rt, g)) * CPR + col];
        bf16x8 kv = __builtin_bit_cast(bf16x8, x);
        f32x8 f = __builtin_convertvector(kv, f32x8) * k_scale;
        x = __builtin_bit_cast(uint4, __builtin_convertvector(f, bf16x8));
      }
      const int kt = j >> 4, ks = col >> 2, grp = col & 3;
      dst[(kt * (D / 32) + ks) * 64 + (j & 15) + 16 * grp] = x;
    }
    return;
  }
  // v: stage the 64 x D block in LDS, then emit transposed fragments.
#pragma unroll
  for (int c = threadIdx.x; c < kKeyBlock * CPR; c += kThreads) {
    const int j = c / CPR, col = c % CPR;
    const int rt = r0 + j;
    uint4 x = make_uint4(0, 0, 0, 0);
    if (rt < valid_end) x = v[slab + size_t(tiled_to_raster(rt, g)) * CPR + col];
    uint32_t* row = reinterpret_cast<uint32_t*>(&tile[j * ROWH + col * 8]);
    row[0] = x.x;
    row[1] = x.y;
    row[2] = x.z;
    row[3] = x.w;
  }
  __syncthreads();
  uint4* dst = vp + slab + size_t(r0) * CPR;
#pragma unroll
  for (int o = threadIdx.x; o < kKeyBlock * CPR; o += kThreads) {
    const int frag = o >> 6, l = o & 63;
    const int ks = frag / (D / 16), dt = frag % (D / 16);
    const int grp = l >> 4, i = l & 15;
    const int col = 16 * dt + i;
    uint32_t w[4];
#pragma unroll
    for (int jj = 0; jj < 8; jj += 2) {
      const int key0 = 32 * ks + 16 * (jj >> 2) + 4 * grp + (jj & 3);
      const uint32_t lo = tile[key0 * ROWH + col];
      const uint32_t hi = tile[(key0 + 1) * ROWH + col];
      w[jj >> 1] = lo | (hi << 16);
    }
    dst[o] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

}  // namespace

hipError_t launch_rows_permute(const Geom& g, const void* src, void* dst, bool to_tiled,
                               hipStream_t stream) {
  dim3 grid(g.S / kKeyBlock, g.B * g.heads);
  if (g.D == 128)
    rows_permute_kernel<128><<<grid, kThreads, 0, stream>>>(g, (const uint4*)src, (uint4*)dst, to_tiled);
  else
    rows_permute_kernel<64><<<grid, kThreads, 0, stream>>>(g, (const uint4*)src, (uint4*)dst, to_tiled);
  return hipGetLastError();
}

hipError_t launch_pack_kv(const Geom& g, const void* k, const void* v, void* k_packed,
                          void* v_packed, float k_scale, hipStream_t stream) {
  dim3 grid(g.S / kKeyBlock, g.B * g.heads, 2);
  if (g.D == 128)
    pack_kv_kernel<128><<<grid, kThreads, 0, stream>>>(g, (const uint4*)k, (const uint4*)v,
                                                       (uint4*)k_packed, (uint4*)v_packed, k_scale);
  else
    pack_kv_kernel<64><<<grid, kThreads, 0, stream>>>(g, (const uint4*)k, (const uint4*)v,
                                                      (uint4*)k_packed, (uint4*)v_packed, k_scale);
  return hipGetLastError();
}

}  // namespace sta
