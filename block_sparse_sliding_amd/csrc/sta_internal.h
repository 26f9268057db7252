// Internal declarations shared by the STA host library and its HIP kernels.
// Not part of the public ABI (include/sta.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sta {

// Tile cube (6, 8, 8) tokens = 384 rows, from the STA README "Usage" section.
constexpr int kTileT = 6;
constexpr int kTileH = 8;
constexpr int kTileW = 8;
constexpr int kTileRows = kTileT * kTileH * kTileW;  // 384
constexpr int kTextSlots = 256;
// Key rows per packed block / per LDS stage of the attention kernel.
constexpr int kKeyBlock = 64;
// Query rows per attention workgroup: one whole tile.
constexpr int kUnitRows = kTileRows;
constexpr int kMaxHeads = 256;
constexpr int kWinBits = 10;  // each packed window component uses 10 bits

// Derived geometry, computed on the host and passed by value to kernels.
struct Geom {
  int32_t B, heads, D;
  int32_t T, H, W;
  int32_t nt, nh, nw;  // tile-grid size: ceil(T/6), ceil(H/8), ceil(W/8)
  int32_t n_tiles;     // nt * nh * nw
  int32_t n_video;     // T * H * W (raster video rows)
  int32_t S;           // n_video + (has_text ? 256 : 0): rows of the caller's tensors
  int32_t n_vt;        // n_tiles * 384: tile-major video rows, padding rows of partial tiles included
  int32_t S_t;         // n_vt + (has_text ? 256 : 0): rows of the tile-major (packed) tensors
  int32_t full;        // 1 when T, H, W are multiples of the tile (no padding rows)
  int32_t has_text;
  int32_t text_length;
  int32_t n_q;         // query units per head: n_tiles (+1 text unit)
  // ceil(2^32 / nw) and ceil(2^32 / nh) (0 when the divisor is 1):
  // floor(n / d) = umulhi(n, m) exactly whenever n * d < 2^32, which holds for
  // every tile index (n_tiles * max(nw, nh) < 2^32 is checked on the host).
  uint32_t mag_nw, mag_nh;
};

// Per-head windows, packed as wt | wh << 10 | ww << 20 (kernel-argument copy).
struct Windows {
  uint32_t w[kMaxHeads];
};

// Start of a window of w tiles along an axis of n tiles for query tile c:
// centred on c and shifted inward at the grid border, so it always holds w
// tiles (the STA README "Usage" example gives every query of the (30,48,80)
// video the same (18,24,24) token box).
__host__ __device__ inline int window_start(int c, int w, int n) {
  int s = c - w / 2;
  s = s < 0 ? 0 : s;
  return s > n - w ? n - w : s;
}
__host__ __device__ inline int win_t(uint32_t p) { return int(p & 1023u); }
__host__ __device__ inline int win_h(uint32_t p) { return int((p >> 10) & 1023u); }
__host__ __device__ inline int win_w(uint32_t p) { return int((p >> 20) & 1023u); }

// Extent of tile (tt, th, tw) inside the video, packed in one int: the frames
// (of 6) | rows (of 8) << 8 | columns (of 8) << 16 of the tile that exist.
constexpr int kFullExtent = kTileT | (kTileH << 8) | (kTileW << 16);
__host__ __device__ inline int tile_extent(int tt, int th, int tw, const Geom& g) {
  int frames = g.T - tt * kTileT, rows = g.H - th * kTileH, cols = g.W - tw * kTileW;
  frames = frames < kTileT ? frames : kTileT;
  rows = rows < kTileH ? rows : kTileH;
  cols = cols < kTileW ? cols : kTileW;
  return frames | (rows << 8) | (cols << 16);
}
__host__ __device__ inline int extent_frames(int e) { return e & 255; }
__host__ __device__ inline int extent_rows(int e) { return (e >> 8) & 255; }
__host__ __device__ inline int extent_cols(int e) { return e >> 16; }
__host__ __device__ inline int extent_tokens(int e) {
  return extent_frames(e) * extent_rows(e) * extent_cols(e);
}
// Compact order of a tile's existing tokens: frame, then row, then column.
// Token r (< extent_tokens(e)) of tile (tt, th, tw) -> its offsets in the tile.
__host__ __device__ inline void compact_token(int r, int e, int& dt, int& dh, int& dw) {
  const int cols = extent_cols(e), plane = extent_rows(e) * cols;
  dt = r / plane;
  const int rem = r - dt * plane;
  dh = rem / cols;
  dw = rem - dh * cols;
}

// Blocks of 64 tokens over a box of tiles [lo, lo + len) per axis, each tile
// counting ceil(tokens / 64). Along an axis every tile but the grid's last is
// full, so the sum has at most eight distinct terms.
__host__ __device__ inline int box_blocks(int lo_t, int len_t, int lo_h, int len_h, int lo_w, int len_w,
                                          const Geom& g) {
  int n_full[3], n_part[3], ext[3];
  const int lo[3] = {lo_t, lo_h, lo_w}, len[3] = {len_t, len_h, len_w};
  const int n[3] = {g.nt, g.nh, g.nw}, size[3] = {g.T, g.H, g.W}, tile[3] = {kTileT, kTileH, kTileW};
  for (int a = 0; a < 3; ++a) {
    ext[a] = size[a] - (n[a] - 1) * tile[a];  // extent of the grid's last tile
    n_part[a] = (lo[a] + len[a] == n[a] && ext[a] < tile[a]) ? 1 : 0;
    n_full[a] = len[a] - n_part[a];
  }
  int sum = 0;
  for (int m = 0; m < 8; ++m) {
    const int ct = (m & 1) ? n_part[0] : n_full[0], ch = (m & 2) ? n_part[1] : n_full[1];
    const int cw = (m & 4) ? n_part[2] : n_full[2];
    const int tok = ((m & 1) ? ext[0] : kTileT) * ((m & 2) ? ext[1] : kTileH) * ((m & 4) ? ext[2] : kTileW);
    sum += ct * ch * cw * ((tok + kKeyBlock - 1) / kKeyBlock);
  }
  return sum;
}

// Tile-major row r (within one [S_t] slab) -> raster row, or -1 for a padding
// row. Tile t owns rows 384t .. 384t + 383; a video size that is not a
// multiple of the tile is covered by the same tile grid, the last tile along
// an axis holding the remainder, and a partial tile's slot holds its existing
// tokens first, in compact order (frame, row, column), then padding rows. For
// a full tile the compact order is (frame, row, column) of 6 x 8 x 8. Text
// rows follow the video in both orders.
// The same for a video size that is a tile multiple (g.full): bit operations
// only inside the tile.
__host__ __device__ inline int tiled_to_raster_full(int r, const Geom& g) {
  if (r >= g.n_vt) return r - g.n_vt + g.n_video;
  const int tile = r / kTileRows;
  const int j = r - tile * kTileRows;
  const int tw = tile % g.nw;
  const int rest = tile / g.nw;
  const int th = rest % g.nh;
  const int tt = rest / g.nh;
  return ((tt * kTileT + (j >> 6)) * g.H + th * kTileH + ((j >> 3) & 7)) * g.W + tw * kTileW + (j & 7);
}
__host__ __device__ inline int tiled_to_raster(int r, const Geom& g) {
  if (r >= g.n_vt) return r - g.n_vt + g.n_video;
  const int tile = r / kTileRows;
  const int j = r - tile * kTileRows;
  const int tw = tile % g.nw;
  const int rest = tile / g.nw;
  const int th = rest % g.nh;
  const int tt = rest / g.nh;
  int dt = j >> 6, dh = (j >> 3) & 7, dw = j & 7;
  if (!g.full) {
    const int e = tile_extent(tt, th, tw, g);
    if (j >= extent_tokens(e)) return -1;
    compact_token(j, e, dt, dh, dw);
  }
  return ((tt * kTileT + dt) * g.H + th * kTileH + dh) * g.W + tw * kTileW + dw;
}

// Launchers (each enqueues one kernel on `stream` and returns hipGetLastError()).
hipError_t launch_rows_permute(const Geom& g, const void* src, void* dst, bool to_tiled,
                               hipStream_t stream);
// V^T fragments: every 64-row tile-major block of v (rows at or after the
// valid text length zeroed) as (2 key halves) x (D/16 column groups) 1 KB
// fragments, the A operand of O^T += V^T P^T (layout documented at the pack
// kernel).
hipError_t launch_pack_v(const Geom& g, const void* v, void* vt, hipStream_t stream);
// The same fragment packing for any [B][heads][S][D] bf16 raster tensor, into
// [B][heads][S_t][D] tile-major fragments; tile-major rows at or after
// valid_end, and padding rows of partial tiles, are written as zeros.
hipError_t launch_pack_rows(const Geom& g, const void* src, void* dst, int valid_end,
                            hipStream_t stream);
hipError_t launch_schedule_lists(const Geom& g, const Windows& win, int32_t* offsets,
                                 int32_t* ids, hipStream_t stream);
// Work order (one query unit per entry, grouped into 8 per-XCD queues: queue x
// holds entries 8k + x). `claim`, when not null, receives kClaimInts zeros:
// the queue heads the attention kernel advances.
hipError_t launch_schedule_work(const Geom& g, const Windows& win, int32_t* work,
                                int32_t* claim, hipStream_t stream);
constexpr int kQueues = 8;        // one per XCD
constexpr int kClaimStride = 64;  // ints between queue heads (own 256-byte line each)
constexpr int kClaimInts = kQueues * kClaimStride;

struct FwdArgs {
  const void* q;         // bf16 raster rows (the caller's q)
  const void* k;         // bf16 raster rows (the caller's k)
  const void* vt;        // packed V^T fragments (launch_pack_v)
  void* out;             // bf16 raster rows (the caller's out)
  float* lse;            // fp32 raster (the caller's lse), or nullptr
  const int32_t* offsets;
  const int32_t* ids;
  const int32_t* work;   // per-XCD queues of query units (launch_schedule_work)
  int32_t* claim;        // queue heads, zeroed by launch_schedule_work
  float q_scale;         // log2(e) / sqrt(D), applied to the fp32 scores
};
hipError_t launch_attention(const Geom& g, const Windows& win, const FwdArgs& a, hipStream_t stream);

// Backward (gradients of the forward for an upstream gradient dout).
struct BwdArgs {
  const void* q;         // bf16 raster rows (the caller's q, k, v, dout)
  const void* k;
  const void* v;
  const void* dout;
  const void* kt;        // packed K^T fragments, text rows past the valid length zero
  const void* qt;        // packed Q^T fragments
  const void* dot;       // packed dout^T fragments
  const float* lse2;     // tile-major lse * log2(e)
  const float* delta;    // tile-major -rowsum(dout * out), negated: it starts the dP accumulators
  void* dq;              // bf16 raster rows (the caller's dq, dk, dv)
  void* dk;
  void* dv;
  const int32_t* offsets;  // forward schedule lists (launch_schedule_lists)
  const int32_t* ids;
  int32_t* claim_q;      // queue heads of the dq and dk/dv launches, zeroed by
  int32_t* claim_kv;     // launch_bwd_prep
  float q_scale;         // log2(e) / sqrt(D)
  float scale;           // 1 / sqrt(D)
};
hipError_t launch_bwd_prep(const Geom& g, const void* out, const void* dout, const float* lse,
                           float* lse2, float* delta, int32_t* claim_q, int32_t* claim_kv,
                           hipStream_t stream);
hipError_t launch_bwd_dq(const Geom& g, const Windows& win, const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dkv(const Geom& g, const Windows& win, const BwdArgs& a, hipStream_t stream);

}  // namespace sta
