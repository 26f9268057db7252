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
// Rows per streamed block / per LDS stage of the attention kernels.
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
  int32_t S_t;         // n_vt + (has_text ? 256 : 0): rows of tile-major tensors
  int32_t full;        // 1 when T, H, W are multiples of the tile (no padding rows)
  int32_t has_text;
  int32_t text_length;
  int32_t n_q;         // query units per head: n_tiles (+1 text unit)
  // ceil(2^32 / nw) and ceil(2^32 / nh) (0 when the divisor is 1):
  // floor(n / d) = umulhi(n, m) exactly whenever n * d < 2^32, which holds for
  // every tile index (n_tiles * max(nw, nh) < 2^32 is checked on the host).
  uint32_t mag_nw, mag_nh;
  // Hilbert-window attention (2D images, T = 1, a 2^hil_m x 2^hil_m tile grid):
  // 0 = the STA box windows; 1 = Hilbert slide windows; 2 = Hilbert windows;
  // kSquareUnits = the STA box windows on a one-frame video (tiles of at
  // most 8x8 tokens), with query units of 2x2 squares of tiles (SquareKeyStream)
  int32_t hilbert, hil_m;
  // tiles per grouped query unit: Hilbert 1, 4 (an aligned 2x2 square of
  // tiles) or 6 consecutive curve positions, ceil(n_tiles / hil_group) video
  // units, the last of which may hold fewer tiles; squares 4, ceil(nh / 2) x
  // ceil(nw / 2) video units, those on an odd last tile row or column holding
  // 2 or 1 tiles. n_q counts the video units plus text_parts text units
  int32_t hil_group;
  // query units that share the text query rows (grouped units: each takes a
  // contiguous run of the key tiles, the last one also the text keys, and
  // their partial results are merged after the attention kernel); 1 otherwise
  int32_t text_parts;
};

constexpr int32_t kSquareUnits = 3;  // Geom::hilbert of STA with 2x2-square query units

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

// Blocks of 64 tokens over a box of tiles [lo, lo + len) per axis: each tile
// has floor(tokens / 64) full blocks (`full`) and, when 64 does not divide its
// tokens, one remainder block (`rem`). Along an axis every tile but the grid's
// last is full, so the sums have at most eight distinct terms.
__host__ __device__ inline void box_block_counts(int lo_t, int len_t, int lo_h, int len_h, int lo_w, int len_w,
                                                 const Geom& g, int& full, int& rem) {
  int n_full[3], n_part[3], ext[3];
  const int lo[3] = {lo_t, lo_h, lo_w}, len[3] = {len_t, len_h, len_w};
  const int n[3] = {g.nt, g.nh, g.nw}, size[3] = {g.T, g.H, g.W}, tile[3] = {kTileT, kTileH, kTileW};
  for (int a = 0; a < 3; ++a) {
    ext[a] = size[a] - (n[a] - 1) * tile[a];  // extent of the grid's last tile
    n_part[a] = (lo[a] + len[a] == n[a] && ext[a] < tile[a]) ? 1 : 0;
    n_full[a] = len[a] - n_part[a];
  }
  full = 0;
  rem = 0;
  for (int m = 0; m < 8; ++m) {
    const int ct = (m & 1) ? n_part[0] : n_full[0], ch = (m & 2) ? n_part[1] : n_full[1];
    const int cw = (m & 4) ? n_part[2] : n_full[2];
    const int tok = ((m & 1) ? ext[0] : kTileT) * ((m & 2) ? ext[1] : kTileH) * ((m & 4) ? ext[2] : kTileW);
    full += ct * ch * cw * (tok / kKeyBlock);
    rem += ct * ch * cw * ((tok % kKeyBlock) != 0 ? 1 : 0);
  }
}
// All blocks of the box: each tile counting ceil(tokens / 64).
__host__ __device__ inline int box_blocks(int lo_t, int len_t, int lo_h, int len_h, int lo_w, int len_w,
                                          const Geom& g) {
  int full, rem;
  box_block_counts(lo_t, len_t, lo_h, len_h, lo_w, len_w, g, full, rem);
  return full + rem;
}

// Hilbert curve of order k on the 2^k x 2^k grid (x = column, y = row), from
// (0, 0) to (2^k - 1, 0): order k visits the quadrants (x low, y low),
// (x low, y high), (x high, y high), (x high, y low), running the order k - 1
// curve transposed, shifted, shifted, and reflected through the anti-diagonal
// ("Boosting 2D Local Attention Efficiency with Hilbert-Guided Sparsity",
// "The Hilbert Curve Advantage": tokens reordered along a Hilbert curve).
// Position d -> cell: the level transforms applied from the innermost digit
// of d (base 4) outwards.
__host__ __device__ inline void hilbert_d2xy(int k, int d, int& x, int& y) {
  x = 0;
  y = 0;
  for (int j = 1; j <= k; ++j) {
    const int h = 1 << (j - 1);
    const int q = (d >> (2 * (j - 1))) & 3;
    if (q == 0) {
      const int t = x;
      x = y;
      y = t;
    } else if (q == 1) {
      y += h;
    } else if (q == 2) {
      x += h;
      y += h;
    } else {
      const int nx = 2 * h - 1 - y, ny = h - 1 - x;
      x = nx;
      y = ny;
    }
  }
}
// Cell -> position: the quadrants peeled from the outermost level inwards.
__host__ __device__ inline int hilbert_xy2d(int k, int x, int y) {
  int d = 0;
  for (int j = k; j >= 1; --j) {
    const int h = 1 << (j - 1);
    int q;
    if (x < h && y < h) {
      q = 0;
      const int t = x;
      x = y;
      y = t;
    } else if (x < h) {
      q = 1;
      y -= h;
    } else if (y >= h) {
      q = 2;
      x -= h;
      y -= h;
    } else {
      q = 3;
      const int nx = h - 1 - y, ny = 2 * h - 1 - x;
      x = nx;
      y = ny;
    }
    d += q * h * h;
  }
  return d;
}
// Key tiles of the query tile at curve position i: positions [first, first + count).
// mode 1 (slide): the STA window rule in one dimension, W tiles centred on i and
// shifted inward at the ends; mode 2 (window): the block of W positions holding i.
__host__ __device__ inline void hilbert_window(int i, int W, int n, int mode, int& first, int& count) {
  if (mode == 1) {
    first = window_start(i, W, n);
    count = W;
  } else {
    first = (i / W) * W;
    count = n - first < W ? n - first : W;
  }
}

// One 64-key block of a query unit's key stream (scalar values).
struct KeyBlock {
  // 0: a full frame of a key tile, block row r at raster base + (r / 8) W + r % 8;
  // 1: consecutive raster rows base + r, valid while r < lim (text);
  // 2: compact token 64 sub + r of the partial key tile with raster origin
  //    base and extent ext, valid while the token exists.
  int kind;
  int base, lim, ext, sub;
  int mask;  // first block row that must not contribute (64: none)
  // the tiles of a grouped query unit (64 rows each, tile i = unit rows
  // 64 i .. 64 i + 63) that see this block: bit i; -1 (every bit) when all of
  // them do, as in every unit of one tile or of the text rows
  int seen;
};

// The key blocks of one query unit, in the order the forward kernel streams
// them: the full blocks of the window's key tiles (n_vfull), the full text
// blocks (n_tfull), then, when the video is not a tile multiple (PAD), one
// remainder block for every key tile whose tokens are not a multiple of 64
// (n_vrem), and last the partial text block when 64 does not divide the text
// length. Blocks before n_plain are whole; only the trailing ones are masked.
// Key tiles are walked by the residues of their coordinates modulo the window
// size (the window starts at (st, sh, sw) and spans (bt, bh, bw) tiles): query
// tiles whose windows overlap then reach each shared key tile at the same
// step of the walk. The text unit walks every tile (a box from the origin).
// block(j) must be called for j = 0, 1, 2, ... after reset().
template <bool PAD>
struct KeyStream {
  int st, sh, sw, bt, bh, bw;
  int n_vfull, n_vrem, n_tfull, n_plain, n_blk, text_len;
  int walk_a, walk_b, walk_c, tile_org, tile_ext, tile_sub, tile_nblk;

  __host__ __device__ void init(const Geom& g, int st_, int bt_, int sh_, int bh_, int sw_, int bw_) {
    st = st_;
    sh = sh_;
    sw = sw_;
    bt = bt_;
    bh = bh_;
    bw = bw_;
    n_vfull = bt * bh * bw * (kTileRows / kKeyBlock);
    n_vrem = 0;
    if (PAD) box_block_counts(st, bt, sh, bh, sw, bw, g, n_vfull, n_vrem);
    text_len = g.has_text ? g.text_length : 0;
    n_tfull = text_len / kKeyBlock;
    n_plain = n_vfull + n_tfull;
    n_blk = n_plain + n_vrem + (text_len % kKeyBlock != 0 ? 1 : 0);
    reset();
  }
  __host__ __device__ void reset() {
    walk_a = 0;
    walk_b = 0;
    walk_c = -1;
    tile_org = 0;
    tile_ext = kFullExtent;
    tile_sub = 0;
    tile_nblk = 0;
  }
  // coordinate in [s, s + w) congruent to r mod w (r in [0, w))
  __host__ __device__ static int residue_coord(int r, int s, int w) {
    const int d = (r - s) % w;
    return s + (d < 0 ? d + w : d);
  }
  // advance the walk to the next key tile; the remainder walk takes only its
  // last, partial block, the first walk only its full blocks
  __host__ __device__ void next_tile(const Geom& g, bool rem_walk) {
    if (++walk_c == bw) {
      walk_c = 0;
      if (++walk_b == bh) {
        walk_b = 0;
        ++walk_a;
      }
    }
    const int kt = residue_coord(walk_a, st, bt), kh = residue_coord(walk_b, sh, bh);
    const int kw = residue_coord(walk_c, sw, bw);
    tile_org = (kt * kTileT * g.H + kh * kTileH) * g.W + kw * kTileW;
    tile_ext = PAD ? tile_extent(kt, kh, kw, g) : kFullExtent;
    const int n_tok = extent_tokens(tile_ext);
    tile_sub = rem_walk ? n_tok / kKeyBlock : 0;
    tile_nblk = rem_walk ? tile_sub + (n_tok % kKeyBlock != 0 ? 1 : 0) : n_tok / kKeyBlock;
  }
  __host__ __device__ KeyBlock block(const Geom& g, int j) {
    KeyBlock s;
    const bool rem_walk = PAD && j >= n_plain;
    if (j < n_vfull || (rem_walk && j < n_plain + n_vrem)) {
      if (PAD && j == n_plain) reset();               // the first remainder block
      while (tile_sub == tile_nblk) next_tile(g, rem_walk);  // skips tiles without such blocks
      const int n_tok = extent_tokens(tile_ext);
      const bool frames = (tile_ext >> 8) == (kFullExtent >> 8);  // every row and column exists
      s.kind = frames ? 0 : 2;
      s.base = frames ? tile_org + tile_sub * g.H * g.W : tile_org;
      s.lim = kKeyBlock;
      s.ext = tile_ext;
      s.sub = tile_sub;
      const int left = n_tok - tile_sub * kKeyBlock;
      s.mask = left < kKeyBlock ? left : kKeyBlock;
      ++tile_sub;
      s.seen = -1;
    } else {
      const int tb = j < n_plain ? j - n_vfull : n_tfull;
      s.kind = 1;
      s.base = g.n_video + tb * kKeyBlock;
      const int left = text_len - tb * kKeyBlock;
      s.lim = left < kKeyBlock ? left : kKeyBlock;
      s.ext = kFullExtent;
      s.sub = 0;
      s.mask = s.lim;
      s.seen = -1;
    }
    return s;
  }
};

// The key blocks of a Hilbert-window query unit (2D image, T = 1): one block per
// key tile (its single 8x8 frame). A video unit is up to G = hil_group
// consecutive curve positions (the last unit of a head may hold fewer); their
// windows, which may differ by a shift, are streamed as their common core
// [first, first + count), walked by the residues of the positions modulo count
// (units whose windows overlap reach a shared tile at the same step), then the
// positions left of the core [lfirst, lfirst + lcount) and right of it
// [rfirst, rfirst + rcount), each seen by a contiguous range of the unit's
// tiles (KeyBlock::seen), then the text blocks as in KeyStream. Every
// row of the unit sees every core block. The text unit streams every tile.
// block(j) may be called in any order.
struct HilbertKeyStream {
  int first, count, lfirst, lcount, rfirst, rcount, m, G, W, mode;
  // slide: the window start of each of the unit's tiles, a large value past
  // its last tile (scalars: an array indexed at run time would put the whole
  // stream in per-lane memory)
  int st0, st1, st2, st3, st4, st5;
  int n_vfull, n_vrem, n_tfull, n_plain, n_blk, text_len;

  // pos0: curve position of the unit's first tile; text: a text unit, part
  // `part` of g.text_parts (tiles [part n / parts, (part + 1) n / parts) of
  // the n = n_tiles, the text keys with the last part)
  __host__ __device__ void init(const Geom& g, int pos0, int W_, bool text, int part = 0) {
    constexpr int kPast = 1 << 29;
    m = g.hil_m;
    W = W_;
    mode = g.hilbert;
    G = text ? 1 : g.hil_group;
    lcount = rcount = 0;
    lfirst = rfirst = 0;
    if (text) {
      first = int(int64_t(part) * g.n_tiles / g.text_parts);
      count = int(int64_t(part + 1) * g.n_tiles / g.text_parts) - first;
      st0 = st1 = st2 = st3 = st4 = st5 = kPast;
    } else {
      int c0;
      hilbert_window(pos0, W, g.n_tiles, mode, first, c0);
      count = c0;
      st0 = first;
      st1 = st2 = st3 = st4 = st5 = kPast;
      // tiles of this unit: G, or what is left of the curve
      const int tiles = g.n_tiles - pos0 < G ? g.n_tiles - pos0 : G;
      if (tiles > 1 && mode == 1) {
        const int n = g.n_tiles;
        st1 = window_start(pos0 + 1, W, n);
        int hi = st1;
        if (tiles > 2) hi = st2 = window_start(pos0 + 2, W, n);
        if (tiles > 3) hi = st3 = window_start(pos0 + 3, W, n);
        if (tiles > 4) hi = st4 = window_start(pos0 + 4, W, n);
        if (tiles > 5) hi = st5 = window_start(pos0 + 5, W, n);
        const int lo = st0;
        first = hi;  // core [hi, lo + W): the starts grow by at most 1 per position
        count = lo + W - hi;
        lfirst = lo;
        lcount = hi - lo;
        rfirst = lo + W;
        rcount = hi - lo;
      }
    }
    n_vfull = count + lcount + rcount;
    n_vrem = 0;
    text_len = g.has_text && (!text || part == g.text_parts - 1) ? g.text_length : 0;
    n_tfull = text_len / kKeyBlock;
    n_plain = n_vfull + n_tfull;
    n_blk = n_plain + (text_len % kKeyBlock != 0 ? 1 : 0);
  }
  __host__ __device__ void reset() {}
  __host__ __device__ KeyBlock block(const Geom& g, int j) const {
    KeyBlock s;
    s.seen = -1;
    if (j < n_vfull) {
      int p;
      if (j < count) {
        int d = (j - first) % count;
        d = d < 0 ? d + count : d;
        p = first + d;
      } else if (j < count + lcount) {
        // left of the core: tiles 0 .. t whose window starts at or before p
        // (the starts never decrease along the curve)
        p = lfirst + (j - count);
        const int t = (st1 <= p ? 1 : 0) + (st2 <= p ? 1 : 0) + (st3 <= p ? 1 : 0) + (st4 <= p ? 1 : 0) +
                      (st5 <= p ? 1 : 0);
        s.seen = (2 << t) - 1;
      } else {
        // right of the core: tiles t .. 3 whose window ends after p
        p = rfirst + (j - count - lcount);
        const int t = (st0 + W <= p ? 1 : 0) + (st1 + W <= p ? 1 : 0) + (st2 + W <= p ? 1 : 0) +
                      (st3 + W <= p ? 1 : 0) + (st4 + W <= p ? 1 : 0);
        s.seen = -(1 << t);
      }
      int tx, ty;
      hilbert_d2xy(m, p, tx, ty);
      s.kind = 0;
      s.base = ty * kTileH * g.W + tx * kTileW;
      s.lim = kKeyBlock;
      s.ext = tile_extent(0, ty, tx, g);
      s.sub = 0;
      s.mask = kKeyBlock;
    } else {
      const int tb = j < n_plain ? j - n_vfull : n_tfull;
      s.kind = 1;
      s.base = g.n_video + tb * kKeyBlock;
      const int left = text_len - tb * kKeyBlock;
      s.lim = left < kKeyBlock ? left : kKeyBlock;
      s.ext = kFullExtent;
      s.sub = 0;
      s.mask = s.lim;
    }
    return s;
  }
};

// The key blocks of an STA query unit of a 2x2 square of tiles (a one-frame
// video, Geom::hilbert == kSquareUnits; a tile is one frame of at most 8x8
// tokens, fewer in the last tile row or column when H or W is not a multiple
// of 8). Unit u of a head
// is square (sy, sx) (square_tiles: panels of square rows, column by column):
// the tiles (2 sy + dy, 2 sx + dx) that exist, in the order (0,0), (0,1), (1,1), (1,0)
// of (dy, dx) (square_tile), unit tile i being unit rows 64 i .. 64 i + 63.
// Along h, the windows of the two tile rows start at sh0 and sh1 = sh0 or
// sh0 + 1 (window_start never grows by more than one per tile), so the tiles
// they cover are a core [sh1, sh0 + wh) seen by both, plus, when sh1 > sh0,
// one row above the core seen by dy = 0 only and one below it seen by dy = 1
// only; the same along w. The unit streams its core first, walked by the
// residues of the key tile coordinates modulo the core's size (units whose
// cores overlap reach a shared tile at the same step), then the rows above
// and below the core across the full width, then the columns left and right
// of the core over its rows, each block with the mask of the unit's tiles
// that see it (KeyBlock::seen), then the text blocks as in KeyStream. With
// partial tiles every block carries its own mask (the tokens of a partial
// tile, the valid text keys), which the kernel applies to every block. The
// core is never empty when wh >= 2 and ww >= 2, or the square has a single
// tile row (column) along the axis where the window is 1, so block 0 is seen
// by every row of the unit. A text unit streams the key tiles of its part in
// raster tile order. block(j) may be called in any order.
__host__ __device__ inline void square_tile(int i, int layout, int& dy, int& dx) {
  // layout: 0 a full square, 1 one tile row (no dy = 1), 2 one tile column
  // (no dx = 1), 3 a single tile
  if (layout == 2) {
    dy = i;
    dx = 0;
  } else {
    dy = i >> 1;
    dx = (i ^ (i >> 1)) & 1;
  }
}

// Square rows per panel of the unit order (below).
constexpr int kSquarePanel = 8;

// Square (sy, sx) of unit u, its tiles (1, 2 or 4) and its layout for
// square_tile. Units run over panels of kSquarePanel square rows (the last
// panel may be lower), each panel column by column, so a run of consecutive
// units (what the resident workgroups of one XCD hold at once) is a compact
// block of squares whose windows overlap in both directions.
__host__ __device__ inline int square_tiles(const Geom& g, int u, int& sy, int& sx, int& layout) {
  const int n_sx = (g.nw + 1) >> 1, n_sy = (g.nh + 1) >> 1;
  const int panel = u / (kSquarePanel * n_sx);
  const int y0 = panel * kSquarePanel;
  const int ph = n_sy - y0 < kSquarePanel ? n_sy - y0 : kSquarePanel;  // this panel's square rows
  const int within = u - y0 * n_sx;
  sx = within / ph;
  sy = y0 + (within - sx * ph);
  const bool h1 = 2 * sy + 1 < g.nh, w1 = 2 * sx + 1 < g.nw;
  layout = h1 ? (w1 ? 0 : 2) : (w1 ? 1 : 3);
  return (h1 ? 2 : 1) * (w1 ? 2 : 1);
}

// PARTIAL: the image has a partial last tile row or column (H or W not a
// multiple of 8); with PARTIAL false every tile is a whole 8x8 frame.
template <bool PARTIAL>
struct SquareKeyStream {
  int ch, cw, Ch, Cw;  // the core: tile rows [ch, ch + Ch), tile columns [cw, cw + Cw)
  int mh, mw;          // 1 when the square's windows differ along h (w): one row (column) on each side
  int layout;          // square_tile's layout
  int first;           // text unit: its first key tile (raster tile order)
  int n_core, n_vfull, n_tfull, n_plain, n_blk, text_len;

  // u: the unit's square, or the text part when `text`
  __host__ __device__ void init(const Geom& g, int u, int wh, int ww, bool text) {
    if (text) {
      first = int(int64_t(u) * g.n_tiles / g.text_parts);
      n_core = int(int64_t(u + 1) * g.n_tiles / g.text_parts) - first;
      ch = cw = Ch = Cw = 0;
      mh = mw = 0;
      layout = 3;
    } else {
      first = 0;
      int sy, sx;
      square_tiles(g, u, sy, sx, layout);
      const int h0 = 2 * sy, w0 = 2 * sx;
      const int sh0 = window_start(h0, wh, g.nh);
      const int sh1 = (layout == 0 || layout == 2) ? window_start(h0 + 1, wh, g.nh) : sh0;
      const int sw0 = window_start(w0, ww, g.nw);
      const int sw1 = (layout == 0 || layout == 1) ? window_start(w0 + 1, ww, g.nw) : sw0;
      mh = sh1 - sh0;
      mw = sw1 - sw0;
      ch = sh1;
      Ch = wh - mh;
      cw = sw1;
      Cw = ww - mw;
      n_core = Ch * Cw;
    }
    // edge blocks: two rows of Cw + 2 mw tiles when mh, two columns of Ch tiles when mw
    n_vfull = n_core + 2 * mh * (Cw + 2 * mw) + 2 * mw * Ch;
    text_len = g.has_text && (!text || u == g.text_parts - 1) ? g.text_length : 0;
    n_tfull = text_len / kKeyBlock;
    n_plain = n_vfull + n_tfull;
    n_blk = n_plain + (text_len % kKeyBlock != 0 ? 1 : 0);
  }
  __host__ __device__ void reset() {}
  __host__ __device__ KeyBlock block(const Geom& g, int j) const {
    KeyBlock s;
    s.seen = -1;
    s.sub = 0;
    if (j < n_vfull) {
      int kh, kw;
      if (Ch == 0) {  // a text unit: key tile first + j in raster tile order
        kh = (first + j) / g.nw;
        kw = first + j - kh * g.nw;
      } else if (j < n_core) {
        const int jh = j / Cw, jw = j - jh * Cw;
        const int dh = (jh - ch) % Ch, dw = (jw - cw) % Cw;
        kh = ch + (dh < 0 ? dh + Ch : dh);
        kw = cw + (dw < 0 ? dw + Cw : dw);
      } else {
        // the tile rows (bit dy) and columns (bit dx) of the square that see the block
        int hsee = 3, wsee = 3;
        const int e = j - n_core, Uw = Cw + 2 * mw;
        if (e < 2 * mh * Uw) {
          const int r = e / Uw, c = e - r * Uw;
          kh = r == 0 ? ch - 1 : ch + Ch;
          hsee = r == 0 ? 1 : 2;
          kw = cw - mw + c;
          wsee = mw == 0 ? 3 : c == 0 ? 1 : c == Uw - 1 ? 2 : 3;
        } else {
          const int e2 = e - 2 * mh * Uw, side = e2 / Ch;
          kh = ch + (e2 - side * Ch);
          kw = side == 0 ? cw - 1 : cw + Cw;
          wsee = side == 0 ? 1 : 2;
        }
        int seen = 0;
        const int tiles = layout == 0 ? 4 : layout == 3 ? 1 : 2;
        for (int i = 0; i < tiles; ++i) {
          int dy, dx;
          square_tile(i, layout, dy, dx);
          seen |= ((hsee >> dy) & (wsee >> dx) & 1) << i;
        }
        s.seen = seen;
      }
      // a whole 8x8 tile is one full frame; a partial one (last tile row or
      // column of an image whose side is not a multiple of 8) holds fewer
      // tokens, fetched in compact order, the rest of its block masked
      s.base = kh * kTileH * g.W + kw * kTileW;
      s.ext = tile_extent(0, kh, kw, g);
      s.lim = PARTIAL ? extent_tokens(s.ext) : kKeyBlock;
      s.kind = !PARTIAL || s.lim == kKeyBlock ? 0 : 2;
      s.mask = s.lim;
    } else {
      const int tb = j < n_plain ? j - n_vfull : n_tfull;
      s.kind = 1;
      s.base = g.n_video + tb * kKeyBlock;
      const int left = text_len - tb * kKeyBlock;
      s.lim = left < kKeyBlock ? left : kKeyBlock;
      s.ext = kFullExtent;
      s.mask = s.lim;
    }
    return s;
  }
};

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
// Raster <-> Hilbert order of the video rows of a 2D image (g.hil_m set; text
// rows copied unchanged): row d of the Hilbert side is the token at curve
// position d of the order hil_m + 3 curve.
hipError_t launch_rows_hilbert(const Geom& g, const void* src, void* dst, bool to_hilbert,
                               hipStream_t stream);
hipError_t launch_schedule_lists(const Geom& g, const Windows& win, int32_t* offsets,
                                 int32_t* ids, hipStream_t stream);
// Work order (one query unit per entry, grouped into 8 per-XCD queues: queue x
// holds entries 8k + x). `claim`, when not null, receives kClaimInts zeros:
// the queue heads the attention kernel advances; `zero_row`, when not null,
// receives kZeroRowBytes zeros.
hipError_t launch_schedule_work(const Geom& g, const Windows& win, int32_t* work,
                                int32_t* claim, void* zero_row, hipStream_t stream);
constexpr int kQueues = 8;        // one per XCD
constexpr int kClaimStride = 64;  // ints between queue heads (own 256-byte line each)
constexpr int kClaimInts = kQueues * kClaimStride;

struct FwdArgs {
  const void* q;         // bf16 raster rows (the caller's q)
  const void* k;         // bf16 raster rows (the caller's k)
  const void* v;         // bf16 raster rows (the caller's v)
  void* out;             // bf16 raster rows (the caller's out)
  float* lse;            // fp32 raster (the caller's lse), or nullptr
  const int32_t* work;   // per-XCD queues of query units (launch_schedule_work)
  int32_t* claim;        // queue heads, zeroed by launch_schedule_work
  const void* zero_row;  // kZeroRowBytes of zeros (written by launch_schedule_work)
  // g.text_parts > 1: partial results of the text units, [B heads][text_parts]
  // [256 rows][D] fp32 (O, not normalised), then [B heads][text_parts][256
  // rows][2] fp32 (reference m in log2 units, row sum l); nullptr otherwise
  float* text_partial;
  float q_scale;         // log2(e) / sqrt(D), applied to the fp32 scores
};
constexpr int kZeroRowBytes = 256;  // one row of D = 128 bf16
hipError_t launch_attention(const Geom& g, const Windows& win, const FwdArgs& a, hipStream_t stream);

// Backward (gradients of the forward for an upstream gradient dout).
struct BwdArgs {
  const void* q;         // bf16 raster rows (the caller's q, k, v, dout)
  const void* k;
  const void* v;
  const void* dout;
  const void* zero_row;  // kZeroRowBytes of zeros (written by launch_bwd_prep)
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
                           void* zero_row, hipStream_t stream);
hipError_t launch_bwd_dq(const Geom& g, const Windows& win, const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dkv(const Geom& g, const Windows& win, const BwdArgs& a, hipStream_t stream);

}  // namespace sta
