// Fused STA attention kernel for gfx950 (CDNA4): bf16 MFMA, fp32 softmax.
//
// What it computes (STA README, "Usage" and "Why is STA Fast?"): for every
// query row, softmax(q k^T / sqrt(D)) v over the keys of whole key tiles in the
// query tile's window, followed by the valid text keys. Because every
// (query tile, key tile) block is fully on or fully off, video blocks need no
// per-element mask; only the last text block is masked, and only when the text
// length is not a multiple of 64 (and, for video sizes that are not tile
// multiples, the last block of a partial key tile).
//
// Work decomposition. A workgroup works on one query unit at a time: a
// 384-row query tile, 8 waves of 48 rows each (three 16-row column groups),
// or the 256 text query slots of one head, 8 waves of 32 rows each; two waves
// per SIMD, one workgroup per CU. The grid is persistent: each workgroup pops
// units from the queue of the XCD it runs on and, once that queue is empty,
// from the other XCDs' queues. The kernel enumerates each unit's key blocks
// itself (KeyStream: the window's key tiles in residue order, then the text),
// reads Q rows from the caller's raster q through the tile map, streams K and
// V rows from the caller's raster k and v into LDS with LDS-DMA (one source
// address per lane, which applies the tile map), and writes O and lse to
// raster positions. Two LDS stages of one 64-key block (K and V), one barrier
// per block; block j + 1 is fetched while block j is computed.
//
// Per block and wave, with v_mfma_f32_16x16x32_bf16:
//   S^T = K Q^T   A = K fragment (lane l: key 16kt + l%16, d 32ks + 8(l/16)
//                 .. +8), B = Q^T fragment (registers, loaded once per unit).
//                 Lane l then holds the scores of query l%16 for keys
//                 16kt + 4(l/16) + r, r = 0..3.
//   softmax       p = 2^(c s - m), c = log2(e)/sqrt(D) applied in fp32 (one
//                 v_fma_f32 and one v_exp_f32 per score), p rounded to bf16;
//                 the row sums accumulate the rounded p (v_dot2_f32_bf16).
//   O^T += V^T P^T  B = P^T from the lane's own registers (half h: keys
//                 32h + 4(l/16) + r and 32h + 16 + 4(l/16) + r), A = V^T
//                 fragment in the same key order, two ds_read_b64_tr_b16 from
//                 V rows in LDS (each gives lane l four consecutive keys of one
//                 column; see the V layout below).
//   The exponentials of key half 1 are scheduled between the MFMAs of half 0.
//   The kernel runs at the chip's power limit (the same cycle count takes
//   about 20% longer on random data than on zeros), so this overlap saves
//   cycles but little time.
//
// Softmax reference. m of a row is the exact maximum of its scaled scores
// over the first key block of the unit, and it never moves: p = 2^(c s - m)
// stays finite while no later score exceeds m by about 127 (log2 units). A
// row whose sum of p reaches 2^32 (some key at least 32 above the reference)
// makes the workgroup redo the unit with m set to the row's maximum over all
// its keys, found by a pass that computes only the scores. With random data
// the redo never happens; large score jumps between key tiles trigger it.
// Any reference gives the same softmax up to rounding.
//
// LDS layouts. K block (64 rows of D bf16): each 1 KB LDS-DMA transfer fills
// a group of 1024 / (2D) consecutive rows, interleaved at 64-byte granularity
// (quad k of every row of the group, then quad k + 1, ...), chunk j of row r
// of a quad at position j XOR (2 * bit 3 of r): every K fragment read (16 rows
// x one 16-byte chunk, served 16 lanes per LDS cycle) covers all 64 banks.
// V block: column-pair major, pair P = columns 32P .. 32P + 31 of all 64 rows,
// 64 bytes per row (4 KB per pair). A transposing read of column unit d (16
// columns) then takes 8 bytes at (lane / 4) * 64 + (lane % 4) * 8 from a
// compile-time offset; the LDS-DMA that fills a pair fetches 64 contiguous
// bytes of each row. An 8-byte LDS read serves lanes 0-31 in one cycle, so
// rows r and r + 4 share banks (a 2-way conflict); permuting each row's
// 16-byte chunks by bit 2 of the row removes it but measured no faster here
// (within +-1.5% across boxes), so the plain layout stays.
//
// Masking. Keys that must not contribute (text slots at or after text_length;
// with PAD, keys past a partial tile's tokens) are fetched from a zero row in
// the workspace, K and V alike, and their scores are replaced by -inf before
// the exponential: their p is exactly 0 and their V rows are zeros, so the
// contents of padded text slots never reach a result. KeyStream puts every
// block that can hold such keys after all whole blocks.
//
// Video sizes that are not tile multiples (PAD): the last tile along an axis
// holds the remainder. A partial key tile streams ceil(tokens / 64) blocks of
// its existing tokens in compact order (frame, row, column). A video unit's
// rows are its tile's existing tokens in compact order; a partial tile of at
// most 128, 192 or 256 tokens runs with 8 waves x 16 rows, 4 waves x 48 or 8
// waves x 32; a wave whose rows all lie past the tokens only loads and
// synchronises; rows past the tokens compute on a valid row and are not
// written.
// Epilogue: O = O^T / l rounded to bf16, lse = (m + log2 l) * ln 2, at raster rows.
#include <type_traits>

#include "sta_device.h"
#include "sta_internal.h"

namespace sta {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = kUnitRows / kWaves;  // 48
constexpr int kQT = kRowsPerWave / 16;            // 3 query column groups per wave
constexpr int kKPrefetch = 4;                     // K fragments in flight in the score loop
constexpr int kVPrefetch = 2;                     // V^T fragments in flight in the P V loop
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRedoSum = 4294967296.0f;  // 2^32: a row sum this large redoes the unit

struct KernelArgs {
  Geom g;
  FwdArgs a;
  Windows win;
};

// The kernel arguments through an opaque copy of the kernarg pointer: loads
// through it are not hoisted out of the unit loop.
__device__ inline const KernelArgs* kernel_args() {
  auto kp = (const __attribute__((address_space(4))) KernelArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(kp));
  return (const KernelArgs*)kp;
}

// GRP: query units of several 64-token tiles of a one-frame video (their rows
// in unit order, 64 per tile). kGrpHilbert, Hilbert-window attention
// (Geom::hilbert 1 or 2): video unit u is the hil_group tiles at Hilbert curve
// positions hil_group * u .. + hil_group - 1, or those of them that exist,
// with key tiles from HilbertKeyStream. kGrpSquares, STA on a one-frame video
// (Geom::hilbert == kSquareUnits): unit u is a 2x2 square of tiles, with key
// tiles from SquareKeyStream. A block that only some of the unit's tiles see
// (KeyBlock::seen) gives the other rows a reference of +inf, so their p is
// exactly 0. With GRP, the text rows may be split over text_parts units by
// key tiles. Everything else is the same kernel.
// kGrpSquaresPartial: squares on an image whose last tile row or column is
// partial (H or W not a multiple of 8).
constexpr int kGrpNone = 0, kGrpHilbert = 1, kGrpSquares = 2, kGrpSquaresPartial = 3;

template <int D, bool PAD, int GRP>
__global__ __launch_bounds__(kThreads, 1) void sta_attention_kernel(KernelArgs) {
  constexpr int KS = D / 32;                  // k-steps of S^T
  constexpr int DT = D / 16;                  // d groups of O^T (and V column units)
  constexpr int ROWB = D * 2;                 // bytes per row
  constexpr int BLK = kKeyBlock * ROWB;       // bytes of one K (or V) block
  constexpr int RPI = 1024 / ROWB;            // K rows per 1 KB LDS-DMA instruction
  constexpr int IPW = BLK / 1024 / kWaves;    // DMA instructions per wave per tensor
  constexpr int VPAIR = kKeyBlock * 64;       // bytes of one V column pair (4 KB)
  static_assert(IPW >= 1 && BLK % (1024 * kWaves) == 0, "block must split over the waves");
  constexpr bool HIL = GRP != kGrpNone;  // grouped units of 64-token tiles
  constexpr bool SQ = GRP == kGrpSquares || GRP == kGrpSquaresPartial;  // 2x2-square units
  constexpr bool SQP = GRP == kGrpSquaresPartial;                       // ... with partial tiles
  static_assert(!HIL || PAD, "grouped units are one-frame tiles");
  __shared__ __attribute__((aligned(1024))) char lds[2][2][BLK];  // [stage][K|V]
  __shared__ int shared_word[2];                                  // claimed unit, redo flag

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (;;) {
    // the previous unit's LDS reads are behind its barriers; this barrier
    // orders the claim (and the next unit's first LDS-DMA writes) after them
    __syncthreads();
    if (threadIdx.x == 0) {
      const KernelArgs* ka = kernel_args();
      unsigned xcc;
      asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
      shared_word[0] = claim_unit(ka->a.work, ka->a.claim, ka->g.B * ka->g.heads * ka->g.n_q, int(xcc));
      shared_word[1] = 0;
    }
    __syncthreads();
    const int unit = __builtin_amdgcn_readfirstlane(shared_word[0]);
    if (unit < 0) break;
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));  // lane-derived values are rebuilt per unit
    const int this_lane = lane;
    const KernelArgs* ka = kernel_args();
    const Geom g = ka->g;
    const FwdArgs a = ka->a;
    const int u = unit % g.n_q;
    const int bh = unit / g.n_q;
    const int hd = bh % g.heads;
    const uint32_t wp = ka->win.w[hd];
    const int n_vunits = HIL ? g.n_q - (g.has_text ? g.text_parts : 0) : g.n_tiles;
    const bool text_unit = g.has_text && u >= n_vunits;  // (grouped: text part u - n_vunits)

    // query tile coordinates and rows (PAD: its existing tokens, compact order)
    int qtt = 0, qth = 0, qtw = 0;
    int q_ext = kFullExtent, q_base = 0;
    int q_rows = text_unit ? kTextSlots : kTileRows;
    int sq_y = 0, sq_x = 0, sq_layout = 0;  // square units: the unit's square
    if (GRP == kGrpHilbert && !text_unit) {
      const int left = g.n_tiles - g.hil_group * u;
      q_rows = kKeyBlock * (left < g.hil_group ? left : g.hil_group);  // 64 rows per tile
    } else if (SQ && !text_unit) {
      q_rows = kKeyBlock * square_tiles(g, u, sq_y, sq_x, sq_layout);
    } else if (!text_unit) {
      const int rest = div_by(u, g.nw, g.mag_nw);
      qtw = u - rest * g.nw;
      qtt = div_by(rest, g.nh, g.mag_nh);
      qth = rest - qtt * g.nh;
      q_base = (qtt * kTileT * g.H + qth * kTileH) * g.W + qtw * kTileW;
      if constexpr (PAD) {
        q_ext = tile_extent(qtt, qth, qtw, g);
        q_rows = extent_tokens(q_ext);
      }
    }
    // raster row of unit row `row` (< q_rows)
    auto query_raster = [&](int row) {
      if (text_unit) return g.n_video + row;
      if constexpr (HIL) {  // row r of unit tile row / 64
        int tx, ty;
        if constexpr (SQ) {
          square_tile(row >> 6, sq_layout, ty, tx);
          ty += 2 * sq_y;
          tx += 2 * sq_x;
          if constexpr (SQP) {
            // tile (ty, tx) holds at most 8x8 tokens; a row past a partial
            // tile's tokens maps to its last one (computed, never written)
            const int e = tile_extent(0, ty, tx, g);
            const int n = extent_tokens(e);
            int r = row & 63;
            r = r < n ? r : n - 1;
            const int cols = extent_cols(e), dh = r / cols;
            return (ty * kTileH + dh) * g.W + tx * kTileW + (r - dh * cols);
          }
        } else {
          hilbert_d2xy(g.hil_m, g.hil_group * u + (row >> 6), tx, ty);
        }
        return (ty * kTileH + ((row >> 3) & 7)) * g.W + tx * kTileW + (row & 7);
      }
      int dt, dh, dw;
      if constexpr (PAD) {
        compact_token(row, q_ext, dt, dh, dw);
      } else {
        dt = row >> 6;
        dh = (row >> 3) & 7;
        dw = row & 7;
      }
      return q_base + (dt * g.H + dh) * g.W + dw;
    };

    // key blocks: the window of the query tile, or every tile for the text unit
    const int wt = win_t(wp), wh = win_h(wp), ww = win_w(wp);
    typename std::conditional<SQ, SquareKeyStream<SQP>,
                              typename std::conditional<HIL, HilbertKeyStream, KeyStream<PAD>>::type>::type keys;
    if constexpr (SQ) {
      keys.init(g, text_unit ? u - n_vunits : u, wh, ww, text_unit);
    } else if constexpr (HIL) {
      // the window length is the w component of the head's window
      keys.init(g, g.hil_group * u, ww, text_unit, text_unit ? u - n_vunits : 0);
    } else {
      if (text_unit)
        keys.init(g, 0, g.nt, 0, g.nh, 0, g.nw);
      else
        keys.init(g, window_start(qtt, wt, g.nt), wt, window_start(qth, wh, g.nh), wh, window_start(qtw, ww, g.nw),
                  ww);
    }
    const int n_plain = keys.n_plain, n_blk = keys.n_blk;

    const size_t slab = size_t(bh) * g.S * D;
    const char* __restrict__ kr = reinterpret_cast<const char*>(a.k) + slab * 2;
    const char* __restrict__ vr = reinterpret_cast<const char*>(a.v) + slab * 2;
    const char* __restrict__ zr = reinterpret_cast<const char*>(a.zero_row);

    // Chunk permutation of K row r inside its 64-byte quad (see the layout above).
    auto sw = [](int row) { return (row >> 2) & 2; };

    // ---- LDS-DMA of one key block into stage st: this wave's IPW groups of K
    // and of V. K group q holds rows q RPI .. + RPI - 1; lane p covers row
    // rin = (p / 4) % RPI and chunk 4 (p / (4 RPI)) + (p % 4 XOR sw). V group q
    // holds rows 16 (q % 4) .. + 15 of column pair q / 4; lane p covers row
    // 16 (q % 4) + p / 4 and bytes 64 (q / 4) + 16 (p % 4) .. + 15 of it.
    auto issue = [&](const KeyBlock& s, int st) {
      const int ln = opaque_lane<true>(this_lane);
      const int rin = (ln >> 2) % RPI;
      const int kchunk_hi = 4 * (ln / (4 * RPI));
      const int vr_lane = ln >> 2, vb_lane = 16 * (ln & 3);
      if (s.kind == 0) {
        // full frames: block row r at raster s.base + (r / 8) W + r % 8; each
        // K group lies in one 8-row run, each V group spans 2 runs
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
          const int q = wave * IPW + i, r0 = q * RPI;
          const int chunk = kchunk_hi + ((ln & 3) ^ sw(r0 + rin));
          const int krow0 = s.base + (r0 >> 3) * g.W + (r0 & 7);
          dma16_buf(kr, unsigned(rin * ROWB + chunk * 16), unsigned(krow0) * ROWB, &lds[st][0][q * 1024]);
          const int vrow0 = s.base + 2 * (q & 3) * g.W;
          const int voff = ((vr_lane >> 3) * g.W + (vr_lane & 7)) * ROWB + vb_lane;
          dma16_buf(vr, unsigned(voff), unsigned(vrow0) * ROWB + 64 * (q >> 2), &lds[st][1][q * 1024]);
        }
      } else if (!PAD || s.kind == 1) {
        // consecutive raster rows s.base + r, valid while r < s.lim
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
          const int q = wave * IPW + i, r = q * RPI + rin;
          const int chunk = kchunk_hi + ((ln & 3) ^ sw(r));
          const char* ks = r < s.lim ? kr + size_t(s.base + r) * ROWB : zr;
          dma16(ks + chunk * 16, &lds[st][0][q * 1024]);
          const int rv = 16 * (q & 3) + vr_lane;
          const char* vs = rv < s.lim ? vr + size_t(s.base + rv) * ROWB : zr;
          dma16(vs + 64 * (q >> 2) + vb_lane, &lds[st][1][q * 1024]);
        }
      } else {
        // PAD: compact token 64 s.sub + r of a partial tile, valid while it exists
        const int n_tok = extent_tokens(s.ext);
        auto src = [&](const char* base, int r) -> const char* {
          const int tok = s.sub * kKeyBlock + r;
          int dt, dh, dw;
          compact_token(tok < n_tok ? tok : 0, s.ext, dt, dh, dw);
          return tok < n_tok ? base + size_t(s.base + (dt * g.H + dh) * g.W + dw) * ROWB : zr;
        };
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
          const int q = wave * IPW + i, r = q * RPI + rin;
          const int chunk = kchunk_hi + ((ln & 3) ^ sw(r));
          dma16(src(kr, r) + chunk * 16, &lds[st][0][q * 1024]);
          dma16(src(vr, 16 * (q & 3) + vr_lane) + 64 * (q >> 2) + vb_lane, &lds[st][1][q * 1024]);
        }
      }
    };

    // The rest runs with QT query column groups per wave: 3 (8 x 48 = 384
    // rows) for a video tile, 2 (8 x 32 = 256 rows) for the text query slots;
    // a partial tile also uses 1 (16 rows per wave) or 3 with only waves 0-3
    // holding rows.
    auto run = [&](auto qt_c) {
      constexpr int QT = decltype(qt_c)::value;
      constexpr int RPW = QT * 16;  // query rows per wave
      const bool active = wave * RPW < q_rows;
      const float qs = a.q_scale;  // log2(e)/sqrt(D), applied to the fp32 scores

      // Q^T fragments for this wave's rows (rows past the unit clamp to its last)
      bf16x8 qf[QT][KS];
#pragma unroll
      for (int c = 0; c < QT; ++c) {
        int row = wave * RPW + c * 16 + (lane & 15);
        row = row < q_rows ? row : q_rows - 1;
        const bf16x8* src = reinterpret_cast<const bf16x8*>(reinterpret_cast<const __bf16*>(a.q) + slab +
                                                            size_t(query_raster(row)) * D + (lane >> 4) * 8);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[c][ks] = src[ks * 4];
      }

      f32x4 acc[QT][DT];
      float l_part[QT];  // this lane's share of the row sum of p
      float m_run[QT];   // reference of the scaled scores (log2 units)
      bf16x2 ones2;
      ones2[0] = (__bf16)1.0f;
      ones2[1] = (__bf16)1.0f;

      // K fragment (row 16kt + lane%16, chunk 4ks + lane/16) of a block sits at
      // kofs + kt * 16 * ROWB + ks * 64 * RPI
      const int l15 = lane & 15;
      const int kofs = (l15 / RPI) * 1024 + (l15 % RPI) * 64 + (((lane >> 4) ^ sw(l15)) << 4);

      // S^T of the block in stage `stage`, keys at or past `mask` (< 64) set to -inf
      auto scores = [&](f32x4 (&s)[QT][4], int stage, int mask) {
        const char* kb = lds[stage][0];
        constexpr int NF = 4 * KS;
        bf16x8 kf[NF];
        auto kload = [&](int f) {
          kf[f] = *reinterpret_cast<const bf16x8*>(kb + kofs + (f & 3) * 16 * ROWB + (f >> 2) * 64 * RPI);
        };
#pragma unroll
        for (int f = 0; f < kKPrefetch; ++f) kload(f);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const int ks = f >> 2, kt = f & 3;
#pragma unroll
          for (int c = 0; c < QT; ++c)
            s[c][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[f], qf[c][ks],
                                                              ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : s[c][kt], 0, 0, 0);
          if (f + kKPrefetch < NF) kload(f + kKPrefetch);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (mask < kKeyBlock) {
          int key0 = 4 * (lane >> 4);
          asm volatile("" : "+v"(key0));  // build the lane masks here, not before the loop
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (key0 + 16 * kt + r >= mask)
#pragma unroll
                for (int c = 0; c < QT; ++c) s[c][kt][r] = -INFINITY;
        }
      };
      // exact scaled row maxima of a block's scores (each row's 64 keys are
      // spread over the 4 lanes l%16 + 16i)
      auto row_max = [&](const f32x4 (&s)[QT][4], float (&mx)[QT]) {
#pragma unroll
        for (int c = 0; c < QT; ++c) {
          float x = s[c][0][0];
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) x = fmaxf(x, s[c][kt][r]);
          mx[c] = swap32_max(swap16_max(x));
        }
      };

      // grouped units: whether some row of this wave lies in a unit tile that
      // sees a block (the wave's rows span unit tiles t_lo .. t_hi)
      auto wave_sees = [&](int seen) {
        const int t_lo = (wave * RPW) >> 6, t_hi = (wave * RPW + RPW - 1) >> 6;
        return ((seen >> t_lo) & ((2 << (t_hi - t_lo)) - 1)) != 0;
      };

      // ---- the main pass; m_run is known (from the max pass) when `known`
      auto main_pass = [&](bool known) {
#pragma unroll
        for (int c = 0; c < QT; ++c) {
#pragma unroll
          for (int d = 0; d < DT; ++d) acc[c][d] = f32x4{0.f, 0.f, 0.f, 0.f};
          l_part[c] = 0.f;
        }
        keys.reset();
        KeyBlock s_cur = keys.block(g, 0);
        issue(s_cur, 0);
        wait_loads();  // the Q rows (and block 0) have landed: no compiler waits inside the loop
        for (int j = 0; j < n_blk; ++j) {
          const int stage = j & 1;
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          __syncthreads();
          const int seen = s_cur.seen;  // of block j
          // grouped units of 32 or 16 rows per wave: a wave none of whose
          // rows sees the block only issues its share of the next block's
          // loads (block 0 is seen by every row; 48-row waves, whose registers
          // leave no room for the branch, compute every block)
          const bool work = !HIL || QT == kQT || wave_sees(seen);
          f32x4 s[QT][4];
          // squares with partial tiles: every block's own mask (they may come anywhere)
          if (work) scores(s, stage, SQP || j >= n_plain ? s_cur.mask : kKeyBlock);
          if (j + 1 < n_blk) {
            s_cur = keys.block(g, j + 1);
            issue(s_cur, stage ^ 1);
          }
          if (work) {
            if (j == 0 && !known) {
              float mx[QT];
              row_max(s, mx);
#pragma unroll
              for (int c = 0; c < QT; ++c) m_run[c] = mx[c] * qs;
            }
            // the reference of each row for this block: +inf for rows that do not see it
            float mb[QT];
#pragma unroll
            for (int c = 0; c < QT; ++c) mb[c] = m_run[c];
            if constexpr (HIL) {
              if (seen != -1) {
#pragma unroll
                for (int c = 0; c < QT; ++c) {
                  const int row = wave * RPW + c * 16 + (lane & 15);
                  mb[c] = ((seen >> (row >> 6)) & 1) != 0 ? m_run[c] : INFINITY;
                }
              }
            }
            // p = 2^(c s - m) rounded to bf16; O^T += V^T P^T; row sums += 1^T P^T.
            // The exponentials of key half 1 are interleaved with the MFMAs of
            // half 0 (they are independent), so the VALU work of that half runs
            // under the matrix core.
            const char* vb = lds[stage][1] + (lane >> 2) * 64 + (lane & 3) * 8;
            // V^T fragment d of half h: keys 32h + 4(l/16) + e and
            // 32h + 16 + 4(l/16) + e of column 16d + l%16
            auto vload = [&](int h, int d) -> bf16x8 {
              const char* p0 = vb + (d >> 1) * VPAIR + 32 * (d & 1) + 32 * h * 64;
              const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0);
              const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 16 * 64));
              return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
            };
            auto probs = [&](int h, bf16x8 (&pb)[QT]) {
#pragma unroll
              for (int c = 0; c < QT; ++c) {
                f32x8 p;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                  p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[c][2 * h][r], qs, -mb[c]));
                  p[4 + r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[c][2 * h + 1][r], qs, -mb[c]));
                }
                pb[c] = __builtin_convertvector(p, bf16x8);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const bf16x2 pair = {pb[c][2 * i], pb[c][2 * i + 1]};
                  l_part[c] = __builtin_amdgcn_fdot2_f32_bf16(pair, ones2, l_part[c], false);
                }
              }
            };
            bf16x8 vf0[DT], vf1[DT], pb0[QT], pb1[QT];
#pragma unroll
            for (int d = 0; d < kVPrefetch; ++d) vf0[d] = vload(0, d);
            probs(0, pb0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int d = 0; d < DT; ++d) {
#pragma unroll
              for (int c = 0; c < QT; ++c)
                acc[c][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf0[d], pb0[c], acc[c][d], 0, 0, 0);
              if (d + kVPrefetch < DT) vf0[d + kVPrefetch] = vload(0, d + kVPrefetch);
            }
            probs(1, pb1);
#pragma unroll
            for (int d = 0; d < kVPrefetch; ++d) vf1[d] = vload(1, d);
            // per MFMA of half 0: one LDS read and up to 3 VALU instructions
#pragma unroll
            for (int i = 0; i < QT * DT; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int d = 0; d < DT; ++d) {
#pragma unroll
              for (int c = 0; c < QT; ++c)
                acc[c][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf1[d], pb1[c], acc[c][d], 0, 0, 0);
              if (d + kVPrefetch < DT) vf1[d + kVPrefetch] = vload(1, d + kVPrefetch);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
      };

      // ---- pass 1 of a redo: the exact row maxima over all keys, scores only
      auto max_pass = [&]() {
        float mx[QT];
#pragma unroll
        for (int c = 0; c < QT; ++c) mx[c] = -INFINITY;
        keys.reset();
        wait_loads();
        for (int j = 0; j < n_blk; ++j) {
          const KeyBlock s_j = keys.block(g, j);
          issue(s_j, 0);
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          __syncthreads();
          if (HIL && !wave_sees(s_j.seen)) {
            __syncthreads();  // every wave has read the stage before it is refilled
            continue;
          }
          f32x4 s[QT][4];
          scores(s, 0, SQP || j >= n_plain ? s_j.mask : kKeyBlock);
          float bm[QT];
          row_max(s, bm);
#pragma unroll
          for (int c = 0; c < QT; ++c) {
            const int row = wave * RPW + c * 16 + (lane & 15);
            const bool sees = !HIL || ((s_j.seen >> (row >> 6)) & 1) != 0;
            mx[c] = sees ? fmaxf(mx[c], bm[c]) : mx[c];
          }
          __syncthreads();  // every wave has read the stage before it is refilled
        }
#pragma unroll
        for (int c = 0; c < QT; ++c) m_run[c] = mx[c] * qs;
      };

      // ---- a wave without rows: the same loads and barriers
      auto idle_main = [&]() {
        keys.reset();
        issue(keys.block(g, 0), 0);
        for (int j = 0; j < n_blk; ++j) {
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          __syncthreads();
          if (j + 1 < n_blk) issue(keys.block(g, j + 1), (j & 1) ^ 1);
        }
      };
      auto idle_max = [&]() {
        keys.reset();
        for (int j = 0; j < n_blk; ++j) {
          issue(keys.block(g, j), 0);
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          __syncthreads();
          __syncthreads();
        }
      };

      if (!active) {
        idle_main();
        __syncthreads();
        if (__builtin_amdgcn_readfirstlane(shared_word[1]) != 0) {
          __syncthreads();
          idle_max();
          idle_main();
        }
        return;
      }
      // a second pass, with the exact row maxima as reference, when some
      // row's sum (relative to the first block's maximum) got large
      for (bool known = false;; known = true) {
        main_pass(known);
        if (known) break;
        bool redo = false;
#pragma unroll
        for (int c = 0; c < QT; ++c) redo |= !(swap32_sum(swap16_sum(l_part[c])) < kRedoSum);
        if (__builtin_amdgcn_ballot_w64(redo) != 0 && lane == 0) shared_word[1] = 1;
        __syncthreads();
        if (__builtin_amdgcn_readfirstlane(shared_word[1]) == 0) break;
        __syncthreads();
        max_pass();
      }

      if constexpr (HIL) {
        // a text unit that holds a part of the keys: O (not normalised), the
        // reference and the row sum, merged by text_merge_kernel
        if (text_unit && g.text_parts > 1) {
          const size_t slot = size_t(bh) * g.text_parts + (u - n_vunits);
          float* __restrict__ op = a.text_partial + slot * kTextSlots * D;
          float* __restrict__ ml =
              a.text_partial + size_t(g.B) * g.heads * g.text_parts * kTextSlots * D + slot * kTextSlots * 2;
#pragma unroll
          for (int c = 0; c < QT; ++c) {
            const float l = swap32_sum(swap16_sum(l_part[c]));
            const int row = wave * RPW + c * 16 + (lane & 15);
            float* dst = op + size_t(row) * D + (lane >> 4) * 4;
#pragma unroll
            for (int d = 0; d < DT; ++d) *reinterpret_cast<f32x4*>(dst + d * 16) = acc[c][d];
            if (lane < 16) *reinterpret_cast<float2*>(ml + 2 * row) = float2{m_run[c], l};
          }
          return;
        }
      }
      // ---- epilogue: O = O^T / l in bf16 and lse, straight to raster positions
      __bf16* __restrict__ outr = reinterpret_cast<__bf16*>(a.out) + slab;
      float* __restrict__ lser = a.lse == nullptr ? nullptr : a.lse + size_t(bh) * g.S;
#pragma unroll
      for (int c = 0; c < QT; ++c) {
        const float l = swap32_sum(swap16_sum(l_part[c]));
        const float inv = __builtin_amdgcn_rcpf(l);
        const int row = wave * RPW + c * 16 + (lane & 15);
        bool written = row < q_rows;
        if constexpr (SQP) {
          // rows past a partial tile's tokens are computed on its last token, not written
          if (!text_unit && written) {
            int ty, tx;
            square_tile(row >> 6, sq_layout, ty, tx);
            written = (row & 63) < extent_tokens(tile_extent(0, ty + 2 * sq_y, tx + 2 * sq_x, g));
          }
        }
        if (written) {
          const int rr = query_raster(row);
          __bf16* dst = outr + size_t(rr) * D + (lane >> 4) * 4;
#pragma unroll
          for (int d = 0; d < DT; ++d) {
            const f32x4 o = acc[c][d] * inv;
            *reinterpret_cast<bf16x4*>(dst + d * 16) = __builtin_convertvector(o, bf16x4);
          }
          if (lser != nullptr && lane < 16) lser[rr] = (m_run[c] + __builtin_amdgcn_logf(l)) * kLn2;
        }
      }
    };
    if constexpr (PAD) {
      if (!text_unit && q_rows <= 16 * kWaves) {  // a small partial tile: 8 (or fewer) waves x 16 rows
        run(std::integral_constant<int, 1>{});
        continue;
      }
    }
    // 8 waves x 32 rows for the text slots and for partial tiles of 193 to 256
    // tokens; otherwise 48 rows per wave (4 waves do the work for at most 192)
    if (text_unit || (PAD && q_rows > 4 * 16 * kQT && q_rows <= kTextSlots))
      run(std::integral_constant<int, kTextSlots / 16 / kWaves>{});
    else
      run(std::integral_constant<int, kQT>{});
  }
}

// The text rows of a grouped call whose text units each took a part of the
// keys: per row, with M = max over the parts of their reference m_p and
// w_p = 2^(m_p - M), out = sum_p w_p O_p / sum_p w_p l_p in bf16 and lse =
// (M + log2 sum_p w_p l_p) ln 2. Grid (B heads, 256 / 4), 4 rows of 64 threads
// per workgroup, D / 64 columns per thread.
template <int D>
__global__ __launch_bounds__(256) void text_merge_kernel(Geom g, const float* __restrict__ part,
                                                         __bf16* __restrict__ out, float* __restrict__ lse) {
  constexpr int CPT = D / 64;
  const int bh = blockIdx.x;
  const int row = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int col = (threadIdx.x & 63) * CPT;
  const int P = g.text_parts;
  const float* ml = part + size_t(g.B) * g.heads * P * kTextSlots * D;
  float M = -INFINITY;
  for (int p = 0; p < P; ++p) M = fmaxf(M, ml[((size_t(bh) * P + p) * kTextSlots + row) * 2]);
  float L = 0.f, o[CPT] = {};
  for (int p = 0; p < P; ++p) {
    const size_t slot = size_t(bh) * P + p;
    const float w = __builtin_amdgcn_exp2f(ml[(slot * kTextSlots + row) * 2] - M);
    L += w * ml[(slot * kTextSlots + row) * 2 + 1];
    const float* op = part + (slot * kTextSlots + row) * D + col;
#pragma unroll
    for (int i = 0; i < CPT; ++i) o[i] += w * op[i];
  }
  const float inv = 1.f / L;
  const size_t orow = size_t(bh) * g.S + g.n_video + row;
#pragma unroll
  for (int i = 0; i < CPT; ++i) out[orow * D + col + i] = __bf16(o[i] * inv);
  if (lse != nullptr && col == 0) lse[orow] = (M + __builtin_amdgcn_logf(L)) * kLn2;
}

// Resident workgroups of the kernel on the current device (cached per device).
template <int D, bool PAD, int GRP>
int persistent_grid() {
  static int cache[kMaxDevices] = {};
  return resident_workgroups(sta_attention_kernel<D, PAD, GRP>, kThreads, cache);
}

template <int D, bool PAD, int GRP = kGrpNone>
hipError_t launch(const Geom& g, const Windows& win, const FwdArgs& a, hipStream_t stream) {
  const int units = g.B * g.heads * g.n_q;
  const int resident = persistent_grid<D, PAD, GRP>();
  if (resident <= 0) return hipErrorInvalidDevice;
  const int grid = units < resident ? units : resident;
  sta_attention_kernel<D, PAD, GRP><<<grid, kThreads, 0, stream>>>(KernelArgs{g, a, win});
  if (GRP != kGrpNone && g.has_text && g.text_parts > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    text_merge_kernel<D><<<dim3(g.B * g.heads, kTextSlots / 4), 256, 0, stream>>>(
        g, a.text_partial, static_cast<__bf16*>(a.out), a.lse);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const Geom& g, const Windows& win, const FwdArgs& a, hipStream_t stream) {
  // one-frame images (grouped units): never a tile multiple
  if (g.hilbert == kSquareUnits && (g.H % kTileH != 0 || g.W % kTileW != 0))
    return g.D == 128 ? launch<128, true, kGrpSquaresPartial>(g, win, a, stream)
                      : launch<64, true, kGrpSquaresPartial>(g, win, a, stream);
  if (g.hilbert == kSquareUnits)
    return g.D == 128 ? launch<128, true, kGrpSquares>(g, win, a, stream)
                      : launch<64, true, kGrpSquares>(g, win, a, stream);
  if (g.hilbert != 0)
    return g.D == 128 ? launch<128, true, kGrpHilbert>(g, win, a, stream)
                      : launch<64, true, kGrpHilbert>(g, win, a, stream);
  if (g.full) return g.D == 128 ? launch<128, false>(g, win, a, stream) : launch<64, false>(g, win, a, stream);
  return g.D == 128 ? launch<128, true>(g, win, a, stream) : launch<64, true>(g, win, a, stream);
}

}  // namespace sta
