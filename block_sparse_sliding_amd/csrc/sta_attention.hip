// Fused STA attention kernel for gfx950 (CDNA4): bf16 MFMA, fp32 online softmax.
//
// What it computes (STA README, "Usage" and "Why is STA Fast?"): for every
// query row, softmax(q k^T / sqrt(D)) v over the keys of whole key tiles in the
// query tile's window, followed by the valid text keys. Because every
// (query tile, key tile) block is fully on or fully off, video blocks need no
// per-element mask; only the last text block is masked, and only when the text
// length is not a multiple of 64.
//
// Work decomposition. A workgroup works on one query unit at a time: a
// 384-row query tile, 8 waves of 48 rows each (three 16-row column groups),
// or the 256 text query slots of one head, 8 waves of 32 rows each; two waves
// per SIMD, one workgroup per CU. The grid is persistent (one workgroup per
// resident slot): each workgroup pops units from the queue of the XCD it runs
// on and, once that queue is empty, from the other XCDs' queues, so the split
// of work between XCDs follows their actual clocks (which differ by several
// percent under load) instead of being fixed at launch. Q rows are read from
// the caller's raster q through the tile map, and O / lse are written back to
// raster positions. Keys stream in 64-key blocks into LDS with LDS-DMA loads,
// double buffered, one barrier per block: K straight from the caller's raster
// k (each lane supplies its own source address, which applies the tile map),
// V as packed V^T fragments (one contiguous 16 KB run per block at D = 128,
// written by the pack kernel). The next block's loads are issued once the
// current block's score MFMAs are under way.
//
// LDS layout of a K block (64 rows of D bf16). Each 1 KB LDS-DMA transfer
// fills one group of 1024 / (2D) consecutive rows. Inside a group the rows
// are interleaved at 64-byte granularity: quad k (16-byte chunks 4k..4k+3) of
// every row of the group, then quad k + 1, and so on; within a quad, chunk j
// of row r sits at position j XOR (2 * bit 3 of r). Every read address is one
// per-lane base plus compile-time offsets. gfx950 serves a ds_read_b128 in
// four LDS cycles of 16 lanes each, lane l in cycle (bit 5 of l, parity of
// bits 2..4 of l) (measured with the LDS bank-conflict counter); with this
// permutation the 16 lanes of every cycle of a K fragment read (16 rows x one
// chunk) cover all 64 banks, for D = 128 and D = 64 alike. Without it, or
// with a permutation that ignores that lane grouping, two lanes of each cycle
// share banks and every K fragment read takes 8 LDS cycles instead of 4.
//
// Per block and wave, with v_mfma_f32_16x16x32_bf16:
//   S^T = K Q^T   A = K fragment (lane l holds K[16kt + l%16][32ks + 8(l/16)
//                 .. +8]), B = Q^T fragment (registers, loaded once per unit),
//                 fp32 accumulation of the exact bf16 products. Lane l then
//                 holds the scores of query l%16 for keys 4(l/16) + r of each
//                 16-key group.
//   softmax       p = 2^(c s - m) with c = log2(e)/sqrt(D) applied in fp32
//                 (one v_fma_f32 and one v_exp_f32 per score; folding c into
//                 a bf16 operand instead would round it and cost accuracy at
//                 large logits), m the running reference in log2 units. The
//                 reference only moves when some scaled score exceeds it by
//                 more than kRescaleSlack (a per-lane v_max3 check and a
//                 ballot); then the accumulator and row sums are rescaled.
//                 The first block sets the reference from its exact row max.
//                 Any reference gives the same softmax; the slack bounds p by
//                 2^slack.
//   O^T += V^T P^T  A = packed V^T fragment (one ds_read_b128; its key order
//                 matches the accumulator layout of S^T), B = P^T from the
//                 lane's own registers after bf16 rounding. The row sums
//                 accumulate the same rounded p with v_dot2_f32_bf16.
// Text rows at or after text_length only ever appear in the last text block:
// their scores are replaced by -inf (a select, so whatever k holds there is
// ignored) and their packed V rows are zeros.
// Video sizes that are not tile multiples (the PAD instantiation): the last
// tile along an axis holds the remainder, and a partial key tile streams
// ceil(tokens / 64) blocks of its existing tokens in compact order (frame,
// row, column; the packed V^T uses the same order). In the last block, keys
// past the tile's tokens are fetched from the last token that exists (every
// source address stays inside the video), their scores are replaced by -inf
// and their packed V rows are zeros. A
// video unit's rows are its tile's existing tokens in compact order (frame,
// row, column; a partial tile of at most 128, 192 or 256 tokens runs with
// 8 waves x 16 rows, 4 waves x 48 or 8 waves x 32; a wave whose rows all lie
// past the tokens only loads and synchronises);
// rows past them compute on a valid row and are not written. The first block
// of every window is frame 0 of an existing tile, so the running max is
// finite from the first block on.
// Epilogue: O = O^T / l rounded to bf16, lse = (m + log2 l) * ln 2, at raster rows.
#include <type_traits>

#include "sta_device.h"
#include "sta_internal.h"

namespace sta {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = kUnitRows / kWaves;  // 48
constexpr int kQT = kRowsPerWave / 16;            // 3 query column groups per wave
constexpr float kRescaleSlack = 8.0f;             // log2 units
constexpr int kKPrefetch = 4;                     // K fragments in flight in the score loop
constexpr float kLn2 = 0.69314718055994530942f;

struct KernelArgs {
  Geom g;
  FwdArgs a;
  Windows win;  // read by the PAD instantiation only
};

// The kernel arguments seen through an opaque copy of the kernarg pointer:
// loads through it cannot be hoisted out of the unit loop, so the per-unit
// code reads them again (scalar loads) instead of keeping them all live in
// SGPRs across the loop.
__device__ inline const KernelArgs* kernel_args() {
  auto kp = (const __attribute__((address_space(4))) KernelArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(kp));
  return (const KernelArgs*)kp;
}

template <int D, bool PAD>
__global__ __launch_bounds__(kThreads, 1) void sta_attention_kernel(KernelArgs) {
  constexpr int KS = D / 32;                // k-steps of S^T
  constexpr int DT = D / 16;                // d groups of O^T
  constexpr int ROWB = D * 2;               // bytes per K row
  constexpr int BLK = kKeyBlock * ROWB;     // bytes of one K (or V^T) block
  constexpr int RPI = 1024 / ROWB;          // K rows per 1 KB LDS-DMA instruction
  constexpr int IPW = BLK / 1024 / kWaves;  // DMA instructions per wave per tensor
  constexpr int BPT = kTileRows / kKeyBlock;  // key blocks per tile (6)
  static_assert(IPW >= 1 && BLK % (1024 * kWaves) == 0, "block must split over the waves");
  __shared__ __attribute__((aligned(1024))) char lds[2][2][BLK];  // [stage][K|V]

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  __shared__ int claimed;
  for (;;) {
  // The previous unit's last LDS reads are behind the body's barriers; this
  // barrier orders the claim (and the next unit's first LDS-DMA writes)
  // after all of them.
  if (threadIdx.x == 0) {
    const KernelArgs* ka = kernel_args();
    unsigned xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    claimed = claim_unit(ka->a.work, ka->a.claim, ka->g.B * ka->g.heads * ka->g.n_q, int(xcc));
  }
  __syncthreads();
  const int unit = __builtin_amdgcn_readfirstlane(claimed);
  if (unit < 0) break;
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));  // lane-derived offsets are rebuilt per unit, not kept live
  const int this_lane = lane;
  const KernelArgs* ka = kernel_args();
  const Geom g = ka->g;
  const FwdArgs a = ka->a;
  const int u = unit % g.n_q;
  const int bh = unit / g.n_q;
  const int hd = bh % g.heads;
  const bool text_unit = g.has_text && u == g.n_tiles;
  const int q_row0 = text_unit ? g.n_vt : u * kTileRows;  // tile-major
  int q_rows = text_unit ? kTextSlots : kTileRows;
  // PAD: the rows of a video unit are the existing tokens of its tile in
  // compact order (frame, row, column), so a partial tile runs as a unit of
  // 128, 192, 256 or 384 rows (the shapes are chosen below)
  int q_ext = kFullExtent, q_base = 0;  // extent and raster origin of the query tile
  if constexpr (PAD) {
    if (!text_unit) {
      const int rest = div_by(u, g.nw, g.mag_nw);
      const int tw = u - rest * g.nw;
      const int tt = div_by(rest, g.nh, g.mag_nh);
      const int th = rest - tt * g.nh;
      q_ext = tile_extent(tt, th, tw, g);
      q_rows = extent_tokens(q_ext);
      q_base = (tt * kTileT * g.H + th * kTileH) * g.W + tw * kTileW;
    }
  }
  // raster row of unit row `row` (< q_rows)
  auto query_raster = [&](int row) {
    if constexpr (PAD) {
      if (!text_unit) {
        int dt, dh, dw;
        compact_token(row, q_ext, dt, dh, dw);
        return q_base + (dt * g.H + dh) * g.W + dw;
      }
    }
    return PAD ? tiled_to_raster(q_row0 + row, g) : tiled_to_raster_full(q_row0 + row, g);
  };
  const size_t slab = size_t(bh) * g.S * D;      // element offset of this (b, head), raster
  const size_t slab_t = size_t(bh) * g.S_t * D;  // the same in the packed tile-major V^T

  const __bf16* __restrict__ qr = reinterpret_cast<const __bf16*>(a.q) + slab;
  const char* __restrict__ kr = reinterpret_cast<const char*>(a.k) + slab * 2;
  const char* __restrict__ vtr = reinterpret_cast<const char*>(a.vt) + slab_t * 2;

  const int l0 = a.offsets[hd * g.n_q + u];
  const int l1 = a.offsets[hd * g.n_q + u + 1];
  // video key blocks: six per listed tile; with PAD, ceil(tokens / 64) per
  // tile, its existing tokens in compact order, summed over the unit's list:
  // the query tile's window (a box of tiles) or, for the text unit, the grid
  int n_vid = (l1 - l0) * BPT;
  if constexpr (PAD) {
    if (text_unit) {
      n_vid = box_blocks(0, g.nt, 0, g.nh, 0, g.nw, g);
    } else {
      const uint32_t p = ka->win.w[hd];
      const int rest = div_by(u, g.nw, g.mag_nw);
      const int tt = div_by(rest, g.nh, g.mag_nh);
      const int th = rest - tt * g.nh, tw = u - rest * g.nw;
      n_vid = box_blocks(window_start(tt, win_t(p), g.nt), win_t(p), window_start(th, win_h(p), g.nh),
                         win_h(p), window_start(tw, win_w(p), g.nw), win_w(p), g);
    }
  }
  const int text_len = g.has_text ? g.text_length : 0;
  const int n_blk = n_vid + (text_len + kKeyBlock - 1) / kKeyBlock;
  const bool ragged = (text_len % kKeyBlock) != 0;

  // Chunk permutation of K row r inside its 64-byte quad (see the layout above).
  auto sw = [](int row) { return (row >> 2) & 2; };

  // The schedule is read through the scalar cache (it is never written while
  // this kernel runs). Key blocks of one tile are consecutive.
  const __attribute__((address_space(4))) int32_t* ids =
      (const __attribute__((address_space(4))) int32_t*)(a.ids + l0);

  // Source rows of key block j (blocks are fetched in order 0, 1, 2, ...; the
  // six blocks of a tile are its six frames, so a tile is decoded once, at its
  // first block): kbase = raster row of the block's 8x8 (h, w) patch origin
  // (video) or first slot (text), krs = raster stride between its 8-row
  // runs, vrow = its first tile-major row (the packed V^T block). With PAD,
  // tile_ext is the packed extent of the current tile (the frames, rows and
  // columns that exist); a tile with only frames missing still has one frame
  // per block, otherwise a block is 64 tokens in compact order (issue_k).
  int tile_kbase = 0, tile_vrow = 0;
  int tile_ext = kFullExtent;  // PAD: packed extent of the current tile
  // PAD: blocks walk the blocks of each listed tile in turn (block j + 1 is
  // always decoded right after block j): cur_t is the next list entry,
  // cur_sub the block within its tile of the last decoded block
  int cur_t = 0, cur_sub = -1;
  auto block_rows = [&](int j, int& kbase, int& krs, int& vrow) {
    if (j < n_vid) {
      int t, sub;
      if constexpr (PAD) {
        sub = cur_sub + 1;
        if (j == 0 || sub * kKeyBlock >= extent_tokens(tile_ext)) {
          sub = 0;
          t = cur_t++;
        }
        cur_sub = sub;
      } else {
        t = j / BPT;
        sub = j - t * BPT;
      }
      if (sub == 0) {
        const int tile = ids[t];
        const int rest = div_by(tile, g.nw, g.mag_nw);
        const int tw = tile - rest * g.nw;
        const int tt = div_by(rest, g.nh, g.mag_nh);
        const int th = rest - tt * g.nh;
        tile_kbase = (tt * kTileT * g.H + th * kTileH) * g.W + tw * kTileW;
        tile_vrow = tile * kTileRows;
        if constexpr (PAD) tile_ext = tile_extent(tt, th, tw, g);
      }
      kbase = tile_kbase + sub * g.H * g.W;
      krs = g.W;
      vrow = tile_vrow + sub * kKeyBlock;
    } else {
      kbase = g.n_video + (j - n_vid) * kKeyBlock;
      vrow = g.n_vt + (j - n_vid) * kKeyBlock;
      krs = kTileW;
      if constexpr (PAD) tile_ext = kFullExtent;
    }
  };

  // Fetch K block j into LDS stage st. Row rr of the block is raster row
  // kbase + (rr/8)*krs + rr%8. Each DMA instruction covers RPI rows that
  // share rr/8, so its source is a wave-uniform row pointer plus a per-lane
  // offset (row within the group, chunk) that is the same for every block.
  auto issue_k = [&](int st, int kbase, int krs) {
    // PAD: per-lane offsets come from a fresh opaque copy of the lane id, so
    // they are rebuilt per block rather than hoisted (and spilled) as 64-bit
    // addresses
    int lane = opaque_lane<PAD>(this_lane);
    if constexpr (PAD) {
      if ((tile_ext >> 8) != (kFullExtent >> 8)) {
        // a tile with missing rows or columns: block row r is token 64 sub + r
        // of the tile in compact order, clamped to the last one that exists
        const int last = extent_tokens(tile_ext) - 1;
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
          const int q = wave * IPW + i;
          const int rin = (lane >> 2) % RPI;
          int dt, dh, dw;
          compact_token(min(cur_sub * kKeyBlock + q * RPI + rin, last), tile_ext, dt, dh, dw);
          const int row = tile_kbase + (dt * g.H + dh) * g.W + dw;
          const int chunk = 4 * (lane / (4 * RPI)) + ((lane & 3) ^ sw(q * RPI + rin));
          dma16(kr + size_t(row) * ROWB + chunk * 16, &lds[st][0][q * 1024]);
        }
        return;
      }
    }
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int q = wave * IPW + i;
      const size_t urow = size_t(kbase + ((q * RPI) >> 3) * krs + ((q * RPI) & 7));
      const int rin = (lane >> 2) % RPI;
      const int chunk = 4 * (lane / (4 * RPI)) + ((lane & 3) ^ sw(q * RPI + rin));
      const unsigned o = unsigned(rin * ROWB + chunk * 16);
      dma16(kr + urow * ROWB + o, &lds[st][0][q * 1024]);
    }
  };
  // Fetch the packed V^T block starting at tile-major row vrow (contiguous).
  auto issue_v = [&](int st, int vrow) {
    int lane = opaque_lane<PAD>(this_lane);
    const char* src = vtr + size_t(vrow) * ROWB;
    const unsigned o = unsigned(lane) * 16u;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int q = wave * IPW + i;
      dma16(src + q * 1024 + o, &lds[st][1][q * 1024]);
    }
  };

  // The rest runs with QT query column groups per wave: 3 (8 x 48 = 384 rows)
  // for a video tile, 2 (8 x 32 = 256 rows) for the text query slots; a
  // partial tile also uses 1 (16 rows per wave) or 3 with only waves 0-3
  // holding rows.
  auto run = [&](auto qt_c) {
    constexpr int QT = decltype(qt_c)::value;
    constexpr int RPW = QT * 16;  // query rows per wave
    // a wave whose rows all lie past a partial tile's tokens only loads and
    // synchronises (its SIMD then runs one wave of the unit instead of two)
    const bool active = !PAD || wave * RPW < q_rows;
    // Q^T fragments for this wave's RPW rows, read from the caller's raster q
    // (row r of the unit: see query_raster; rows past the unit are clamped to
    // a valid row and their results discarded).
    const float qs = a.q_scale;  // log2(e)/sqrt(D), applied to the fp32 scores
    bf16x8 qf[QT][KS];
  #pragma unroll
    for (int c = 0; c < QT; ++c) {
      int row = wave * RPW + c * 16 + (lane & 15);
      row = row < q_rows ? row : q_rows - 1;
      const int rr = query_raster(row);
      const bf16x8* src = reinterpret_cast<const bf16x8*>(qr + size_t(rr) * D + (lane >> 4) * 8);
  #pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[c][ks] = src[ks * 4];
    }

    f32x4 acc[QT][DT];
    float l_part[QT];  // this lane's share of the row sum of p
    float m_run[QT];   // reference max of the scaled scores (log2 units)
  #pragma unroll
    for (int c = 0; c < QT; ++c) {
  #pragma unroll
      for (int d = 0; d < DT; ++d) acc[c][d] = f32x4{0.f, 0.f, 0.f, 0.f};
      l_part[c] = 0.f;
      m_run[c] = 0.f;
    }
    bf16x2 ones2;
    ones2[0] = (__bf16)1.0f;
    ones2[1] = (__bf16)1.0f;

    // K fragment (row 16kt + lane%16, chunk 4ks + lane/16) of a block sits at
    // kofs + kt * 16 * ROWB + ks * 64 * RPI; V^T fragment (h, dt) at
    // (h * DT + dt) * 1024 + lane * 16.
    const int l15 = lane & 15;
    const int kofs = (l15 / RPI) * 1024 + (l15 % RPI) * 64 + (((lane >> 4) ^ sw(l15)) << 4);

    auto issue = [&](int j, int st) {
      int kbase, krs, vrow;
      block_rows(j, kbase, krs, vrow);
      issue_k(st, kbase, krs);
      issue_v(st, vrow);
    };

    issue(0, 0);
    if (!active) {
      // the same loads and barriers as the loop below; once every wave has
      // passed barrier j, no wave reads the other stage any more
      for (int j = 0; j < n_blk; ++j) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (j + 1 < n_blk) issue(j + 1, (j & 1) ^ 1);
      }
      return;
    }
    for (int j = 0; j < n_blk; ++j) {
      const int stage = j & 1;
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();

      // ---- raw scores S^T = K Q^T (fp32); p = 2^(c s - m) below
      const char* kb = lds[stage][0];
      f32x4 s[QT][4];
      {
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
        if (ragged && j == n_blk - 1) {
          int key0 = (j - n_vid) * kKeyBlock + 4 * (lane >> 4);
          asm volatile("" : "+v"(key0));  // build the 16 lane masks here, not before the loop
  #pragma unroll
          for (int kt = 0; kt < 4; ++kt)
  #pragma unroll
            for (int r = 0; r < 4; ++r)
              if (key0 + 16 * kt + r >= text_len)
  #pragma unroll
                for (int c = 0; c < QT; ++c) s[c][kt][r] = -INFINITY;
        }
        if constexpr (PAD) {
          // the last block of a tile whose token count is not a multiple of
          // 64: keys past the tile's tokens (the tile state still describes
          // block j; block j + 1 is decoded below)
          const int n_tok = extent_tokens(tile_ext);
          if (j < n_vid && (cur_sub + 1) * kKeyBlock > n_tok) {
            int key0 = cur_sub * kKeyBlock + 4 * (lane >> 4);
            asm volatile("" : "+v"(key0));
  #pragma unroll
            for (int kt = 0; kt < 4; ++kt)
  #pragma unroll
              for (int r = 0; r < 4; ++r)
                if (key0 + 16 * kt + r >= n_tok)
  #pragma unroll
                  for (int c = 0; c < QT; ++c) s[c][kt][r] = -INFINITY;
          }
        }
      }
      if (j + 1 < n_blk) issue(j + 1, stage ^ 1);
      // per-lane max of the scaled scores; the reference moves only past the
      // slack, and then only m, l and the accumulator change (the scores are
      // raw, so nothing is recomputed)
      float lm[QT];
      bool need = false;
  #pragma unroll
      for (int c = 0; c < QT; ++c) {
        float x = fmaxf(fmaxf(s[c][0][0], s[c][0][1]), s[c][0][2]);
        x = fmaxf(fmaxf(x, s[c][0][3]), s[c][1][0]);
        x = fmaxf(fmaxf(x, s[c][1][1]), s[c][1][2]);
        x = fmaxf(fmaxf(x, s[c][1][3]), s[c][2][0]);
        x = fmaxf(fmaxf(x, s[c][2][1]), s[c][2][2]);
        x = fmaxf(fmaxf(x, s[c][2][3]), s[c][3][0]);
        x = fmaxf(fmaxf(x, s[c][3][1]), s[c][3][2]);
        lm[c] = fmaxf(x, s[c][3][3]) * qs;
        need |= lm[c] - m_run[c] > kRescaleSlack;
      }
      const bool first = j == 0;
      if (first || __builtin_amdgcn_ballot_w64(need) != 0) {
  #pragma unroll
        for (int c = 0; c < QT; ++c) {
          // exact row max across the 4 lanes holding this query
          const float mx = swap32_max(swap16_max(lm[c]));
          if (first) {
            m_run[c] = mx;  // nothing accumulated yet
          } else if (mx > m_run[c]) {
            const float alpha = __builtin_amdgcn_exp2f(m_run[c] - mx);
            m_run[c] = mx;
            l_part[c] *= alpha;
  #pragma unroll
            for (int d = 0; d < DT; ++d) acc[c][d] *= alpha;
          }
        }
      }

      // ---- p = 2^(c s - m) rounded to bf16; O^T += V^T P^T; row sums += 1^T P^T
      const bf16x8* vl = reinterpret_cast<const bf16x8*>(lds[stage][1]);
  #pragma unroll
      for (int h = 0; h < 2; ++h) {
        bf16x8 pb[QT];
  #pragma unroll
        for (int c = 0; c < QT; ++c) {
          f32x8 p;
  #pragma unroll
          for (int r = 0; r < 4; ++r) {
            p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[c][2 * h][r], qs, -m_run[c]));
            p[4 + r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[c][2 * h + 1][r], qs, -m_run[c]));
          }
          pb[c] = __builtin_convertvector(p, bf16x8);
          // row sum of the rounded p, two at a time
  #pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bf16x2 pair = {pb[c][2 * i], pb[c][2 * i + 1]};
            l_part[c] = __builtin_amdgcn_fdot2_f32_bf16(pair, ones2, l_part[c], false);
          }
        }
  #pragma unroll
        for (int d = 0; d < DT; ++d) {
          const bf16x8 vf = vl[(h * DT + d) * 64 + lane];
  #pragma unroll
          for (int c = 0; c < QT; ++c)
            acc[c][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[c], acc[c][d], 0, 0, 0);
        }
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
      if (row < q_rows) {
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
    if (q_rows <= 16 * kWaves) {  // a small partial tile: 8 (or 4) waves x 16 rows
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

// Resident workgroups of the kernel on the current device (cached per device).
template <int D, bool PAD>
int persistent_grid() {
  static int cache[kMaxDevices] = {};
  return resident_workgroups(sta_attention_kernel<D, PAD>, kThreads, cache);
}

template <int D, bool PAD>
hipError_t launch(const Geom& g, const Windows& win, const FwdArgs& a, hipStream_t stream) {
  const int units = g.B * g.heads * g.n_q;
  const int resident = persistent_grid<D, PAD>();
  if (resident <= 0) return hipErrorInvalidDevice;
  const int grid = units < resident ? units : resident;
  sta_attention_kernel<D, PAD><<<grid, kThreads, 0, stream>>>(KernelArgs{g, a, win});
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const Geom& g, const Windows& win, const FwdArgs& a, hipStream_t stream) {
  if (g.full) return g.D == 128 ? launch<128, false>(g, win, a, stream) : launch<64, false>(g, win, a, stream);
  return g.D == 128 ? launch<128, true>(g, win, a, stream) : launch<64, true>(g, win, a, stream);
}

}  // namespace sta
