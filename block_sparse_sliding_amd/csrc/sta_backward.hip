// STA backward for gfx950: dq, dk, dv of the fused forward, bf16 MFMA with
// fp32 accumulation.
//
// What it computes: the gradients of softmax(q k^T / sqrt(D)) v under the STA
// mask (STA README, "Usage" and "Why is STA Fast?": whole key tiles of each
// query tile's window, then the valid text keys) for an upstream gradient
// dout. With c = 1/sqrt(D), P the forward's probabilities (recomputed from
// the saved lse) and delta_i = dout_i . out_i:
//   dP = dout v^T,   dS = P * (dP - delta),
//   dq = c dS k,     dk = c dS^T q,     dv = P^T dout.
// The page shows only the forward call; these follow from its definition.
//
// Three passes over the inputs, each a launch on the caller's stream:
//   prep   lse2 = lse * log2(e) and -delta, per row in tile-major order;
//   pack   K^T, Q^T and dout^T as MFMA A-operand fragments (the forward's V^T
//          packing, applied to these tensors);
//   dq     query-stationary: the forward's loop with S^T = K Q^T and
//          dP^T = V dout^T from LDS (K and V raw, same swizzled layout), then
//          dq^T += K^T dS^T with K^T fragments from LDS;
//   dk/dv  key-stationary: units of 256 keys (32 per wave) or 128 keys (16
//          per wave), their K and V rows held as MFMA B operands, streaming
//          every query block that sees the keys: S = Q K^T and dP = dout V^T
//          with Q and dout raw in LDS, then dv^T += dout^T P and
//          dk^T += Q^T dS with Q^T / dout^T fragments, each 64-row block in
//          two halves of 32 queries (so two key groups fit the registers and
//          every fragment read from LDS feeds two MFMAs).
// The packed fragments present their 64 rows in the order in which a
// 16x16x32 MFMA accumulator leaves its rows in the lanes, so P and dS go from
// the accumulator straight into the B operand, as in the forward's PV step.
//
// Key-side work: a key tile is seen by the query tiles whose clamped window
// holds it. Along one axis the window start clamp(c - w/2, 0, n - w) never
// decreases with c, so those query tiles form a box (an interval per axis),
// found per unit by a scan over the axis; text query rows see every video key
// and every valid text key. Text key slots at or after text_length are seen by
// no query and get zero gradients.
//
// Video sizes that are not tile multiples (the PAD instantiations): the last
// tile along an axis holds the remainder, and a partial tile's tile-major
// slot holds its existing tokens first, in compact order (frame, row,
// column), then padding. Stationary rows and keys are those tokens; streamed
// tiles contribute ceil(tokens / 64) blocks whose raw rows are fetched per
// lane through the compact map, clamped to the last token (every address
// stays inside the video). Packed padding rows are zeros and prep gives
// padding query rows lse2 = +inf and -delta = 0, so their P and dS are
// exactly 0 wherever they are streamed; padding key rows add nothing to dq
// (their packed K^T rows are zero and their dS finite, computed on a copy of
// a key of the same tile), and padding rows of dq, dk, dv are not written.
#include <type_traits>

#include "sta_device.h"
#include "sta_internal.h"

namespace sta {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kQueryBlock = 64;                     // query rows per streamed block (dk/dv)
constexpr int kKPrefetch = 4;                       // A fragments in flight (dq contractions)
constexpr int kKvPrefetch = 2;                      // A fragments in flight (dk/dv contractions)
constexpr float kLog2e = 1.44269504088896340736f;

static_assert(kKeyBlock == kQueryBlock, "one packed block size for keys and queries");
static_assert(kTileRows == 256 + 128 && kTextSlots == 256, "dk/dv unit shapes below");

struct KernelArgs {
  Geom g;
  Windows win;
  BwdArgs a;
};

__device__ inline const KernelArgs* kernel_args() {
  auto kp = (const __attribute__((address_space(4))) KernelArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(kp));
  return (const KernelArgs*)kp;
}

// Next entry of the unit order for a workgroup on XCD `xcd`, or -1 once every
// queue is empty. Entry e = 8k + y is item k of queue y; the heads in claim
// (one per 256-byte line) count the items taken. Same protocol as the
// forward's queues: each fetch-add hands out a distinct item.
__device__ inline int claim_entry(int32_t* claim, int total, int xcd) {
  for (int t = 0; t < kQueues; ++t) {
    const int y = (xcd + t) & (kQueues - 1);
    const int n_y = (total - y + kQueues - 1) / kQueues;
    if (n_y <= 0) continue;
    const int k = __hip_atomic_fetch_add(claim + y * kClaimStride, 1, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    if (k < n_y) return kQueues * k + y;
  }
  return -1;
}

// Unit of entry e when the first `heavy` units are dealt round-robin over the
// 8 queues and every queue then takes one contiguous run of the remaining
// units (queue y holds ceil((total - y) / 8) entries, as claim_entry
// assumes). Neighbouring units, which read mostly the same blocks, thus run
// at about the same time on one XCD and share its L2.
__device__ inline int entry_unit(int e, int total, int heavy) {
  if (e < heavy) return e;
  const int x = e & (kQueues - 1), k = e / kQueues;
  auto len = [&](int y) { return (total - y + kQueues - 1) / kQueues; };
  auto n_heavy = [&](int y) { return heavy > y ? (heavy - y + kQueues - 1) / kQueues : 0; };
  int base = 0;
  for (int y = 0; y < x; ++y) base += len(y) - n_heavy(y);
  return heavy + base + (k - n_heavy(x));
}

__device__ inline int xcd_id() {
  unsigned xcc;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  return int(xcc);
}

// The interval of query coordinates whose window (window_start) holds key
// coordinate kc.
__device__ inline void seeing_interval(int kc, int w, int n, int& lo, int& len) {
  int first = n, last = -1;
  for (int c = 0; c < n; ++c) {
    const int s = window_start(c, w, n);
    if (s <= kc && kc < s + w) {
      first = c < first ? c : first;
      last = c;
    }
  }
  lo = first;
  len = last - first + 1;
}

// ---------------------------------------------------------------- prep
// grid (S_t / 64, B*heads), 256 threads: 4 threads per tile-major row.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(Geom g, const __bf16* __restrict__ out,
                                                      const __bf16* __restrict__ dout,
                                                      const float* __restrict__ lse,
                                                      float* __restrict__ lse2,
                                                      float* __restrict__ delta) {
  constexpr int PER = D / 4;  // elements per thread
  const size_t bh = blockIdx.y;
  const int r = blockIdx.x * 64 + (threadIdx.x >> 2);
  const int part = threadIdx.x & 3;
  const int rr = tiled_to_raster(r, g);
  if (rr < 0) {  // padding row of a partial tile: P = 2^(s c' - inf) = 0 wherever it is streamed
    if (part == 0) {
      delta[bh * g.S_t + r] = -0.f;
      lse2[bh * g.S_t + r] = INFINITY;
    }
    return;
  }
  const size_t base = (bh * g.S + rr) * D + part * PER;
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < PER; i += 8) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(out + base + i);
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(dout + base + i);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(float(a[e]), float(b[e]), acc);
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  if (part == 0) {
    delta[bh * g.S_t + r] = -acc;  // stored negated: it starts the dP accumulators
    lse2[bh * g.S_t + r] = lse[bh * g.S + rr] * kLog2e;
  }
}

// ---------------------------------------------------------------- dq
// Query units per (b, head): two per video tile (rows 0..255 with 8 waves x
// 32 rows, rows 256..383 with 8 waves x 16 rows; with PAD, a unit of at most
// 128 existing rows also runs 8 x 16), plus the 256 text query slots (8 waves
// x 32 rows). Unit order: text units first, then the tiles.
__device__ inline int dq_units_per_head(const Geom& g) { return 2 * g.n_tiles + (g.has_text ? 1 : 0); }

template <int D, bool PAD>
__global__ __launch_bounds__(kThreads, 1) void bwd_dq_kernel(KernelArgs) {
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  constexpr int ROWB = D * 2;
  constexpr int BLK = kKeyBlock * ROWB;
  constexpr int RPI = 1024 / ROWB;
  constexpr int IPW = BLK / 1024 / kWaves;
  constexpr int BPT = kTileRows / kKeyBlock;
  static_assert(IPW >= 1 && BLK % (1024 * kWaves) == 0, "block must split over the waves");
  // [stage][K raw | V raw | K^T packed]
  __shared__ __attribute__((aligned(1024))) char lds[2][3][BLK];
  __shared__ int claimed;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  for (;;) {
    // every wave has read the previous claim and finished the previous
    // unit's LDS reads (a unit may stream no block, so its body need not
    // contain a barrier)
    __syncthreads();
    if (threadIdx.x == 0) {
      const KernelArgs* ka = kernel_args();
      const int n_qu = dq_units_per_head(ka->g);
      claimed = claim_entry(ka->a.claim_q, ka->g.B * ka->g.heads * n_qu, xcd_id());
    }
    __syncthreads();
    const int entry = __builtin_amdgcn_readfirstlane(claimed);
    if (entry < 0) break;
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    const int this_lane = lane;
    const KernelArgs* ka = kernel_args();
    const Geom g = ka->g;
    const BwdArgs a = ka->a;

    // entry -> unit: the B*heads text units first, then (bh, tile, part)
    const int n_text_units = g.has_text ? g.B * g.heads : 0;
    const int unit = entry_unit(entry, g.B * g.heads * dq_units_per_head(g), n_text_units);
    int bh, u;  // u: list index into the forward schedule (tile, or n_tiles for text)
    int q_row0, q_rows;
    if (unit < n_text_units) {
      bh = unit;
      u = g.n_tiles;
      q_row0 = g.n_vt;
      q_rows = kTextSlots;
    } else {
      const int e = unit - n_text_units;
      bh = e / (2 * g.n_tiles);
      const int r = e - bh * 2 * g.n_tiles;
      u = r >> 1;
      q_row0 = u * kTileRows + (r & 1) * 256;
      q_rows = (r & 1) ? kTileRows - 256 : 256;
    }
    // PAD: the rows of a video unit are its tile's existing tokens in compact
    // order (frame, row, column), part 1 starting at token 256; n_valid of
    // them exist (possibly none: the unit then streams nothing)
    int q_ext = kFullExtent, q_base = 0, n_valid = q_rows;
    if constexpr (PAD) {
      if (unit >= n_text_units) {
        const int rest = div_by(u, g.nw, g.mag_nw);
        const int tw = u - rest * g.nw;
        const int tt = div_by(rest, g.nh, g.mag_nh);
        const int th = rest - tt * g.nh;
        q_ext = tile_extent(tt, th, tw, g);
        q_base = (tt * kTileT * g.H + th * kTileH) * g.W + tw * kTileW;
        n_valid = min(extent_tokens(q_ext) - (q_row0 - u * kTileRows), q_rows);
      }
    }
    // unit row `row` -> raster row and tile-major row (the index of lse2 and
    // delta); rows at or past n_valid map to the last existing one
    auto query_rows = [&](int row, int& raster, int& tiled) {
      if constexpr (PAD) {
        if (unit >= n_text_units) {
          const int first = q_row0 - u * kTileRows;  // 0 or 256
          int dt, dh, dw;
          compact_token(first + (row < n_valid ? row : n_valid - 1), q_ext, dt, dh, dw);
          raster = q_base + (dt * g.H + dh) * g.W + dw;
          tiled = u * kTileRows + first + (row < n_valid ? row : n_valid - 1);  // compact layout
          return;
        }
      }
      raster = PAD ? tiled_to_raster(q_row0 + row, g) : tiled_to_raster_full(q_row0 + row, g);
      tiled = q_row0 + row;
    };
    const int hd = bh % g.heads;
    const size_t slab = size_t(bh) * g.S * D;
    const __bf16* __restrict__ qr = reinterpret_cast<const __bf16*>(a.q) + slab;
    const __bf16* __restrict__ dor = reinterpret_cast<const __bf16*>(a.dout) + slab;
    const char* __restrict__ kr = reinterpret_cast<const char*>(a.k) + slab * 2;
    const char* __restrict__ vr = reinterpret_cast<const char*>(a.v) + slab * 2;
    const size_t slab_t = size_t(bh) * g.S_t * D;  // packed tile-major tensors
    const char* __restrict__ ktr = reinterpret_cast<const char*>(a.kt) + slab_t * 2;
    const float* __restrict__ lse2 = a.lse2 + size_t(bh) * g.S_t;
    const float* __restrict__ dlt = a.delta + size_t(bh) * g.S_t;

    const int l0 = a.offsets[hd * g.n_q + u];
    const int l1 = a.offsets[hd * g.n_q + u + 1];
    // video key blocks: six per listed tile; with PAD, ceil(tokens / 64) per
    // tile (as in the forward)
    int n_vid = (l1 - l0) * BPT;
    if constexpr (PAD) {
      if (unit < n_text_units) {
        n_vid = box_blocks(0, g.nt, 0, g.nh, 0, g.nw, g);
      } else {  // the list is the query tile's window, a box
        const uint32_t p = ka->win.w[hd];
        const int rest = div_by(u, g.nw, g.mag_nw);
        const int tt = div_by(rest, g.nh, g.mag_nh);
        const int th = rest - tt * g.nh, tw = u - rest * g.nw;
        n_vid = box_blocks(window_start(tt, win_t(p), g.nt), win_t(p), window_start(th, win_h(p), g.nh),
                           win_h(p), window_start(tw, win_w(p), g.nw), win_w(p), g);
      }
    }
    const int text_len = g.has_text ? g.text_length : 0;
    const int n_blk = n_valid > 0 ? n_vid + (text_len + kKeyBlock - 1) / kKeyBlock : 0;
    const bool ragged = (text_len % kKeyBlock) != 0;
    auto sw = [](int row) { return (row >> 2) & 2; };
    const __attribute__((address_space(4))) int32_t* ids =
        (const __attribute__((address_space(4))) int32_t*)(a.ids + l0);

    // with PAD, tile_ext: packed extent of the current key tile (the frames,
    // rows and columns that exist); its blocks are 64 compact tokens each
    int tile_kbase = 0, tile_vrow = 0;
    int tile_ext = kFullExtent;  // PAD: packed extent of the current tile
    int cur_t = 0, cur_sub = -1;  // PAD: the forward's walk over existing frames
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
    // raw rows kbase + (rr/8)*krs + rr%8 of tensor `src` into LDS region `dst`
    // (the forward's swizzled K layout)
    auto issue_raw = [&](const char* src, char* dst, int kbase, int krs) {
      // PAD: per-lane offsets from a fresh opaque lane id, rebuilt per block
      // rather than hoisted (and spilled) as 64-bit addresses
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
            dma16(src + size_t(row) * ROWB + chunk * 16, dst + q * 1024);
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
        dma16(src + urow * ROWB + o, dst + q * 1024);
      }
    };
    auto issue_packed = [&](const char* src, char* dst, int vrow) {
      int lane = opaque_lane<PAD>(this_lane);
      const char* p = src + size_t(vrow) * ROWB;
      const unsigned o = unsigned(lane) * 16u;
#pragma unroll
      for (int i = 0; i < IPW; ++i) {
        const int q = wave * IPW + i;
        dma16(p + q * 1024 + o, dst + q * 1024);
      }
    };

    auto run = [&](auto qt_c) {
      constexpr int QT = decltype(qt_c)::value;
      constexpr int RPW = QT * 16;
      const float qs = a.q_scale;
      bf16x8 qf[QT][KS], dof[QT][KS];
      float l2[QT], dl[QT];  // lse2 and -delta of this lane's query rows
#pragma unroll
      for (int c = 0; c < QT; ++c) {
        const int row = wave * RPW + c * 16 + (lane & 15);  // < q_rows for every unit shape
        int rr, rt;
        query_rows(row, rr, rt);
        const bf16x8* qs8 = reinterpret_cast<const bf16x8*>(qr + size_t(rr) * D + (lane >> 4) * 8);
        const bf16x8* ds8 = reinterpret_cast<const bf16x8*>(dor + size_t(rr) * D + (lane >> 4) * 8);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          qf[c][ks] = qs8[ks * 4];
          dof[c][ks] = ds8[ks * 4];
        }
        l2[c] = lse2[rt];
        dl[c] = dlt[rt];
      }
      f32x4 acc[QT][DT];
#pragma unroll
      for (int c = 0; c < QT; ++c)
#pragma unroll
        for (int d = 0; d < DT; ++d) acc[c][d] = f32x4{0.f, 0.f, 0.f, 0.f};

      const int l15 = lane & 15;
      const int kofs = (l15 / RPI) * 1024 + (l15 % RPI) * 64 + (((lane >> 4) ^ sw(l15)) << 4);
      auto issue = [&](int j, int st) {
        int kbase, krs, vrow;
        block_rows(j, kbase, krs, vrow);
        issue_raw(kr, lds[st][0], kbase, krs);
        issue_raw(vr, lds[st][1], kbase, krs);
        issue_packed(ktr, lds[st][2], vrow);
      };

      // A x B^T-style score product over one raw block in LDS: out[c][kt] =
      // init[c] + sum over d of blk[16 kt + l%16][d] * frag[c][d]
      auto scores = [&](const char* blk, const bf16x8 (&frag)[QT][KS], const f32x4 (&init)[QT],
                        f32x4 (&out)[QT][4]) {
        constexpr int NF = 4 * KS;
        bf16x8 kf[NF];
        auto kload = [&](int f) {
          kf[f] = *reinterpret_cast<const bf16x8*>(blk + kofs + (f & 3) * 16 * ROWB + (f >> 2) * 64 * RPI);
        };
#pragma unroll
        for (int f = 0; f < kKPrefetch; ++f) kload(f);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const int ks = f >> 2, kt = f & 3;
#pragma unroll
          for (int c = 0; c < QT; ++c)
            out[c][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[f], frag[c][ks],
                                                                  ks == 0 ? init[c] : out[c][kt], 0, 0, 0);
          if (f + kKPrefetch < NF) kload(f + kKPrefetch);
          __builtin_amdgcn_sched_barrier(0);
        }
      };

      if (!PAD || n_blk > 0) issue(0, 0);
      // a wave whose rows all lie past a partial tile's tokens only loads
      if (PAD && wave * RPW >= n_valid) {
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
        f32x4 s[QT][4], dp[QT][4];
        f32x4 zero[QT], nd[QT];  // dP^T starts at -delta of its query (column)
#pragma unroll
        for (int c = 0; c < QT; ++c) {
          float x = dl[c];
          asm volatile("" : "+v"(x));  // built here, per block, not kept live across the loop
          zero[c] = f32x4{0.f, 0.f, 0.f, 0.f};
          nd[c] = f32x4{x, x, x, x};
        }
        scores(lds[stage][0], qf, zero, s);
        scores(lds[stage][1], dof, nd, dp);
        if (j + 1 < n_blk) issue(j + 1, stage ^ 1);
        // P = 2^(c' s - lse2), dS = P (dP - delta) with dP - delta from the MFMAs
#pragma unroll
        for (int c = 0; c < QT; ++c)
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[c][kt][r], qs, -l2[c]));
              dp[c][kt][r] = p * dp[c][kt][r];
            }
        // keys at or after the text length (last text block only): dS = 0 by
        // select, so whatever k and v hold there cannot reach dq
        if (ragged && j == n_blk - 1) {
          int key0 = (j - n_vid) * kKeyBlock + 4 * (lane >> 4);
          asm volatile("" : "+v"(key0));
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (key0 + 16 * kt + r >= text_len)
#pragma unroll
                for (int c = 0; c < QT; ++c) dp[c][kt][r] = 0.f;
        }
        // dq^T += K^T dS^T
        const bf16x8* ktl = reinterpret_cast<const bf16x8*>(lds[stage][2]);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          bf16x8 db[QT];
#pragma unroll
          for (int c = 0; c < QT; ++c) {
            f32x8 x;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              x[r] = dp[c][2 * h][r];
              x[4 + r] = dp[c][2 * h + 1][r];
            }
            db[c] = __builtin_convertvector(x, bf16x8);
          }
#pragma unroll
          for (int d = 0; d < DT; ++d) {
            const bf16x8 kf = ktl[(h * DT + d) * 64 + lane];
#pragma unroll
            for (int c = 0; c < QT; ++c)
              acc[c][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, db[c], acc[c][d], 0, 0, 0);
          }
        }
      }
      // dq = c * acc, rows to raster positions
      __bf16* __restrict__ dqr = reinterpret_cast<__bf16*>(a.dq) + slab;
#pragma unroll
      for (int c = 0; c < QT; ++c) {
        const int row = wave * RPW + c * 16 + (lane & 15);
        if (PAD && row >= n_valid) continue;  // no such token
        int rr, rt;
        query_rows(row, rr, rt);
        __bf16* dst = dqr + size_t(rr) * D + (lane >> 4) * 4;
#pragma unroll
        for (int d = 0; d < DT; ++d) {
          const f32x4 o = acc[c][d] * a.scale;
          *reinterpret_cast<bf16x4*>(dst + d * 16) = __builtin_convertvector(o, bf16x4);
        }
      }
    };
    if (q_rows == 256 && !(PAD && n_valid <= 128))  // PAD: a small partial tile runs 8 x 16 rows
      run(std::integral_constant<int, 2>{});
    else
      run(std::integral_constant<int, 1>{});
  }
}

// ---------------------------------------------------------------- dk, dv
// Key units per (b, head): per video tile keys 0..255 (8 waves x 32 keys) and
// keys 256..383 (8 waves x 16 keys; with PAD, a unit of at most 128 existing
// keys also runs 8 x 16), plus the 256 text slots (8 waves x 32).
// Unit order: the text units first (each streams every query row), then
// (bh, tile, part).
__device__ inline int kv_units_per_head(const Geom& g) { return 2 * g.n_tiles + (g.has_text ? 1 : 0); }

template <int D, bool PAD>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkv_kernel(KernelArgs) {
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  constexpr int ROWB = D * 2;
  constexpr int BLK = kQueryBlock * ROWB;
  constexpr int RPI = 1024 / ROWB;
  constexpr int IPW = BLK / 1024 / kWaves;
  constexpr int BPT = kTileRows / kQueryBlock;
  static_assert(IPW >= 1 && BLK % (1024 * kWaves) == 0, "block must split over the waves");
  // [stage][Q raw | dout raw | Q^T packed | dout^T packed], then lse2 and delta
  __shared__ __attribute__((aligned(1024))) char lds[2][4][BLK];
  __shared__ __attribute__((aligned(16))) float rowv[2][2][kQueryBlock];
  __shared__ int claimed;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  for (;;) {
    __syncthreads();  // as in the dq kernel
    if (threadIdx.x == 0) {
      const KernelArgs* ka = kernel_args();
      const int n_ku = kv_units_per_head(ka->g);
      claimed = claim_entry(ka->a.claim_kv, ka->g.B * ka->g.heads * n_ku, xcd_id());
    }
    __syncthreads();
    const int entry = __builtin_amdgcn_readfirstlane(claimed);
    if (entry < 0) break;
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    const int this_lane = lane;
    const KernelArgs* ka = kernel_args();
    const Geom g = ka->g;
    const BwdArgs a = ka->a;

    const int n_text_units = g.has_text ? g.B * g.heads : 0;
    const int unit = entry_unit(entry, g.B * g.heads * kv_units_per_head(g), n_text_units);
    int bh, key_row0, unit_keys;
    bool text_unit;
    int box_t = 0, box_h = 0, box_w = 0, lo_t = 0, lo_h = 0, lo_w = 0;
    // PAD: the keys of a video unit are its tile's existing tokens in compact
    // order (frame, row, column), part 1 starting at token 256; n_keys of them
    // exist (none or fewer: the unit then streams nothing or writes fewer rows)
    int k_ext = kFullExtent, k_base = 0, k_first = 0, n_keys = 0;
    if (unit < n_text_units) {
      bh = unit;
      key_row0 = g.n_vt;
      unit_keys = kTextSlots;
      text_unit = true;
    } else {
      const int e = unit - n_text_units;
      bh = e / (2 * g.n_tiles);
      const int r = e - bh * 2 * g.n_tiles;
      const int tile = r >> 1;
      key_row0 = tile * kTileRows + (r & 1) * 256;
      unit_keys = (r & 1) ? kTileRows - 256 : 256;
      text_unit = false;
      const uint32_t p = ka->win.w[bh % g.heads];
      const int rest = div_by(tile, g.nw, g.mag_nw);
      const int tw = tile - rest * g.nw;
      const int tt = div_by(rest, g.nh, g.mag_nh);
      const int th = rest - tt * g.nh;
      seeing_interval(tt, win_t(p), g.nt, lo_t, box_t);
      seeing_interval(th, win_h(p), g.nh, lo_h, box_h);
      seeing_interval(tw, win_w(p), g.nw, lo_w, box_w);
      if constexpr (PAD) {
        k_ext = tile_extent(tt, th, tw, g);
        k_base = (tt * kTileT * g.H + th * kTileH) * g.W + tw * kTileW;
        k_first = (r & 1) * 256;
        n_keys = min(extent_tokens(k_ext) - k_first, unit_keys);
      }
    }
    const size_t slab = size_t(bh) * g.S * D;
    const size_t slab_t = size_t(bh) * g.S_t * D;  // packed tile-major tensors
    const int text_len = g.has_text ? g.text_length : 0;
    // text key slots at or after text_len are seen by nobody
    const int valid_keys = text_unit ? min(max(g.n_vt + text_len - key_row0, 0), unit_keys)
                                     : (PAD ? max(n_keys, 0) : unit_keys);
    // streamed video query blocks: six per query tile of the box (or of the
    // video, for a text unit); with PAD, ceil(tokens / 64) per tile
    int n_vblk = text_unit ? g.n_tiles * BPT : box_t * box_h * box_w * BPT;
    if constexpr (PAD) {
      n_vblk = text_unit ? box_blocks(0, g.nt, 0, g.nh, 0, g.nw, g)
                         : box_blocks(lo_t, box_t, lo_h, box_h, lo_w, box_w, g);
    }
    const int n_blk = valid_keys == 0 ? 0 : n_vblk + (g.has_text ? kTextSlots / kQueryBlock : 0);

    const char* __restrict__ qr = reinterpret_cast<const char*>(a.q) + slab * 2;
    const char* __restrict__ dor = reinterpret_cast<const char*>(a.dout) + slab * 2;
    const char* __restrict__ qtr = reinterpret_cast<const char*>(a.qt) + slab_t * 2;
    const char* __restrict__ dotr = reinterpret_cast<const char*>(a.dot) + slab_t * 2;
    const char* __restrict__ lse2 = reinterpret_cast<const char*>(a.lse2 + size_t(bh) * g.S_t);
    const char* __restrict__ dlt = reinterpret_cast<const char*>(a.delta + size_t(bh) * g.S_t);
    auto sw = [](int row) { return (row >> 2) & 2; };

    // query block j: raster origin of its rows and its first tile-major row;
    // with PAD, tile_ext describes the current query tile as in the dq kernel
    int tile_qbase = 0, tile_vrow = 0;
    int tile_ext = kFullExtent;  // PAD: packed extent of the current tile
    int cur_t = 0, cur_sub = -1;  // PAD: the walk over existing frames of the dq kernel
    auto block_rows = [&](int j, int& qbase, int& qrs, int& vrow) {
      if (j < n_vblk) {
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
          int tt, th, tw;
          if (text_unit) {
            const int rest = div_by(t, g.nw, g.mag_nw);
            tw = t - rest * g.nw;
            tt = div_by(rest, g.nh, g.mag_nh);
            th = rest - tt * g.nh;
          } else {
            const int rest = t / box_w;
            tw = lo_w + (t - rest * box_w);
            tt = lo_t + rest / box_h;
            th = lo_h + (rest - (rest / box_h) * box_h);
          }
          tile_qbase = (tt * kTileT * g.H + th * kTileH) * g.W + tw * kTileW;
          tile_vrow = ((tt * g.nh + th) * g.nw + tw) * kTileRows;
          if constexpr (PAD) tile_ext = tile_extent(tt, th, tw, g);
        }
        qbase = tile_qbase + sub * g.H * g.W;
        qrs = g.W;
        vrow = tile_vrow + sub * kQueryBlock;
      } else {
        qbase = g.n_video + (j - n_vblk) * kQueryBlock;
        vrow = g.n_vt + (j - n_vblk) * kQueryBlock;
        qrs = kTileW;
        if constexpr (PAD) tile_ext = kFullExtent;
      }
    };
    auto issue_raw = [&](const char* src, char* dst, int qbase, int qrs) {
      int lane = opaque_lane<PAD>(this_lane);  // as in the dq kernel
      if constexpr (PAD) {
        if ((tile_ext >> 8) != (kFullExtent >> 8)) {  // compact order, as in the dq kernel
          const int last = extent_tokens(tile_ext) - 1;
#pragma unroll
          for (int i = 0; i < IPW; ++i) {
            const int q = wave * IPW + i;
            const int rin = (lane >> 2) % RPI;
            int dt, dh, dw;
            compact_token(min(cur_sub * kQueryBlock + q * RPI + rin, last), tile_ext, dt, dh, dw);
            const int row = tile_qbase + (dt * g.H + dh) * g.W + dw;
            const int chunk = 4 * (lane / (4 * RPI)) + ((lane & 3) ^ sw(q * RPI + rin));
            dma16(src + size_t(row) * ROWB + chunk * 16, dst + q * 1024);
          }
          return;
        }
      }
#pragma unroll
      for (int i = 0; i < IPW; ++i) {
        const int q = wave * IPW + i;
        const size_t urow = size_t(qbase + ((q * RPI) >> 3) * qrs + ((q * RPI) & 7));
        const int rin = (lane >> 2) % RPI;
        const int chunk = 4 * (lane / (4 * RPI)) + ((lane & 3) ^ sw(q * RPI + rin));
        unsigned o = unsigned(rin * ROWB + chunk * 16);
        asm volatile("" : "+v"(o));  // keep base + offset per block (no hoisted 64-bit address)
        dma16(src + urow * ROWB + o, dst + q * 1024);
      }
    };
    auto issue_packed = [&](const char* src, char* dst, int vrow) {
      const char* p = src + size_t(vrow) * ROWB;
      unsigned o = unsigned(lane) * 16u;
      asm volatile("" : "+v"(o));
#pragma unroll
      for (int i = 0; i < IPW; ++i) {
        const int q = wave * IPW + i;
        dma16(p + q * 1024 + o, dst + q * 1024);
      }
    };
    auto issue = [&](int j, int st) {
      int qbase, qrs, vrow;
      block_rows(j, qbase, qrs, vrow);
      issue_raw(qr, lds[st][0], qbase, qrs);
      issue_raw(dor, lds[st][1], qbase, qrs);
      issue_packed(qtr, lds[st][2], vrow);
      issue_packed(dotr, lds[st][3], vrow);
      unsigned o4 = unsigned(lane) * 4u;
      asm volatile("" : "+v"(o4));
      if (wave == 0) dma4(lse2 + size_t(vrow) * 4 + o4, reinterpret_cast<char*>(rowv[st][0]));
      if (wave == 1) dma4(dlt + size_t(vrow) * 4 + o4, reinterpret_cast<char*>(rowv[st][1]));
    };

    const float qs = a.q_scale;
    const int l15 = lane & 15;
    const int qofs = (l15 / RPI) * 1024 + (l15 % RPI) * 64 + (((lane >> 4) ^ sw(l15)) << 4);

    auto run = [&](auto kt_c) {
      constexpr int KT = decltype(kt_c)::value;  // 16-key groups per wave
      // this wave's keys: K and V rows as B operands (lane: key l%16, d chunk l/16)
      int kras[KT];
      bool key_ok[KT];
      bf16x8 kf[KT][KS], vf[KT][KS];
#pragma unroll
      for (int kg = 0; kg < KT; ++kg) {
        const int local = wave * 16 * KT + 16 * kg + (lane & 15);
        const int key = key_row0 + local;
        key_ok[kg] = !text_unit || key < g.n_vt + text_len;
        kras[kg] = PAD ? tiled_to_raster(key, g) : tiled_to_raster_full(key, g);
        int ksrc = kras[kg];
        if constexpr (PAD) {
          if (!text_unit) {  // compact order; a key past n_keys computes on the last one, never written
            int dt, dh, dw;
            compact_token(k_first + (local < n_keys ? local : n_keys - 1), k_ext, dt, dh, dw);
            ksrc = k_base + (dt * g.H + dh) * g.W + dw;
            kras[kg] = local < n_keys ? ksrc : -1;
          }
        }
        const bf16x8* k8 = reinterpret_cast<const bf16x8*>(reinterpret_cast<const __bf16*>(a.k) + slab +
                                                           size_t(ksrc) * D + (lane >> 4) * 8);
        const bf16x8* v8 = reinterpret_cast<const bf16x8*>(reinterpret_cast<const __bf16*>(a.v) + slab +
                                                           size_t(ksrc) * D + (lane >> 4) * 8);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          kf[kg][ks] = k8[ks * 4];
          vf[kg][ks] = v8[ks * 4];
        }
      }
      f32x4 dk[KT][DT], dv[KT][DT];
#pragma unroll
      for (int kg = 0; kg < KT; ++kg)
#pragma unroll
        for (int d = 0; d < DT; ++d) {
          dk[kg][d] = f32x4{0.f, 0.f, 0.f, 0.f};
          dv[kg][d] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

      // out[kg][i] = init[i] + sum over d of blk[16 (2 hq + i) + l%16][d] * frag[kg][d]
      auto scores = [&](const char* blk, int hq, const bf16x8 (&frag)[KT][KS], const f32x4 (&init)[2],
                        f32x4 (&out)[KT][2]) {
        constexpr int NF = 2 * KS;
        bf16x8 af[NF];
        auto aload = [&](int f) {
          af[f] = *reinterpret_cast<const bf16x8*>(blk + qofs + (2 * hq + (f & 1)) * 16 * ROWB + (f >> 1) * 64 * RPI);
        };
#pragma unroll
        for (int f = 0; f < kKvPrefetch; ++f) aload(f);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const int ks = f >> 1, i = f & 1;
#pragma unroll
          for (int kg = 0; kg < KT; ++kg)
            out[kg][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[f], frag[kg][ks],
                                                                 ks == 0 ? init[i] : out[kg][i], 0, 0, 0);
          if (f + kKvPrefetch < NF) aload(f + kKvPrefetch);
          __builtin_amdgcn_sched_barrier(0);
        }
      };

      if (n_blk > 0) issue(0, 0);
      // a wave whose keys all lie past a partial tile's tokens only loads
      if (PAD && !text_unit && wave * 16 * KT >= n_keys) {
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
        const f32x4* l2v = reinterpret_cast<const f32x4*>(rowv[stage][0]);
        const f32x4* dlv = reinterpret_cast<const f32x4*>(rowv[stage][1]);
        const bf16x8* qtl = reinterpret_cast<const bf16x8*>(lds[stage][2]);
        const bf16x8* dotl = reinterpret_cast<const bf16x8*>(lds[stage][3]);
#pragma unroll
        for (int hq = 0; hq < 2; ++hq) {
          f32x4 s[KT][2], dp[KT][2];
          // rows of the accumulators: query 16 (2 hq + i) + 4 (l/16) + r; dP
          // starts at -delta of those rows
          const f32x4 zero[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
          const f32x4 nd[2] = {dlv[(2 * hq) * 4 + (lane >> 4)], dlv[(2 * hq + 1) * 4 + (lane >> 4)]};
          scores(lds[stage][0], hq, kf, zero, s);
          scores(lds[stage][1], hq, vf, nd, dp);
          if (hq == 0 && j + 1 < n_blk) issue(j + 1, stage ^ 1);
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const f32x4 l2 = l2v[(2 * hq + i) * 4 + (lane >> 4)];
#pragma unroll
            for (int kg = 0; kg < KT; ++kg)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kg][i][r], qs, -l2[r]));
                dp[kg][i][r] = p * dp[kg][i][r];
                s[kg][i][r] = p;
              }
          }
          if (text_unit) {
#pragma unroll
            for (int kg = 0; kg < KT; ++kg)
              if (!key_ok[kg])
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                  for (int r = 0; r < 4; ++r) {
                    s[kg][i][r] = 0.f;
                    dp[kg][i][r] = 0.f;
                  }
          }
          bf16x8 pb[KT], db[KT];
#pragma unroll
          for (int kg = 0; kg < KT; ++kg) {
            f32x8 x, y;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              x[r] = s[kg][0][r];
              x[4 + r] = s[kg][1][r];
              y[r] = dp[kg][0][r];
              y[4 + r] = dp[kg][1][r];
            }
            pb[kg] = __builtin_convertvector(x, bf16x8);
            db[kg] = __builtin_convertvector(y, bf16x8);
          }
          // dv^T += dout^T P, dk^T += Q^T dS over this half's 32 queries
#pragma unroll
          for (int d = 0; d < DT; ++d) {
            const bf16x8 fo = dotl[(hq * DT + d) * 64 + lane];
            const bf16x8 fq = qtl[(hq * DT + d) * 64 + lane];
#pragma unroll
            for (int kg = 0; kg < KT; ++kg) {
              dv[kg][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fo, pb[kg], dv[kg][d], 0, 0, 0);
              dk[kg][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fq, db[kg], dk[kg][d], 0, 0, 0);
            }
          }
        }
      }
      // dk = c * acc, dv = acc; C row = d (4 (l/16) + r of each 16-group), column = key
#pragma unroll
      for (int kg = 0; kg < KT; ++kg) {
        if (PAD && kras[kg] < 0) continue;
        __bf16* dkr = reinterpret_cast<__bf16*>(a.dk) + slab + size_t(kras[kg]) * D + (lane >> 4) * 4;
        __bf16* dvr = reinterpret_cast<__bf16*>(a.dv) + slab + size_t(kras[kg]) * D + (lane >> 4) * 4;
#pragma unroll
        for (int d = 0; d < DT; ++d) {
          *reinterpret_cast<bf16x4*>(dkr + d * 16) = __builtin_convertvector(dk[kg][d] * a.scale, bf16x4);
          *reinterpret_cast<bf16x4*>(dvr + d * 16) = __builtin_convertvector(dv[kg][d], bf16x4);
        }
      }
    };
    if (unit_keys == 256 && !(PAD && !text_unit && n_keys <= 128))  // PAD: a small partial tile runs 8 x 16 keys
      run(std::integral_constant<int, 2>{});
    else
      run(std::integral_constant<int, 1>{});
  }
}

template <int D, bool PAD>
hipError_t launch_dq(const Geom& g, const Windows& win, const BwdArgs& a, hipStream_t stream) {
  static int cache[kMaxDevices] = {};
  const int units = g.B * g.heads * (2 * g.n_tiles + (g.has_text ? 1 : 0));
  const int resident = resident_workgroups(bwd_dq_kernel<D, PAD>, kThreads, cache);
  if (resident <= 0) return hipErrorInvalidDevice;
  const int grid = units < resident ? units : resident;
  bwd_dq_kernel<D, PAD><<<grid, kThreads, 0, stream>>>(KernelArgs{g, win, a});
  return hipGetLastError();
}
template <int D, bool PAD>
hipError_t launch_dkv(const Geom& g, const Windows& win, const BwdArgs& a, hipStream_t stream) {
  static int cache[kMaxDevices] = {};
  const int units = g.B * g.heads * (2 * g.n_tiles + (g.has_text ? 1 : 0));
  const int resident = resident_workgroups(bwd_dkv_kernel<D, PAD>, kThreads, cache);
  if (resident <= 0) return hipErrorInvalidDevice;
  const int grid = units < resident ? units : resident;
  bwd_dkv_kernel<D, PAD><<<grid, kThreads, 0, stream>>>(KernelArgs{g, win, a});
  return hipGetLastError();
}

__global__ void zero_claims_kernel(int32_t* a, int32_t* b) {
  a[threadIdx.x] = 0;
  b[threadIdx.x] = 0;
}

}  // namespace

hipError_t launch_bwd_prep(const Geom& g, const void* out, const void* dout, const float* lse,
                           float* lse2, float* delta, int32_t* claim_q, int32_t* claim_kv,
                           hipStream_t stream) {
  dim3 grid(g.S_t / 64, g.B * g.heads);
  if (g.D == 128)
    bwd_prep_kernel<128><<<grid, 256, 0, stream>>>(g, (const __bf16*)out, (const __bf16*)dout, lse, lse2, delta);
  else
    bwd_prep_kernel<64><<<grid, 256, 0, stream>>>(g, (const __bf16*)out, (const __bf16*)dout, lse, lse2, delta);
  zero_claims_kernel<<<1, kClaimInts, 0, stream>>>(claim_q, claim_kv);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const Geom& g, const Windows& win, const BwdArgs& a, hipStream_t stream) {
  if (g.full) return g.D == 128 ? launch_dq<128, false>(g, win, a, stream) : launch_dq<64, false>(g, win, a, stream);
  return g.D == 128 ? launch_dq<128, true>(g, win, a, stream) : launch_dq<64, true>(g, win, a, stream);
}

hipError_t launch_bwd_dkv(const Geom& g, const Windows& win, const BwdArgs& a, hipStream_t stream) {
  if (g.full) return g.D == 128 ? launch_dkv<128, false>(g, win, a, stream) : launch_dkv<64, false>(g, win, a, stream);
  return g.D == 128 ? launch_dkv<128, true>(g, win, a, stream) : launch_dkv<64, true>(g, win, a, stream);
}

}  // namespace sta
