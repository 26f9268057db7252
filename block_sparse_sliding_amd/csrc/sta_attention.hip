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
// Work decomposition. A workgroup of 4 waves (one per SIMD) works on one query
// unit at a time: a 384-row query tile (96 rows per wave), or the 256 text
// query slots of one head (64 rows per wave). The grid is persistent: each
// workgroup pops units from the queue of the XCD it runs on and, once that
// queue is empty, from the other XCDs' queues. The key tiles of a unit's
// window are enumerated in the kernel (residue order, see key_tile), so no
// schedule list is read. Q rows are read from the caller's raster q through
// the tile map, K and V rows from the caller's raster k and v (LDS-DMA, one
// source address per lane, which applies the tile map), and O / lse are
// written to raster positions.
//
// Products: v_mfma_f32_32x32x16_bf16 throughout.
//   S^T = K Q^T    A = K fragment (lane l: key 32h + l%32, d 16ks + 8(l/32)
//                  .. +8), B = Q^T fragment (registers, loaded once per unit).
//                  Lane l then holds the scores of query l%32 for keys
//                  8(i/4) + 4(l/32) + i%4, i = 0..15, of each 32-key half.
//   O^T += V^T P^T A = V^T fragment read with ds_read_b64_tr_b16 from V rows
//                  in LDS (the transposing read turns 4 keys x 16 columns of
//                  row-major V into the k-contiguous operand), B = P^T from
//                  the lane's own registers: the 16 scores of a half are two
//                  16-key chunks in exactly the key order the A operand uses.
//                  The accumulators live in AGPRs (inline-asm MFMAs with "+a"
//                  operands); the score MFMAs write VGPRs.
//
// Software pipeline. Each 64-key block is two 32-key halves; half-step hh
// issues, for all 96 rows of the wave, the score MFMAs of half hh + 1 and the
// P V MFMAs of half hh - 1, and between consecutive MFMAs one slice of the
// softmax of half hh: p = 2^(c s - m) (one v_fma_f32, one v_exp_f32), pairs
// rounded to bf16 (v_cvt_pk_bf16_f32, the P operand) and summed into the row
// sum (v_dot2_f32_bf16 with ones). The fma, exp and pack of one score sit in
// three consecutive MFMA slots, so no VALU instruction waits on the one
// before it; one wave per SIMD then keeps the matrix core busy while it
// issues the softmax. K and V each have two LDS stages; the K stream runs one
// block ahead of the V stream, and one barrier per block orders the LDS-DMA
// writes against the reads.
//
// Softmax reference. The reference m of a row is the exact maximum of its
// scaled scores over the first 32 keys of the unit, and it never moves:
// p = 2^(c s - m) stays within fp32 as long as no later score exceeds m by
// about 127 (log2 units). At the end of a unit, a row whose sum of p reaches
// 2^32 (some later key scored at least 32 above the first half's maximum)
// makes the workgroup redo the unit with m set to the row's maximum over all
// its keys, found by a pass that computes only the scores. With random data
// the redo never happens; large score jumps between key tiles trigger it.
//
// LDS layouts (row-major rows of D bf16 = 2D bytes, grouped by 1 KB: RPG rows
// per group, 4 for D = 128 and 8 for D = 64; a group is one LDS-DMA
// instruction). Inside a group, 16-byte chunk c of group row rr sits at
// (c / 4) * RPG * 64 + rr * 64 + 16 * (c % 4) for V, and at the same place
// with c % 4 replaced by (c % 4) XOR ((row / 4) % 4) for K. A score-MFMA K
// read (16 lanes per LDS cycle, rows {0-3, 12-15, 20-23, 24-27} or the other
// parity class, one chunk) then covers all 64 banks, and so does a V^T
// transposing read (4 rows x 64 bytes per 32 lanes); every read address is one
// of a few per-lane bases plus a compile-time offset.
//
// Masking. Keys that must not contribute (text slots at or after text_length;
// with PAD, keys past a partial tile's tokens) are fetched from a zero row in
// the workspace, K and V alike, and their scores are replaced by -inf before
// the exponential; their p is exactly 0 and their V rows are zeros, so the
// contents of padded text slots never reach a result.
//
// Video sizes that are not tile multiples (PAD): the last tile along an axis
// holds the remainder. A partial key tile streams ceil(tokens / 64) blocks of
// its existing tokens in compact order (frame, row, column); its full blocks
// take their place in the walk, and its last, partial block is deferred to a
// tail of masked blocks after all whole ones (KeyStream), so the main loop
// runs the unmasked half-steps only and the masked variant appears in the
// tail alone (one loop holding both would exceed the register file). A video unit's
// rows are its tile's existing tokens in compact order; a tile of at most 128
// or 256 tokens runs with 32 or 64 rows per wave, and a wave whose rows all lie
// past the tokens only loads and synchronises. Rows past the tokens compute on
// a valid row and are not written.
// Epilogue: O = O^T / l rounded to bf16, lse = (m + log2 l) * ln 2, at raster rows.
#include <type_traits>

#include "sta_device.h"
#include "sta_internal.h"

namespace sta {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kWaves = 4;  // one wave per SIMD
constexpr int kThreads = kWaves * 64;
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

// O^T += V^T P^T on AGPR accumulators (the compiler's hazard checks do not see
// inline asm: every VGPR this reads was written at least two instructions
// earlier, see the slot order, and the accumulators are read only after an
// explicit wait).
// (The host pass of this single-source file checks asm constraints against
// the host target, where "a" means a general register: the statements exist
// in the device pass only.)
#if defined(__HIP_DEVICE_COMPILE__)
#define STA_PV_MFMA_ASM(NOP, acc, vf, pf) \
  asm volatile(NOP "v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(vf), "v"(pf))
#else
#define STA_PV_MFMA_ASM(NOP, acc, vf, pf) ((void)(acc), (void)(vf), (void)(pf))
#endif
#define STA_PV_MFMA(acc, vf, pf) STA_PV_MFMA_ASM("", acc, vf, pf)

// LDS-DMA of 16 bytes per lane from base + soff (wave-uniform) + voff (per
// lane) into lds_dst + 16 lane, through a buffer resource over base (the
// uniform part stays in scalar registers). The instruction is written as
// inline asm on purpose: the compiler treats an LDS-DMA it can see as a store
// to all of LDS and makes every later LDS read wait for it (vmcnt(0)), which
// would expose the whole memory latency inside the MFMA loop. The kernel
// orders these writes itself: every read of a block follows the s_waitcnt
// vmcnt(0) and the barrier that close the block before it. (M0 holds the LDS
// destination: it is saved and restored around the load, and one wait state
// separates its write from the load that reads it. The statements exist in
// the device pass only, as the host pass checks the constraints against the
// host target.)
__device__ inline void dma16_buf(const char* base, int voff, int soff, char* lds_dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  const unsigned long long b = reinterpret_cast<unsigned long long>(base);
  const i32x4 rsrc = {int(unsigned(b)), int(unsigned(b >> 32) & 0xffffu), 0x7fffffff, 0x00020000};
  const unsigned m0 = unsigned(reinterpret_cast<unsigned long long>((lds_void*)lds_dst));
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rsrc), "s"(m0), "s"(soff)
      : "memory");
#else
  (void)base, (void)voff, (void)soff, (void)lds_dst;
#endif
}

template <int D>
struct Lay {
  static constexpr int ROWB = 2 * D;        // bytes per row
  static constexpr int RPG = 1024 / ROWB;   // rows per 1 KB group
  static constexpr int KS = D / 16;         // k-steps of the score MFMAs
  static constexpr int DT = D / 32;         // 32-column tiles of O
  static constexpr int BLKB = 64 * ROWB;    // bytes of a 64-row K or V block
  static constexpr int GPB = 64 / RPG;      // 1 KB groups per block
  static constexpr int GPW = GPB / kWaves;  // groups per wave
  static constexpr int NVF = 2 * DT;        // V^T fragments per half (2 chunks of 16 keys x DT)
  static constexpr int NF = NVF + KS;       // fragments per half-step
  static constexpr int SPS = 16 / NF;       // scores (per lane and query group) per MFMA slot
  static constexpr int QSEG = RPG * 64;     // bytes between chunk quads inside a group
  static_assert(GPW >= 1 && GPB % kWaves == 0, "groups split evenly over the waves");
};

template <int D, bool PAD>
__global__ __launch_bounds__(kThreads, 1) void sta_attention_kernel(KernelArgs) {
  using L = Lay<D>;
  constexpr int ROWB = L::ROWB, RPG = L::RPG, KS = L::KS, DT = L::DT, BLKB = L::BLKB;
  // K stages at [0, 2 BLKB), V stages at [2 BLKB, 5 BLKB)
  __shared__ __attribute__((aligned(1024))) char lds[5 * BLKB];
  __shared__ int shared_word[2];

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
    const bool text_unit = g.has_text && u == g.n_tiles;

    // query tile coordinates and rows (PAD: its existing tokens, compact order)
    int qtt = 0, qth = 0, qtw = 0;
    int q_ext = kFullExtent, q_base = 0;
    int q_rows = text_unit ? kTextSlots : kTileRows;
    if (!text_unit) {
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
    KeyStream<PAD> keys;
    if (text_unit)
      keys.init(g, 0, g.nt, 0, g.nh, 0, g.nw);
    else
      keys.init(g, window_start(qtt, wt, g.nt), wt, window_start(qth, wh, g.nh), wh, window_start(qtw, ww, g.nw), ww);
    const int n_plain = keys.n_plain, n_blk = keys.n_blk;

    const size_t slab = size_t(bh) * g.S * D;
    const char* __restrict__ kr = reinterpret_cast<const char*>(a.k) + slab * 2;
    const char* __restrict__ vr = reinterpret_cast<const char*>(a.v) + slab * 2;
    const char* __restrict__ zr = reinterpret_cast<const char*>(a.zero_row);

    auto decode = [&](int j) { return keys.block(g, j); };
    auto reset_walk = [&]() { keys.reset(); };

    // ---- LDS-DMA of one block (this wave's GPW groups). Lane p of a group
    // covers group row rr = (p / 4) % RPG and chunk 4 (p / (4 RPG)) + p % 4,
    // XOR-ed with the row's (row / 4) % 4 for K. The source of a full frame's
    // rows (the common case) is a wave-uniform row pointer plus a per-lane
    // offset; text rows past the valid length and, with PAD, keys past a
    // partial tile's tokens come from the zero row.
    auto issue = [&](const KeyBlock& s, int stage_off, bool is_k) {
      const int ln = opaque_lane<true>(this_lane);
      const int rr = (ln >> 2) % RPG, j4 = ln & 3, q4 = 4 * (ln / (4 * RPG));
      const char* base = is_k ? kr : vr;
      char* dst = lds + stage_off + wave * L::GPW * 1024;
      auto chunk = [&](int G) {  // this lane's chunk for group G
        const int x = ((G * RPG + rr) >> 2) & 3;
        return q4 + (is_k ? (j4 ^ x) : j4);
      };
      if (s.kind == 0) {
#pragma unroll
        for (int i = 0; i < L::GPW; ++i) {
          const int G = wave * L::GPW + i, r0 = G * RPG;
          // rows r0 .. r0 + RPG - 1 lie in one 8-row run of the frame
          const int row0 = s.base + (r0 >> 3) * g.W + (r0 & 7);
          dma16_buf(base, rr * ROWB + chunk(G) * 16, row0 * ROWB, dst + i * 1024);
        }
      } else if (!PAD || s.kind == 1) {
#pragma unroll
        for (int i = 0; i < L::GPW; ++i) {
          const int G = wave * L::GPW + i, r = G * RPG + rr;
          const char* src = r < s.lim ? base + size_t(s.base + r) * ROWB : zr;
          dma16(src + chunk(G) * 16, dst + i * 1024);
        }
      } else {
        const int n_tok = extent_tokens(s.ext);
#pragma unroll
        for (int i = 0; i < L::GPW; ++i) {
          const int G = wave * L::GPW + i, tok = s.sub * kKeyBlock + G * RPG + rr;
          int dt, dh, dw;
          compact_token(tok < n_tok ? tok : 0, s.ext, dt, dh, dw);
          const char* src = tok < n_tok ? base + size_t(s.base + (dt * g.H + dh) * g.W + dw) * ROWB : zr;
          dma16(src + chunk(G) * 16, dst + i * 1024);
        }
      }
    };

    // One group (op < GPW: K group op, else V group op - GPW) of a full-frame
    // block (kind 0), for DMA spread over the MFMA slots of a half-step.
    auto issue_frame_op = [&](const KeyBlock& s, int k_stage_off, int v_stage_off, int op) {
      const bool is_k = op < L::GPW;
      const int i = is_k ? op : op - L::GPW;
      const int ln = opaque_lane<true>(this_lane);
      const int rr = (ln >> 2) % RPG, j4 = ln & 3, q4 = 4 * (ln / (4 * RPG));
      const int G = wave * L::GPW + i, r0 = G * RPG;
      const int x = ((G * RPG + rr) >> 2) & 3;
      const int chunk = q4 + (is_k ? (j4 ^ x) : j4);
      const int row0 = s.base + (r0 >> 3) * g.W + (r0 & 7);
      dma16_buf(is_k ? kr : vr, rr * ROWB + chunk * 16, row0 * ROWB,
                lds + (is_k ? k_stage_off : v_stage_off) + wave * L::GPW * 1024 + i * 1024);
    };

    // ---- per-lane LDS read bases
    const int kl = lane & 31, kx = (kl >> 2) & 3;
    const int k_lane = (kl / RPG) * 1024 + (kl % RPG) * 64;
    const int kb_even = k_lane + (((lane >> 5)) ^ kx) * 16;
    const int kb_odd = k_lane + ((2 | (lane >> 5)) ^ kx) * 16;
    const int vi = lane & 15;
    const int vrow = 4 * (lane >> 5) + (vi >> 2);  // row inside a 16-key chunk
    const int vb = 2 * BLKB + (vrow / RPG) * 1024 + (vrow % RPG) * 64 + 32 * ((lane >> 4) & 1) + 8 * (vi & 1) +
                   16 * ((vi & 3) >> 1);
    const char* lds_ke = lds + kb_even;
    const char* lds_ko = lds + kb_odd;
    const char* lds_v = lds + vb;

    const float qs = a.q_scale;  // log2(e)/sqrt(D)
    const bf16x2 ones2 = {(__bf16)1.0f, (__bf16)1.0f};

    // The rest runs with QG query groups of 32 rows per wave: 3 for a video
    // tile, 2 for the text slots (and partial tiles of 129..256 tokens), 1 for
    // partial tiles of at most 128 tokens.
    auto run = [&](auto qg_c) {
      constexpr int QG = decltype(qg_c)::value;
      constexpr int RPW = 32 * QG;
      constexpr int NF = L::NF, NVF = L::NVF, SPS = L::SPS;
      constexpr int SLOTS = NF * QG;  // MFMAs per half-step
      constexpr int NSC = 16 * QG;    // scores per lane per half-step
      const bool active = wave * RPW < q_rows;
      (void)active;

      // Q^T fragments: lane l, group c, step ks: row 32 c + l % 32 of this wave,
      // columns 16 ks + 8 (l / 32) .. + 8 (rows past the unit clamp to its last)
      bf16x8 qf[QG][KS];
#pragma unroll
      for (int c = 0; c < QG; ++c) {
        int row = wave * RPW + 32 * c + (lane & 31);
        row = row < q_rows ? row : q_rows - 1;
        const __bf16* src = reinterpret_cast<const __bf16*>(a.q) + slab + size_t(query_raster(row)) * D +
                            8 * (lane >> 5);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[c][ks] = *reinterpret_cast<const bf16x8*>(src + 16 * ks);
      }

      f32x16 acc[QG][DT];
      float lsum[QG], m_run[QG];

      // K fragment ks of K half kh in K stage kst (compile-time offsets when
      // the stage is)
      auto kfrag = [&](int kst, int kh, int ks) -> bf16x8 {
        return *reinterpret_cast<const bf16x8*>(((ks & 1) ? lds_ko : lds_ke) + kst * BLKB + (32 * kh) / RPG * 1024 +
                                                (ks >> 1) * L::QSEG);
      };
      // V^T fragment f (chunk f / DT, tile f % DT) of V half vh at V offset voff
      auto vfrag_at = [&](int voff, int vh, int f) -> bf16x8 {
        const int kc = f / DT, dt = f % DT;
        const char* p = lds_v + voff + (32 * vh + 16 * kc) / RPG * 1024 + dt * L::QSEG;
        const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
        const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 8 / RPG * 1024));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      };

      // softmax pipeline state: t = c s - m of the last scores (stage A),
      // e = exponentials by group and element parity (stage B)
      float vt[2 * SPS];
      float ve[QG][2];
      // slot k, stage A of scores SPS k .. SPS k + SPS - 1, B of the SPS
      // before, C (pack + row sum) of those before that; score sc is element
      // i = sc / QG of group c = sc % QG
      auto vstage = [&](int k, f32x16 (&s)[QG], uint32_t (&pw)[QG][8], bool do_a, bool do_mask, int lim_lane) {
#pragma unroll
        for (int x = 0; x < SPS; ++x) {
          const int c2 = SPS * (k - 2) + x;  // stage C
          if (c2 >= 0 && c2 < NSC && ((c2 / QG) & 1)) {
            const int c = c2 % QG, i = c2 / QG;
            const bf16x2 pr = __builtin_convertvector((f32x2){ve[c][0], ve[c][1]}, bf16x2);
            lsum[c] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones2, lsum[c], false);
            pw[c][i >> 1] = __builtin_bit_cast(uint32_t, pr);
          }
        }
#pragma unroll
        for (int x = 0; x < SPS; ++x) {
          const int b1 = SPS * (k - 1) + x;  // stage B
          if (b1 >= 0 && b1 < NSC) ve[b1 % QG][(b1 / QG) & 1] = __builtin_amdgcn_exp2f(vt[b1 % (2 * SPS)]);
        }
        if (do_a) {
#pragma unroll
          for (int x = 0; x < SPS; ++x) {
            const int a0 = SPS * k + x;  // stage A
            const int i = a0 / QG;
            const float t = __builtin_fmaf(s[a0 % QG][i], qs, -m_run[a0 % QG]);
            // masked half: key 8 (i / 4) + 4 (l / 32) + i % 4 at or past the limit
            vt[a0 % (2 * SPS)] = (do_mask && 8 * (i >> 2) + (i & 3) >= lim_lane) ? -INFINITY : t;
          }
        }
      };

      // One half-step: SLOTS MFMA slots over NF fragments x QG groups.
      // Fragment f + PF is read when fragment f is first used; V^T fragments
      // of the next half-step are read during the last slots. Scores of
      // s_cur pass through the softmax stages, one group of SPS per slot; the
      // last scores' B and C stages run in the first slots of the next
      // half-step (carried through vt / ve). DO_S, DO_PV, DO_P: whether the
      // step scores the next half, multiplies the previous half's P by V, and
      // has scores of its own. voff / nvoff: byte offsets of the V stages of
      // this step's and the next step's P V; kst: K stage of the next half.
      constexpr int PF = 3;
      auto no_hook = [](int) {};
      auto step = [&](auto do_s_c, auto do_pv_c, auto do_p_c, auto do_mask_c, auto kst, int voff, int vh, int kh,
                      int nvoff, int nvh, int lim, bf16x8 (&fr)[PF], f32x16 (&s_next)[QG], f32x16 (&s_cur)[QG],
                      uint32_t (&p_prev)[QG][8], uint32_t (&p_cur)[QG][8], auto&& hook) {
        constexpr bool DO_S = decltype(do_s_c)::value, DO_PV = decltype(do_pv_c)::value;
        constexpr bool DO_P = decltype(do_p_c)::value, DO_MASK = decltype(do_mask_c)::value;
        const int KST = kst;
        // masked half: this lane's keys 8 (i / 4) + 4 (l / 32) + i % 4 at or past lim are dead
        const int lim_lane = lim - 4 * (lane >> 5);
        // opaque stage offsets (32-bit LDS byte offsets): every V^T read is
        // one of them plus an immediate
        int vcur = vb + voff + (32 * vh) / RPG * 1024;
        int vnext = vb + nvoff + (32 * nvh) / RPG * 1024;
        asm volatile("" : "+v"(vcur), "+v"(vnext));
        auto vfrag = [&](int vb0, int f) -> bf16x8 {
          const int kc = f / DT, dt = f % DT;
          const char* p = lds + vb0 + (16 * kc) / RPG * 1024 + dt * L::QSEG;
          const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
          const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 8 / RPG * 1024));
          return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        bf16x8 ring[NF + PF];
#pragma unroll
        for (int i = 0; i < PF; ++i) ring[i] = fr[i];
#pragma unroll
        for (int k = 0; k < SLOTS; ++k) {
          const int f = k / QG, c = k % QG;
          if (c == 0) {
            const int nf = f + PF;
            if (nf < NVF) {
              if (DO_PV) ring[nf] = vfrag(vcur, nf);
            } else if (nf < NF) {
              if (DO_S) ring[nf] = kfrag(KST, kh, nf - NVF);
            } else {
              ring[nf] = vfrag(vnext, nf - NF);  // next half-step's V^T
            }
          }
          if (f < NVF) {
            if constexpr (DO_PV) {
              const int kc = f / DT, dt = f % DT;
              const bf16x8 pb = __builtin_bit_cast(
                  bf16x8, (uint4){p_prev[c][4 * kc], p_prev[c][4 * kc + 1], p_prev[c][4 * kc + 2], p_prev[c][4 * kc + 3]});
              if (kc == 1 && dt == 0)  // its last dwords may have been packed in slot 0 or 1
                STA_PV_MFMA_ASM("s_nop 1\n\t", acc[c][dt], ring[f], pb);
              else
                STA_PV_MFMA(acc[c][dt], ring[f], pb);
            }
          } else if constexpr (DO_S) {
            const int ks = f - NVF;
            s_next[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[f], qf[c][ks], ks == 0 ? f32x16{} : s_next[c],
                                                                0, 0, 0);
          }
          hook(k);
          if constexpr (DO_PV) {  // a previous half exists: finish its last scores
            if (k == 0) vstage(SLOTS, s_cur, p_prev, false, false, 0);
            if (k == 1) vstage(SLOTS + 1, s_cur, p_prev, false, false, 0);
          }
          if constexpr (DO_P) vstage(k, s_cur, p_cur, true, DO_MASK, lim_lane);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < PF; ++i) fr[i] = ring[NF + i];
      };

      // replace the scores of keys at or past `lim` (0..32, within a half) by -inf
      auto mask_half = [&](f32x16 (&s)[QG], int lim) {
        int key0 = 4 * (lane >> 5);
        asm volatile("" : "+v"(key0));
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const bool dead = key0 + 8 * (i >> 2) + (i & 3) >= lim;
#pragma unroll
          for (int c = 0; c < QG; ++c) s[c][i] = dead ? -INFINITY : s[c][i];
        }
      };

      // scores of one half of the block in K stage kst, with masking
      auto scores = [&](f32x16 (&s)[QG], int kst, int kh, int mask) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 x = kfrag(kst, kh, ks);
#pragma unroll
          for (int c = 0; c < QG; ++c)
            s[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, qf[c][ks], ks == 0 ? f32x16{} : s[c], 0, 0, 0);
        }
        if (mask - 32 * kh < 32) mask_half(s, mask - 32 * kh);
      };

      // Streaming (main pass): blocks 0 and 1 are fetched before the first
      // barrier; after the barrier of block j (which follows the wait for
      // this wave's own loads) block j + 2 is fetched, K into K stage j % 2
      // and V into V stage (j + 2) % 3. K(j) was last read in half-step 2j
      // and V(j - 1) in half-step 2j, both before that barrier; K(j + 2) is
      // first read in half-step 2j + 3 and V(j + 2) at the end of half-step
      // 2j + 4, both after the next barrier.
      auto voff_of = [](int j) { return (j % 3) * BLKB; };

      // ---- an idle wave of a partial unit: the same loads and barriers
      auto idle_main = [&]() {
        reset_walk();
        const KeyBlock s0 = decode(0);
        issue(s0, 0, true);
        issue(s0, 2 * BLKB + voff_of(0), false);
        if (n_blk > 1) {
          const KeyBlock s1 = decode(1);
          issue(s1, BLKB, true);
          issue(s1, 2 * BLKB + voff_of(1), false);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        for (int j = 0; j < n_blk; ++j) {
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          __syncthreads();
          if (j + 2 < n_blk) {
            const KeyBlock s2 = decode(j + 2);
            issue(s2, (j & 1) * BLKB, true);
            issue(s2, 2 * BLKB + voff_of(j + 2), false);
          }
        }
      };
      auto idle_max = [&]() {
        reset_walk();
        for (int j = 0; j < n_blk; ++j) {
          const KeyBlock s = decode(j);
          issue(s, 0, true);
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          __syncthreads();
          __syncthreads();
        }
      };

      // ---- pass 1 (rare): the exact row maxima over all keys, scores only
      auto max_pass = [&]() {
        float mx[QG];
#pragma unroll
        for (int c = 0; c < QG; ++c) mx[c] = -INFINITY;
        reset_walk();
        for (int j = 0; j < n_blk; ++j) {
          const KeyBlock s = decode(j);
          issue(s, 0, true);
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          __syncthreads();
#pragma unroll
          for (int kh = 0; kh < 2; ++kh) {
            f32x16 sc[QG];
            scores(sc, 0, kh, s.mask);
#pragma unroll
            for (int c = 0; c < QG; ++c)
#pragma unroll
              for (int i = 0; i < 16; ++i) mx[c] = fmaxf(mx[c], sc[c][i]);
          }
          __syncthreads();  // every wave has read the stage before it is refilled
        }
#pragma unroll
        for (int c = 0; c < QG; ++c) m_run[c] = swap32_max(mx[c]) * qs;
      };

      // ---- the pipelined pass; m_run was set by max_pass when `known`
      auto main_pass = [&](bool known) {
        using T = std::true_type;
        using F = std::false_type;
#pragma unroll
        for (int c = 0; c < QG; ++c) {
#pragma unroll
          for (int d = 0; d < DT; ++d) acc[c][d] = f32x16{};
          lsum[c] = 0.f;
        }
        reset_walk();
        const KeyBlock s0 = decode(0);
        issue(s0, 0, true);
        issue(s0, 2 * BLKB + voff_of(0), false);
        int mask1 = 64;  // mask of block j + 1 in body(j)
        int mask2 = 64;  // mask of block j + 2
        if (n_blk > 1) {
          const KeyBlock s1 = decode(1);
          issue(s1, BLKB, true);
          issue(s1, 2 * BLKB + voff_of(1), false);
          mask1 = s1.mask;
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        f32x16 sa[QG], sb[QG];
        uint32_t pa[QG][8], pb[QG][8];
        scores(sa, 0, 0, s0.mask);  // S(0), masked
        if (!known) {
          // the reference: exact maximum of each row's scaled scores over half 0
#pragma unroll
          for (int c = 0; c < QG; ++c) {
            float x = sa[c][0];
#pragma unroll
            for (int i = 1; i < 16; ++i) x = fmaxf(x, sa[c][i]);
            m_run[c] = swap32_max(x) * qs;
          }
        }
        bf16x8 fr[PF];
#pragma unroll
        for (int i = 0; i < PF; ++i) fr[i] = vfrag_at(voff_of(0), 0, i);
        asm volatile("s_nop 2" ::: "memory");  // accumulator writes before the first asm MFMA
        // half-step 0: S(1) (K(0) half 1) and P(0); no P V yet
        step(T{}, F{}, T{}, F{}, std::integral_constant<int, 0>{}, voff_of(0), 0, 1, voff_of(0), 0, 64, fr, sb, sa,
             pb, pa, no_hook);
        if (s0.mask < 64) mask_half(sb, s0.mask - 32);  // S(1): block 0 half 1
        // body(j): half-steps 2j + 1 (scores K(j + 1) half 0 into S(2j + 2),
        // P V of half 2j = V(j) half 0, softmax of S(2j + 1): block j half 1)
        // and 2j + 2 (scores K(j + 1) half 1, P V of half 2j + 1, softmax of
        // S(2j + 2): block j + 1 half 0). mask_a, mask_b: the masks of the
        // halves consumed (64 when nothing is masked).
        // Block j + 2 is fetched after the barrier; a block of full frames
        // (the common case) one group at a time, spread over the MFMA slots
        // of the first half-step, any other block at once.
        auto body = [&](auto mask_first_c, auto mask_second_c, auto kst, int j, int mask_a, int mask_b) {
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          __syncthreads();
          KeyBlock s2{};
          bool spread = false;
          const int k_off = (j & 1) * BLKB, v_off = 2 * BLKB + voff_of(j + 2);
          if (j + 2 < n_blk) {
            s2 = decode(j + 2);
            mask2 = s2.mask;
            spread = s2.kind == 0;
            if (!spread) {
              issue(s2, k_off, true);
              issue(s2, v_off, false);
            }
          }
          auto dma = [&](int k) {
            constexpr int NOPS = 2 * L::GPW;
            constexpr int SP = (SLOTS - 2) / NOPS > 0 ? (SLOTS - 2) / NOPS : 1;
            if (k >= 2 && (k - 2) % SP == 0 && (k - 2) / SP < NOPS && spread)
              issue_frame_op(s2, k_off, v_off, (k - 2) / SP);
          };
          const int vj = voff_of(j), vj1 = voff_of(j + 1);
          step(T{}, T{}, T{}, mask_first_c, kst, vj, 0, 0, vj, 1, mask_a, fr, sa, sb, pa, pb, dma);
          step(T{}, T{}, T{}, mask_second_c, kst, vj, 1, 1, vj1, 0, mask_b, fr, sb, sa, pb, pa, no_hook);
        };
        int mask0 = s0.mask;  // mask of block j in body(j)
        auto advance = [&]() {
          mask0 = mask1;
          mask1 = mask2;
          mask2 = 64;
        };
        // bodies j with j + 1 < n_plain consume unmasked halves only
        int j = 0;
        for (; j + 2 < n_plain; j += 2) {
          body(F{}, F{}, std::integral_constant<int, 1>{}, j, 64, 64);
          advance();
          body(F{}, F{}, std::integral_constant<int, 0>{}, j + 1, 64, 64);
          advance();
        }
        if (j + 1 < n_plain) {
          body(F{}, F{}, std::integral_constant<int, 1>{}, j, 64, 64);
          advance();
          ++j;
        }
        if constexpr (!PAD) {
          // only the last block can be masked: body(n_blk - 2) consumes its half 0
          if (j + 1 < n_blk) {
            body(F{}, T{}, 1 - (j & 1), j, 64, mask1);
            advance();
            ++j;
          }
        } else {
          for (; j + 1 < n_blk; ++j) {  // the masked tail
            body(T{}, T{}, 1 - (j & 1), j, mask0 - 32, mask1);
            advance();
          }
        }
        // the last block j = n_blk - 1: half-step 2j + 1 (P V of half 2j,
        // softmax of block j half 1, masked) and 2j + 2 (P V of half 2j + 1)
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        const int vj = voff_of(j);
        step(F{}, T{}, T{}, T{}, 0, vj, 0, 0, vj, 1, mask0 - 32, fr, sa, sb, pa, pb, no_hook);
        step(F{}, T{}, F{}, F{}, 0, vj, 1, 0, vj, 1, 64, fr, sb, sa, pb, pa, no_hook);
        asm volatile("s_nop 15\n\ts_nop 7" ::: "memory");  // last MFMA results before any read
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
      // row's sum (relative to its first half's maximum) got large
      for (bool known = false;; known = true) {
        main_pass(known);
        if (known) break;
        bool redo = false;
#pragma unroll
        for (int c = 0; c < QG; ++c) redo |= !(swap32_sum(lsum[c]) < kRedoSum);
        if (__builtin_amdgcn_ballot_w64(redo) != 0 && lane == 0) shared_word[1] = 1;
        __syncthreads();
        if (__builtin_amdgcn_readfirstlane(shared_word[1]) == 0) break;
        __syncthreads();
        max_pass();
      }

      // ---- epilogue: O = O^T / l (bf16) and lse at raster rows; lane l holds
      // query 32 c + l % 32, columns 32 dt + 8 g + 4 (l / 32) + 0..3 in
      // accumulator registers 4 g .. 4 g + 3
      __bf16* __restrict__ outr = reinterpret_cast<__bf16*>(a.out) + slab;
      float* __restrict__ lser = a.lse == nullptr ? nullptr : a.lse + size_t(bh) * g.S;
#pragma unroll
      for (int c = 0; c < QG; ++c) {
        const float l = swap32_sum(lsum[c]);
        const float inv = __builtin_amdgcn_rcpf(l);
        const int row = wave * RPW + 32 * c + (lane & 31);
        if (row < q_rows) {
          const int rr = query_raster(row);
          __bf16* dst = outr + size_t(rr) * D + 4 * (lane >> 5);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              const f32x4 o = {acc[c][dt][4 * gq] * inv, acc[c][dt][4 * gq + 1] * inv, acc[c][dt][4 * gq + 2] * inv,
                               acc[c][dt][4 * gq + 3] * inv};
              *reinterpret_cast<bf16x4*>(dst + 32 * dt + 8 * gq) = __builtin_convertvector(o, bf16x4);
            }
          if (lser != nullptr && lane < 32) lser[rr] = (m_run[c] + __builtin_amdgcn_logf(l)) * kLn2;
        }
      }
    };
    if (text_unit || (PAD && q_rows > 4 * 32 && q_rows <= kTextSlots))
      run(std::integral_constant<int, 2>{});
    else if (PAD && q_rows <= 4 * 32)
      run(std::integral_constant<int, 1>{});
    else
      run(std::integral_constant<int, 3>{});
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
