// Tile-window schedule, built on the device.
//
// For each head and query tile the key tiles of its window: per axis the
// window of w tiles starts at clamp(c - w/2, 0, n - w), i.e. it is centred on
// the query tile and shifted inward at the grid border so that it always
// holds w tiles. (The STA README "Usage" section states that window (3,3,3)
// gives every query the same (18,24,24) token box of the (30,48,80) video.)
// The text query unit of a head sees every tile.
//
// The work order holds one queue of query units per XCD, heaviest first,
// spreading every class of equal-cost units evenly over the 8 queues with
// each queue taking a contiguous run of each class.
#include "sta_internal.h"

namespace sta {
namespace {

// Offset inside a window [s, s + w) of the coordinate congruent to r mod w
// (r in [0, w)). Listing a window's tiles by the residues of their absolute
// coordinates, rather than by their offsets from the window start, makes
// query tiles whose windows overlap read each shared key tile at the same
// step of their key loop; workgroups on one XCD run in step, so the shared
// tile is then fetched into that XCD's L2 once rather than once per query
// tile.
__device__ inline int residue_offset(int r, int s, int w) {
  const int d = (r - s) % w;
  return d < 0 ? d + w : d;
}

__device__ inline int64_t head_list_len(const Geom& g, uint32_t p) {
  const int64_t wv = int64_t(win_t(p)) * win_h(p) * win_w(p);
  return int64_t(g.n_tiles) * wv + (g.has_text ? g.n_tiles : 0);
}

// grid (n_q, heads): one workgroup writes one query unit's key-tile list.
__global__ __launch_bounds__(256) void schedule_lists_kernel(Geom g, Windows win,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ ids) {
  const int u = blockIdx.x;
  const int hd = blockIdx.y;
  int64_t base = 0;
  for (int h2 = 0; h2 < hd; ++h2) base += head_list_len(g, win.w[h2]);
  const uint32_t p = win.w[hd];
  const int wt = win_t(p), wh = win_h(p), ww = win_w(p);
  const int wv = wt * wh * ww;
  if (u < g.n_tiles) {
    const int64_t off = base + int64_t(u) * wv;
    if (threadIdx.x == 0) offsets[hd * g.n_q + u] = int32_t(off);
    const int tw = u % g.nw, th = (u / g.nw) % g.nh, tt = u / (g.nw * g.nh);
    const int st = window_start(tt, wt, g.nt), sh = window_start(th, wh, g.nh),
              sw = window_start(tw, ww, g.nw);
    for (int j = threadIdx.x; j < wv; j += blockDim.x) {
      const int a = j / (wh * ww), b = (j / ww) % wh, c = j % ww;
      ids[off + j] = ((st + residue_offset(a, st, wt)) * g.nh + (sh + residue_offset(b, sh, wh))) *
                         g.nw +
                     (sw + residue_offset(c, sw, ww));
    }
  } else {
    const int64_t off = base + int64_t(g.n_tiles) * wv;
    if (threadIdx.x == 0) offsets[hd * g.n_q + u] = int32_t(off);
    for (int j = threadIdx.x; j < g.n_tiles; j += blockDim.x) ids[off + j] = j;
  }
  if (hd == g.heads - 1 && u == g.n_q - 1 && threadIdx.x == 0)
    offsets[g.heads * g.n_q] = int32_t(base + head_list_len(g, p));
}

constexpr int kWorkThreads = 256;
constexpr int kMaxClasses = 2 * kMaxHeads;
constexpr int kXcds = kQueues;
static_assert(kXcds == 8, "the queue index is the XCD id mod 8");

// grid ceil(units / 256). Query units fall into classes of equal cost, one
// per (head, video|text). Entry i = 8k + x is item k of XCD x's queue; each
// queue takes, class by class in decreasing cost, an equal share of every
// class: a contiguous run of that class's units (so the XCD's L2 serves
// neighbouring tiles), with the remainders of uneven classes rotated over the
// XCDs. Heavy classes therefore spread evenly over the XCDs and run first,
// and all XCDs work through the same head at about the same time. The
// attention kernel's workgroups pop their own XCD's queue and, once it is
// empty, the other queues, so XCDs that run at a higher clock take more units.
// Every workgroup rebuilds the small class table in LDS, then each thread
// resolves one entry to its query unit; block 0 also zeroes the queue heads.
__global__ __launch_bounds__(kWorkThreads) void schedule_work_kernel(Geom g, Windows win,
                                                                     int32_t* __restrict__ work,
                                                                     int32_t* __restrict__ claim,
                                                                     int32_t* __restrict__ zero_row) {
  if (claim != nullptr && blockIdx.x == 0)
    for (int i = threadIdx.x; i < kClaimInts; i += kWorkThreads) claim[i] = 0;
  if (zero_row != nullptr && blockIdx.x == 0)
    for (int i = threadIdx.x; i < kZeroRowBytes / 4; i += kWorkThreads) zero_row[i] = 0;
  __shared__ long long cost[kMaxClasses];
  __shared__ int count[kMaxClasses];
  __shared__ int order[kMaxClasses];  // order[rank] = class
  __shared__ int rot[kMaxClasses];    // first XCD that takes a remainder unit of class c
  const int C = 2 * g.heads;
  for (int c = threadIdx.x; c < C; c += kWorkThreads) {
    const int hd = c >> 1, text = c & 1;
    const uint32_t p = win.w[hd];
    const long long keys_extra = g.has_text ? g.text_length : 0;
    if (!text) {
      count[c] = g.B * g.n_tiles;
      cost[c] = (long long)kTileRows *
                ((long long)win_t(p) * win_h(p) * win_w(p) * kTileRows + keys_extra);
    } else {  // the text rows, split over text_parts units by key tiles
      count[c] = g.has_text ? g.B * g.text_parts : 0;
      cost[c] = (long long)kTextSlots * ((long long)g.n_tiles * kTileRows + keys_extra) / g.text_parts;
    }
  }
  __syncthreads();
  // classes ordered by decreasing cost, ties by class index
  for (int c = threadIdx.x; c < C; c += kWorkThreads) {
    int rank = 0, rem_before = 0;
    for (int c2 = 0; c2 < C; ++c2) {
      const bool before = cost[c2] > cost[c] || (cost[c2] == cost[c] && c2 < c);
      rank += before ? 1 : 0;
      rem_before += before ? (count[c2] & (kXcds - 1)) : 0;
    }
    order[rank] = c;
    rot[c] = rem_before & (kXcds - 1);
  }
  __syncthreads();
  const int total = g.B * g.heads * g.n_q;
  const int i = blockIdx.x * kWorkThreads + threadIdx.x;
  if (i >= total) return;
  const int x = i & (kXcds - 1), k = i / kXcds;
  int acc = 0;
  for (int rk = 0; rk < C; ++rk) {
    const int c = order[rk];
    const int n = count[c];
    if (n == 0) continue;
    const int base = n / kXcds, rem = n & (kXcds - 1), r = rot[c];
    const int len = base + ((((x - r) & (kXcds - 1)) < rem) ? 1 : 0);
    if (k < acc + len) {
      int before = 0;
      for (int x2 = 0; x2 < x; ++x2) before += (((x2 - r) & (kXcds - 1)) < rem) ? 1 : 0;
      const int idx = x * base + before + (k - acc);
      const int hd = c >> 1;
      int unit;
      if ((c & 1) == 0) {
        const int b = idx / g.n_tiles, qt = idx % g.n_tiles;
        unit = (b * g.heads + hd) * g.n_q + qt;
      } else {
        const int b = idx / g.text_parts, part = idx % g.text_parts;
        unit = (b * g.heads + hd) * g.n_q + g.n_tiles + part;
      }
      work[i] = unit;
      return;
    }
    acc += len;
  }
}

}  // namespace

hipError_t launch_schedule_lists(const Geom& g, const Windows& win, int32_t* offsets,
                                 int32_t* ids, hipStream_t stream) {
  dim3 grid(g.n_q, g.heads);
  schedule_lists_kernel<<<grid, 256, 0, stream>>>(g, win, offsets, ids);
  return hipGetLastError();
}

hipError_t launch_schedule_work(const Geom& g, const Windows& win, int32_t* work,
                                int32_t* claim, void* zero_row, hipStream_t stream) {
  const int total = g.B * g.heads * g.n_q;
  dim3 grid((total + kWorkThreads - 1) / kWorkThreads);
  schedule_work_kernel<<<grid, kWorkThreads, 0, stream>>>(g, win, work, claim,
                                                           static_cast<int32_t*>(zero_row));
  return hipGetLastError();
}

}  // namespace sta
