// Host side of the STA C ABI (include/sta.h): argument validation, geometry,
// workspace carving and the launch sequence on the caller's stream.
//
// Validation is plain C++ and runs before any HIP call, so argument errors
// are reported synchronously and can be exercised without a GPU.
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/sta.h"
#include "sta_internal.h"

namespace {

using sta::Geom;
using sta::Windows;

constexpr size_t kAlign = 256;
// smallest Hilbert slide window (in tiles) run with six-tile query units
constexpr int kHilbertGroup6Window = 6;
// Text units of grouped calls: at most this many, each with at least this many key tiles
constexpr int kHilbertTextParts = 8;
constexpr int kHilbertTextPartTiles = 128;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// STA_LOG set (and not "0") in the environment: every forward and backward
// call prints its derived schedule to stderr before it enqueues anything.
bool log_enabled() {
  static const bool on = [] {
    const char* e = std::getenv("STA_LOG");
    return e != nullptr && e[0] != '\0' && std::strcmp(e, "0") != 0;
  }();
  return on;
}

// One line: the call, its geometry, the query units and their kind, the
// window of head 0 and how many heads have other windows, the workspace.
void log_schedule(const char* call, const sta::Geom& g, const sta::Windows& win, int64_t units_per_head,
                  size_t workspace) {
  if (!log_enabled()) return;
  const char* kind = g.hilbert == sta::kSquareUnits ? "2x2-square"
                     : g.hilbert != 0               ? "hilbert"
                                                    : "single-tile";
  int other = 0;
  for (int h = 1; h < g.heads; ++h) other += win.w[h] != win.w[0] ? 1 : 0;
  std::fprintf(stderr,
               "[sta] %s: B=%d heads=%d D=%d video=(%d,%d,%d) tiles=(%d,%d,%d)=%d text=%d/%d S=%d "
               "units/head=%lld (%s%s, text parts %d) window[0]=(%d,%d,%d) heads with another window=%d "
               "workspace=%zu bytes\n",
               call, g.B, g.heads, g.D, g.T, g.H, g.W, g.nt, g.nh, g.nw, g.n_tiles, g.text_length,
               g.has_text ? 256 : 0, g.S, static_cast<long long>(units_per_head), kind,
               g.full ? "" : ", partial tiles", g.text_parts, sta::win_t(win.w[0]), sta::win_h(win.w[0]),
               sta::win_w(win.w[0]), other, workspace);
}

sta_status make_geom(const sta_dims* d, int32_t has_text, int32_t text_length, Geom* g) {
  if (d == nullptr) return STA_ERR_NULL;
  if (d->batch <= 0 || d->heads <= 0) return STA_ERR_NULL;
  if (d->heads > STA_MAX_HEADS) return STA_ERR_SHAPE;
  if (d->head_dim != 64 && d->head_dim != 128) return STA_ERR_SHAPE;
  if (d->T <= 0 || d->H <= 0 || d->W <= 0) return STA_ERR_SHAPE;
  // sizes that are not tile multiples are covered by the same tile grid, the
  // last tile along an axis holding the remainder
  const int64_t nt = (d->T + sta::kTileT - 1) / sta::kTileT;
  const int64_t nh = (d->H + sta::kTileH - 1) / sta::kTileH;
  const int64_t nw = (d->W + sta::kTileW - 1) / sta::kTileW;
  if (nt > 1023 || nh > 1023 || nw > 1023) return STA_ERR_SHAPE;
  // tile decoding divides tile indices by nw and nh with 32-bit reciprocals
  if (nt * nh * nw * (nh > nw ? nh : nw) >= (int64_t(1) << 32)) return STA_ERR_SHAPE;
  const int64_t n_video = int64_t(d->T) * d->H * d->W;
  const int64_t S = n_video + (has_text ? STA_TEXT_SLOTS : 0);
  const int64_t n_vt = nt * nh * nw * sta::kTileRows;
  const int64_t S_t = n_vt + (has_text ? STA_TEXT_SLOTS : 0);
  // per-slab element offsets and row indices are 32-bit inside the kernels
  if (S_t * d->head_dim >= (int64_t(1) << 31)) return STA_ERR_SHAPE;
  const int64_t n_q = nt * nh * nw + (has_text ? 1 : 0);
  if (int64_t(d->batch) * d->heads * n_q >= (int64_t(1) << 31)) return STA_ERR_SHAPE;
  if (int64_t(d->batch) * d->heads * (S_t / sta::kKeyBlock) >= (int64_t(1) << 31)) return STA_ERR_SHAPE;
  if (has_text) {
    if (text_length < 0 || text_length > STA_TEXT_SLOTS) return STA_ERR_TEXT;
  } else if (text_length != 0) {
    return STA_ERR_TEXT;
  }
  g->B = d->batch;
  g->heads = d->heads;
  g->D = d->head_dim;
  g->T = d->T;
  g->H = d->H;
  g->W = d->W;
  g->nt = int32_t(nt);
  g->nh = int32_t(nh);
  g->nw = int32_t(nw);
  g->n_tiles = int32_t(nt * nh * nw);
  g->n_video = int32_t(n_video);
  g->S = int32_t(S);
  g->n_vt = int32_t(n_vt);
  g->S_t = int32_t(S_t);
  g->full = (n_vt == n_video) ? 1 : 0;
  g->has_text = has_text ? 1 : 0;
  g->text_length = text_length;
  g->n_q = int32_t(n_q);
  auto magic = [](int64_t d) { return d == 1 ? 0u : uint32_t(((int64_t(1) << 32) + d - 1) / d); };
  g->mag_nw = magic(nw);
  g->mag_nh = magic(nh);
  g->hilbert = 0;
  g->hil_m = 0;
  g->hil_group = 1;
  g->text_parts = 1;
  return STA_OK;
}

// Text query rows of a grouped call: they see every key tile, and as one unit
// they would stream all of them alone, longer than the rest of the call on a
// large image. Their keys are split over up to 8 units of at least 128 tiles
// each, merged afterwards.
int32_t grouped_text_parts(const Geom& g) {
  if (!g.has_text) return 1;
  const int parts = g.n_tiles / kHilbertTextPartTiles;
  return parts < 1 ? 1 : parts > kHilbertTextParts ? kHilbertTextParts : parts;
}

// STA on a one-frame video (a 2D image under the one-frame reading): each tile
// holds at most 8x8 tokens, so a single-tile query unit keeps one wave per
// SIMD busy. When every head's window spans at least two tiles along
// each axis that has two tile rows (columns), query units become 2x2 squares
// of tiles (Geom::hilbert = kSquareUnits), whose windows share a non-empty
// core; the text rows are split by key tiles when split_text. Leaves g
// unchanged otherwise.
void plan_square_units(Geom* g, const Windows& win, bool split_text) {
  if (g->T != 1) return;
  if (g->nh < 2 && g->nw < 2) return;
  for (int h = 0; h < g->heads; ++h) {
    const uint32_t p = win.w[h];
    if ((sta::win_h(p) < 2 && g->nh > 1) || (sta::win_w(p) < 2 && g->nw > 1)) return;
  }
  g->hilbert = sta::kSquareUnits;
  g->hil_group = 4;
  g->text_parts = split_text ? grouped_text_parts(*g) : 1;
  g->n_q = ((g->nh + 1) / 2) * ((g->nw + 1) / 2) + (g->has_text ? g->text_parts : 0);
}

// A 2D image for the Hilbert entry points: one frame, square, its side 8 * 2^m
// tokens (a 2^m x 2^m tile grid); sets g->hil_m.
sta_status make_hilbert_geom(const sta_dims* d, int32_t has_text, int32_t text_length, Geom* g) {
  sta_status st = make_geom(d, has_text, text_length, g);
  if (st != STA_OK) return st;
  if (d->T != 1 || d->H != d->W || d->H % sta::kTileH != 0) return STA_ERR_SHAPE;
  const int side = d->H / sta::kTileH;
  if ((side & (side - 1)) != 0) return STA_ERR_SHAPE;
  int m = 0;
  while ((1 << m) < side) ++m;
  g->hil_m = m;
  g->text_parts = grouped_text_parts(*g);
  // the most query units any grouping gives (single tiles); sizes the workspace
  g->n_q = g->n_tiles + (g->has_text ? g->text_parts : 0);
  return STA_OK;
}

// Hilbert windows: one length per head in [1, min(n_tiles, 1023)] tiles, kept
// as the w component of a (1, 1, W) window (which also prices the work order).
sta_status make_hilbert_windows(const Geom& g, const int32_t* lens, int32_t mode, Windows* win) {
  if (lens == nullptr) return STA_ERR_NULL;
  if (mode != STA_HILBERT_SLIDE && mode != STA_HILBERT_WINDOW) return STA_ERR_WINDOW;
  std::memset(win, 0, sizeof(*win));
  for (int h = 0; h < g.heads; ++h) {
    const int32_t w = lens[h];
    if (w < 1 || w > g.n_tiles || w > 1023) return STA_ERR_WINDOW;
    win->w[h] = 1u | (1u << 10) | (uint32_t(w) << 20);
  }
  return STA_OK;
}

sta_status make_windows(const Geom& g, const int32_t* ws, Windows* win, int64_t* n_ids) {
  if (ws == nullptr) return STA_ERR_NULL;
  int64_t total = 0;
  std::memset(win, 0, sizeof(*win));
  for (int h = 0; h < g.heads; ++h) {
    const int32_t wt = ws[3 * h], wh = ws[3 * h + 1], ww = ws[3 * h + 2];
    if (wt < 1 || wt > g.nt || wh < 1 || wh > g.nh || ww < 1 || ww > g.nw) return STA_ERR_WINDOW;
    win->w[h] = uint32_t(wt) | (uint32_t(wh) << 10) | (uint32_t(ww) << 20);
    total += int64_t(g.n_tiles) * wt * wh * ww + (g.has_text ? g.n_tiles : 0);
  }
  if (total >= (int64_t(1) << 31)) return STA_ERR_SHAPE;
  *n_ids = total;
  return STA_OK;
}

// Forward workspace: the work order (one int32 per query unit), the queue
// heads and a zero row (the source of keys that must not contribute).
struct Carve {
  size_t work, claim, zero_row, text_partial, total;
};

Carve carve(const Geom& g) {
  Carve c{};
  size_t at = 0;
  c.work = at; at = align_up(at + size_t(g.B) * g.heads * g.n_q * 4);
  c.claim = at; at = align_up(at + size_t(sta::kClaimInts) * 4);
  c.zero_row = at; at = align_up(at + size_t(sta::kZeroRowBytes));
  // partial results of split text units (FwdArgs::text_partial)
  c.text_partial = at;
  if (g.text_parts > 1)
    at = align_up(at + size_t(g.B) * g.heads * g.text_parts * STA_TEXT_SLOTS * (g.D + 2) * 4);
  c.total = at;
  return c;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

sta_status hip_status(hipError_t e) { return e == hipSuccess ? STA_OK : STA_ERR_HIP; }

}  // namespace

extern "C" {

const char* sta_status_str(sta_status s) {
  switch (s) {
    case STA_OK: return "STA_OK";
    case STA_ERR_NULL: return "STA_ERR_NULL: NULL pointer or non-positive batch/heads";
    case STA_ERR_SHAPE: return "STA_ERR_SHAPE: unsupported video size, head_dim, head count or size";
    case STA_ERR_WINDOW: return "STA_ERR_WINDOW: window component outside [1, tiles on that axis]";
    case STA_ERR_TEXT: return "STA_ERR_TEXT: text_length outside [0, 256] or non-zero without text";
    case STA_ERR_ALIGN: return "STA_ERR_ALIGN: device pointer not 16-byte aligned";
    case STA_ERR_WORKSPACE: return "STA_ERR_WORKSPACE: workspace missing or too small";
    case STA_ERR_HIP: return "STA_ERR_HIP: HIP runtime error at launch";
    case STA_ERR_ALIAS: return "STA_ERR_ALIAS: output overlaps an input";
    case STA_ERR_SCRATCH:
      return "STA_ERR_SCRATCH: the shape needs more workspace than sta_forward_noalloc's fixed scratch";
  }
  return "STA_ERR_UNKNOWN";
}

int64_t sta_seq_len(const sta_dims* dims, int32_t has_text) {
  Geom g;
  if (make_geom(dims, has_text, 0, &g) != STA_OK) return 0;
  return g.S;
}

int64_t sta_tiled_seq_len(const sta_dims* dims, int32_t has_text) {
  Geom g;
  if (make_geom(dims, has_text, 0, &g) != STA_OK) return 0;
  return g.S_t;
}

size_t sta_workspace_bytes(const sta_dims* dims, const int32_t* window_sizes, int32_t has_text) {
  Geom g;
  if (make_geom(dims, has_text, 0, &g) != STA_OK) return 0;
  Windows win;
  int64_t n_ids = 0;
  if (make_windows(g, window_sizes, &win, &n_ids) != STA_OK) return 0;
  plan_square_units(&g, win, true);
  return carve(g).total;
}

sta_status sta_schedule_sizes(const sta_dims* dims, const int32_t* window_sizes, int32_t has_text,
                              int64_t* n_offsets, int64_t* n_ids, int64_t* n_work) {
  Geom g;
  sta_status st = make_geom(dims, has_text, 0, &g);
  if (st != STA_OK) return st;
  if (n_offsets == nullptr || n_ids == nullptr || n_work == nullptr) return STA_ERR_NULL;
  Windows win;
  int64_t ids = 0;
  st = make_windows(g, window_sizes, &win, &ids);
  if (st != STA_OK) return st;
  *n_offsets = int64_t(g.heads) * g.n_q + 1;
  *n_ids = ids;
  *n_work = int64_t(g.B) * g.heads * g.n_q;
  return STA_OK;
}

sta_status sta_build_schedule(const sta_dims* dims, const int32_t* window_sizes, int32_t text_length,
                              int32_t has_text, int32_t* offsets, int32_t* ids, int32_t* work,
                              void* stream) {
  Geom g;
  sta_status st = make_geom(dims, has_text, text_length, &g);
  if (st != STA_OK) return st;
  Windows win;
  int64_t n_ids = 0;
  st = make_windows(g, window_sizes, &win, &n_ids);
  if (st != STA_OK) return st;
  if (offsets == nullptr || ids == nullptr || work == nullptr) return STA_ERR_NULL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  st = hip_status(sta::launch_schedule_lists(g, win, offsets, ids, s));
  if (st != STA_OK) return st;
  return hip_status(sta::launch_schedule_work(g, win, work, nullptr, nullptr, s));
}

sta_status sta_tile_gather(const sta_dims* dims, int32_t has_text, const void* x_raster,
                           void* x_tiled, void* stream) {
  Geom g;
  sta_status st = make_geom(dims, has_text, 0, &g);
  if (st != STA_OK) return st;
  if (x_raster == nullptr || x_tiled == nullptr) return STA_ERR_NULL;
  if (!aligned16(x_raster) || !aligned16(x_tiled)) return STA_ERR_ALIGN;
  const size_t raster_bytes = size_t(g.B) * g.heads * g.S * g.D * 2;
  const size_t tiled_bytes = size_t(g.B) * g.heads * g.S_t * g.D * 2;
  if (overlaps(x_raster, raster_bytes, x_tiled, tiled_bytes)) return STA_ERR_ALIAS;
  return hip_status(sta::launch_rows_permute(g, x_raster, x_tiled, true,
                                             reinterpret_cast<hipStream_t>(stream)));
}

sta_status sta_tile_scatter(const sta_dims* dims, int32_t has_text, const void* x_tiled,
                            void* x_raster, void* stream) {
  Geom g;
  sta_status st = make_geom(dims, has_text, 0, &g);
  if (st != STA_OK) return st;
  if (x_raster == nullptr || x_tiled == nullptr) return STA_ERR_NULL;
  if (!aligned16(x_raster) || !aligned16(x_tiled)) return STA_ERR_ALIGN;
  const size_t raster_bytes = size_t(g.B) * g.heads * g.S * g.D * 2;
  const size_t tiled_bytes = size_t(g.B) * g.heads * g.S_t * g.D * 2;
  if (overlaps(x_raster, raster_bytes, x_tiled, tiled_bytes)) return STA_ERR_ALIAS;
  return hip_status(sta::launch_rows_permute(g, x_tiled, x_raster, false,
                                             reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// The forward's launches for a validated geometry and windows.
sta_status forward_launch(Geom g, const Windows& win, const void* q, const void* k, const void* v,
                          void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream,
                          void* const* events) {
  sta_status st = STA_OK;
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return STA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      (lse != nullptr && !aligned16(lse)))
    return STA_ERR_ALIGN;
  const Carve c = carve(g);
  if (workspace == nullptr || workspace_bytes < c.total) return STA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return STA_ERR_ALIGN;
  const size_t tbytes = size_t(g.B) * g.heads * g.S * g.D * 2;
  const size_t lbytes = size_t(g.B) * g.heads * g.S * 4;
  for (const void* in : {q, k, v, static_cast<const void*>(workspace)}) {
    const size_t n = in == workspace ? c.total : tbytes;
    if (overlaps(out, tbytes, in, n)) return STA_ERR_ALIAS;
    if (lse != nullptr && overlaps(lse, lbytes, in, n)) return STA_ERR_ALIAS;
  }
  if (lse != nullptr && overlaps(lse, lbytes, out, tbytes)) return STA_ERR_ALIAS;
  log_schedule("sta_forward", g, win, g.n_q, c.total);

  char* ws = static_cast<char*>(workspace);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // optional timing events: recorded before the first launch and after each one
  auto mark = [&](int i) -> sta_status {
    if (events == nullptr) return STA_OK;
    return hip_status(hipEventRecord(reinterpret_cast<hipEvent_t>(events[i]), s));
  };
  st = mark(0);
  if (st != STA_OK) return st;
  int32_t* work = reinterpret_cast<int32_t*>(ws + c.work);
  int32_t* claim = reinterpret_cast<int32_t*>(ws + c.claim);
  // the work order counts query units: with grouped units, a head has
  // n_q - text_parts video units
  Geom gs = g;
  if (g.hilbert != 0) gs.n_tiles = g.n_q - (g.has_text ? g.text_parts : 0);
  st = hip_status(sta::launch_schedule_work(gs, win, work, claim, ws + c.zero_row, s));
  if (st == STA_OK) st = mark(1);
  if (st != STA_OK) return st;
  sta::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.work = work;
  a.claim = claim;
  a.zero_row = ws + c.zero_row;
  a.text_partial = g.text_parts > 1 ? reinterpret_cast<float*>(ws + c.text_partial) : nullptr;
  a.q_scale = float(1.4426950408889634 / std::sqrt(double(g.D)));  // log2(e)/sqrt(D)
  st = hip_status(sta::launch_attention(g, win, a, s));
  if (st == STA_OK) st = mark(2);
  return st;
}

// split_text: grouped calls may split their text rows (sta_forward_noalloc
// keeps them whole when its scratch cannot hold the partial results)
sta_status forward_impl(const sta_dims* dims, const void* q, const void* k, const void* v,
                        const int32_t* window_sizes, int32_t text_length, int32_t has_text,
                        void* out, float* lse, void* workspace, size_t workspace_bytes,
                        void* stream, void* const* events, bool split_text = true) {
  Geom g;
  sta_status st = make_geom(dims, has_text, text_length, &g);
  if (st != STA_OK) return st;
  Windows win;
  int64_t n_ids = 0;
  st = make_windows(g, window_sizes, &win, &n_ids);
  if (st != STA_OK) return st;
  plan_square_units(&g, win, split_text);
  return forward_launch(g, win, q, k, v, out, lse, workspace, workspace_bytes, stream, events);
}

}  // namespace

extern "C" {

sta_status sta_forward(const sta_dims* dims, const void* q, const void* k, const void* v,
                       const int32_t* window_sizes, int32_t text_length, int32_t has_text,
                       void* out, float* lse, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return forward_impl(dims, q, k, v, window_sizes, text_length, has_text, out, lse, workspace,
                      workspace_bytes, stream, nullptr);
}

sta_status sta_forward_timed(const sta_dims* dims, const void* q, const void* k, const void* v,
                             const int32_t* window_sizes, int32_t text_length, int32_t has_text,
                             void* out, float* lse, void* workspace, size_t workspace_bytes,
                             void* stream, void* const* events) {
  if (events == nullptr) return STA_ERR_NULL;
  for (int i = 0; i < STA_TIMED_EVENTS; ++i)
    if (events[i] == nullptr) return STA_ERR_NULL;
  return forward_impl(dims, q, k, v, window_sizes, text_length, has_text, out, lse, workspace,
                      workspace_bytes, stream, events);
}

}  // extern "C"

// ------------------------------------------------- Hilbert-window attention
extern "C" {

size_t sta_hilbert_workspace_bytes(const sta_dims* dims, int32_t has_text) {
  Geom g;
  if (make_hilbert_geom(dims, has_text, 0, &g) != STA_OK) return 0;
  return carve(g).total;
}

sta_status sta_hilbert_forward(const sta_dims* dims, const void* q, const void* k, const void* v,
                               const int32_t* window_lens, int32_t mode, int32_t text_length,
                               int32_t has_text, void* out, float* lse, void* workspace,
                               size_t workspace_bytes, void* stream) {
  Geom g;
  sta_status st = make_hilbert_geom(dims, has_text, text_length, &g);
  if (st != STA_OK) return st;
  Windows win;
  st = make_hilbert_windows(g, window_lens, mode, &win);
  if (st != STA_OK) return st;
  g.hilbert = mode;
  // Query units of several consecutive curve positions when every head's
  // windows allow it. Slide windows of at least kHilbertGroup6Window tiles: six
  // positions (384 rows, the shape of a video tile unit; their windows share a
  // core of at least W - 5 tiles, and the last unit of a head holds what is
  // left). Slide windows of at least 4 tiles, or windows of a multiple of 4
  // tiles: four (an aligned 2x2 square of tiles, 256 rows; slide windows then
  // share a core, fixed windows are the same for the four). Single tiles
  // otherwise.
  bool group4 = g.n_tiles % 4 == 0, group6 = mode == STA_HILBERT_SLIDE;
  for (int h = 0; h < g.heads; ++h) {
    const int w = window_lens[h];
    group4 = group4 && (mode == STA_HILBERT_SLIDE ? w >= 4 : w % 4 == 0);
    group6 = group6 && w >= kHilbertGroup6Window;
  }
  g.hil_group = group6 ? 6 : group4 ? 4 : 1;
  g.n_q = (g.n_tiles + g.hil_group - 1) / g.hil_group + (g.has_text ? g.text_parts : 0);
  return forward_launch(g, win, q, k, v, out, lse, workspace, workspace_bytes, stream, nullptr);
}

namespace {
sta_status hilbert_rows(const sta_dims* dims, int32_t has_text, const void* src, void* dst, bool to_hilbert,
                        void* stream) {
  Geom g;
  sta_status st = make_hilbert_geom(dims, has_text, 0, &g);
  if (st != STA_OK) return st;
  if (src == nullptr || dst == nullptr) return STA_ERR_NULL;
  if (!aligned16(src) || !aligned16(dst)) return STA_ERR_ALIGN;
  const size_t bytes = size_t(g.B) * g.heads * g.S * g.D * 2;
  if (overlaps(src, bytes, dst, bytes)) return STA_ERR_ALIAS;
  return hip_status(sta::launch_rows_hilbert(g, src, dst, to_hilbert, reinterpret_cast<hipStream_t>(stream)));
}
}  // namespace

sta_status sta_hilbert_gather(const sta_dims* dims, int32_t has_text, const void* x_raster,
                              void* x_hilbert, void* stream) {
  return hilbert_rows(dims, has_text, x_raster, x_hilbert, true, stream);
}

sta_status sta_hilbert_scatter(const sta_dims* dims, int32_t has_text, const void* x_hilbert,
                               void* x_raster, void* stream) {
  return hilbert_rows(dims, has_text, x_hilbert, x_raster, false, stream);
}

}  // extern "C"

// ------------------------------------------- forward without a workspace
namespace {

// (Plain C++ builds of this file, which check the host logic with the HIP
// calls stubbed, lack the HIP compiler's spellings of these two.)
#ifndef __align__
#define __align__(n) __attribute__((aligned(n)))
#endif
#ifndef HIP_SYMBOL
#define HIP_SYMBOL(x) x
#endif

// The workspace of sta_forward_noalloc: a fixed array in device memory, one
// per GPU. In host code `scratch` is only a stand-in for the symbol; its
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) char scratch[STA_NOALLOC_SCRATCH_BYTES];
constexpr int kScratchDevices = 64;
std::atomic<void*> g_scratch_addr[kScratchDevices];

sta_status scratch_address(void** addr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return STA_ERR_HIP;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // the current device is the one the array's address is taken on
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return STA_ERR_HIP;
    g_scratch_addr[dev].store(p, std::memory_order_release);
  }
  *addr = p;
  return STA_OK;
}

}  // namespace

extern "C" {

sta_status sta_forward_noalloc(const sta_dims* dims, const void* q, const void* k, const void* v,
                               const int32_t* window_sizes, int32_t text_length, int32_t has_text,
                               void* out, float* lse, void* stream) {
  Geom g;
  sta_status st = make_geom(dims, has_text, text_length, &g);
  if (st != STA_OK) return st;
  Windows win;
  int64_t n_ids = 0;
  st = make_windows(g, window_sizes, &win, &n_ids);
  if (st != STA_OK) return st;
  // square units with split text rows when their partial results fit the
  // scratch, else with whole text units
  Geom gs = g;
  plan_square_units(&gs, win, true);
  const bool split_text = carve(gs).total <= STA_NOALLOC_SCRATCH_BYTES;
  plan_square_units(&g, win, false);
  if (carve(g).total > STA_NOALLOC_SCRATCH_BYTES) return STA_ERR_SCRATCH;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != STA_OK) return st;
  return forward_impl(dims, q, k, v, window_sizes, text_length, has_text, out, lse, ws,
                      STA_NOALLOC_SCRATCH_BYTES, stream, nullptr, split_text);
}

}  // extern "C"

// ---------------------------------------------------------------- backward
namespace {

struct BwdCarve {
  size_t lse2, delta, offsets, ids, claim_q, claim_kv, zero_row, total;
};

BwdCarve bwd_carve(const Geom& g, int64_t n_ids) {
  BwdCarve c{};
  const size_t rows = size_t(g.B) * g.heads * g.S_t * 4;  // tile-major rows
  size_t at = 0;
  c.lse2 = at; at = align_up(at + rows);
  c.delta = at; at = align_up(at + rows);
  c.offsets = at; at = align_up(at + (size_t(g.heads) * g.n_q + 1) * 4);
  c.ids = at; at = align_up(at + size_t(n_ids) * 4);
  c.claim_q = at; at = align_up(at + size_t(sta::kClaimInts) * 4);
  c.claim_kv = at; at = align_up(at + size_t(sta::kClaimInts) * 4);
  c.zero_row = at; at = align_up(at + size_t(sta::kZeroRowBytes));
  c.total = at;
  return c;
}

sta_status backward_impl(const sta_dims* dims, const void* q, const void* k, const void* v,
                         const void* out, const float* lse, const void* dout,
                         const int32_t* window_sizes, int32_t text_length, int32_t has_text,
                         void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                         void* stream, void* const* events) {
  Geom g;
  sta_status st = make_geom(dims, has_text, text_length, &g);
  if (st != STA_OK) return st;
  // key units (3 per tile, 2 for the text slots) are numbered in 32 bits
  if (int64_t(g.B) * g.heads * (3 * int64_t(g.n_tiles) + 2) >= (int64_t(1) << 31)) return STA_ERR_SHAPE;
  Windows win;
  int64_t n_ids = 0;
  st = make_windows(g, window_sizes, &win, &n_ids);
  if (st != STA_OK) return st;
  for (const void* p : {q, k, v, out, static_cast<const void*>(lse), dout,
                        static_cast<const void*>(dq), static_cast<const void*>(dk),
                        static_cast<const void*>(dv)})
    if (p == nullptr) return STA_ERR_NULL;
  for (const void* p : {q, k, v, out, static_cast<const void*>(lse), dout,
                        static_cast<const void*>(dq), static_cast<const void*>(dk),
                        static_cast<const void*>(dv)})
    if (!aligned16(p)) return STA_ERR_ALIGN;
  const BwdCarve c = bwd_carve(g, n_ids);
  if (workspace == nullptr || workspace_bytes < c.total) return STA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return STA_ERR_ALIGN;
  const size_t tbytes = size_t(g.B) * g.heads * g.S * g.D * 2;
  const size_t lbytes = size_t(g.B) * g.heads * g.S * 4;
  const void* ins[] = {q, k, v, out, lse, dout, workspace};
  const size_t in_n[] = {tbytes, tbytes, tbytes, tbytes, lbytes, tbytes, c.total};
  void* outs[] = {dq, dk, dv};
  for (int o = 0; o < 3; ++o) {
    for (int i = 0; i < 7; ++i)
      if (overlaps(outs[o], tbytes, ins[i], in_n[i])) return STA_ERR_ALIAS;
    for (int o2 = o + 1; o2 < 3; ++o2)
      if (overlaps(outs[o], tbytes, outs[o2], tbytes)) return STA_ERR_ALIAS;
  }
  // one-frame videos whose windows allow the forward's 2x2-square units: the
  // dq pass uses them too (Geom::hilbert marks it; the key lists, indexed by
  // n_q, stay those of single tiles for the dk/dv pass)
  {
    Geom gs = g;
    plan_square_units(&gs, win, false);
    if (gs.hilbert == sta::kSquareUnits) g.hilbert = sta::kSquareUnits;
  }
  // dq units: two parts per tile, or one square of tiles, (+ the text slots)
  log_schedule("sta_backward", g, win,
               g.hilbert == sta::kSquareUnits ? int64_t((g.nh + 1) / 2) * ((g.nw + 1) / 2) + (g.has_text ? 1 : 0)
                                              : 2 * int64_t(g.n_tiles) + (g.has_text ? 1 : 0),
               c.total);

  char* ws = static_cast<char*>(workspace);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  auto mark = [&](int i) -> sta_status {
    if (events == nullptr) return STA_OK;
    return hip_status(hipEventRecord(reinterpret_cast<hipEvent_t>(events[i]), s));
  };
  sta::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.zero_row = ws + c.zero_row;
  a.lse2 = reinterpret_cast<float*>(ws + c.lse2);
  a.delta = reinterpret_cast<float*>(ws + c.delta);
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + c.offsets);
  int32_t* ids = reinterpret_cast<int32_t*>(ws + c.ids);
  a.offsets = offsets;
  a.ids = ids;
  a.claim_q = reinterpret_cast<int32_t*>(ws + c.claim_q);
  a.claim_kv = reinterpret_cast<int32_t*>(ws + c.claim_kv);
  a.q_scale = float(1.4426950408889634 / std::sqrt(double(g.D)));  // log2(e)/sqrt(D)
  a.scale = float(1.0 / std::sqrt(double(g.D)));

  st = mark(0);
  if (st == STA_OK)
    st = hip_status(sta::launch_bwd_prep(g, out, dout, lse, reinterpret_cast<float*>(ws + c.lse2),
                                         reinterpret_cast<float*>(ws + c.delta), a.claim_q,
                                         a.claim_kv, ws + c.zero_row, s));
  if (st == STA_OK) st = mark(1);
  if (st == STA_OK) st = hip_status(sta::launch_schedule_lists(g, win, offsets, ids, s));
  if (st == STA_OK) st = mark(2);
  if (st == STA_OK) st = hip_status(sta::launch_bwd_dq(g, win, a, s));
  if (st == STA_OK) st = mark(3);
  if (st == STA_OK) st = hip_status(sta::launch_bwd_dkv(g, win, a, s));
  if (st == STA_OK) st = mark(4);
  return st;
}

}  // namespace

extern "C" {

size_t sta_backward_workspace_bytes(const sta_dims* dims, const int32_t* window_sizes,
                                    int32_t has_text) {
  Geom g;
  if (make_geom(dims, has_text, 0, &g) != STA_OK) return 0;
  Windows win;
  int64_t n_ids = 0;
  if (make_windows(g, window_sizes, &win, &n_ids) != STA_OK) return 0;
  return bwd_carve(g, n_ids).total;
}

sta_status sta_backward(const sta_dims* dims, const void* q, const void* k, const void* v,
                        const void* out, const float* lse, const void* dout,
                        const int32_t* window_sizes, int32_t text_length, int32_t has_text,
                        void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                        void* stream) {
  return backward_impl(dims, q, k, v, out, lse, dout, window_sizes, text_length, has_text, dq, dk,
                       dv, workspace, workspace_bytes, stream, nullptr);
}

sta_status sta_backward_timed(const sta_dims* dims, const void* q, const void* k, const void* v,
                              const void* out, const float* lse, const void* dout,
                              const int32_t* window_sizes, int32_t text_length, int32_t has_text,
                              void* dq, void* dk, void* dv, void* workspace,
                              size_t workspace_bytes, void* stream, void* const* events) {
  if (events == nullptr) return STA_ERR_NULL;
  for (int i = 0; i < STA_BWD_TIMED_EVENTS; ++i)
    if (events[i] == nullptr) return STA_ERR_NULL;
  return backward_impl(dims, q, k, v, out, lse, dout, window_sizes, text_length, has_text, dq, dk,
                       dv, workspace, workspace_bytes, stream, events);
}

}  // extern "C"
