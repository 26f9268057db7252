// Host side of the STA C ABI (include/sta.h): argument validation, geometry,
// workspace carving and the launch sequence on the caller's stream.
//
// Validation is plain C++ and runs before any HIP call, so argument errors
// are reported synchronously and can be exercised without a GPU.
#include <cmath>
#include <cstring>

#include "../../include/sta.h"
#include "sta_internal.h"

namespace {

using sta::Geom;
using sta::Windows;

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

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

struct Carve {
  size_t vt, offsets, ids, work, claim, total;
};

Carve carve(const Geom& g, int64_t n_ids) {
  Carve c{};
  const size_t tensor = size_t(g.B) * g.heads * g.S_t * g.D * 2;  // packed, tile-major
  size_t at = 0;
  c.vt = at; at = align_up(at + tensor);
  c.offsets = at; at = align_up(at + (size_t(g.heads) * g.n_q + 1) * 4);
  c.ids = at; at = align_up(at + size_t(n_ids) * 4);
  c.work = at; at = align_up(at + size_t(g.B) * g.heads * g.n_q * 4);
  c.claim = at; at = align_up(at + size_t(sta::kClaimInts) * 4);
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
  return carve(g, n_ids).total;
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
  return hip_status(sta::launch_schedule_work(g, win, work, nullptr, s));
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

sta_status forward_impl(const sta_dims* dims, const void* q, const void* k, const void* v,
                        const int32_t* window_sizes, int32_t text_length, int32_t has_text,
                        void* out, float* lse, void* workspace, size_t workspace_bytes,
                        void* stream, void* const* events) {
  Geom g;
  sta_status st = make_geom(dims, has_text, text_length, &g);
  if (st != STA_OK) return st;
  Windows win;
  int64_t n_ids = 0;
  st = make_windows(g, window_sizes, &win, &n_ids);
  if (st != STA_OK) return st;
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return STA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      (lse != nullptr && !aligned16(lse)))
    return STA_ERR_ALIGN;
  const Carve c = carve(g, n_ids);
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

  char* ws = static_cast<char*>(workspace);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // optional timing events: recorded before the first launch and after each one
  auto mark = [&](int i) -> sta_status {
    if (events == nullptr) return STA_OK;
    return hip_status(hipEventRecord(reinterpret_cast<hipEvent_t>(events[i]), s));
  };
  st = mark(0);
  if (st != STA_OK) return st;
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + c.offsets);
  int32_t* ids = reinterpret_cast<int32_t*>(ws + c.ids);
  int32_t* work = reinterpret_cast<int32_t*>(ws + c.work);
  int32_t* claim = reinterpret_cast<int32_t*>(ws + c.claim);

  st = hip_status(sta::launch_pack_v(g, v, ws + c.vt, s));
  if (st == STA_OK) st = mark(1);
  if (st != STA_OK) return st;
  st = hip_status(sta::launch_schedule_lists(g, win, offsets, ids, s));
  if (st == STA_OK) st = mark(2);
  if (st != STA_OK) return st;
  st = hip_status(sta::launch_schedule_work(g, win, work, claim, s));
  if (st == STA_OK) st = mark(3);
  if (st != STA_OK) return st;
  sta::FwdArgs a;
  a.q = q;
  a.k = k;
  a.vt = ws + c.vt;
  a.out = out;
  a.lse = lse;
  a.offsets = offsets;
  a.ids = ids;
  a.work = work;
  a.claim = claim;
  a.q_scale = float(1.4426950408889634 / std::sqrt(double(g.D)));  // log2(e)/sqrt(D)
  st = hip_status(sta::launch_attention(g, win, a, s));
  if (st == STA_OK) st = mark(4);
  return st;
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

// ---------------------------------------------------------------- backward
namespace {

struct BwdCarve {
  size_t kt, qt, dot, lse2, delta, offsets, ids, claim_q, claim_kv, total;
};

BwdCarve bwd_carve(const Geom& g, int64_t n_ids) {
  BwdCarve c{};
  const size_t tensor = size_t(g.B) * g.heads * g.S_t * g.D * 2;  // packed, tile-major
  const size_t rows = size_t(g.B) * g.heads * g.S_t * 4;          // tile-major rows
  size_t at = 0;
  c.kt = at; at = align_up(at + tensor);
  c.qt = at; at = align_up(at + tensor);
  c.dot = at; at = align_up(at + tensor);
  c.lse2 = at; at = align_up(at + rows);
  c.delta = at; at = align_up(at + rows);
  c.offsets = at; at = align_up(at + (size_t(g.heads) * g.n_q + 1) * 4);
  c.ids = at; at = align_up(at + size_t(n_ids) * 4);
  c.claim_q = at; at = align_up(at + size_t(sta::kClaimInts) * 4);
  c.claim_kv = at; at = align_up(at + size_t(sta::kClaimInts) * 4);
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
  a.kt = ws + c.kt;
  a.qt = ws + c.qt;
  a.dot = ws + c.dot;
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
                                         a.claim_kv, s));
  if (st == STA_OK) st = mark(1);
  if (st == STA_OK)
    st = hip_status(sta::launch_pack_rows(g, k, ws + c.kt, g.n_vt + (g.has_text ? g.text_length : 0), s));
  if (st == STA_OK) st = hip_status(sta::launch_pack_rows(g, q, ws + c.qt, g.S_t, s));
  if (st == STA_OK) st = hip_status(sta::launch_pack_rows(g, dout, ws + c.dot, g.S_t, s));
  if (st == STA_OK) st = mark(2);
  if (st == STA_OK) st = hip_status(sta::launch_schedule_lists(g, win, offsets, ids, s));
  if (st == STA_OK) st = mark(3);
  if (st == STA_OK) st = hip_status(sta::launch_bwd_dq(g, win, a, s));
  if (st == STA_OK) st = mark(4);
  if (st == STA_OK) st = hip_status(sta::launch_bwd_dkv(g, win, a, s));
  if (st == STA_OK) st = mark(5);
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
