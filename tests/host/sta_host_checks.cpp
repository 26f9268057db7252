// Host-only checks of the STA library's host code (argument validation,
// geometry, workspace carving, the launch sequence) and of the index helpers
// that its kernels share with the host. tests/test_host_sanitized.py builds
// this file together with the library's host source under AddressSanitizer
// and UndefinedBehaviorSanitizer with the host C++ compiler. No GPU and no
// HIP runtime take part: the kernel launchers and hipEventRecord are replaced
// by stubs that record their arguments, and no "device" pointer is ever
// dereferenced (the fake addresses used here are only compared).
//
//   sta_host_checks validate
//       self-checking cases; prints "ok <n>" and exits 0, or names the first
//       failing case and exits 1
//   sta_host_checks dump <B> <heads> <D> <T> <H> <W> <has_text> <ell> <wt> <wh> <ww>
//       prints the helpers' values for one geometry (every head gets the
//       window (wt, wh, ww)); the Python test compares them with maps built
//       from the oracle's token coordinates
//   sta_host_checks hcurve <k> | hstream <side> <has_text> <ell> <W> <mode>
//       the Hilbert curve and the Hilbert units' key streams (compared with
//       the Hilbert oracle by the Python test)
//   sta_host_checks stream <T> <H> <W> <has_text> <ell> <wt> <wh> <ww>
//       checks the forward kernel's key stream of every query unit and prints
//       its key rows (compared with the oracle's mask by the Python test)
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/sta.h"
#include "../../block_sparse_sliding_amd/csrc/sta_internal.h"

namespace {

struct Launch {
  std::string name;
  std::vector<uintptr_t> ptrs;  // pointer arguments, in declaration order
  sta::Geom g;
};
std::vector<Launch> g_launches;
int g_events = 0;

uintptr_t P(const void* p) { return reinterpret_cast<uintptr_t>(p); }
void record(const char* name, const sta::Geom& g, std::vector<uintptr_t> ptrs) {
  g_launches.push_back(Launch{name, std::move(ptrs), g});
}

}  // namespace

// ---- stubs for the device side of the library
extern "C" hipError_t hipEventRecord(hipEvent_t, hipStream_t) {
  ++g_events;
  return hipSuccess;
}
// the no-workspace forward's scratch: one fake device address, looked up once
int g_symbol_lookups = 0;
extern "C" hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}
extern "C" hipError_t hipGetSymbolAddress(void** p, const void*) {
  ++g_symbol_lookups;
  *p = reinterpret_cast<void*>(uintptr_t(40) * 64 * (uintptr_t(1) << 30));
  return hipSuccess;
}

namespace sta {
hipError_t launch_rows_permute(const Geom& g, const void* src, void* dst, bool, hipStream_t) {
  record("rows_permute", g, {P(src), P(dst)});
  return hipSuccess;
}
hipError_t launch_rows_hilbert(const Geom& g, const void* src, void* dst, bool, hipStream_t) {
  record("rows_hilbert", g, {P(src), P(dst)});
  return hipSuccess;
}
hipError_t launch_schedule_lists(const Geom& g, const Windows&, int32_t* offsets, int32_t* ids,
                                 hipStream_t) {
  record("schedule_lists", g, {P(offsets), P(ids)});
  return hipSuccess;
}
hipError_t launch_schedule_work(const Geom& g, const Windows&, int32_t* work, int32_t* claim,
                                void* zero_row, hipStream_t) {
  record("schedule_work", g, {P(work), P(claim), P(zero_row)});
  return hipSuccess;
}
hipError_t launch_attention(const Geom& g, const Windows&, const FwdArgs& a, hipStream_t) {
  record("attention", g, {P(a.q), P(a.k), P(a.v), P(a.out), P(a.lse), P(a.work), P(a.claim),
                          P(a.zero_row), P(a.text_partial)});
  return hipSuccess;
}
hipError_t launch_bwd_prep(const Geom& g, const void* out, const void* dout, const float* lse,
                           float* lse2, float* delta, int32_t* claim_q, int32_t* claim_kv,
                           void* zero_row, hipStream_t) {
  record("bwd_prep", g, {P(out), P(dout), P(lse), P(lse2), P(delta), P(claim_q), P(claim_kv), P(zero_row)});
  return hipSuccess;
}
hipError_t launch_bwd_dq(const Geom& g, const Windows&, const BwdArgs& a, hipStream_t) {
  record("bwd_dq", g, {P(a.zero_row), P(a.lse2), P(a.delta), P(a.offsets), P(a.ids), P(a.claim_q),
                       P(a.claim_kv)});
  return hipSuccess;
}
hipError_t launch_bwd_dkv(const Geom& g, const Windows&, const BwdArgs& a, hipStream_t) {
  record("bwd_dkv", g, {P(a.zero_row), P(a.lse2), P(a.delta), P(a.offsets), P(a.ids), P(a.claim_q),
                        P(a.claim_kv)});
  return hipSuccess;
}
}  // namespace sta

namespace {

int g_checks = 0;
#define CHECK(cond, ...)                                                     \
  do {                                                                       \
    ++g_checks;                                                              \
    if (!(cond)) {                                                           \
      std::fprintf(stderr, "FAIL %s:%d: %s: ", __FILE__, __LINE__, #cond);   \
      std::fprintf(stderr, __VA_ARGS__);                                     \
      std::fprintf(stderr, "\n");                                            \
      std::exit(1);                                                          \
    }                                                                        \
  } while (0)

// Fake, well-separated, 256-byte aligned "device" addresses (never dereferenced).
constexpr uintptr_t kGiB = uintptr_t(1) << 30;
void* fake(int slot) { return reinterpret_cast<void*>(uintptr_t(slot + 1) * 64 * kGiB); }

std::vector<int32_t> windows_for(int heads, int wt, int wh, int ww) {
  std::vector<int32_t> w;
  for (int h = 0; h < heads; ++h) w.insert(w.end(), {wt, wh, ww});
  return w;
}

sta_status fwd(const sta_dims* d, const int32_t* win, int ell, int text, void* q, void* k, void* v,
               void* out, float* lse, void* ws, size_t ws_bytes, void* const* events = nullptr) {
  g_launches.clear();
  if (events != nullptr)
    return sta_forward_timed(d, q, k, v, win, ell, text, out, lse, ws, ws_bytes, nullptr, events);
  return sta_forward(d, q, k, v, win, ell, text, out, lse, ws, ws_bytes, nullptr);
}

// Every pointer that a launch got which is not one of the caller's tensors
// lies inside the workspace, at a 256-byte aligned offset.
void check_in_workspace(const Launch& l, const std::vector<uintptr_t>& caller, uintptr_t ws,
                        size_t bytes) {
  for (uintptr_t p : l.ptrs) {
    bool is_caller = p == 0;
    for (uintptr_t c : caller) is_caller |= p == c;
    if (is_caller) continue;
    CHECK(p >= ws && p < ws + bytes, "%s: pointer %#zx outside workspace [%#zx, +%zu)",
          l.name.c_str(), size_t(p), size_t(ws), bytes);
    CHECK(((p - ws) & 255) == 0, "%s: workspace offset %zu not 256-aligned", l.name.c_str(),
          size_t(p - ws));
  }
}

void validate() {
  const sta_dims d{1, 2, 128, 30, 48, 80};
  std::vector<int32_t> w = windows_for(2, 3, 3, 3);
  void *q = fake(0), *k = fake(1), *v = fake(2), *out = fake(3), *ws = fake(8);
  float* lse = static_cast<float*>(fake(4));
  const size_t need = sta_workspace_bytes(&d, w.data(), 1);
  CHECK(need > 0, "workspace bytes");

  struct Case {
    const char* what;
    sta_status expect;
    sta_status got;
  };
  std::vector<Case> cases;
  auto add = [&](const char* what, sta_status expect, sta_status got) {
    cases.push_back({what, expect, got});
    CHECK(g_launches.empty(), "%s: launched %zu kernels on a rejected call", what,
          g_launches.size());
  };
  const sta_dims d0{0, 2, 128, 30, 48, 80}, dh0{1, 0, 128, 30, 48, 80}, dd{1, 2, 96, 30, 48, 80};
  const sta_dims dt0{1, 2, 128, 0, 48, 80}, dhn{1, 2, 128, 30, -8, 80};
  const sta_dims dbig{1, 2, 128, 6 * 1024, 8, 8}, dheads{1, 257, 128, 30, 48, 80};
  std::vector<int32_t> w257 = windows_for(257, 1, 1, 1);
  add("null dims", STA_ERR_NULL, fwd(nullptr, w.data(), 226, 1, q, k, v, out, lse, ws, need));
  add("batch 0", STA_ERR_NULL, fwd(&d0, w.data(), 226, 1, q, k, v, out, lse, ws, need));
  add("heads 0", STA_ERR_NULL, fwd(&dh0, w.data(), 226, 1, q, k, v, out, lse, ws, need));
  add("null q", STA_ERR_NULL, fwd(&d, w.data(), 226, 1, nullptr, k, v, out, lse, ws, need));
  add("null v", STA_ERR_NULL, fwd(&d, w.data(), 226, 1, q, k, nullptr, out, lse, ws, need));
  add("null out", STA_ERR_NULL, fwd(&d, w.data(), 226, 1, q, k, v, nullptr, lse, ws, need));
  add("null windows", STA_ERR_NULL, fwd(&d, nullptr, 226, 1, q, k, v, out, lse, ws, need));
  add("head_dim 96", STA_ERR_SHAPE, fwd(&dd, w.data(), 226, 1, q, k, v, out, lse, ws, need));
  add("T 0", STA_ERR_SHAPE, fwd(&dt0, w.data(), 226, 1, q, k, v, out, lse, ws, need));
  add("H -8", STA_ERR_SHAPE, fwd(&dhn, w.data(), 226, 1, q, k, v, out, lse, ws, need));
  add("1024 tiles on t", STA_ERR_SHAPE, fwd(&dbig, w.data(), 0, 0, q, k, v, out, lse, ws, need));
  add("257 heads", STA_ERR_SHAPE, fwd(&dheads, w257.data(), 0, 1, q, k, v, out, lse, ws, need));
  for (int axis = 0; axis < 3; ++axis)
    for (int bad : {0, -1, 7, 11}) {
      std::vector<int32_t> wb = w;
      const int n_axis[3] = {5, 6, 10};
      if (bad >= 1 && bad <= n_axis[axis]) continue;
      wb[3 + axis] = bad;
      add("window out of range", STA_ERR_WINDOW,
          fwd(&d, wb.data(), 226, 1, q, k, v, out, lse, ws, need));
    }
  add("ell 257", STA_ERR_TEXT, fwd(&d, w.data(), 257, 1, q, k, v, out, lse, ws, need));
  add("ell -1", STA_ERR_TEXT, fwd(&d, w.data(), -1, 1, q, k, v, out, lse, ws, need));
  add("ell without text", STA_ERR_TEXT, fwd(&d, w.data(), 5, 0, q, k, v, out, lse, ws, need));
  char* qc = static_cast<char*>(q);
  add("q misaligned", STA_ERR_ALIGN, fwd(&d, w.data(), 226, 1, qc + 1, k, v, out, lse, ws, need));
  add("out misaligned", STA_ERR_ALIGN,
      fwd(&d, w.data(), 226, 1, q, k, v, static_cast<char*>(out) + 8, lse, ws, need));
  add("lse misaligned", STA_ERR_ALIGN,
      fwd(&d, w.data(), 226, 1, q, k, v, out, lse + 1, ws, need));
  add("workspace small", STA_ERR_WORKSPACE,
      fwd(&d, w.data(), 226, 1, q, k, v, out, lse, ws, need - 1));
  add("workspace null", STA_ERR_WORKSPACE,
      fwd(&d, w.data(), 226, 1, q, k, v, out, lse, nullptr, need));
  add("workspace misaligned", STA_ERR_ALIGN,
      fwd(&d, w.data(), 226, 1, q, k, v, out, lse, static_cast<char*>(ws) + 16, need));
  add("out over q", STA_ERR_ALIAS, fwd(&d, w.data(), 226, 1, q, k, v, q, lse, ws, need));
  add("lse over out", STA_ERR_ALIAS,
      fwd(&d, w.data(), 226, 1, q, k, v, out, static_cast<float*>(out) + 256, ws, need));
  add("out over workspace", STA_ERR_ALIAS,
      fwd(&d, w.data(), 226, 1, q, k, v, static_cast<char*>(ws) + 1024, lse, ws, need));
  void* null_events[STA_TIMED_EVENTS] = {};
  add("timed, null event", STA_ERR_NULL,
      fwd(&d, w.data(), 226, 1, q, k, v, out, lse, ws, need, null_events));
  for (const Case& c : cases)
    CHECK(c.got == c.expect, "%s: expected %d (%s), got %d (%s)", c.what, int(c.expect),
          sta_status_str(c.expect), int(c.got), sta_status_str(c.got));

  // Valid forward calls on every workload shape: the launch sequence runs on
  // the caller's tensors and workspace regions only; the timed variant records
  // one event before the first launch and one after each.
  struct Shape {
    sta_dims d;
    int text, ell, wt, wh, ww;
  };
  const Shape shapes[] = {
      {{1, 1, 64, 18, 24, 24}, 0, 0, 1, 3, 3},    {{1, 24, 128, 30, 48, 80}, 1, 226, 3, 3, 3},
      {{1, 24, 128, 48, 72, 128}, 1, 128, 3, 3, 3}, {{1, 24, 128, 33, 45, 80}, 1, 226, 3, 3, 3},
      {{2, 3, 64, 7, 9, 11}, 1, 50, 2, 2, 2},     {{1, 2, 128, 1, 128, 128}, 0, 0, 1, 5, 5},
      {{3, 5, 128, 1, 1, 1}, 1, 256, 1, 1, 1},
  };
  for (const Shape& s : shapes) {
    std::vector<int32_t> ws_win = windows_for(s.d.heads, s.wt, s.wh, s.ww);
    const size_t n = sta_workspace_bytes(&s.d, ws_win.data(), s.text);
    CHECK(n > 0, "workspace bytes of a valid shape");
    void* events[STA_TIMED_EVENTS];
    for (int i = 0; i < STA_TIMED_EVENTS; ++i) events[i] = fake(20 + i);
    g_events = 0;
    sta_status st = fwd(&s.d, ws_win.data(), s.ell, s.text, q, k, v, out, lse, ws, n, events);
    CHECK(st == STA_OK, "valid forward returned %s", sta_status_str(st));
    CHECK(g_events == STA_TIMED_EVENTS, "timed forward recorded %d events", g_events);
    CHECK(!g_launches.empty() && g_launches.back().name == "attention", "attention launched last");
    for (const Launch& l : g_launches)
      check_in_workspace(l, {P(q), P(k), P(v), P(out), P(lse)}, P(ws), n);
    // the backward: same rules, with its own workspace
    const size_t nb = sta_backward_workspace_bytes(&s.d, ws_win.data(), s.text);
    CHECK(nb > 0, "backward workspace bytes of a valid shape");
    g_launches.clear();
    void *dq = fake(10), *dk = fake(11), *dv = fake(12), *dout = fake(13);
    st = sta_backward(&s.d, q, k, v, out, lse, dout, ws_win.data(), s.ell, s.text, dq, dk, dv, ws,
                      nb, nullptr);
    CHECK(st == STA_OK, "valid backward returned %s", sta_status_str(st));
    CHECK(g_launches.size() >= 2 && g_launches.back().name == "bwd_dkv", "backward sequence");
    for (const Launch& l : g_launches)
      check_in_workspace(l, {P(q), P(k), P(v), P(out), P(lse), P(dout), P(dq), P(dk), P(dv)},
                         P(ws), nb);
    g_launches.clear();
    st = sta_backward(&s.d, q, k, v, out, lse, dout, ws_win.data(), s.ell, s.text, dq, dk, dv, ws,
                      nb - 1, nullptr);
    CHECK(st == STA_ERR_WORKSPACE && g_launches.empty(), "backward, workspace short by one byte");
    st = sta_backward(&s.d, q, k, v, out, lse, dout, ws_win.data(), s.ell, s.text, dq, dq, dv, ws,
                      nb, nullptr);
    CHECK(st == STA_ERR_ALIAS && g_launches.empty(), "backward, dk over dq");
  }
  // Hilbert entry points: shape, window and mode errors before any launch
  {
    const sta_dims ok{1, 2, 64, 1, 32, 32};
    const int32_t lens[2] = {3, 16};
    const size_t n = sta_hilbert_workspace_bytes(&ok, 1);
    CHECK(n > 0, "hilbert workspace");
    struct HCase {
      sta_dims d;
      int32_t l0, l1, mode;
      sta_status expect;
      const char* what;
    } hc[] = {
        {{1, 2, 64, 1, 32, 32}, 3, 16, STA_HILBERT_SLIDE, STA_OK, "valid slide"},
        {{1, 2, 64, 1, 32, 32}, 4, 16, STA_HILBERT_WINDOW, STA_OK, "valid window"},
        {{1, 2, 64, 2, 32, 32}, 3, 16, STA_HILBERT_SLIDE, STA_ERR_SHAPE, "two frames"},
        {{1, 2, 64, 1, 32, 64}, 3, 16, STA_HILBERT_SLIDE, STA_ERR_SHAPE, "not square"},
        {{1, 2, 64, 1, 24, 24}, 3, 9, STA_HILBERT_SLIDE, STA_ERR_SHAPE, "3x3 tile grid"},
        {{1, 2, 64, 1, 36, 36}, 3, 9, STA_HILBERT_SLIDE, STA_ERR_SHAPE, "side not a tile multiple"},
        {{1, 2, 64, 1, 32, 32}, 0, 16, STA_HILBERT_SLIDE, STA_ERR_WINDOW, "window 0"},
        {{1, 2, 64, 1, 32, 32}, 3, 17, STA_HILBERT_SLIDE, STA_ERR_WINDOW, "window past the grid"},
        {{1, 2, 64, 1, 32, 32}, 3, 16, 0, STA_ERR_WINDOW, "mode 0"},
        {{1, 2, 64, 1, 32, 32}, 3, 16, 3, STA_ERR_WINDOW, "mode 3"},
    };
    for (const HCase& c : hc) {
      const int32_t l[2] = {c.l0, c.l1};
      g_launches.clear();
      const sta_status st = sta_hilbert_forward(&c.d, q, k, v, l, c.mode, 100, 1, out, lse, ws, n, nullptr);
      CHECK(st == c.expect, "hilbert %s: expected %s, got %s", c.what, sta_status_str(c.expect), sta_status_str(st));
      CHECK((st == STA_OK) == !g_launches.empty(), "hilbert %s: launches", c.what);
      if (st == STA_OK)
        for (const Launch& l2 : g_launches) check_in_workspace(l2, {P(q), P(k), P(v), P(out), P(lse)}, P(ws), n);
    }
    CHECK(sta_hilbert_forward(&ok, q, k, v, lens, STA_HILBERT_SLIDE, 100, 1, out, lse, ws, n - 1, nullptr) ==
              STA_ERR_WORKSPACE,
          "hilbert workspace short by one byte");
    // large images split the text rows' keys over several units, whose
    // partial results sit in the workspace: it must hold them whole (the size
    // query covers single-tile units, so it may exceed what a call uses)
    for (int side : {128, 256, 512}) {
      const sta_dims big{2, 3, 128, 1, side, side};
      const int32_t bl[3] = {27, 9, 64};
      const size_t nb = sta_hilbert_workspace_bytes(&big, 1);
      g_launches.clear();
      CHECK(sta_hilbert_forward(&big, q, k, v, bl, STA_HILBERT_SLIDE, 226, 1, out, lse, ws, nb, nullptr) == STA_OK,
            "hilbert %d^2 forward", side);
      const Launch& l = g_launches.back();
      const sta::Geom& gb = l.g;
      const int parts = gb.n_tiles / 128 < 8 ? gb.n_tiles / 128 : 8;
      CHECK(l.name == "attention" && gb.text_parts == parts && gb.hil_group == 6, "hilbert %d^2: %d text parts",
            side, gb.text_parts);
      check_in_workspace(l, {P(q), P(k), P(v), P(out), P(lse)}, P(ws), nb);
      const uintptr_t tp = l.ptrs.back();
      CHECK(tp != 0 && tp + size_t(2) * 3 * parts * 256 * (128 + 2) * 4 <= P(ws) + nb,
            "hilbert %d^2: text partials inside the workspace", side);
    }
    CHECK(sta_hilbert_gather(&ok, 1, q, q, nullptr) == STA_ERR_ALIAS, "hilbert gather in place");
    CHECK(sta_hilbert_gather(&ok, 1, q, out, nullptr) == STA_OK && g_launches.back().name == "rows_hilbert",
          "hilbert gather");
    const sta_dims bad{1, 2, 64, 1, 40, 40};
    CHECK(sta_hilbert_scatter(&bad, 1, q, out, nullptr) == STA_ERR_SHAPE, "hilbert scatter, 5x5 tiles");
  }
  // the forward without a workspace: its kernels get the scratch array only
  {
    const uintptr_t scratch = uintptr_t(40) * 64 * (uintptr_t(1) << 30);
    const sta_dims d{2, 24, 128, 30, 48, 80};
    std::vector<int32_t> w = windows_for(d.heads, 3, 3, 3);
    for (int call = 0; call < 2; ++call) {
      g_launches.clear();
      sta_status st = sta_forward_noalloc(&d, q, k, v, w.data(), 226, 1, out, lse, nullptr);
      CHECK(st == STA_OK, "noalloc forward returned %s", sta_status_str(st));
      CHECK(!g_launches.empty() && g_launches.back().name == "attention", "noalloc: attention launched last");
      for (const Launch& l : g_launches)
        check_in_workspace(l, {P(q), P(k), P(v), P(out), P(lse)}, scratch, STA_NOALLOC_SCRATCH_BYTES);
    }
    CHECK(g_symbol_lookups == 1, "scratch address looked up %d times", g_symbol_lookups);
    // a shape whose workspace exceeds the scratch is rejected before any launch
    const sta_dims big{16, 256, 64, 60, 64, 64};
    std::vector<int32_t> wb = windows_for(big.heads, 1, 1, 1);
    CHECK(sta_workspace_bytes(&big, wb.data(), 0) > STA_NOALLOC_SCRATCH_BYTES, "big shape");
    g_launches.clear();
    sta_status st = sta_forward_noalloc(&big, q, k, v, wb.data(), 0, 0, out, lse, nullptr);
    CHECK(st == STA_ERR_SCRATCH && g_launches.empty(), "noalloc, oversize: %s", sta_status_str(st));
    // argument errors are those of sta_forward
    st = sta_forward_noalloc(&d, q, k, v, w.data(), 300, 1, out, lse, nullptr);
    CHECK(st == STA_ERR_TEXT && g_launches.empty(), "noalloc, bad text length: %s", sta_status_str(st));
    st = sta_forward_noalloc(&d, q, k, v, w.data(), 226, 1, q, lse, nullptr);
    CHECK(st == STA_ERR_ALIAS && g_launches.empty(), "noalloc, out over q: %s", sta_status_str(st));
  }
  std::printf("ok %d\n", g_checks);
}

void dump(int argc, char** argv) {
  if (argc != 13) {
    std::fprintf(stderr, "dump needs 11 integers\n");
    std::exit(2);
  }
  int a[11];
  for (int i = 0; i < 11; ++i) a[i] = std::atoi(argv[2 + i]);
  const sta_dims d{a[0], a[1], a[2], a[3], a[4], a[5]};
  const int text = a[6], ell = a[7];
  std::vector<int32_t> w = windows_for(d.heads, a[8], a[9], a[10]);
  // geometry through the public calls, then the Geom the launches received
  int64_t n_off = 0, n_ids = 0, n_work = 0;
  CHECK(sta_schedule_sizes(&d, w.data(), text, &n_off, &n_ids, &n_work) == STA_OK, "sizes");
  std::printf("sizes %lld %lld %lld %lld %lld\n", (long long)sta_seq_len(&d, text),
              (long long)sta_tiled_seq_len(&d, text), (long long)n_off, (long long)n_ids,
              (long long)n_work);
  const size_t n = sta_workspace_bytes(&d, w.data(), text);
  g_launches.clear();
  CHECK(fwd(&d, w.data(), ell, text, fake(0), fake(1), fake(2), fake(3),
            static_cast<float*>(fake(4)), fake(8), n) == STA_OK,
        "forward on the dumped geometry");
  const sta::Geom g = g_launches.back().g;
  std::printf("geom %d %d %d %d %d %d %d %d %d %d %d\n", g.nt, g.nh, g.nw, g.n_tiles, g.n_video,
              g.S, g.n_vt, g.S_t, g.full, g.n_q, g.text_length);
  // window placement: every start on each axis, for every window size
  const int nax[3] = {g.nt, g.nh, g.nw};
  for (int ax = 0; ax < 3; ++ax)
    for (int wl = 1; wl <= nax[ax]; ++wl)
      for (int c = 0; c < nax[ax]; ++c)
        std::printf("ws %d %d %d %d\n", ax, wl, c, sta::window_start(c, wl, nax[ax]));
  // tile extents, and the blocks of each query tile's window and of the grid
  for (int t = 0; t < g.n_tiles; ++t) {
    const int tw = t % g.nw, th = (t / g.nw) % g.nh, tt = t / (g.nw * g.nh);
    const int e = sta::tile_extent(tt, th, tw, g);
    const int st = sta::window_start(tt, a[8], g.nt), sh = sta::window_start(th, a[9], g.nh),
              sw = sta::window_start(tw, a[10], g.nw);
    std::printf("tile %d %d %d %d %d %d\n", t, sta::extent_frames(e), sta::extent_rows(e),
                sta::extent_cols(e), sta::extent_tokens(e),
                sta::box_blocks(st, a[8], sh, a[9], sw, a[10], g));
  }
  std::printf("grid %d\n", sta::box_blocks(0, g.nt, 0, g.nh, 0, g.nw, g));
  // tile-major row -> raster row (-1 for padding), and the multiples-only form
  for (int r = 0; r < g.S_t; ++r) {
    const int x = sta::tiled_to_raster(r, g);
    if (g.full) CHECK(x == sta::tiled_to_raster_full(r, g), "tiled_to_raster_full row %d", r);
    std::printf("%d\n", x);
  }
}

// The forward kernel's key stream of every query unit (sta::KeyStream, the
// same code the kernel runs): checks the block order (blocks before n_plain
// whole, masked ones after), the bounds of every key row, and that no key is
// streamed twice; prints each unit's valid key rows as sorted half-open
// ranges "unit <u> <n_blk> <n_plain> <lo>:<hi> ...".
template <bool PAD>
void stream_units(const sta::Geom& g, int wt, int wh, int ww) {
  for (int u = 0; u < g.n_q; ++u) {
    const bool text_unit = g.has_text && u == g.n_tiles;
    sta::KeyStream<PAD> ks;
    if (text_unit) {
      ks.init(g, 0, g.nt, 0, g.nh, 0, g.nw);
    } else {
      const int tw = u % g.nw, th = (u / g.nw) % g.nh, tt = u / (g.nw * g.nh);
      ks.init(g, sta::window_start(tt, wt, g.nt), wt, sta::window_start(th, wh, g.nh), wh,
              sta::window_start(tw, ww, g.nw), ww);
    }
    std::vector<int> keys;
    for (int j = 0; j < ks.n_blk; ++j) {
      const sta::KeyBlock b = ks.block(g, j);
      CHECK(b.mask >= 1 && b.mask <= sta::kKeyBlock, "unit %d block %d mask %d", u, j, b.mask);
      CHECK(j >= ks.n_plain || b.mask == sta::kKeyBlock, "unit %d block %d masked before n_plain %d", u, j,
            ks.n_plain);
      CHECK(PAD || b.kind != 2, "unit %d block %d: compact block without partial tiles", u, j);
      for (int r = 0; r < b.mask; ++r) {
        int row;
        if (b.kind == 0) {
          row = b.base + (r >> 3) * g.W + (r & 7);
        } else if (b.kind == 1) {
          CHECK(b.mask == b.lim, "unit %d block %d text limit", u, j);
          row = b.base + r;
          CHECK(row >= g.n_video && row < g.n_video + g.text_length, "unit %d block %d text row %d", u, j, row);
        } else {
          const int tok = b.sub * sta::kKeyBlock + r;
          CHECK(tok < sta::extent_tokens(b.ext), "unit %d block %d token %d past the tile", u, j, tok);
          int dt, dh, dw;
          sta::compact_token(tok, b.ext, dt, dh, dw);
          row = b.base + (dt * g.H + dh) * g.W + dw;
        }
        CHECK(row >= 0 && row < g.S, "unit %d block %d row %d outside the sequence", u, j, row);
        keys.push_back(row);
      }
    }
    std::sort(keys.begin(), keys.end());
    for (size_t i = 1; i < keys.size(); ++i) CHECK(keys[i] != keys[i - 1], "unit %d key %d twice", u, keys[i]);
    std::printf("unit %d %d %d", u, ks.n_blk, ks.n_plain);
    for (size_t i = 0; i < keys.size();) {
      size_t e = i + 1;
      while (e < keys.size() && keys[e] == keys[e - 1] + 1) ++e;
      std::printf(" %d:%d", keys[i], keys[e - 1] + 1);
      i = e;
    }
    std::printf("\n");
  }
}

void stream(int argc, char** argv) {
  if (argc != 10) {
    std::fprintf(stderr, "stream needs 8 integers\n");
    std::exit(2);
  }
  int a[8];
  for (int i = 0; i < 8; ++i) a[i] = std::atoi(argv[2 + i]);
  const sta_dims d{1, 1, 128, a[0], a[1], a[2]};
  const int text = a[3], ell = a[4];
  std::vector<int32_t> w = windows_for(1, a[5], a[6], a[7]);
  const size_t n = sta_workspace_bytes(&d, w.data(), text);
  CHECK(fwd(&d, w.data(), ell, text, fake(0), fake(1), fake(2), fake(3), static_cast<float*>(fake(4)), fake(8),
            n) == STA_OK,
        "forward on the streamed geometry");
  const sta::Geom g = g_launches.back().g;
  CHECK(g.hilbert == 0, "stream: single-tile units expected");
  if (g.full)
    stream_units<false>(g, a[5], a[6], a[7]);
  else
    stream_units<true>(g, a[5], a[6], a[7]);
}

// The Hilbert curve helpers: "hcurve <k>" prints x y of every position of the
// order-k curve (and checks the inverse); "hstream <side> <has_text> <ell> <W>
// <mode>" prints every Hilbert unit's key rows like `stream`, with the query
// tile's coordinates.
void hcurve(int argc, char** argv) {
  if (argc != 3) {
    std::fprintf(stderr, "hcurve needs the order\n");
    std::exit(2);
  }
  const int k = std::atoi(argv[2]);
  for (int d = 0; d < (1 << (2 * k)); ++d) {
    int x, y;
    sta::hilbert_d2xy(k, d, x, y);
    CHECK(sta::hilbert_xy2d(k, x, y) == d, "order %d position %d: inverse", k, d);
    std::printf("%d %d\n", x, y);
  }
}

void hstream(int argc, char** argv) {
  if (argc != 7) {
    std::fprintf(stderr, "hstream needs 5 integers\n");
    std::exit(2);
  }
  const int side = std::atoi(argv[2]), text = std::atoi(argv[3]), ell = std::atoi(argv[4]);
  const int W = std::atoi(argv[5]), mode = std::atoi(argv[6]);
  const sta_dims d{1, 1, 128, 1, side, side};
  const int32_t lens[1] = {W};
  const size_t n = sta_hilbert_workspace_bytes(&d, text);
  CHECK(n > 0, "hilbert workspace bytes");
  g_launches.clear();
  CHECK(sta_hilbert_forward(&d, fake(0), fake(1), fake(2), lens, mode, ell, text, fake(3),
                            static_cast<float*>(fake(4)), fake(8), n, nullptr) == STA_OK,
        "hilbert forward on the streamed geometry");
  const sta::Geom g = g_launches.back().g;
  CHECK(g.hilbert == mode && (8 << g.hil_m) == side && !g.full, "hilbert geometry");
  const int G = g.hil_group, n_vunits = (g.n_tiles + G - 1) / G;
  CHECK(G == 1 || G == 4 || G == 6, "hilbert group %d", G);
  CHECK(G != 6 || (mode == 1 && W >= 6), "six-tile units need a slide window of at least 6");
  const int parts = g.has_text ? g.text_parts : 0;
  CHECK(g.has_text ? (parts >= 1 && parts <= 8 && (parts == 1 || g.n_tiles / parts >= 128)) : g.text_parts == 1,
        "hilbert text parts %d", g.text_parts);
  CHECK(g.n_q == n_vunits + parts, "hilbert units %d", g.n_q);
  // one line per query tile; the text units' parts are listed together
  for (int u = 0; u < n_vunits + (g.has_text ? 1 : 0); ++u) {
    const bool text_unit = g.has_text && u == n_vunits;
    const int tiles = text_unit ? 1 : std::min(G, g.n_tiles - G * u);
    for (int t = 0; t < tiles; ++t) {
      int tx = -1, ty = -1;
      if (!text_unit) sta::hilbert_d2xy(g.hil_m, G * u + t, tx, ty);
      std::vector<int> keys;
      for (int part = 0; part < (text_unit ? parts : 1); ++part) {
        sta::HilbertKeyStream ks;
        ks.init(g, G * u, W, text_unit, part);
        for (int j = 0; j < ks.n_blk; ++j) {
          const sta::KeyBlock b = ks.block(g, j);
          CHECK(j >= ks.n_plain || b.mask == sta::kKeyBlock, "unit %d block %d masked early", u, j);
          CHECK(j != 0 || b.seen == -1, "unit %d: block 0 not seen by all", u);
          if (((b.seen >> t) & 1) == 0) continue;
          for (int r = 0; r < b.mask; ++r) {
            int row;
            if (b.kind == 0) {
              CHECK(sta::extent_tokens(b.ext) == 64, "unit %d block %d: tile of %d tokens", u, j,
                    sta::extent_tokens(b.ext));
              row = b.base + (r >> 3) * g.W + (r & 7);
            } else {
              CHECK(b.kind == 1, "unit %d block %d kind %d", u, j, b.kind);
              row = b.base + r;
            }
            CHECK(row >= 0 && row < g.S, "unit %d block %d row %d outside the sequence", u, j, row);
            keys.push_back(row);
          }
        }
      }
      std::sort(keys.begin(), keys.end());
      for (size_t i = 1; i < keys.size(); ++i) CHECK(keys[i] != keys[i - 1], "unit %d key %d twice", u, keys[i]);
      std::printf("unit %d %d %d %d", u, t, tx, ty);
      for (size_t i = 0; i < keys.size();) {
        size_t e = i + 1;
        while (e < keys.size() && keys[e] == keys[e - 1] + 1) ++e;
        std::printf(" %d:%d", keys[i], keys[e - 1] + 1);
        i = e;
      }
      std::printf("\n");
    }
  }
}


// "sqstream <H> <W> <has_text> <ell> <wh> <ww>": STA on a one-frame video (any H, W)
// (T = 1) as the forward plans it; with square units, one line per query tile
// of every unit, "unit u i tile_h tile_w" then its key rows as in `stream`,
// and one line for the text rows (tile -1 -1, every part's keys); "single"
// when the forward keeps single-tile units.
void sqstream(int argc, char** argv) {
  if (argc != 8) {
    std::fprintf(stderr, "sqstream needs 6 integers\n");
    std::exit(2);
  }
  int a[6];
  for (int i = 0; i < 6; ++i) a[i] = std::atoi(argv[2 + i]);
  const sta_dims d{1, 1, 128, 1, a[0], a[1]};
  const int text = a[2], ell = a[3];
  std::vector<int32_t> w = windows_for(1, 1, a[4], a[5]);
  const size_t n = sta_workspace_bytes(&d, w.data(), text);
  CHECK(n > 0, "square workspace bytes");
  g_launches.clear();
  CHECK(fwd(&d, w.data(), ell, text, fake(0), fake(1), fake(2), fake(3), static_cast<float*>(fake(4)), fake(8),
            n) == STA_OK,
        "forward on the streamed geometry");
  const sta::Geom g = g_launches.back().g;
  if (g.hilbert == 0) {
    std::printf("single\n");
    return;
  }
  CHECK(g.hilbert == sta::kSquareUnits && g.hil_group == 4 && g.T == 1, "square geometry");
  const int n_su = ((g.nh + 1) / 2) * ((g.nw + 1) / 2);
  const int parts = g.has_text ? g.text_parts : 0;
  CHECK(g.n_q == n_su + parts, "square units %d", g.n_q);
  CHECK(g.has_text ? (parts >= 1 && parts <= 8 && (parts == 1 || g.n_tiles / parts >= 128)) : g.text_parts == 1,
        "square text parts %d", g.text_parts);
  std::vector<int> covered(g.n_tiles, 0);
  for (int u = 0; u < n_su + (g.has_text ? 1 : 0); ++u) {
    const bool text_unit = g.has_text && u == n_su;
    int sy = 0, sx = 0, layout = 3, tiles = 1;
    if (!text_unit) tiles = sta::square_tiles(g, u, sy, sx, layout);
    for (int i = 0; i < tiles; ++i) {
      int th = -1, tw = -1;
      if (!text_unit) {
        int dy, dx;
        sta::square_tile(i, layout, dy, dx);
        th = 2 * sy + dy;
        tw = 2 * sx + dx;
        CHECK(th < g.nh && tw < g.nw, "unit %d tile %d outside the grid", u, i);
        ++covered[th * g.nw + tw];
      }
      std::vector<int> keys;
      for (int part = 0; part < (text_unit ? parts : 1); ++part) {
        // the kernel's stream: with partial tiles when H or W is not a multiple of 8
        sta::SquareKeyStream<true> ks;
        sta::SquareKeyStream<false> kw;
        const bool partial = g.H % 8 != 0 || g.W % 8 != 0;
        ks.init(g, text_unit ? part : u, a[4], a[5], text_unit);
        kw.init(g, text_unit ? part : u, a[4], a[5], text_unit);
        CHECK(ks.n_blk == kw.n_blk, "unit %d: block counts differ", u);
        for (int j = 0; j < ks.n_blk; ++j) {
          const sta::KeyBlock b = partial ? ks.block(g, j) : kw.block(g, j);
          if (!partial) {
            const sta::KeyBlock bp = ks.block(g, j);
            CHECK(bp.kind == b.kind && bp.base == b.base && bp.mask == b.mask && bp.seen == b.seen,
                  "unit %d block %d: streams differ on whole tiles", u, j);
          }
          CHECK(b.mask >= 1 && b.mask <= sta::kKeyBlock, "unit %d block %d mask %d", u, j, b.mask);
          CHECK(j != 0 || b.seen == -1, "unit %d: block 0 not seen by all", u);
          CHECK(b.seen == -1 || (b.seen & ~((1 << tiles) - 1)) == 0, "unit %d block %d: seen bits past the unit", u, j);
          CHECK(b.seen != 0, "unit %d block %d seen by no tile", u, j);
          if (((b.seen >> i) & 1) == 0) continue;
          for (int r = 0; r < b.mask; ++r) {
            int row;
            if (b.kind == 0) {
              CHECK(sta::extent_tokens(b.ext) == 64 && b.mask == 64, "unit %d block %d: tile of %d tokens", u, j,
                    sta::extent_tokens(b.ext));
              row = b.base + (r >> 3) * g.W + (r & 7);
            } else if (b.kind == 2) {
              CHECK(b.sub == 0 && b.mask == sta::extent_tokens(b.ext) && b.mask < 64, "unit %d block %d partial", u, j);
              int dt, dh, dw;
              sta::compact_token(r, b.ext, dt, dh, dw);
              CHECK(dt == 0, "unit %d block %d frame %d", u, j, dt);
              row = b.base + dh * g.W + dw;
            } else {
              CHECK(b.kind == 1, "unit %d block %d kind %d", u, j, b.kind);
              row = b.base + r;
            }
            CHECK(row >= 0 && row < g.S, "unit %d block %d row %d outside the sequence", u, j, row);
            keys.push_back(row);
          }
        }
      }
      std::sort(keys.begin(), keys.end());
      for (size_t k = 1; k < keys.size(); ++k) CHECK(keys[k] != keys[k - 1], "unit %d key %d twice", u, keys[k]);
      std::printf("unit %d %d %d %d", u, i, th, tw);
      for (size_t k = 0; k < keys.size();) {
        size_t e = k + 1;
        while (e < keys.size() && keys[e] == keys[e - 1] + 1) ++e;
        std::printf(" %d:%d", keys[k], keys[e - 1] + 1);
        k = e;
      }
      std::printf("\n");
    }
  }
  for (int t = 0; t < g.n_tiles; ++t) CHECK(covered[t] == 1, "tile %d in %d units", t, covered[t]);
}
}  // namespace

int main(int argc, char** argv) {
  if (argc >= 2 && std::strcmp(argv[1], "validate") == 0) {
    validate();
    return 0;
  }
  if (argc >= 2 && std::strcmp(argv[1], "dump") == 0) {
    dump(argc, argv);
    return 0;
  }
  if (argc >= 2 && std::strcmp(argv[1], "stream") == 0) {
    stream(argc, argv);
    return 0;
  }
  if (argc >= 2 && std::strcmp(argv[1], "hcurve") == 0) {
    hcurve(argc, argv);
    return 0;
  }
  if (argc >= 2 && std::strcmp(argv[1], "hstream") == 0) {
    hstream(argc, argv);
    return 0;
  }
  if (argc >= 2 && std::strcmp(argv[1], "sqstream") == 0) {
    sqstream(argc, argv);
    return 0;
  }
  std::fprintf(stderr, "usage: %s validate | dump B heads D T H W has_text ell wt wh ww | stream T H W has_text ell wt wh ww\n",
               argv[0]);
  return 2;
}
