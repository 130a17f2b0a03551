// Host side of the C ABI declared in include/flce.h: argument validation, the BT-chunk plan,
// workspace carving and the per-chunk launch sequence. Everything is enqueued on the caller's
// stream; nothing here allocates or synchronises during flce_forward_backward.
//
// The chunk plan answers the two chunk-size observations of "Torch compiled FLCE is 2x faster than
// the current FLCE" (Liger-Kernel issue #227): the chunk size trades time against memory (Chillee's
// 256 vs 512 comparison), and B*T that varies from call to call and is not a multiple of the chunk
// size must not cost a recompile (wizyoung's ragged benchmark). Here the code object is the same for
// every BT; chunks are balanced so that the last one is not a sliver that still pays a full
// grad_W read-modify-write, and grad_W is accumulated in place (the same thread notes that the
// compiled version does not do its addmm in place).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <vector>

#include "flce.h"
#include "flce_internal.h"

struct flce_ctx {
  int device;
  int ncu;        // compute units of the device
  int64_t chunk_rows_max;
  int* d_status;  // device status word written by the label pre-pass
  // kernel timing (flce_profile_begin/end): event pairs recorded around each launch
  bool prof_on = false;
  std::vector<hipEvent_t> prof_events;
  std::vector<int> prof_kinds;
};

namespace {

constexpr int64_t kDefaultChunk = 4096;
constexpr int kDefaultCUs = 256;  // MI355X, for workspace sizes asked without a handle
constexpr int64_t kMaxH = 1 << 16;
constexpr int64_t kMaxV = int64_t(1) << 20;  // keeps every per-tile buffer range below 2 GiB
constexpr int64_t kMaxBT = (int64_t(1) << 31) - 1;

int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

int64_t chunk_max_of(const flce_ctx* h) {
  return h ? h->chunk_rows_max : kDefaultChunk;
}
int ncu_of(const flce_ctx* h) {
  return h ? h->ncu : kDefaultCUs;
}

void plan(int64_t BT, int64_t cmax, int64_t* n, int64_t* rows) {
  if (BT <= 0) {
    *n = 0;
    *rows = 0;
    return;
  }
  const int64_t nn = (BT + cmax - 1) / cmax;
  int64_t c = round_up((BT + nn - 1) / nn, flce::kRowAlign);
  if (c > cmax) c = cmax;
  *n = nn;
  *rows = c;
}

int dx_splits(int64_t rows, int64_t H, int64_t V_pad, int dtype, int ncu) {
  // Split K (= V) only when it shortens the wave-quantised schedule: with T tiles on ncu CUs and
  // s splits the time goes as ceil(T*s / ncu) / s, plus a small per-split cost for the reduction.
  const int64_t tiles = ((rows + flce::kTile - 1) / flce::kTile) * ((H + flce::kTile - 1) / flce::kTile);
  const int64_t nk = V_pad * (dtype == 0 ? 2 : 4) / flce::kStepBytes;
  int best = 1;
  double best_cost = 1e30;
  for (int s = 1; s <= 32; ++s) {
    if (s > 1 && nk / s < 16) break;  // keep at least 16 k-steps per split
    const double waves = (double)((tiles * s + ncu - 1) / ncu);
    const double cost = waves / s + 0.02 * (s - 1);
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = s;
    }
  }
  return best;
}

struct Layout {
  size_t off_e, off_m, off_s, off_y, off_sl, off_og, off_loss, off_part, off_xt, off_params, total;
  int splits;
  int64_t chunk_rows;
};

// Workspace carving. The forward-only path (backward = false) needs no q/dZ chunk and no split-K
// partials.
Layout layout(int64_t BT, int64_t H, int64_t V, int dtype, int64_t cmax, int ncu, bool backward = true) {
  Layout L{};
  int64_t n, rows;
  plan(BT, cmax, &n, &rows);
  const int64_t V_pad = round_up(V, flce::kTile);
  const int64_t nseg = V_pad / flce::kSeg;
  const size_t esz = dtype == 0 ? 2 : 4;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) / 256 * 256;
    return o;
  };
  L.chunk_rows = rows;
  L.splits = backward && rows > 0 ? dx_splits(rows, H, V_pad, dtype, ncu) : 1;
  L.off_params = take(sizeof(flce::DevParams));
  L.off_e = take(backward ? (size_t)rows * V_pad * esz : 0);
  L.off_m = take((size_t)rows * nseg * 4);
  L.off_s = take((size_t)rows * nseg * 4);
  L.off_y = take((size_t)BT * 4);
  L.off_sl = take((size_t)BT * 4);
  L.off_og = take((size_t)BT * 4);
  L.off_loss = take((size_t)BT * 4);
  L.off_part = take(L.splits > 1 ? (size_t)L.splits * rows * H * 4 : 0);
  L.off_xt = take((size_t)rows * H * esz);
  L.total = off;
  return L;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_sizes(int64_t BT, int64_t H, int64_t V, int dtype) {
  if (BT < 0 || H <= 0 || V <= 0) return FLCE_ERR_INVALID_ARG;
  if (dtype != FLCE_BF16 && dtype != FLCE_FP32) return FLCE_ERR_INVALID_ARG;
  if (H % 8 != 0 || H > kMaxH || V > kMaxV || BT > kMaxBT) return FLCE_ERR_UNSUPPORTED;
  return FLCE_OK;
}

struct DeviceGuard {
  int prev = -1;
  bool ok = true;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) {
      ok = false;
      return;
    }
    if (prev != dev && hipSetDevice(dev) != hipSuccess) ok = false;
  }
  ~DeviceGuard() {
    int cur;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

// One call's problem description, workspace views and launch bookkeeping. Each launch is
// optionally bracketed by a pre-created event pair on the call's stream (kernel timing diagnostics).
struct Call {
  flce_ctx* h;
  hipStream_t stream;
  flce::Problem p;
  flce::Work w;
  template <class F>
  bool run(int kind, F&& launch) {
    const size_t k = h->prof_kinds.size();
    const bool rec = h->prof_on && 2 * (k + 1) <= h->prof_events.size();
    if (rec && hipEventRecord(h->prof_events[2 * k], stream) != hipSuccess) return false;
    if (launch() != hipSuccess) return false;
    if (rec) {
      if (hipEventRecord(h->prof_events[2 * k + 1], stream) != hipSuccess) return false;
      h->prof_kinds.push_back(kind);
    }
    return true;
  }
};

Call make_call(flce_ctx* h, const Layout& L, int64_t BT, int64_t H, int64_t V, int dtype, int64_t ignore_index,
               float softcap, int reduction, void* workspace, void* stream) {
  Call c;
  c.h = h;
  c.stream = (hipStream_t)stream;
  flce::Problem& p = c.p;
  p.BT = BT;
  p.H = H;
  p.V = V;
  p.V_pad = round_up(V, flce::kTile);
  p.nseg = p.V_pad / flce::kSeg;
  p.dtype = dtype;
  p.ignore_index = ignore_index;
  p.softcap = softcap;
  p.reduction = reduction;
  p.ncu = h->ncu;
  char* base = (char*)workspace;
  flce::Work& w = c.w;
  w.ws_e = base + L.off_e;
  w.seg_m = (float*)(base + L.off_m);
  w.seg_s = (float*)(base + L.off_s);
  w.y32 = (int*)(base + L.off_y);
  w.s_label = (float*)(base + L.off_sl);
  w.og = (float*)(base + L.off_og);
  w.loss_row = (float*)(base + L.off_loss);
  w.dx_part = L.splits > 1 ? (float*)(base + L.off_part) : nullptr;
  w.params = (flce::DevParams*)(base + L.off_params);
  w.xt = base + L.off_xt;
  w.chunk_cap = L.chunk_rows;
  return c;
}

}  // namespace

extern "C" {

int flce_create(flce_handle* out, int device, const flce_config* cfg) {
  if (!out) return FLCE_ERR_INVALID_ARG;
  *out = nullptr;
  int64_t cmax = kDefaultChunk;
  if (cfg) {
    for (int i = 0; i < 3; ++i)
      if (cfg->reserved[i] != 0) return FLCE_ERR_INVALID_ARG;
    if (cfg->chunk_rows_max < 0) return FLCE_ERR_INVALID_ARG;
    if (cfg->chunk_rows_max > 0) cmax = round_up(cfg->chunk_rows_max, flce::kRowAlign);
  }
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || device < 0 || device >= count) return FLCE_ERR_HIP;
  DeviceGuard g(device);
  if (!g.ok) return FLCE_ERR_HIP;
  int ncu = 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || ncu <= 0)
    return FLCE_ERR_HIP;
  int* st = nullptr;
  if (hipMalloc(&st, 256) != hipSuccess) return FLCE_ERR_HIP;
  if (hipMemset(st, 0, 256) != hipSuccess) {
    (void)hipFree(st);
    return FLCE_ERR_HIP;
  }
  flce_ctx* h = new flce_ctx;
  h->device = device;
  h->ncu = ncu;
  h->chunk_rows_max = cmax;
  h->d_status = st;
  *out = h;
  return FLCE_OK;
}

int flce_destroy(flce_handle h) {
  if (!h) return FLCE_OK;
  int rc = FLCE_OK;
  {
    DeviceGuard g(h->device);
    if (h->d_status && hipFree(h->d_status) != hipSuccess) rc = FLCE_ERR_HIP;
    for (hipEvent_t e : h->prof_events) (void)hipEventDestroy(e);
  }
  delete h;
  return rc;
}

int flce_workspace_size(flce_handle h, int64_t BT, int64_t H, int64_t V, int dtype, size_t* bytes) {
  if (!bytes) return FLCE_ERR_INVALID_ARG;
  const int rc = check_sizes(BT, H, V, dtype);
  if (rc != FLCE_OK) return rc;
  *bytes = layout(BT, H, V, dtype, chunk_max_of(h), ncu_of(h)).total;
  return FLCE_OK;
}

int flce_chunk_plan(flce_handle h, int64_t BT, int64_t* n_chunks, int64_t* chunk_rows) {
  if (!n_chunks || !chunk_rows || BT < 0) return FLCE_ERR_INVALID_ARG;
  plan(BT, chunk_max_of(h), n_chunks, chunk_rows);
  return FLCE_OK;
}

int flce_forward_backward(flce_handle h, const void* hidden, const void* W, const int64_t* labels,
                          int64_t BT, int64_t H, int64_t V, int dtype, int64_t ignore_index,
                          float softcap, int reduction, float* loss, void* grad_hidden, float* grad_W,
                          void* workspace, size_t workspace_bytes, void* stream_ptr) {
  if (!h) return FLCE_ERR_INVALID_ARG;
  int rc = check_sizes(BT, H, V, dtype);
  if (rc != FLCE_OK) return rc;
  if (reduction == FLCE_NONE) return FLCE_ERR_UNSUPPORTED;
  if (reduction != FLCE_MEAN && reduction != FLCE_SUM) return FLCE_ERR_INVALID_ARG;
  if (!(softcap >= 0.0f) || !std::isfinite(softcap)) return FLCE_ERR_INVALID_ARG;
  if (!W || !loss || !grad_W || !workspace) return FLCE_ERR_INVALID_ARG;
  if (BT > 0 && (!hidden || !labels || !grad_hidden)) return FLCE_ERR_INVALID_ARG;
  if (!aligned(W, 16) || !aligned(loss, 4) || !aligned(grad_W, 16) || !aligned(workspace, 256))
    return FLCE_ERR_INVALID_ARG;
  if (BT > 0 && (!aligned(hidden, 16) || !aligned(labels, 8) || !aligned(grad_hidden, 16)))
    return FLCE_ERR_INVALID_ARG;
  const Layout L = layout(BT, H, V, dtype, h->chunk_rows_max, h->ncu);
  if (workspace_bytes < L.total) return FLCE_ERR_WORKSPACE_TOO_SMALL;

  DeviceGuard g(h->device);
  if (!g.ok) return FLCE_ERR_HIP;
  Call call = make_call(h, L, BT, H, V, dtype, ignore_index, softcap, reduction, workspace, stream_ptr);
  const hipStream_t stream = call.stream;
  const flce::Problem& p = call.p;
  const flce::Work& w = call.w;
#define FLCE_LAUNCH(kind, expr)                                        \
  do {                                                                 \
    if (!call.run(kind, [&]() { return (expr); })) return FLCE_ERR_HIP; \
  } while (0)

  FLCE_LAUNCH(FLCE_K_PREPASS, flce::launch_prepass(p, labels, w, h->d_status, stream));
  if (BT == 0) {
    FLCE_LAUNCH(FLCE_K_FINALIZE, flce::launch_zero_f32(grad_W, V * H, stream));
    FLCE_LAUNCH(FLCE_K_FINALIZE, flce::launch_finalize(p, w, loss, stream));
    return FLCE_OK;
  }
  int64_t n_chunks, crows;
  plan(BT, h->chunk_rows_max, &n_chunks, &crows);
  for (int64_t ci = 0; ci < n_chunks; ++ci) {
    const int64_t row0 = ci * crows;
    const int64_t rows = (BT - row0) < crows ? (BT - row0) : crows;
    FLCE_LAUNCH(FLCE_K_TRANSPOSE, flce::launch_transpose(p, hidden, w, row0, rows, stream));
    FLCE_LAUNCH(FLCE_K_FWD, flce::launch_fwd(p, W, w, row0, rows, true, stream));
    FLCE_LAUNCH(FLCE_K_MERGE, flce::launch_merge(p, w, row0, rows, stream));
    int splits = L.splits > 1 ? dx_splits(rows, H, p.V_pad, dtype, h->ncu) : 1;
    if (splits > L.splits) splits = L.splits;
    FLCE_LAUNCH(FLCE_K_DX, flce::launch_dx(p, W, w, grad_hidden, row0, rows, splits, stream));
    if (splits > 1)
      FLCE_LAUNCH(FLCE_K_DX_REDUCE, flce::launch_dx_reduce(p, w, grad_hidden, row0, rows, splits, stream));
    FLCE_LAUNCH(FLCE_K_DW, flce::launch_dw(p, hidden, w, grad_W, row0, rows, ci > 0, stream));
  }
  FLCE_LAUNCH(FLCE_K_FINALIZE, flce::launch_finalize(p, w, loss, stream));
#undef FLCE_LAUNCH
  return FLCE_OK;
}

int flce_forward_workspace_size(flce_handle h, int64_t BT, int64_t H, int64_t V, int dtype, size_t* bytes) {
  if (!bytes) return FLCE_ERR_INVALID_ARG;
  const int rc = check_sizes(BT, H, V, dtype);
  if (rc != FLCE_OK) return rc;
  *bytes = layout(BT, H, V, dtype, chunk_max_of(h), ncu_of(h), false).total;
  return FLCE_OK;
}

int flce_forward(flce_handle h, const void* hidden, const void* W, const int64_t* labels, int64_t BT, int64_t H,
                 int64_t V, int dtype, int64_t ignore_index, float softcap, int reduction, float* loss,
                 float* loss_rows, float* lse_rows, void* workspace, size_t workspace_bytes, void* stream_ptr) {
  if (!h) return FLCE_ERR_INVALID_ARG;
  int rc = check_sizes(BT, H, V, dtype);
  if (rc != FLCE_OK) return rc;
  if (reduction != FLCE_NONE && reduction != FLCE_MEAN && reduction != FLCE_SUM) return FLCE_ERR_INVALID_ARG;
  if (!(softcap >= 0.0f) || !std::isfinite(softcap)) return FLCE_ERR_INVALID_ARG;
  if (!W || !workspace) return FLCE_ERR_INVALID_ARG;
  if (reduction == FLCE_NONE ? (BT > 0 && !loss_rows) : !loss) return FLCE_ERR_INVALID_ARG;
  if (BT > 0 && (!hidden || !labels)) return FLCE_ERR_INVALID_ARG;
  if (!aligned(W, 16) || !aligned(workspace, 256) || !aligned(loss, 4) || !aligned(loss_rows, 4) ||
      !aligned(lse_rows, 4))
    return FLCE_ERR_INVALID_ARG;
  if (BT > 0 && (!aligned(hidden, 16) || !aligned(labels, 8))) return FLCE_ERR_INVALID_ARG;
  const Layout L = layout(BT, H, V, dtype, h->chunk_rows_max, h->ncu, false);
  if (workspace_bytes < L.total) return FLCE_ERR_WORKSPACE_TOO_SMALL;

  DeviceGuard g(h->device);
  if (!g.ok) return FLCE_ERR_HIP;
  // per-row terms need no scale; the pre-pass's 1/N only matters for the reduced mean
  const int red = reduction == FLCE_NONE ? FLCE_SUM : reduction;
  Call call = make_call(h, L, BT, H, V, dtype, ignore_index, softcap, red, workspace, stream_ptr);
  const hipStream_t stream = call.stream;
  const flce::Problem& p = call.p;
  const flce::Work& w = call.w;
#define FLCE_LAUNCH(kind, expr)                                        \
  do {                                                                 \
    if (!call.run(kind, [&]() { return (expr); })) return FLCE_ERR_HIP; \
  } while (0)

  FLCE_LAUNCH(FLCE_K_PREPASS, flce::launch_prepass(p, labels, w, h->d_status, stream));
  int64_t n_chunks, crows;
  plan(BT, h->chunk_rows_max, &n_chunks, &crows);
  for (int64_t ci = 0; ci < n_chunks && BT > 0; ++ci) {
    const int64_t row0 = ci * crows;
    const int64_t rows = (BT - row0) < crows ? (BT - row0) : crows;
    FLCE_LAUNCH(FLCE_K_TRANSPOSE, flce::launch_transpose(p, hidden, w, row0, rows, stream));
    FLCE_LAUNCH(FLCE_K_FWD, flce::launch_fwd(p, W, w, row0, rows, false, stream));
    FLCE_LAUNCH(FLCE_K_ROWS, flce::launch_rows(p, w, row0, rows, loss_rows, lse_rows, stream));
  }
  if (reduction != FLCE_NONE) FLCE_LAUNCH(FLCE_K_FINALIZE, flce::launch_finalize(p, w, loss, stream));
#undef FLCE_LAUNCH
  return FLCE_OK;
}

int flce_status(flce_handle h, void* stream) {
  if (!h) return FLCE_ERR_INVALID_ARG;
  DeviceGuard g(h->device);
  if (!g.ok) return FLCE_ERR_HIP;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return FLCE_ERR_HIP;
  int st = 0;
  if (hipMemcpy(&st, h->d_status, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess) return FLCE_ERR_HIP;
  return st ? FLCE_ERR_LABEL_RANGE : FLCE_OK;
}

int flce_profile_begin(flce_handle h, int max_launches) {
  if (!h || max_launches <= 0) return FLCE_ERR_INVALID_ARG;
  DeviceGuard g(h->device);
  if (!g.ok) return FLCE_ERR_HIP;
  for (hipEvent_t e : h->prof_events) (void)hipEventDestroy(e);
  h->prof_events.clear();
  h->prof_kinds.clear();
  h->prof_kinds.reserve(max_launches);
  for (int i = 0; i < 2 * max_launches; ++i) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return FLCE_ERR_HIP;
    h->prof_events.push_back(e);
  }
  h->prof_on = true;
  return FLCE_OK;
}

int flce_profile_end(flce_handle h, void* stream, double* ms_out, int64_t* count_out) {
  if (!h || !ms_out || !count_out) return FLCE_ERR_INVALID_ARG;
  DeviceGuard g(h->device);
  if (!g.ok) return FLCE_ERR_HIP;
  h->prof_on = false;
  for (int k = 0; k < FLCE_K_COUNT; ++k) {
    ms_out[k] = 0.0;
    count_out[k] = 0;
  }
  int rc = FLCE_OK;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) rc = FLCE_ERR_HIP;
  for (size_t i = 0; rc == FLCE_OK && i < h->prof_kinds.size(); ++i) {
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, h->prof_events[2 * i], h->prof_events[2 * i + 1]) != hipSuccess) {
      rc = FLCE_ERR_HIP;
      break;
    }
    ms_out[h->prof_kinds[i]] += ms;
    count_out[h->prof_kinds[i]] += 1;
  }
  for (hipEvent_t e : h->prof_events) (void)hipEventDestroy(e);
  h->prof_events.clear();
  h->prof_kinds.clear();
  return rc;
}

const char* flce_error_string(int code) {
  switch (code) {
    case FLCE_OK: return "ok";
    case FLCE_ERR_INVALID_ARG: return "invalid argument";
    case FLCE_ERR_UNSUPPORTED: return "unsupported problem (H must be a multiple of 8; size limits)";
    case FLCE_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than flce_workspace_size";
    case FLCE_ERR_HIP: return "HIP runtime error";
    case FLCE_ERR_LABEL_RANGE: return "a label is outside [0, V) and is not ignore_index";
    default: return "unknown error code";
  }
}

}  // extern "C"
