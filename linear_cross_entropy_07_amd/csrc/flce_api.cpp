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
#include <utility>
#include <vector>

#include "flce.h"
#include "flce_internal.h"

struct flce_ctx {
  int device;
  int ncu;        // compute units of the device
  int64_t chunk_rows_max;
  int* d_status;  // device status word written by the label pre-pass
  void* scratch;  // this device's copy of the library's static scratch (flce_forward_backward_static)
  // kernel timing (flce_profile_begin/end): event pairs recorded around each launch
  bool prof_on = false;
  std::vector<hipEvent_t> prof_events;
  std::vector<int> prof_kinds;
};

namespace {

constexpr int64_t kDefaultChunk = 4096;
constexpr int64_t kAutoChunkWork = int64_t(1) << 24;   // rows x H: 256 tiles of 256 x 256 in grad_hidden
constexpr int64_t kAutoChunkBytes = int64_t(1) << 31;  // [rows][V] buffer bound for chunks above the default
constexpr int kDefaultCUs = 256;  // MI355X, for workspace sizes asked without a handle
constexpr int64_t kMaxH = 1 << 16;
constexpr int64_t kMaxV = int64_t(1) << 20;  // keeps every per-tile buffer range below 2 GiB
constexpr int64_t kMaxBT = (int64_t(1) << 31) - 1;

int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

// Row cap of the chunk plan: the handle's, if one was configured. Otherwise at least 4096 rows, and
// more for a narrow hidden size: enough that one chunk's grad_hidden product [rows][H] has 256 tiles
// of 256 x 256 (one per CU of the chip) without splitting the vocabulary, as long as the chunk's
// [rows][V] buffer stays within 2 GiB.
int64_t chunk_cap(const flce_ctx* h, int64_t H, int64_t V, int dtype) {
  if (h && h->chunk_rows_max > 0) return h->chunk_rows_max;
  const int64_t esz = dtype == 0 ? 2 : 4;
  const int64_t by_work = round_up((kAutoChunkWork + H - 1) / H, flce::kRowAlign);
  const int64_t by_mem = kAutoChunkBytes / (round_up(V, flce::kTile) * esz) / flce::kRowAlign * flce::kRowAlign;
  const int64_t c = by_work < by_mem ? by_work : by_mem;
  return c > kDefaultChunk ? c : kDefaultChunk;
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
  size_t off_e, off_m, off_s, off_y, off_sl, off_loss, off_cref, off_lse, off_fs, off_part, off_xt, off_xf, off_params,
      off_tail, total;
  bool tail = false;  // room for grad_W's split last wave
  int splits;
  int64_t chunk_rows;
};

// Workspace carving. The forward-only path (backward = false) needs no q chunk, no per-row lse or
// factors, no split-K partials and no scaled copy of the chunk's hidden rows.
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
  L.off_loss = take((size_t)BT * 4);
  L.off_cref = take((size_t)BT * 4);
  L.off_lse = take(backward ? (size_t)BT * 4 : 0);
  L.off_fs = take(backward ? (size_t)BT * 4 : 0);
  L.off_part = take(L.splits > 1 ? (size_t)L.splits * rows * H * 4 : 0);
  L.off_xt = take((size_t)rows * H * esz);
  L.off_xf = take(backward ? (size_t)rows * H * esz : 0);
  // grad_W's split last wave (its partial 256 x 256 fp32 tiles), for calls of several chunks: a
  // one-chunk call keeps each grad_W tile one sum in K order, as the recompute mode does
  int tail = 0;
  const int tsplits = backward && n > 1 ? flce::dw_tail_plan(V, H, rows, dtype, ncu, &tail) : 1;
  L.tail = tsplits > 1;
  L.off_tail = take(L.tail ? (size_t)tail * tsplits * flce::kTile * flce::kTile * 4 : 0);
  L.total = off;
  return L;
}

constexpr int64_t kDefaultVSlice = 8192;

// Width of the vocabulary slices of the recompute mode: a multiple of the tile width, at most V
// rounded up (0 selects the default).
int64_t vslice_of(int64_t vs, int64_t V) {
  if (vs <= 0) vs = kDefaultVSlice;
  vs = round_up(vs, flce::kTile);
  const int64_t vmax = round_up(V, flce::kTile);
  return vs < vmax ? vs : vmax;
}

// Rows of the recompute mode's single pass: all BT rows, rounded up to the row alignment.
int64_t recompute_rows(int64_t BT) { return round_up(BT, flce::kRowAlign); }

// Workspace of the recompute mode, whose one pass covers all R = recompute_rows(BT) rows: q of one
// vocabulary slice [R][slice], the statistics of the whole vocabulary [R][V_pad/128] (pass 1), the
// fp32 grad_hidden accumulator [R][H], hidden^T [H][R] and f times the hidden rows [R][H]; per row:
// label, label logit, loss term, reference, lse and f. No buffer spans the whole vocabulary for more
// than its 128-wide segment statistics.
Layout layout_recompute(int64_t BT, int64_t H, int64_t V, int dtype, int64_t vs) {
  Layout L{};
  const int64_t rows = recompute_rows(BT);
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
  L.splits = 1;
  L.off_params = take(sizeof(flce::DevParams));
  L.off_e = take((size_t)rows * vslice_of(vs, V) * esz);
  L.off_m = take((size_t)rows * nseg * 4);
  L.off_s = take((size_t)rows * nseg * 4);
  L.off_y = take((size_t)BT * 4);
  L.off_sl = take((size_t)BT * 4);
  L.off_loss = take((size_t)BT * 4);
  L.off_cref = take((size_t)BT * 4);
  L.off_lse = take((size_t)BT * 4);
  L.off_fs = take((size_t)BT * 4);
  L.off_part = take((size_t)rows * H * 4);
  L.off_xt = take((size_t)rows * H * esz);
  L.off_xf = take((size_t)rows * H * esz);
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

// Rows of one call: where row r's hidden, grad_hidden and label live.
struct Rows {
  int64_t B = 0, T = 0, shift = 0, BT = 0;
  flce::RowMap hmap{}, gmap{}, lmap{};
};

// The plain layout: hidden and grad_hidden [BT][H], labels [BT].
Rows plain_rows(int64_t BT, int64_t H) {
  Rows r;
  r.B = BT;
  r.T = 1;
  r.BT = BT;
  r.hmap = flce::RowMap{H, 0, 0, 1};
  r.gmap = r.hmap;
  r.lmap = flce::RowMap{1, 0, 0, 1};
  return r;
}

// True if rows (b, t) of extents (n0, n1) with element strides (s0, s1) and `width` elements each
// never share an element: with the strides ordered (s0 <= s1), the inner stride steps past a row
// and the outer stride steps past the whole inner span, s1 >= (n0 - 1) * s0 + width (checked
// without overflow).
bool no_overlap(int64_t n0, int64_t s0, int64_t n1, int64_t s1, int64_t width) {
  if (n0 <= 1) s0 = 0, n0 = 1;
  if (n1 <= 1) s1 = 0, n1 = 1;
  if (n0 == 1 && n1 == 1) return true;
  if (n0 == 1) return s1 >= width;
  if (n1 == 1) return s0 >= width;
  if (s0 > s1) {
    std::swap(s0, s1);
    std::swap(n0, n1);
  }
  return s0 >= width && s1 >= width && (s1 - width) / s0 >= n0 - 1;
}

// Validates a flce_rows description (see include/flce.h) and derives the row maps.
int check_rows(const flce_rows* d, int64_t H, int dtype, bool grads, Rows* out) {
  if (!d) return FLCE_ERR_INVALID_ARG;
  if (d->batch < 0 || d->seq < 0 || (d->shift != 0 && d->shift != 1)) return FLCE_ERR_INVALID_ARG;
  for (int i = 0; i < 2; ++i)
    if (d->hidden_stride[i] < 0 || d->label_stride[i] < 0 || (grads && d->grad_hidden_stride[i] < 0))
      return FLCE_ERR_INVALID_ARG;
  const int64_t per = d->seq > d->shift ? d->seq - d->shift : 0;
  if (d->batch > 0 && per > 0 && d->batch > kMaxBT / per) return FLCE_ERR_UNSUPPORTED;
  // 16-byte aligned rows: element strides of hidden and grad_hidden are multiples of 16 bytes
  const int64_t al = dtype == FLCE_BF16 ? 8 : 4;
  for (int i = 0; i < 2; ++i)
    if (d->hidden_stride[i] % al != 0 || (grads && d->grad_hidden_stride[i] % al != 0))
      return FLCE_ERR_INVALID_ARG;
  // every grad_hidden row is written (rows of the call, and the skipped last positions when the
  // labels are shifted), so no two of them may share an element
  if (grads && !no_overlap(d->batch, d->grad_hidden_stride[0], d->seq, d->grad_hidden_stride[1], H))
    return FLCE_ERR_INVALID_ARG;
  Rows r;
  r.B = d->batch;
  r.T = d->seq;
  r.shift = d->shift;
  r.BT = d->batch * per;
  const uint32_t up = (uint32_t)(per > 0 ? per : 1);
  r.hmap = flce::RowMap{d->hidden_stride[0], d->hidden_stride[1], 0, up};
  r.gmap = flce::RowMap{d->grad_hidden_stride[0], d->grad_hidden_stride[1], 0, up};
  r.lmap = flce::RowMap{d->label_stride[0], d->label_stride[1], d->shift * d->label_stride[1], up};
  *out = r;
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

Call make_call(flce_ctx* h, const Layout& L, const Rows& R, int64_t H, int64_t V, int dtype,
               int64_t ignore_index, float softcap, int reduction, float grad_scale, int flags, void* workspace,
               void* stream) {
  Call c;
  c.h = h;
  c.stream = (hipStream_t)stream;
  flce::Problem& p = c.p;
  p.BT = R.BT;
  p.hmap = R.hmap;
  p.gmap = R.gmap;
  p.lmap = R.lmap;
  p.grad_scale = grad_scale;
  p.acc_gh = (flags & FLCE_ACCUMULATE_GRAD_HIDDEN) != 0;
  p.acc_gw = (flags & FLCE_ACCUMULATE_GRAD_W) != 0;
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
  w.loss_row = (float*)(base + L.off_loss);
  w.cref = (float*)(base + L.off_cref);
  w.lse = (float*)(base + L.off_lse);
  w.fscale = (float*)(base + L.off_fs);
  w.dx_part = L.splits > 1 ? (float*)(base + L.off_part) : nullptr;
  w.params = (flce::DevParams*)(base + L.off_params);
  w.xt = base + L.off_xt;
  w.xf = base + L.off_xf;
  w.dw_tail = L.tail ? (float*)(base + L.off_tail) : nullptr;
  w.chunk_cap = L.chunk_rows;
  return c;
}

#define FLCE_LAUNCH(kind, expr)                                        \
  do {                                                                 \
    if (!call.run(kind, [&]() { return (expr); })) return FLCE_ERR_HIP; \
  } while (0)

// The fused forward + backward over the rows R (sizes already checked).
// cmax: the chunk cap (0 = the handle's).
int run_fused(flce_ctx* h, int64_t cmax, const void* hidden, const void* W, const int64_t* labels, const Rows& R,
              int64_t H, int64_t V, int dtype, int64_t ignore_index, float softcap, int reduction, float grad_scale,
              int flags, float* loss, void* grad_hidden, float* grad_W, void* workspace, size_t workspace_bytes,
              void* stream_ptr) {
  const int64_t BT = R.BT;
  if (reduction == FLCE_NONE) return FLCE_ERR_UNSUPPORTED;
  if (reduction != FLCE_MEAN && reduction != FLCE_SUM) return FLCE_ERR_INVALID_ARG;
  if (!(softcap >= 0.0f) || !std::isfinite(softcap)) return FLCE_ERR_INVALID_ARG;
  // one of the two gradients may be left out (a frozen weight or a frozen input); not both
  const bool need_gh = (flags & FLCE_NO_GRAD_HIDDEN) == 0, need_gw = (flags & FLCE_NO_GRAD_W) == 0;
  if (!need_gh && !need_gw) return FLCE_ERR_INVALID_ARG;
  if ((!need_gh && (flags & FLCE_ACCUMULATE_GRAD_HIDDEN)) || (!need_gw && (flags & FLCE_ACCUMULATE_GRAD_W)))
    return FLCE_ERR_INVALID_ARG;
  if (!W || !loss || (need_gw && !grad_W) || !workspace) return FLCE_ERR_INVALID_ARG;
  // grad_hidden is written on every row of the call and on the skipped last positions
  const bool gh_rows = need_gh && (BT > 0 || (R.shift == 1 && R.B > 0 && R.T > 0));
  if ((BT > 0 && (!hidden || !labels)) || (gh_rows && !grad_hidden)) return FLCE_ERR_INVALID_ARG;
  if (!aligned(W, 16) || !aligned(loss, 4) || (need_gw && !aligned(grad_W, 16)) || !aligned(workspace, 256))
    return FLCE_ERR_INVALID_ARG;
  if (BT > 0 && (!aligned(hidden, 16) || !aligned(labels, 8))) return FLCE_ERR_INVALID_ARG;
  if (gh_rows && !aligned(grad_hidden, 16)) return FLCE_ERR_INVALID_ARG;
  if (cmax <= 0) cmax = chunk_cap(h, H, V, dtype);  // 0: the handle's chunk cap
  const Layout L = layout(BT, H, V, dtype, cmax, h->ncu, true);
  if (workspace_bytes < L.total) return FLCE_ERR_WORKSPACE_TOO_SMALL;

  DeviceGuard g(h->device);
  if (!g.ok) return FLCE_ERR_HIP;
  Call call = make_call(h, L, R, H, V, dtype, ignore_index, softcap, reduction, grad_scale, flags, workspace,
                        stream_ptr);
  const hipStream_t stream = call.stream;
  const flce::Problem& p = call.p;
  const flce::Work& w = call.w;

  FLCE_LAUNCH(FLCE_K_PREPASS, flce::launch_prepass(p, labels, w, h->d_status, stream));
  // the last position of each sequence is no row when labels are shifted: its gradient is zero
  if (need_gh && R.shift == 1 && R.T > 0 && !p.acc_gh)
    FLCE_LAUNCH(FLCE_K_ZERO, flce::launch_zero_rows(p, grad_hidden, R.B, (R.T - 1) * R.gmap.st, stream));
  if (BT == 0) {
    if (need_gw && !p.acc_gw) FLCE_LAUNCH(FLCE_K_ZERO, flce::launch_zero_f32(grad_W, V * H, stream));
    FLCE_LAUNCH(FLCE_K_FINALIZE, flce::launch_finalize(p, w, loss, stream));
    return FLCE_OK;
  }
  int64_t n_chunks, crows;
  plan(BT, cmax, &n_chunks, &crows);
  for (int64_t ci = 0; ci < n_chunks; ++ci) {
    const int64_t row0 = ci * crows;
    const int64_t rows = (BT - row0) < crows ? (BT - row0) : crows;
    FLCE_LAUNCH(FLCE_K_TRANSPOSE, flce::launch_transpose(p, hidden, w, row0, rows, stream));
    FLCE_LAUNCH(FLCE_K_ROWREF, flce::launch_rowref(p, hidden, W, w, row0, rows, stream));
    FLCE_LAUNCH(FLCE_K_FWD, flce::launch_fwd(p, W, w, row0, rows, true, stream));
    FLCE_LAUNCH(FLCE_K_LSE, flce::launch_lse(p, w, row0, rows, true, stream));
    FLCE_LAUNCH(FLCE_K_ROWFIX, flce::launch_rowfix(p, hidden, w, row0, rows, stream, flce::VSlice{}, 3));
    if (need_gh) {
      int splits = L.splits > 1 ? dx_splits(rows, H, p.V_pad, dtype, h->ncu) : 1;
      if (splits > L.splits) splits = L.splits;
      FLCE_LAUNCH(FLCE_K_DX, flce::launch_dx(p, W, w, grad_hidden, row0, rows, splits, stream));
      if (splits > 1)
        FLCE_LAUNCH(FLCE_K_DX_REDUCE, flce::launch_dx_reduce(p, w, grad_hidden, row0, rows, splits, stream));
    }
    if (need_gw) FLCE_LAUNCH(FLCE_K_DW, flce::launch_dw(p, w, grad_W, rows, ci > 0 || p.acc_gw, stream));
  }
  FLCE_LAUNCH(FLCE_K_FINALIZE, flce::launch_finalize(p, w, loss, stream));
  return FLCE_OK;
}

// The recompute mode over the rows R (plain layout; sizes already checked), vocabulary slices
// outermost over all rows at once: the forward pass over the whole vocabulary gives each row's lse
// and maximum, hence its final reference and its factor f; then per vocabulary slice the logits are
// formed again into q against that reference (the label entry folded in when the label lies in the
// slice) and used at once for the slice's grad_W rows, written once, and for the fp32 grad_hidden
// sum over slices, which is multiplied by f at the end.
int run_recompute(flce_ctx* h, const void* hidden, const void* W, const int64_t* labels, const Rows& R, int64_t H,
                  int64_t V, int dtype, int64_t ignore_index, float softcap, int reduction, int64_t v_slice,
                  float* loss, void* grad_hidden, float* grad_W, void* workspace, size_t workspace_bytes,
                  void* stream_ptr) {
  const int64_t BT = R.BT;
  if (reduction == FLCE_NONE) return FLCE_ERR_UNSUPPORTED;
  if (reduction != FLCE_MEAN && reduction != FLCE_SUM) return FLCE_ERR_INVALID_ARG;
  if (!(softcap >= 0.0f) || !std::isfinite(softcap)) return FLCE_ERR_INVALID_ARG;
  if (v_slice < 0) return FLCE_ERR_INVALID_ARG;
  if (!W || !loss || !grad_W || !workspace) return FLCE_ERR_INVALID_ARG;
  if (BT > 0 && (!hidden || !labels || !grad_hidden)) return FLCE_ERR_INVALID_ARG;
  if (!aligned(W, 16) || !aligned(loss, 4) || !aligned(grad_W, 16) || !aligned(workspace, 256))
    return FLCE_ERR_INVALID_ARG;
  if (BT > 0 && (!aligned(hidden, 16) || !aligned(labels, 8) || !aligned(grad_hidden, 16)))
    return FLCE_ERR_INVALID_ARG;
  const int64_t vs = vslice_of(v_slice, V);
  const Layout L = layout_recompute(BT, H, V, dtype, vs);
  if (workspace_bytes < L.total) return FLCE_ERR_WORKSPACE_TOO_SMALL;

  DeviceGuard g(h->device);
  if (!g.ok) return FLCE_ERR_HIP;
  Call call = make_call(h, L, R, H, V, dtype, ignore_index, softcap, reduction, 1.0f, 0, workspace, stream_ptr);
  const hipStream_t stream = call.stream;
  const flce::Problem& p = call.p;
  flce::Work& w = call.w;
  w.dx_part = (float*)((char*)workspace + L.off_part);

  FLCE_LAUNCH(FLCE_K_PREPASS, flce::launch_prepass(p, labels, w, h->d_status, stream));
  if (BT == 0) {
    FLCE_LAUNCH(FLCE_K_ZERO, flce::launch_zero_f32(grad_W, V * H, stream));
    FLCE_LAUNCH(FLCE_K_FINALIZE, flce::launch_finalize(p, w, loss, stream));
    return FLCE_OK;
  }
  const int64_t row0 = 0, rows = BT;
  FLCE_LAUNCH(FLCE_K_TRANSPOSE, flce::launch_transpose(p, hidden, w, row0, rows, stream));
  FLCE_LAUNCH(FLCE_K_ROWREF, flce::launch_rowref(p, hidden, W, w, row0, rows, stream));
  // pass 1: row statistics over the whole vocabulary -> lse, the loss terms, the final references
  FLCE_LAUNCH(FLCE_K_FWD, flce::launch_fwd(p, W, w, row0, rows, false, stream));
  FLCE_LAUNCH(FLCE_K_LSE, flce::launch_lse(p, w, row0, rows, false, stream));
  FLCE_LAUNCH(FLCE_K_ROWFIX, flce::launch_rowfix(p, hidden, w, row0, rows, stream, flce::VSlice{}, 1));
  // pass 2: per vocabulary slice over all rows
  for (int64_t v0 = 0, si = 0; v0 < V; v0 += vs, ++si) {
    const flce::VSlice sl{v0, (V - v0) < vs ? (V - v0) : vs};
    FLCE_LAUNCH(FLCE_K_FWD, flce::launch_fwd(p, W, w, row0, rows, true, stream, sl, true));
    FLCE_LAUNCH(FLCE_K_ROWFIX, flce::launch_rowfix(p, hidden, w, row0, rows, stream, sl, 2));
    FLCE_LAUNCH(FLCE_K_DX, flce::launch_dx(p, W, w, grad_hidden, row0, rows, 1, stream, sl, si == 0 ? 1 : 2));
    FLCE_LAUNCH(FLCE_K_DW, flce::launch_dw(p, w, grad_W, rows, false, stream, sl));
  }
  FLCE_LAUNCH(FLCE_K_DX_REDUCE, flce::launch_dx_reduce(p, w, grad_hidden, row0, rows, 1, stream));
  FLCE_LAUNCH(FLCE_K_FINALIZE, flce::launch_finalize(p, w, loss, stream));
  return FLCE_OK;
}

// The forward alone over the rows R (sizes already checked).
int run_forward(flce_ctx* h, const void* hidden, const void* W, const int64_t* labels, const Rows& R, int64_t H,
                int64_t V, int dtype, int64_t ignore_index, float softcap, int reduction, float* loss,
                float* loss_rows, float* lse_rows, void* workspace, size_t workspace_bytes, void* stream_ptr) {
  const int64_t BT = R.BT;
  if (reduction != FLCE_NONE && reduction != FLCE_MEAN && reduction != FLCE_SUM) return FLCE_ERR_INVALID_ARG;
  if (!(softcap >= 0.0f) || !std::isfinite(softcap)) return FLCE_ERR_INVALID_ARG;
  if (!W || !workspace) return FLCE_ERR_INVALID_ARG;
  if (reduction == FLCE_NONE ? (BT > 0 && !loss_rows) : !loss) return FLCE_ERR_INVALID_ARG;
  if (BT > 0 && (!hidden || !labels)) return FLCE_ERR_INVALID_ARG;
  if (!aligned(W, 16) || !aligned(workspace, 256) || !aligned(loss, 4) || !aligned(loss_rows, 4) ||
      !aligned(lse_rows, 4))
    return FLCE_ERR_INVALID_ARG;
  if (BT > 0 && (!aligned(hidden, 16) || !aligned(labels, 8))) return FLCE_ERR_INVALID_ARG;
  const int64_t cmax = chunk_cap(h, H, V, dtype);
  const Layout L = layout(BT, H, V, dtype, cmax, h->ncu, false);
  if (workspace_bytes < L.total) return FLCE_ERR_WORKSPACE_TOO_SMALL;

  DeviceGuard g(h->device);
  if (!g.ok) return FLCE_ERR_HIP;
  // per-row terms need no scale; the pre-pass's 1/N only matters for the reduced mean
  const int red = reduction == FLCE_NONE ? FLCE_SUM : reduction;
  Call call = make_call(h, L, R, H, V, dtype, ignore_index, softcap, red, 1.0f, 0, workspace, stream_ptr);
  const hipStream_t stream = call.stream;
  const flce::Problem& p = call.p;
  const flce::Work& w = call.w;

  FLCE_LAUNCH(FLCE_K_PREPASS, flce::launch_prepass(p, labels, w, h->d_status, stream));
  int64_t n_chunks, crows;
  plan(BT, cmax, &n_chunks, &crows);
  for (int64_t ci = 0; ci < n_chunks && BT > 0; ++ci) {
    const int64_t row0 = ci * crows;
    const int64_t rows = (BT - row0) < crows ? (BT - row0) : crows;
    FLCE_LAUNCH(FLCE_K_TRANSPOSE, flce::launch_transpose(p, hidden, w, row0, rows, stream));
    FLCE_LAUNCH(FLCE_K_ROWREF, flce::launch_rowref(p, hidden, W, w, row0, rows, stream));
    FLCE_LAUNCH(FLCE_K_FWD, flce::launch_fwd(p, W, w, row0, rows, false, stream));
    FLCE_LAUNCH(FLCE_K_ROWS, flce::launch_rows(p, w, row0, rows, loss_rows, lse_rows, stream));
  }
  if (reduction != FLCE_NONE) FLCE_LAUNCH(FLCE_K_FINALIZE, flce::launch_finalize(p, w, loss, stream));
  return FLCE_OK;
}
#undef FLCE_LAUNCH

}  // namespace

extern "C" {

int flce_create(flce_handle* out, int device, const flce_config* cfg) {
  if (!out) return FLCE_ERR_INVALID_ARG;
  *out = nullptr;
  int64_t cmax = 0;  // automatic (chunk_cap)
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
  // this device's copy of the static scratch, looked up once per device with the device current
  void* scratch = nullptr;
  if (flce::scratch_for_device(device, &scratch) != hipSuccess) return FLCE_ERR_HIP;
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
  h->scratch = scratch;
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
  *bytes = layout(BT, H, V, dtype, chunk_cap(h, H, V, dtype), ncu_of(h)).total;
  return FLCE_OK;
}

int flce_chunk_plan(flce_handle h, int64_t BT, int64_t H, int64_t V, int dtype, int64_t* n_chunks,
                    int64_t* chunk_rows) {
  if (!n_chunks || !chunk_rows) return FLCE_ERR_INVALID_ARG;
  const int rc = check_sizes(BT, H, V, dtype);
  if (rc != FLCE_OK) return rc;
  plan(BT, chunk_cap(h, H, V, dtype), n_chunks, chunk_rows);
  return FLCE_OK;
}

int flce_forward_backward(flce_handle h, const void* hidden, const void* W, const int64_t* labels,
                          int64_t BT, int64_t H, int64_t V, int dtype, int64_t ignore_index,
                          float softcap, int reduction, float* loss, void* grad_hidden, float* grad_W,
                          void* workspace, size_t workspace_bytes, void* stream_ptr) {
  if (!h) return FLCE_ERR_INVALID_ARG;
  const int rc = check_sizes(BT, H, V, dtype);
  if (rc != FLCE_OK) return rc;
  return run_fused(h, 0, hidden, W, labels, plain_rows(BT, H), H, V, dtype, ignore_index, softcap, reduction, 1.0f,
                   0, loss, grad_hidden, grad_W, workspace, workspace_bytes, stream_ptr);
}

int flce_forward_backward_static(flce_handle h, const void* hidden, const void* W, const int64_t* labels,
                                 int64_t BT, int64_t H, int64_t V, int dtype, int64_t ignore_index,
                                 float softcap, int reduction, float* loss, void* grad_hidden, float* grad_W,
                                 void* stream) {
  if (!h) return FLCE_ERR_INVALID_ARG;
  const int rc = check_sizes(BT, H, V, dtype);
  if (rc != FLCE_OK) return rc;
  if (!h->scratch) return FLCE_ERR_HIP;
  // the largest chunk (a multiple of 256 rows, at most the handle's cap) whose workspace fits the scratch
  int64_t cmax = chunk_cap(h, H, V, dtype);
  while (cmax >= flce::kRowAlign && layout(BT, H, V, dtype, cmax, h->ncu).total > flce::kScratchBytes)
    cmax -= flce::kRowAlign;
  if (cmax < flce::kRowAlign) return FLCE_ERR_WORKSPACE_TOO_SMALL;
  return run_fused(h, cmax, hidden, W, labels, plain_rows(BT, H), H, V, dtype, ignore_index, softcap, reduction,
                   1.0f, 0, loss, grad_hidden, grad_W, h->scratch, flce::kScratchBytes, stream);
}

int flce_workspace_size_rows(flce_handle h, const flce_rows* rows, int64_t H, int64_t V, int dtype,
                             size_t* bytes) {
  if (!bytes || !rows) return FLCE_ERR_INVALID_ARG;
  Rows R;
  int rc = check_rows(rows, H, dtype, true, &R);
  if (rc == FLCE_OK) rc = check_sizes(R.BT, H, V, dtype);
  if (rc != FLCE_OK) return rc;
  *bytes = layout(R.BT, H, V, dtype, chunk_cap(h, H, V, dtype), ncu_of(h), true).total;
  return FLCE_OK;
}

int flce_forward_backward_rows(flce_handle h, const void* hidden, const void* W, const int64_t* labels,
                               const flce_rows* rows, int64_t H, int64_t V, int dtype, int64_t ignore_index,
                               float softcap, int reduction, float grad_scale, int flags, float* loss,
                               void* grad_hidden, float* grad_W, void* workspace, size_t workspace_bytes,
                               void* stream_ptr) {
  if (!h || !rows) return FLCE_ERR_INVALID_ARG;
  Rows R;
  int rc = check_rows(rows, H, dtype, true, &R);
  if (rc == FLCE_OK) rc = check_sizes(R.BT, H, V, dtype);
  if (rc != FLCE_OK) return rc;
  if (!std::isfinite(grad_scale)) return FLCE_ERR_INVALID_ARG;
  if (flags & ~(FLCE_ACCUMULATE_GRAD_HIDDEN | FLCE_ACCUMULATE_GRAD_W | FLCE_NO_GRAD_HIDDEN | FLCE_NO_GRAD_W))
    return FLCE_ERR_INVALID_ARG;
  return run_fused(h, 0, hidden, W, labels, R, H, V, dtype, ignore_index, softcap, reduction, grad_scale, flags,
                   loss, grad_hidden, grad_W, workspace, workspace_bytes, stream_ptr);
}

int flce_recompute_workspace_size(flce_handle h, int64_t BT, int64_t H, int64_t V, int dtype, int64_t v_slice,
                                  size_t* bytes) {
  if (!bytes || v_slice < 0) return FLCE_ERR_INVALID_ARG;
  const int rc = check_sizes(BT, H, V, dtype);
  if (rc != FLCE_OK) return rc;
  *bytes = layout_recompute(BT, H, V, dtype, vslice_of(v_slice, V)).total;
  return FLCE_OK;
}

int flce_forward_backward_recompute(flce_handle h, const void* hidden, const void* W, const int64_t* labels,
                                    int64_t BT, int64_t H, int64_t V, int dtype, int64_t ignore_index,
                                    float softcap, int reduction, int64_t v_slice, float* loss, void* grad_hidden,
                                    float* grad_W, void* workspace, size_t workspace_bytes, void* stream_ptr) {
  if (!h) return FLCE_ERR_INVALID_ARG;
  const int rc = check_sizes(BT, H, V, dtype);
  if (rc != FLCE_OK) return rc;
  return run_recompute(h, hidden, W, labels, plain_rows(BT, H), H, V, dtype, ignore_index, softcap, reduction,
                       v_slice, loss, grad_hidden, grad_W, workspace, workspace_bytes, stream_ptr);
}

int flce_forward_workspace_size(flce_handle h, int64_t BT, int64_t H, int64_t V, int dtype, size_t* bytes) {
  if (!bytes) return FLCE_ERR_INVALID_ARG;
  const int rc = check_sizes(BT, H, V, dtype);
  if (rc != FLCE_OK) return rc;
  *bytes = layout(BT, H, V, dtype, chunk_cap(h, H, V, dtype), ncu_of(h), false).total;
  return FLCE_OK;
}

int flce_forward(flce_handle h, const void* hidden, const void* W, const int64_t* labels, int64_t BT, int64_t H,
                 int64_t V, int dtype, int64_t ignore_index, float softcap, int reduction, float* loss,
                 float* loss_rows, float* lse_rows, void* workspace, size_t workspace_bytes, void* stream_ptr) {
  if (!h) return FLCE_ERR_INVALID_ARG;
  const int rc = check_sizes(BT, H, V, dtype);
  if (rc != FLCE_OK) return rc;
  return run_forward(h, hidden, W, labels, plain_rows(BT, H), H, V, dtype, ignore_index, softcap, reduction, loss,
                     loss_rows, lse_rows, workspace, workspace_bytes, stream_ptr);
}

int flce_forward_rows(flce_handle h, const void* hidden, const void* W, const int64_t* labels, const flce_rows* rows,
                      int64_t H, int64_t V, int dtype, int64_t ignore_index, float softcap, int reduction,
                      float* loss, float* loss_rows, float* lse_rows, void* workspace, size_t workspace_bytes,
                      void* stream_ptr) {
  if (!h || !rows) return FLCE_ERR_INVALID_ARG;
  Rows R;
  int rc = check_rows(rows, H, dtype, false, &R);
  if (rc == FLCE_OK) rc = check_sizes(R.BT, H, V, dtype);
  if (rc != FLCE_OK) return rc;
  return run_forward(h, hidden, W, labels, R, H, V, dtype, ignore_index, softcap, reduction, loss, loss_rows,
                     lse_rows, workspace, workspace_bytes, stream_ptr);
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
    case FLCE_ERR_WORKSPACE_TOO_SMALL:
      return "workspace smaller than flce_workspace_size (flce_forward_backward_static: the problem needs more "
             "than the library's static scratch even in 256-row chunks)";
    case FLCE_ERR_HIP: return "HIP runtime error";
    case FLCE_ERR_LABEL_RANGE: return "a label is outside [0, V) and is not ignore_index";
    default: return "unknown error code";
  }
}

}  // extern "C"
