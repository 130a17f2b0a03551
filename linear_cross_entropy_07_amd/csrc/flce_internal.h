// Internal interface between the host scheduler (flce_api.cpp) and the kernels (flce_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace flce {

// Tile geometry shared by host planning and kernels.
constexpr int kTile = 256;      // rows/cols of every GEMM block tile
constexpr int kSeg = 128;       // width (in V) of one row-statistics segment (one wave's M extent)
constexpr int kRowAlign = 256;  // chunk sizes are multiples of this
#ifndef FLCE_STEP_BYTES
#define FLCE_STEP_BYTES 64
#endif
#ifndef FLCE_STAGES
#define FLCE_STAGES 4
#endif
constexpr int kStepBytes = FLCE_STEP_BYTES;  // bytes of K per GEMM pipeline step (64 or 128)
constexpr int kPipeStages = FLCE_STAGES;     // LDS stages of the GEMM pipeline

// Row r of a call -> element offset of its first element in a tensor of sequences: r = b * per + t
// (per = rows per sequence), offset = b * sb + t * st + base. The plain [BT][ld] layout is
// {sb = ld, st = 0, base = 0, per = 1}. Row indices and per fit in 31 bits.
struct RowMap {
  int64_t sb, st, base;
  uint32_t per;
  __host__ __device__ __forceinline__ int64_t operator()(int64_t r) const {
    const uint32_t b = (uint32_t)r / per, t = (uint32_t)r - b * per;
    return (int64_t)b * sb + (int64_t)t * st + base;
  }
};

// Per-call device parameters written by the label pre-pass and read by later kernels.
struct DevParams {
  int n_valid;   // N = number of rows whose label is in [0, V)
  float ginv;    // grad_scale * (1/N (mean, N > 0), 0 (mean, N == 0), 1 (sum))
  int status;    // bit 0: a label outside [0, V) that is not ignore_index was seen
  int pad;
};

// Views of the workspace for one call (carved by the host).
struct Work {
  void* ws_e;          // chunk_rows x V_pad q = exp(s - c) (softcap derivative), bf16 or fp32, in blocks
                       // of 256 rows x one 64-byte K step, ordered by tile of rows, then by v
  float* seg_m;        // [chunk_rows][nseg]: segment max
  float* seg_s;        // [chunk_rows][nseg]: segment sum of exp(s - segment max)
  int* y32;            // [BT] label or -1 for rows that do not count
  float* s_label;      // [BT] softcapped label logit (written by the logits epilogue)
  float* loss_row;     // [BT]
  float* cref;         // [BT] reference c of each row (label logit, or the row maximum)
  float* lse;          // [BT] log-sum-exp of each row
  float* fscale;       // [BT] f = g exp(c - lse): dZ = f q away from the label
  float* dx_part;      // [splits][chunk_rows][H] fp32 split-K partials of grad_hidden (may be null)
  void* xt;            // [H][chunk_cap] the current chunk of hidden, transposed
  void* xf;            // [chunk_cap][H] f times the current chunk's rows of hidden (grad_W operand)
  float* dw_tail;      // [tail][splits][256][256] fp32 partial tiles of grad_W's split last wave (null: no split)
  int64_t chunk_cap;   // row capacity of one chunk (a multiple of 256)
  DevParams* params;   // in the workspace
};

struct Problem {
  int64_t BT, H, V, V_pad, nseg;
  int dtype;           // 0 bf16, 1 fp32
  int64_t ignore_index;
  float softcap;
  int reduction;       // 1 mean, 2 sum
  int ncu;             // compute units of the device (sizes persistent grids)
  RowMap hmap;         // rows of hidden (elements)
  RowMap gmap;         // rows of grad_hidden (elements)
  RowMap lmap;         // labels (elements)
  float grad_scale;    // multiplies both gradients
  bool acc_gh, acc_gw; // add into grad_hidden / grad_W instead of overwriting
};

// A slice of the vocabulary: W rows v0 .. v0 + vn - 1 (vn < 0: the whole vocabulary). Slices other
// than the last are multiples of the tile width, so tiles and 128-wide segments line up with those
// of the whole vocabulary.
struct VSlice {
  int64_t v0 = 0, vn = -1;
};

// Launchers (all enqueue on `stream`, return hipError_t of the launch).
hipError_t launch_prepass(const Problem& p, const int64_t* labels, const Work& w, int* status_out,
                          hipStream_t stream);
hipError_t launch_transpose(const Problem& p, const void* hidden, const Work& w, int64_t row0, int64_t rows,
                            hipStream_t stream);
// store_q: write q (else the forward-only path); qonly: write q but no statistics or label logits.
hipError_t launch_fwd(const Problem& p, const void* W, const Work& w, int64_t row0, int64_t rows,
                      bool store_q, hipStream_t stream, VSlice vs = VSlice{}, bool qonly = false);
hipError_t launch_rows(const Problem& p, const Work& w, int64_t row0, int64_t rows, float* loss_rows,
                       float* lse_rows, hipStream_t stream);
// per-row reference (label logit) of a chunk
hipError_t launch_rowref(const Problem& p, const void* hidden, const void* W, const Work& w, int64_t row0,
                         int64_t rows, hipStream_t stream);
// per-row lse and loss term; references moved to the row maximum where needed, with rescale_q the
// stored q of those rows rescaled to match
hipError_t launch_lse(const Problem& p, const Work& w, int64_t row0, int64_t rows, bool rescale_q,
                      hipStream_t stream);
// mode bit 1: f and hidden_f; bit 2: the label entry of q (labels within the slice vs)
hipError_t launch_rowfix(const Problem& p, const void* hidden, const Work& w, int64_t row0, int64_t rows,
                         hipStream_t stream, VSlice vs, int mode);
// part_mode: 0 the normal output, 1 write the fp32 [rows][H] partials (one split), 2 add to them.
hipError_t launch_dx(const Problem& p, const void* W, const Work& w, void* grad_hidden, int64_t row0,
                     int64_t rows, int splits, hipStream_t stream, VSlice vs = VSlice{}, int part_mode = 0);
// grad_hidden rows that are no rows of the call (the last position of each sequence when labels are
// shifted): zero-filled. B sequences, element offset `off` of the row in sequence 0.
hipError_t launch_zero_rows(const Problem& p, void* grad_hidden, int64_t B, int64_t off, hipStream_t stream);
hipError_t launch_dx_reduce(const Problem& p, const Work& w, void* grad_hidden, int64_t row0, int64_t rows,
                            int splits, hipStream_t stream);
// grad_W's last wave: the number of K parts its tiles are split into (1: none) and, through `tail`,
// how many tiles that wave has, for a launch over V x H with `rows` of K on `ncu` CUs.
int dw_tail_plan(int64_t V, int64_t H, int64_t rows, int dtype, int ncu, int* tail);
hipError_t launch_dw(const Problem& p, const Work& w, float* grad_W, int64_t rows, bool accumulate,
                     hipStream_t stream, VSlice vs = VSlice{});
hipError_t launch_finalize(const Problem& p, const Work& w, float* loss, hipStream_t stream);
hipError_t launch_zero_f32(float* ptr, int64_t n, hipStream_t stream);

// Library-owned static device scratch (the allocation-free entry point's workspace): kScratchBytes
// per device, held by the loaded code object until the process ends. scratch_for_device() must be
// called with `device` current; it looks the array's address up once per device and returns it.
constexpr size_t kScratchBytes = size_t(256) << 20;
constexpr int kMaxDevices = 64;
hipError_t scratch_for_device(int device, void** out);

}  // namespace flce
