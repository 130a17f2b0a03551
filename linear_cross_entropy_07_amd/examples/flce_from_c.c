/*
 * flce_from_c.c - calling libflce.so from plain C99 through include/flce.h, with device memory from
 * the HIP runtime and no other framework.
 *
 * usage: flce_from_c <inputs.bin> <outputs.bin>
 *
 * inputs.bin  (little endian): int64 BT, H, V; float softcap; int32 reduction (FLCE_MEAN or
 *             FLCE_SUM); int64 B (sequences for the sequence call, dividing BT); float grad_scale;
 *             then hidden [BT][H] and W [V][H] as bf16 bit patterns (uint16), labels [BT] int64.
 * outputs.bin: four calls on the same data, then int32 status of each call (flce_status):
 *             1. flce_forward_backward: float loss; grad_hidden [BT][H] bf16 bit patterns; grad_W
 *                [V][H] float;
 *             2. flce_forward with FLCE_NONE: loss_rows [BT] float, lse_rows [BT] float;
 *             3. flce_forward_backward_recompute with 256-wide vocabulary slices: as 1;
 *             4. flce_forward_backward_rows over the rows as B sequences of T = BT / B positions,
 *                each position scored against the next one's label (shift 1), gradients times
 *                grad_scale: as 1 (the last position of each sequence gets a zero gradient row).
 * Exit code 0 on success; on any error a message names the failing call.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "flce.h"

#define HIP_OK(call)                                                            \
  do {                                                                          \
    hipError_t e_ = (call);                                                     \
    if (e_ != hipSuccess) {                                                     \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));         \
      return 1;                                                                 \
    }                                                                           \
  } while (0)

#define FLCE_OK_(call)                                                          \
  do {                                                                          \
    int r_ = (call);                                                            \
    if (r_ != FLCE_OK) {                                                        \
      fprintf(stderr, "%s failed: %d (%s)\n", #call, r_, flce_error_string(r_)); \
      return 1;                                                                 \
    }                                                                           \
  } while (0)

static int read_all(FILE* f, void* p, size_t n) { return fread(p, 1, n, f) == n; }
static int write_all(FILE* f, const void* p, size_t n) { return fwrite(p, 1, n, f) == n; }

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s <inputs.bin> <outputs.bin>\n", argv[0]);
    return 2;
  }
  FILE* in = fopen(argv[1], "rb");
  if (!in) {
    fprintf(stderr, "cannot open %s\n", argv[1]);
    return 1;
  }
  int64_t dims[3], nseq;
  float softcap, grad_scale;
  int32_t reduction;
  if (!read_all(in, dims, sizeof dims) || !read_all(in, &softcap, sizeof softcap) ||
      !read_all(in, &reduction, sizeof reduction) || !read_all(in, &nseq, sizeof nseq) ||
      !read_all(in, &grad_scale, sizeof grad_scale)) {
    fprintf(stderr, "short header\n");
    return 1;
  }
  const int64_t BT = dims[0], H = dims[1], V = dims[2];
  if (BT <= 0 || H <= 0 || V <= 0 || nseq <= 0 || BT % nseq != 0) {
    fprintf(stderr, "bad sizes\n");
    return 1;
  }
  const size_t nx = (size_t)BT * H, nw = (size_t)V * H;
  uint16_t* x = malloc(nx * 2);
  uint16_t* w = malloc(nw * 2);
  int64_t* y = malloc((size_t)BT * 8);
  uint16_t* gh = malloc(nx * 2);
  float* gw = malloc(nw * 4);
  float* rows = malloc((size_t)BT * 4);
  float* lse = malloc((size_t)BT * 4);
  if (!x || !w || !y || !gh || !gw || !rows || !lse) {
    fprintf(stderr, "out of host memory\n");
    return 1;
  }
  if (!read_all(in, x, nx * 2) || !read_all(in, w, nw * 2) || !read_all(in, y, (size_t)BT * 8)) {
    fprintf(stderr, "short inputs\n");
    return 1;
  }
  fclose(in);

  void *d_x, *d_w, *d_y, *d_gh, *d_ws, *d_fws, *d_rws, *d_sws;
  float *d_loss, *d_gw, *d_rows, *d_lse;
  HIP_OK(hipSetDevice(0));
  HIP_OK(hipMalloc(&d_x, nx * 2));
  HIP_OK(hipMalloc(&d_w, nw * 2));
  HIP_OK(hipMalloc(&d_y, (size_t)BT * 8));
  HIP_OK(hipMalloc(&d_gh, nx * 2));
  HIP_OK(hipMalloc((void**)&d_gw, nw * 4));
  HIP_OK(hipMalloc((void**)&d_loss, 4));
  HIP_OK(hipMalloc((void**)&d_rows, (size_t)BT * 4));
  HIP_OK(hipMalloc((void**)&d_lse, (size_t)BT * 4));
  HIP_OK(hipMemcpy(d_x, x, nx * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_w, w, nw * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_y, y, (size_t)BT * 8, hipMemcpyHostToDevice));

  flce_handle h = NULL;
  FLCE_OK_(flce_create(&h, 0, NULL));
  size_t ws_bytes = 0, fws_bytes = 0;
  FLCE_OK_(flce_workspace_size(h, BT, H, V, FLCE_BF16, &ws_bytes));
  FLCE_OK_(flce_forward_workspace_size(h, BT, H, V, FLCE_BF16, &fws_bytes));
  HIP_OK(hipMalloc(&d_ws, ws_bytes));
  HIP_OK(hipMalloc(&d_fws, fws_bytes));
  const int64_t T = BT / nseq;
  const flce_rows R = {nseq, T, 1, {T * H, H}, {T * H, H}, {T, 1}};
  size_t rws_bytes = 0, sws_bytes = 0;
  FLCE_OK_(flce_recompute_workspace_size(h, BT, H, V, FLCE_BF16, 256, &rws_bytes));
  FLCE_OK_(flce_workspace_size_rows(h, &R, H, V, FLCE_BF16, &sws_bytes));
  HIP_OK(hipMalloc(&d_rws, rws_bytes));
  HIP_OK(hipMalloc(&d_sws, sws_bytes));
  FILE* out = fopen(argv[2], "wb");
  if (!out) {
    fprintf(stderr, "cannot open %s\n", argv[2]);
    return 1;
  }
#define COPY_OUT_(nbytes, host, dev)                                            \
  do {                                                                          \
    HIP_OK(hipMemcpy(host, dev, nbytes, hipMemcpyDeviceToHost));                \
    if (!write_all(out, host, nbytes)) {                                        \
      fprintf(stderr, "cannot write %s\n", argv[2]);                           \
      return 1;                                                                 \
    }                                                                           \
  } while (0)
  float loss = 0.0f;
  int32_t st[4];

  /* 1. the fused forward + backward and 2. the forward alone with per-row terms, on the null stream */
  FLCE_OK_(flce_forward_backward(h, d_x, d_w, (const int64_t*)d_y, BT, H, V, FLCE_BF16, -100, softcap, reduction,
                                 d_loss, d_gh, d_gw, d_ws, ws_bytes, NULL));
  st[0] = flce_status(h, NULL);
  COPY_OUT_(4, &loss, d_loss);
  const float loss_fused = loss;
  COPY_OUT_(nx * 2, gh, d_gh);
  COPY_OUT_(nw * 4, gw, d_gw);
  FLCE_OK_(flce_forward(h, d_x, d_w, (const int64_t*)d_y, BT, H, V, FLCE_BF16, -100, softcap, FLCE_NONE, NULL,
                        d_rows, d_lse, d_fws, fws_bytes, NULL));
  st[1] = flce_status(h, NULL);
  COPY_OUT_((size_t)BT * 4, rows, d_rows);
  COPY_OUT_((size_t)BT * 4, lse, d_lse);
  /* 3. the same results with the logits formed twice and one 256-wide vocabulary slice kept */
  FLCE_OK_(flce_forward_backward_recompute(h, d_x, d_w, (const int64_t*)d_y, BT, H, V, FLCE_BF16, -100, softcap,
                                           reduction, 256, d_loss, d_gh, d_gw, d_rws, rws_bytes, NULL));
  st[2] = flce_status(h, NULL);
  COPY_OUT_(4, &loss, d_loss);
  COPY_OUT_(nx * 2, gh, d_gh);
  COPY_OUT_(nw * 4, gw, d_gw);
  /* 4. the rows as sequences: next-token labels by addressing, scaled gradients */
  FLCE_OK_(flce_forward_backward_rows(h, d_x, d_w, (const int64_t*)d_y, &R, H, V, FLCE_BF16, -100, softcap,
                                      reduction, grad_scale, 0, d_loss, d_gh, d_gw, d_sws, sws_bytes, NULL));
  st[3] = flce_status(h, NULL);
  COPY_OUT_(4, &loss, d_loss);
  COPY_OUT_(nx * 2, gh, d_gh);
  COPY_OUT_(nw * 4, gw, d_gw);
  if (!write_all(out, st, sizeof st)) {
    fprintf(stderr, "cannot write %s\n", argv[2]);
    return 1;
  }
  fclose(out);
  FLCE_OK_(flce_destroy(h));
  hipFree(d_x);
  hipFree(d_w);
  hipFree(d_y);
  hipFree(d_gh);
  hipFree(d_gw);
  hipFree(d_loss);
  hipFree(d_rows);
  hipFree(d_lse);
  hipFree(d_ws);
  hipFree(d_fws);
  hipFree(d_rws);
  hipFree(d_sws);
  free(x);
  free(w);
  free(y);
  free(gh);
  free(gw);
  free(rows);
  free(lse);
  printf("flce_from_c: BT=%lld H=%lld V=%lld loss %.7f (sequences %.7f) status %d %d %d %d\n", (long long)BT,
         (long long)H, (long long)V, loss_fused, loss, st[0], st[1], st[2], st[3]);
  return 0;
}
