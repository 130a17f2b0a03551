// Peak calibration microbenchmarks for the benchmark: an MFMA-only loop and a device copy. They
// measure the ceilings this GPU sustains; nothing in the FLCE library calls them.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <vector>

#include "flce_calib.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kChains = 8;  // independent accumulators per wave (the GEMMs keep 4 x 2 blocks)
constexpr int kOps = 4;     // distinct operand vectors per lane and operand, cycled from one MFMA to the next

// A 32-bit mixing function (xorshift-multiply rounds); only its bits are used, as signs.
__device__ __forceinline__ unsigned mix32(unsigned h) {
  h ^= h >> 16;
  h *= 0x7feb352du;
  h ^= h >> 15;
  h *= 0x846ca68bu;
  h ^= h >> 16;
  return h;
}

// Operands are +-2^-10 with random signs per lane, element and vector, and consecutive MFMAs of a wave
// use different vectors, so the multipliers see changing data as in a real GEMM (a constant operand
// barely toggles them and draws less power). Every product is +-2^-20, so an MFMA adds a multiple of
// 2^-20 of magnitude at most 16 * 2^-20 to each accumulator element; with at most 2^16 iterations every
// partial sum is a multiple of 2^-20 below 1 in magnitude, exact in fp32. The operand cycle repeats
// every kOps iterations, so for iteration counts that are multiples of kOps each accumulator element is
// (iters / kOps) times one fixed sum, and the output (the same fixed-order fp32 sum of 128 such values)
// for 2n iterations is exactly twice the output for n.
// With `full_random` the operands are instead random bf16 bit patterns: random sign, exponent 2^-12 ..
// 2^-9 and 7 random mantissa bits per element (every multiplier bit toggles, as with real data; the
// magnitudes keep every sum far from overflow, but the exactness above no longer holds).
__device__ __forceinline__ __bf16 operand(unsigned lane_id, unsigned seed, unsigned v, int e, bool full_random) {
  const unsigned h = mix32(lane_id * 0x9e3779b9u ^ seed ^ (v * 8u + (unsigned)e + 1u) * 0x85ebca77u);
  if (!full_random) return (__bf16)((h & 1u) ? -0.0009765625f : 0.0009765625f);
  const unsigned short bits = (unsigned short)(((h & 1u) << 15) | ((115u + ((h >> 1) & 3u)) << 7) | ((h >> 3) & 127u));
  return __builtin_bit_cast(__bf16, bits);
}

__global__ __launch_bounds__(512) void k_mfma_loop(int iters, unsigned seed, int full_random, float* out) {
  const unsigned lane_id = (unsigned)blockIdx.x * blockDim.x + threadIdx.x;
  bf16x8_t A[kOps], B[kOps];
#pragma unroll
  for (int v = 0; v < kOps; ++v)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      A[v][e] = operand(lane_id, seed, 2u * v, e, full_random != 0);
      B[v][e] = operand(lane_id, seed, 2u * v + 1u, e, full_random != 0);
    }
  f32x16_t acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  for (int it = 0; it < iters; it += kOps) {
#pragma unroll
    for (int u = 0; u < kOps; ++u)
#pragma unroll
      for (int c = 0; c < kChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[(c + u) % kOps], B[(c + 3 * u + 1) % kOps], acc[c],
                                                          0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void k_copy16(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst,
                                                size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

struct Device {
  int prev = -1;
  bool ok = false;
  explicit Device(int d) {
    if (hipGetDevice(&prev) != hipSuccess) return;
    ok = hipSetDevice(d) == hipSuccess;
  }
  ~Device() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

// Runs `launch` once untimed and `reps` times timed on `stream`; returns the best duration in ms.
template <class F>
bool time_best(hipStream_t stream, int reps, F launch, double* best_ms) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return false;
  bool ok = launch() == hipSuccess && hipStreamSynchronize(stream) == hipSuccess;
  double best = 1e300;
  for (int r = 0; ok && r < reps; ++r) {
    ok = hipEventRecord(e0, stream) == hipSuccess && launch() == hipSuccess &&
         hipEventRecord(e1, stream) == hipSuccess && hipEventSynchronize(e1) == hipSuccess;
    float ms = 0.0f;
    if (ok) ok = hipEventElapsedTime(&ms, e0, e1) == hipSuccess;
    if (ok && ms < best) best = ms;
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  *best_ms = best;
  return ok;
}

}  // namespace

extern "C" {

int flce_calib_mfma_bf16(int device, int blocks, int iters, int reps, unsigned seed, int full_random,
                         double* tflops_out, double* ms_out, double* check_out) {
  if (blocks < 1 || iters < kOps || iters % kOps != 0 || reps < 1 || iters > (1 << 16) || !tflops_out || !ms_out)
    return -1;
  Device g(device);
  if (!g.ok) return -4;
  float* out = nullptr;
  hipStream_t stream = nullptr;
  int rc = 0;
  if (hipMalloc(&out, (size_t)blocks * 512 * sizeof(float)) != hipSuccess) return -4;
  if (hipStreamCreate(&stream) != hipSuccess) {
    (void)hipFree(out);
    return -4;
  }
  double ms = 0.0;
  const bool ok = time_best(stream, reps, [&]() {
    k_mfma_loop<<<blocks, 512, 0, stream>>>(iters, seed, full_random, out);
    return hipGetLastError();
  }, &ms);
  if (!ok) {
    rc = -4;
  } else {
    const double flops = (double)blocks * 8 /* waves */ * iters * kChains * 32768.0;
    *tflops_out = flops / (ms * 1e-3) / 1e12;
    *ms_out = ms;
    if (check_out) {
      float v = 0.0f;
      if (hipMemcpy(&v, out, sizeof(float), hipMemcpyDeviceToHost) != hipSuccess) rc = -4;
      *check_out = v;
    }
  }
  (void)hipStreamDestroy(stream);
  (void)hipFree(out);
  return rc;
}

int flce_calib_copy(int device, size_t bytes, int reps, double* gbs_out, double* ms_out, int* ok_out) {
  if (bytes < 16 || reps < 1 || !gbs_out || !ms_out) return -1;
  const size_t n = bytes / 16;
  Device g(device);
  if (!g.ok) return -4;
  u32x4_t* src = nullptr;
  u32x4_t* dst = nullptr;
  hipStream_t stream = nullptr;
  int rc = 0;
  if (hipMalloc(&src, n * 16) != hipSuccess) return -4;
  if (hipMalloc(&dst, n * 16) != hipSuccess) {
    (void)hipFree(src);
    return -4;
  }
  if (hipStreamCreate(&stream) != hipSuccess) rc = -4;
  // a byte pattern in the source, a different one in the destination
  if (rc == 0 && (hipMemsetAsync(src, 0x5a, n * 16, stream) != hipSuccess ||
                  hipMemsetAsync(dst, 0x00, n * 16, stream) != hipSuccess))
    rc = -4;
  double ms = 0.0;
  if (rc == 0) {
    int ncu = 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || ncu <= 0)
      ncu = 256;
    const int grid = ncu * 8;
    const bool ok = time_best(stream, reps, [&]() {
      k_copy16<<<grid, 256, 0, stream>>>(src, dst, n);
      return hipGetLastError();
    }, &ms);
    if (!ok) rc = -4;
  }
  if (rc == 0) {
    *gbs_out = 2.0 * (double)(n * 16) / (ms * 1e-3) / 1e9;
    *ms_out = ms;
    if (ok_out) {
      // compare a sample of 16-byte elements spread over the buffer
      const size_t samples = n < 4096 ? n : 4096;
      std::vector<u32x4_t> a(1), b(1);
      int same = 1;
      for (size_t k = 0; k < samples && same; ++k) {
        const size_t i = k * (n / samples);
        if (hipMemcpy(a.data(), src + i, 16, hipMemcpyDeviceToHost) != hipSuccess ||
            hipMemcpy(b.data(), dst + i, 16, hipMemcpyDeviceToHost) != hipSuccess) {
          rc = -4;
          break;
        }
        for (int e = 0; e < 4; ++e) same &= a[0][e] == b[0][e];
      }
      *ok_out = same;
    }
  }
  if (stream) (void)hipStreamDestroy(stream);
  (void)hipFree(src);
  (void)hipFree(dst);
  return rc;
}

}  // extern "C"
