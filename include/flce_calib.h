/* Peak calibration for the benchmark (measurement only; libflce_calib.so, not part of the FLCE path).
 *
 * The fused linear + cross-entropy step is priced against the chip's published peaks (2.5 PF/s bf16
 * dense MFMA, 8 TB/s HBM). These two microbenchmarks measure what this GPU sustains instead, so a
 * result can also be stated as a fraction of the measured ceiling:
 *   - an MFMA-only loop: blocks of 8 waves, each wave running 8 independent chains of
 *     v_mfma_f32_32x32x16_bf16 on register operands that change from one MFMA to the next (the
 *     instruction, block shape and accumulator count of the library's GEMMs), no memory traffic
 *     inside the loop;
 *   - a device-to-device copy kernel, 16 bytes per lane per access.
 * Both allocate their own device buffers with hipMalloc, run on a stream they create, synchronise, and
 * free everything before returning. Not for use inside graph capture or in an allocation-free context.
 */
#ifndef FLCE_CALIB_H
#define FLCE_CALIB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* MFMA-only loop on HIP device `device`: `blocks` blocks of 512 threads, `iters` loop iterations of 8
 * MFMAs per wave, launched `reps` times after one warm-up launch. Operands are drawn per lane, element
 * and vector from `seed` (a hash) and cycled over 4 vectors per operand, so that consecutive MFMAs see
 * different data, as in a GEMM. full_random = 0: +-2^-10 (random signs; the arithmetic is exact, see
 * check_out). full_random = 1: random bf16 bit patterns (random sign, exponent 2^-12 .. 2^-9, 7 random
 * mantissa bits), so every multiplier bit toggles as with real data; check_out is then just a value.
 *   tflops_out   host, 1 double: the best launch's bf16 TFLOP/s (32768 flop per MFMA)
 *   ms_out       host, 1 double: that launch's duration in ms
 *   check_out    host, 1 double or NULL: the loop's output value for lane 0 of block 0. With
 *                full_random = 0 the arithmetic is exact, so for the same blocks and seed the value for
 *                2*iters is exactly twice the value for iters: a caller can confirm that the MFMAs ran,
 *                and how many
 * Returns 0, -1 (blocks < 1, iters not a positive multiple of 4, iters > 2^16, reps < 1, NULL outputs)
 * or -4 (a HIP call failed). */
int flce_calib_mfma_bf16(int device, int blocks, int iters, int reps, unsigned seed, int full_random,
                         double* tflops_out, double* ms_out, double* check_out);

/* Device-to-device copy of `bytes` bytes (rounded down to a multiple of 16, at least 16) on HIP device
 * `device`, launched `reps` times after one warm-up launch.
 *   gbs_out      host, 1 double: the best launch's (read + write) bytes per second, in GB/s (1e9)
 *   ms_out       host, 1 double: that launch's duration in ms
 *   ok_out       host, 1 int or NULL: 1 if the destination equals the source after the last launch
 * Returns 0, -1 (bytes < 16, reps < 1, NULL outputs) or -4 (a HIP call failed, e.g. out of memory). */
int flce_calib_copy(int device, size_t bytes, int reps, double* gbs_out, double* ms_out, int* ok_out);

#ifdef __cplusplus
}
#endif

#endif /* FLCE_CALIB_H */
