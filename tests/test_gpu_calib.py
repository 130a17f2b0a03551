"""The benchmark's peak calibration (libflce_calib.so) on the GPU: the MFMA-only loop's output is exact
(twice the iterations give exactly twice the value, and the value is not zero), the copy's destination
equals its source, and both rates lie within the published ceilings (2.5 PF/s bf16 dense at 2.4 GHz,
8 TB/s)."""
import ctypes
import math

import pytest

from gpu_helpers import announce, device
from linear_cross_entropy_07_amd import build_lib

pytestmark = pytest.mark.gpu


def _lib():
    L = ctypes.CDLL(build_lib.CALIB_LIB)
    d = ctypes.c_double
    L.flce_calib_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint,
                                       ctypes.c_int, ctypes.POINTER(d), ctypes.POINTER(d), ctypes.POINTER(d)]
    L.flce_calib_copy.argtypes = [ctypes.c_int, ctypes.c_size_t, ctypes.c_int, ctypes.POINTER(d),
                                  ctypes.POINTER(d), ctypes.POINTER(ctypes.c_int)]
    return L


def _mfma(L, dev, blocks, iters, seed=1, full_random=0):
    d = ctypes.c_double
    tf, ms, chk = d(), d(), d()
    assert L.flce_calib_mfma_bf16(dev.index, blocks, iters, 2, seed, full_random, ctypes.byref(tf),
                                  ctypes.byref(ms), ctypes.byref(chk)) == 0
    return tf.value, ms.value, chk.value


@pytest.mark.parametrize("blocks,iters", [(1, 4), (256, 1000), (1024, 20000)])
def test_mfma_loop_is_exact_and_within_the_peak(blocks, iters):
    dev = device()
    announce("MFMA-only loop", f"blocks={blocks} iters={iters}")
    L = _lib()
    tf, ms, chk = _mfma(L, dev, blocks, iters)
    tf2, ms2, chk2 = _mfma(L, dev, blocks, 2 * iters)
    print(f"   {tf:.1f} TFLOP/s in {ms:.3f} ms (x2 iterations: {tf2:.1f} in {ms2:.3f}); output {chk} / {chk2}",
          flush=True)
    assert chk != 0.0 and chk2 == 2.0 * chk
    assert _mfma(L, dev, blocks, iters, seed=2)[2] != chk  # the seed changes the data
    assert 0.0 < tf <= 2500.0 * 1.01 and 0.0 < tf2 <= 2500.0 * 1.01
    if blocks == 1024:
        assert tf > 1000.0  # a full chip of matrix cores, whatever the clock under load
        tfr, msr, chkr = _mfma(L, dev, blocks, iters, full_random=1)
        print(f"   random bf16 operands: {tfr:.1f} TFLOP/s in {msr:.3f} ms; output {chkr}", flush=True)
        assert 1000.0 < tfr <= 2500.0 * 1.01 and math.isfinite(chkr) and chkr != chk


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 1 << 30])
def test_copy_is_a_copy_within_the_hbm_ceiling(nbytes):
    dev = device()
    announce("device copy", f"{nbytes} bytes")
    L, d = _lib(), ctypes.c_double
    gbs, ms, ok = d(), d(), ctypes.c_int()
    assert L.flce_calib_copy(dev.index, nbytes, 2, ctypes.byref(gbs), ctypes.byref(ms), ctypes.byref(ok)) == 0
    print(f"   {gbs.value:.1f} GB/s in {ms.value:.3f} ms", flush=True)
    assert ok.value == 1
    assert 0.0 < gbs.value
    if nbytes == 1 << 30:
        assert 1000.0 < gbs.value <= 8000.0 * 1.01


def test_argument_errors():
    device()
    L, d = _lib(), ctypes.c_double
    x, y, z = d(), d(), d()
    assert L.flce_calib_mfma_bf16(0, 0, 4, 1, 1, 0, ctypes.byref(x), ctypes.byref(y), None) == -1
    assert L.flce_calib_mfma_bf16(0, 1, 6, 1, 1, 0, ctypes.byref(x), ctypes.byref(y), None) == -1
    assert L.flce_calib_mfma_bf16(0, 1, (1 << 16) + 4, 1, 1, 0, ctypes.byref(x), ctypes.byref(y), None) == -1
    assert L.flce_calib_mfma_bf16(0, 1, 4, 1, 1, 0, None, ctypes.byref(y), None) == -1
    assert L.flce_calib_copy(0, 15, 1, ctypes.byref(x), ctypes.byref(z), None) == -1
