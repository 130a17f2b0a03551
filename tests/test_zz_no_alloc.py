"""flce_forward_backward_static (the entry point for callers that cannot allocate) called through the
C ABI, against flce_forward_backward on a handle with the chunk cap the static entry point picks: two
calls in a row, the second smaller, bitwise equal, and the second also against the CPU float64 oracle.
Sizes whose workspace exceeds the static scratch are refused before anything is enqueued."""
import ctypes

import pytest
import torch

import oracle
from gpu_helpers import TOL, announce, device, rel_fro
from linear_cross_entropy_07_amd import flce, inputs

pytestmark = pytest.mark.gpu

SCRATCH = 256 << 20  # FLCE_STATIC_SCRATCH_BYTES


def _static_chunk_cap(dev, BT, H, V, dtype):
    """The chunk cap the static entry point uses: the largest multiple of 256 up to 4096 whose
    workspace fits the scratch."""
    for c in range(4096, 0, -256):
        e = flce.FLCE(dev, chunk_rows_max=c)  # keep the handle alive while its size is asked for
        if e.workspace_size(BT, H, V, dtype) <= SCRATCH:
            return c
    return 0


def _static_call(e, X, W, y, softcap, out):
    loss, gh, gw = out
    BT, H = X.shape
    rc = flce.lib().flce_forward_backward_static(
        e.handle, X.data_ptr(), W.data_ptr(), y.data_ptr(), BT, H, W.shape[0], flce._DTYPES[X.dtype], -100,
        float(softcap), flce.FLCE_MEAN, loss.data_ptr(), gh.data_ptr(), gw.data_ptr(),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return rc


@pytest.mark.parametrize("first,second", [
    (dict(BT=8192, H=1024, V=64000, dtype="bf16", softcap=0.0), dict(BT=700, H=256, V=3000, dtype="bf16", softcap=25.0)),
    (dict(BT=3000, H=512, V=20000, dtype="fp32", softcap=10.0), dict(BT=300, H=64, V=1000, dtype="fp32", softcap=0.0)),
])
def test_static_entry_matches_the_workspace_entry(first, second):
    dev = device()
    e = flce.FLCE(dev)
    for k, shp in enumerate((first, second)):
        sc = shp.pop("softcap")
        w = inputs.custom(**shp, ignore_frac=0.05, w_std=0.05, name="static")
        X, W, y = inputs.make_inputs(w, seed=40 + k)
        BT, H, V = w.BT, w.H, w.V
        Xd, Wd, yd = X.to(dev), W.to(dev), y.to(dev)
        cap = _static_chunk_cap(dev, BT, H, V, Xd.dtype)
        announce("flce_forward_backward_static call", k + 1, f"BT={BT} H={H} V={V} {w.dtype} softcap={sc}",
                 f"chunk cap {cap}")
        assert cap >= 256
        out = (torch.empty((), dtype=torch.float32, device=dev), torch.empty_like(Xd),
               torch.empty((V, H), dtype=torch.float32, device=dev))
        for t in out:
            t.fill_(float("nan"))
        assert _static_call(e, Xd, Wd, yd, sc, out) == 0
        e_ref = flce.FLCE(dev, chunk_rows_max=cap)
        ref = e_ref.forward_backward(Xd, Wd, yd, softcap=sc)
        torch.cuda.synchronize()
        assert e.status() == 0
        same = [torch.equal(a, b) for a, b in zip(out, ref)]
        print(f"   loss {float(out[0]):.6f}; bitwise equal to flce_forward_backward (loss, gh, gW): {same}",
              flush=True)
        assert all(same)
        if k == 1:
            ol, odx, odw = oracle.flce_forward_backward(X, W, y, -100, sc, "mean")
            tol = TOL[w.dtype]
            assert abs(float(out[0]) - ol) <= tol["loss"] * ol
            assert rel_fro(out[1].double().cpu().numpy(), odx) <= tol["grad"]
            assert rel_fro(out[2].double().cpu().numpy(), odw) <= tol["grad"]


def test_static_entry_refuses_sizes_beyond_the_scratch():
    dev = device()
    announce("flce_forward_backward_static refuses V = 2^20 (256 rows need 512 MiB)")
    e = flce.FLCE(dev)
    p = torch.empty(64, dtype=torch.float32, device=dev)
    ptr = p.data_ptr()
    rc = flce.lib().flce_forward_backward_static(e.handle, ptr, ptr, ptr, 4, 64, 1 << 20, flce.FLCE_BF16, -100,
                                                  0.0, flce.FLCE_MEAN, ptr, ptr, ptr, None)
    assert rc == -3  # FLCE_ERR_WORKSPACE_TOO_SMALL, nothing enqueued
    assert "static scratch" in flce.lib().flce_error_string(rc).decode()
