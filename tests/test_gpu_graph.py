"""The compute entry points enqueue kernels only (no allocation, no synchronisation, no memset), so a
caller can capture them into a HIP graph and replay it. Each replay is checked bit for bit against the
eager call, with eager work and synchronisation between replays, and after the inputs are overwritten
in place (a replay reads the live input buffers)."""
import numpy as np
import pytest
import torch

from gpu_helpers import announce, device
from linear_cross_entropy_07_amd import flce, inputs

pytestmark = pytest.mark.gpu


def _buffers(e, X, W):
    BT, H = X.shape
    V = W.shape[0]
    out = (torch.empty((), dtype=torch.float32, device=e.device), torch.empty_like(X),
           torch.empty((V, H), dtype=torch.float32, device=e.device))
    ws = e.workspace(e.workspace_size(BT, H, V, X.dtype))
    return out, ws


def _same(a, b):
    return all(torch.equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("softcap", [0.0, 30.0])
def test_fused_call_in_a_hip_graph(softcap):
    dev = device()
    announce("HIP graph capture of flce_forward_backward, 1000x256x5000 bf16, 4 chunks", f"softcap={softcap}")
    w = inputs.custom(BT=1000, H=256, V=5000, dtype="bf16", ignore_frac=0.05, w_std=0.05, name="graph")
    X, W, y = inputs.make_inputs(w, seed=31)
    X2, _, y2 = inputs.make_inputs(w, seed=32)
    e = flce.FLCE(dev, chunk_rows_max=256)
    Xd, Wd, yd = X.to(dev), W.to(dev), y.to(dev)
    ref1 = [t.clone() for t in e.forward_backward(Xd, Wd, yd, softcap=softcap)]
    ref2 = [t.clone() for t in e.forward_backward(X2.to(dev), Wd, y2.to(dev), softcap=softcap)]
    torch.cuda.synchronize()

    out, ws = _buffers(e, Xd, Wd)
    xin, yin = Xd.clone(), yd.clone()
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream, as torch recommends
        e.forward_backward(xin, Wd, yin, softcap=softcap, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        e.forward_backward(xin, Wd, yin, softcap=softcap, out=out, workspace=ws)
    torch.cuda.synchronize()

    junk = torch.randn(2048, 2048, device=dev)
    for r in range(3):
        for t in out:
            t.fill_(float("nan"))
        _ = junk @ junk  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same(out, ref1), f"replay {r}"
        assert e.status() == 0
    # new contents in the captured input buffers: the replay follows them
    xin.copy_(X2.to(dev))
    yin.copy_(y2.to(dev))
    g.replay()
    torch.cuda.synchronize()
    assert _same(out, ref2)
    xin.copy_(Xd)
    yin.copy_(yd)
    g.replay()
    torch.cuda.synchronize()
    assert _same(out, ref1)
    print(f"   5 replays bitwise equal to the eager calls; loss {float(ref1[0]):.6f} / {float(ref2[0]):.6f}",
          flush=True)
    assert not np.isnan(float(out[0]))
