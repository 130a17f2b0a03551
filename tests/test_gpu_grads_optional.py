"""Only the gradients that will be used are computed: the autograd wrapper under torch.no_grad (or with
no input requiring a gradient) runs the forward alone, and with only one of hidden / W requiring a
gradient the other gradient's GEMM is not launched (kernel launch counts from the library's own
per-launch profile). Results against the CPU float64 oracle. Also: a call on a side stream given
explicitly gives the same bits as the call on the current stream."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import TOL, announce, device, rel_fro
from linear_cross_entropy_07_amd import flce, inputs

pytestmark = pytest.mark.gpu


def _case(dtype="bf16", softcap=0.0, BT=700, H=256, V=3000, seed=3):
    w = inputs.custom(BT=BT, H=H, V=V, dtype=dtype, softcap=softcap, ignore_frac=0.1, w_std=0.05, name="opt")
    return inputs.make_inputs(w, seed=seed)


def _counts(e, fn):
    e.profile_begin(4096)
    out = fn()
    kt = e.profile_end()
    return out, {k: c for k, (_, c) in kt.items()}


@pytest.mark.parametrize("softcap", [0.0, 20.0])
def test_no_grad_loss_runs_the_forward_only(softcap):
    dev = device()
    announce("flce_loss under torch.no_grad: forward only", f"softcap={softcap}")
    X, W, y = _case(softcap=softcap)
    e = flce.engine(dev)
    Xd, Wd, yd = X.to(dev).requires_grad_(), W.to(dev).requires_grad_(), y.to(dev)
    with torch.no_grad():
        loss, cnt = _counts(e, lambda: flce.flce_loss(Xd, Wd, yd, softcap=softcap))
    torch.cuda.synchronize()
    print(f"   launches {cnt}", flush=True)
    assert cnt["dx"] == 0 and cnt["dw"] == 0 and cnt["rowfix"] == 0 and cnt["fwd"] >= 1
    assert not loss.requires_grad
    ol = oracle.flce_forward(X, W, y, -100, softcap, "mean")[0]
    assert abs(float(loss.detach()) - ol) <= TOL["bf16"]["loss"] * ol
    # no input requiring a gradient: the same forward-only path with grad mode on
    loss2, cnt2 = _counts(e, lambda: flce.flce_loss(X.to(dev), W.to(dev), yd, softcap=softcap))
    assert cnt2["dx"] == 0 and cnt2["dw"] == 0 and float(loss2) == float(loss)


@pytest.mark.parametrize("which", ["hidden", "W", "both"])
@pytest.mark.parametrize("shape3d", [False, True])
def test_only_the_needed_gradient_is_computed(which, shape3d):
    dev = device()
    announce("flce_loss with", which, "requiring a gradient", "[B,T,H] shifted" if shape3d else "[BT,H]")
    X, W, y = _case(softcap=15.0, BT=3 * 257)
    e = flce.engine(dev)
    Xd = X.to(dev).requires_grad_(which in ("hidden", "both"))
    Wd = W.to(dev).requires_grad_(which in ("W", "both"))
    yd = y.to(dev)
    if shape3d:
        Xin, yin = Xd.view(3, 257, -1), yd.view(3, 257)
        Xs = X.view(3, 257, -1)[:, :-1].reshape(-1, X.shape[1])
        ys = y.view(3, 257)[:, 1:].reshape(-1)
    else:
        Xin, yin, Xs, ys = Xd, yd, X, y
    loss, cnt = _counts(e, lambda: flce.flce_loss(Xin, Wd, yin, softcap=15.0, shift=shape3d))
    (loss * 0.5).backward()
    torch.cuda.synchronize()
    print(f"   launches {cnt}", flush=True)
    assert (cnt["dx"] > 0) == (which in ("hidden", "both"))
    assert (cnt["dw"] > 0) == (which in ("W", "both"))
    ol, odx, odw = oracle.flce_forward_backward(Xs, W, ys, -100, 15.0, "mean")
    assert abs(float(loss.detach()) - ol) <= TOL["bf16"]["loss"] * ol
    if which in ("hidden", "both"):
        g = Xd.grad.double().cpu().numpy()
        if shape3d:
            g3 = g.reshape(3, 257, -1)
            assert not g3[:, -1].any()
            g = g3[:, :-1].reshape(-1, g.shape[1])
        assert rel_fro(g, 0.5 * odx) <= TOL["bf16"]["grad"]
    else:
        assert Xd.grad is None
    if which in ("W", "both"):
        assert rel_fro(Wd.grad.double().cpu().numpy(), 0.5 * odw) <= TOL["bf16"]["grad"]
    else:
        assert Wd.grad is None


def test_skip_flags_match_the_full_call_bitwise():
    dev = device()
    announce("forward_backward with one gradient left out vs both, bitwise")
    X, W, y = _case(dtype="fp32", BT=1000, H=128, V=2500)
    e = flce.FLCE(dev, chunk_rows_max=256)
    Xd, Wd, yd = X.to(dev), W.to(dev), y.to(dev)
    l, gh, gw = [t.clone() for t in e.forward_backward(Xd, Wd, yd)]
    l1, gh1, gw1 = e.forward_backward(Xd, Wd, yd, grad_W=False)
    assert gw1 is None and torch.equal(l1, l) and torch.equal(gh1, gh)
    l2, gh2, gw2 = e.forward_backward(Xd, Wd, yd, grad_hidden=False)
    assert gh2 is None and torch.equal(l2, l) and torch.equal(gw2, gw)
    with pytest.raises(ValueError):
        e.forward_backward(Xd, Wd, yd, grad_hidden=False, grad_W=False)


def test_side_stream_call_matches_current_stream():
    dev = device()
    announce("forward_backward on an explicit side stream vs the current stream")
    X, W, y = _case(BT=1500, H=512, V=7000, seed=9)
    e = flce.FLCE(dev, chunk_rows_max=512)
    Xd, Wd, yd = X.to(dev), W.to(dev), y.to(dev)
    ref = [t.clone() for t in e.forward_backward(Xd, Wd, yd)]
    torch.cuda.synchronize()
    e._ws = None  # the side-stream call allocates its workspace afresh
    side = torch.cuda.Stream(device=dev)
    Xn = Xd * 1.0  # produced on the current stream just before the call
    out = e.forward_backward(Xn, Wd, yd, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    del Xn
    junk = [torch.empty(1 << 24, device=dev).fill_(7.0) for _ in range(4)]  # reuse freed memory if any
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(out, ref))
    del junk
