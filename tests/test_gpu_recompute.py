"""GPU parity of the recompute mode (flce_forward_backward_recompute) against the CPU float64 oracle,
and its exact relations to the fused call: the loss is bitwise that of flce_forward_backward, grad_W
bitwise that of flce_forward_backward with all rows in one chunk (the recompute mode's single pass),
grad_hidden differs only by the order of its fp32 sums. Vocabulary slices with a ragged last slice,
a ragged row count, bf16 and fp32, with and without softcap; the workspace does not depend on the
handle's chunk cap."""
import pytest
import torch

from gpu_helpers import announce, check_against_oracle, device
from linear_cross_entropy_07_amd import flce, inputs

pytestmark = pytest.mark.gpu

_ENG = {}


def eng(chunk=0):
    dev = device()
    if chunk not in _ENG:
        _ENG[chunk] = flce.FLCE(dev, chunk_rows_max=chunk)
    return _ENG[chunk]


def _run_device(e, X, W, y, softcap, reduction, v_slice):
    """The recompute call on e, the fused call on e (row chunks of e's cap) and on a handle whose one
    chunk holds all rows; asserts the exact relations; returns the recompute results."""
    dev = e.device
    Xd, Wd, yd = X.to(dev), W.to(dev), y.to(dev)
    rl, rgh, rgw = e.forward_backward_recompute(Xd, Wd, yd, -100, softcap, reduction, v_slice)
    fl = e.forward_backward(Xd, Wd, yd, -100, softcap, reduction)[0].clone()
    one = eng(max(256, X.shape[0]))
    assert one.chunk_plan(X.shape[0], X.shape[1], W.shape[0], X.dtype)[0] == 1
    fl1, fgh, fgw = one.forward_backward(Xd, Wd, yd, -100, softcap, reduction)
    torch.cuda.synchronize(dev)
    assert torch.equal(rl, fl), (float(rl), float(fl))
    assert torch.equal(rl, fl1), (float(rl), float(fl1))
    assert torch.equal(rgw, fgw)
    d = float((rgh.float() - fgh.float()).norm() / fgh.float().norm().clamp_min(1e-30))
    print(f"   grad_hidden recompute vs fused: rel {d:.2e}", flush=True)
    return rl, rgh, rgw, d


def _run(e, X, W, y, softcap, reduction, v_slice):
    rl, rgh, rgw, _ = _run_device(e, X, W, y, softcap, reduction, v_slice)
    return float(rl.cpu()), rgh.double().cpu().numpy(), rgw.double().cpu().numpy()


@pytest.mark.parametrize("softcap", [0.0, 30.0])
@pytest.mark.parametrize("v_slice", [256, 1024])
def test_bf16_slices(softcap, v_slice):
    w = inputs.custom(BT=1000, H=256, V=3001, dtype="bf16", ignore_frac=0.1, w_std=0.05, name="recompute")
    announce("recompute bf16", w.BT, w.H, w.V, "v_slice", v_slice, "softcap", softcap)
    X, W, y = inputs.make_inputs(w, seed=51)
    got = _run(eng(256), X, W, y, softcap, "mean", v_slice)
    check_against_oracle(got, X, W, y, "bf16", softcap=softcap, reduction="mean")


@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_fp32_slices(reduction):
    w = inputs.custom(BT=700, H=96, V=1000, dtype="fp32", ignore_frac=0.1, name="recompute_fp32")
    announce("recompute fp32", reduction, "v_slice 256")
    X, W, y = inputs.make_inputs(w, seed=52)
    got = _run(eng(256), X, W, y, 3.0, reduction, 256)
    check_against_oracle(got, X, W, y, "fp32", softcap=3.0, reduction=reduction)


def test_single_slice_and_edges():
    e = eng()
    dev = e.device
    announce("recompute: one slice wider than V, BT = 0, all rows ignored")
    w = inputs.custom(BT=300, H=128, V=1000, dtype="bf16", ignore_frac=0.1, w_std=0.05, name="recompute_one")
    X, W, y = inputs.make_inputs(w, seed=53)
    got = _run(e, X, W, y, 0.0, "mean", 1 << 20)
    check_against_oracle(got, X, W, y, "bf16")
    X0 = torch.empty(0, 128, dtype=torch.bfloat16, device=dev)
    y0 = torch.empty(0, dtype=torch.int64, device=dev)
    loss, _, gw = e.forward_backward_recompute(X0, W.to(dev), y0)
    assert float(loss.cpu()) == 0.0 and torch.all(gw == 0).item()
    yi = torch.full((300,), -100, dtype=torch.int64)
    loss, gh, gw = e.forward_backward_recompute(X.to(dev), W.to(dev), yi.to(dev), v_slice=256)
    assert float(loss.cpu()) == 0.0 and torch.all(gh == 0).item() and torch.all(gw == 0).item()
    with pytest.raises(flce.FlceError):
        e.forward_backward_recompute(X.to(dev), W.to(dev), y.to(dev), v_slice=-1)


def test_llama_head_equals_fused_call():
    """Full-size Llama-3-8B head: the loss bitwise that of the fused call, grad_W bitwise that of the
    fused call with all 8192 rows in one chunk, grad_hidden within bf16 rounding of it (the fused
    call's whole tensors are checked against the oracle elsewhere)."""
    e = eng()
    w = inputs.WORKLOADS["llama3_8b_head"]
    announce("recompute: llama3_8b_head, v_slice 8192")
    X, W, y = inputs.make_inputs(w, seed=0)
    _, gh, _, d = _run_device(e, X, W, y, 0.0, "mean", 8192)
    assert torch.isfinite(gh.float()).all().item()
    assert d <= 5e-3


@pytest.mark.parametrize("softcap,far", [(0.0, 60.0), (30.0, 120.0)])
def test_label_far_below_the_row_maximum(softcap, far):
    """Rows whose label logit lies more than the reference span below their maximum: the recompute mode
    forms their numerators against the row maximum directly (the fused call rescales stored ones, so
    the two agree to rounding here, not bitwise); against the oracle."""
    e = eng()
    dev = e.device
    X, W, y = inputs.far_label_case(700, 128, 3000, "bf16", far=far, near=40.0, every=5, seed=12)
    announce("recompute: label far below the row maximum", f"softcap={softcap}", "v_slice 1024")
    rl, rgh, rgw = e.forward_backward_recompute(X.to(dev), W.to(dev), y.to(dev), -100, softcap, "mean", 1024)
    torch.cuda.synchronize(dev)
    got = (float(rl.cpu()), rgh.double().cpu().numpy(), rgw.double().cpu().numpy())
    check_against_oracle(got, X, W, y, "bf16", softcap=softcap, reduction="mean")


def test_workspace_does_not_depend_on_the_chunk_cap():
    """One pass over all rows: the handle's chunk cap changes neither the workspace size nor the bits."""
    dev = device()
    announce("recompute: chunk cap 256 vs default, workspace and bits")
    w = inputs.custom(BT=900, H=128, V=2000, dtype="bf16", ignore_frac=0.1, w_std=0.05, name="recompute_cap")
    X, W, y = inputs.make_inputs(w, seed=54)
    a, b = eng(256), eng()
    assert (flce.recompute_workspace_size(900, 128, 2000, torch.bfloat16, 512, a._h)
            == flce.recompute_workspace_size(900, 128, 2000, torch.bfloat16, 512, b._h))
    Xd, Wd, yd = X.to(dev), W.to(dev), y.to(dev)
    ra = [t.clone() for t in a.forward_backward_recompute(Xd, Wd, yd, v_slice=512)]
    rb = b.forward_backward_recompute(Xd, Wd, yd, v_slice=512)
    torch.cuda.synchronize(dev)
    assert all(torch.equal(u, v) for u, v in zip(ra, rb))
