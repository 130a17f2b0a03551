"""GPU parity of the sequence entry points (flce_forward_backward_rows, flce_forward_rows) against
the CPU float64 oracle: hidden [B,T,H] at arbitrary strides, labels [B,T] at their own strides, the
next-token label shift done by addressing, a gradient scale, and accumulation into existing
gradients. Shapes span several tiles and chunks with ragged tails; V = 300 (bf16) and V = 250 (fp32)
take the grad_hidden epilogue of whole tiles, V = 3001 (bf16) and V = 1000 (fp32) the split-K
reduction."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import TOL, announce, device, rel_fro
from linear_cross_entropy_07_amd import flce, inputs

pytestmark = pytest.mark.gpu

_ENG = {}
IGN = -100


def eng(chunk=0):
    dev = device()
    if chunk not in _ENG:
        _ENG[chunk] = flce.FLCE(dev, chunk_rows_max=chunk)
    return _ENG[chunk]


def _seq_inputs(B, T, H, V, dtype, seed, ignore_frac=0.1):
    w = inputs.custom(BT=B * T, H=H, V=V, dtype=dtype, ignore_frac=ignore_frac, w_std=0.05, name="seq")
    X, W, y = inputs.make_inputs(w, seed=seed)
    return X.reshape(B, T, H), W, y.reshape(B, T)


def _place_hidden(X3, layout, dev):
    """hidden on the device in the given layout (values equal to X3)."""
    B, T, H = X3.shape
    if layout == "contiguous":
        return X3.to(dev)
    if layout == "padded":  # rows of a wider buffer: position stride H + 64
        big = torch.zeros(B, T, H + 64, dtype=X3.dtype, device=dev)
        big[..., :H] = X3.to(dev)
        return big[..., :H]
    if layout == "seq_major":  # a [T, B, H] buffer seen as [B, T, H]: strides (H, B*H, 1)
        return X3.transpose(0, 1).contiguous().to(dev).transpose(0, 1)
    raise ValueError(layout)


def _place_labels(Y2, layout, dev):
    if layout == "contiguous":
        return Y2.to(dev)
    B, T = Y2.shape  # every other entry of a [B, 2T] buffer: strides (2T, 2)
    big = torch.full((B, 2 * T), 7, dtype=torch.int64, device=dev)
    big[:, ::2] = Y2.to(dev)
    return big[:, ::2]


def _grad_buffer(X3, layout, dev, fill):
    """grad_hidden [B,T,H] in the given layout; returns (view, backing buffer)."""
    B, T, H = X3.shape
    if layout == "padded":
        big = torch.full((B, T, H + 8), fill, dtype=X3.dtype, device=dev)
        return big[..., :H], big
    if layout == "seq_major":
        big = torch.full((T, B, H), fill, dtype=X3.dtype, device=dev)
        return big.transpose(0, 1), big
    big = torch.full((B, T, H), fill, dtype=X3.dtype, device=dev)
    return big, big


def _check(e, X3, W, Y2, dtype, shift=True, softcap=0.0, reduction="mean", grad_scale=1.0, layout="contiguous",
           labels_layout="contiguous", acc_gh=False, acc_gw=False, seed=0):
    dev = e.device
    B, T, H = X3.shape
    V = W.shape[0]
    tol = TOL[dtype]
    rng = np.random.default_rng(seed)
    hidden = _place_hidden(X3, layout, dev)
    labels = _place_labels(Y2, labels_layout, dev)
    # initial gradients: NaN where everything is overwritten, values of the gradients' size to add to
    gh, gbig = _grad_buffer(X3, layout, dev, float("nan"))
    gw = torch.full((V, H), float("nan"), dtype=torch.float32, device=dev)
    ref = oracle.flce_sequences(X3, W, Y2, int(shift), IGN, softcap, reduction, grad_scale)
    gh0 = gw0 = None
    if acc_gh:
        s = float(np.abs(ref[1]).mean()) + 1e-30
        gh0 = torch.tensor(rng.standard_normal((B, T, H)) * s, dtype=X3.dtype)
        gh.copy_(gh0.to(dev))
    if acc_gw:
        s = float(np.abs(ref[2]).mean()) + 1e-30
        gw0 = torch.tensor(rng.standard_normal((V, H)) * s, dtype=torch.float32)
        gw.copy_(gw0.to(dev))
    if acc_gh or acc_gw:
        ref = oracle.flce_sequences(X3, W, Y2, int(shift), IGN, softcap, reduction, grad_scale, gh0, gw0)
    loss, gh_out, gw_out = e.forward_backward_seq(hidden, W.to(dev), labels, shift, IGN, softcap, reduction,
                                                  grad_scale, gh, gw, acc_gh, acc_gw)
    assert gh_out.data_ptr() == gh.data_ptr() and gw_out.data_ptr() == gw.data_ptr()
    gl = float(loss.cpu())
    gdx = gh.double().cpu().numpy()
    gdw = gw.double().cpu().numpy()
    ol, odx, odw = ref[0], ref[1], ref[2]
    err_l = abs(gl - ol) / abs(ol)
    err_dx, err_dw = rel_fro(gdx, odx), rel_fro(gdw, odw)
    print(f"   loss gpu {gl:.7f} oracle {ol:.7f} rel {err_l:.2e}; dX {err_dx:.2e}; dW {err_dw:.2e}", flush=True)
    assert err_l <= tol["loss"]
    assert err_dx <= tol["grad"] and err_dw <= tol["grad"]
    # the last position of every sequence gets no gradient of its own
    if shift:
        last = gh[:, -1, :].cpu()
        if acc_gh:
            assert torch.equal(last, gh0[:, -1, :])
        else:
            assert torch.all(last == 0).item()
    # nothing outside the B x T x H rows of grad_hidden is touched
    if layout == "padded":
        assert torch.isnan(gbig[..., H:]).all().item()


@pytest.mark.parametrize("V", [300, 3001])
@pytest.mark.parametrize("softcap", [0.0, 30.0])
def test_shifted_contiguous_bf16(V, softcap):
    X3, W, Y2 = _seq_inputs(3, 171, 128, V, "bf16", seed=40)
    announce("rows: shifted [3,171,128]", V, softcap)
    _check(eng(), X3, W, Y2, "bf16", softcap=softcap)


@pytest.mark.parametrize("V", [300, 3001])
@pytest.mark.parametrize("layout", ["padded", "seq_major"])
def test_strided_layouts_multichunk(layout, V):
    X3, W, Y2 = _seq_inputs(3, 171, 128, V, "bf16", seed=41)
    announce("rows: layout", layout, "strided labels, chunk 256 (510 rows -> 2 chunks)", V)
    _check(eng(256), X3, W, Y2, "bf16", layout=layout, labels_layout="strided")


@pytest.mark.parametrize("acc", [(True, True), (True, False), (False, True)])
@pytest.mark.parametrize("V", [300, 3001])
def test_accumulate_and_grad_scale_bf16(acc, V):
    X3, W, Y2 = _seq_inputs(2, 200, 64, V, "bf16", seed=42)
    announce("rows: accumulate", acc, "grad_scale 0.25, padded", V)
    _check(eng(256), X3, W, Y2, "bf16", grad_scale=0.25, layout="padded", acc_gh=acc[0], acc_gw=acc[1], seed=1)


@pytest.mark.parametrize("V", [1000, 250])
@pytest.mark.parametrize("layout", ["contiguous", "seq_major"])
@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_fp32_shifted(layout, reduction, V):
    """V = 250 keeps K = V too short to split: the fp32 grad_hidden tile epilogue; V = 1000 splits K."""
    X3, W, Y2 = _seq_inputs(4, 100, 96, V, "fp32", seed=43)
    announce("rows: fp32", layout, reduction, V, "chunk 256")
    _check(eng(256), X3, W, Y2, "fp32", softcap=3.0, reduction=reduction, grad_scale=-1.5, layout=layout,
           labels_layout="strided", acc_gh=True, acc_gw=True, seed=2)


def test_no_shift_sequences_equal_plain_call_bitwise():
    """Rows already in the plain layout give exactly the plain call's results."""
    e = eng()
    dev = e.device
    X3, W, Y2 = _seq_inputs(4, 150, 128, 3001, "bf16", seed=44)
    announce("rows: [4,150,128] without shift vs the plain call")
    Xd, Wd = X3.to(dev), W.to(dev)
    l1, g1, w1 = e.forward_backward_seq(Xd, Wd, Y2.to(dev), shift=False)
    l2, g2, w2 = e.forward_backward(Xd.reshape(-1, 128), Wd, Y2.reshape(-1).to(dev))
    assert torch.equal(l1, l2) and torch.equal(g1.reshape(-1, 128), g2) and torch.equal(w1, w2)


def test_forward_seq_rows_and_loss():
    e = eng(256)
    dev = e.device
    X3, W, Y2 = _seq_inputs(3, 171, 128, 1000, "bf16", seed=45)
    announce("rows: forward only, seq_major + strided labels")
    hidden = _place_hidden(X3, "seq_major", dev)
    labels = _place_labels(Y2, "strided", dev)
    rows, lse = e.forward_seq(hidden, W.to(dev), labels, reduction="none", return_lse=True)
    assert tuple(rows.shape) == (3, 170)
    _, _, _, o_rows, o_lse = oracle.flce_sequences(X3, W, Y2, 1, IGN, 0.0, "mean")
    for got, ref, what in ((rows, o_rows, "rows"), (lse, o_lse, "lse")):
        g = got.reshape(-1).double().cpu().numpy()
        err = np.abs(g - ref) / np.maximum(np.abs(ref), 1.0)
        print(f"   {what}: max rel err {err.max():.2e}", flush=True)
        assert np.all(err <= TOL["bf16"]["loss"])
    loss = e.forward_seq(hidden, W.to(dev), labels)
    fused, _, _ = e.forward_backward_seq(hidden, W.to(dev), labels)
    assert torch.equal(loss, fused)


def test_sequence_edge_cases():
    e = eng()
    dev = e.device
    announce("rows: T = 1 with shift (no rows), B = 0, accumulate with no rows")
    W = (torch.randn(300, 64) * 0.1).to(torch.bfloat16).to(dev)
    X3 = torch.randn(5, 1, 64).to(torch.bfloat16).to(dev)
    Y2 = torch.randint(0, 300, (5, 1)).to(dev)
    gh = torch.full_like(X3, float("nan"))
    gw = torch.full((300, 64), float("nan"), device=dev)
    loss, _, _ = e.forward_backward_seq(X3, W, Y2, grad_hidden=gh, grad_W=gw)
    assert float(loss.cpu()) == 0.0 and torch.all(gh == 0).item() and torch.all(gw == 0).item()
    gh.fill_(2.0)
    gw.fill_(3.0)
    e.forward_backward_seq(X3, W, Y2, grad_hidden=gh, grad_W=gw, accumulate_grad_hidden=True,
                           accumulate_grad_W=True)
    assert torch.all(gh == 2.0).item() and torch.all(gw == 3.0).item()
    X0 = torch.empty(0, 4, 64, dtype=torch.bfloat16, device=dev)
    Y0 = torch.empty(0, 4, dtype=torch.int64, device=dev)
    loss, gh0, gw0 = e.forward_backward_seq(X0, W, Y0)
    assert float(loss.cpu()) == 0.0 and gh0.numel() == 0 and torch.all(gw0 == 0).item()


def test_llama_head_sequences_equal_plain_call_bitwise():
    """Full-size Llama-3-8B head as 8 sequences of 1025 positions with the shift (8192 rows): the
    same results, bit for bit, as the plain call on the same rows gathered in the same order
    (whose sampled rows the full-size tests check against the oracle)."""
    e = eng()
    dev = e.device
    w = inputs.WORKLOADS["llama3_8b_head"]
    announce("rows: llama3_8b_head as [8, 1025, 4096] shifted vs plain [8192, 4096]")
    X, W, y = inputs.make_inputs(w, seed=0, BT=8 * 1025)
    X3, Y2 = X.reshape(8, 1025, w.H).to(dev), y.reshape(8, 1025).to(dev)
    Wd = W.to(dev)
    l1, g1, w1 = e.forward_backward_seq(X3, Wd, Y2)
    Xp = X3[:, :-1, :].reshape(-1, w.H).contiguous()
    yp = Y2[:, 1:].reshape(-1).contiguous()
    l2, g2, w2 = e.forward_backward(Xp, Wd, yp)
    assert torch.equal(l1, l2)
    assert torch.equal(g1[:, :-1, :].reshape(-1, w.H), g2)
    assert torch.all(g1[:, -1, :] == 0).item()
    assert torch.equal(w1, w2)


def test_autograd_wrapper_on_sequences():
    """flce_loss on hidden [B,T,H] with shift: the training-loop usage (loss / accumulation steps,
    then backward) gives the oracle's scaled gradients, zero on the last positions."""
    from linear_cross_entropy_07_amd.flce import flce_loss

    dev = device()
    X3, W, Y2 = _seq_inputs(2, 129, 64, 300, "bf16", seed=46)
    announce("rows: autograd wrapper, [2,129,64] shifted, loss / 4")
    h = X3.to(dev).requires_grad_(True)
    Wd = W.to(dev).requires_grad_(True)
    loss = flce_loss(h, Wd, Y2.to(dev), shift=True)
    (loss / 4).backward()
    ol, odx, odw, _, _ = oracle.flce_sequences(X3, W, Y2, 1, IGN, 0.0, "mean", 0.25)
    assert abs(float(loss.detach().cpu()) - ol) <= TOL["bf16"]["loss"] * ol
    assert rel_fro(h.grad.double().cpu().numpy(), odx) <= TOL["bf16"]["grad"]
    assert rel_fro(Wd.grad.double().cpu().numpy(), odw) <= TOL["bf16"]["grad"]
    assert torch.all(h.grad[:, -1, :] == 0).item()
