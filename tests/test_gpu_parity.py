"""GPU parity of the HIP path against the CPU float64 oracle, element by element, on shapes that span
several tiles with ragged tails in BT, H and V, plus the edge cases of the method."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import TOL, announce, check_against_oracle, device, rel_fro, run_gpu
from linear_cross_entropy_07_amd import flce, inputs

pytestmark = pytest.mark.gpu

_ENG = {}


def eng(chunk=0):
    dev = device()
    if chunk not in _ENG:
        _ENG[chunk] = flce.FLCE(dev, chunk_rows_max=chunk)
    return _ENG[chunk]


def test_tiny_fp32_workload():
    w = inputs.WORKLOADS["tiny_fp32"]
    announce("tiny_fp32", w)
    X, W, y = inputs.make_inputs(w, seed=0)
    check_against_oracle(run_gpu(eng(), X, W, y), X, W, y, "fp32")


@pytest.mark.parametrize("softcap", [0.0, 3.0])
@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_fp32_multichunk_ragged(softcap, reduction):
    w = inputs.custom(BT=700, H=96, V=1000, dtype="fp32", ignore_frac=0.1, name="fp32_ragged")
    announce(w, softcap, reduction, "chunk 256")
    X, W, y = inputs.make_inputs(w, seed=1)
    check_against_oracle(run_gpu(eng(256), X, W, y, softcap=softcap, reduction=reduction), X, W, y, "fp32",
                         softcap=softcap, reduction=reduction)


@pytest.mark.parametrize("softcap", [0.0, 30.0])
@pytest.mark.parametrize("reduction", ["mean", "sum"])
@pytest.mark.parametrize("shape", [(300, 128, 1000), (513, 264, 3001), (1000, 256, 5000)])
def test_bf16_small(shape, softcap, reduction):
    BT, H, V = shape
    w = inputs.custom(BT=BT, H=H, V=V, dtype="bf16", ignore_frac=0.1, w_std=0.05, name="bf16_small")
    announce(w, softcap, reduction)
    X, W, y = inputs.make_inputs(w, seed=2)
    check_against_oracle(run_gpu(eng(), X, W, y, softcap=softcap, reduction=reduction), X, W, y, "bf16",
                         softcap=softcap, reduction=reduction)


def test_bf16_multichunk_ragged():
    w = inputs.custom(BT=1000, H=256, V=5000, dtype="bf16", ignore_frac=0.05, w_std=0.05, name="bf16_chunks")
    announce(w, "chunk 256 -> 4 chunks (256, 256, 256, 232)")
    X, W, y = inputs.make_inputs(w, seed=3)
    check_against_oracle(run_gpu(eng(256), X, W, y), X, W, y, "bf16")


def test_bf16_gpt2_slice_v_tail():
    w = inputs.with_bt(inputs.WORKLOADS["gpt2_head"], 512)
    announce(w)
    X, W, y = inputs.make_inputs(w, seed=4)
    check_against_oracle(run_gpu(eng(), X, W, y), X, W, y, "bf16")


def test_bf16_large_logits_zipf_rmsnorm():
    # the Llama-head input recipe (RMS-normalised hidden, Zipf labels) at a reduced V and H,
    # with W scaled up so that the softmax is sharp
    w = inputs.custom(BT=512, H=512, V=4000, dtype="bf16", ignore_frac=0.05, labels="zipf1.1",
                      x_rmsnorm=True, w_std=0.2, name="sharp")
    announce(w)
    X, W, y = inputs.make_inputs(w, seed=5)
    check_against_oracle(run_gpu(eng(), X, W, y), X, W, y, "bf16")


@pytest.mark.parametrize("dtype,a", [("fp32", 64.0), ("fp32", 128.0), ("bf16", 1024.0)])
def test_logit_shift_metamorphic(dtype, a):
    """A ones-column in X and a constant-a column in W shift every logit by a, which the softmax ignores.
    The GPU result on the shifted problem must match the oracle on the unshifted one: loss, the original
    columns of dX and dW, dW's new column = sum_t dZ[t, v], and dX's new column = a * sum_v dZ = 0 (up to
    the cancellation error of a sum of V terms of size g, amplified by a). exp would overflow fp32 at
    a = 128 without the max subtraction."""
    BT, H, V = 300, 64, 1000
    rng = np.random.default_rng(6)
    X = rng.standard_normal((BT, H)).astype(np.float32)
    W = (rng.standard_normal((V, H)) / 8).astype(np.float32)
    y = rng.integers(0, V, BT)
    tdt = torch.float32 if dtype == "fp32" else torch.bfloat16
    # the unshifted problem on exactly the values the GPU sees
    Xr = torch.from_numpy(X).to(tdt)
    Wr = torch.from_numpy(W).to(tdt)
    Xa = torch.cat([Xr, torch.ones((BT, 1), dtype=tdt), torch.zeros((BT, 7), dtype=tdt)], 1).contiguous()
    Wa = torch.cat([Wr, torch.full((V, 1), a, dtype=tdt), torch.zeros((V, 7), dtype=tdt)], 1).contiguous()
    yt = torch.from_numpy(y)
    announce("shift", dtype, a)
    gl, gdx, gdw = run_gpu(eng(), Xa, Wa, yt)
    ol, odx, odw, det = oracle.flce_forward_backward(Xr, Wr, yt, return_details=True)
    tol = TOL[dtype]
    e = (abs(gl - ol) / ol, rel_fro(gdx[:, :H], odx), rel_fro(gdw[:, :H], odw),
         rel_fro(gdw[:, H], det["dZ"].sum(axis=0)))
    print(f"   loss {gl:.7f} vs {ol:.7f}: rel {e[0]:.2e}; dX {e[1]:.2e}; dW {e[2]:.2e}; dW shift col {e[3]:.2e}",
          flush=True)
    assert e[0] <= tol["loss"] and e[1] <= tol["grad"] and e[2] <= tol["grad"] and e[3] <= tol["grad"]
    # sum_v |dZ[t, v]| <= 2 g, so the ones column of dX is bounded by a * 2/N * (relative rounding)
    ulp = 2.0 ** -23 if dtype == "fp32" else 2.0 ** -8
    assert np.abs(gdx[:, H]).max() <= a * 2.0 / BT * ulp * 64 * 4
    assert not np.any(gdx[:, H + 1:]) and not np.any(gdw[:, H + 1:])


@pytest.mark.parametrize("shape,softcap", [((300, 64, 1 << 20), 30.0), ((300, 65536, 1000), 0.0)],
                         ids=["V=2^20", "H=65536"])
def test_maximum_sizes(shape, softcap):
    """The largest vocabulary (2^20) and hidden size (65536) the library accepts, against the oracle."""
    BT, H, V = shape
    w = inputs.custom(BT=BT, H=H, V=V, dtype="bf16", ignore_frac=0.1, w_std=0.05, name="max_size")
    announce(w, softcap)
    X, W, y = inputs.make_inputs(w, seed=14)
    check_against_oracle(run_gpu(eng(), X, W, y, softcap=softcap), X, W, y, "bf16", softcap=softcap)
    # one more row or column than that is refused before anything runs
    dev = device()
    with pytest.raises(flce.FlceError) as ei:
        if V == 1 << 20:
            eng().forward_backward(X[:4].to(dev), torch.zeros(V + 1, H, dtype=torch.bfloat16, device=dev),
                                   y[:4].to(dev))
        else:
            eng().forward_backward(torch.zeros(4, H + 8, dtype=torch.bfloat16, device=dev),
                                   torch.zeros(V, H + 8, dtype=torch.bfloat16, device=dev), y[:4].to(dev))
    assert ei.value.code == -2


def test_bt_zero():
    dev = device()
    announce("BT=0")
    X = torch.empty((0, 64), dtype=torch.bfloat16, device=dev)
    W = torch.randn((100, 64), device=dev).to(torch.bfloat16)
    y = torch.empty((0,), dtype=torch.int64, device=dev)
    loss, gh, gw = eng().forward_backward(X, W, y)
    torch.cuda.synchronize()
    assert float(loss) == 0.0 and gh.numel() == 0 and not torch.any(gw != 0)


@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_all_rows_ignored(reduction):
    announce("all ignored", reduction)
    w = inputs.custom(BT=300, H=64, V=500, dtype="bf16", name="ign")
    X, W, _ = inputs.make_inputs(w, seed=7)
    y = torch.full((300,), -100, dtype=torch.int64)
    gl, gdx, gdw = run_gpu(eng(), X, W, y, reduction=reduction)
    assert gl == 0.0 and not np.any(gdx) and not np.any(gdw)


def test_ignored_rows_give_exact_zero_rows_and_custom_ignore_index():
    announce("ignore_index=7 rows zero")
    w = inputs.custom(BT=400, H=128, V=700, dtype="bf16", w_std=0.05, name="ign7")
    X, W, y = inputs.make_inputs(w, seed=8)
    y[::5] = 7  # label 7 is the ignore_index here
    gl, gdx, gdw = run_gpu(eng(), X, W, y, ignore_index=7)
    assert not np.any(gdx[::5])
    check_against_oracle((gl, gdx, gdw), X, W, y, "bf16", ignore_index=7)


def test_single_row_single_class_and_min_hidden():
    announce("BT=1, V=1, H=8")
    X = torch.randn(1, 8).to(torch.bfloat16)
    W = torch.randn(1, 8).to(torch.bfloat16)
    y = torch.zeros(1, dtype=torch.int64)
    gl, gdx, gdw = run_gpu(eng(), X, W, y)
    assert gl == 0.0 and np.abs(gdx).max() == 0.0 and np.abs(gdw).max() == 0.0
    w = inputs.custom(BT=1, H=8, V=3, dtype="fp32", name="one")
    X, W, y = inputs.make_inputs(w, seed=9)
    check_against_oracle(run_gpu(eng(), X, W, y), X, W, y, "fp32")


def test_zero_weight_closed_form_on_gpu():
    announce("W=0 -> loss ln V, dX = 0")
    w = inputs.custom(BT=300, H=64, V=777, dtype="bf16", ignore_frac=0.1, name="w0")
    X, _, y = inputs.make_inputs(w, seed=10)
    W = torch.zeros((777, 64), dtype=torch.bfloat16)
    for cap in (0.0, 5.0):
        gl, gdx, gdw = run_gpu(eng(), X, W, y, softcap=cap)
        assert abs(gl - np.log(777)) <= 1e-3 * np.log(777)
        assert not np.any(gdx)
        check_against_oracle((gl, gdx, gdw), X, W, y, "bf16", softcap=cap)


def test_out_of_range_label_sets_status_and_counts_as_ignored():
    dev = device()
    announce("label out of range")
    w = inputs.custom(BT=64, H=64, V=100, dtype="fp32", name="oor")
    X, W, y = inputs.make_inputs(w, seed=11)
    y_bad = y.clone()
    y_bad[3] = 100
    y_bad[9] = -5
    e = eng()
    gl, gdx, gdw = run_gpu(e, X, W, y_bad)
    assert e.status() == -5  # FLCE_ERR_LABEL_RANGE
    y_ign = y.clone()
    y_ign[3] = -100
    y_ign[9] = -100
    check_against_oracle((gl, gdx, gdw), X, W, y_ign, "fp32")
    run_gpu(e, X, W, y)
    assert e.status() == 0


def test_chunking_invariance_and_determinism():
    """Per-row work does not depend on the chunk plan: the loss is bitwise equal across chunk sizes;
    repeated calls are bitwise identical."""
    announce("chunk invariance 1000 rows: 4096 vs 256 vs 512")
    w = inputs.custom(BT=1000, H=256, V=3000, dtype="bf16", ignore_frac=0.05, w_std=0.05, name="inv")
    X, W, y = inputs.make_inputs(w, seed=12)
    a = run_gpu(eng(), X, W, y)
    b = run_gpu(eng(256), X, W, y)
    c = run_gpu(eng(512), X, W, y)
    a2 = run_gpu(eng(), X, W, y)
    assert a[0] == b[0] == c[0]
    assert rel_fro(b[1], a[1]) < 5e-3 and rel_fro(b[2], a[2]) < 1e-5
    assert a2[0] == a[0] and np.array_equal(a2[1], a[1]) and np.array_equal(a2[2], a[2])


def test_grad_w_split_last_wave():
    """grad_W tiles of a sparse last wave are computed as K parts and added in a fixed order (calls of
    several chunks): 3000 rows in chunks of 1024 give 12 grad_W tiles per chunk, each split 4 ways, the
    later chunks accumulating. Against the oracle, and bitwise repeatable."""
    announce("grad_W last-wave split: BT 3000, H 256, V 3000, chunks of 1024")
    w = inputs.custom(BT=3000, H=256, V=3000, dtype="bf16", ignore_frac=0.05, w_std=0.05, name="tail")
    X, W, y = inputs.make_inputs(w, seed=14)
    e = eng(1024)
    a = run_gpu(e, X, W, y)
    b = run_gpu(e, X, W, y)
    assert a[0] == b[0] and np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])
    check_against_oracle(a, X, W, y, "bf16")


def test_autograd_wrapper_scales_by_upstream_grad():
    dev = device()
    announce("autograd wrapper, loss / 4")
    w = inputs.custom(BT=256, H=64, V=500, dtype="fp32", ignore_frac=0.1, name="ag")
    X, W, y = inputs.make_inputs(w, seed=13)
    Xd = X.to(dev).requires_grad_(True)
    Wd = W.to(dev).requires_grad_(True)
    loss = flce.flce_loss(Xd, Wd, y.to(dev))
    (loss / 4).backward()
    ol, odx, odw = oracle.flce_forward_backward(X, W, y)
    assert abs(float(loss) - ol) <= 1e-5 * ol
    assert rel_fro(Xd.grad.double().cpu().numpy(), odx / 4) < 1e-4
    assert rel_fro(Wd.grad.double().cpu().numpy(), odw / 4) < 1e-4


def test_workspace_too_small_is_rejected():
    dev = device()
    announce("workspace too small")
    X = torch.randn(64, 64, device=dev)
    W = torch.randn(100, 64, device=dev)
    y = torch.zeros(64, dtype=torch.int64, device=dev)
    e = eng()
    ws = torch.empty(1024, dtype=torch.uint8, device=dev)
    with pytest.raises(flce.FlceError) as ei:
        e.forward_backward(X, W, y, workspace=ws)
    assert ei.value.code == -3


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("softcap,far,near,every", [(0.0, 60.0, 40.0, 5), (30.0, 120.0, 40.0, 5),
                                                    (0.0, 70.0, 70.0, 1)])
def test_label_far_below_the_row_maximum(dtype, softcap, far, near, every):
    """Rows whose label logit lies more than the library's reference span (48) below their largest logit
    (their stored softmax numerators are re-referenced to the row maximum after the statistics are
    known), next to rows 40 below it (large numerators, no re-reference), in several chunks; with
    every=1 all rows are of the first kind."""
    X, W, y = inputs.far_label_case(700, 128, 3000, dtype, far=far, near=near, every=every, seed=11)
    announce("label far below the row maximum", dtype, f"softcap={softcap} far={far} near={near} every={every}",
             "chunk 256")
    check_against_oracle(run_gpu(eng(256), X, W, y, softcap=softcap), X, W, y, dtype, softcap=softcap)
