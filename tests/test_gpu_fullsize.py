"""Full-size GPU parity at the workloads' real shapes, in the launch configuration the benchmark times
(default chunk plan): the whole loss, the whole grad_hidden and the whole grad_W of one call against the
CPU float64 oracle (flce_blocked: every row's logits built in blocks of rows), plus the worst per-row
error of each gradient, and relations that hold at any size (mean = sum / N, loss additivity over a
split of the rows, <grad_W, W> = <grad_hidden, hidden>, ignored rows exactly zero).

Workloads: the Llama-3-8B head, the Gemma2 head (softcap 30), the GPT-2 head, one GPU's vocabulary share
of the Llama head, and the ragged B*T sweep's two endpoints (4096, 32768) plus three of its seeded draws.
The oracle runs on the host's cores; each case prints its phases as it goes."""
import time

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import TOL, announce, device, rel_fro
from linear_cross_entropy_07_amd import flce, inputs

pytestmark = [pytest.mark.gpu, pytest.mark.fullsize]


def _row_errors(got, ref):
    """Relative error of each row whose reference is nonzero; rows whose reference is zero must be zero."""
    nr = np.linalg.norm(ref, axis=1)
    nz = nr > 0
    assert not np.any(got[~nz]), "rows with a zero reference gradient must be exactly zero"
    return np.linalg.norm(got[nz] - ref[nz], axis=1) / nr[nz]


def _fullsize_check(X, W, y, softcap, label):
    dev = device()
    e = flce.FLCE(dev)
    BT, H = X.shape
    V = W.shape[0]
    announce(label, f"BT={BT} H={H} V={V} softcap={softcap} chunks={e.chunk_plan(BT, H, V)}")
    Xd, Wd, yd = X.to(dev), W.to(dev), y.to(dev)
    loss, gh, gw = e.forward_backward(Xd, Wd, yd, softcap=softcap)
    torch.cuda.synchronize()
    assert e.status() == 0
    loss = float(loss)
    gh_c = gh.double().cpu().numpy()
    gw_c = gw.double().cpu().numpy()
    tol = TOL["bf16"]

    # relations that hold at any size, from further GPU calls on the same inputs
    lsum = float(e.forward_backward(Xd, Wd, yd, softcap=softcap, reduction="sum")[0])
    half = BT // 2
    l1 = float(e.forward_backward(Xd[:half].contiguous(), Wd, yd[:half].contiguous(), softcap=softcap,
                                  reduction="sum")[0])
    l2 = float(e.forward_backward(Xd[half:].contiguous(), Wd, yd[half:].contiguous(), softcap=softcap,
                                  reduction="sum")[0])
    a = float((gw.double() * Wd.double()).sum())
    b = float((gh.double() * Xd.double()).sum())
    del gh, gw, Xd, Wd, yd
    torch.cuda.empty_cache()

    t0 = time.perf_counter()
    print(f"   GPU call done (loss {loss:.6f}); oracle on the host ...", flush=True)
    o_loss, o_dx, o_dw, d = oracle.flce_blocked(X, W, y, -100, softcap, "mean", block_rows=1024)
    print(f"   oracle done in {time.perf_counter() - t0:.1f} s (loss {o_loss:.6f}, N={d['N']})", flush=True)
    N = d["N"]
    valid = (y != -100).numpy()

    err_l = abs(loss - o_loss) / abs(o_loss)
    err_dx = rel_fro(gh_c, o_dx)
    err_dw = rel_fro(gw_c, o_dw)
    rows_dx = _row_errors(gh_c, o_dx)
    rows_dw = _row_errors(gw_c, o_dw)
    print(f"   loss rel {err_l:.2e}; grad_hidden rel Frobenius {err_dx:.2e} (worst row {rows_dx.max():.2e}); "
          f"grad_W rel Frobenius {err_dw:.2e} (worst row {rows_dw.max():.2e})", flush=True)
    assert err_l <= tol["loss"]
    assert err_dx <= tol["grad"]
    assert err_dw <= tol["grad"]
    # no single row may be off by more than the whole-tensor bar either
    assert rows_dx.max() <= tol["grad"]
    assert rows_dw.max() <= tol["grad"]
    assert not np.any(gh_c[~valid]), "ignored rows must get exactly zero gradient"

    assert abs(lsum / N - loss) <= 1e-5 * loss
    assert abs(l1 + l2 - lsum) <= 1e-5 * lsum
    print(f"   <dW,W> {a:.6e} <dX,X> {b:.6e}", flush=True)
    assert abs(a - b) <= 2e-2 * max(abs(a), abs(b)) + 1e-6
    assert np.isfinite(gw_c).all() and np.isfinite(gh_c).all()


@pytest.mark.parametrize("name", ["llama3_8b_head", "gemma2_head", "gpt2_head", "llama3_8b_head_vshard8"])
def test_fullsize_workload(name):
    w = inputs.WORKLOADS[name]
    X, W, y = inputs.make_inputs(w, seed=0)
    _fullsize_check(X, W, y, w.softcap, name)


def _ragged_cases():
    """The sweep's endpoints (first and last call) and three of its 20 draws, chosen by a fixed seed."""
    bts = inputs.ragged_bt_list(0, 20)
    picks = sorted(np.random.default_rng(7).choice(np.arange(1, len(bts) - 1), 3, replace=False).tolist())
    return [0, len(bts) - 1] + picks


@pytest.mark.parametrize("i", _ragged_cases())
def test_ragged_sweep_call(i):
    bts = inputs.ragged_bt_list(0, 20)
    X, W, y = inputs.make_ragged_call(bts[i], seed=100 + i)
    _fullsize_check(X, W, y, 0.0, f"ragged call {i}")
