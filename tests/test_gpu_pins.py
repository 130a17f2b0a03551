"""GPU checks of the HIP path against properties fixed by the mathematics, independent of the oracle:
central finite differences of the library's own loss against its gradients, row and vocabulary
permutations, and the chunk plan at a ragged full-size B*T (the per-row work does not depend on it)."""
import numpy as np
import pytest
import torch

from gpu_helpers import announce, device, rel_fro, run_gpu
from linear_cross_entropy_07_amd import flce, inputs

pytestmark = pytest.mark.gpu


def _tiny_fp32(rng, BT, H, V, w_scale):
    X = torch.from_numpy(rng.standard_normal((BT, H)).astype(np.float32))
    W = torch.from_numpy((rng.standard_normal((V, H)) * w_scale / np.sqrt(H)).astype(np.float32))
    y = torch.from_numpy(rng.integers(0, V, size=BT).astype(np.int64))
    return X, W, y


@pytest.mark.parametrize("softcap", [0.0, 2.5])
def test_finite_differences_fp32(softcap):
    """d loss / d x_ij and d loss / d w_vj by central differences of the GPU loss (fp32, BT=4, H=8,
    V=16) agree with the GPU gradients (a coarse check: the loss itself is fp32)."""
    dev = device()
    announce("finite differences fp32 4x8x16", f"softcap={softcap}")
    rng = np.random.default_rng(21)
    X, W, y = _tiny_fp32(rng, 4, 8, 16, 3.0)
    y[1] = -100
    e = flce.FLCE(dev)
    Xd, Wd, yd = X.to(dev), W.to(dev), y.to(dev)
    _, gh, gw = e.forward_backward(Xd, Wd, yd, softcap=softcap)
    gh, gw = gh.double().cpu().numpy(), gw.double().cpu().numpy()

    def loss_at(Xp, Wp):
        return float(e.forward(Xp, Wp, yd, softcap=softcap))

    eps = 1e-2
    worst = 0.0
    for (A, G, is_x) in ((Xd, gh, True), (Wd, gw, False)):
        for idx in np.ndindex(*A.shape):
            Ap, Am = A.clone(), A.clone()
            Ap[idx] += eps
            Am[idx] -= eps
            lp = loss_at(Ap, Wd) if is_x else loss_at(Xd, Ap)
            lm = loss_at(Am, Wd) if is_x else loss_at(Xd, Am)
            fd = (lp - lm) / (2 * eps)
            err = abs(fd - G[idx])
            worst = max(worst, err / (1e-3 + abs(G[idx])))
            assert err <= 1e-3 + 1e-2 * abs(G[idx]), (is_x, idx, fd, G[idx])
    print(f"   worst |fd - grad| / (1e-3 + |grad|) = {worst:.2e}", flush=True)
    # the ignored row has an exactly zero gradient
    assert not np.any(gh[1])


def test_row_permutation_bf16():
    """Permuting the rows (with their labels) permutes grad_hidden and leaves the loss and grad_W
    unchanged up to the order of the sums over rows."""
    dev = device()
    announce("row permutation bf16 700x256x3001")
    w = inputs.custom(BT=700, H=256, V=3001, dtype="bf16", ignore_frac=0.1, w_std=0.05, name="perm_rows")
    X, W, y = inputs.make_inputs(w, seed=22)
    perm = torch.from_numpy(np.random.default_rng(22).permutation(w.BT))
    e = flce.FLCE(dev)
    a = run_gpu(e, X, W, y)
    b = run_gpu(e, X[perm].contiguous(), W, y[perm].contiguous())
    assert abs(a[0] - b[0]) <= 1e-6 * abs(a[0])
    assert rel_fro(b[1], a[1][perm.numpy()]) <= 1e-6
    assert rel_fro(b[2], a[2]) <= 1e-5


def test_vocab_permutation_fp32():
    """Permuting the rows of W (labels remapped) permutes grad_W and leaves the loss and grad_hidden
    unchanged: softmax cross-entropy does not depend on the order of the classes (fp32, so that the
    16-bit storage of a different segment grouping does not enter)."""
    dev = device()
    announce("vocabulary permutation fp32 300x64x1000")
    w = inputs.custom(BT=300, H=64, V=1000, dtype="fp32", ignore_frac=0.1, name="perm_vocab")
    X, W, y = inputs.make_inputs(w, seed=23)
    pi = np.random.default_rng(23).permutation(w.V)      # new row k of W is old row pi[k]
    inv = np.argsort(pi)                                  # old class c is new class inv[c]
    y2 = y.clone()
    valid = y2 != -100
    y2[valid] = torch.from_numpy(inv)[y2[valid]]
    e = flce.FLCE(dev)
    a = run_gpu(e, X, W, y)
    b = run_gpu(e, X, W[torch.from_numpy(pi)].contiguous(), y2)
    assert abs(a[0] - b[0]) <= 1e-6 * abs(a[0])
    assert rel_fro(b[1], a[1]) <= 1e-5
    assert rel_fro(b[2], a[2][pi]) <= 1e-5


def test_chunk_plans_at_ragged_full_size():
    """At a ragged B*T of the Llama-3-8B head shape (6269 rows: 2 chunks of 3328 with the default
    plan, 4 of 1792 with chunk_rows_max 2048) the loss is bitwise the same and the gradients agree to
    the rounding of their last sums."""
    dev = device()
    BT = 6269
    announce(f"chunk plans at BT={BT}, H=4096, V=128256: chunk_rows_max 4096 vs 2048")
    X, W, y = inputs.make_ragged_call(BT, seed=24)
    a = run_gpu(flce.FLCE(dev), X, W, y)
    b = run_gpu(flce.FLCE(dev, chunk_rows_max=2048), X, W, y)
    print(f"   loss {a[0]:.7f} / {b[0]:.7f}; dX rel {rel_fro(b[1], a[1]):.2e}; dW rel {rel_fro(b[2], a[2]):.2e}",
          flush=True)
    assert a[0] == b[0]
    assert rel_fro(b[1], a[1]) <= 5e-3
    assert rel_fro(b[2], a[2]) <= 1e-5
