"""Pins for the CPU float64 oracle (no GPU).

Each test ties the oracle to something other than itself: closed forms of the
loss and gradients, central finite differences of the oracle's own loss, an
independent library implementation (PyTorch CPU float64 cross_entropy +
autograd), invariants that hold exactly, and metamorphic relations. A final
group plants mistakes in the oracle and checks that the pins catch them.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import flce_oracle as O

IGN = -100


def _rand_case(rng, BT, H, V, ignore=0, w_scale=1.0):
    X = rng.standard_normal((BT, H))
    W = rng.standard_normal((V, H)) * w_scale / math.sqrt(H)
    y = rng.integers(0, V, size=BT)
    if ignore:
        y[rng.permutation(BT)[:ignore]] = IGN
    return X, W, y


def _torch_reference(X, W, y, softcap, reduction):
    """Independent implementation: torch float64 linear + (softcap) + F.cross_entropy + autograd."""
    Xt = torch.tensor(X, dtype=torch.float64, requires_grad=True)
    Wt = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    yt = torch.tensor(y, dtype=torch.int64)
    z = torch.nn.functional.linear(Xt, Wt)
    if softcap > 0:
        z = softcap * torch.tanh(z / softcap)
    loss = torch.nn.functional.cross_entropy(z, yt, ignore_index=IGN, reduction=reduction)
    loss.backward()
    return loss.item(), Xt.grad.numpy(), Wt.grad.numpy()


def _rel(a, b):
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("softcap", [0.0, 5.0])
@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_zero_weight_closed_form(softcap, reduction):
    """W = 0: every logit is 0, softmax is uniform, loss = ln V per valid row; dX = 0;
    dW[v] = g * ((1/V) sum_valid x_t - sum_{valid t, y_t = v} x_t)."""
    rng = np.random.default_rng(1)
    BT, H, V = 13, 6, 11
    X = rng.standard_normal((BT, H))
    W = np.zeros((V, H))
    y = rng.integers(0, V, size=BT)
    y[[2, 7]] = IGN
    valid = y != IGN
    N = int(valid.sum())
    loss, dX, dW = oracle.flce_forward_backward(X, W, y, IGN, softcap, reduction)
    g = 1.0 / N if reduction == "mean" else 1.0
    expect_loss = math.log(V) * (1.0 if reduction == "mean" else N)
    assert abs(loss - expect_loss) <= 1e-13 * expect_loss
    assert np.all(dX == 0.0)
    expect_dW = np.zeros((V, H))
    xs = X[valid].sum(axis=0)
    for v in range(V):
        expect_dW[v] = g * (xs / V - X[valid & (y == v)].sum(axis=0))
    np.testing.assert_allclose(dW, expect_dW, rtol=0, atol=1e-14)


def test_single_class_is_zero():
    """V = 1: softmax is 1 at the label, so the loss and every gradient are 0."""
    rng = np.random.default_rng(2)
    X = rng.standard_normal((5, 4))
    W = rng.standard_normal((1, 4))
    y = np.zeros(5, dtype=np.int64)
    loss, dX, dW = oracle.flce_forward_backward(X, W, y)
    assert loss == 0.0
    assert np.abs(dX).max() < 1e-15 and np.abs(dW).max() < 1e-15


def test_two_class_softplus_closed_form():
    """V = 2, H = 1: loss = softplus(z_other - z_label), dX = sigma * (w_other - w_label),
    dW_label = -sigma * x, dW_other = sigma * x with sigma = logistic(z_other - z_label)."""
    x, a, b = 1.5, 0.5, -0.25
    X = np.array([[x]])
    W = np.array([[a], [b]])
    for label, (wl, wo) in ((0, (a, b)), (1, (b, a))):
        loss, dX, dW = oracle.flce_forward_backward(X, W, np.array([label]))
        u = x * (wo - wl)
        sig = 1.0 / (1.0 + math.exp(-u))
        assert abs(loss - math.log1p(math.exp(u))) < 1e-15
        assert abs(dX[0, 0] - sig * (wo - wl)) < 1e-15
        assert abs(dW[label, 0] + sig * x) < 1e-15
        assert abs(dW[1 - label, 0] - sig * x) < 1e-15


def test_no_valid_rows_gives_zero():
    rng = np.random.default_rng(3)
    X, W, _ = _rand_case(rng, 6, 4, 9)
    y = np.full(6, IGN)
    for red in ("mean", "sum"):
        loss, dX, dW = oracle.flce_forward_backward(X, W, y, reduction=red)
        assert loss == 0.0 and not dX.any() and not dW.any()


def test_label_out_of_range_raises():
    X, W, _ = _rand_case(np.random.default_rng(4), 3, 4, 5)
    with pytest.raises(ValueError):
        oracle.flce_forward_backward(X, W, np.array([0, 5, 1]))
    with pytest.raises(ValueError):
        oracle.flce_forward_backward(X, W, np.array([0, -1, 1]))


# ---------------------------------------------------------------- finite differences

@pytest.mark.parametrize("softcap", [0.0, 1.5])
@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_finite_differences(softcap, reduction):
    """Central differences of the oracle's loss match its analytic dX and dW entry by entry."""
    rng = np.random.default_rng(5)
    BT, H, V = 4, 8, 16
    X, W, y = _rand_case(rng, BT, H, V, w_scale=3.0)
    y[1] = IGN
    _, dX, dW = oracle.flce_forward_backward(X, W, y, IGN, softcap, reduction)
    h = 1e-5

    def L(Xp, Wp):
        return oracle.flce_forward_backward(Xp, Wp, y, IGN, softcap, reduction)[0]

    fdX = np.zeros_like(X)
    for i in range(BT):
        for j in range(H):
            Xp, Xm = X.copy(), X.copy()
            Xp[i, j] += h
            Xm[i, j] -= h
            fdX[i, j] = (L(Xp, W) - L(Xm, W)) / (2 * h)
    fdW = np.zeros_like(W)
    for i in range(V):
        for j in range(H):
            Wp, Wm = W.copy(), W.copy()
            Wp[i, j] += h
            Wm[i, j] -= h
            fdW[i, j] = (L(X, Wp) - L(X, Wm)) / (2 * h)
    np.testing.assert_allclose(dX, fdX, rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dW, fdW, rtol=1e-6, atol=1e-8)
    assert np.all(dX[1] == 0.0)


# ---------------------------------------------------------------- library cross-check

@pytest.mark.parametrize("softcap", [0.0, 4.0])
@pytest.mark.parametrize("reduction", ["mean", "sum"])
@pytest.mark.parametrize("shape", [(256, 64, 1000), (64, 32, 50), (7, 8, 3)])
def test_matches_torch_cross_entropy(softcap, reduction, shape):
    BT, H, V = shape
    rng = np.random.default_rng(6)
    X, W, y = _rand_case(rng, BT, H, V, ignore=max(1, BT // 10), w_scale=4.0)
    loss, dX, dW = oracle.flce_forward_backward(X, W, y, IGN, softcap, reduction)
    tl, tdX, tdW = _torch_reference(X, W, y, softcap, reduction)
    assert abs(loss - tl) <= 1e-12 * abs(tl)
    assert _rel(dX, tdX) < 1e-12
    assert _rel(dW, tdW) < 1e-12


# ---------------------------------------------------------------- forward-only oracle

@pytest.mark.parametrize("softcap", [0.0, 4.0])
@pytest.mark.parametrize("shape", [(256, 64, 1000), (7, 8, 3)])
def test_forward_rows_match_torch(softcap, shape):
    """Per-row NLL and lse against torch float64 cross_entropy(reduction='none') and logsumexp."""
    BT, H, V = shape
    rng = np.random.default_rng(16)
    X, W, y = _rand_case(rng, BT, H, V, ignore=max(1, BT // 10), w_scale=4.0)
    rows, lse = oracle.flce_forward(X, W, y, IGN, softcap, "none")
    z = torch.nn.functional.linear(torch.tensor(X), torch.tensor(W))
    if softcap > 0:
        z = softcap * torch.tanh(z / softcap)
    t_rows = torch.nn.functional.cross_entropy(z, torch.tensor(y), ignore_index=IGN, reduction="none").numpy()
    t_lse = torch.logsumexp(z, dim=1).numpy()
    np.testing.assert_allclose(rows, t_rows, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, t_lse, rtol=1e-12, atol=0)
    assert np.all(rows[y == IGN] == 0.0)
    for red in ("mean", "sum"):
        loss, lse2 = oracle.flce_forward(X, W, y, IGN, softcap, red)
        tl = torch.nn.functional.cross_entropy(z, torch.tensor(y), ignore_index=IGN, reduction=red).item()
        assert abs(loss - tl) <= 1e-12 * abs(tl)
        np.testing.assert_array_equal(lse2, lse)


def test_forward_zero_weight_closed_form():
    """W = 0: every row's lse is ln V, every valid row's term is ln V, ignored rows give 0."""
    rng = np.random.default_rng(17)
    X, _, y = _rand_case(rng, 33, 8, 21, ignore=4)
    W = np.zeros((21, 8))
    rows, lse = oracle.flce_forward(X, W, y, IGN, 0.0, "none")
    np.testing.assert_allclose(lse, math.log(21), rtol=1e-15)
    np.testing.assert_allclose(rows, np.where(y == IGN, 0.0, math.log(21)), rtol=1e-15)
    loss, _ = oracle.flce_forward(X, W, y, IGN, 0.0, "mean")
    assert abs(loss - math.log(21)) < 1e-14


# ---------------------------------------------------------------- invariants and metamorphic relations

@pytest.mark.parametrize("softcap", [0.0, 3.0])
def test_invariants(softcap):
    rng = np.random.default_rng(7)
    X, W, y = _rand_case(rng, 40, 16, 30, ignore=5, w_scale=5.0)
    loss, dX, dW, t = oracle.flce_forward_backward(X, W, y, IGN, softcap, "mean", return_details=True)
    # each valid row of dlogits sums to 0 only without the softcap factor; sum over v of dS is 0,
    # so without softcap sum_v dW[v, h] = 0 for every h
    if softcap == 0.0:
        assert np.abs(t["dZ"].sum(axis=1)).max() < 1e-15
        assert np.abs(dW.sum(axis=0)).max() < 1e-14
    # <dW, W> = <dX, X> = sum dZ * Z holds with or without softcap
    assert abs((dW * W).sum() - (dX * X).sum()) < 1e-12
    # ignored rows contribute nothing
    ign = y == IGN
    assert np.all(dX[ign] == 0.0) and np.all(t["loss_rows"][ign] == 0.0)
    # sum = mean * N
    ls, dXs, dWs = oracle.flce_forward_backward(X, W, y, IGN, softcap, "sum")
    N = int((~ign).sum())
    assert abs(ls - loss * N) < 1e-12 * ls
    np.testing.assert_allclose(dXs, dX * N, rtol=1e-12, atol=1e-15)


def test_ignored_row_content_is_irrelevant():
    rng = np.random.default_rng(8)
    X, W, y = _rand_case(rng, 10, 8, 12)
    y[3] = IGN
    a = oracle.flce_forward_backward(X, W, y)
    X2 = X.copy()
    X2[3] = rng.standard_normal(8) * 100
    b = oracle.flce_forward_backward(X2, W, y)
    assert a[0] == b[0]
    np.testing.assert_array_equal(a[1], b[1])
    np.testing.assert_allclose(a[2], b[2], rtol=0, atol=1e-15)


@pytest.mark.parametrize("a", [64.0, 128.0, 1024.0])
def test_logit_shift_invariance(a):
    """Append a ones-column to X and a constant-a column to W: every logit shifts by a, which the
    softmax ignores (no softcap). Loss and the original gradient columns are unchanged; the new
    dX column is a * sum_v dZ = 0 and the new dW column is sum_t dZ[t, v]."""
    rng = np.random.default_rng(9)
    X, W, y = _rand_case(rng, 20, 8, 25, ignore=2, w_scale=3.0)
    loss, dX, dW, t = oracle.flce_forward_backward(X, W, y, return_details=True)
    Xa = np.concatenate([X, np.ones((20, 1)), np.zeros((20, 7))], axis=1)
    Wa = np.concatenate([W, np.full((25, 1), a), np.zeros((25, 7))], axis=1)
    la, dXa, dWa = oracle.flce_forward_backward(Xa, Wa, y)
    assert abs(la - loss) < 1e-12 * abs(loss) + 1e-13 * a
    np.testing.assert_allclose(dXa[:, :8], dX, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(dWa[:, :8], dW, rtol=1e-9, atol=1e-12)
    assert np.abs(dXa[:, 8]).max() < 1e-9
    np.testing.assert_allclose(dWa[:, 8], t["dZ"].sum(axis=0), rtol=0, atol=1e-9)


def test_row_permutation():
    rng = np.random.default_rng(10)
    X, W, y = _rand_case(rng, 16, 8, 20, ignore=3)
    perm = rng.permutation(16)
    a = oracle.flce_forward_backward(X, W, y)
    b = oracle.flce_forward_backward(X[perm], W, y[perm])
    assert abs(a[0] - b[0]) < 1e-13
    np.testing.assert_allclose(b[1], a[1][perm], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(b[2], a[2], rtol=1e-11, atol=1e-15)


def test_vocab_permutation():
    rng = np.random.default_rng(11)
    X, W, y = _rand_case(rng, 16, 8, 20, ignore=3)
    perm = rng.permutation(20)          # new row i of W is old row perm[i]
    inv = np.argsort(perm)
    y2 = np.where(y == IGN, IGN, inv[np.where(y == IGN, 0, y)])
    a = oracle.flce_forward_backward(X, W, y)
    b = oracle.flce_forward_backward(X, W[perm], y2)
    assert abs(a[0] - b[0]) < 1e-13
    np.testing.assert_allclose(b[2], a[2][perm], rtol=1e-12, atol=1e-15)


def test_softcap_limits():
    rng = np.random.default_rng(12)
    X, W, y = _rand_case(rng, 30, 16, 40, ignore=3, w_scale=30.0)
    c = 2.0
    loss = oracle.flce_forward_backward(X, W, y, IGN, c)[0]
    assert loss <= math.log(40) + 2 * c
    big = oracle.flce_forward_backward(X, W, y, IGN, 1e6)
    off = oracle.flce_forward_backward(X, W, y, IGN, 0.0)
    assert abs(big[0] - off[0]) < 1e-6 * abs(off[0])
    assert _rel(big[1], off[1]) < 1e-6 and _rel(big[2], off[2]) < 1e-6


def test_loss_expectation_at_tiny_workload():
    """x ~ N(0,1), W ~ N(0, 1/H) gives logits ~ N(0, |x|^2/H) roughly; E[loss] is close to
    ln V + sigma^2/2 for uniform labels (a coarse statistical sanity band)."""
    from linear_cross_entropy_07_amd import inputs

    w = inputs.WORKLOADS["tiny_fp32"]
    X, W, y = inputs.make_inputs(w, seed=0)
    loss = oracle.flce_forward_backward(X, W, y)[0]
    sigma2 = float((X.double() ** 2).sum(1).mean()) / w.H
    assert abs(loss - (math.log(w.V) + sigma2 / 2)) < 0.1


def test_flce_rows_matches_full():
    rng = np.random.default_rng(13)
    X, W, y = _rand_case(rng, 30, 8, 25, ignore=4)
    loss, dX, dW, t = oracle.flce_forward_backward(X, W, y, return_details=True)
    rows = [0, 5, 17, 29]
    r = oracle.flce_rows(X, W, y, rows, n_valid=t["N"])
    np.testing.assert_allclose(r["dX"], dX[rows], rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(r["lse"], t["lse"][rows], rtol=1e-14)


def _vocab_rows_case():
    rng = np.random.default_rng(15)
    X, W, y = _rand_case(rng, 37, 8, 29, ignore=5, w_scale=3.0)
    y[30:36] = 3  # one vocabulary row that is the label of many rows
    return X, W, y, [0, 3, 11, 28]


@pytest.mark.parametrize("softcap", [0.0, 2.5])
@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_vocab_rows_match_torch(softcap, reduction):
    """Selected grad_W rows, computed in row blocks, against torch autograd and the full oracle."""
    X, W, y, vrows = _vocab_rows_case()
    _, _, tdW = _torch_reference(X, W, y, softcap, reduction)
    r = oracle.flce_vocab_rows(X, W, y, vrows, softcap=softcap, reduction=reduction, block_rows=8)
    assert _rel(r["dW"], tdW[vrows]) < 1e-12
    full = oracle.flce_forward_backward(X, W, y, softcap=softcap, reduction=reduction, return_details=True)
    np.testing.assert_allclose(r["dW"], full[2][vrows], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(r["lse"], full[3]["lse"], rtol=1e-14)
    assert r["N"] == full[3]["N"]


@pytest.mark.parametrize("mutation", ["no_softcap", "transposed_logits_use", "lse_without_max"])
def test_vocab_rows_pin_catches_planted_mistakes(monkeypatch, mutation):
    X, W, y, vrows = _vocab_rows_case()
    _, _, tdW = _torch_reference(X, W, y, 2.5, "mean")
    if mutation == "no_softcap":
        monkeypatch.setattr(O, "apply_softcap", lambda Z, c: Z)
    elif mutation == "transposed_logits_use":
        monkeypatch.setattr(O, "logits", lambda X, W: (X @ W.T)[:, ::-1].copy())
    else:
        monkeypatch.setattr(O, "row_logsumexp", lambda S: (S.max(1), np.log(np.exp(S).sum(1)) + 0.01))
    r = oracle.flce_vocab_rows(X, W, y, vrows, softcap=2.5, block_rows=8)
    assert _rel(r["dW"], tdW[vrows]) > 1e-6


# ---------------------------------------------------------------- planted mistakes must be caught

def _pins_pass(monkeypatch=None):
    rng = np.random.default_rng(14)
    X, W, y = _rand_case(rng, 9, 8, 12, ignore=2, w_scale=3.0)
    for softcap in (0.0, 2.5):
        loss, dX, dW = O.flce_forward_backward(X, W, y, IGN, softcap, "mean")
        tl, tdX, tdW = _torch_reference(X, W, y, softcap, "mean")
        if abs(loss - tl) > 1e-10 or _rel(dX, tdX) > 1e-10 or _rel(dW, tdW) > 1e-10:
            return False
    return True


def test_pins_accept_the_oracle():
    assert _pins_pass()


@pytest.mark.parametrize("mutation", ["no_softcap", "transposed_logits_use", "drop_onehot",
                                      "wrong_sign", "lse_without_max", "softcap_grad_dropped"])
def test_pins_catch_planted_mistakes(monkeypatch, mutation):
    if mutation == "no_softcap":
        monkeypatch.setattr(O, "apply_softcap", lambda Z, c: Z)
    elif mutation == "transposed_logits_use":
        monkeypatch.setattr(O, "logits", lambda X, W: (X @ W.T)[:, ::-1].copy())
    elif mutation == "lse_without_max":
        monkeypatch.setattr(O, "row_logsumexp", lambda S: (S.max(1), np.log(np.exp(S).sum(1)) + 0.01))
    else:
        real = O._row_terms

        def patched(*a, **k):
            t = real(*a, **k)
            X, W, y, ign, softcap = a[0], a[1], a[2], a[3], a[4]
            if mutation == "drop_onehot":
                rows = np.nonzero(t["valid"])[0]
                t["dZ"][rows, y[rows]] += t["g"][rows] * (1.0 if softcap == 0 else 0.5)
            elif mutation == "wrong_sign":
                t["dZ"] = -t["dZ"]
            elif mutation == "softcap_grad_dropped" and softcap > 0:
                Z = O.apply_softcap(O.logits(X, W), softcap)
                t["dZ"] = t["dZ"] / (1.0 - (Z / softcap) ** 2)
            return t

        monkeypatch.setattr(O, "_row_terms", patched)
    assert not _pins_pass()


# ---------------------------------------------------------------- batches of sequences (label shift)

def _torch_sequences(X3, W, Y2, shift, softcap, reduction, grad_scale, dX0, dW0):
    """Independent implementation: the training-loop form, with torch float64 autograd. The logits
    of all positions are formed, sliced to the first T-1 positions and the labels to the last T-1
    (shift), cross_entropy is taken, and loss * grad_scale is back-propagated into grads that
    already hold dX0 / dW0."""
    Xt = torch.tensor(X3, dtype=torch.float64, requires_grad=True)
    Wt = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    Xt.grad = torch.tensor(dX0, dtype=torch.float64)
    Wt.grad = torch.tensor(dW0, dtype=torch.float64)
    z = torch.nn.functional.linear(Xt, Wt)  # [B, T, V]
    if softcap > 0:
        z = softcap * torch.tanh(z / softcap)
    yt = torch.tensor(Y2, dtype=torch.int64)
    if shift:
        z, yt = z[:, :-1, :], yt[:, 1:]
    loss = torch.nn.functional.cross_entropy(z.reshape(-1, z.shape[-1]), yt.reshape(-1), ignore_index=IGN,
                                             reduction=reduction)
    (loss * grad_scale).backward()
    return loss.item(), Xt.grad.numpy(), Wt.grad.numpy()


def _seq_case(rng, B, T, H, V, ignore):
    X3 = rng.standard_normal((B, T, H))
    W = rng.standard_normal((V, H)) * 3.0 / math.sqrt(H)
    Y2 = rng.integers(0, V, size=(B, T))
    flat = Y2.reshape(-1)
    flat[rng.permutation(B * T)[:ignore]] = IGN
    return X3, W, flat.reshape(B, T)


@pytest.mark.parametrize("shift", [1, 0])
@pytest.mark.parametrize("softcap", [0.0, 3.0])
@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_sequences_match_torch_training_loop(shift, softcap, reduction):
    rng = np.random.default_rng(30)
    X3, W, Y2 = _seq_case(rng, 3, 11, 16, 37, ignore=5)
    dX0 = rng.standard_normal(X3.shape)
    dW0 = rng.standard_normal(W.shape)
    for scale, init in ((1.0, False), (0.25, True), (-2.0, True)):
        loss, dX, dW, rows, lse = oracle.flce_sequences(X3, W, Y2, shift, IGN, softcap, reduction, scale,
                                                        dX0 if init else None, dW0 if init else None)
        tl, tdX, tdW = _torch_sequences(X3, W, Y2, shift, softcap, reduction, scale,
                                        dX0 if init else np.zeros_like(X3), dW0 if init else np.zeros_like(W))
        assert abs(loss - tl) <= 1e-12 * abs(tl)
        assert _rel(dX, tdX) < 1e-12 and _rel(dW, tdW) < 1e-12
        assert rows.shape == (3 * (11 - shift),) and lse.shape == rows.shape
    # the last position of each sequence gets no gradient of its own under the shift
    _, dX, _, _, _ = oracle.flce_sequences(X3, W, Y2, shift, IGN, softcap, reduction)
    if shift:
        assert np.all(dX[:, -1, :] == 0.0)


def test_sequences_rows_are_the_shifted_pairs():
    """Row b*(T-1)+t of the shifted form is the pair (hidden (b, t), label (b, t+1)) of the plain form."""
    rng = np.random.default_rng(31)
    X3, W, Y2 = _seq_case(rng, 2, 6, 8, 13, ignore=2)
    _, _, _, rows, lse = oracle.flce_sequences(X3, W, Y2, 1, IGN, 0.0, "mean")
    X = X3[:, :-1, :].reshape(-1, 8)
    y = Y2[:, 1:].reshape(-1)
    r2, l2 = oracle.flce_forward(X, W, y, IGN, 0.0, "none")
    np.testing.assert_array_equal(rows, r2)
    np.testing.assert_array_equal(lse, l2)


@pytest.mark.parametrize("mutation", ["shift_backwards", "no_shift", "scale_on_loss", "init_dropped"])
def test_sequence_pin_catches_planted_mistakes(monkeypatch, mutation):
    """A plausible mistake in the sequence form must fail the training-loop comparison."""
    rng = np.random.default_rng(32)
    X3, W, Y2 = _seq_case(rng, 2, 7, 8, 11, ignore=1)
    dX0, dW0 = rng.standard_normal(X3.shape), rng.standard_normal(W.shape)
    real = O.flce_forward_backward

    def wrong_rows(X, W_, y, *a, **k):
        # the oracle flattens positions 0..T-2 with labels 1..T-1; re-pair them wrongly
        y = np.asarray(y).reshape(2, 6)
        if mutation == "shift_backwards":
            y = np.concatenate([Y2[:, :1], Y2[:, :5]], axis=1)
        elif mutation == "no_shift":
            y = Y2[:, :6]
        return real(X, W_, y.reshape(-1), *a, **k)

    scale = 0.5
    if mutation in ("shift_backwards", "no_shift"):
        monkeypatch.setattr(O, "flce_forward_backward", wrong_rows)
        got = O.flce_sequences(X3, W, Y2, 1, IGN, 0.0, "mean", scale, dX0, dW0)
    elif mutation == "scale_on_loss":
        got = list(O.flce_sequences(X3, W, Y2, 1, IGN, 0.0, "mean", 1.0, dX0, dW0))
        got[0] *= scale
    else:
        got = O.flce_sequences(X3, W, Y2, 1, IGN, 0.0, "mean", scale)
    tl, tdX, tdW = _torch_sequences(X3, W, Y2, 1, 0.0, "mean", scale, dX0, dW0)
    ok = abs(got[0] - tl) <= 1e-12 * abs(tl) and _rel(got[1], tdX) < 1e-12 and _rel(got[2], tdW) < 1e-12
    assert not ok


# ---------------------------------------------------------------- the blocked full-size oracle
@pytest.mark.parametrize("softcap", [0.0, 4.0])
@pytest.mark.parametrize("reduction", ["mean", "sum"])
@pytest.mark.parametrize("block_rows", [1, 5, 16, 37, 64])
def test_blocked_matches_torch(softcap, reduction, block_rows):
    """flce_blocked (row blocks, N over the whole call, dW summed over blocks) against the independent
    PyTorch float64 implementation, with block sizes that leave a ragged last block (37 rows)."""
    rng = np.random.default_rng(70 + block_rows)
    X, W, y = _rand_case(rng, 37, 12, 23, ignore=5, w_scale=3.0)
    tl, tdx, tdw = _torch_reference(X, W, y, softcap, reduction)
    loss, dX, dW, d = oracle.flce_blocked(X, W, y, IGN, softcap, reduction, block_rows=block_rows)
    assert abs(loss - tl) <= 1e-12 * abs(tl)
    assert np.allclose(dX, tdx, rtol=0, atol=1e-13)
    assert np.allclose(dW, tdw, rtol=0, atol=1e-13)
    assert d["N"] == 32 and np.all(d["loss_rows"][y == IGN] == 0.0)
    # per-row lse against torch's logsumexp of the (softcapped) logits
    z = torch.tensor(X) @ torch.tensor(W).T
    if softcap > 0:
        z = softcap * torch.tanh(z / softcap)
    assert np.allclose(d["lse"], torch.logsumexp(z, 1).numpy(), rtol=0, atol=1e-12)


def test_blocked_no_valid_rows_and_block_larger_than_call():
    rng = np.random.default_rng(5)
    X, W, y = _rand_case(rng, 9, 8, 7)
    y[:] = IGN
    loss, dX, dW, d = oracle.flce_blocked(X, W, y, IGN, block_rows=4)
    assert loss == 0.0 and not dX.any() and not dW.any() and d["N"] == 0
    X, W, y = _rand_case(rng, 9, 8, 7, ignore=2)
    tl, tdx, tdw = _torch_reference(X, W, y, 0.0, "mean")
    loss, dX, dW, _ = oracle.flce_blocked(X, W, y, IGN, block_rows=1000)
    assert abs(loss - tl) <= 1e-12 * tl and np.allclose(dX, tdx, atol=1e-13) and np.allclose(dW, tdw, atol=1e-13)


@pytest.mark.parametrize("mutation", ["drop_tail", "overlap", "per_block_N", "skip_first"])
def test_blocked_pin_catches_planted_mistakes(monkeypatch, mutation):
    """Mistakes at the block boundaries or in the cross-block divisor, planted in the oracle, must make
    the pin against torch fail."""
    if mutation == "drop_tail":      # the last, shorter block is never visited
        monkeypatch.setattr(O, "_row_blocks", lambda n, b: [(i, i + b) for i in range(0, n - n % b, b)])
    elif mutation == "overlap":      # blocks share a row: its dW contribution counts twice
        monkeypatch.setattr(O, "_row_blocks", lambda n, b: [(i, min(i + b + 1, n)) for i in range(0, n, b)])
    elif mutation == "skip_first":   # off by one at the start of every block
        monkeypatch.setattr(O, "_row_blocks", lambda n, b: [(i + 1, min(i + b, n)) for i in range(0, n, b)])
    else:                            # the mean's divisor counted per block instead of per call
        orig = O._row_terms
        monkeypatch.setattr(O, "_row_terms", lambda X, W, y, ig, c, r, n: orig(X, W, y, ig, c, r, None))
    rng = np.random.default_rng(71)
    X, W, y = _rand_case(rng, 37, 12, 23, ignore=5, w_scale=3.0)
    tl, tdx, tdw = _torch_reference(X, W, y, 0.0, "mean")
    loss, dX, dW, _ = oracle.flce_blocked(X, W, y, IGN, 0.0, "mean", block_rows=8)
    ok = abs(loss - tl) <= 1e-12 * abs(tl) and np.allclose(dX, tdx, atol=1e-13) and np.allclose(dW, tdw, atol=1e-13)
    assert not ok
