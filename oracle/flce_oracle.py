"""Plain CPU float64 oracle for fused linear + cross-entropy (FLCE), forward and backward.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this module; it is
used by the tests, by the smoke check and by the benchmark's CPU-baseline leg.

What is computed follows the PR description on the page "[AOTAutograd] tweak
min-cut partitioner to avoid saving softmax output" (PyTorch PR #126348): the
linear layer produces the softmax input (the logits), a per-row maximum and a
per-row sum of exponentials are formed from it in two separate passes, the
negative log-likelihood needs only the label's entry of each row, and the
backward pass needs the whole softmax, which is a function of the logits and the
small per-row max/sum tensors. The weight has the `nn.Linear(H, V, bias=False)`
layout shown in that PR's test (W is [V, H], no bias). The optional logit
softcap is the Gemma2 one mentioned in the comments of "Torch compiled FLCE is
2x faster than the current FLCE" (Liger-Kernel issue #227); the pages name it
without a formula, and this oracle takes s = c * tanh(z / c), with c = 0 meaning
"off".

Everything is done the plain way, on fully materialised float64 logits:

    z   = X W^T                       (one BLAS call; the definition of the linear layer)
    s   = c tanh(z / c)  or  z
    m   = max_v s                      (first pass over the row)
    lse = m + ln sum_v exp(s - m)      (second pass over the row)
    l_t = lse_t - s_{t, y_t}           for rows whose label is not ignore_index
    loss = sum_t l_t / N  (mean over the N valid rows)   or   sum_t l_t (sum)

    backward with d loss = 1:
    g_t   = 1/N (mean) or 1 (sum) on valid rows, 0 on ignored rows
    ds_tv = g_t (exp(s_tv - lse_t) - [v == y_t])
    dz_tv = ds_tv (1 - (s_tv / c)^2)   when the softcap is on (d/dz c tanh(z/c) = 1 - tanh^2)
    dX = dZ W,   dW = dZ^T X           (two BLAS calls)

Readings taken where the pages are silent (the same list is kept with the design notes):
  * mean is over the valid rows of the whole call; with N = 0 the loss and all
    gradients are 0 (PyTorch would give NaN);
  * a label outside [0, V) that is not ignore_index is an error here;
  * no intermediate is rounded to bf16: the inputs' exact values are widened to
    float64 and every step stays in float64.

There is no online softmax, chunking or fusion here: rows are independent, and
each row's whole logits vector is built. Most functions build the [BT, V] logits
matrix of the rows asked for at once; flce_vocab_rows and flce_blocked, which
must cover every row of a full-size call, build it in blocks of rows.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "logits",
    "apply_softcap",
    "row_logsumexp",
    "valid_mask",
    "flce_forward_backward",
    "flce_rows",
    "flce_vocab_rows",
    "flce_blocked",
    "flce_sequences",
]


def _f64(a) -> np.ndarray:
    """Widen an array (numpy, or a CPU torch tensor of any float dtype) to float64."""
    if hasattr(a, "detach"):  # a torch tensor: bf16 has no numpy dtype, so widen in torch first
        import torch

        return a.detach().to(device="cpu", dtype=torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def _labels(y) -> np.ndarray:
    if hasattr(y, "detach"):
        y = y.detach().cpu().numpy()
    return np.asarray(y, dtype=np.int64).reshape(-1)


def logits(X: np.ndarray, W: np.ndarray) -> np.ndarray:
    """Step 1 of the PR description: the linear layer, z = X W^T, W in nn.Linear's [V, H] layout."""
    return X @ W.T


def apply_softcap(Z: np.ndarray, softcap: float) -> np.ndarray:
    """Gemma2 logit softcap c tanh(z / c) (named in Liger-Kernel issue #227; formula is this oracle's reading)."""
    if softcap > 0.0:
        return softcap * np.tanh(Z / softcap)
    return Z


def row_logsumexp(S: np.ndarray):
    """Steps 2 and 3 of the PR description: one pass for the row max, a second for the row sum.

    Returns (m, lse) with lse = m + ln sum_v exp(s_v - m).
    """
    m = S.max(axis=1)
    total = np.exp(S - m[:, None]).sum(axis=1)
    return m, m + np.log(total)


def valid_mask(y: np.ndarray, V: int, ignore_index: int) -> np.ndarray:
    """Rows that take part in the loss: label != ignore_index. Any other label must lie in [0, V)."""
    valid = y != ignore_index
    bad = valid & ((y < 0) | (y >= V))
    if bad.any():
        raise ValueError(f"label out of range [0, {V}) at rows {np.nonzero(bad)[0][:8].tolist()}")
    return valid


def _check(X, W, y, softcap, reduction):
    if X.ndim != 2 or W.ndim != 2 or X.shape[1] != W.shape[1]:
        raise ValueError(f"bad shapes X{X.shape} W{W.shape}")
    if y.shape[0] != X.shape[0]:
        raise ValueError("labels must have one entry per row of X")
    if not (softcap >= 0.0):  # also rejects NaN
        raise ValueError("softcap must be >= 0 (0 = off)")
    if reduction not in ("mean", "sum"):
        raise ValueError("reduction must be 'mean' or 'sum'")


def _row_terms(X, W, y, ignore_index, softcap, reduction, n_valid):
    """Per-row forward quantities and dZ for the rows of X (all of them materialised)."""
    V = W.shape[0]
    valid = valid_mask(y, V, ignore_index)
    N = int(valid.sum()) if n_valid is None else int(n_valid)
    Z = logits(X, W)
    S = apply_softcap(Z, softcap)
    m, lse = row_logsumexp(S)
    rows = np.arange(X.shape[0])
    y_safe = np.where(valid, y, 0)
    s_label = S[rows, y_safe]
    loss_rows = np.where(valid, lse - s_label, 0.0)

    if reduction == "mean":
        g = np.where(valid, 1.0 / N, 0.0) if N > 0 else np.zeros(X.shape[0])
    else:
        g = np.where(valid, 1.0, 0.0)
    P = np.exp(S - lse[:, None])  # the softmax, rebuilt from the logits and lse
    dS = P
    dS[rows[valid], y_safe[valid]] -= 1.0
    dS *= g[:, None]
    if softcap > 0.0:
        dZ = dS * (1.0 - (S / softcap) ** 2)
    else:
        dZ = dS
    return dict(valid=valid, N=N, m=m, lse=lse, s_label=s_label, loss_rows=loss_rows, g=g, dZ=dZ)


def flce_forward_backward(X, W, y, ignore_index: int = -100, softcap: float = 0.0,
                          reduction: str = "mean", return_details: bool = False):
    """Loss, dL/dX and dL/dW of mean/sum NLL over softmax(softcap(X W^T)), with dL/dloss = 1.

    X: [BT, H], W: [V, H], y: [BT] integer labels. Inputs of any float dtype are
    widened exactly to float64. Returns (loss: float, dX: [BT, H] f64, dW: [V, H] f64)
    and, with return_details, a dict of per-row quantities (lse, loss_rows, dZ, ...).
    """
    X = _f64(X)
    W = _f64(W)
    y = _labels(y)
    _check(X, W, y, softcap, reduction)
    t = _row_terms(X, W, y, ignore_index, softcap, reduction, None)
    total = float(t["loss_rows"].sum())
    if reduction == "mean":
        loss = total / t["N"] if t["N"] > 0 else 0.0
    else:
        loss = total
    dX = t["dZ"] @ W
    dW = t["dZ"].T @ X
    if return_details:
        return loss, dX, dW, t
    return loss, dX, dW


def flce_forward(X, W, y, ignore_index: int = -100, softcap: float = 0.0, reduction: str = "mean"):
    """Forward only: the NLL of the PR description without any gradient.

    Steps 1-5 of the module docstring on fully materialised float64 logits. Returns (out, lse):
    out is the loss (a float) for 'mean' and 'sum', or the per-row terms l_t [BT] (lse_t - s_{t,y_t},
    0 on ignored rows) for 'none'; lse [BT] is the row log-sum-exp of every row, ignored rows
    included.
    """
    X = _f64(X)
    W = _f64(W)
    y = _labels(y)
    _check(X, W, y, softcap, "mean" if reduction == "none" else reduction)
    V = W.shape[0]
    valid = valid_mask(y, V, ignore_index)
    S = apply_softcap(logits(X, W), softcap)
    _, lse = row_logsumexp(S)
    y_safe = np.where(valid, y, 0)
    loss_rows = np.where(valid, lse - S[np.arange(X.shape[0]), y_safe], 0.0)
    if reduction == "none":
        return loss_rows, lse
    total = float(loss_rows.sum())
    N = int(valid.sum())
    if reduction == "mean":
        return (total / N if N > 0 else 0.0), lse
    return total, lse


def flce_rows(X, W, y, rows, n_valid: int, ignore_index: int = -100, softcap: float = 0.0,
              reduction: str = "mean"):
    """Per-row results for a subset of the rows of a larger call.

    Rows of the method are independent except for the mean's divisor N, which is
    the number of valid rows of the whole call and is passed in. Returns a dict
    with, for each requested row: lse, loss_row (lse - s_label, 0 if ignored) and
    the dX row. Used to check sampled rows of full-size runs.
    """
    rows = np.asarray(rows, dtype=np.int64)
    Xr = _f64(X[rows] if not hasattr(X, "detach") else X[rows.tolist()])
    Wf = _f64(W)
    yr = _labels(y)[rows]
    _check(Xr, Wf, yr, softcap, reduction)
    t = _row_terms(Xr, Wf, yr, ignore_index, softcap, reduction, n_valid)
    return dict(lse=t["lse"], loss_rows=t["loss_rows"], dX=t["dZ"] @ Wf, valid=t["valid"],
                s_label=t["s_label"])


def flce_vocab_rows(X, W, y, vrows, ignore_index: int = -100, softcap: float = 0.0,
                    reduction: str = "mean", block_rows: int = 1024, threads: int = 0):
    """Selected rows of dL/dW for a call of any size: dW[v, :] = sum_t dz_tv x_t for v in vrows.

    Every dz_tv needs the row's lse over the whole vocabulary, so the full float64 logits row of
    every t is built, in blocks of block_rows rows so that host memory stays bounded (rows are
    independent; within a row nothing is streamed: max, then the sum of exponentials, as in
    row_logsumexp). Blocks run on a thread pool (numpy releases the GIL in BLAS and ufuncs); their
    contributions are summed in block order. Returns dict(dW=[len(vrows), H] f64, lse=[BT], N).
    """
    from concurrent.futures import ThreadPoolExecutor
    import os

    Xf = _f64(X)
    Wf = _f64(W)
    yl = _labels(y)
    _check(Xf, Wf, yl, softcap, reduction)
    vrows = np.asarray(vrows, dtype=np.int64)
    V = Wf.shape[0]
    if vrows.size and (vrows.min() < 0 or vrows.max() >= V):
        raise ValueError("vocabulary rows out of range")
    valid = valid_mask(yl, V, ignore_index)
    N = int(valid.sum())
    if reduction == "mean":
        g = np.where(valid, 1.0 / N, 0.0) if N > 0 else np.zeros(Xf.shape[0])
    else:
        g = np.where(valid, 1.0, 0.0)

    def block(b0):
        b1 = min(b0 + block_rows, Xf.shape[0])
        S = apply_softcap(logits(Xf[b0:b1], Wf), softcap)
        _, lse = row_logsumexp(S)
        Sv = S[:, vrows]
        dS = np.exp(Sv - lse[:, None])
        onehot = (yl[b0:b1, None] == vrows[None, :]) & valid[b0:b1, None]
        dS -= onehot
        dS *= g[b0:b1, None]
        dZ = dS * (1.0 - (Sv / softcap) ** 2) if softcap > 0.0 else dS
        return lse, dZ.T @ Xf[b0:b1]

    starts = list(range(0, Xf.shape[0], block_rows))
    nthr = threads or min(len(starts), len(os.sched_getaffinity(0)), 16) or 1
    with ThreadPoolExecutor(max_workers=nthr) as ex:
        parts = list(ex.map(block, starts))
    dW = np.zeros((vrows.size, Wf.shape[1]))
    for _, d in parts:
        dW += d
    lse = np.concatenate([l for l, _ in parts]) if parts else np.zeros(0)
    return dict(dW=dW, lse=lse, N=N)


def _row_blocks(n: int, block_rows: int):
    """Consecutive row ranges [b0, b1) that cover rows 0 .. n-1 once, block_rows rows each (the last
    one shorter when block_rows does not divide n)."""
    return [(b0, min(b0 + block_rows, n)) for b0 in range(0, n, block_rows)]


def flce_blocked(X, W, y, ignore_index: int = -100, softcap: float = 0.0, reduction: str = "mean",
                 block_rows: int = 1024):
    """flce_forward_backward for a call of any size, with host memory bounded by a block of rows.

    Rows of the method are independent except for the mean's divisor N, so N is counted over the
    whole call first; then each block of block_rows rows goes through exactly the per-row steps of
    flce_forward_backward (its whole float64 logits rows built, the two-pass max and sum, the loss
    terms, dZ) and contributes dX_b = dZ_b W and dZ_b^T X_b, the latter summed into dW in block
    order. The loss is the sum of all rows' terms (in row order) over N, or that sum.
    Returns (loss, dX [BT, H] f64, dW [V, H] f64, dict(lse [BT], loss_rows [BT], N)).
    """
    Xf = _f64(X)
    Wf = _f64(W)
    yl = _labels(y)
    _check(Xf, Wf, yl, softcap, reduction)
    if block_rows <= 0:
        raise ValueError("block_rows must be positive")
    BT, H = Xf.shape
    V = Wf.shape[0]
    N = int(valid_mask(yl, V, ignore_index).sum())
    dX = np.zeros((BT, H))
    dW = np.zeros((V, H))
    lse = np.zeros(BT)
    loss_rows = np.zeros(BT)
    for b0, b1 in _row_blocks(BT, block_rows):
        t = _row_terms(Xf[b0:b1], Wf, yl[b0:b1], ignore_index, softcap, reduction, N)
        dX[b0:b1] = t["dZ"] @ Wf
        dW += t["dZ"].T @ Xf[b0:b1]
        lse[b0:b1] = t["lse"]
        loss_rows[b0:b1] = t["loss_rows"]
    total = float(loss_rows.sum())
    if reduction == "mean":
        loss = total / N if N > 0 else 0.0
    else:
        loss = total
    return loss, dX, dW, dict(lse=lse, loss_rows=loss_rows, N=N)


def flce_sequences(X3, W, Y2, shift: int = 1, ignore_index: int = -100, softcap: float = 0.0,
                   reduction: str = "mean", grad_scale: float = 1.0, dX_init=None, dW_init=None):
    """The same loss over a batch of sequences, with the next-token shift done by indexing.

    X3: [B, T, H], Y2: [B, T]. With shift = 1 the position t < T-1 of sequence b is scored against
    the label at (b, t+1) and the last position is not scored: the shift that the training loop in
    torchtune issue #1228 ("[FEATURE REQUEST] Compile model+loss_fn together") makes by slicing the
    logits and labels; shift = 0 scores every position against its own label. The gradients are
    multiplied by grad_scale (the upstream gradient of the loss, e.g. the loss / accumulation-steps
    division of that loop) and added to dX_init / dW_init when given. The last positions get no
    gradient of their own (0 + dX_init there).

    Returns (loss, dX3 [B, T, H] f64, dW [V, H] f64, loss_rows [B * (T - shift)], lse [B * (T - shift)]),
    rows numbered b * (T - shift) + t.
    """
    X3 = _f64(X3)
    W = _f64(W)
    if hasattr(Y2, "detach"):
        Y2 = Y2.detach().cpu().numpy()
    Y2 = np.asarray(Y2, dtype=np.int64)
    if X3.ndim != 3 or Y2.shape != X3.shape[:2] or shift not in (0, 1):
        raise ValueError(f"bad shapes X{X3.shape} Y{Y2.shape} or shift {shift}")
    B, T, H = X3.shape
    P = max(T - shift, 0)
    X = X3[:, :P, :].reshape(B * P, H)
    y = Y2[:, shift:shift + P].reshape(B * P)
    loss, dX, dW, t = flce_forward_backward(X, W, y, ignore_index, softcap, reduction, return_details=True)
    dX3 = np.zeros((B, T, H)) if dX_init is None else _f64(dX_init).copy()
    dX3[:, :P, :] += grad_scale * dX.reshape(B, P, H)
    dW_out = grad_scale * dW if dW_init is None else _f64(dW_init) + grad_scale * dW
    return loss, dX3, dW_out, t["loss_rows"], t["lse"]
