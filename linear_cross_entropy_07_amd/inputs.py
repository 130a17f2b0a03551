"""Seeded synthetic inputs for fused linear + cross-entropy workloads.

This module only draws random numbers; it holds none of the method's arithmetic,
so both the oracle-side tests and the HIP-side benchmark may use it. Every
workload is drawn with `numpy.random.default_rng(seed)` (PCG64) in the order
hidden, W, labels, ignore mask; values are drawn in float32 and then rounded to
the workload's dtype (bf16 with round-to-nearest-even through torch).

The shapes stand in for the workloads the pages discuss (no dataset or trained
weight is used):
  * gpt2_head: the llm.c GPT-2-small LM head (C = 768, V = 50257, B = 32, T = 1024)
    from the PR description of "[AOTAutograd] tweak min-cut partitioner to avoid
    saving softmax output";
  * llama3_8b_head / ragged: H = 4096, V = 128256 and the ragged B*T protocol from
    the benchmark comment in "Torch compiled FLCE is 2x faster than the current FLCE";
  * gemma2_head: a softcapped Gemma2-style head (softcap mentioned in the same thread);
  * llama3_8b_head_vshard8: one GPU's share of the Llama head split by vocabulary over 8 GPUs
    (V = 128256 / 8 = 16032 rows of W), at its real shape.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

IGNORE_INDEX = -100


@dataclass(frozen=True)
class Workload:
    name: str
    BT: int
    H: int
    V: int
    dtype: str            # "bf16" or "fp32"
    softcap: float        # 0 = off
    ignore_frac: float    # exact count round(frac * BT) of rows set to ignore_index
    labels: str           # "uniform" or "zipf1.1"
    x_rmsnorm: bool       # hidden ~ N(0,1) then x / sqrt(mean(x^2)) per row (fp32, no eps)
    w_std: float          # W ~ N(0, w_std^2); 0 means 1/sqrt(H)
    reduction: str = "mean"


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 256, 64, 1000, "fp32", 0.0, 0.10, "uniform", False, 0.0),
    "gpt2_head": Workload("gpt2_head", 32768, 768, 50257, "bf16", 0.0, 0.0, "uniform", False, 0.02),
    "llama3_8b_head": Workload("llama3_8b_head", 8192, 4096, 128256, "bf16", 0.0, 0.05, "zipf1.1", True, 0.02),
    "gemma2_head": Workload("gemma2_head", 8192, 3584, 256000, "bf16", 30.0, 0.05, "uniform", False, 0.02),
    "ragged": Workload("ragged", 0, 4096, 128256, "bf16", 0.0, 0.05, "uniform", False, 0.02),
    "llama3_8b_head_vshard8": Workload("llama3_8b_head_vshard8", 8192, 4096, 16032, "bf16", 0.0, 0.05, "zipf1.1",
                                       True, 0.02),
}


def _to_dtype(a: np.ndarray, dtype: str):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "fp32":
        return t
    raise ValueError(dtype)


def _draw_hidden(rng, BT, H, rmsnorm):
    x = rng.standard_normal((BT, H), dtype=np.float32)
    if rmsnorm:
        x = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True, dtype=np.float32))
    return x


def _draw_weight(rng, V, H, w_std):
    std = np.float32(w_std if w_std > 0 else 1.0 / np.sqrt(H))
    w = rng.standard_normal((V, H), dtype=np.float32)
    w *= std
    return w


def _draw_labels(rng, BT, V, kind, ignore_frac):
    if kind == "uniform":
        y = rng.integers(0, V, size=BT, dtype=np.int64)
    elif kind == "zipf1.1":
        p = np.arange(1, V + 1, dtype=np.float64) ** -1.1
        p /= p.sum()
        y = rng.choice(V, size=BT, p=p).astype(np.int64)
    else:
        raise ValueError(kind)
    n_ign = int(round(ignore_frac * BT))
    if n_ign:
        y[rng.permutation(BT)[:n_ign]] = IGNORE_INDEX
    return y


def make_inputs(w: Workload, seed: int = 0, BT: int | None = None):
    """Draw (hidden [BT,H], W [V,H], labels [BT] int64) as CPU torch tensors for workload w."""
    import torch

    BT = w.BT if BT is None else BT
    rng = np.random.default_rng(seed)
    x = _draw_hidden(rng, BT, w.H, w.x_rmsnorm)
    W = _draw_weight(rng, w.V, w.H, w.w_std)
    y = _draw_labels(rng, BT, w.V, w.labels, w.ignore_frac)
    return _to_dtype(x, w.dtype), _to_dtype(W, w.dtype), torch.from_numpy(y)


def custom(BT, H, V, dtype="bf16", softcap=0.0, ignore_frac=0.0, labels="uniform",
           x_rmsnorm=False, w_std=0.0, name="custom", reduction="mean") -> Workload:
    return Workload(name, BT, H, V, dtype, softcap, ignore_frac, labels, x_rmsnorm, w_std, reduction)


def ragged_bt_list(seed: int = 0, draws: int = 20):
    """B*T values of the ragged sweep: 4096, then 4096 + U[0, 28672] + U[0, 1000] per draw, then 32768."""
    rng = np.random.default_rng(seed)
    mid = [int(4096 + rng.integers(0, 28673) + rng.integers(0, 1001)) for _ in range(draws)]
    return [4096] + mid + [32768]


def make_ragged_call(BT: int, seed: int, W_seed: int = 0):
    """One call of the ragged sweep: W fixed by W_seed, fresh hidden/labels from seed."""
    w = WORKLOADS["ragged"]
    rng_w = np.random.default_rng(W_seed)
    W = _draw_weight(rng_w, w.V, w.H, w.w_std)
    rng = np.random.default_rng(seed)
    x = _draw_hidden(rng, BT, w.H, False)
    y = _draw_labels(rng, BT, w.V, "uniform", w.ignore_frac)
    import torch

    return _to_dtype(x, "bf16"), _to_dtype(W, "bf16"), torch.from_numpy(y)


def with_bt(w: Workload, BT: int) -> Workload:
    return replace(w, BT=BT)


def far_label_case(BT: int, H: int, V: int, dtype: str = "bf16", far: float = 60.0, near: float = 40.0,
                   every: int = 5, ignore_frac: float = 0.05, seed: int = 0):
    """Inputs where some rows' label logit lies far below the row's largest logit.

    Two vocabulary rows a = 7 and b = V - 3 hold +alpha u and -alpha u for a random unit vector u. Hidden
    rows 0, every, 2 every, ... are beta u plus small noise, with label b: their logit at a exceeds
    their label logit by 2 alpha beta, which is `far` for every other planted row and `near` for the
    rest. Other rows and weights are the usual Gaussian draws (W ~ N(0, 0.05^2)); round(ignore_frac *
    BT) rows that are not planted are set to ignore_index."""
    import torch

    rng = np.random.default_rng(seed)
    x = rng.standard_normal((BT, H), dtype=np.float32)
    W = (rng.standard_normal((V, H), dtype=np.float32) * np.float32(0.05)).astype(np.float32)
    y = rng.integers(0, V, size=BT, dtype=np.int64)
    u = rng.standard_normal(H).astype(np.float64)
    u /= np.linalg.norm(u)
    a, b, alpha = 7, V - 3, 4.0
    W[a] = (alpha * u).astype(np.float32)
    W[b] = (-alpha * u).astype(np.float32)
    planted = np.arange(0, BT, every)
    for k, r in enumerate(planted):
        beta = (far if k % 2 == 0 else near) / (2.0 * alpha)
        x[r] = (beta * u + 0.01 * rng.standard_normal(H)).astype(np.float32)
        y[r] = b
    others = np.setdiff1d(np.arange(BT), planted)
    n_ign = min(int(round(ignore_frac * BT)), others.size)
    if n_ign:
        y[rng.permutation(others)[:n_ign]] = IGNORE_INDEX
    return _to_dtype(x, dtype), _to_dtype(W, dtype), torch.from_numpy(y)
