"""GPU parity on seeded random small shapes: B*T, H (any multiple of 8) and V with tails in every
tile dimension, both dtypes, softcap on and off, both reductions, several chunk sizes and ignore
fractions, through the fused call and the forward-only call, each checked against the CPU float64
oracle."""
import numpy as np
import pytest

import oracle
from gpu_helpers import TOL, announce, check_against_oracle, device, run_gpu
from linear_cross_entropy_07_amd import flce, inputs

pytestmark = pytest.mark.gpu

_ENG = {}


def eng(chunk):
    dev = device()
    if chunk not in _ENG:
        _ENG[chunk] = flce.FLCE(dev, chunk_rows_max=chunk)
    return _ENG[chunk]


def _cases(n=16, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = "fp32" if i % 4 == 3 else "bf16"
        out.append(dict(
            BT=int(rng.integers(1, 700)), H=int(8 * rng.integers(1, 41)), V=int(rng.integers(2, 3200)),
            dtype=dtype, softcap=float(rng.choice([0.0, 0.0, 5.0, 30.0])),
            reduction=str(rng.choice(["mean", "sum"])), chunk=int(rng.choice([0, 256, 512])),
            ignore=float(rng.choice([0.0, 0.1, 0.5])), seed=int(rng.integers(0, 1 << 30))))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"{c['dtype']}-{c['BT']}x{c['H']}x{c['V']}")
def test_random_shape(case):
    c = case
    w = inputs.custom(BT=c["BT"], H=c["H"], V=c["V"], dtype=c["dtype"], softcap=c["softcap"],
                      ignore_frac=c["ignore"], w_std=0.05 if c["dtype"] == "bf16" else 0.0, name="random")
    announce("random shape", c)
    X, W, y = inputs.make_inputs(w, seed=c["seed"])
    e = eng(c["chunk"])
    got = run_gpu(e, X, W, y, softcap=c["softcap"], reduction=c["reduction"])
    check_against_oracle(got, X, W, y, c["dtype"], softcap=c["softcap"], reduction=c["reduction"])
    # the forward-only call on the same inputs: per-row terms and lse against the oracle
    dev = e.device
    rows, lse = e.forward(X.to(dev), W.to(dev), y.to(dev), softcap=c["softcap"], reduction="none",
                          return_lse=True)
    o_rows, o_lse = oracle.flce_forward(X, W, y, -100, c["softcap"], "none")
    tol = TOL[c["dtype"]]["loss"]
    for g, r in ((rows, o_rows), (lse, o_lse)):
        g = g.double().cpu().numpy()
        assert np.all(np.abs(g - r) <= tol * np.maximum(np.abs(r), 1.0))
