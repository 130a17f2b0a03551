"""The C ABI from plain C: examples/flce_from_c (C99, HIP runtime C API for device memory, no
PyTorch in the process) calls flce_forward_backward, flce_forward, flce_forward_backward_recompute
and flce_forward_backward_rows through include/flce.h; its outputs are checked against the CPU
float64 oracle."""
import os
import struct
import subprocess
import tempfile

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import TOL, announce, device, rel_fro
from linear_cross_entropy_07_amd import build_lib, inputs

pytestmark = pytest.mark.gpu


def _bits(t: torch.Tensor) -> bytes:
    return t.contiguous().view(torch.int16).numpy().tobytes()


@pytest.mark.parametrize("softcap,reduction", [(0.0, 1), (30.0, 2)])
def test_c_caller_matches_oracle(softcap, reduction):
    device()  # skips without a GPU; the C program itself runs in a child process
    if not os.path.exists(build_lib.EXAMPLE_BIN):
        pytest.fail(f"{build_lib.EXAMPLE_BIN} is not built; run __graft_entry__.build()")
    BT, H, V, B, scale = 300, 128, 1000, 3, 0.5
    w = inputs.custom(BT=BT, H=H, V=V, dtype="bf16", ignore_frac=0.1, w_std=0.05, name="c_abi")
    X, W, y = inputs.make_inputs(w, seed=21)
    announce("C caller", BT, H, V, "softcap", softcap, "reduction", reduction)
    with tempfile.TemporaryDirectory() as d:
        fin, fout = os.path.join(d, "in.bin"), os.path.join(d, "out.bin")
        with open(fin, "wb") as f:
            f.write(struct.pack("<qqqfiqf", BT, H, V, softcap, reduction, B, scale))
            f.write(_bits(X))
            f.write(_bits(W))
            f.write(y.numpy().astype("<i8").tobytes())
        res = subprocess.run([build_lib.EXAMPLE_BIN, fin, fout], capture_output=True, text=True, timeout=120)
        print(res.stdout, res.stderr, flush=True)
        assert res.returncode == 0
        raw = open(fout, "rb").read()
    off = 0

    def take(n, dt):
        nonlocal off
        a = np.frombuffer(raw, dtype=dt, count=n, offset=off)
        off += a.nbytes
        return a

    def grads():
        loss = float(take(1, "<f4")[0])
        gh = torch.from_numpy(take(BT * H, "<i2").copy()).view(torch.bfloat16).double().numpy().reshape(BT, H)
        gw = take(V * H, "<f4").astype(np.float64).reshape(V, H)
        return loss, gh, gw

    fused = grads()
    rows = take(BT, "<f4").astype(np.float64)
    lse = take(BT, "<f4").astype(np.float64)
    recompute = grads()
    seqs = grads()
    st = take(4, "<i4")
    assert off == len(raw)
    red = "mean" if reduction == 1 else "sum"
    ol, odx, odw = oracle.flce_forward_backward(X, W, y, -100, softcap, red)
    o_rows, o_lse = oracle.flce_forward(X, W, y, -100, softcap, "none")
    T = BT // B
    sl, sdx3, sdw, _, _ = oracle.flce_sequences(X.reshape(B, T, H), W, y.reshape(B, T), 1, -100, softcap, red,
                                                grad_scale=scale)
    tol = TOL["bf16"]
    for (loss, gh, gw), (rl, rdx, rdw) in ((fused, (ol, odx, odw)), (recompute, (ol, odx, odw)),
                                           (seqs, (sl, sdx3.reshape(BT, H), sdw))):
        assert abs(loss - rl) <= tol["loss"] * abs(rl)
        assert rel_fro(gh, rdx) <= tol["grad"] and rel_fro(gw, rdw) <= tol["grad"]
    # the last position of each sequence is no row of the sequence call: its gradient row is zero
    assert not np.any(seqs[1].reshape(B, T, H)[:, -1, :])
    for got, ref in ((rows, o_rows), (lse, o_lse)):
        assert np.all(np.abs(got - ref) <= tol["loss"] * np.maximum(np.abs(ref), 1.0))
    assert list(st) == [0, 0, 0, 0]
