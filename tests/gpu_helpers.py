"""Shared helpers for the GPU parity tests: run the HIP path and the oracle on the same inputs."""
import numpy as np
import torch

import oracle
from linear_cross_entropy_07_amd import build_lib

# Tolerances of the target: loss relative error and gradient relative Frobenius error.
TOL = {"bf16": dict(loss=1e-3, grad=2e-2), "fp32": dict(loss=1e-5, grad=1e-4)}


def device():
    import pytest

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    build_lib.ensure_built()
    return torch.device("cuda", 0)


def announce(*a):
    print("[case]", *a, flush=True)


def rel_fro(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    if nb == 0.0:
        return 0.0 if not np.any(a) else float("inf")
    return float(np.linalg.norm(a - b) / nb)


def run_gpu(eng, X, W, y, ignore_index=-100, softcap=0.0, reduction="mean"):
    dev = eng.device
    loss, gh, gw = eng.forward_backward(X.to(dev), W.to(dev), y.to(dev), ignore_index, softcap, reduction)
    torch.cuda.synchronize(dev)
    return float(loss.cpu()), gh.double().cpu().numpy(), gw.double().cpu().numpy()


def check_against_oracle(gpu, X, W, y, dtype, ignore_index=-100, softcap=0.0, reduction="mean"):
    ol, odx, odw = oracle.flce_forward_backward(X, W, y, ignore_index, softcap, reduction)
    gl, gdx, gdw = gpu
    tol = TOL[dtype]
    err_l = abs(gl - ol) / max(abs(ol), 1e-30) if ol != 0.0 else abs(gl)
    err_dx, err_dw = rel_fro(gdx, odx), rel_fro(gdw, odw)
    print(f"   loss gpu {gl:.7f} oracle {ol:.7f} rel {err_l:.2e}; dX {err_dx:.2e}; dW {err_dw:.2e}",
          flush=True)
    if ol == 0.0:
        assert gl == 0.0
    else:
        assert err_l <= tol["loss"], (gl, ol)
    assert err_dx <= tol["grad"], err_dx
    assert err_dw <= tol["grad"], err_dw
    return ol, odx, odw
