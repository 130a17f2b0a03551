"""Python binding of libflce.so (ctypes): argument marshalling only.

Every step of the computation runs in the library's HIP kernels; this module checks tensor
properties, allocates outputs and the workspace with torch (device memory is torch's), passes raw
pointers and the current HIP stream, and turns return codes into exceptions. There is no fallback:
without the built library, or without a GPU, calls raise.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading

import torch

from . import build_lib

FLCE_BF16, FLCE_FP32 = 0, 1
FLCE_NONE, FLCE_MEAN, FLCE_SUM = 0, 1, 2
_REDUCTIONS = {"mean": FLCE_MEAN, "sum": FLCE_SUM}
_FWD_REDUCTIONS = {"none": FLCE_NONE, "mean": FLCE_MEAN, "sum": FLCE_SUM}
_DTYPES = {torch.bfloat16: FLCE_BF16, torch.float32: FLCE_FP32}

ERRORS = {0: "FLCE_OK", -1: "FLCE_ERR_INVALID_ARG", -2: "FLCE_ERR_UNSUPPORTED",
          -3: "FLCE_ERR_WORKSPACE_TOO_SMALL", -4: "FLCE_ERR_HIP", -5: "FLCE_ERR_LABEL_RANGE"}


class FlceError(RuntimeError):
    def __init__(self, code: int, what: str = ""):
        self.code = code
        msg = ERRORS.get(code, str(code))
        if _LIB is not None:
            msg += ": " + _LIB.flce_error_string(code).decode()
        super().__init__(f"{what}: {msg}" if what else msg)


class _Config(ctypes.Structure):
    _fields_ = [("chunk_rows_max", ctypes.c_int64), ("reserved", ctypes.c_int64 * 3)]


_LIB = None
_LOCK = threading.Lock()


def header_functions() -> list[str]:
    """Names of the functions declared in include/flce.h."""
    text = open(os.path.join(build_lib.INCLUDE, "flce.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(flce_\w+)\s*\(", text, re.M)))


def lib() -> ctypes.CDLL:
    """Load libflce.so (built in-tree); raises if it has not been built."""
    global _LIB
    with _LOCK:
        if _LIB is None:
            if not os.path.exists(build_lib.LIB):
                raise FileNotFoundError(f"{build_lib.LIB} is not built; run __graft_entry__.build()")
            L = ctypes.CDLL(build_lib.LIB)
            vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
            L.flce_create.argtypes = [ctypes.POINTER(vp), i32, ctypes.POINTER(_Config)]
            L.flce_destroy.argtypes = [vp]
            L.flce_workspace_size.argtypes = [vp, i64, i64, i64, i32, ctypes.POINTER(ctypes.c_size_t)]
            L.flce_chunk_plan.argtypes = [vp, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]
            L.flce_forward_backward.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i64, ctypes.c_float,
                                                i32, vp, vp, vp, vp, ctypes.c_size_t, vp]
            L.flce_forward_workspace_size.argtypes = [vp, i64, i64, i64, i32, ctypes.POINTER(ctypes.c_size_t)]
            L.flce_forward.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i64, ctypes.c_float, i32,
                                       vp, vp, vp, vp, ctypes.c_size_t, vp]
            L.flce_status.argtypes = [vp, vp]
            L.flce_profile_begin.argtypes = [vp, i32]
            L.flce_profile_end.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]
            L.flce_error_string.argtypes = [i32]
            L.flce_error_string.restype = ctypes.c_char_p
            for f in ("flce_create", "flce_destroy", "flce_workspace_size", "flce_chunk_plan",
                      "flce_forward_backward", "flce_forward_workspace_size", "flce_forward", "flce_status",
                      "flce_profile_begin", "flce_profile_end"):
                getattr(L, f).restype = i32
            _LIB = L
    return _LIB


def _check(rc: int, what: str):
    if rc != 0:
        raise FlceError(rc, what)


def workspace_size(BT: int, H: int, V: int, dtype=torch.bfloat16, handle=None) -> int:
    out = ctypes.c_size_t()
    _check(lib().flce_workspace_size(handle, BT, H, V, _DTYPES[dtype], ctypes.byref(out)),
           "flce_workspace_size")
    return out.value


def forward_workspace_size(BT: int, H: int, V: int, dtype=torch.bfloat16, handle=None) -> int:
    out = ctypes.c_size_t()
    _check(lib().flce_forward_workspace_size(handle, BT, H, V, _DTYPES[dtype], ctypes.byref(out)),
           "flce_forward_workspace_size")
    return out.value


def chunk_plan(BT: int, handle=None):
    n, c = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().flce_chunk_plan(handle, BT, ctypes.byref(n), ctypes.byref(c)), "flce_chunk_plan")
    return n.value, c.value


class FLCE:
    """A library handle bound to one device."""

    def __init__(self, device=None, chunk_rows_max: int = 0):
        if device is None:
            device = torch.device("cuda", torch.cuda.current_device())
        device = torch.device(device)
        if device.type != "cuda":
            raise ValueError("FLCE runs on a HIP device")
        self.device = device if device.index is not None else torch.device("cuda", torch.cuda.current_device())
        cfg = _Config(chunk_rows_max, (ctypes.c_int64 * 3)(0, 0, 0))
        h = ctypes.c_void_p()
        _check(lib().flce_create(ctypes.byref(h), self.device.index, ctypes.byref(cfg)), "flce_create")
        self._h = h
        self._ws = None

    @property
    def handle(self):
        return self._h

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().flce_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace_size(self, BT, H, V, dtype=torch.bfloat16) -> int:
        return workspace_size(BT, H, V, dtype, self._h)

    def chunk_plan(self, BT):
        return chunk_plan(BT, self._h)

    def workspace(self, nbytes: int) -> torch.Tensor:
        """A cached uint8 device buffer of at least nbytes (grown when too small)."""
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = None
            self._ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        return self._ws

    def _check_inputs(self, hidden: torch.Tensor, W: torch.Tensor, labels: torch.Tensor):
        if hidden.dim() != 2 or W.dim() != 2 or labels.dim() != 1:
            raise ValueError("hidden [BT,H], W [V,H], labels [BT] expected")
        BT, H = hidden.shape
        V = W.shape[0]
        if W.shape[1] != H or labels.shape[0] != BT:
            raise ValueError(f"shape mismatch: hidden {tuple(hidden.shape)}, W {tuple(W.shape)}, "
                             f"labels {tuple(labels.shape)}")
        if hidden.dtype != W.dtype or hidden.dtype not in _DTYPES:
            raise TypeError("hidden and W must both be bfloat16 or both float32")
        if labels.dtype != torch.int64:
            raise TypeError("labels must be int64")
        for name, t in (("hidden", hidden), ("W", W), ("labels", labels)):
            if t.device != self.device:
                raise ValueError(f"{name} is on {t.device}, handle is on {self.device}")
            if not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")
        return BT, H, V

    def forward_backward(self, hidden: torch.Tensor, W: torch.Tensor, labels: torch.Tensor,
                         ignore_index: int = -100, softcap: float = 0.0, reduction: str = "mean",
                         out=None, workspace: torch.Tensor | None = None, stream=None):
        """Run the fused forward + backward; returns (loss [0-dim fp32], grad_hidden, grad_W fp32)."""
        BT, H, V = self._check_inputs(hidden, W, labels)
        if reduction not in _REDUCTIONS:
            raise ValueError("reduction must be 'mean' or 'sum'")
        dt = _DTYPES[hidden.dtype]
        need = self.workspace_size(BT, H, V, hidden.dtype)
        if workspace is None:
            workspace = self.workspace(need)
        if out is None:
            loss = torch.empty((), dtype=torch.float32, device=self.device)
            gh = torch.empty_like(hidden)
            gw = torch.empty((V, H), dtype=torch.float32, device=self.device)
        else:
            loss, gh, gw = out
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        rc = lib().flce_forward_backward(
            self._h, hidden.data_ptr(), W.data_ptr(), labels.data_ptr(), BT, H, V, dt,
            int(ignore_index), float(softcap), _REDUCTIONS[reduction], loss.data_ptr(),
            gh.data_ptr(), gw.data_ptr(), workspace.data_ptr(), workspace.numel(),
            ctypes.c_void_p(stream.cuda_stream))
        _check(rc, "flce_forward_backward")
        return loss, gh, gw

    def forward(self, hidden: torch.Tensor, W: torch.Tensor, labels: torch.Tensor, ignore_index: int = -100,
                softcap: float = 0.0, reduction: str = "mean", return_lse: bool = False,
                workspace: torch.Tensor | None = None, stream=None):
        """Forward only. Returns the loss (0-dim fp32) for 'mean'/'sum', or the per-row loss terms
        [BT] fp32 for 'none'; with return_lse also the per-row log-sum-exp [BT] fp32."""
        BT, H, V = self._check_inputs(hidden, W, labels)
        if reduction not in _FWD_REDUCTIONS:
            raise ValueError("reduction must be 'none', 'mean' or 'sum'")
        dt = _DTYPES[hidden.dtype]
        need = forward_workspace_size(BT, H, V, hidden.dtype, self._h)
        if workspace is None:
            workspace = self.workspace(need)
        loss = torch.empty((), dtype=torch.float32, device=self.device) if reduction != "none" else None
        rows = torch.empty(BT, dtype=torch.float32, device=self.device) if reduction == "none" else None
        lse = torch.empty(BT, dtype=torch.float32, device=self.device) if return_lse else None
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        ptr = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
        rc = lib().flce_forward(
            self._h, hidden.data_ptr(), W.data_ptr(), labels.data_ptr(), BT, H, V, dt, int(ignore_index),
            float(softcap), _FWD_REDUCTIONS[reduction], ptr(loss), ptr(rows), ptr(lse),
            workspace.data_ptr(), workspace.numel(), ctypes.c_void_p(stream.cuda_stream))
        _check(rc, "flce_forward")
        out = loss if reduction != "none" else rows
        return (out, lse) if return_lse else out

    KERNELS = ("prepass", "fwd", "merge", "dx", "dx_reduce", "dw", "finalize", "transpose", "rows")

    def profile_begin(self, max_launches: int = 4096):
        """Bracket every following kernel launch with HIP events on its stream (diagnostics)."""
        _check(lib().flce_profile_begin(self._h, max_launches), "flce_profile_begin")

    def profile_end(self, stream=None) -> dict:
        """Synchronise and return {kernel: (total_ms, launches)} since profile_begin."""
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        n = len(self.KERNELS)
        ms = (ctypes.c_double * n)()
        cnt = (ctypes.c_int64 * n)()
        _check(lib().flce_profile_end(self._h, ctypes.c_void_p(stream.cuda_stream), ms, cnt),
               "flce_profile_end")
        return {k: (ms[i], cnt[i]) for i, k in enumerate(self.KERNELS)}

    def status(self, stream=None) -> int:
        """Synchronise and return the status code of the last call (0 or FLCE_ERR_LABEL_RANGE)."""
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        return lib().flce_status(self._h, ctypes.c_void_p(stream.cuda_stream))


_ENGINES: dict = {}


def engine(device=None) -> FLCE:
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    if dev.index is None:
        dev = torch.device("cuda", torch.cuda.current_device())
    if dev not in _ENGINES:
        _ENGINES[dev] = FLCE(dev)
    return _ENGINES[dev]


class _FLCEFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, hidden, W, labels, ignore_index, softcap, reduction):
        loss, gh, gw = engine(hidden.device).forward_backward(hidden, W, labels, ignore_index, softcap,
                                                               reduction)
        ctx.save_for_backward(gh, gw)
        ctx.w_dtype = W.dtype
        return loss

    @staticmethod
    def backward(ctx, grad_out):
        gh, gw = ctx.saved_tensors
        return gh * grad_out.to(gh.dtype), (gw * grad_out).to(ctx.w_dtype), None, None, None, None


def flce_loss(hidden, W, labels, ignore_index: int = -100, softcap: float = 0.0, reduction: str = "mean"):
    """Loss of softmax cross-entropy over hidden @ W.T (optionally softcapped) with autograd support.

    The gradients are produced in the same fused call as the loss and scaled by the upstream
    gradient in backward (e.g. a gradient-accumulation divisor)."""
    return _FLCEFunction.apply(hidden, W, labels, ignore_index, softcap, reduction)
