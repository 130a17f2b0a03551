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


class Rows(ctypes.Structure):
    """flce_rows: B sequences of T positions at element strides; shift = 1 scores position t
    against the label at t + 1 and leaves the last position out."""
    _fields_ = [("batch", ctypes.c_int64), ("seq", ctypes.c_int64), ("shift", ctypes.c_int64),
                ("hidden_stride", ctypes.c_int64 * 2), ("grad_hidden_stride", ctypes.c_int64 * 2),
                ("label_stride", ctypes.c_int64 * 2)]


FLCE_ACCUMULATE_GRAD_HIDDEN, FLCE_ACCUMULATE_GRAD_W, FLCE_NO_GRAD_HIDDEN, FLCE_NO_GRAD_W = 1, 2, 4, 8


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
            L.flce_chunk_plan.argtypes = [vp, i64, i64, i64, i32, ctypes.POINTER(i64), ctypes.POINTER(i64)]
            L.flce_forward_backward.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i64, ctypes.c_float,
                                                i32, vp, vp, vp, vp, ctypes.c_size_t, vp]
            L.flce_forward_workspace_size.argtypes = [vp, i64, i64, i64, i32, ctypes.POINTER(ctypes.c_size_t)]
            L.flce_forward.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i64, ctypes.c_float, i32,
                                       vp, vp, vp, vp, ctypes.c_size_t, vp]
            rp = ctypes.POINTER(Rows)
            L.flce_workspace_size_rows.argtypes = [vp, rp, i64, i64, i32, ctypes.POINTER(ctypes.c_size_t)]
            L.flce_forward_backward_rows.argtypes = [vp, vp, vp, vp, rp, i64, i64, i32, i64, ctypes.c_float, i32,
                                                     ctypes.c_float, i32, vp, vp, vp, vp, ctypes.c_size_t, vp]
            L.flce_forward_rows.argtypes = [vp, vp, vp, vp, rp, i64, i64, i32, i64, ctypes.c_float, i32,
                                            vp, vp, vp, vp, ctypes.c_size_t, vp]
            L.flce_recompute_workspace_size.argtypes = [vp, i64, i64, i64, i32, i64, ctypes.POINTER(ctypes.c_size_t)]
            L.flce_forward_backward_recompute.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i64, ctypes.c_float,
                                                          i32, i64, vp, vp, vp, vp, ctypes.c_size_t, vp]
            L.flce_forward_backward_static.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i64, ctypes.c_float,
                                                       i32, vp, vp, vp, vp]
            L.flce_status.argtypes = [vp, vp]
            L.flce_profile_begin.argtypes = [vp, i32]
            L.flce_profile_end.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]
            L.flce_error_string.argtypes = [i32]
            L.flce_error_string.restype = ctypes.c_char_p
            for f in ("flce_create", "flce_destroy", "flce_workspace_size", "flce_chunk_plan",
                      "flce_forward_backward", "flce_forward_workspace_size", "flce_forward", "flce_status",
                      "flce_workspace_size_rows", "flce_forward_backward_rows", "flce_forward_rows",
                      "flce_recompute_workspace_size", "flce_forward_backward_recompute",
                      "flce_profile_begin", "flce_profile_end", "flce_forward_backward_static"):
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


def recompute_workspace_size(BT: int, H: int, V: int, dtype=torch.bfloat16, v_slice: int = 0, handle=None) -> int:
    out = ctypes.c_size_t()
    _check(lib().flce_recompute_workspace_size(handle, BT, H, V, _DTYPES[dtype], v_slice, ctypes.byref(out)),
           "flce_recompute_workspace_size")
    return out.value


def workspace_size_rows(rows: Rows, H: int, V: int, dtype=torch.bfloat16, handle=None) -> int:
    out = ctypes.c_size_t()
    _check(lib().flce_workspace_size_rows(handle, ctypes.byref(rows), H, V, _DTYPES[dtype], ctypes.byref(out)),
           "flce_workspace_size_rows")
    return out.value


def chunk_plan(BT: int, H: int, V: int, dtype=torch.bfloat16, handle=None):
    """(number of chunks, rows per chunk) of the library's row plan for this problem."""
    n, c = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().flce_chunk_plan(handle, BT, H, V, _DTYPES[dtype], ctypes.byref(n), ctypes.byref(c)),
           "flce_chunk_plan")
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

    def chunk_plan(self, BT, H, V, dtype=torch.bfloat16):
        return chunk_plan(BT, H, V, dtype, self._h)

    def _stream(self, stream, tensors):
        """The stream a call enqueues on. Another stream than the current one first waits for the
        current stream (which produced the inputs and the tensors allocated for the call), and every
        tensor of the call, the cached workspace included, is marked as used on it, so that torch's
        caching allocator does not hand that memory out again while the stream may still use it."""
        cur = torch.cuda.current_stream(self.device)
        if stream is None or stream == cur:
            return cur
        stream.wait_stream(cur)
        for t in tensors:
            if t is not None:
                t.record_stream(stream)
        return stream

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
                         out=None, workspace: torch.Tensor | None = None, stream=None,
                         grad_hidden: bool = True, grad_W: bool = True):
        """Run the fused forward + backward; returns (loss [0-dim fp32], grad_hidden, grad_W fp32).
        With grad_hidden=False or grad_W=False that gradient is not computed (its GEMM does not run)
        and None is returned in its place."""
        BT, H, V = self._check_inputs(hidden, W, labels)
        if reduction not in _REDUCTIONS:
            raise ValueError("reduction must be 'mean' or 'sum'")
        if not (grad_hidden or grad_W):
            raise ValueError("no gradient asked for: use forward()")
        dt = _DTYPES[hidden.dtype]
        need = self.workspace_size(BT, H, V, hidden.dtype)
        if workspace is None:
            workspace = self.workspace(need)
        if out is None:
            loss = torch.empty((), dtype=torch.float32, device=self.device)
            gh = torch.empty_like(hidden) if grad_hidden else None
            gw = torch.empty((V, H), dtype=torch.float32, device=self.device) if grad_W else None
        else:
            loss, gh, gw = out
            gh, gw = (gh if grad_hidden else None), (gw if grad_W else None)
        stream = self._stream(stream, (hidden, W, labels, loss, gh, gw, workspace))
        ptr = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
        if grad_hidden and grad_W:
            rc = lib().flce_forward_backward(
                self._h, hidden.data_ptr(), W.data_ptr(), labels.data_ptr(), BT, H, V, dt,
                int(ignore_index), float(softcap), _REDUCTIONS[reduction], loss.data_ptr(),
                gh.data_ptr(), gw.data_ptr(), workspace.data_ptr(), workspace.numel(),
                ctypes.c_void_p(stream.cuda_stream))
            _check(rc, "flce_forward_backward")
        else:
            # the plain [BT, H] layout as one sequence of BT positions, with one gradient left out
            rows = Rows(1, BT, 0, (ctypes.c_int64 * 2)(0, H), (ctypes.c_int64 * 2)(0, H),
                        (ctypes.c_int64 * 2)(0, 1))
            flags = (0 if grad_hidden else FLCE_NO_GRAD_HIDDEN) | (0 if grad_W else FLCE_NO_GRAD_W)
            rc = lib().flce_forward_backward_rows(
                self._h, hidden.data_ptr(), W.data_ptr(), labels.data_ptr(), ctypes.byref(rows), H, V, dt,
                int(ignore_index), float(softcap), _REDUCTIONS[reduction], 1.0, flags, loss.data_ptr(),
                ptr(gh), ptr(gw), workspace.data_ptr(), workspace.numel(), ctypes.c_void_p(stream.cuda_stream))
            _check(rc, "flce_forward_backward_rows")
        return loss, gh, gw

    def forward_backward_recompute(self, hidden: torch.Tensor, W: torch.Tensor, labels: torch.Tensor,
                                   ignore_index: int = -100, softcap: float = 0.0, reduction: str = "mean",
                                   v_slice: int = 0, out=None, workspace: torch.Tensor | None = None, stream=None):
        """The recompute mode (logits formed twice; vocabulary slices outermost over all rows, one
        slice of dZ numerators kept at a time); returns (loss, grad_hidden, grad_W fp32) like
        forward_backward."""
        BT, H, V = self._check_inputs(hidden, W, labels)
        if reduction not in _REDUCTIONS:
            raise ValueError("reduction must be 'mean' or 'sum'")
        need = recompute_workspace_size(BT, H, V, hidden.dtype, v_slice, self._h)
        if workspace is None:
            workspace = self.workspace(need)
        if out is None:
            loss = torch.empty((), dtype=torch.float32, device=self.device)
            gh = torch.empty_like(hidden)
            gw = torch.empty((V, H), dtype=torch.float32, device=self.device)
        else:
            loss, gh, gw = out
        stream = self._stream(stream, (hidden, W, labels, loss, gh, gw, workspace))
        rc = lib().flce_forward_backward_recompute(
            self._h, hidden.data_ptr(), W.data_ptr(), labels.data_ptr(), BT, H, V, _DTYPES[hidden.dtype],
            int(ignore_index), float(softcap), _REDUCTIONS[reduction], int(v_slice), loss.data_ptr(),
            gh.data_ptr(), gw.data_ptr(), workspace.data_ptr(), workspace.numel(), ctypes.c_void_p(stream.cuda_stream))
        _check(rc, "flce_forward_backward_recompute")
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
        stream = self._stream(stream, (hidden, W, labels, loss, rows, lse, workspace))
        ptr = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
        rc = lib().flce_forward(
            self._h, hidden.data_ptr(), W.data_ptr(), labels.data_ptr(), BT, H, V, dt, int(ignore_index),
            float(softcap), _FWD_REDUCTIONS[reduction], ptr(loss), ptr(rows), ptr(lse),
            workspace.data_ptr(), workspace.numel(), ctypes.c_void_p(stream.cuda_stream))
        _check(rc, "flce_forward")
        out = loss if reduction != "none" else rows
        return (out, lse) if return_lse else out

    def _seq_rows(self, hidden: torch.Tensor, W: torch.Tensor, labels: torch.Tensor, shift: bool,
                  grad_hidden: torch.Tensor | None = None) -> tuple:
        if hidden.dim() != 3 or W.dim() != 2 or labels.dim() != 2:
            raise ValueError("hidden [B,T,H], W [V,H], labels [B,T] expected")
        B, T, H = hidden.shape
        V = W.shape[0]
        if W.shape[1] != H or tuple(labels.shape) != (B, T):
            raise ValueError(f"shape mismatch: hidden {tuple(hidden.shape)}, W {tuple(W.shape)}, "
                             f"labels {tuple(labels.shape)}")
        if hidden.dtype != W.dtype or hidden.dtype not in _DTYPES:
            raise TypeError("hidden and W must both be bfloat16 or both float32")
        if labels.dtype != torch.int64:
            raise TypeError("labels must be int64")
        for name, t in (("hidden", hidden), ("W", W), ("labels", labels), ("grad_hidden", grad_hidden)):
            if t is not None and t.device != self.device:
                raise ValueError(f"{name} is on {t.device}, handle is on {self.device}")
        if not W.is_contiguous():
            raise ValueError("W must be contiguous")
        if hidden.stride(2) != 1 or (grad_hidden is not None and grad_hidden.stride(2) != 1):
            raise ValueError("hidden and grad_hidden rows must be contiguous (unit stride along H)")
        if grad_hidden is not None and (tuple(grad_hidden.shape) != (B, T, H) or grad_hidden.dtype != hidden.dtype):
            raise ValueError("grad_hidden must match hidden's shape and dtype")
        g = grad_hidden if grad_hidden is not None else hidden
        r = Rows(B, T, 1 if shift else 0, (ctypes.c_int64 * 2)(hidden.stride(0), hidden.stride(1)),
                 (ctypes.c_int64 * 2)(g.stride(0), g.stride(1)),
                 (ctypes.c_int64 * 2)(labels.stride(0), labels.stride(1)))
        return r, B, T, H, V

    def forward_backward_seq(self, hidden: torch.Tensor, W: torch.Tensor, labels: torch.Tensor, shift: bool = True,
                             ignore_index: int = -100, softcap: float = 0.0, reduction: str = "mean",
                             grad_scale: float = 1.0, grad_hidden: torch.Tensor | None = None,
                             grad_W: torch.Tensor | None = None, accumulate_grad_hidden: bool = False,
                             accumulate_grad_W: bool = False, loss: torch.Tensor | None = None,
                             workspace: torch.Tensor | None = None, stream=None, need_grad_hidden: bool = True,
                             need_grad_W: bool = True):
        """Fused forward + backward over a batch of sequences hidden [B,T,H] (any strides with H
        contiguous) and labels [B,T]; with shift, position t is scored against label t+1 and the
        last position gets no gradient of its own. Gradients are multiplied by grad_scale and
        written into (or, with the accumulate flags, added to) grad_hidden [B,T,H] and grad_W
        [V,H] fp32, allocated when not given. need_grad_hidden=False / need_grad_W=False leave that
        gradient out (its GEMM does not run; None is returned for it). Returns (loss, grad_hidden,
        grad_W)."""
        if reduction not in _REDUCTIONS:
            raise ValueError("reduction must be 'mean' or 'sum'")
        if not (need_grad_hidden or need_grad_W):
            raise ValueError("no gradient asked for: use forward_seq()")
        if accumulate_grad_hidden and grad_hidden is None or accumulate_grad_W and grad_W is None:
            raise ValueError("accumulating needs the gradient tensor to add to")
        if (accumulate_grad_hidden and not need_grad_hidden) or (accumulate_grad_W and not need_grad_W):
            raise ValueError("cannot accumulate into a gradient that is left out")
        if not need_grad_hidden:
            grad_hidden = None
        elif grad_hidden is None:
            grad_hidden = torch.empty(hidden.shape, dtype=hidden.dtype, device=self.device)
        rows, B, T, H, V = self._seq_rows(hidden, W, labels, shift, grad_hidden)
        if not need_grad_W:
            grad_W = None
        elif grad_W is None:
            grad_W = torch.empty((V, H), dtype=torch.float32, device=self.device)
        if grad_W is not None and (tuple(grad_W.shape) != (V, H) or grad_W.dtype != torch.float32
                                   or not grad_W.is_contiguous() or grad_W.device != self.device):
            raise ValueError("grad_W must be a contiguous [V,H] float32 tensor on the handle's device")
        if loss is None:
            loss = torch.empty((), dtype=torch.float32, device=self.device)
        flags = (FLCE_ACCUMULATE_GRAD_HIDDEN if accumulate_grad_hidden else 0) | \
                (FLCE_ACCUMULATE_GRAD_W if accumulate_grad_W else 0) | \
                (0 if need_grad_hidden else FLCE_NO_GRAD_HIDDEN) | (0 if need_grad_W else FLCE_NO_GRAD_W)
        need = workspace_size_rows(rows, H, V, hidden.dtype, self._h)
        if workspace is None:
            workspace = self.workspace(need)
        stream = self._stream(stream, (hidden, W, labels, loss, grad_hidden, grad_W, workspace))
        ptr = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
        rc = lib().flce_forward_backward_rows(
            self._h, hidden.data_ptr(), W.data_ptr(), labels.data_ptr(), ctypes.byref(rows), H, V,
            _DTYPES[hidden.dtype], int(ignore_index), float(softcap), _REDUCTIONS[reduction], float(grad_scale),
            flags, loss.data_ptr(), ptr(grad_hidden), ptr(grad_W), workspace.data_ptr(),
            workspace.numel(), ctypes.c_void_p(stream.cuda_stream))
        _check(rc, "flce_forward_backward_rows")
        return loss, grad_hidden, grad_W

    def forward_seq(self, hidden: torch.Tensor, W: torch.Tensor, labels: torch.Tensor, shift: bool = True,
                    ignore_index: int = -100, softcap: float = 0.0, reduction: str = "mean",
                    return_lse: bool = False, workspace: torch.Tensor | None = None, stream=None):
        """Forward only over a batch of sequences (as forward_backward_seq). Returns the loss, or
        for 'none' the per-row terms [B, T - shift]; with return_lse also lse [B, T - shift]."""
        if reduction not in _FWD_REDUCTIONS:
            raise ValueError("reduction must be 'none', 'mean' or 'sum'")
        rows, B, T, H, V = self._seq_rows(hidden, W, labels, shift)
        P = max(T - rows.shift, 0)
        need = forward_workspace_size(B * P, H, V, hidden.dtype, self._h)
        if workspace is None:
            workspace = self.workspace(need)
        loss = torch.empty((), dtype=torch.float32, device=self.device) if reduction != "none" else None
        per = torch.empty((B, P), dtype=torch.float32, device=self.device) if reduction == "none" else None
        lse = torch.empty((B, P), dtype=torch.float32, device=self.device) if return_lse else None
        stream = self._stream(stream, (hidden, W, labels, loss, per, lse, workspace))
        ptr = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
        rc = lib().flce_forward_rows(
            self._h, hidden.data_ptr(), W.data_ptr(), labels.data_ptr(), ctypes.byref(rows), H, V,
            _DTYPES[hidden.dtype], int(ignore_index), float(softcap), _FWD_REDUCTIONS[reduction], ptr(loss),
            ptr(per), ptr(lse), workspace.data_ptr(), workspace.numel(), ctypes.c_void_p(stream.cuda_stream))
        _check(rc, "flce_forward_rows")
        out = loss if reduction != "none" else per
        return (out, lse) if return_lse else out

    KERNELS = ("prepass", "fwd", "lse", "dx", "dx_reduce", "dw", "finalize", "transpose", "rows", "zero",
               "rowref", "rowfix")

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
    """The loss with its gradients computed in the same fused call: only the gradients autograd will
    ask for are computed and kept (hidden's, W's or both)."""

    @staticmethod
    def forward(ctx, hidden, W, labels, ignore_index, softcap, reduction, shift):
        e = engine(hidden.device)
        need_gh, need_gw = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        if hidden.dim() == 3:
            loss, gh, gw = e.forward_backward_seq(hidden, W, labels, shift, ignore_index, softcap, reduction,
                                                  need_grad_hidden=need_gh, need_grad_W=need_gw)
        else:
            loss, gh, gw = e.forward_backward(hidden, W, labels, ignore_index, softcap, reduction,
                                              grad_hidden=need_gh, grad_W=need_gw)
        ctx.save_for_backward(gh, gw)
        ctx.w_dtype = W.dtype
        return loss

    @staticmethod
    def backward(ctx, grad_out):
        gh, gw = ctx.saved_tensors
        dh = gh * grad_out.to(gh.dtype) if gh is not None else None
        dw = (gw * grad_out).to(ctx.w_dtype) if gw is not None else None
        return dh, dw, None, None, None, None, None


def flce_loss(hidden, W, labels, ignore_index: int = -100, softcap: float = 0.0, reduction: str = "mean",
              shift: bool = False):
    """Loss of softmax cross-entropy over hidden @ W.T (optionally softcapped) with autograd support.

    hidden is [BT, H] with labels [BT], or [B, T, H] (any strides, H contiguous) with labels [B, T];
    for the latter, shift=True scores position t against label t+1 and leaves the last position out
    (its gradient is zero). The gradients are produced in the same fused call as the loss and scaled
    by the upstream gradient in backward (e.g. a gradient-accumulation divisor)."""
    if shift and hidden.dim() != 3:
        raise ValueError("shift needs hidden [B, T, H] and labels [B, T]")
    if not (torch.is_grad_enabled() and (hidden.requires_grad or W.requires_grad)):
        # no gradient will be asked for (evaluation, torch.no_grad): the forward alone, one GEMM
        e = engine(hidden.device)
        if hidden.dim() == 3:
            return e.forward_seq(hidden, W, labels, shift, ignore_index, softcap, reduction)
        return e.forward(hidden, W, labels, ignore_index, softcap, reduction)
    return _FLCEFunction.apply(hidden, W, labels, ignore_index, softcap, reduction, bool(shift))
