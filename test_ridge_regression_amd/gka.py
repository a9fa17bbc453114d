"""Thin Python binding of libgka.so (argument marshalling only; every step runs in the HIP kernels).

The names mirror the C ABI in include/gka.h:

  fwd_chunked(q, k, v, gamma, a, iters, chunk, state=None, ...)   -> gka_fwd_chunked
  step(q, k, v, gamma, a, iters, state)                             -> gka_step

Tensors are torch device tensors (PyTorch supplies device memory and the current stream).
If the shared library is missing, loading fails loudly: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# GKA_LIBRARY names another build of the library (a sanitizer build of the host code, say)
LIB_PATH = os.environ.get("GKA_LIBRARY") or os.path.join(_HERE, "libgka.so")

GKA_BF16 = 0
GKA_FP32 = 1
GKA_MAX_ITERS = 64
STATUS = {0: "GKA_OK", 1: "GKA_ERR_NULL", 2: "GKA_ERR_SHAPE", 3: "GKA_ERR_VALUE",
          4: "GKA_ERR_DTYPE", 5: "GKA_ERR_WORKSPACE", 6: "GKA_ERR_HIP", 7: "GKA_ERR_ALIAS",
          8: "GKA_ERR_SCRATCH"}
GKA_STATIC_SCRATCH_BYTES = 64 << 20
EXPORTED = ["gka_fwd_workspace_bytes", "gka_fwd_chunked", "gka_step", "gka_fwd_chunked_beta",
            "gka_step_beta", "gka_fwd_chunked_residuals", "gka_step_residuals",
            "gka_fwd_varlen", "gka_fwd_varlen_workspace_bytes", "gka_bwd",
            "gka_bwd_workspace_bytes", "gka_fwd_chunked_static", "gka_status_str",
            "gka_abi_version"]


class GkaParams(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("D", ctypes.c_int32), ("chunk", ctypes.c_int32), ("iters", ctypes.c_int32),
                ("a", ctypes.c_float), ("dtype", ctypes.c_int32), ("segments", ctypes.c_int32)]


class GkaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libgka.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is not built; run `python -m test_ridge_regression_amd.build` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(GkaParams)
    vp, fp = ctypes.c_void_p, ctypes.c_void_p
    lib.gka_fwd_workspace_bytes.argtypes = [P]
    lib.gka_fwd_workspace_bytes.restype = ctypes.c_size_t
    lib.gka_fwd_chunked.argtypes = [P, vp, vp, vp, fp, vp, fp, fp, fp, fp, vp, ctypes.c_size_t, vp,
                                    ctypes.c_void_p]
    lib.gka_fwd_chunked.restype = ctypes.c_int
    lib.gka_step.argtypes = [P, vp, vp, vp, fp, vp, fp, fp, fp, vp]
    lib.gka_step.restype = ctypes.c_int
    lib.gka_fwd_chunked_beta.argtypes = [P, vp, vp, vp, fp, fp, vp, fp, fp, fp, fp, vp,
                                         ctypes.c_size_t, vp, ctypes.c_void_p]
    lib.gka_fwd_chunked_beta.restype = ctypes.c_int
    lib.gka_step_beta.argtypes = [P, vp, vp, vp, fp, fp, vp, fp, fp, fp, vp]
    lib.gka_step_beta.restype = ctypes.c_int
    lib.gka_fwd_chunked_residuals.argtypes = [P, vp, vp, vp, fp, fp, vp, fp, fp, fp, fp, fp, vp,
                                              ctypes.c_size_t, vp]
    lib.gka_fwd_chunked_residuals.restype = ctypes.c_int
    lib.gka_step_residuals.argtypes = [P, vp, vp, vp, fp, fp, vp, fp, fp, fp, fp, vp]
    lib.gka_step_residuals.restype = ctypes.c_int
    lib.gka_fwd_varlen.argtypes = [P, vp, ctypes.c_int64, vp, vp, vp, fp, fp, vp, fp, fp, fp, fp,
                                   vp, ctypes.c_size_t, vp]
    lib.gka_fwd_varlen.restype = ctypes.c_int
    lib.gka_fwd_varlen_workspace_bytes.argtypes = [P]
    lib.gka_fwd_varlen_workspace_bytes.restype = ctypes.c_size_t
    lib.gka_bwd_workspace_bytes.argtypes = [P]
    lib.gka_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.gka_bwd.argtypes = [P, vp, vp, vp, fp, fp, vp, vp, vp, vp, fp, fp, vp, ctypes.c_size_t,
                            vp]
    lib.gka_bwd.restype = ctypes.c_int
    lib.gka_fwd_chunked_static.argtypes = [P, vp, vp, vp, fp, fp, vp, fp, fp, fp, fp, vp]
    lib.gka_fwd_chunked_static.restype = ctypes.c_int
    lib.gka_status_str.argtypes = [ctypes.c_int]
    lib.gka_status_str.restype = ctypes.c_char_p
    lib.gka_abi_version.argtypes = []
    lib.gka_abi_version.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise GkaError(status, load().gka_status_str(status).decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GKA_BF16
    if t.dtype == torch.float32:
        return GKA_FP32
    return -1


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _require_io(q, k, v, gamma, o, state, gamma_shape, n_states):
    """Marshalling checks the C side cannot make, in this order: dense tensors of matching
    element types, the shapes of gamma (``gamma_shape``) and of the carried state (``n_states``
    heads' worth: h, u [n_states..., D, D], n2 [n_states...]), and that every tensor lives on
    q's CUDA device. A host tensor would hand a host pointer to a kernel, and a short gamma or
    state would be read (the state also written) past its end; neither is visible from C."""
    ts = [q, k, v, gamma, o] + ([state.h, state.u, state.n2] if state is not None else [])
    for t in ts:
        if not t.is_contiguous():
            raise ValueError("libgka takes dense contiguous tensors")
    if not (q.dtype == k.dtype == v.dtype == o.dtype):
        raise ValueError("q, k, v and o must share one dtype (bfloat16 or float32)")
    if gamma.dtype != torch.float32 or (state is not None and not (
            state.h.dtype == state.u.dtype == state.n2.dtype == torch.float32)):
        raise ValueError("gamma and the state are float32")
    if k.shape != q.shape or v.shape != q.shape or o.shape != q.shape:
        raise ValueError("q, k, v, o must have the same shape")
    if tuple(gamma.shape) != tuple(gamma_shape):
        raise ValueError(f"gamma must have shape {tuple(gamma_shape)}, got {tuple(gamma.shape)}")
    if state is not None:
        D = q.shape[-1]
        n = tuple(n_states)
        if (tuple(state.h.shape) != n + (D, D) or tuple(state.u.shape) != n + (D, D)
                or tuple(state.n2.shape) != n):
            raise ValueError(f"state must be h, u {n + (D, D)} and n2 {n}")
    _require_device(q, ts)


def _require_device(q, ts):
    """Every tensor in ``ts`` (None entries skipped) on q's device, which must be a GPU."""
    if not q.is_cuda:
        raise ValueError("libgka takes GPU (device) tensors")
    for t in ts:
        if t is not None and (not t.is_cuda or t.device != q.device):
            raise ValueError(f"every tensor must be on {q.device}; got one on {t.device}")


def _require_beta(beta, shape):
    """The write gate: None, or a dense float32 tensor of the gates' shape."""
    if beta is None:
        return
    if beta.dtype != torch.float32 or not beta.is_contiguous() or tuple(beta.shape) != tuple(shape):
        raise ValueError(f"beta must be a dense float32 tensor of shape {tuple(shape)}")


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


@dataclasses.dataclass
class GkaState:
    """Carried state of B x H heads: h, u float32 [B, H, D, D] (u is [value][key]), n2 float32
    [B, H] = ||H||_F^2. Owned by the caller; updated in place by the library."""
    h: torch.Tensor
    u: torch.Tensor
    n2: torch.Tensor

    @staticmethod
    def zeros(B: int, H: int, D: int, device="cuda") -> "GkaState":
        return GkaState(torch.zeros(B, H, D, D, device=device, dtype=torch.float32),
                        torch.zeros(B, H, D, D, device=device, dtype=torch.float32),
                        torch.zeros(B, H, device=device, dtype=torch.float32))


def make_params(B, T, H, D, chunk, iters, a, dtype_code, segments=0) -> GkaParams:
    return GkaParams(int(B), int(T), int(H), int(D), int(chunk), int(iters), float(a),
                     int(dtype_code), int(segments))


def workspace_bytes(B, T, H, D, chunk, iters, a, dtype_code, segments=0) -> int:
    p = make_params(B, T, H, D, chunk, iters, a, dtype_code, segments)
    return int(load().gka_fwd_workspace_bytes(ctypes.byref(p)))


def varlen_workspace_bytes(B, T, H, D, chunk, iters, a, dtype_code, segments=0) -> int:
    """gka_fwd_varlen_workspace_bytes: B sequences, every length <= T."""
    p = make_params(B, T, H, D, chunk, iters, a, dtype_code, segments)
    return int(load().gka_fwd_varlen_workspace_bytes(ctypes.byref(p)))


def fwd_chunked(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gamma: torch.Tensor, a: float,
                iters: int, chunk: int = 64, state: Optional[GkaState] = None,
                return_hnorm: bool = False, segments: int = 0, out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, stream=None, phase_events=None,
                beta: Optional[torch.Tensor] = None):
    """gka_fwd_chunked on [B, T, H, D] tensors; returns o (and per-token ||H_t||_F [B,T,H]).

    ``state`` (optional) is read as the initial state and overwritten with the final one.
    ``phase_events`` (optional) is a ctypes array of 4 hipEvent_t handles recorded at the
    phase boundaries (see include/gka.h). ``beta`` (optional, float32 [B, T, H]) is the
    per-token write gate; with it the call goes to gka_fwd_chunked_beta.
    """
    lib = load()
    B, T, H, D = q.shape
    p = make_params(B, T, H, D, chunk, iters, a, _dtype_code(q), segments)
    o = torch.empty_like(q) if out is None else out
    _require_io(q, k, v, gamma, o, state, (B, T, H), (B, H))
    _require_beta(beta, (B, T, H))
    hn = torch.empty(B, T, H, device=q.device, dtype=torch.float32) if return_hnorm else None
    need = int(lib.gka_fwd_workspace_bytes(ctypes.byref(p)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    _require_device(q, [beta, workspace])
    rest = (_ptr(o), _ptr(state.h if state else None), _ptr(state.u if state else None),
            _ptr(state.n2 if state else None), _ptr(hn), _ptr(workspace),
            ctypes.c_size_t(workspace.numel() if workspace is not None else 0),
            _stream(stream), phase_events)
    if beta is None:
        st = lib.gka_fwd_chunked(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma), *rest)
    else:
        st = lib.gka_fwd_chunked_beta(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma),
                                      _ptr(beta), *rest)
    _check(st)
    return (o, hn) if return_hnorm else o


def fwd_chunked_beta(q, k, v, gamma, beta, a, iters, **kw):
    """gka_fwd_chunked_beta: fwd_chunked with the per-token write gate beta [B, T, H]."""
    return fwd_chunked(q, k, v, gamma, a, iters, beta=beta, **kw)


def fwd_chunked_static(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gamma: torch.Tensor,
                       a: float, iters: int, chunk: int = 64, state: Optional[GkaState] = None,
                       beta: Optional[torch.Tensor] = None, segments: int = 0,
                       out: Optional[torch.Tensor] = None, hnorm: Optional[torch.Tensor] = None,
                       stream=None):
    """gka_fwd_chunked_static: fwd_chunked without a workspace (the library's static scratch
    holds the segment states). The call allocates nothing when ``out`` (and ``hnorm``, the
    optional per-token ||H_t||_F [B, T, H] output) are given; returns o."""
    lib = load()
    B, T, H, D = q.shape
    p = make_params(B, T, H, D, chunk, iters, a, _dtype_code(q), segments)
    o = torch.empty_like(q) if out is None else out
    _require_io(q, k, v, gamma, o, state, (B, T, H), (B, H))
    _require_beta(beta, (B, T, H))
    if hnorm is not None and (hnorm.dtype != torch.float32 or not hnorm.is_contiguous()
                              or tuple(hnorm.shape) != (B, T, H)):
        raise ValueError(f"hnorm must be a dense float32 tensor of shape {(B, T, H)}")
    _require_device(q, [beta, hnorm])
    st = lib.gka_fwd_chunked_static(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma), _ptr(beta), _ptr(o),
        _ptr(state.h if state else None), _ptr(state.u if state else None),
        _ptr(state.n2 if state else None), _ptr(hnorm), _stream(stream))
    _check(st)
    return o


def step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gamma: torch.Tensor, a: float,
         iters: int, state: GkaState, out: Optional[torch.Tensor] = None, stream=None,
         beta: Optional[torch.Tensor] = None):
    """gka_step on [B, H, D] tensors; updates ``state`` in place and returns o [B, H, D].
    ``beta`` (optional, float32 [B, H]) is the write gate; with it the call goes to
    gka_step_beta."""
    lib = load()
    B, H, D = q.shape
    p = make_params(B, 1, H, D, 64, iters, a, _dtype_code(q))
    o = torch.empty_like(q) if out is None else out
    _require_io(q, k, v, gamma, o, state, (B, H), (B, H))
    _require_beta(beta, (B, H))
    _require_device(q, [beta])
    rest = (_ptr(o), _ptr(state.h), _ptr(state.u), _ptr(state.n2), _stream(stream))
    if beta is None:
        st = lib.gka_step(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma), *rest)
    else:
        st = lib.gka_step_beta(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma),
                               _ptr(beta), *rest)
    _check(st)
    return o


def step_beta(q, k, v, gamma, beta, a, iters, state, **kw):
    """gka_step_beta: step with the write gate beta [B, H]."""
    return step(q, k, v, gamma, a, iters, state, beta=beta, **kw)


def fwd_chunked_residuals(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                          gamma: torch.Tensor, a: float, iters: int, chunk: int = 64,
                          state: Optional[GkaState] = None, beta: Optional[torch.Tensor] = None,
                          return_hnorm: bool = False, segments: int = 0,
                          out: Optional[torch.Tensor] = None,
                          resid: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None, stream=None):
    """gka_fwd_chunked_residuals: the forward plus ||q_t - A_t x_i|| for i = 0..iters.

    Returns (o, resid) -- resid float32 [B, T, H, iters + 1] -- or (o, resid, hnorm)."""
    lib = load()
    B, T, H, D = q.shape
    p = make_params(B, T, H, D, chunk, iters, a, _dtype_code(q), segments)
    o = torch.empty_like(q) if out is None else out
    _require_io(q, k, v, gamma, o, state, (B, T, H), (B, H))
    _require_beta(beta, (B, T, H))
    if resid is None:
        resid = torch.empty(B, T, H, iters + 1, device=q.device, dtype=torch.float32)
    elif (resid.dtype != torch.float32 or not resid.is_contiguous()
          or tuple(resid.shape) != (B, T, H, iters + 1)):
        raise ValueError("resid must be a dense float32 [B, T, H, iters + 1] tensor")
    hn = torch.empty(B, T, H, device=q.device, dtype=torch.float32) if return_hnorm else None
    need = int(lib.gka_fwd_workspace_bytes(ctypes.byref(p)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    _require_device(q, [beta, resid, workspace])
    st = lib.gka_fwd_chunked_residuals(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma), _ptr(beta), _ptr(o),
        _ptr(state.h if state else None), _ptr(state.u if state else None),
        _ptr(state.n2 if state else None), _ptr(hn), _ptr(resid), _ptr(workspace),
        ctypes.c_size_t(workspace.numel() if workspace is not None else 0), _stream(stream))
    _check(st)
    return (o, resid, hn) if return_hnorm else (o, resid)


def step_residuals(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gamma: torch.Tensor,
                   a: float, iters: int, state: GkaState, beta: Optional[torch.Tensor] = None,
                   out: Optional[torch.Tensor] = None, stream=None):
    """gka_step_residuals: one decode step plus ||q - A x_i||, i = 0..iters; returns
    (o [B, H, D], resid float32 [B, H, iters + 1])."""
    lib = load()
    B, H, D = q.shape
    p = make_params(B, 1, H, D, 64, iters, a, _dtype_code(q))
    o = torch.empty_like(q) if out is None else out
    _require_io(q, k, v, gamma, o, state, (B, H), (B, H))
    _require_beta(beta, (B, H))
    _require_device(q, [beta])
    resid = torch.empty(B, H, iters + 1, device=q.device, dtype=torch.float32)
    st = lib.gka_step_residuals(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma),
                                _ptr(beta), _ptr(o), _ptr(state.h), _ptr(state.u),
                                _ptr(state.n2), _ptr(resid), _stream(stream))
    _check(st)
    return o, resid


def fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gamma: torch.Tensor,
               cu_seqlens: torch.Tensor, max_seqlen: int, a: float, iters: int, chunk: int = 64,
               state: Optional[GkaState] = None, beta: Optional[torch.Tensor] = None,
               return_hnorm: bool = False, segments: int = 0, out: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None, stream=None, total: Optional[int] = None):
    """gka_fwd_varlen on a packed batch: q, k, v [total, H, D]; gamma (and beta) [total, H];
    cu_seqlens int32 [B + 1] on the device; every length <= max_seqlen. ``state`` (optional)
    holds one carried state per sequence ([B, H, D, D], [B, H]). ``total`` defaults to the
    number of rows of q. Returns o (and per-row ||H_t||_F [total, H])."""
    lib = load()
    rows, H, D = q.shape
    B = cu_seqlens.numel() - 1
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_contiguous() or B < 1:
        raise ValueError("cu_seqlens must be a dense int32 tensor of B + 1 offsets")
    total = rows if total is None else int(total)
    p = make_params(B, max_seqlen, H, D, chunk, iters, a, _dtype_code(q), segments)
    o = torch.empty_like(q) if out is None else out
    _require_io(q, k, v, gamma, o, state, (rows, H), (B, H))
    _require_beta(beta, (rows, H))
    hn = torch.empty(rows, H, device=q.device, dtype=torch.float32) if return_hnorm else None
    need = int(lib.gka_fwd_varlen_workspace_bytes(ctypes.byref(p)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    _require_device(q, [cu_seqlens, beta, workspace])
    st = lib.gka_fwd_varlen(
        ctypes.byref(p), _ptr(cu_seqlens), ctypes.c_int64(total), _ptr(q), _ptr(k), _ptr(v),
        _ptr(gamma), _ptr(beta), _ptr(o), _ptr(state.h if state else None),
        _ptr(state.u if state else None), _ptr(state.n2 if state else None), _ptr(hn),
        _ptr(workspace), ctypes.c_size_t(workspace.numel() if workspace is not None else 0),
        _stream(stream))
    _check(st)
    return (o, hn) if return_hnorm else o


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gamma: torch.Tensor,
        dout: torch.Tensor, a: float, iters: int, beta: Optional[torch.Tensor] = None,
        workspace: Optional[torch.Tensor] = None, stream=None):
    """gka_bwd: gradients of sum <dout, o> for the forward from the zero state.
    Returns (dq, dk, dv, dgamma, dbeta) -- dq, dk, dv in the dtype of q, the rest float32."""
    lib = load()
    B, T, H, D = q.shape
    p = make_params(B, T, H, D, 64, iters, a, _dtype_code(q))
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    _require_io(q, k, v, gamma, dq, None, (B, T, H), (B, H))
    if dout.shape != q.shape or dout.dtype != q.dtype or not dout.is_contiguous():
        raise ValueError("dout must match q")
    _require_beta(beta, (B, T, H))
    dgamma = torch.empty(B, T, H, device=q.device, dtype=torch.float32)
    dbeta = torch.empty(B, T, H, device=q.device, dtype=torch.float32)
    need = int(lib.gka_bwd_workspace_bytes(ctypes.byref(p)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=q.device, dtype=torch.uint8)
    _require_device(q, [dout, beta, workspace])
    st = lib.gka_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma), _ptr(beta),
                     _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dgamma), _ptr(dbeta),
                     _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream(stream))
    _check(st)
    return dq, dk, dv, dgamma, dbeta


def lib_bwd_workspace(w) -> int:
    """gka_bwd_workspace_bytes for a workload description (B, T, H, D, iters, a, dtype)."""
    p = make_params(w.B, w.T, w.H, w.D, 64, w.iters, w.a,
                    GKA_BF16 if w.dtype == "bf16" else GKA_FP32)
    return int(load().gka_bwd_workspace_bytes(ctypes.byref(p)))
