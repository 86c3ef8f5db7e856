"""Spatial-spectral coupling on AMD Instinct MI355X (gfx950).

The coupling of deep functional-map pipelines, Pi_NM Phi_M =
softmax(F_N F_M^T / sqrt(d)) Phi_M, is scaled dot-product attention with the
target descriptors as queries, the source descriptors as keys and the source
Laplace-Beltrami basis as values ("Spatial-Spectral Coupling as Attention",
project page, section "How it works").  This package is a thin ctypes
binding over `libssc.so`, whose hand-written HIP kernels compute both the
exact dense coupling and the Geo-FlashAttention coupling (section
"Geo-FlashAttention"), forward and backward.  Every step runs in the library;
Python only checks arguments, allocates outputs and workspaces with torch and
passes device pointers plus the current HIP stream.

The five entry points carry the C ABI's names (declared in include/ssc.h):
coupling_dense_fwd, coupling_dense_bwd, patch_score_topk, coupling_geo_fwd,
coupling_geo_bwd.  `dense_coupling` and `geo_coupling` wrap them as
autograd functions.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "CouplingError", "KernelTimer", "dense_route", "lib", "library_path", "workspace_bytes", "kpad",
    "coupling_dense_fwd", "coupling_dense_bwd", "patch_score_topk",
    "coupling_geo_fwd", "coupling_geo_bwd", "dense_coupling", "geo_coupling",
    "coupling_linear_fwd", "coupling_linear_bwd", "linear_coupling",
    "fmap_solve_fwd", "fmap_solve_bwd", "fmap_solve", "fps_partition",
    "coupling_performer_fwd", "coupling_performer_bwd", "performer_coupling",
    "OP_DENSE_FWD", "OP_DENSE_BWD", "OP_PATCH_TOPK", "OP_GEO_FWD", "OP_GEO_BWD",
    "OP_LINEAR_FWD", "OP_LINEAR_BWD", "OP_FMAP_FWD", "OP_FMAP_BWD", "OP_FPS", "OP_PERFORMER_FWD",
    "OP_PERFORMER_BWD",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
# SSC_LIBRARY selects another build of the library (the debug or the
# host-sanitized one); by default the in-tree libssc.so.
library_path = os.environ.get("SSC_LIBRARY") or os.path.join(_HERE, "libssc.so")

(OP_DENSE_FWD, OP_DENSE_BWD, OP_PATCH_TOPK, OP_GEO_FWD, OP_GEO_BWD, OP_LINEAR_FWD, OP_LINEAR_BWD,
 OP_FMAP_FWD, OP_FMAP_BWD, OP_FPS, OP_PERFORMER_FWD, OP_PERFORMER_BWD) = range(12)
_F32, _BF16 = 0, 1
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported shape", 3: "workspace too small",
           4: "HIP launch failed"}


class CouplingError(RuntimeError):
    """A non-zero status from libssc.so."""

    def __init__(self, fn: str, status: int, hip: int = 0):
        msg = f"{fn}: {_STATUS.get(status, 'status %d' % status)}"
        if status == 4:
            msg += f" (hipError_t {hip})"
        super().__init__(msg)
        self.status = status


_lib = None
_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "ssc_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i, _i]),
    "ssc_status_string": (ctypes.c_char_p, [_i]),
    "ssc_last_hip_error": (_i, []),
    "ssc_debug_build": (_i, []),
    "ssc_query": (_i, [_i, _i]),
    "ssc_dense_split": (_i, [_i]),
    "ssc_timer_arm": (_i, [ctypes.c_char_p, _i]),
    "ssc_timer_read": (_i, [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int)]),
    "coupling_dense_fwd": (_i, [_i, _i, _i, _i, _i, _vp, _vp, _vp, _f, _vp, _vp, _vp, _sz, _vp]),
    "coupling_dense_bwd": (_i, [_i, _i, _i, _i, _i, _vp, _vp, _vp, _f, _vp, _vp, _vp, _vp, _vp, _vp,
                                _vp, _sz, _vp]),
    "patch_score_topk": (_i, [_i, _i, _i, _i, _vp, _vp, _i, _i, _vp, _vp, _i, _vp, _vp, _vp, _sz, _vp]),
    "patch_score_topk_noalloc": (_i, [_i, _i, _i, _i, _vp, _vp, _i, _i, _vp, _vp, _i, _vp, _vp, _vp]),
    "coupling_geo_fwd": (_i, [_i, _i, _i, _i, _i, _vp, _i, _i, _vp, _i, _vp, _vp, _vp, _vp, _f, _vp,
                              _vp, _vp, _sz, _vp]),
    "coupling_geo_bwd": (_i, [_i, _i, _i, _i, _i, _vp, _i, _i, _vp, _i, _vp, _vp, _vp, _vp, _f, _vp,
                              _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "coupling_linear_fwd": (_i, [_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "coupling_linear_bwd": (_i, [_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                 _vp]),
    "fmap_solve_fwd": (_i, [_i, _i, _i, _vp, _vp, _vp, _vp, _sz, _vp]),
    "fmap_solve_bwd": (_i, [_i, _i, _i, _vp, _vp, _vp, _vp, _sz, _vp]),
    "fps_partition": (_i, [_i, _i, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _sz, _vp]),
    "coupling_performer_fwd": (_i, [_i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _f, _vp, _vp, _vp, _sz, _vp]),
    "coupling_performer_bwd": (_i, [_i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _f, _vp, _vp, _vp, _vp, _vp, _vp,
                                    _vp, _sz, _vp]),
}


def lib() -> ctypes.CDLL:
    """Load libssc.so (raises if it has not been built: there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(
                f"{library_path} is missing: build it with "
                "`python -m spatial_spectral_coupling_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(library_path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def kpad(k: int) -> int:
    """Internal padded width of the basis (0 if k is unsupported)."""
    return int(lib().ssc_query(0, int(k)))


class dense_route:
    """Route of the bf16 dense couplings on this thread inside a `with`
    block: "auto" (by size, the default), "dense" (always the dense kernels)
    or "split" (always the one-patch geo route, whose planner splits short
    item lists along their key stream).  The setting is per thread: calls
    that torch's autograd engine makes from its own thread (the backward of
    `dense_coupling`) keep the default."""

    _MODES = {"auto": -1, "dense": 0, "split": 1}

    def __init__(self, mode: str):
        if mode not in self._MODES:
            raise ValueError(f"dense route must be one of {sorted(self._MODES)}")
        self.mode = self._MODES[mode]

    def __enter__(self):
        self.prev = int(lib().ssc_dense_split(self.mode))
        return self

    def __exit__(self, *exc):
        lib().ssc_dense_split(self.prev)
        return False


class KernelTimer:
    """HIP-event timing of one kernel family inside the library, recorded on
    the stream each launch uses: `with KernelTimer("dkv", 64) as t: ...;
    t.read()` returns (summed ms, number of launches)."""

    def __init__(self, family: str, capacity: int = 256):
        self.family, self.capacity = family, capacity
        self.total_ms, self.count = 0.0, 0

    def __enter__(self):
        st = lib().ssc_timer_arm(self.family.encode(), int(self.capacity))
        if st != 0:
            raise CouplingError("ssc_timer_arm", st, lib().ssc_last_hip_error())
        return self

    def read(self):
        ms, n = ctypes.c_float(0), ctypes.c_int(0)
        st = lib().ssc_timer_read(ctypes.byref(ms), ctypes.byref(n))
        if st != 0:
            raise CouplingError("ssc_timer_read", st, lib().ssc_last_hip_error())
        if n.value < 0:
            raise RuntimeError("kernel timer overflow: raise the capacity")
        self.total_ms, self.count = float(ms.value), int(n.value)
        return self.total_ms, self.count

    def __exit__(self, *exc):
        lib().ssc_timer_arm(None, 0)
        return False


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _BF16
    if t.dtype == torch.float32:
        return _F32
    raise TypeError(f"inputs must be bfloat16 or float32, got {t.dtype}")


def workspace_bytes(op: int, dtype: torch.dtype, n_N: int, n_M: int, d: int, k: int,
                    P_N: int = 0, P_M: int = 0, s: int = 0) -> int:
    code = _BF16 if dtype == torch.bfloat16 else _F32
    return int(lib().ssc_workspace_bytes(op, code, n_N, n_M, d, k, P_N, P_M, s))


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_dev(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous (row-major)")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on the same device")
    return dev


def _stream(dev) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ws(nbytes: int, dev) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=dev)


def _call(name: str, *args):
    st = getattr(lib(), name)(*args)
    if st != 0:
        raise CouplingError(name, st, lib().ssc_last_hip_error())


def _scale(scale, d):
    return float(1.0 / math.sqrt(d) if scale is None else scale)


def _same_dtype(*ts):
    t0 = ts[0]
    for t in ts[1:]:
        if t.dtype != t0.dtype:
            raise TypeError("Q, K, V (and dO) must share one dtype")
    return _dt(t0)


def _i32(t: torch.Tensor, name: str):
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32")


def _want(t: Optional[torch.Tensor], name: str, shape, dtype):
    """Shape and dtype of a tensor the library reads or writes by raw pointer
    (a mismatch would make a kernel read or write past the buffer)."""
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _mat(t: torch.Tensor, name: str):
    if t.dim() != 2:
        raise ValueError(f"{name} must be a matrix, got {t.dim()} dimensions")
    return t.shape


def _offsets(off: torch.Tensor, name: str) -> int:
    _i32(off, name)
    if off.dim() != 1 or off.numel() < 2:
        raise ValueError(f"{name} must be a vector of P + 1 >= 2 offsets")
    return off.numel() - 1


# ---------------------------------------------------------------------------
# the five entry points
# ---------------------------------------------------------------------------
def coupling_dense_fwd(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, scale: Optional[float] = None,
                       O: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None
                       ) -> Tuple[torch.Tensor, torch.Tensor]:
    """O = softmax(Q K^T * scale) V (fp32) and lse (natural log), no map stored."""
    code = _same_dtype(Q, K, V)
    n_N, d = _mat(Q, "Q")
    n_M, k = _mat(V, "V")
    _want(K, "K", (n_M, d), Q.dtype)
    _want(O, "O", (n_N, k), torch.float32)
    _want(lse, "lse", (n_N,), torch.float32)
    dev = _check_dev(Q, K, V, O, lse)
    O = torch.empty(n_N, k, dtype=torch.float32, device=dev) if O is None else O
    lse = torch.empty(n_N, dtype=torch.float32, device=dev) if lse is None else lse
    ws = _ws(lib().ssc_workspace_bytes(OP_DENSE_FWD, code, n_N, n_M, d, k, 0, 0, 0), dev)
    _call("coupling_dense_fwd", code, n_N, n_M, d, k, _p(Q), _p(K), _p(V), _scale(scale, d),
          _p(O), _p(lse), _p(ws), ws.numel(), _stream(dev))
    return O, lse


def _check_bwd_inputs(Q, K, V, O, dO, lse):
    n_N, d = _mat(Q, "Q")
    n_M, k = _mat(V, "V")
    _want(K, "K", (n_M, d), Q.dtype)
    _want(O, "O", (n_N, k), torch.float32)
    _want(dO, "dO", (n_N, k), Q.dtype)
    _want(lse, "lse", (n_N,), torch.float32)
    return n_N, n_M, d, k


def coupling_dense_bwd(Q, K, V, O, dO, lse, scale: Optional[float] = None, need_dV: bool = True):
    """dQ, dK, dV (fp32) of <dO, O> for the dense coupling.  With need_dV
    False the library skips the dV products and dV is returned as None (the
    basis V = Phi_M is fixed in the functional-map pipelines)."""
    code = _same_dtype(Q, K, V, dO)
    n_N, n_M, d, k = _check_bwd_inputs(Q, K, V, O, dO, lse)
    dev = _check_dev(Q, K, V, O, dO, lse)
    dQ = torch.empty(n_N, d, dtype=torch.float32, device=dev)
    dK = torch.empty(n_M, d, dtype=torch.float32, device=dev)
    dV = torch.empty(n_M, k, dtype=torch.float32, device=dev) if need_dV else None
    ws = _ws(lib().ssc_workspace_bytes(OP_DENSE_BWD, code, n_N, n_M, d, k, 0, 0, 0), dev)
    _call("coupling_dense_bwd", code, n_N, n_M, d, k, _p(Q), _p(K), _p(V), _scale(scale, d),
          _p(O), _p(dO), _p(lse), _p(dQ), _p(dK), _p(dV), _p(ws), ws.numel(), _stream(dev))
    return dQ, dK, dV


def patch_score_topk(Q, offN, K, offM, s: int, return_scores: bool = False):
    """Top-s source patches per target patch from patch-mean descriptors.

    Q, K are patch-sorted; offN, offM int32 offsets (length P + 1) on the
    device.  Returns idx [P_N x s] int32 (and scores [P_N x P_M] fp64).
    """
    code = _same_dtype(Q, K)
    P_N, P_M = _offsets(offN, "offN"), _offsets(offM, "offM")
    n_N, d = _mat(Q, "Q")
    n_M, dk = _mat(K, "K")
    if dk != d:
        raise ValueError("Q and K must have the same width d")
    dev = _check_dev(Q, K, offN, offM)
    idx = torch.empty(P_N, s, dtype=torch.int32, device=dev)
    scores = torch.empty(P_N, P_M, dtype=torch.float64, device=dev) if return_scores else None
    ws = _ws(lib().ssc_workspace_bytes(OP_PATCH_TOPK, code, n_N, n_M, d, 1, P_N, P_M, s), dev)
    _call("patch_score_topk", code, d, n_N, P_N, _p(offN), _p(Q), n_M, P_M, _p(offM), _p(K), int(s),
          _p(idx), _p(scores), _p(ws), ws.numel(), _stream(dev))
    return (idx, scores) if return_scores else idx


def _check_selection(offN, offM, idx):
    P_N, P_M = _offsets(offN, "offN"), _offsets(offM, "offM")
    _i32(idx, "idx")
    if idx.dim() != 2 or idx.shape[0] != P_N:
        raise ValueError(f"idx must be P_N x s = {P_N} x s, got {tuple(idx.shape)}")
    return P_N, P_M, idx.shape[1]


def coupling_geo_fwd(Q, K, V, offN, offM, idx, scale: Optional[float] = None):
    """Geo-FlashAttention forward on patch-sorted rows: O (fp32), lse."""
    code = _same_dtype(Q, K, V)
    n_N, d = _mat(Q, "Q")
    n_M, k = _mat(V, "V")
    _want(K, "K", (n_M, d), Q.dtype)
    P_N, P_M, s = _check_selection(offN, offM, idx)
    dev = _check_dev(Q, K, V, offN, offM, idx)
    O = torch.empty(n_N, k, dtype=torch.float32, device=dev)
    lse = torch.empty(n_N, dtype=torch.float32, device=dev)
    ws = _ws(lib().ssc_workspace_bytes(OP_GEO_FWD, code, n_N, n_M, d, k, P_N, P_M, s), dev)
    _call("coupling_geo_fwd", code, d, k, n_N, P_N, _p(offN), n_M, P_M, _p(offM), s, _p(idx),
          _p(Q), _p(K), _p(V), _scale(scale, d), _p(O), _p(lse), _p(ws), ws.numel(), _stream(dev))
    return O, lse


def coupling_geo_bwd(Q, K, V, offN, offM, idx, O, dO, lse, scale: Optional[float] = None, need_dV: bool = True):
    """Geo-FlashAttention backward for the fixed selection idx: dQ, dK, dV
    (fp32); dV is skipped (None) with need_dV False."""
    code = _same_dtype(Q, K, V, dO)
    n_N, n_M, d, k = _check_bwd_inputs(Q, K, V, O, dO, lse)
    P_N, P_M, s = _check_selection(offN, offM, idx)
    dev = _check_dev(Q, K, V, offN, offM, idx, O, dO, lse)
    dQ = torch.empty(n_N, d, dtype=torch.float32, device=dev)
    dK = torch.empty(n_M, d, dtype=torch.float32, device=dev)
    dV = torch.empty(n_M, k, dtype=torch.float32, device=dev) if need_dV else None
    ws = _ws(lib().ssc_workspace_bytes(OP_GEO_BWD, code, n_N, n_M, d, k, P_N, P_M, s), dev)
    _call("coupling_geo_bwd", code, d, k, n_N, P_N, _p(offN), n_M, P_M, _p(offM), s, _p(idx),
          _p(Q), _p(K), _p(V), _scale(scale, d), _p(O), _p(dO), _p(lse), _p(dQ), _p(dK), _p(dV),
          _p(ws), ws.numel(), _stream(dev))
    return dQ, dK, dV


# ---------------------------------------------------------------------------
# autograd wrappers
# ---------------------------------------------------------------------------
class _Dense(torch.autograd.Function):
    @staticmethod
    def forward(ctx, Q, K, V, scale):
        O, lse = coupling_dense_fwd(Q, K, V, scale)
        ctx.save_for_backward(Q, K, V, O, lse)
        ctx.scale = scale
        return O

    @staticmethod
    def backward(ctx, dO):
        Q, K, V, O, lse = ctx.saved_tensors
        need_dV = bool(ctx.needs_input_grad[2])
        dQ, dK, dV = coupling_dense_bwd(Q, K, V, O, dO.to(Q.dtype).contiguous(), lse, ctx.scale, need_dV=need_dV)
        return dQ.to(Q.dtype), dK.to(K.dtype), dV.to(V.dtype) if need_dV else None, None


class _Geo(torch.autograd.Function):
    @staticmethod
    def forward(ctx, Q, K, V, offN, offM, idx, scale):
        O, lse = coupling_geo_fwd(Q, K, V, offN, offM, idx, scale)
        ctx.save_for_backward(Q, K, V, offN, offM, idx, O, lse)
        ctx.scale = scale
        return O

    @staticmethod
    def backward(ctx, dO):
        Q, K, V, offN, offM, idx, O, lse = ctx.saved_tensors
        need_dV = bool(ctx.needs_input_grad[2])
        dQ, dK, dV = coupling_geo_bwd(Q, K, V, offN, offM, idx, O, dO.to(Q.dtype).contiguous(), lse,
                                      ctx.scale, need_dV=need_dV)
        return dQ.to(Q.dtype), dK.to(K.dtype), dV.to(V.dtype) if need_dV else None, None, None, None, None


def dense_coupling(Q, K, V, scale: Optional[float] = None):
    """Differentiable Pi_NM Phi_M (dense, exact)."""
    return _Dense.apply(Q, K, V, _scale(scale, Q.shape[1]))


def geo_coupling(Q, K, V, offN, offM, s: int, scale: Optional[float] = None):
    """Differentiable Geo-FlashAttention coupling; selection recomputed per call."""
    idx = patch_score_topk(Q.detach(), offN, K.detach(), offM, s)
    return _Geo.apply(Q, K, V, offN, offM, idx, _scale(scale, Q.shape[1]))


# ---------------------------------------------------------------------------
# linear-attention (ELU feature map) coupling
# ---------------------------------------------------------------------------
def coupling_linear_fwd(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """O = phi(Q)(phi(K)^T V) / (phi(Q) phi(K)^T 1), phi = elu + 1 (bf16 in, fp32
    out), and the per-row normaliser den."""
    code = _same_dtype(Q, K, V)
    n_N, d = _mat(Q, "Q")
    n_M, k = _mat(V, "V")
    _want(K, "K", (n_M, d), Q.dtype)
    dev = _check_dev(Q, K, V)
    O = torch.empty(n_N, k, dtype=torch.float32, device=dev)
    den = torch.empty(n_N, dtype=torch.float32, device=dev)
    ws = _ws(lib().ssc_workspace_bytes(OP_LINEAR_FWD, code, n_N, n_M, d, k, 0, 0, 0), dev)
    _call("coupling_linear_fwd", code, n_N, n_M, d, k, _p(Q), _p(K), _p(V), _p(O), _p(den), _p(ws),
          ws.numel(), _stream(dev))
    return O, den


def coupling_linear_bwd(Q, K, V, O, dO, den):
    """dQ, dK, dV (fp32) of <dO, O> for the linear coupling."""
    code = _same_dtype(Q, K, V, dO)
    n_N, n_M, d, k = _check_bwd_inputs(Q, K, V, O, dO, den)
    dev = _check_dev(Q, K, V, O, dO, den)
    dQ = torch.empty(n_N, d, dtype=torch.float32, device=dev)
    dK = torch.empty(n_M, d, dtype=torch.float32, device=dev)
    dV = torch.empty(n_M, k, dtype=torch.float32, device=dev)
    ws = _ws(lib().ssc_workspace_bytes(OP_LINEAR_BWD, code, n_N, n_M, d, k, 0, 0, 0), dev)
    _call("coupling_linear_bwd", code, n_N, n_M, d, k, _p(Q), _p(K), _p(V), _p(O), _p(dO), _p(den),
          _p(dQ), _p(dK), _p(dV), _p(ws), ws.numel(), _stream(dev))
    return dQ, dK, dV


class _LinearCoupling(torch.autograd.Function):
    @staticmethod
    def forward(ctx, Q, K, V):
        O, den = coupling_linear_fwd(Q, K, V)
        ctx.save_for_backward(Q, K, V, O, den)
        return O

    @staticmethod
    def backward(ctx, dO):
        Q, K, V, O, den = ctx.saved_tensors
        dQ, dK, dV = coupling_linear_bwd(Q, K, V, O, dO.to(Q.dtype).contiguous(), den)
        return dQ.to(Q.dtype), dK.to(K.dtype), dV.to(V.dtype)


def linear_coupling(Q, K, V):
    """Differentiable linear-attention coupling (autograd wrapper)."""
    return _LinearCoupling.apply(Q, K, V)


def fmap_solve_fwd(PhiN: torch.Tensor, O: torch.Tensor) -> torch.Tensor:
    """Least-squares functional map C = (PhiN^T PhiN)^-1 PhiN^T O (k x k,
    fp32) from the coupling's output O = Pi Phi_M (n x k fp32) and the target
    basis PhiN (n x k bf16)."""
    code = _same_dtype(PhiN)
    n, k = _mat(PhiN, "PhiN")
    _want(O, "O", (n, k), torch.float32)
    dev = _check_dev(PhiN, O)
    C = torch.empty(k, k, dtype=torch.float32, device=dev)
    ws = _ws(lib().ssc_workspace_bytes(OP_FMAP_FWD, code, n, 0, 0, k, 0, 0, 0), dev)
    _call("fmap_solve_fwd", code, n, k, _p(PhiN), _p(O), _p(C), _p(ws), ws.numel(), _stream(dev))
    return C


def fmap_solve_bwd(PhiN: torch.Tensor, dC: torch.Tensor) -> torch.Tensor:
    """dO = PhiN (PhiN^T PhiN)^-1 dC (n x k fp32) for an upstream gradient dC
    (k x k fp32); the basis is held fixed."""
    code = _same_dtype(PhiN)
    n, k = _mat(PhiN, "PhiN")
    _want(dC, "dC", (k, k), torch.float32)
    dev = _check_dev(PhiN, dC)
    dO = torch.empty(n, k, dtype=torch.float32, device=dev)
    ws = _ws(lib().ssc_workspace_bytes(OP_FMAP_BWD, code, n, 0, 0, k, 0, 0, 0), dev)
    _call("fmap_solve_bwd", code, n, k, _p(PhiN), _p(dC.contiguous()), _p(dO), _p(ws), ws.numel(), _stream(dev))
    return dO


class _FmapSolve(torch.autograd.Function):
    @staticmethod
    def forward(ctx, PhiN, O):
        ctx.save_for_backward(PhiN)
        return fmap_solve_fwd(PhiN, O)

    @staticmethod
    def backward(ctx, dC):
        (PhiN,) = ctx.saved_tensors
        return None, fmap_solve_bwd(PhiN, dC.float().contiguous())


def fmap_solve(PhiN, O):
    """Differentiable functional-map solve (gradient for O only)."""
    return _FmapSolve.apply(PhiN, O)


def fps_partition(x: torch.Tensor, off: torch.Tensor, adj: torch.Tensor, P: int):
    """Geodesic farthest-point sampling of P seeds on a mesh given by fp64
    positions x [n x 3] and its CSR adjacency (off [n+1], adj [nnz] int32,
    both directions of every edge).  Returns (seeds [P] int32, labels [n]
    int32 = index of the nearest seed, dist [n] fp64)."""
    dev = _check_dev(x, off, adj) if adj.numel() else _check_dev(x, off)
    if x.dtype != torch.float64 or x.dim() != 2 or x.shape[1] != 3:
        raise TypeError("x must be n x 3 float64")
    if off.dtype != torch.int32 or adj.dtype != torch.int32:
        raise TypeError("off and adj must be int32")
    n, nnz = x.shape[0], adj.numel()
    if off.numel() != n + 1:
        raise ValueError("off must have n + 1 entries")
    seeds = torch.empty(P, dtype=torch.int32, device=dev)
    labels = torch.empty(n, dtype=torch.int32, device=dev)
    dist = torch.empty(n, dtype=torch.float64, device=dev)
    ws = _ws(lib().ssc_workspace_bytes(OP_FPS, 0, n, nnz, 0, 0, P, 0, 0), dev)
    _call("fps_partition", n, nnz, _p(x), _p(off), _p(adj) if nnz else None, P, _p(seeds), _p(labels), _p(dist),
          _p(ws), ws.numel(), _stream(dev))
    return seeds, labels, dist


def _directions(W, d, dtype):
    """Feature count m of the Performer directions W [m x d]."""
    m, _ = _mat(W, "W")
    _want(W, "W", (m, d), dtype)
    return m


def coupling_performer_fwd(Q, K, V, W, scale: Optional[float] = None):
    """Performer (FAVOR+) coupling: O = phi(Q) (phi(K)^T V) / den and ln den
    (fp32), with m random directions W [m x d] bf16 (m in {64, 128})."""
    code = _same_dtype(Q, K, V, W)
    n_N, d = _mat(Q, "Q")
    n_M, k = _mat(V, "V")
    _want(K, "K", (n_M, d), Q.dtype)
    m = _directions(W, d, Q.dtype)
    dev = _check_dev(Q, K, V, W)
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    O = torch.empty(n_N, k, dtype=torch.float32, device=dev)
    lnden = torch.empty(n_N, dtype=torch.float32, device=dev)
    ws = _ws(lib().ssc_workspace_bytes(OP_PERFORMER_FWD, code, n_N, n_M, d, k, m, 0, 0), dev)
    _call("coupling_performer_fwd", code, n_N, n_M, d, k, m, _p(Q), _p(K), _p(V), _p(W), sc, _p(O), _p(lnden),
          _p(ws), ws.numel(), _stream(dev))
    return O, lnden


def coupling_performer_bwd(Q, K, V, W, O, dO, lnden, scale: Optional[float] = None):
    """dQ, dK, dV (fp32) of <dO, O> for the Performer coupling (W fixed)."""
    code = _same_dtype(Q, K, V, W, dO)
    n_N, n_M, d, k = _check_bwd_inputs(Q, K, V, O, dO, lnden)
    m = _directions(W, d, Q.dtype)
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dev = _check_dev(Q, K, V, W, O, dO, lnden)
    dQ = torch.empty(n_N, d, dtype=torch.float32, device=dev)
    dK = torch.empty(n_M, d, dtype=torch.float32, device=dev)
    dV = torch.empty(n_M, k, dtype=torch.float32, device=dev)
    ws = _ws(lib().ssc_workspace_bytes(OP_PERFORMER_BWD, code, n_N, n_M, d, k, m, 0, 0), dev)
    _call("coupling_performer_bwd", code, n_N, n_M, d, k, m, _p(Q), _p(K), _p(V), _p(W), sc, _p(O), _p(dO),
          _p(lnden), _p(dQ), _p(dK), _p(dV), _p(ws), ws.numel(), _stream(dev))
    return dQ, dK, dV


class _PerformerCoupling(torch.autograd.Function):
    @staticmethod
    def forward(ctx, Q, K, V, W, scale):
        O, lnden = coupling_performer_fwd(Q, K, V, W, scale)
        ctx.save_for_backward(Q, K, V, W, O, lnden)
        ctx.scale = scale
        return O

    @staticmethod
    def backward(ctx, dO):
        Q, K, V, W, O, lnden = ctx.saved_tensors
        dQ, dK, dV = coupling_performer_bwd(Q, K, V, W, O, dO.to(Q.dtype).contiguous(), lnden, ctx.scale)
        return dQ.to(Q.dtype), dK.to(K.dtype), dV.to(V.dtype), None, None


def performer_coupling(Q, K, V, W, scale: Optional[float] = None):
    """Differentiable Performer coupling (autograd wrapper; W gets no gradient)."""
    return _PerformerCoupling.apply(Q, K, V, W, scale)
