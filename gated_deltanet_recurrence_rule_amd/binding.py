"""ctypes binding of libgdn's C ABI (include/gdn.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the computation runs in the library's kernels.  There is
no fallback -- if libgdn.so is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdn.so")

GDN_BF16 = 0
GDN_F32 = 1

# update rules (gdn_variant in include/gdn.h)
GDN_GATED_DELTA = 0
GDN_DELTA = 1
GDN_GATED_LINEAR = 2
GDN_LINEAR = 3
VARIANTS = {"gated_delta": GDN_GATED_DELTA, "delta": GDN_DELTA, "gated_linear": GDN_GATED_LINEAR,
            "linear": GDN_LINEAR}

_lib = None


class GdnError(RuntimeError):
    """A libgdn call returned a non-zero status."""

    def __init__(self, status: int, text: str):
        super().__init__(f"libgdn status {status}: {text}")
        self.status = status


def load() -> ctypes.CDLL:
    """Load libgdn.so from the package directory (raises if it was never built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first (python -m "
                           "gated_deltanet_recurrence_rule_amd.build or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    vp, fp, i32, i64, sz = (ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                            ctypes.c_size_t)
    lib.gdn_decode_step.argtypes = [vp, vp, vp, fp, fp, fp, vp, i32, i32, i32, i32, i32, ctypes.c_int,
                                    ctypes.c_float, vp]
    lib.gdn_decode_step.restype = ctypes.c_int
    lib.gdn_decode_step_v.argtypes = [vp, vp, vp, fp, fp, fp, vp, i32, i32, i32, i32, i32, ctypes.c_int,
                                      ctypes.c_float, ctypes.c_int, vp]
    lib.gdn_decode_step_v.restype = ctypes.c_int
    lib.gdn_prefill_workspace_size.argtypes = [i32, i64, i32, i32, i32, i32, ctypes.c_int]
    lib.gdn_prefill_workspace_size.restype = sz
    lib.gdn_prefill.argtypes = [vp, vp, vp, fp, fp, vp, vp, i32, i64, fp, vp, fp, i32, i32, i32, i32,
                                ctypes.c_int, ctypes.c_float, vp, sz, vp]
    lib.gdn_prefill.restype = ctypes.c_int
    lib.gdn_prefill_v.argtypes = [vp, vp, vp, fp, fp, vp, vp, i32, i64, fp, vp, fp, i32, i32, i32, i32,
                                  ctypes.c_int, ctypes.c_float, ctypes.c_int, vp, sz, vp]
    lib.gdn_prefill_v.restype = ctypes.c_int
    lib.gdn_status_str.argtypes = [ctypes.c_int]
    lib.gdn_status_str.restype = ctypes.c_char_p
    lib.gdn_last_error.argtypes = []
    lib.gdn_last_error.restype = ctypes.c_char_p
    lib.gdn_prefill_kernel_name.argtypes = [i32, i64, i32, i32, i32, i32, ctypes.c_int]
    lib.gdn_prefill_kernel_name.restype = ctypes.c_char_p
    lib.gdn_version.argtypes = []
    lib.gdn_version.restype = ctypes.c_int32
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        lib = load()
        raise GdnError(status, f"{lib.gdn_status_str(status).decode()}: {lib.gdn_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise TypeError(f"q, k, v must be bfloat16 or float32, got {t.dtype}")


def _variant_code(variant) -> int:
    if isinstance(variant, str):
        if variant not in VARIANTS:
            raise ValueError(f"unknown variant {variant!r}; one of {sorted(VARIANTS)}")
        return VARIANTS[variant]
    return int(variant)


def _need_opt(t: Optional[torch.Tensor], name: str, dtype):
    if t is not None:
        _need(t, name, dtype)


def _need(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: Optional[torch.Tensor],
                beta: Optional[torch.Tensor], S: torch.Tensor, *, scale: float = 1.0,
                o: Optional[torch.Tensor] = None, variant="gated_delta") -> torch.Tensor:
    """One token for every sequence and V head; S [N, HV, dk, dv] fp32 is updated in place.

    q, k [N, HQK, dk]; v [N, HV, dv] (bf16 or fp32, one type); g, beta [N, HV] fp32.
    Returns o [N, HV, dv] in v's dtype.  variant: "gated_delta" (default), "delta",
    "gated_linear" or "linear" (gdn_variant); the library decides which of g / beta
    may be None for it.
    """
    N, HQK, dk = q.shape
    HV, dv = v.shape[1], v.shape[2]
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype)
    _need_opt(g, "g", torch.float32)
    _need_opt(beta, "beta", torch.float32)
    _need(S, "S", torch.float32)
    if o is None:
        o = torch.empty((N, HV, dv), dtype=v.dtype, device=v.device)
    _need(o, "o", v.dtype)
    var = _variant_code(variant)
    lib = load()
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S), _ptr(o), N, HQK, HV, dk, dv,
            _dtype_code(q), float(scale))
    if var == GDN_GATED_DELTA:
        _check(lib.gdn_decode_step(*args, _stream(q.device)))
    else:
        _check(lib.gdn_decode_step_v(*args, var, _stream(q.device)))
    return o


def prefill_workspace_size(N: int, total_T: int, HQK: int, HV: int, dk: int, dv: int,
                           dtype: torch.dtype) -> int:
    code = GDN_BF16 if dtype == torch.bfloat16 else GDN_F32
    return int(load().gdn_prefill_workspace_size(N, total_T, HQK, HV, dk, dv, code))


def prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: Optional[torch.Tensor],
            beta: Optional[torch.Tensor], *, cu_seqlens: Optional[torch.Tensor] = None,
            cu_seqlens_host=None, N: Optional[int] = None, S0: Optional[torch.Tensor] = None,
            scale: float = 1.0, o: Optional[torch.Tensor] = None,
            S_T: Optional[torch.Tensor] = None, output_state: bool = True,
            workspace: Optional[torch.Tensor] = None,
            variant="gated_delta") -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Whole sequences of a packed batch.

    q, k [total_T, HQK, dk]; v [total_T, HV, dv]; g, beta [total_T, HV] fp32.
    cu_seqlens: int32 device tensor [N + 1] (or None with N given: equal lengths).
    cu_seqlens_host: optional host copy (list / numpy / CPU tensor) for validation.
    S0 [N, HV, dk, dv] fp32 or None.  Returns (o [total_T, HV, dv], S_T or None).
    variant: as for decode_step.
    """
    total_T, HQK, dk = q.shape
    HV, dv = v.shape[1], v.shape[2]
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype)
    _need_opt(g, "g", torch.float32)
    _need_opt(beta, "beta", torch.float32)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32)
        n_seq = int(cu_seqlens.shape[0] - 1)
    else:
        if N is None:
            raise ValueError("give cu_seqlens or N")
        n_seq = int(N)
    host = None
    if cu_seqlens_host is not None:
        import numpy as np
        host = np.ascontiguousarray(np.asarray(cu_seqlens_host, dtype=np.int32))
        if host.shape[0] != n_seq + 1:
            raise ValueError("cu_seqlens_host must have N + 1 entries")
    if S0 is not None:
        _need(S0, "S0", torch.float32)
    if o is None:
        o = torch.empty((total_T, HV, dv), dtype=v.dtype, device=v.device)
    _need(o, "o", v.dtype)
    if S_T is None and output_state:
        S_T = torch.empty((n_seq, HV, dk, dv), dtype=torch.float32, device=v.device)
    if S_T is not None:
        _need(S_T, "S_T", torch.float32)
    lib = load()
    code = _dtype_code(q)
    need = int(lib.gdn_prefill_workspace_size(n_seq, total_T, HQK, HV, dk, dv, code))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=v.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    host_ptr = None if host is None else host.ctypes.data_as(ctypes.c_void_p)
    var = _variant_code(variant)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), host_ptr, n_seq, total_T,
            _ptr(S0), _ptr(o), _ptr(S_T), HQK, HV, dk, dv, code, float(scale))
    if var == GDN_GATED_DELTA:
        _check(lib.gdn_prefill(*args, _ptr(workspace), ws_bytes, _stream(q.device)))
    else:
        _check(lib.gdn_prefill_v(*args, var, _ptr(workspace), ws_bytes, _stream(q.device)))
    return o, S_T


def prefill_kernel_name(N: int, total_T: int, HQK: int, HV: int, dk: int, dv: int,
                        dtype: torch.dtype) -> str:
    code = GDN_BF16 if dtype == torch.bfloat16 else GDN_F32
    return load().gdn_prefill_kernel_name(N, total_T, HQK, HV, dk, dv, code).decode()


def version() -> int:
    return int(load().gdn_version())
