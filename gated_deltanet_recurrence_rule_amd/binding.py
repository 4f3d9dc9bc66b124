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


class BlockOps(ctypes.Structure):
    """gdn_block_ops: gates from raw projections and the gated RMS norm (include/gdn.h)."""
    _fields_ = [("A_log", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p), ("beta_logits", ctypes.c_int32),
                ("z", ctypes.c_void_p), ("norm_w", ctypes.c_void_p), ("norm_eps", ctypes.c_float),
                ("alpha_sigmoid", ctypes.c_int32)]


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
    ops_p = ctypes.POINTER(BlockOps)
    lib.gdn_decode_step_ex.argtypes = [vp, vp, vp, fp, fp, fp, vp, i32, i32, i32, i32, i32, ctypes.c_int,
                                       ctypes.c_float, ctypes.c_int, ops_p, vp]
    lib.gdn_decode_step_ex.restype = ctypes.c_int
    lib.gdn_prefill_workspace_size.argtypes = [i32, i64, i32, i32, i32, i32, ctypes.c_int]
    lib.gdn_prefill_workspace_size.restype = sz
    lib.gdn_prefill_workspace_size_lens.argtypes = [i32, i64, vp, i32, i32, i32, i32, ctypes.c_int]
    lib.gdn_prefill_workspace_size_lens.restype = sz
    lib.gdn_prefill.argtypes = [vp, vp, vp, fp, fp, vp, vp, i32, i64, fp, vp, fp, i32, i32, i32, i32,
                                ctypes.c_int, ctypes.c_float, vp, sz, vp]
    lib.gdn_prefill.restype = ctypes.c_int
    lib.gdn_prefill_v.argtypes = [vp, vp, vp, fp, fp, vp, vp, i32, i64, fp, vp, fp, i32, i32, i32, i32,
                                  ctypes.c_int, ctypes.c_float, ctypes.c_int, vp, sz, vp]
    lib.gdn_prefill_v.restype = ctypes.c_int
    lib.gdn_prefill_ex.argtypes = [vp, vp, vp, fp, fp, vp, vp, i32, i64, fp, vp, fp, i32, i32, i32, i32,
                                   ctypes.c_int, ctypes.c_float, ctypes.c_int, ops_p, vp, sz, vp]
    lib.gdn_prefill_ex.restype = ctypes.c_int
    lib.gdn_prefill_noalloc.argtypes = [vp, vp, vp, fp, fp, vp, vp, i32, i64, fp, vp, fp, i32, i32, i32, i32,
                                        ctypes.c_int, ctypes.c_float, ctypes.c_int, ops_p, vp]
    lib.gdn_prefill_noalloc.restype = ctypes.c_int
    lib.gdn_conv_silu.argtypes = [vp, vp, vp, vp, i32, i64, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                  ctypes.c_int, vp]
    lib.gdn_conv_silu.restype = ctypes.c_int
    lib.gdn_gated_rmsnorm.argtypes = [vp, vp, vp, ctypes.c_float, vp, i64, i32, ctypes.c_int, vp]
    lib.gdn_gated_rmsnorm.restype = ctypes.c_int
    lib.gdn_status_str.argtypes = [ctypes.c_int]
    lib.gdn_status_str.restype = ctypes.c_char_p
    lib.gdn_last_error.argtypes = []
    lib.gdn_last_error.restype = ctypes.c_char_p
    lib.gdn_prefill_kernel_name.argtypes = [i32, i64, vp, i32, i32, i32, i32, ctypes.c_int]
    lib.gdn_prefill_kernel_name.restype = ctypes.c_char_p
    lib.gdn_prefill_narrow_count.argtypes = [i32, i64, vp, i32, i32, i32, i32, ctypes.c_int]
    lib.gdn_prefill_narrow_count.restype = ctypes.c_int32
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


def _need_opt(t: Optional[torch.Tensor], name: str, dtype, shape=None, device=None):
    if t is not None:
        _need(t, name, dtype, shape, device)


def _block_ops(A_log, dt_bias, beta_logits, z, norm_w, norm_eps, io_dtype, alpha_sigmoid=False, *,
               HV, dv, z_shape, device):
    """A BlockOps for the given parts, or None when none is asked for."""
    if A_log is None and dt_bias is None and not beta_logits and z is None and not alpha_sigmoid:
        return None
    _need_opt(A_log, "A_log", torch.float32, (HV,), device)
    _need_opt(dt_bias, "dt_bias", torch.float32, (HV,), device)
    _need_opt(z, "z", io_dtype, z_shape, device)
    _need_opt(norm_w, "norm_w", torch.float32, (dv,), device)
    if dt_bias is not None and A_log is None and not alpha_sigmoid:
        raise ValueError("dt_bias is only used with A_log or alpha_sigmoid")
    return BlockOps(None if A_log is None else A_log.data_ptr(),
                    None if dt_bias is None else dt_bias.data_ptr(), 1 if beta_logits else 0,
                    None if z is None else z.data_ptr(), None if norm_w is None else norm_w.data_ptr(),
                    float(norm_eps), 1 if alpha_sigmoid else 0)


def _need(t: torch.Tensor, name: str, dtype=None, shape=None, device=None):
    """t must be a contiguous device tensor of the given dtype, shape and device: the C ABI sees
    only pointers, so a tensor smaller than its sizes imply would be read or written past its
    end by the kernels."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the call runs on {device}")


def _dims(t: torch.Tensor, name: str, n: int):
    if t.dim() != n:
        raise ValueError(f"{name} must have {n} dimensions, got shape {tuple(t.shape)}")
    return tuple(int(x) for x in t.shape)


def decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: Optional[torch.Tensor],
                beta: Optional[torch.Tensor], S: torch.Tensor, *, scale: float = 1.0,
                o: Optional[torch.Tensor] = None, variant="gated_delta", A_log=None, dt_bias=None,
                beta_logits: bool = False, z=None, norm_w=None, norm_eps: float = 1e-6,
                alpha_sigmoid: bool = False) -> torch.Tensor:
    """One token for every sequence and V head; S [N, HV, dk, dv] fp32 is updated in place.

    q, k [N, HQK, dk]; v [N, HV, dv] (bf16 or fp32, one type); g, beta [N, HV] fp32.
    Returns o [N, HV, dv] in v's dtype.  variant: "gated_delta" (default), "delta",
    "gated_linear" or "linear" (gdn_variant); the library decides which of g / beta
    may be None for it.  Block parts (gdn_block_ops): A_log, dt_bias [HV] fp32 make g the
    raw decay projection; beta_logits makes beta the raw projection b; z [N, HV, dv] with
    norm_w [dv] and norm_eps applies the gated RMS norm to o; alpha_sigmoid (with dt_bias as
    the bias) makes g the raw a of alpha = sigmoid(a + bias) instead.
    """
    N, HQK, dk = _dims(q, "q", 3)
    _, HV, dv = _dims(v, "v", 3)
    dev = q.device
    _need(q, "q", q.dtype, device=dev)
    _need(k, "k", q.dtype, (N, HQK, dk), dev)
    _need(v, "v", q.dtype, (N, HV, dv), dev)
    _need_opt(g, "g", torch.float32, (N, HV), dev)
    _need_opt(beta, "beta", torch.float32, (N, HV), dev)
    _need(S, "S", torch.float32, (N, HV, dk, dv), dev)
    if o is None:
        o = torch.empty((N, HV, dv), dtype=v.dtype, device=dev)
    _need(o, "o", v.dtype, (N, HV, dv), dev)
    var = _variant_code(variant)
    lib = load()
    ops = _block_ops(A_log, dt_bias, beta_logits, z, norm_w, norm_eps, v.dtype, alpha_sigmoid,
                     HV=HV, dv=dv, z_shape=(N, HV, dv), device=dev)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S), _ptr(o), N, HQK, HV, dk, dv,
            _dtype_code(q), float(scale))
    if ops is not None:
        _check(lib.gdn_decode_step_ex(*args, var, ctypes.byref(ops), _stream(q.device)))
    elif var == GDN_GATED_DELTA:
        _check(lib.gdn_decode_step(*args, _stream(q.device)))
    else:
        _check(lib.gdn_decode_step_v(*args, var, _stream(q.device)))
    return o


def _host_offsets(cu_seqlens_host, N: int):
    import numpy as np
    host = np.ascontiguousarray(np.asarray(cu_seqlens_host, dtype=np.int32))
    if host.shape != (N + 1,):
        raise ValueError("cu_seqlens_host must have N + 1 entries")
    return host


def prefill_workspace_size(N: int, total_T: int, HQK: int, HV: int, dk: int, dv: int,
                           dtype: torch.dtype, cu_seqlens_host=None) -> int:
    """Workspace bytes for these sizes; with the host lengths (N + 1 offsets), for the plan
    gdn_prefill takes given those lengths (gdn_prefill_workspace_size_lens)."""
    code = GDN_BF16 if dtype == torch.bfloat16 else GDN_F32
    if cu_seqlens_host is None:
        return int(load().gdn_prefill_workspace_size(N, total_T, HQK, HV, dk, dv, code))
    host = _host_offsets(cu_seqlens_host, N)
    return int(load().gdn_prefill_workspace_size_lens(N, total_T, host.ctypes.data, HQK, HV, dk, dv, code))


def prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: Optional[torch.Tensor],
            beta: Optional[torch.Tensor], *, cu_seqlens: Optional[torch.Tensor] = None,
            cu_seqlens_host=None, N: Optional[int] = None, S0: Optional[torch.Tensor] = None,
            scale: float = 1.0, o: Optional[torch.Tensor] = None,
            S_T: Optional[torch.Tensor] = None, output_state: bool = True,
            workspace: Optional[torch.Tensor] = None,
            variant="gated_delta", A_log=None, dt_bias=None, beta_logits: bool = False, z=None,
            norm_w=None, norm_eps: float = 1e-6,
            alpha_sigmoid: bool = False) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Whole sequences of a packed batch.

    q, k [total_T, HQK, dk]; v [total_T, HV, dv]; g, beta [total_T, HV] fp32.
    cu_seqlens: int32 device tensor [N + 1] (or None with N given: equal lengths).
    cu_seqlens_host: optional host copy (list / numpy / CPU tensor) for validation.
    S0 [N, HV, dk, dv] fp32 or None.  Returns (o [total_T, HV, dv], S_T or None).
    variant and the block parts: as for decode_step (z is [total_T, HV, dv]).
    """
    return _prefill(q, k, v, g, beta, cu_seqlens, cu_seqlens_host, N, S0, scale, o, S_T, output_state, workspace,
                    variant, A_log, dt_bias, beta_logits, z, norm_w, norm_eps, alpha_sigmoid, noalloc=False)


def prefill_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: Optional[torch.Tensor],
                    beta: Optional[torch.Tensor], *, cu_seqlens: Optional[torch.Tensor] = None,
                    cu_seqlens_host=None, N: Optional[int] = None, S0: Optional[torch.Tensor] = None,
                    scale: float = 1.0, o: torch.Tensor, S_T: Optional[torch.Tensor] = None,
                    variant="gated_delta", A_log=None, dt_bias=None, beta_logits: bool = False, z=None,
                    norm_w=None, norm_eps: float = 1e-6,
                    alpha_sigmoid: bool = False) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """prefill through gdn_prefill_noalloc: the library's static device scratch stands in for
    the workspace, so nothing is allocated (o and, if wanted, S_T are given by the caller)."""
    return _prefill(q, k, v, g, beta, cu_seqlens, cu_seqlens_host, N, S0, scale, o, S_T, False, None,
                    variant, A_log, dt_bias, beta_logits, z, norm_w, norm_eps, alpha_sigmoid, noalloc=True)


def _prefill(q, k, v, g, beta, cu_seqlens, cu_seqlens_host, N, S0, scale, o, S_T, output_state, workspace,
             variant, A_log, dt_bias, beta_logits, z, norm_w, norm_eps, alpha_sigmoid, *, noalloc):
    total_T, HQK, dk = _dims(q, "q", 3)
    _, HV, dv = _dims(v, "v", 3)
    dev = q.device
    _need(q, "q", q.dtype, device=dev)
    _need(k, "k", q.dtype, (total_T, HQK, dk), dev)
    _need(v, "v", q.dtype, (total_T, HV, dv), dev)
    _need_opt(g, "g", torch.float32, (total_T, HV), dev)
    _need_opt(beta, "beta", torch.float32, (total_T, HV), dev)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, device=dev)
        if cu_seqlens.dim() != 1 or cu_seqlens.shape[0] < 1:
            raise ValueError("cu_seqlens must be a 1-D tensor of N + 1 entries")
        n_seq = int(cu_seqlens.shape[0] - 1)
        if N is not None and int(N) != n_seq:
            raise ValueError(f"N = {N} but cu_seqlens has {n_seq + 1} entries")
    else:
        if N is None:
            raise ValueError("give cu_seqlens or N")
        n_seq = int(N)
    host = None if cu_seqlens_host is None else _host_offsets(cu_seqlens_host, n_seq)
    _need_opt(S0, "S0", torch.float32, (n_seq, HV, dk, dv), dev)
    if o is None:
        o = torch.empty((total_T, HV, dv), dtype=v.dtype, device=dev)
    _need(o, "o", v.dtype, (total_T, HV, dv), dev)
    if S_T is None and output_state:
        S_T = torch.empty((n_seq, HV, dk, dv), dtype=torch.float32, device=dev)
    _need_opt(S_T, "S_T", torch.float32, (n_seq, HV, dk, dv), dev)
    lib = load()
    code = _dtype_code(q)
    if noalloc:
        need = 0
    elif host is not None and cu_seqlens is not None:
        need = int(lib.gdn_prefill_workspace_size_lens(n_seq, total_T, host.ctypes.data, HQK, HV, dk, dv, code))
    else:
        need = int(lib.gdn_prefill_workspace_size(n_seq, total_T, HQK, HV, dk, dv, code))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _need(workspace, "workspace", device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    host_ptr = None if host is None else host.ctypes.data_as(ctypes.c_void_p)
    var = _variant_code(variant)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), host_ptr, n_seq, total_T,
            _ptr(S0), _ptr(o), _ptr(S_T), HQK, HV, dk, dv, code, float(scale))
    ops = _block_ops(A_log, dt_bias, beta_logits, z, norm_w, norm_eps, v.dtype, alpha_sigmoid,
                     HV=HV, dv=dv, z_shape=(total_T, HV, dv), device=dev)
    if noalloc:
        _check(lib.gdn_prefill_noalloc(*args, var, None if ops is None else ctypes.byref(ops), _stream(q.device)))
    elif ops is not None:
        _check(lib.gdn_prefill_ex(*args, var, ctypes.byref(ops), _ptr(workspace), ws_bytes,
                                  _stream(q.device)))
    elif var == GDN_GATED_DELTA:
        _check(lib.gdn_prefill(*args, _ptr(workspace), ws_bytes, _stream(q.device)))
    else:
        _check(lib.gdn_prefill_v(*args, var, _ptr(workspace), ws_bytes, _stream(q.device)))
    return o, S_T


def _host_seqlens(cu_seqlens_host, n_seq):
    if cu_seqlens_host is None:
        return None, None
    import numpy as np
    host = np.ascontiguousarray(np.asarray(cu_seqlens_host, dtype=np.int32))
    if host.shape[0] != n_seq + 1:
        raise ValueError("cu_seqlens_host must have N + 1 entries")
    return host, host.ctypes.data_as(ctypes.c_void_p)


def conv_silu(x: torch.Tensor, w: torch.Tensor, *, HQK: int, HV: int, dk: int, dv: int,
              cu_seqlens: Optional[torch.Tensor] = None, cu_seqlens_host=None, N: Optional[int] = None,
              state_in: Optional[torch.Tensor] = None, state_out: Optional[torch.Tensor] = None,
              q: Optional[torch.Tensor] = None, k: Optional[torch.Tensor] = None,
              v: Optional[torch.Tensor] = None):
    """Causal depthwise convolution (width 4) + SiLU of the concatenated q | k | v channels.

    x [total_T, 2 HQK dk + HV dv] (bf16 or fp32); w [Ctot, 4] fp32; state_in / state_out
    [N, 3, Ctot] in x's dtype (None: zeros / not written; they may be the same tensor).
    Returns (q [total_T, HQK, dk], k, v [total_T, HV, dv]) in x's dtype.
    """
    total_T, Ct = _dims(x, "x", 2)
    if Ct != 2 * HQK * dk + HV * dv:
        raise ValueError("x's width must be 2 HQK dk + HV dv")
    dev = x.device
    _need(x, "x", device=dev)
    code = _dtype_code(x)
    _need(w, "w", torch.float32, (Ct, 4), dev)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, device=dev)
        if cu_seqlens.dim() != 1 or cu_seqlens.shape[0] < 1:
            raise ValueError("cu_seqlens must be a 1-D tensor of N + 1 entries")
        n_seq = int(cu_seqlens.shape[0] - 1)
    else:
        if N is None:
            raise ValueError("give cu_seqlens or N")
        n_seq = int(N)
    _need_opt(state_in, "state_in", x.dtype, (n_seq, 3, Ct), dev)
    _need_opt(state_out, "state_out", x.dtype, (n_seq, 3, Ct), dev)
    q = torch.empty((total_T, HQK, dk), dtype=x.dtype, device=dev) if q is None else q
    k = torch.empty((total_T, HQK, dk), dtype=x.dtype, device=dev) if k is None else k
    v = torch.empty((total_T, HV, dv), dtype=x.dtype, device=dev) if v is None else v
    for t, nm, shp in ((q, "q", (total_T, HQK, dk)), (k, "k", (total_T, HQK, dk)), (v, "v", (total_T, HV, dv))):
        _need(t, nm, x.dtype, shp, dev)
    host, host_ptr = _host_seqlens(cu_seqlens_host, n_seq)
    _check(load().gdn_conv_silu(_ptr(x), _ptr(w), _ptr(cu_seqlens), host_ptr, n_seq, total_T, _ptr(state_in),
                                _ptr(state_out), _ptr(q), _ptr(k), _ptr(v), HQK, HV, dk, dv, code,
                                _stream(dev)))
    return q, k, v


def gated_rmsnorm(x: torch.Tensor, z: torch.Tensor, w: torch.Tensor, eps: float = 1e-6,
                  y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = w * x / sqrt(mean(x^2) + eps) * silu(z) over the last dimension (dv); y may be x."""
    dev = x.device
    _need(x, "x", device=dev)
    if x.dim() < 1:
        raise ValueError("x must have a last dimension (dv)")
    dv = x.shape[-1]
    _need(z, "z", x.dtype, tuple(x.shape), dev)
    _need(w, "w", torch.float32, (dv,), dev)
    y = torch.empty_like(x) if y is None else y
    _need(y, "y", x.dtype, tuple(x.shape), dev)
    _check(load().gdn_gated_rmsnorm(_ptr(x), _ptr(z), _ptr(w), float(eps), _ptr(y), x.numel() // max(dv, 1), dv,
                                    _dtype_code(x), _stream(x.device)))
    return y


def prefill_kernel_name(N: int, total_T: int, HQK: int, HV: int, dk: int, dv: int,
                        dtype: torch.dtype, cu_seqlens_host=None) -> str:
    """The kernel gdn_prefill runs, with the workspace prefill() allocates for these sizes
    (and host lengths, if given)."""
    code = GDN_BF16 if dtype == torch.bfloat16 else GDN_F32
    host = None if cu_seqlens_host is None else _host_offsets(cu_seqlens_host, N)
    ptr = None if host is None else host.ctypes.data
    return load().gdn_prefill_kernel_name(N, total_T, ptr, HQK, HV, dk, dv, code).decode()


def prefill_narrow_count(cu_seqlens_host, HQK: int, HV: int, dk: int, dv: int, dtype: torch.dtype) -> int:
    """How many sequences gdn_prefill runs on 32-column workgroups when it gets these host
    lengths (N + 1 offsets)."""
    import numpy as np
    host = np.ascontiguousarray(np.asarray(cu_seqlens_host, dtype=np.int32))
    if host.ndim != 1 or host.size < 2:
        raise ValueError("cu_seqlens_host must hold N + 1 offsets")
    code = GDN_BF16 if dtype == torch.bfloat16 else GDN_F32
    total_T = int(host[-1]) - int(host[0])
    return int(load().gdn_prefill_narrow_count(host.size - 1, total_T, host.ctypes.data, HQK, HV, dk, dv, code))


def version() -> int:
    return int(load().gdn_version())
