"""Seeded synthetic inputs for the gated delta-rule scan.

This module only draws random numbers and lays them out; it holds none of the
recurrence's arithmetic.  Both the HIP path (tests, bench) and the float64
oracle receive exactly the arrays made here, so the two sides always see the
same values.

Shapes and distributions follow the five workloads the library is measured on:

  tiny       fp32, N=1, T=64, 4 heads, dk=dv=32, S0 = none
  decode     bf16, N=256 sequences, 16 QK / 32 V heads, dk=dv=128, one token,
             fp32 state S ~ N(0, 0.05) updated in place (512 MiB)
  prefill    bf16, N=1, T=8192, 16 heads, dk=dv=128, S0 = none
  qwen3next  bf16, N=4, T=16384, 16 QK / 32 V heads, dk=dv=128, S0 ~ N(0, 0.05)
  varlen     bf16, 64 sequences with log-uniform lengths in [128, 32768] plus one
             sequence of 262144 tokens; 16 QK / 32 V heads; 10% of tokens have
             g = 0 and (independently) 10% have beta = 1

Recipe shared by all of them: q, k ~ N(0, 1), each (token, head) vector scaled to
unit L2 norm in float32 (the workloads state that q and k arrive normalised);
v ~ N(0, 1); g = log(sigmoid(x)) with x ~ N(mu, sd), so alpha = exp(g) lies in
(0, 1]; beta = sigmoid(N(0, 1)).  bf16 values are fp32 draws rounded to nearest
even.  The head shapes (dk = dv = 128, 16 QK heads shared by 32 V heads) are the
Qwen3-Next layer quoted on the learn-llm page "13_linear_attention_viz"
(hybrid-layout widget); the gate ranges follow the handbook page
"7. Gated DeltaNet: the token-by-token recurrence" (section "Run it", gate
ranges measured on real input) and the learn-llm page's note that the gate bias
starts at 3.0 (alpha ~ 0.95).
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
from typing import Optional

import numpy as np

BF16 = "bf16"
F32 = "f32"


# ---------------------------------------------------------------- bf16 helpers
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return raw uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen raw bfloat16 bits to float32 exactly."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------- containers
@dataclasses.dataclass
class Inputs:
    """One batch of packed inputs.

    Layout (row-major, last index fastest):
      q, k   [total_T, HQK, dk]   raw bf16 bits (uint16) or float32
      v      [total_T, HV, dv]    raw bf16 bits (uint16) or float32
      g, beta[total_T, HV]        float32 (log-decay <= 0, write strength in [0, 1])
      cu_seqlens [N + 1] int32    sequence i owns tokens [cu[i], cu[i+1])
      S0     [N, HV, dk, dv] float32 or None
    """

    name: str
    dtype: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    cu_seqlens: np.ndarray
    S0: Optional[np.ndarray]
    HQK: int
    HV: int
    dk: int
    dv: int
    scale: float = 1.0

    @property
    def N(self) -> int:
        return int(self.cu_seqlens.shape[0] - 1)

    @property
    def total_T(self) -> int:
        return int(self.cu_seqlens[-1])

    def as_f64_rows(self, name: str, t0: int, t1: int) -> np.ndarray:
        """Exact values of tokens [t0, t1) of q, k or v, widened to float64."""
        a = getattr(self, name)[t0:t1]
        if a.dtype == np.uint16:
            a = bf16_bits_to_f32(a)
        return a.astype(np.float64)

    def as_f64(self, name: str) -> np.ndarray:
        """The exact values of one input tensor, widened to float64."""
        a = getattr(self, name)
        if a is None:
            return None
        if a.dtype == np.uint16:
            a = bf16_bits_to_f32(a)
        return a.astype(np.float64)


# ---------------------------------------------------------------- draws
# Large arrays are drawn in row blocks, each from its own generator seeded by
# (seed, array id, block index), so the values do not depend on how many
# threads fill them.
_BLOCK_ELEMS = 1 << 21
_THREADS = max(1, min(16, os.cpu_count() or 1))


def _block_rng(seed: int, array_id: int, block: int) -> np.random.Generator:
    return np.random.default_rng([seed, array_id, block])


def _fill_blocks(seed: int, array_id: int, shape, out_dtype, make):
    """out[rows of block b] = make(rng_b, block_shape) for every block, in parallel."""
    shape = tuple(int(x) for x in shape)
    out = np.empty(shape, dtype=out_dtype)
    rows = shape[0]
    per_row = int(np.prod(shape[1:], dtype=np.int64)) if len(shape) > 1 else 1
    brows = max(1, _BLOCK_ELEMS // max(1, per_row))
    nblk = (rows + brows - 1) // brows

    def job(b):
        r0, r1 = b * brows, min(rows, (b + 1) * brows)
        out[r0:r1] = make(_block_rng(seed, array_id, b), (r1 - r0,) + shape[1:])

    if nblk <= 1:
        for b in range(nblk):
            job(b)
    else:
        with concurrent.futures.ThreadPoolExecutor(max_workers=_THREADS) as ex:
            list(ex.map(job, range(nblk)))
    return out


def _unit_rows(rng: np.random.Generator, shape) -> np.ndarray:
    """Standard-normal vectors (last axis) scaled to unit length in float32."""
    x = rng.standard_normal(shape, dtype=np.float32)
    flat = x.reshape(-1, shape[-1])
    n = np.sqrt(np.einsum("ij,ij->i", flat, flat))[:, None]
    flat /= np.maximum(n, np.float32(1e-12))
    return x


@dataclasses.dataclass(frozen=True)
class NormSpread:
    """How q and k rows are scaled after being drawn unit-norm: each (token, head) row gets
    a norm log-uniform in [lo, hi]; a fraction p_zero of the rows is set to zero, and a
    fraction p_tiny is given the norm `tiny` (below the library's 1e-12 floor)."""
    lo: float = 1e-2
    hi: float = 1e2
    p_zero: float = 0.05
    p_tiny: float = 0.02
    tiny: float = 1e-13


def _spread_rows(rng: np.random.Generator, shape, spread: NormSpread) -> np.ndarray:
    """Unit rows (see _unit_rows) times random per-row norms drawn as `spread` says."""
    x = _unit_rows(rng, shape)
    rows = int(np.prod(shape[:-1], dtype=np.int64))
    norm = np.exp(rng.uniform(math.log(spread.lo), math.log(spread.hi), size=rows)).astype(np.float32)
    u = rng.random(rows)
    norm[u < spread.p_zero] = 0.0
    norm[(u >= spread.p_zero) & (u < spread.p_zero + spread.p_tiny)] = np.float32(spread.tiny)
    x.reshape(rows, shape[-1])[:] *= norm[:, None]
    return x


def _log_sigmoid(x: np.ndarray) -> np.ndarray:
    # log(sigmoid(x)) = -log1p(exp(-x)), written to stay finite for any x
    x = x.astype(np.float64)
    return (np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))).astype(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def _pack(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == BF16 else np.ascontiguousarray(x, dtype=np.float32)


def make_inputs(name: str, seed: int, seqlens, HQK: int, HV: int, dk: int, dv: int, dtype: str,
                g_mu: float, g_sd: float, s0_sd: Optional[float], p_g0: float = 0.0,
                p_beta1: float = 0.0, scale: float = 1.0,
                qk_spread: Optional[NormSpread] = None) -> Inputs:
    """Draw one packed batch with the shared recipe (see the module docstring).

    qk_spread: None keeps q and k unit-norm (the workloads' statement); a NormSpread
    scales their rows instead, for tests of the library's own normalisation."""
    seqlens = np.asarray(seqlens, dtype=np.int64)
    cu = np.zeros(len(seqlens) + 1, dtype=np.int64)
    np.cumsum(seqlens, out=cu[1:])
    if cu[-1] >= 2**31:
        raise ValueError("total length exceeds int32 cu_seqlens")
    T = int(cu[-1])
    io = np.uint16 if dtype == BF16 else np.float32
    rows = _unit_rows if qk_spread is None else (lambda r, s: _spread_rows(r, s, qk_spread))
    q = _fill_blocks(seed, 0, (T, HQK, dk), io, lambda r, s: _pack(rows(r, s), dtype))
    k = _fill_blocks(seed, 1, (T, HQK, dk), io, lambda r, s: _pack(rows(r, s), dtype))
    v = _fill_blocks(seed, 2, (T, HV, dv), io,
                     lambda r, s: _pack(r.standard_normal(s, dtype=np.float32), dtype))
    g = _fill_blocks(seed, 3, (T, HV), np.float32,
                     lambda r, s: _log_sigmoid(r.normal(g_mu, g_sd, size=s).astype(np.float32)))
    beta = _fill_blocks(seed, 4, (T, HV), np.float32,
                        lambda r, s: _sigmoid(r.standard_normal(s, dtype=np.float32)))
    rng = np.random.default_rng([seed, 5])
    if p_g0 > 0.0:
        g[rng.random(T) < p_g0, :] = 0.0
    if p_beta1 > 0.0:
        beta[rng.random(T) < p_beta1, :] = 1.0
    S0 = None
    if s0_sd is not None and len(seqlens) > 0:
        S0 = _fill_blocks(seed, 6, (len(seqlens) * HV, dk, dv), np.float32,
                          lambda r, s: r.standard_normal(s, dtype=np.float32) * np.float32(s0_sd))
        S0 = S0.reshape(len(seqlens), HV, dk, dv)
    return Inputs(name, dtype, q, k, v, g, beta, cu.astype(np.int32), S0, HQK, HV, dk, dv, scale)


def varlen_lengths(seed: int = 5, n: int = 64, lo: int = 128, hi: int = 32768, tail: int = 262144):
    """64 lengths log-uniform in [lo, hi] (rounded), then one long sequence appended last."""
    rng = np.random.default_rng(seed + 1000)
    lens = np.round(np.exp(rng.uniform(math.log(lo), math.log(hi), size=n))).astype(np.int64)
    return list(lens) + ([tail] if tail else [])


# ---------------------------------------------------------------- named workloads
def tiny(seed: int = 1) -> Inputs:
    """fp32, N=1, T=64, 4 heads (no sharing), dk=dv=32, S0 = none, alpha ~ 0.95."""
    return make_inputs("tiny", seed, [64], 4, 4, 32, 32, F32, 3.0, 1.0, None)


def decode(seed: int = 2, N: int = 256, HQK: int = 16, HV: int = 32, d: int = 128,
           dtype: str = BF16) -> Inputs:
    """One decode token for N sequences; state S ~ N(0, 0.05) passed as S0 (updated in place)."""
    return make_inputs("decode", seed, [1] * N, HQK, HV, d, d, dtype, 3.0, 1.0, 0.05)


def prefill(seed: int = 3, T: int = 8192, H: int = 16, d: int = 128, dtype: str = BF16) -> Inputs:
    """Single sequence, HQK = HV = H, S0 = none, g = log sigmoid(N(2, 1.5))."""
    return make_inputs("prefill", seed, [T], H, H, d, d, dtype, 2.0, 1.5, None)


def qwen3next(seed: int = 4, N: int = 4, T: int = 16384, HQK: int = 16, HV: int = 32, d: int = 128,
              dtype: str = BF16) -> Inputs:
    """N sequences of T tokens, 16 QK heads shared by 32 V heads, S0 ~ N(0, 0.05)."""
    return make_inputs("qwen3next", seed, [T] * N, HQK, HV, d, d, dtype, 2.0, 1.5, 0.05)


def varlen(seed: int = 5, n: int = 64, lo: int = 128, hi: int = 32768, tail: int = 262144,
           HQK: int = 16, HV: int = 32, d: int = 128, dtype: str = BF16) -> Inputs:
    """Packed variable-length batch with 10% alpha=1 tokens and 10% beta=1 tokens."""
    lens = varlen_lengths(seed, n, lo, hi, tail)
    return make_inputs("varlen", seed, lens, HQK, HV, d, d, dtype, 2.0, 1.5, 0.05,
                       p_g0=0.1, p_beta1=0.1)


def random_small(seed: int, seqlens, HQK: int, HV: int, dk: int, dv: int, dtype: str = BF16,
                 s0: bool = True, g_mu: float = 2.0, g_sd: float = 1.5, p_g0: float = 0.0,
                 p_beta1: float = 0.0, qk_spread: Optional[NormSpread] = None,
                 scale: float = 1.0) -> Inputs:
    """Small random batch for parity tests (any lengths, including zero)."""
    return make_inputs("random", seed, seqlens, HQK, HV, dk, dv, dtype, g_mu, g_sd,
                       0.05 if s0 else None, p_g0=p_g0, p_beta1=p_beta1, qk_spread=qk_spread,
                       scale=scale)


# ---------------------------------------------------------------- the block around the scan
@dataclasses.dataclass
class BlockInputs:
    """Raw inputs of the GatedDeltaNet block's parts around the scan.

      x          [total_T, 2 HQK dk + HV dv]  concatenated q | k | v channels before the
                                              short convolution (bf16 bits or float32)
      conv_w     [Ctot, 4] float32            convolution weights, column 3 = current token
      conv_state [N, 3, Ctot] or None         the three inputs before each sequence
      a, b       [total_T, HV] float32        raw decay / write-strength projections
      A_log, dt_bias [HV] float32             per-head decay parameters
      z          [total_T, HV, dv]            output gate (bf16 bits or float32)
      norm_w     [dv] float32                 gated-norm weight
    """

    dtype: str
    x: np.ndarray
    conv_w: np.ndarray
    conv_state: Optional[np.ndarray]
    a: np.ndarray
    b: np.ndarray
    A_log: np.ndarray
    dt_bias: np.ndarray
    z: np.ndarray
    norm_w: np.ndarray
    cu_seqlens: np.ndarray
    HQK: int
    HV: int
    dk: int
    dv: int

    def as_f64(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        if a is None:
            return None
        if a.dtype == np.uint16:
            a = bf16_bits_to_f32(a)
        return a.astype(np.float64)


def block_inputs(seed: int, seqlens, HQK: int, HV: int, dk: int, dv: int, dtype: str = BF16,
                 conv_state: bool = True) -> BlockInputs:
    """Synthetic raw projections and block parameters.

    Recipe: x, z ~ N(0, 1); conv weights ~ U(-0.5, 0.5) (the default initialisation range
    of a width-4 depthwise convolution); a, b ~ N(0, 1); exp(A_log) ~ U(0.01, 1.3) (the
    handbook page "7. Gated DeltaNet: the token-by-token recurrence", section "Run it",
    prints per-head forgetting speeds exp(A_log) from 0.00 to 1.29); dt_bias ~ N(1, 0.5)
    around the block's initial value 1; norm weight 1 + N(0, 0.1) around its initial 1;
    conv state ~ N(0, 1).
    """
    seqlens = np.asarray(seqlens, dtype=np.int64)
    cu = np.zeros(len(seqlens) + 1, dtype=np.int64)
    np.cumsum(seqlens, out=cu[1:])
    T, N = int(cu[-1]), len(seqlens)
    Ct = 2 * HQK * dk + HV * dv
    io = np.uint16 if dtype == BF16 else np.float32
    normal = lambda r, s: _pack(r.standard_normal(s, dtype=np.float32), dtype)
    x = _fill_blocks(seed, 10, (T, Ct), io, normal)
    z = _fill_blocks(seed, 11, (T, HV, dv), io, normal)
    a = _fill_blocks(seed, 12, (T, HV), np.float32, lambda r, s: r.standard_normal(s, dtype=np.float32))
    b = _fill_blocks(seed, 13, (T, HV), np.float32, lambda r, s: r.standard_normal(s, dtype=np.float32))
    rng = np.random.default_rng([seed, 14])
    conv_w = rng.uniform(-0.5, 0.5, size=(Ct, 4)).astype(np.float32)
    A_log = np.log(rng.uniform(0.01, 1.3, size=HV)).astype(np.float32)
    dt_bias = rng.normal(1.0, 0.5, size=HV).astype(np.float32)
    norm_w = (1.0 + rng.normal(0.0, 0.1, size=dv)).astype(np.float32)
    st = _fill_blocks(seed, 15, (N, 3, Ct), io, normal) if conv_state and N > 0 else None
    return BlockInputs(dtype, x, conv_w, st, a, b, A_log, dt_bias, z, norm_w, cu.astype(np.int32),
                       HQK, HV, dk, dv)
