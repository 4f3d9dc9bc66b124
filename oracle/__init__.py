"""Float64 CPU oracle for the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The GPU library never imports, links or calls it,
and it imports nothing from the library: the two share no code.  Inputs reach
both sides from the seeded generators in
``gated_deltanet_recurrence_rule_amd.workloads`` (random draws only), or from the
tests themselves.

Three statements of the method live here, all float64:

* ``run`` -- the C token loop in ``gdn_oracle.c`` (OpenMP over independent
  (sequence, V head) units).  This is THE oracle.
* ``delta_rule_np`` -- the same rule stated a second way, in [LLV]'s transposed
  form (the table multiplied by alpha (I - beta k k^T) each token), used to
  catch mistakes in the C code.
* ``chunked_np`` -- the chunk-parallel rewriting of the same recurrence, used
  only to pin the algebra that the GPU prefill implements (the handbook page
  says that real implementations split the sequence into chunks and are
  mathematically equivalent to the loop; it gives no formulas, so they are
  derived in that function's docstring).

``oracle/shell.py`` states, in float64 as well, the parts of the GatedDeltaNet
block that touch only the scan's inputs or output (the gates from raw
projections, the short causal convolution + SiLU, the gated RMS norm).

Sources: [HB7] handbook page "7. Gated DeltaNet: the token-by-token recurrence"
(anrans.github.io/ai-infra-handbooks/en/transformer/deltanet/, and its Chinese
twin); [LLV] learn-llm page 13_linear_attention_viz (learn-llm.fim.ai).

Parity unpinned: the value of the normalisation floor eps (1e-12, the documented
default of torch.nn.functional.normalize named by [LLV]) -- the pages never show
it and no printed example exercises it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn_oracle.so")
SRC_PATH = os.path.join(_HERE, "gdn_oracle.c")
EPS = 1e-12

_lib = None


def build(force: bool = True) -> str:
    """Compile gdn_oracle.c with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-Wall",
                               SRC_PATH, "-o", tmp, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        lib = ctypes.CDLL(LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        lib.gdn_oracle_run.argtypes = [dp, dp, dp, dp, dp, ctypes.POINTER(i64), i64, dp, dp, dp,
                                       i64, i64, i64, i64, ctypes.c_double, ctypes.c_int,
                                       ctypes.c_int]
        lib.gdn_oracle_run.restype = ctypes.c_int
        lib.gdn_oracle_threads.argtypes = []
        lib.gdn_oracle_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def threads() -> int:
    """OpenMP threads the C oracle uses."""
    return int(_load().gdn_oracle_threads())


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def run(q, k, v, g, beta, cu_seqlens, S0=None, *, scale=1.0, delta=True, normalize=True):
    """Token-loop oracle (C, float64).

    q, k [total_T, HQK, dk]; v [total_T, HV, dv]; g, beta [total_T, HV];
    cu_seqlens [N + 1]; S0 [N, HV, dk, dv] or None (zeros).
    Returns (o [total_T, HV, dv], S_T [N, HV, dk, dv]) as float64.
    """
    q, k, v, g, beta, S0 = (_f64(x) for x in (q, k, v, g, beta, S0))
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    T, HQK, dk = q.shape
    HV, dv = v.shape[1], v.shape[2]
    N = cu.shape[0] - 1
    if k.shape != q.shape or v.shape[0] != T or g.shape != (T, HV) or beta.shape != (T, HV):
        raise ValueError("inconsistent shapes")
    if N > 0 and cu[-1] != T:
        raise ValueError("cu_seqlens[-1] must equal total_T")
    if S0 is not None and S0.shape != (N, HV, dk, dv):
        raise ValueError("S0 shape")
    o = np.zeros((T, HV, dv), dtype=np.float64)
    S_T = np.zeros((N, HV, dk, dv), dtype=np.float64)
    rc = _load().gdn_oracle_run(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), N, _ptr(S0),
                                _ptr(o), _ptr(S_T), HQK, HV, dk, dv, float(scale), int(delta),
                                int(normalize))
    if rc != 0:
        raise ValueError(f"gdn_oracle_run failed ({rc})")
    return o, S_T


def run_inputs(inp, *, S0="inputs", delta=True, normalize=True, scale=None):
    """Oracle on a ``workloads.Inputs`` batch (bf16 values widened exactly)."""
    s0 = inp.as_f64("S0") if isinstance(S0, str) else S0
    return run(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"), inp.as_f64("g"),
               inp.as_f64("beta"), inp.cu_seqlens, s0,
               scale=inp.scale if scale is None else scale, delta=delta, normalize=normalize)


# --------------------------------------------------------------------------- numpy twin
def _unit(x, normalize):
    if not normalize:
        return x
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, EPS)


def delta_rule_np(q, k, v, g, beta, S0=None, *, scale=1.0, delta=True, normalize=True):
    """One sequence, numpy float64: q, k [T, HQK, dk]; v [T, HV, dv]; g, beta [T, HV].

    A second, independent statement of the rule, checked against the C token loop: the
    transposed form that [LLV] gives in its update-rule table (Gated DeltaNet row), where
    the table is M = S^T [dv, dk] and every token multiplies it on the right by the matrix
    alpha (I - beta k k^T) -- a decay together with a projection away from k -- before
    adding the new association beta v k^T:

        M_t = M_{t-1} (alpha_t (I - beta_t k_t k_t^T)) + beta_t v_t k_t^T,   o_t = M_t q_t.

    Without the look-up (delta=False) the projection drops out: M_t = alpha_t M_{t-1} +
    beta_t v_t k_t^T.  V head h reads QK head h // (HV // HQK).  Each head runs its own
    explicit loop over tokens.  Returns (o [T, HV, dv], S [HV, dk, dv]) in [HB7]'s
    orientation (S = M^T).
    """
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    T, HQK, dk = q.shape
    HV, dv = v.shape[1:]
    group = HV // HQK
    o = np.zeros((T, HV, dv))
    S_out = np.zeros((HV, dk, dv))
    eye = np.eye(dk)
    for h in range(HV):
        hq = h // group
        M = np.zeros((dv, dk)) if S0 is None else np.array(S0[h], dtype=np.float64).T
        for t in range(T):
            key = _unit(k[t, hq], normalize)
            query = scale * _unit(q[t, hq], normalize)
            alpha = np.exp(g[t, h])
            if delta:
                M = M @ (alpha * (eye - beta[t, h] * np.outer(key, key))) + beta[t, h] * np.outer(v[t, h], key)
            else:
                M = alpha * M + beta[t, h] * np.outer(v[t, h], key)
            o[t, h] = M @ query
        S_out[h] = M.T
    return o, S_out


# --------------------------------------------------------------------------- chunked form
def chunked_np(q, k, v, g, beta, S0=None, *, C=64, scale=1.0):
    """One sequence, float64, the recurrence rewritten over chunks of C tokens.

    Derivation (from [HB7] "The formula"; the pages only say that chunked
    implementations exist and equal the loop).  Inside one chunk with start
    state S_0 and tokens i = 1..n, let G_i = g_1 + ... + g_i, gamma_i = exp(G_i),
    and delta_i = beta_i (v_i - a_i S_{i-1}^T k_i).  Then S_i = a_i S_{i-1} + k_i delta_i^T,
    so by induction

        S_r = gamma_r S_0 + sum_{i<=r} exp(G_r - G_i) k_i delta_i^T,

    and substituting a_i S_{i-1} into delta_i gives a unit lower-triangular system

        (I + A) Delta = diag(beta) (V - diag(gamma) K S_0),
        A_ij = beta_i exp(G_i - G_j) (k_i . k_j)   for j < i (zero otherwise).

    With T = (I + A)^{-1}: Delta = U - W S_0, U = T diag(beta) V,
    W = T diag(beta gamma) K.  The outputs and the next chunk's start state are

        O   = diag(gamma) Q S_0 + P Delta,  P_ri = exp(G_r - G_i) (q_r . k_i), i <= r,
        S_n = gamma_n S_0 + K^T diag(exp(G_n - G_i)) Delta.

    Here the triangular system is solved by numpy's dense solver.
    """
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    T, HQK, dk = q.shape
    HV, dv = v.shape[1:]
    rep = HV // HQK
    kh = np.repeat(_unit(k, True), rep, axis=1)
    qh = np.repeat(_unit(q, True) * scale, rep, axis=1)
    S = np.zeros((HV, dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, HV, dv))
    for h in range(HV):
        Sh = S[h]
        for c0 in range(0, T, C):
            c1 = min(T, c0 + C)
            K, Q, V = kh[c0:c1, h], qh[c0:c1, h], v[c0:c1, h]
            b = beta[c0:c1, h]
            G = np.cumsum(g[c0:c1, h])
            gam = np.exp(G)
            decay = np.exp(G[:, None] - G[None, :])          # exp(G_i - G_j)
            lower = np.tril(np.ones((c1 - c0, c1 - c0)), -1)
            A = lower * decay * (K @ K.T) * b[:, None]
            rhs = b[:, None] * (V - gam[:, None] * (K @ Sh))
            Delta = np.linalg.solve(np.eye(c1 - c0) + A, rhs)
            P = np.tril(decay * (Q @ K.T))
            o[c0:c1, h] = gam[:, None] * (Q @ Sh) + P @ Delta
            Sh = gam[-1] * Sh + K.T @ (np.exp(G[-1] - G)[:, None] * Delta)
        S[h] = Sh
    return o, S


# --------------------------------------------------------------------------- tolerances
def v_norm(v) -> float:
    """RMS per-vector norm of v over all (token, head) vectors: the scale of the output gate."""
    v = np.asarray(v, dtype=np.float64)
    if v.size == 0:
        return 1.0
    return float(np.sqrt(np.mean(np.sum(v * v, axis=-1))))
