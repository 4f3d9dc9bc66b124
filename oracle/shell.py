"""Float64 CPU oracle for the work around the scan -- TEST INFRASTRUCTURE ONLY.

Like the rest of ``oracle/``, only the test suite, ``__graft_entry__.smoke()``
and the benchmark's CPU-baseline leg may use this module; the GPU library never
imports or calls it and it imports nothing from the library.

The handbook page "7. Gated DeltaNet: the token-by-token recurrence" ([HB7])
shows the GatedDeltaNet block that wraps the delta rule (its listing of the
block's forward pass and the table of the block's parts that follows it).
Three of those parts touch only the scan's inputs or its output, and they are
stated here in float64, in the order the page applies them:

* ``gates_np``        -- the decay and write-strength gates from their raw
                         projections: g = -exp(A_log) softplus(a + dt_bias),
                         beta = sigmoid(b)  ([HB7] table row "in_proj_a, dt_bias,
                         A_log" and row "in_proj_b -> sigmoid"); or, as the
                         learn-llm page 13_linear_attention_viz ([LLV]) describes
                         its RecurrentMixer (an a projection with a bias started at
                         3.0, so that alpha = sigmoid(3) ~ 0.95 at the start of
                         training), alpha = sigmoid(a + bias), i.e.
                         g = log sigmoid(a + bias).
* ``conv_silu_np``    -- the depthwise causal short convolution (window 4,
                         every channel on its own) followed by SiLU, on the
                         concatenated q | k | v channels ([HB7] table row
                         "in_proj_qkv + conv1d" and the note under the table:
                         the output at position t uses inputs t-3 .. t).
* ``gated_rmsnorm_np`` -- the per-head RMS normalisation of the read, scaled by
                         a per-channel weight and multiplied by silu(z) ([HB7]
                         table row "in_proj_z + GatedRMSNorm").

Readings (the page leaves these open):
* GatedRMSNorm's body is not shown.  Taken: y = w * o / sqrt(mean(o^2) + eps)
  * silu(z) over each head's dv values, w of length dv shared by all heads (the
  block builds it as GatedRMSNorm(dv, eps)); normalise first, then gate, as the
  table row says.  eps is an argument.
* The convolution's carried state: the last three inputs of each sequence
  (oldest first), zeros for a fresh sequence -- what the page's zero padding of
  width 3 gives at the start of a sequence.
* Rounding: where the GPU path hands a bf16 tensor from one kernel to the next
  (the convolution's outputs feed the scan as bf16 q, k, v), ``round_bf16`` rounds
  the float64 value to the nearest bfloat16, ties to even.

Parity unpinned: the GatedRMSNorm reading above (order of weight and gate, the
weight's shape) -- the page names the operation without its formula.
"""
from __future__ import annotations

import numpy as np

CONV_WIDTH = 4  # [HB7]: window of 4, each position sees itself and the previous 3 tokens


def softplus(x):
    """log(1 + exp(x)) in float64 without overflow."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x * sigmoid(x)


def gates_np(a, b, A_log, dt_bias, *, alpha_sigmoid=False):
    """Raw projections a, b [T, HV] and per-head A_log, dt_bias [HV] -> (g, beta) [T, HV].

    [HB7] block listing / parts table: g = -exp(A_log) * softplus(a + dt_bias) (always
    <= 0, so the decay exp(g) lies in (0, 1]); beta = sigmoid(b).
    alpha_sigmoid=True ([LLV] RecurrentMixer): alpha = sigmoid(a + dt_bias), so
    g = log sigmoid(a + dt_bias) = -softplus(-(a + dt_bias)); A_log is not used.
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    dt_bias = np.asarray(dt_bias, dtype=np.float64)
    if alpha_sigmoid:
        g = -softplus(-(a + dt_bias[None, :]))
    else:
        A_log = np.asarray(A_log, dtype=np.float64)
        g = -np.exp(A_log)[None, :] * softplus(a + dt_bias[None, :])
    return g, sigmoid(b)


def conv_silu_np(x, w, cu_seqlens, state=None, *, act=True):
    """Depthwise causal convolution of width 4 + SiLU over a packed batch.

    x [T, C] (the concatenated q | k | v channels of every token); w [C, 4] with
    w[c, 3] the weight of the current token and w[c, 0] of the token three back;
    cu_seqlens [N + 1]; state [N, 3, C] = the three inputs before each sequence
    (oldest first) or None for zeros.

    For token t of sequence n, with e the sequence's inputs prefixed by its state,
        y[t, c] = silu( sum_{j=0..3} w[c, j] * e[t - 3 + j, c] )
    ([HB7]: the convolution pads 3 positions and keeps the first T outputs, so
    position t sees inputs t-3 .. t only; every channel has its own 4 weights).
    act=False returns the sum before the SiLU.

    Returns (y [T, C], state_out [N, 3, C] = the last three entries of e).
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, C = x.shape
    N = cu.shape[0] - 1
    if w.shape != (C, CONV_WIDTH):
        raise ValueError("w must be [C, 4]")
    st = np.zeros((N, CONV_WIDTH - 1, C)) if state is None else np.asarray(state, dtype=np.float64)
    y = np.zeros((T, C))
    st_out = np.zeros((N, CONV_WIDTH - 1, C))
    for n in range(N):
        t0, t1 = int(cu[n]), int(cu[n + 1])
        e = np.concatenate([st[n], x[t0:t1]], axis=0)  # e[i] = input at position i - 3
        for i in range(t1 - t0):
            acc = np.zeros(C)
            for j in range(CONV_WIDTH):
                acc = acc + w[:, j] * e[i + j]
            y[t0 + i] = silu(acc) if act else acc
        st_out[n] = e[-(CONV_WIDTH - 1):]
    return y, st_out


def gated_rmsnorm_np(o, z, w, eps):
    """o, z [..., dv]; w [dv]: y = w * o / sqrt(mean(o^2) + eps) * silu(z) per head vector."""
    o = np.asarray(o, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    ms = np.mean(o * o, axis=-1, keepdims=True)
    return w * (o / np.sqrt(ms + eps)) * silu(z)


BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127  # largest finite bfloat16


def round_bf16(x):
    """Round float64 values to the nearest bfloat16, ties to even; returned as float64.

    bfloat16 keeps 8 significant bits over float32's exponent range.  A value x with
    x = m 2^e, 0.5 <= |m| < 1, lies among bfloat16 numbers spaced 2^(e - 8) apart; below
    the normal range (e <= -126) the spacing stays at that of the subnormals, 2^-133.  So
    x rounds to rint(x / s) s with s = 2^(max(e, -125) - 8), rint taking halves to even
    (the parity of the count of steps is the parity of the last stored bit).  A result
    beyond the largest finite bfloat16 -- which happens from the midpoint
    (2 - 2^-8) 2^127 up, ties going to the even neighbour 2^128 -- is an infinity of the
    same sign.  NaN and infinities pass through.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, dtype=np.float64, copy=True)
    fin = np.isfinite(x)
    xf = x[fin]
    _, e = np.frexp(xf)
    step = np.ldexp(1.0, np.maximum(e, -125) - 8)
    r = np.rint(xf / step) * step
    r = np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, xf), r)
    out[fin] = r
    return out if out.ndim else out[()]
