"""Helpers shared by the test modules: golden-fixture readers and tolerance checks."""
import os

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def golden_path(name):
    return os.path.join(ROOT, "tests", "golden", name)


def read_golden_kv(name):
    out = {}
    with open(golden_path(name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            out[key] = [float(x) for x in val.split()]
    return out


def read_golden_rows(name):
    rows = []
    with open(golden_path(name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------- device transfer
def to_device(inp, device="cuda"):
    """Upload a workloads.Inputs batch; bf16 bits are reinterpreted, never re-rounded."""
    import torch

    def tok(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)

    d = dict(q=tok(inp.q), k=tok(inp.k), v=tok(inp.v),
             g=torch.from_numpy(inp.g).to(device), beta=torch.from_numpy(inp.beta).to(device),
             cu=torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(device))
    d["S0"] = None if inp.S0 is None else torch.from_numpy(inp.S0).to(device)
    return d


def to_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


# ---------------------------------------------------------------- parity gate
# Achieved errors of every assert_parity call, keyed by the running test: the session
# summary (conftest.py) prints the worst of each test beside its gate.
PARITY_LOG = {}


def _log_parity(dtype, err_o_rel, err_s):
    """err_o_rel / err_s: None where the call compared no reads / no table."""
    key = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    rec = PARITY_LOG.setdefault(key, {"dtype": dtype, "o": None, "s": None, "units": 0})
    for name, val in (("o", err_o_rel), ("s", err_s)):
        if val is not None:
            rec[name] = val if rec[name] is None else max(rec[name], val)
    rec["units"] += 1


def tolerances(dtype):
    """(output max-abs factor on |v|, state relative Frobenius bound)."""
    return (2e-3, 1e-3) if dtype == "bf16" else (1e-5, 1e-5)


def assert_parity(o, S, o_ref, S_ref, v_ref, dtype, what="", grows=False):
    """bf16 inputs: max|o - o_ref| <= 2e-3 |v| and |S - S_ref|_F / |S_ref|_F <= 1e-3;
    fp32 inputs: both bounds 1e-5.  |v| is the RMS per-vector norm of v.

    grows=True (the rules without the look-up, whose table and reads grow with the
    sequence): the output bound is taken relative to the larger of |v| and the RMS
    per-vector norm of the oracle's reads, since the kernel's rounding errors scale with
    the table it reads from."""
    import oracle

    fo, fs = tolerances(dtype)
    vn = oracle.v_norm(v_ref)
    if grows and o_ref.size:
        vn = max(vn, oracle.v_norm(o_ref))
    err_o = float(np.abs(o - o_ref).max()) if o_ref.size else None
    err_s = None
    if S_ref is not None and S_ref.size:
        den = float(np.linalg.norm(S_ref))
        err_s = float(np.linalg.norm(S - S_ref)) / max(den, 1e-30)
    _log_parity(dtype, None if err_o is None else err_o / max(vn, 1e-30), err_s)
    if err_o is not None:
        assert np.isfinite(o).all(), f"{what}: non-finite output"
        assert err_o <= fo * vn, f"{what}: output max-abs error {err_o:.3e} > {fo * vn:.3e}"
    if err_s is not None:
        assert err_s <= fs, f"{what}: state relative Frobenius error {err_s:.3e} > {fs:.1e}"


def rows_f64(a):
    """Exact float64 values of raw bf16 bits (uint16) or float32 rows."""
    from gated_deltanet_recurrence_rule_amd.workloads import bf16_bits_to_f32

    if a.dtype == np.uint16:
        a = bf16_bits_to_f32(a)
    return a.astype(np.float64)


def oracle_units(inp, seqs, heads):
    """Oracle on a subset of (sequence, V head) units of a batch.

    Each selected V head gets its own copy of its QK head, so the subset runs as
    an ungrouped batch.  Returns {(seq, head): (o [len, dv], S_T [dk, dv])}.
    """
    import oracle

    rep = inp.HV // inp.HQK
    heads = list(heads)
    qk_idx = [h // rep for h in heads]
    out = {}
    S0 = inp.S0
    for n in seqs:
        t0, t1 = int(inp.cu_seqlens[n]), int(inp.cu_seqlens[n + 1])
        q = rows_f64(inp.q[t0:t1][:, qk_idx])
        k = rows_f64(inp.k[t0:t1][:, qk_idx])
        v = rows_f64(inp.v[t0:t1][:, heads])
        g = inp.g[t0:t1][:, heads].astype(np.float64)
        b = inp.beta[t0:t1][:, heads].astype(np.float64)
        s0 = None if S0 is None else S0[n][heads].astype(np.float64)[None]
        o, S = oracle.run(q, k, v, g, b, [0, t1 - t0], s0, scale=inp.scale)
        for i, h in enumerate(heads):
            out[(n, h)] = (o[:, i], S[0, i])
    return out
