"""C-ABI checks that need no GPU: the library loads, exports every declared entry
point, and rejects every malformed argument before touching the device.

Validation runs before any HIP call, so these run on a machine without a GPU.
The pointers passed are host addresses of poisoned buffers: the library must
return the error and leave them untouched.
"""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "gated_deltanet_recurrence_rule_amd", "libgdn.so")

OK, E_NULL, E_SHAPE, E_DTYPE, E_UNSUP, E_ALIGN, E_SEQ, E_WS, E_HIP = 0, -1, -2, -3, -4, -5, -6, -7, -8


def declared_functions():
    src = open(os.path.join(ROOT, "include", "gdn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module", autouse=True)
def _no_visible_gpu():
    """The calls here pass host addresses and must be rejected before any launch; should one be
    accepted by mistake, it must not reach a real device.  (Counting devices does not
    initialise the runtime.)"""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("host-pointer ABI checks run only where no GPU is visible")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libgdn.so is not built (run __graft_entry__.build())")
    from gated_deltanet_recurrence_rule_amd import binding
    return binding.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) >= {"gdn_decode_step", "gdn_prefill", "gdn_prefill_workspace_size",
                          "gdn_status_str", "gdn_last_error", "gdn_version"}
    for n in names:
        assert hasattr(lib, n), n


def test_exports_variant_entry_points(lib):
    assert {"gdn_decode_step_v", "gdn_prefill_v"} <= set(declared_functions())


def test_status_strings(lib):
    for s in (OK, E_NULL, E_SHAPE, E_DTYPE, E_UNSUP, E_ALIGN, E_SEQ, E_WS, E_HIP):
        assert lib.gdn_status_str(s)
    assert lib.gdn_version() >= 100


class Bufs:
    """Poisoned host buffers standing in for device tensors (never dereferenced)."""

    def __init__(self, T=8, N=2, HQK=2, HV=4, dk=32, dv=32):
        self.T, self.N, self.HQK, self.HV, self.dk, self.dv = T, N, HQK, HV, dk, dv
        self.q = np.full(T * HQK * dk + 16, 7.0, np.float32)
        self.k = np.full_like(self.q, 7.0)
        self.v = np.full(T * HV * dv + 16, 7.0, np.float32)
        self.g = np.full(T * HV + 16, 7.0, np.float32)
        self.b = np.full_like(self.g, 7.0)
        self.o = np.full_like(self.v, 7.0)
        self.S = np.full(N * HV * dk * dv + 16, 7.0, np.float32)
        self.ST = np.full_like(self.S, 7.0)
        cu = np.linspace(0, T, N + 1).astype(np.int32)
        self.cu = cu

    def p(self, a, off=0):
        return ctypes.c_void_p(a.ctypes.data + off)

    def untouched(self):
        return all(np.all(x == 7.0) for x in (self.q, self.k, self.v, self.g, self.b, self.o,
                                               self.S, self.ST))


def _prefill(lib, B, **kw):
    a = dict(q=B.p(B.q), k=B.p(B.k), v=B.p(B.v), g=B.p(B.g), b=B.p(B.b), cu=B.p(B.cu),
             cu_host=B.p(B.cu), N=B.N, T=B.T, S0=B.p(B.S), o=B.p(B.o), ST=B.p(B.ST), HQK=B.HQK,
             HV=B.HV, dk=B.dk, dv=B.dv, dtype=1, scale=1.0, ws=None, ws_bytes=0)
    a.update(kw)
    return lib.gdn_prefill(a["q"], a["k"], a["v"], a["g"], a["b"], a["cu"], a["cu_host"], a["N"],
                           a["T"], a["S0"], a["o"], a["ST"], a["HQK"], a["HV"], a["dk"], a["dv"],
                           a["dtype"], a["scale"], a["ws"], a["ws_bytes"], None)


def _decode(lib, B, **kw):
    a = dict(q=B.p(B.q), k=B.p(B.k), v=B.p(B.v), g=B.p(B.g), b=B.p(B.b), S=B.p(B.S), o=B.p(B.o),
             N=B.N, HQK=B.HQK, HV=B.HV, dk=B.dk, dv=B.dv, dtype=1, scale=1.0)
    a.update(kw)
    return lib.gdn_decode_step(a["q"], a["k"], a["v"], a["g"], a["b"], a["S"], a["o"], a["N"],
                               a["HQK"], a["HV"], a["dk"], a["dv"], a["dtype"], a["scale"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), E_NULL), (dict(k=None), E_NULL), (dict(v=None), E_NULL), (dict(g=None), E_NULL),
    (dict(b=None), E_NULL), (dict(o=None), E_NULL), (dict(S=None), E_NULL),
    (dict(N=-1), E_SHAPE), (dict(HQK=0), E_SHAPE), (dict(HQK=3), E_SHAPE), (dict(HV=-4), E_SHAPE),
    (dict(dk=48), E_UNSUP), (dict(dv=256), E_UNSUP), (dict(dk=16), E_UNSUP),
    (dict(dtype=7), E_DTYPE),
])
def test_decode_rejects(lib, kw, status):
    B = Bufs()
    assert _decode(lib, B, **kw) == status
    assert lib.gdn_last_error()
    assert B.untouched()


def test_decode_rejects_misaligned(lib):
    B = Bufs()
    for name in ("q", "k", "v", "o", "S"):
        assert _decode(lib, B, **{name: B.p(getattr(B, name), 4)}) == E_ALIGN
    assert _decode(lib, B, g=B.p(B.g, 2)) == E_ALIGN
    assert B.untouched()


def test_decode_zero_sequences_is_a_noop(lib):
    B = Bufs()
    assert _decode(lib, B, N=0, q=None, k=None, v=None, g=None, b=None, o=None, S=None) == OK
    assert B.untouched()


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), E_NULL), (dict(o=None), E_NULL), (dict(g=None), E_NULL),
    (dict(T=-1), E_SHAPE), (dict(N=-2), E_SHAPE), (dict(HQK=3), E_SHAPE),
    (dict(dk=100), E_UNSUP), (dict(dtype=-1), E_DTYPE),
    (dict(T=9), E_SEQ),                                     # cu[N] != total_T
    (dict(cu=None, cu_host=None, N=3), E_SEQ),              # N does not divide total_T
])
def test_prefill_rejects(lib, kw, status):
    B = Bufs()
    assert _prefill(lib, B, **kw) == status
    assert B.untouched()


def test_prefill_rejects_bad_host_seqlens(lib):
    B = Bufs(T=8, N=3)
    for cu in ([1, 4, 6, 8], [0, 5, 4, 8], [0, 2, 4, 7]):
        arr = np.array(cu, np.int32)
        assert _prefill(lib, B, cu_host=B.p(arr)) == E_SEQ
    assert B.untouched()


def test_prefill_rejects_misaligned(lib):
    B = Bufs()
    for name, buf in (("q", B.q), ("v", B.v), ("o", B.o), ("S0", B.S), ("ST", B.ST)):
        assert _prefill(lib, B, **{name: B.p(buf, 4)}) == E_ALIGN, name
    assert _prefill(lib, B, cu=B.p(B.cu, 2)) == E_ALIGN
    assert B.untouched()


def test_prefill_workspace_contract(lib):
    B = Bufs()
    need = lib.gdn_prefill_workspace_size(B.N, B.T, B.HQK, B.HV, B.dk, B.dv, 0)
    if need > 0:
        assert _prefill(lib, B, dtype=0, ws=None, ws_bytes=need - 1) == E_WS
    assert B.untouched()


def test_prefill_zero_sequences_is_a_noop(lib):
    B = Bufs()
    z = np.zeros(1, np.int32)
    assert _prefill(lib, B, N=0, T=0, cu=B.p(z), cu_host=B.p(z), q=None, k=None, v=None,
                    g=None, b=None, o=None, S0=None, ST=None) == OK
    assert B.untouched()


def _decode_v(lib, B, variant, **kw):
    a = dict(q=B.p(B.q), k=B.p(B.k), v=B.p(B.v), g=B.p(B.g), b=B.p(B.b), S=B.p(B.S), o=B.p(B.o),
             N=B.N, HQK=B.HQK, HV=B.HV, dk=B.dk, dv=B.dv, dtype=1, scale=1.0)
    a.update(kw)
    return lib.gdn_decode_step_v(a["q"], a["k"], a["v"], a["g"], a["b"], a["S"], a["o"], a["N"],
                                 a["HQK"], a["HV"], a["dk"], a["dv"], a["dtype"], a["scale"], variant,
                                 None)


def _prefill_v(lib, B, variant, **kw):
    a = dict(q=B.p(B.q), k=B.p(B.k), v=B.p(B.v), g=B.p(B.g), b=B.p(B.b), cu=B.p(B.cu),
             cu_host=B.p(B.cu), N=B.N, T=B.T, S0=B.p(B.S), o=B.p(B.o), ST=B.p(B.ST), HQK=B.HQK,
             HV=B.HV, dk=B.dk, dv=B.dv, dtype=1, scale=1.0, ws=None, ws_bytes=0)
    a.update(kw)
    return lib.gdn_prefill_v(a["q"], a["k"], a["v"], a["g"], a["b"], a["cu"], a["cu_host"], a["N"],
                             a["T"], a["S0"], a["o"], a["ST"], a["HQK"], a["HV"], a["dk"], a["dv"],
                             a["dtype"], a["scale"], variant, a["ws"], a["ws_bytes"], None)


GATED_DELTA, DELTA, GATED_LINEAR, LINEAR = 0, 1, 2, 3


@pytest.mark.parametrize("call", [_decode_v, _prefill_v])
@pytest.mark.parametrize("variant,kw,status", [
    (7, {}, E_UNSUP), (-1, {}, E_UNSUP),
    (GATED_DELTA, dict(g=None), E_NULL), (GATED_DELTA, dict(b=None), E_NULL),
    (DELTA, dict(b=None), E_NULL), (GATED_LINEAR, dict(g=None), E_NULL),
    (DELTA, dict(g=None, HQK=3), E_SHAPE), (LINEAR, dict(g=None, b=None, dk=48), E_UNSUP),
    (GATED_LINEAR, dict(b=None, g=None), E_NULL),
])
def test_variant_rejects(lib, call, variant, kw, status):
    B = Bufs()
    assert call(lib, B, variant, **kw) == status
    assert lib.gdn_last_error()
    assert B.untouched()


@pytest.mark.parametrize("variant", [DELTA, GATED_LINEAR, LINEAR])
def test_variant_zero_sequences_is_a_noop(lib, variant):
    B = Bufs()
    z = np.zeros(1, np.int32)
    assert _decode_v(lib, B, variant, N=0, q=None, k=None, v=None, g=None, b=None, o=None,
                     S=None) == OK
    assert _prefill_v(lib, B, variant, N=0, T=0, cu=B.p(z), cu_host=B.p(z), q=None, k=None, v=None,
                      g=None, b=None, o=None, S0=None, ST=None) == OK
    assert B.untouched()


# ------------------------------------------------------------------ block parts
def test_exports_block_entry_points(lib):
    assert {"gdn_decode_step_ex", "gdn_prefill_ex", "gdn_conv_silu", "gdn_gated_rmsnorm"} <= set(declared_functions())
    assert lib.gdn_status_str(-9) and lib.gdn_status_str(-10)


E_ALIAS, E_VALUE = -9, -10


def _ops(B, **kw):
    from gated_deltanet_recurrence_rule_amd.binding import BlockOps
    a = dict(A_log=None, dt_bias=None, beta_logits=0, z=None, norm_w=None, norm_eps=1e-6, alpha_sigmoid=0)
    a.update(kw)
    return BlockOps(a["A_log"], a["dt_bias"], a["beta_logits"], a["z"], a["norm_w"], a["norm_eps"],
                    a["alpha_sigmoid"])


def _decode_ex(lib, B, variant, ops, **kw):
    a = dict(q=B.p(B.q), k=B.p(B.k), v=B.p(B.v), g=B.p(B.g), b=B.p(B.b), S=B.p(B.S), o=B.p(B.o),
             N=B.N, HQK=B.HQK, HV=B.HV, dk=B.dk, dv=B.dv, dtype=1, scale=1.0)
    a.update(kw)
    return lib.gdn_decode_step_ex(a["q"], a["k"], a["v"], a["g"], a["b"], a["S"], a["o"], a["N"], a["HQK"],
                                  a["HV"], a["dk"], a["dv"], a["dtype"], a["scale"], variant,
                                  None if ops is None else ctypes.byref(ops), None)


def _prefill_ex(lib, B, variant, ops, **kw):
    a = dict(q=B.p(B.q), k=B.p(B.k), v=B.p(B.v), g=B.p(B.g), b=B.p(B.b), cu=B.p(B.cu),
             cu_host=B.p(B.cu), N=B.N, T=B.T, S0=B.p(B.S), o=B.p(B.o), ST=B.p(B.ST), HQK=B.HQK,
             HV=B.HV, dk=B.dk, dv=B.dv, dtype=1, scale=1.0, ws=None, ws_bytes=0)
    a.update(kw)
    return lib.gdn_prefill_ex(a["q"], a["k"], a["v"], a["g"], a["b"], a["cu"], a["cu_host"], a["N"], a["T"],
                              a["S0"], a["o"], a["ST"], a["HQK"], a["HV"], a["dk"], a["dv"], a["dtype"],
                              a["scale"], variant, None if ops is None else ctypes.byref(ops), a["ws"],
                              a["ws_bytes"], None)


@pytest.mark.parametrize("call", [_decode_ex, _prefill_ex])
@pytest.mark.parametrize("case,variant,status", [
    ("A_log_ungated", DELTA, E_UNSUP), ("A_log_linear", LINEAR, E_UNSUP),
    ("logits_without_beta", GATED_LINEAR, E_NULL), ("z_without_w", GATED_DELTA, E_NULL),
    ("negative_eps", GATED_DELTA, E_VALUE), ("nan_eps", GATED_DELTA, E_VALUE),
    ("z_misaligned", GATED_DELTA, E_ALIGN), ("z_overlaps_o", GATED_DELTA, E_ALIAS),
    ("alpha_ungated", DELTA, E_UNSUP), ("alpha_and_A_log", GATED_DELTA, E_VALUE),
])
def test_block_ops_rejects(lib, call, case, variant, status):
    B = Bufs()
    w = np.ones(B.dv + 4, np.float32)
    z = np.full_like(B.v, 7.0)
    kw, okw = {}, {}
    if case.startswith("A_log"):
        okw = dict(A_log=B.p(w).value)
        kw = dict(g=None) if variant == DELTA else dict(g=None, b=None)
    elif case == "logits_without_beta":
        okw, kw = dict(beta_logits=1), dict(b=None)
    elif case == "z_without_w":
        okw = dict(z=B.p(z).value)
    elif case == "negative_eps":
        okw = dict(z=B.p(z).value, norm_w=B.p(w).value, norm_eps=-1.0)
    elif case == "nan_eps":
        okw = dict(z=B.p(z).value, norm_w=B.p(w).value, norm_eps=float("nan"))
    elif case == "z_misaligned":
        okw = dict(z=B.p(z, 4).value, norm_w=B.p(w).value)
    elif case == "z_overlaps_o":
        okw = dict(z=B.p(B.o, 64).value, norm_w=B.p(w).value)
    elif case == "alpha_ungated":
        okw, kw = dict(alpha_sigmoid=1), dict(g=None)
    elif case == "alpha_and_A_log":
        okw = dict(alpha_sigmoid=1, A_log=B.p(w).value)
    assert call(lib, B, variant, _ops(B, **okw), **kw) == status, lib.gdn_last_error()
    assert B.untouched() and np.all(z == 7.0)


def test_prefill_ex_rejects_norm_in_place_on_z(lib):
    B = Bufs()
    w = np.ones(B.dv, np.float32)
    assert _prefill_ex(lib, B, GATED_DELTA, _ops(B, z=B.p(B.o).value, norm_w=B.p(w).value)) == E_ALIAS
    assert B.untouched()


def test_block_ops_zero_tokens_is_a_noop(lib):
    B = Bufs()
    z = np.zeros(1, np.int32)
    ops = _ops(B, A_log=None, beta_logits=1)
    assert _decode_ex(lib, B, GATED_DELTA, ops, N=0, q=None, k=None, v=None, g=None, b=None, o=None,
                      S=None) == OK
    assert _prefill_ex(lib, B, GATED_DELTA, ops, N=0, T=0, cu=B.p(z), cu_host=B.p(z), q=None, k=None,
                       v=None, g=None, b=None, o=None, S0=None, ST=None) == OK
    assert B.untouched()


class ConvBufs:
    def __init__(self, T=9, N=2, HQK=1, HV=2, dk=32, dv=32):
        self.T, self.N, self.HQK, self.HV, self.dk, self.dv = T, N, HQK, HV, dk, dv
        self.Ct = 2 * HQK * dk + HV * dv
        self.x = np.full(T * self.Ct + 16, 7.0, np.float32)
        self.w = np.full(self.Ct * 4 + 16, 7.0, np.float32)
        self.s = np.full(N * 3 * self.Ct + 64, 7.0, np.float32)
        self.q = np.full(T * HQK * dk + 16, 7.0, np.float32)
        self.k = np.full_like(self.q, 7.0)
        self.v = np.full(T * HV * dv + 16, 7.0, np.float32)
        self.cu = np.array([0, 4, T], np.int32)

    def p(self, a, off=0):
        return ctypes.c_void_p(a.ctypes.data + off)

    def untouched(self):
        return all(np.all(a == 7.0) for a in (self.x, self.w, self.s, self.q, self.k, self.v))


def _conv(lib, C, **kw):
    a = dict(x=C.p(C.x), w=C.p(C.w), cu=C.p(C.cu), cu_host=C.p(C.cu), N=C.N, T=C.T, si=C.p(C.s),
             so=None, q=C.p(C.q), k=C.p(C.k), v=C.p(C.v), HQK=C.HQK, HV=C.HV, dk=C.dk, dv=C.dv, dtype=1)
    a.update(kw)
    return lib.gdn_conv_silu(a["x"], a["w"], a["cu"], a["cu_host"], a["N"], a["T"], a["si"], a["so"], a["q"],
                             a["k"], a["v"], a["HQK"], a["HV"], a["dk"], a["dv"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=4), E_DTYPE), (dict(HQK=0), E_SHAPE), (dict(N=-1), E_SHAPE), (dict(dk=48), E_UNSUP),
    (dict(x=None), E_NULL), (dict(w=None), E_NULL), (dict(v=None), E_NULL),
    (dict(T=10), E_SEQ), (dict(cu=None, cu_host=None, T=9, N=2), E_SEQ),
])
def test_conv_rejects(lib, kw, status):
    C = ConvBufs()
    assert _conv(lib, C, **kw) == status
    assert C.untouched()


def test_conv_rejects_misaligned_and_overlap(lib):
    C = ConvBufs()
    for name, buf in (("x", C.x), ("w", C.w), ("q", C.q), ("si", C.s)):
        assert _conv(lib, C, **{name: C.p(buf, 4)}) == E_ALIGN, name
    assert _conv(lib, C, so=C.p(C.s, 16)) == E_ALIAS
    assert _conv(lib, C, N=0, T=0, cu=C.p(np.zeros(1, np.int32)), cu_host=None) == OK
    assert C.untouched()


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=2), E_DTYPE), (dict(rows=-1), E_SHAPE), (dict(dv=48), E_UNSUP), (dict(eps=-1e-3), E_VALUE),
    (dict(eps=float("nan")), E_VALUE), (dict(x=None), E_NULL), (dict(w=None), E_NULL),
    ("y_is_z", E_ALIAS), ("y_inside_x", E_ALIAS), ("x_misaligned", E_ALIGN),
])
def test_gated_rmsnorm_rejects(lib, kw, status):
    x = np.full(8 * 32 + 64, 7.0, np.float32)
    z = np.full_like(x, 7.0)
    y = np.full_like(x, 7.0)
    w = np.full(32, 7.0, np.float32)
    p = lambda a, off=0: ctypes.c_void_p(a.ctypes.data + off)
    a = dict(x=p(x), z=p(z), w=p(w), eps=1e-6, y=p(y), rows=8, dv=32, dtype=1)
    if kw == "y_is_z":
        kw = dict(y=p(z))
    elif kw == "y_inside_x":
        kw = dict(y=p(x, 64))
    elif kw == "x_misaligned":
        kw = dict(x=p(x, 4))
    a.update(kw)
    assert lib.gdn_gated_rmsnorm(a["x"], a["z"], a["w"], a["eps"], a["y"], a["rows"], a["dv"], a["dtype"],
                                 None) == status
    assert all(np.all(t == 7.0) for t in (x, z, y, w))


# ------------------------------------------------------------------ split sequences
def test_split_workspace_plan(lib):
    """Host planning of split sequences (no GPU here, so the device is taken to have 256
    compute units).  The plan minimises the modelled time in chunk periods; the expected plans
    below are what that model gives, worked out by hand:
    1 x 8192 tokens, 16 heads, d = 128, bf16: u = 32 workgroups of 64 columns, 128 chunks.
    P = 9: the maps of segments 1-7 (7 x 64 workgroups) take 2 rounds of the 224 units beside
    segment 0's scan, so w0 = 2 and a = ceil(128 / 10) = 13 chunks per unit; the segment pass
    (8 x 32 workgroups) 1 round; 3 x 13 + 7 x 1.2 + 3 = 50.4 periods against 0.87 x 128 unsplit.
    Workspace: 7 maps of 128 x 256 and 8 start tables of 128 x 128 per head."""
    def plan_bytes(N, HV, P, dk=128, dv=128):
        maps = N * (P - 2) * HV * dk * (dv + dk) * 4
        starts = N * (P - 1) * HV * dk * dv * 4
        return (maps + 255) // 256 * 256 + (starts + 255) // 256 * 256

    assert lib.gdn_prefill_workspace_size(1, 8192, 16, 16, 128, 128, 0) == plan_bytes(1, 16, 9)
    assert lib.gdn_prefill_kernel_name(1, 8192, None, 16, 16, 128, 128, 0) == b"prefill_chunked_split"
    # 24 chunks: P = 5 with w0 = 1 (3 maps fit one round), a = 5: 2 x 5 + 3 x 1.2 + 3 = 16.6
    # periods against 0.87 x 24 = 20.9
    assert lib.gdn_prefill_workspace_size(1, 1500, 16, 16, 128, 128, 0) == plan_bytes(1, 16, 5)
    # 16 chunks: P = 4, w0 = 1, a = 4: 8 + 2.4 + 3 = 13.4 < 0.97 x 13.92
    assert lib.gdn_prefill_workspace_size(1, 1000, 16, 16, 128, 128, 0) == plan_bytes(1, 16, 4)
    # 7 chunks: nothing beats 0.87 x 7 once the fixed cost of the two extra launches is paid
    assert lib.gdn_prefill_workspace_size(1, 400, 16, 16, 128, 128, 0) == 0
    assert lib.gdn_prefill_kernel_name(1, 400, None, 16, 16, 128, 128, 0) == b"prefill_chunked"
    # 2 x 16384 tokens, 32 heads: u = 128, so the maps of one middle segment take 2 rounds of
    # the other 128 units: P = 3, w0 = 2, a = 64: 3 x 64 + 1.2 x 2 + 3 = 197.4 against 222.7
    # (the launch order takes the first 256 bytes)
    assert lib.gdn_prefill_workspace_size(2, 32768, 16, 32, 128, 128, 0) == 256 + plan_bytes(2, 32, 3)
    assert lib.gdn_prefill_kernel_name(2, 32768, None, 16, 32, 128, 128, 0) == b"prefill_chunked_split"
    assert lib.gdn_prefill_narrow_count(2, 32768, None, 16, 32, 128, 128, 0) == 0
    # the 4 x 16384 batch fills the device (256 workgroups): no split
    assert lib.gdn_prefill_workspace_size(4, 65536, 16, 32, 128, 128, 0) == 256
    assert lib.gdn_prefill_kernel_name(4, 65536, None, 16, 32, 128, 128, 0) == b"prefill_chunked"
    # a batch of more than half the units (3 x 16384, 32 heads: 192 workgroups) never splits
    assert lib.gdn_prefill_workspace_size(3, 49152, 16, 32, 128, 128, 0) == 256
    # fp32 runs the token-serial kernel: never split
    assert lib.gdn_prefill_workspace_size(1, 8192, 16, 16, 128, 128, 1) == 0


def test_narrow_workgroup_rule(lib):
    """Host rule for 32-column workgroups (no GPU here: 256 compute units assumed), as reported
    for a workspace of gdn_prefill_workspace_size_lens bytes.  A batch whose 64-column
    workgroups fill at most half the units narrows all (host lengths or not); of two long
    sequences of similar length the longer is narrowed; a batch with one sequence that would
    outlast the rest has that one split instead (0); uniform batches that fill more, two equally
    long sequences, small split batches, fp32, and a large batch without host lengths narrow
    none."""
    import ctypes

    def count(lens, HQK=16, HV=32, dk=128, dv=128, dtype=0, host=True):
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        ptr = cu.ctypes.data_as(ctypes.c_void_p) if host else None
        return lib.gdn_prefill_narrow_count(len(lens), int(cu[-1]), ptr, HQK, HV, dk, dv, dtype)

    from gated_deltanet_recurrence_rule_amd import workloads as W
    assert count([1000, 900, 300, 200]) == 1
    assert count([200, 900, 1000, 300]) == 1  # the rule does not need sorted lengths
    assert count([1000] * 6 + [100] * 100, HQK=2, HV=4) == 6
    assert count([4000] * 6 + [100] * 100, HQK=2, HV=4) == 0  # long enough to split the six instead
    assert count([10000, 9000, 300, 200]) == 0  # the two longest split
    assert count(list(W.varlen_lengths())) == 0  # its 262144-token sequence is split instead
    assert count([262144] + [1000] * 10) == 0
    assert count([8192, 1000, 300, 257]) == 0
    assert count([16384] * 4) == 0
    assert count([16384] * 3) == 0  # a third of the device idle, but no sequence outlasts the others
    assert count([32768, 32768, 100]) == 0  # the second long sequence would stay on 64 columns
    assert count([8192, 100]) == 2  # 128 workgroups of 64 columns: all on 32 (a split does not pay)
    assert count([8192, 100], host=False) == 2
    assert count([8192], HQK=16, HV=16) == 0  # 32 workgroups: split into 9 segments instead
    assert count([8192, 1000, 300, 257], dtype=1) == 0  # fp32: token-serial kernel
    assert count([1000, 900, 300, 200], host=False) == 0


def test_longest_sequence_split_plan(lib):
    """With the host lengths, a packed batch that the sizes alone leave unsplit may have its
    longest sequences cut into segments (no GPU here: 256 compute units assumed).
    The 65-sequence batch (64 lengths of 128 .. 32768 tokens and one of 262144), 32 V heads of
    d = 128: the model takes P = 5, so the workspace grows by 3 maps of 128 x 256 and 4 start
    tables of 128 x 128 per head for that one sequence; the kernel is then the split one.
    Batches with no dominant sequence keep gdn_prefill_workspace_size's plan."""
    import ctypes
    from gated_deltanet_recurrence_rule_amd import workloads as W

    def sizes(lens, HQK=16, HV=32, dtype=0, sort=False):
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        ptr = cu.ctypes.data_as(ctypes.c_void_p)
        N, T = len(lens), int(cu[-1])
        base = lib.gdn_prefill_workspace_size(N, T, HQK, HV, 128, 128, dtype)
        lens_ws = lib.gdn_prefill_workspace_size_lens(N, T, ptr, HQK, HV, 128, 128, dtype)
        name = lib.gdn_prefill_kernel_name(N, T, ptr, HQK, HV, 128, 128, dtype)
        return base, lens_ws, name

    per_head = 3 * 128 * 256 * 4 + 4 * 128 * 128 * 4
    base, lens_ws, name = sizes(list(W.varlen_lengths()))
    assert base == 512 and lens_ws == base + 32 * per_head and name == b"prefill_chunked_split"
    base, lens_ws, name = sizes([300, 1000, 8192, 257])
    assert lens_ws == base + 32 * per_head and name == b"prefill_chunked_split"
    # the two longest of three: P = 3, one map and two start tables per head for each
    base, lens_ws, name = sizes([32768, 32768, 100])
    assert lens_ws == base + 2 * 32 * (128 * 256 * 4 + 2 * 128 * 128 * 4) and name == b"prefill_chunked_split"
    for lens in ([16384] * 4, [16384] * 3, [1000, 900, 300, 200]):
        base, lens_ws, name = sizes(lens)
        assert lens_ws == base and name == b"prefill_chunked", lens
    base, lens_ws, name = sizes(list(W.varlen_lengths()), dtype=1)  # fp32: token-serial, no workspace
    assert base == lens_ws and name == b"prefill_recurrent"
    # more sequences than the order kernel ranks (16384): launched in the given order, so the
    # longest is split only when the lengths never increase
    many = [1 << 20] + [64] * 16400
    base, lens_ws, name = sizes(many)
    assert base == 0 and lens_ws == 32 * per_head and name == b"prefill_chunked_split"
    base, lens_ws, name = sizes(many[1:] + many[:1])
    assert base == 0 and lens_ws == 0 and name == b"prefill_chunked"
    # without host lengths: the sizes' plan
    N, T = 65, int(sum(W.varlen_lengths()))
    assert lib.gdn_prefill_workspace_size_lens(N, T, None, 16, 32, 128, 128, 0) == 512
    assert lib.gdn_prefill_kernel_name(N, T, None, 16, 32, 128, 128, 0) == b"prefill_chunked"


def test_split_workspace_too_small_is_rejected(lib):
    B = Bufs(T=8192, N=1, HQK=1, HV=2, dk=128, dv=128)
    need = lib.gdn_prefill_workspace_size(1, 8192, 1, 2, 128, 128, 0)
    assert need > 0
    # no pointer: a host array claimed to span need - 1 bytes would overlap the other buffers
    assert _prefill(lib, B, dtype=0, ws=None, ws_bytes=need - 1) == E_WS
    assert B.untouched()


# ------------------------------------------------------------------ overlapping buffers
# Every call below must fail its checks before any launch (the buffers are host memory).
@pytest.mark.parametrize("out,into,off", [
    ("o", "q", 0), ("o", "k", 64), ("o", "v", 16), ("o", "g", 0), ("o", "b", 16),
    ("S", "q", 0), ("S", "v", 64), ("S", "b", 0), ("S", "o", 16), ("o", "S", 0),
])
def test_decode_rejects_overlap(lib, out, into, off):
    B = Bufs()
    assert _decode(lib, B, **{out: B.p(getattr(B, into), off)}) == E_ALIAS, lib.gdn_last_error()
    assert B.untouched()


def test_decode_ex_rejects_z_or_weights_inside_outputs(lib):
    B = Bufs()
    w = np.ones(B.dv + 4, np.float32)
    z = np.full_like(B.v, 7.0)
    assert _decode_ex(lib, B, GATED_DELTA, _ops(B, z=B.p(B.o).value, norm_w=B.p(w).value)) == E_ALIAS
    assert _decode_ex(lib, B, GATED_DELTA, _ops(B, z=B.p(z).value, norm_w=B.p(B.S, 32).value)) == E_ALIAS
    assert _decode_ex(lib, B, GATED_DELTA, _ops(B, A_log=B.p(B.o, 16).value)) == E_ALIAS
    assert B.untouched() and np.all(z == 7.0)


@pytest.mark.parametrize("out,into,off", [
    ("o", "q", 0), ("o", "k", 16), ("o", "v", 0), ("o", "g", 64), ("o", "b", 0), ("o", "S", 0),
    ("o", "cu", 0), ("ST", "q", 32), ("ST", "v", 0), ("ST", "o", 0), ("ST", "S", 16), ("ST", "cu", 0),
])
def test_prefill_rejects_overlap(lib, out, into, off):
    """o and S_T must be disjoint from every input and from each other; S_T may be exactly S0
    (covered on the GPU), but not a shifted view of it."""
    B = Bufs()
    src = B.cu if into == "cu" else getattr(B, into)
    key = "S0" if out == "S" else out
    assert _prefill(lib, B, **{key: B.p(src, off)}) == E_ALIAS, lib.gdn_last_error()
    assert B.untouched()


def test_prefill_rejects_workspace_overlap(lib):
    B = Bufs()
    need = lib.gdn_prefill_workspace_size(B.N, B.T, B.HQK, B.HV, B.dk, B.dv, 1)
    assert need > 0  # the launch-order part of two sequences
    for name in ("q", "o", "S", "ST"):
        assert _prefill(lib, B, ws=B.p(getattr(B, name)), ws_bytes=need) == E_ALIAS, name
    assert B.untouched()


def test_conv_rejects_outputs_overlapping(lib):
    C = ConvBufs()
    assert _conv(lib, C, q=C.p(C.x)) == E_ALIAS
    assert _conv(lib, C, k=C.p(C.q, 16)) == E_ALIAS
    assert _conv(lib, C, v=C.p(C.w)) == E_ALIAS
    assert _conv(lib, C, so=C.p(C.v)) == E_ALIAS
    assert C.untouched()


# ------------------------------------------------------------------ the Python binding's checks
class _DevTensor:
    """Stands in for a contiguous device tensor in the binding's argument checks, which raise
    before any pointer is taken (so nothing here reaches the library)."""

    def __init__(self, shape, dtype):
        import torch
        self.shape = tuple(shape)
        self.dtype = dtype
        self.device = torch.device("cuda", 0)
        self.is_cuda = True

    def is_contiguous(self):
        return True

    def dim(self):
        return len(self.shape)


def _prefill_args(T=128, N=2, HQK=2, HV=4, dk=64, dv=32):
    import torch
    t = lambda *s, dt=torch.bfloat16: _DevTensor(s, dt)
    return dict(q=t(T, HQK, dk), k=t(T, HQK, dk), v=t(T, HV, dv), g=t(T, HV, dt=torch.float32),
                beta=t(T, HV, dt=torch.float32), cu_seqlens=t(N + 1, dt=torch.int32),
                S0=t(N, HV, dk, dv, dt=torch.float32), o=t(T, HV, dv), S_T=t(N, HV, dk, dv, dt=torch.float32))


@pytest.mark.parametrize("name,shape", [
    ("k", (128, 2, 32)), ("k", (127, 2, 64)), ("v", (120, 4, 32)), ("g", (128, 2)), ("beta", (128, 4, 1)),
    ("S0", (2, 4, 64, 64)), ("S0", (3, 4, 64, 32)), ("o", (128, 4, 64)), ("S_T", (1, 4, 64, 32)),
])
def test_binding_prefill_rejects_mis_shaped(name, shape):
    import torch
    from gated_deltanet_recurrence_rule_amd import binding
    a = _prefill_args()
    a[name] = _DevTensor(shape, a[name].dtype)
    q, k, v, g, beta = a.pop("q"), a.pop("k"), a.pop("v"), a.pop("g"), a.pop("beta")
    with pytest.raises(ValueError, match=name):
        binding.prefill(q, k, v, g, beta, **a)


def test_binding_prefill_rejects_seqlens_mismatch():
    from gated_deltanet_recurrence_rule_amd import binding
    a = _prefill_args()
    q, k, v, g, beta = a.pop("q"), a.pop("k"), a.pop("v"), a.pop("g"), a.pop("beta")
    with pytest.raises(ValueError, match="N = 3"):
        binding.prefill(q, k, v, g, beta, N=3, **a)
    with pytest.raises(ValueError, match="cu_seqlens_host"):
        binding.prefill(q, k, v, g, beta, cu_seqlens_host=[0, 128], **a)


@pytest.mark.parametrize("name,shape", [
    ("k", (5, 2, 32)), ("v", (5, 4, 16)), ("g", (4, 4)), ("beta", (5, 2)), ("S", (5, 4, 64, 16)),
    ("S", (5, 4, 32, 32)), ("o", (5, 2, 32)), ("z", (5, 4, 64)), ("A_log", (2,)), ("norm_w", (64,)),
])
def test_binding_decode_rejects_mis_shaped(name, shape):
    import torch
    from gated_deltanet_recurrence_rule_amd import binding
    t = lambda *s, dt=torch.bfloat16: _DevTensor(s, dt)
    N, HQK, HV, dk, dv = 5, 2, 4, 64, 32
    a = dict(q=t(N, HQK, dk), k=t(N, HQK, dk), v=t(N, HV, dv), g=t(N, HV, dt=torch.float32),
             beta=t(N, HV, dt=torch.float32), S=t(N, HV, dk, dv, dt=torch.float32), o=t(N, HV, dv),
             z=t(N, HV, dv), A_log=t(HV, dt=torch.float32), norm_w=t(dv, dt=torch.float32))
    a[name] = _DevTensor(shape, a[name].dtype)
    with pytest.raises(ValueError, match=name):
        binding.decode_step(a["q"], a["k"], a["v"], a["g"], a["beta"], a["S"], o=a["o"], z=a["z"],
                            A_log=a["A_log"], norm_w=a["norm_w"])


@pytest.mark.parametrize("name,shape", [
    ("w", (2 * 64 + 4 * 32, 3)), ("state_in", (2, 3, 100)), ("state_out", (3, 3, 256)), ("q", (10, 2, 32)),
    ("v", (10, 4, 64)),
])
def test_binding_conv_rejects_mis_shaped(name, shape):
    import torch
    from gated_deltanet_recurrence_rule_amd import binding
    t = lambda *s, dt=torch.bfloat16: _DevTensor(s, dt)
    T, N, HQK, HV, dk, dv = 10, 2, 1, 4, 64, 32
    Ct = 2 * HQK * dk + HV * dv
    a = dict(w=t(Ct, 4, dt=torch.float32), state_in=t(N, 3, Ct), state_out=t(N, 3, Ct), q=t(T, HQK, dk),
             k=t(T, HQK, dk), v=t(T, HV, dv))
    a[name] = _DevTensor(shape, a[name].dtype)
    with pytest.raises(ValueError, match=name):
        binding.conv_silu(t(T, Ct), a.pop("w"), HQK=HQK, HV=HV, dk=dk, dv=dv, N=N, **a)


# ------------------------------------------------------------------ the allocation-free prefill
def test_noalloc_rejects_workspace_beyond_its_scratch(lib):
    """gdn_prefill_noalloc's static scratch holds 24 MiB: a split batch (4096 tokens, 16 QK / 32 V
    heads of dv = 64) that needs ~29 MiB is rejected with GDN_ERR_WORKSPACE before anything runs
    (the device count here is taken as 256 compute units), and N = 0 is a no-op that touches no
    device."""
    T, H, HV, dk, dv = 4096, 16, 32, 128, 64
    assert lib.gdn_prefill_workspace_size(1, T, H, HV, dk, dv, 0) > 24 << 20
    q = np.full(T * H * dk // 2 + 16, 7.0, np.float32)      # bf16 sizes, in floats
    k = np.full_like(q, 7.0)
    v = np.full(T * HV * dv // 2 + 16, 7.0, np.float32)
    o = np.full_like(v, 7.0)
    g = np.full(T * HV + 16, 7.0, np.float32)
    b = np.full_like(g, 7.0)
    p = lambda a: ctypes.c_void_p(a.ctypes.data)
    st = lib.gdn_prefill_noalloc(p(q), p(k), p(v), p(g), p(b), None, None, 1, T, None, p(o), None, H, HV, dk, dv,
                                 0, 1.0, 0, None, None)
    assert st == E_WS, lib.gdn_last_error()
    assert b"static scratch" in lib.gdn_last_error()
    z = np.zeros(1, np.int32)
    assert lib.gdn_prefill_noalloc(None, None, None, None, None, p(z), p(z), 0, 0, None, None, None, H, H, dk, dv,
                                   0, 1.0, 0, None, None) == OK
    assert all(np.all(a == 7.0) for a in (q, k, v, o, g, b))
