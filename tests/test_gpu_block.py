"""GPU parity of the block parts around the scan against the float64 oracle.

The handbook page "7. Gated DeltaNet: the token-by-token recurrence" wraps the delta rule
in a block (its forward listing and parts table): a causal short convolution + SiLU in
front, gates from raw projections, a gated RMS norm behind.  libgdn runs the gates inside
the scan kernels (gdn_block_ops), the convolution as gdn_conv_silu and the norm as
gdn_gated_rmsnorm (fused into decode, after the scan in prefill).

Tolerances.  Elementwise parts: bf16 outputs within one bf16 unit in the last place of the
oracle's value rounded to bf16 (fp32 arithmetic may land on the other side of a rounding
boundary), fp32 outputs within 1e-5 relative + 1e-6 absolute.  For the convolution, whose
four-term sum can cancel, each bound also admits the fp32 rounding of that sum:
8 * 2^-24 * sum_j |w_j e_j| (four roundings of at most 2^-24 of the running magnitude, times
silu's slope, at most 1.1, with room to spare).  The carried convolution
state is a copy of inputs and must match exactly.  The scan keeps its own gate (output
max-abs <= 2e-3 |v| for bf16, 1e-5 |v| for fp32; state relative Frobenius 1e-3 / 1e-5).
A normed read y = w o / rho silu(z), rho = sqrt(mean o^2 + eps), moves by at most
|w silu(z)| (d/rho)(1 + |o| / rho) when every element of o moves by at most d; d is the
scan's output bound plus, where prefill rounds o to bf16 before the norm, 2^-8 |o|.  That
bound plus one bf16 rounding of y (2^-8 |y|) is the normed output's gate.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
from oracle import shell
from gated_deltanet_recurrence_rule_amd import binding, workloads as W
from gdn_testutil import assert_parity, to_device, to_f64

pytestmark = pytest.mark.gpu

EPS = 1e-6


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    binding.load()


def _dev(a, dtype):
    """Upload a generator array (bf16 bits reinterpreted, never re-rounded)."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _elementwise_ok(got, ref, dtype, what, floor=0.0):
    """bf16: within one bf16 ulp of the oracle rounded to bf16; fp32: 1e-5 rel + 1e-6 abs;
    both widened by `floor` (the fp32 rounding of a sum that may cancel)."""
    if dtype == "bf16":
        r = shell.round_bf16(ref)
        ulp = np.ldexp(1.0, np.frexp(np.abs(r))[1] - 8)     # spacing of bf16 values at |r|
        bad = np.abs(got - r) > ulp * 1.0001 + floor
        assert not bad.any(), f"{what}: {bad.sum()} elements off by more than one bf16 ulp"
        exact = float(np.mean(got == r))
        assert exact > 0.99, f"{what}: only {exact:.4f} of the elements round like the oracle"
    else:
        err = np.abs(got - ref) - (1e-5 * np.abs(ref) + 1e-6 + floor)
        assert (err <= 0).all(), f"{what}: max excess {err.max():.3e}"


def _conv_floor(x, w, cu, state):
    """8 * 2^-24 * sum_j |w_j e_j| for every output of the convolution (module docstring)."""
    mag, _ = shell.conv_silu_np(np.abs(x), np.abs(w), cu, None if state is None else np.abs(state), act=False)
    return 8.0 * 2.0 ** -24 * mag


# ------------------------------------------------------------------ convolution
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("lens,state,inplace", [
    ([0, 1, 2, 3, 70, 200], True, False),
    ([130, 0, 5], False, False),
    ([64, 1, 300], True, True),
])
def test_conv_silu(dtype, lens, state, inplace):
    _say(f"conv_silu {dtype} lens={lens} state={state} inplace={inplace}")
    HQK, HV, dk, dv = 2, 4, 64, 128
    bi = W.block_inputs(61, lens, HQK, HV, dk, dv, dtype, conv_state=state)
    x, w, cu = _dev(bi.x, dtype), _dev(bi.conv_w, dtype), _dev(bi.cu_seqlens, dtype)
    st_in = _dev(bi.conv_state, dtype)
    N = len(lens)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    st_out = st_in if inplace else torch.full((N, 3, x.shape[1]), 7.0, dtype=tdt, device="cuda")
    q, k, v = binding.conv_silu(x, w, HQK=HQK, HV=HV, dk=dk, dv=dv, cu_seqlens=cu,
                                cu_seqlens_host=bi.cu_seqlens, state_in=st_in, state_out=st_out)
    torch.cuda.synchronize()
    y_ref, s_ref = shell.conv_silu_np(bi.as_f64("x"), bi.conv_w, bi.cu_seqlens, bi.as_f64("conv_state"))
    fl = _conv_floor(bi.as_f64("x"), bi.conv_w, bi.cu_seqlens, bi.as_f64("conv_state"))
    Cq = HQK * dk
    T = bi.x.shape[0]
    _elementwise_ok(to_f64(q).reshape(T, -1), y_ref[:, :Cq], dtype, "conv q", fl[:, :Cq])
    _elementwise_ok(to_f64(k).reshape(T, -1), y_ref[:, Cq:2 * Cq], dtype, "conv k", fl[:, Cq:2 * Cq])
    _elementwise_ok(to_f64(v).reshape(T, -1), y_ref[:, 2 * Cq:], dtype, "conv v", fl[:, 2 * Cq:])
    np.testing.assert_array_equal(to_f64(st_out), s_ref)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_conv_silu_decode_tokens(dtype):
    """N sequences of one token each, no cu_seqlens, state in place: a decode step's convolution."""
    _say(f"conv_silu decode {dtype}")
    N, HQK, HV, d = 48, 16, 32, 128
    bi = W.block_inputs(62, [1] * N, HQK, HV, d, d, dtype)
    x, w, st = _dev(bi.x, dtype), _dev(bi.conv_w, dtype), _dev(bi.conv_state, dtype)
    q, k, v = binding.conv_silu(x, w, HQK=HQK, HV=HV, dk=d, dv=d, N=N, state_in=st, state_out=st)
    torch.cuda.synchronize()
    y_ref, s_ref = shell.conv_silu_np(bi.as_f64("x"), bi.conv_w, bi.cu_seqlens, bi.as_f64("conv_state"))
    fl = _conv_floor(bi.as_f64("x"), bi.conv_w, bi.cu_seqlens, bi.as_f64("conv_state"))
    got = np.concatenate([to_f64(t).reshape(N, -1) for t in (q, k, v)], axis=1)
    _elementwise_ok(got, y_ref, dtype, "conv decode", fl)
    np.testing.assert_array_equal(to_f64(st), s_ref)


# ------------------------------------------------------------------ gated RMS norm
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("dv", [32, 64, 128])
@pytest.mark.parametrize("inplace", [False, True])
def test_gated_rmsnorm(dtype, dv, inplace):
    _say(f"gated_rmsnorm {dtype} dv={dv} inplace={inplace}")
    bi = W.block_inputs(63, [333], 1, 3, 32, dv, dtype)         # 999 rows: a ragged last block
    o = bi.z[::-1].copy()                                        # any bf16 / fp32 values serve as the read
    x, z, w = _dev(o, dtype), _dev(bi.z, dtype), _dev(bi.norm_w, dtype)
    y = binding.gated_rmsnorm(x, z, w, EPS, y=x if inplace else None)
    torch.cuda.synchronize()
    xo = o.astype(np.float64) if dtype == "f32" else W.bf16_bits_to_f32(o).astype(np.float64)
    ref = shell.gated_rmsnorm_np(xo, bi.as_f64("z"), bi.norm_w, EPS)
    _elementwise_ok(to_f64(y), ref, dtype, "gated norm")


# ------------------------------------------------------------------ fused gates and norm
def _oracle_scan(inp, bi, *, raw_gates, S0=None):
    g, beta = (inp.as_f64("g"), inp.as_f64("beta"))
    if raw_gates:
        g, beta = shell.gates_np(bi.a, bi.b, bi.A_log, bi.dt_bias)
    s0 = inp.as_f64("S0") if S0 is None else S0
    return oracle.run(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"), g, beta, inp.cu_seqlens, s0,
                      scale=inp.scale)


def _norm_bound(o_ref, d, bi_z, norm_w, y_ref):
    """Elementwise bound on the normed read (module docstring)."""
    rho = np.sqrt(np.mean(o_ref * o_ref, axis=-1, keepdims=True) + EPS)
    gate = np.abs(norm_w * shell.silu(bi_z))
    return gate * (d / rho) * (1.0 + np.abs(o_ref) / rho) + 2.0 ** -8 * np.abs(y_ref) + 1e-30


def _check_normed(y, o_ref, v_ref, bi, dtype, rounded_o, what):
    fo = 2e-3 if dtype == "bf16" else 1e-5
    d = fo * oracle.v_norm(v_ref)
    if rounded_o:
        d = d + 2.0 ** -8 * np.abs(o_ref).max(axis=-1, keepdims=True)
    y_ref = shell.gated_rmsnorm_np(o_ref, bi.as_f64("z"), bi.norm_w, EPS)
    bound = _norm_bound(o_ref, d, bi.as_f64("z"), bi.norm_w, y_ref)
    excess = np.abs(y - y_ref) - bound
    assert (excess <= 0).all(), f"{what}: normed read off by {excess.max():.3e} beyond its bound"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("norm", [False, True])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 32), (32, 64)])
def test_decode_block_ops(dtype, norm, dk, dv):
    """Decode with g, beta given as raw projections (A_log, dt_bias, sigmoid) and the fused norm."""
    _say(f"decode block ops {dtype} norm={norm} dk={dk} dv={dv}")
    N, HQK, HV = 40, 2, 4
    inp = W.make_inputs("dec", 64, [1] * N, HQK, HV, dk, dv, dtype, 3.0, 1.0, 0.05)
    bi = W.block_inputs(65, [1] * N, HQK, HV, dk, dv, dtype)
    dd = to_device(inp)
    S = dd["S0"].clone()
    kw = dict(A_log=_dev(bi.A_log, dtype), dt_bias=_dev(bi.dt_bias, dtype), beta_logits=True)
    if norm:
        kw.update(z=_dev(bi.z, dtype), norm_w=_dev(bi.norm_w, dtype), norm_eps=EPS)
    o = binding.decode_step(dd["q"], dd["k"], dd["v"], _dev(bi.a, dtype), _dev(bi.b, dtype), S, **kw)
    torch.cuda.synchronize()
    o_ref, S_ref = _oracle_scan(inp, bi, raw_gates=True)
    if norm:
        assert_parity(None, to_f64(S), np.zeros((0,)), S_ref, inp.as_f64("v"), dtype, "decode block state")
        _check_normed(to_f64(o), o_ref, inp.as_f64("v"), bi, dtype, False, "decode normed read")
    else:
        assert_parity(to_f64(o), to_f64(S), o_ref, S_ref, inp.as_f64("v"), dtype, "decode raw gates")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("norm", [False, True])
def test_prefill_block_ops(dtype, norm):
    """Prefill (chunked MFMA kernel for bf16, token-serial for fp32) with raw gates and the norm."""
    lens = [0, 1, 63, 64, 65, 260]
    _say(f"prefill block ops {dtype} norm={norm} lens={lens}")
    HQK, HV, d = 2, 4, 128
    inp = W.random_small(66, lens, HQK, HV, d, d, dtype=dtype, s0=True)
    bi = W.block_inputs(67, lens, HQK, HV, d, d, dtype)
    dd = to_device(inp)
    kw = dict(A_log=_dev(bi.A_log, dtype), dt_bias=_dev(bi.dt_bias, dtype), beta_logits=True)
    if norm:
        kw.update(z=_dev(bi.z, dtype), norm_w=_dev(bi.norm_w, dtype), norm_eps=EPS)
    o, S = binding.prefill(dd["q"], dd["k"], dd["v"], _dev(bi.a, dtype), _dev(bi.b, dtype),
                           cu_seqlens=dd["cu"], cu_seqlens_host=inp.cu_seqlens, S0=dd["S0"],
                           scale=inp.scale, **kw)
    torch.cuda.synchronize()
    o_ref, S_ref = _oracle_scan(inp, bi, raw_gates=True)
    if norm:
        assert_parity(None, to_f64(S), np.zeros((0,)), S_ref, inp.as_f64("v"), dtype, "prefill block state")
        _check_normed(to_f64(o), o_ref, inp.as_f64("v"), bi, dtype, dtype == "bf16", "prefill normed read")
    else:
        assert_parity(to_f64(o), to_f64(S), o_ref, S_ref, inp.as_f64("v"), dtype, "prefill raw gates")


def test_block_end_to_end_bf16():
    """x -> convolution + SiLU -> scan with raw gates -> gated norm, against the oracle's chain
    (which rounds the convolution's outputs to bf16 where the GPU path hands them over)."""
    lens = [200, 0, 70]
    HQK, HV, d = 2, 4, 128
    _say(f"block end to end bf16 lens={lens}")
    bi = W.block_inputs(68, lens, HQK, HV, d, d, "bf16")
    inp = W.random_small(69, lens, HQK, HV, d, d, dtype="bf16", s0=True)   # S0 only
    x, w, cu = _dev(bi.x, "bf16"), _dev(bi.conv_w, "bf16"), _dev(bi.cu_seqlens, "bf16")
    q, k, v = binding.conv_silu(x, w, HQK=HQK, HV=HV, dk=d, dv=d, cu_seqlens=cu,
                                cu_seqlens_host=bi.cu_seqlens, state_in=_dev(bi.conv_state, "bf16"))
    o, S = binding.prefill(q, k, v, _dev(bi.a, "bf16"), _dev(bi.b, "bf16"), cu_seqlens=cu,
                           cu_seqlens_host=bi.cu_seqlens, S0=_dev(inp.S0, "bf16"),
                           A_log=_dev(bi.A_log, "bf16"), dt_bias=_dev(bi.dt_bias, "bf16"), beta_logits=True,
                           z=_dev(bi.z, "bf16"), norm_w=_dev(bi.norm_w, "bf16"), norm_eps=EPS)
    torch.cuda.synchronize()
    y, _ = shell.conv_silu_np(bi.as_f64("x"), bi.conv_w, bi.cu_seqlens, bi.as_f64("conv_state"))
    y = shell.round_bf16(y)
    T, Cq = y.shape[0], HQK * d
    qr, kr = y[:, :Cq].reshape(T, HQK, d), y[:, Cq:2 * Cq].reshape(T, HQK, d)
    vr = y[:, 2 * Cq:].reshape(T, HV, d)
    g, beta = shell.gates_np(bi.a, bi.b, bi.A_log, bi.dt_bias)
    o_ref, S_ref = oracle.run(qr, kr, vr, g, beta, bi.cu_seqlens, inp.as_f64("S0"))
    assert_parity(None, to_f64(S), np.zeros((0,)), S_ref, vr, "bf16", "block state")
    _check_normed(to_f64(o), o_ref, vr, bi, "bf16", True, "block normed read")


def test_block_ops_rejected_on_device():
    inp = W.random_small(70, [10], 1, 2, 128, 128, dtype="bf16", s0=False)
    dd = to_device(inp)
    A = torch.zeros(2, device="cuda")
    with pytest.raises(binding.GdnError):     # A_log with an ungated rule
        binding.prefill(dd["q"], dd["k"], dd["v"], None, dd["beta"], cu_seqlens=dd["cu"], variant="delta",
                        A_log=A)
    with pytest.raises(binding.GdnError):     # z without its weight
        binding.prefill(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], cu_seqlens=dd["cu"],
                        z=torch.zeros_like(dd["v"]))


def test_block_full_size_qwen3next():
    """The chain at the measured size (4 x 16384 tokens, 16 QK / 32 V heads, 8192 conv channels):
    the GPU runs every token and channel; the oracle checks sampled channels of the convolution
    and sampled (sequence, V head) units of the scan + gated norm."""
    HQK, HV, d, T1, N = 16, 32, 128, 16384, 4
    _say("block full size: 4 x 16384, 16 QK / 32 V heads")
    bi = W.block_inputs(71, [T1] * N, HQK, HV, d, d, "bf16")
    inp = W.qwen3next()                                          # S0 of the same shape
    x, w, cu = _dev(bi.x, "bf16"), _dev(bi.conv_w, "bf16"), _dev(bi.cu_seqlens, "bf16")
    st = _dev(bi.conv_state, "bf16")
    st_out = torch.empty_like(st)
    q, k, v = binding.conv_silu(x, w, HQK=HQK, HV=HV, dk=d, dv=d, cu_seqlens=cu,
                                cu_seqlens_host=bi.cu_seqlens, state_in=st, state_out=st_out)
    o, S = binding.prefill(q, k, v, _dev(bi.a, "bf16"), _dev(bi.b, "bf16"), cu_seqlens=cu,
                           cu_seqlens_host=bi.cu_seqlens, S0=_dev(inp.S0, "bf16"),
                           A_log=_dev(bi.A_log, "bf16"), dt_bias=_dev(bi.dt_bias, "bf16"), beta_logits=True,
                           z=_dev(bi.z, "bf16"), norm_w=_dev(bi.norm_w, "bf16"), norm_eps=EPS)
    torch.cuda.synchronize()
    Cq = HQK * d
    xs = W.bf16_bits_to_f32(bi.x)                               # exact inputs, float32 view
    sts = W.bf16_bits_to_f32(bi.conv_state)

    def conv_ref(chans):
        y, s = shell.conv_silu_np(xs[:, chans].astype(np.float64), bi.conv_w[chans], bi.cu_seqlens,
                                  sts[:, :, chans].astype(np.float64))
        return y, s

    def conv_floor(chans):
        return _conv_floor(xs[:, chans].astype(np.float64), bi.conv_w[chans], bi.cu_seqlens,
                           sts[:, :, chans].astype(np.float64))

    # convolution: 48 channels spread over q, k and v, every token
    rng = np.random.default_rng(72)
    chans = np.sort(rng.choice(x.shape[1], 48, replace=False))
    y_ref, s_ref = conv_ref(chans)
    qkv = torch.cat([q.reshape(q.shape[0], -1), k.reshape(k.shape[0], -1), v.reshape(v.shape[0], -1)], dim=1)
    _elementwise_ok(to_f64(qkv[:, torch.from_numpy(chans).cuda()]), y_ref, "bf16", "full-size conv",
                    conv_floor(chans))
    np.testing.assert_array_equal(to_f64(st_out[:, :, torch.from_numpy(chans).cuda()]), s_ref)

    # scan + gated norm on sampled units: the oracle convolves just the channels they read
    g_all, b_all = shell.gates_np(bi.a, bi.b, bi.A_log, bi.dt_bias)
    for h in (0, 17):
        hq = h // (HV // HQK)
        qc = np.arange(hq * d, (hq + 1) * d)
        kc = Cq + qc
        vc = 2 * Cq + np.arange(h * d, (h + 1) * d)
        y, _ = conv_ref(np.concatenate([qc, kc, vc]))
        y = shell.round_bf16(y)
        for n in (0, 3):
            t0, t1 = int(bi.cu_seqlens[n]), int(bi.cu_seqlens[n + 1])
            qn, kn, vn = (y[t0:t1, i * d:(i + 1) * d][:, None, :] for i in range(3))
            o_ref, S_ref = oracle.run(qn, kn, vn, g_all[t0:t1, h:h + 1], b_all[t0:t1, h:h + 1], [0, t1 - t0],
                                      inp.S0[n, h:h + 1].astype(np.float64)[None])
            assert_parity(None, to_f64(S[n, h])[None, None], np.zeros((0,)), S_ref, vn, "bf16",
                          f"full-size block state seq {n} head {h}")
            sub = W.BlockInputs("bf16", None, None, None, None, None, None, None, bi.z[t0:t1, h:h + 1],
                                bi.norm_w, None, 1, 1, d, d)
            _check_normed(to_f64(o[t0:t1, h:h + 1]), o_ref, vn, sub, "bf16", True,
                          f"full-size normed read seq {n} head {h}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("call", ["decode", "prefill"])
def test_alpha_sigmoid_gate(dtype, call):
    """The learn-llm page's decay form alpha = sigmoid(a + bias), its bias near the page's
    initial 3.0 (alpha ~ 0.95); prefill on ragged sequences (chunked MFMA kernel for bf16)."""
    _say(f"alpha sigmoid gate {call} {dtype}")
    HQK, HV, d = 2, 4, 128
    lens = [1] * 24 if call == "decode" else [0, 1, 63, 64, 65, 260]
    if call == "decode":
        inp = W.make_inputs("dec", 73, lens, HQK, HV, d, d, dtype, 3.0, 1.0, 0.05)
    else:
        inp = W.random_small(73, lens, HQK, HV, d, d, dtype=dtype, s0=True)
    bi = W.block_inputs(74, lens, HQK, HV, d, d, dtype)
    bias = (bi.dt_bias + 2.0).astype(np.float32)               # ~ N(3, 0.5)
    dd = to_device(inp)
    kw = dict(alpha_sigmoid=True, dt_bias=_dev(bias, dtype), beta_logits=True)
    if call == "decode":
        S = dd["S0"].clone()
        o = binding.decode_step(dd["q"], dd["k"], dd["v"], _dev(bi.a, dtype), _dev(bi.b, dtype), S, **kw)
    else:
        o, S = binding.prefill(dd["q"], dd["k"], dd["v"], _dev(bi.a, dtype), _dev(bi.b, dtype), cu_seqlens=dd["cu"],
                               cu_seqlens_host=inp.cu_seqlens, S0=dd["S0"], **kw)
    torch.cuda.synchronize()
    g, beta = shell.gates_np(bi.a, bi.b, None, bias, alpha_sigmoid=True)
    o_ref, S_ref = oracle.run(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"), g, beta, inp.cu_seqlens,
                              inp.as_f64("S0"))
    assert_parity(to_f64(o), to_f64(S), o_ref, S_ref, inp.as_f64("v"), dtype, f"alpha sigmoid {call}")
