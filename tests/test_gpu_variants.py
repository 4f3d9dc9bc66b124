"""GPU parity of the update-rule variants (gdn_variant) against the float64 oracle.

The learn-llm page "13_linear_attention_viz" tabulates four update rules: Gated
DeltaNet, DeltaNet (no decay), Mamba2-style decayed linear attention (no look-up)
and plain linear attention (neither).  The oracle computes all four from its
`delta` flag and the gates it is given: an ungated variant is the oracle with
g = 0 (a = 1), a variant called without beta is the oracle with beta = 1.
Tolerances are the same as for the default rule.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
from gated_deltanet_recurrence_rule_amd import binding, workloads as W
from gdn_testutil import assert_parity, to_device, to_f64

pytestmark = pytest.mark.gpu

GATED = {"delta": False, "gated_linear": True, "linear": False}
DELTA = {"delta": True, "gated_linear": False, "linear": False}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    binding.load()


def _oracle(inp, variant, with_beta, *, S0=None):
    g = inp.as_f64("g") if GATED[variant] else np.zeros_like(inp.g, dtype=np.float64)
    b = inp.as_f64("beta") if with_beta else np.ones_like(inp.beta, dtype=np.float64)
    s0 = inp.as_f64("S0") if S0 is None else S0
    return oracle.run(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"), g, b, inp.cu_seqlens, s0,
                      scale=inp.scale, delta=DELTA[variant])


def _args(d, variant, with_beta):
    # ungated variants get g = NULL; "delta" keeps beta (it needs it), the linear ones
    # are run both with and without it
    return (d["g"] if GATED[variant] else None), (d["beta"] if with_beta else None)


CASES = [("delta", True), ("gated_linear", True), ("gated_linear", False), ("linear", False)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("variant,with_beta", CASES)
def test_decode_variant(dtype, variant, with_beta):
    _say(f"decode variant={variant} beta={with_beta} dtype={dtype}")
    inp = W.make_inputs("dec", 51, [1] * 6, 2, 4, 128, 128, dtype, 3.0, 1.0, 0.05)
    d = to_device(inp)
    S = d["S0"].clone()
    g, b = _args(d, variant, with_beta)
    o = binding.decode_step(d["q"], d["k"], d["v"], g, b, S, variant=variant)
    torch.cuda.synchronize()
    o_ref, S_ref = _oracle(inp, variant, with_beta)
    assert_parity(to_f64(o), to_f64(S), o_ref, S_ref, inp.as_f64("v"), dtype, f"decode {variant}",
                  grows=not DELTA[variant])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("variant,with_beta", CASES)
def test_prefill_variant(dtype, variant, with_beta):
    """Ragged batch spanning several 64-token chunks; bf16 runs the chunked MFMA kernel
    (without the look-up it skips the triangular solve), fp32 the token-serial one."""
    lens = [0, 1, 63, 64, 65, 300]
    _say(f"prefill variant={variant} beta={with_beta} dtype={dtype} lens={lens}")
    inp = W.random_small(52, lens, 2, 4, 128, 128, dtype=dtype, s0=True)
    d = to_device(inp)
    g, b = _args(d, variant, with_beta)
    o, S = binding.prefill(d["q"], d["k"], d["v"], g, b, cu_seqlens=d["cu"],
                           cu_seqlens_host=inp.cu_seqlens, S0=d["S0"], scale=inp.scale,
                           variant=variant)
    torch.cuda.synchronize()
    o_ref, S_ref = _oracle(inp, variant, with_beta)
    assert_parity(to_f64(o), to_f64(S), o_ref, S_ref, inp.as_f64("v"), dtype, f"prefill {variant}",
                  grows=not DELTA[variant])


def test_prefill_variant_ignores_unused_gates():
    """An ungated variant given a g tensor, and a linear one given beta = 1 explicitly,
    match the same call with NULL gates exactly."""
    inp = W.random_small(53, [130, 70], 2, 4, 128, 128, dtype="bf16", s0=True)
    d = to_device(inp)
    ones = torch.ones_like(d["beta"])
    kw = dict(cu_seqlens=d["cu"], cu_seqlens_host=inp.cu_seqlens, S0=d["S0"], scale=inp.scale)
    o1, S1 = binding.prefill(d["q"], d["k"], d["v"], d["g"], ones, variant="linear", **kw)
    o2, S2 = binding.prefill(d["q"], d["k"], d["v"], None, None, variant="linear", **kw)
    o3, S3 = binding.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], variant="delta", **kw)
    o4, S4 = binding.prefill(d["q"], d["k"], d["v"], None, d["beta"], variant="delta", **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    assert torch.equal(o3, o4) and torch.equal(S3, S4)


def test_variant_null_gate_rules_on_device():
    inp = W.random_small(54, [10], 1, 2, 128, 128, dtype="bf16", s0=False)
    d = to_device(inp)
    with pytest.raises(binding.GdnError):
        binding.prefill(d["q"], d["k"], d["v"], None, d["beta"], cu_seqlens=d["cu"],
                        variant="gated_linear")
    with pytest.raises(binding.GdnError):
        binding.prefill(d["q"], d["k"], d["v"], d["g"], None, cu_seqlens=d["cu"], variant="delta")
    with pytest.raises(ValueError):
        binding.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu"], variant="mamba")
