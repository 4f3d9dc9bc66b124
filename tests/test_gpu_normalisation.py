"""GPU parity of the library's own q, k normalisation (the prologue of every kernel).

The library divides q and k by max(|x|_2, 1e-12) per (token, QK head) before use (the
handbook page "7. Gated DeltaNet: the token-by-token recurrence", section "Common
questions": why q and k are normalised to unit length first; the l2norm lines of its
qwen/deltanet.py listing).  The measured workloads hand it rows that are already unit
length, where dropping the step would go unseen.  Here q and k rows get norms
log-uniform in [1e-2, 1e2], 5% of the rows are all zero (they must normalise to zero)
and 2% have norm 1e-13, below the floor (they must come out with norm 1e-13 / 1e-12 =
0.1, not 1).  Both scale = 1 and the listing's scale = 1/sqrt(dk) are run.  Every
kernel family is covered: decode, the token-serial prefill (fp32, and bf16 shapes the
chunked kernel does not take), the chunked bf16 prefill, and its split-sequence path.

Each case also checks that the inputs are sharp enough: the oracle run without
normalisation must miss the normalised oracle by far more than the parity gate.
"""
import math
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
from gated_deltanet_recurrence_rule_amd import binding, workloads as W
from gdn_testutil import assert_parity, to_device, to_f64, tolerances

pytestmark = pytest.mark.gpu

SPREAD = W.NormSpread(lo=1e-2, hi=1e2, p_zero=0.05, p_tiny=0.02, tiny=1e-13)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    binding.load()


def _miss(a, ref):
    """Largest deviation, infinite where a is not finite (the un-normalised rule diverges when
    beta |k|^2 > 2, which long runs of large keys reach)."""
    d = np.abs(a - ref)
    return float("inf") if not np.isfinite(d).all() else (float(d.max()) if d.size else 0.0)


def _sharp(inp, o_ref, S_ref):
    """The un-normalised oracle must miss the normalised one by more than 20x the gate."""
    o_raw, S_raw = oracle.run_inputs(inp, normalize=False)
    fo, fs = tolerances(inp.dtype)
    vn = oracle.v_norm(inp.as_f64("v"))
    miss_o = _miss(o_raw, o_ref) / vn
    miss_s = _miss(S_raw, S_ref) / max(float(np.abs(S_ref).max()), 1e-30)
    assert miss_o > 20 * fo or miss_s > 20 * fs, (miss_o, miss_s)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv", [(32, 64), (64, 32), (128, 128)])
@pytest.mark.parametrize("scaled", [False, True])
def test_decode_unnormalised(dtype, dk, dv, scaled):
    scale = 1.0 / math.sqrt(dk) if scaled else 1.0
    _say(f"decode unnormalised q,k dtype={dtype} dk={dk} dv={dv} scale={scale:.4f}")
    inp = W.make_inputs("dec", 910 + dk + dv, [1] * 200, 4, 8, dk, dv, dtype, 3.0, 1.0, 0.05,
                        qk_spread=SPREAD, scale=scale)
    d = to_device(inp)
    S = d["S0"].clone()
    o = binding.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], S, scale=scale)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.run_inputs(inp)
    _sharp(inp, o_ref, S_ref)
    assert_parity(to_f64(o), to_f64(S), o_ref, S_ref, inp.as_f64("v"), dtype, "decode unnormalised")


@pytest.mark.parametrize("dtype,dk,dv", [("f32", 128, 128), ("f32", 32, 64), ("bf16", 64, 128), ("bf16", 32, 32)])
@pytest.mark.parametrize("scaled", [False, True])
def test_prefill_recurrent_unnormalised(dtype, dk, dv, scaled):
    scale = 1.0 / math.sqrt(dk) if scaled else 1.0
    _say(f"token-serial prefill unnormalised dtype={dtype} dk={dk} dv={dv} scale={scale:.4f}")
    inp = W.random_small(920 + dk, [150, 0, 61], 2, 4, dk, dv, dtype=dtype, qk_spread=SPREAD, scale=scale)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    assert binding.prefill_kernel_name(inp.N, inp.total_T, inp.HQK, inp.HV, dk, dv, tdt) == "prefill_recurrent"
    d = to_device(inp)
    o, S = binding.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu"],
                           cu_seqlens_host=inp.cu_seqlens, S0=d["S0"], scale=scale)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.run_inputs(inp)
    _sharp(inp, o_ref, S_ref)
    assert_parity(to_f64(o), to_f64(S), o_ref, S_ref, inp.as_f64("v"), dtype, "recurrent unnormalised")


@pytest.mark.parametrize("scaled", [False, True])
@pytest.mark.parametrize("lens,HQK,HV,dv", [([300, 77, 130], 2, 4, 128), ([64, 1, 190], 1, 3, 64)])
def test_prefill_chunked_unnormalised(lens, HQK, HV, dv, scaled):
    scale = 1.0 / math.sqrt(128) if scaled else 1.0
    _say(f"chunked prefill unnormalised lens={lens} HQK={HQK} HV={HV} dv={dv} scale={scale:.4f}")
    inp = W.random_small(930 + HV, lens, HQK, HV, 128, dv, dtype="bf16", qk_spread=SPREAD, scale=scale)
    assert binding.prefill_kernel_name(inp.N, inp.total_T, HQK, HV, 128, dv, torch.bfloat16) == "prefill_chunked"
    d = to_device(inp)
    o, S = binding.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu"],
                           cu_seqlens_host=inp.cu_seqlens, S0=d["S0"], scale=scale)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.run_inputs(inp)
    _sharp(inp, o_ref, S_ref)
    assert_parity(to_f64(o), to_f64(S), o_ref, S_ref, inp.as_f64("v"), "bf16", "chunked unnormalised")


@pytest.mark.parametrize("variant", ["gated_delta", "gated_linear"])
def test_prefill_split_unnormalised(variant):
    """One 4096-token sequence with two V heads: the split-sequence path (maps, chain, segments)."""
    scale = 1.0 / math.sqrt(128)
    _say(f"split prefill unnormalised variant={variant}")
    inp = W.random_small(940, [4096], 1, 2, 128, 128, dtype="bf16", qk_spread=SPREAD, scale=scale)
    assert binding.prefill_kernel_name(inp.N, inp.total_T, 1, 2, 128, 128, torch.bfloat16) == "prefill_chunked_split"
    look = variant == "gated_delta"
    d = to_device(inp)
    o, S = binding.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"] if look else None, cu_seqlens=d["cu"],
                           cu_seqlens_host=inp.cu_seqlens, S0=d["S0"], scale=scale, variant=variant)
    torch.cuda.synchronize()
    b = inp.as_f64("beta") if look else np.ones_like(inp.beta, dtype=np.float64)
    o_ref, S_ref = oracle.run(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"), inp.as_f64("g"), b,
                              inp.cu_seqlens, inp.as_f64("S0"), scale=scale, delta=look)
    o_raw, _ = oracle.run(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"), inp.as_f64("g"), b,
                          inp.cu_seqlens, inp.as_f64("S0"), scale=scale, delta=look, normalize=False)
    assert _miss(o_raw, o_ref) > 40e-3 * oracle.v_norm(inp.as_f64("v"))
    assert_parity(to_f64(o), to_f64(S), o_ref, S_ref, inp.as_f64("v"), "bf16", f"split unnormalised {variant}",
                  grows=not look)
