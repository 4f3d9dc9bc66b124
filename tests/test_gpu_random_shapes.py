"""GPU parity on seeded random shapes: head dims, head sharing, dtypes, ragged lengths
(including empty sequences), with and without a start table, against the float64 oracle.
The shapes are drawn once from a fixed seed, so every run checks the same cases.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
from gated_deltanet_recurrence_rule_amd import binding, workloads as W
from gdn_testutil import assert_parity, to_device, to_f64

pytestmark = pytest.mark.gpu


def _cases(n=14, seed=2025):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dk = int(rng.choice([32, 64, 128]))
        dv = int(rng.choice([32, 64, 128]))
        if i % 3 == 0:
            dk = 128                      # keep the chunked kernel well represented
        HQK = int(rng.choice([1, 2, 4]))
        HV = HQK * int(rng.choice([1, 2, 3]))
        N = int(rng.integers(1, 6))
        lens = [int(x) for x in rng.choice([0, 1, 17, 63, 64, 65, 128, 190, 257], size=N)]
        dtype = "bf16" if rng.random() < 0.7 else "f32"
        s0 = bool(rng.random() < 0.6)
        out.append((i, lens, HQK, HV, dk, dv, dtype, s0))
    return out


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    binding.load()


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"case{c[0]}")
def test_random_prefill(case):
    i, lens, HQK, HV, dk, dv, dtype, s0 = case
    print(f"random case {i}: lens={lens} HQK={HQK} HV={HV} dk={dk} dv={dv} {dtype} s0={s0}", flush=True)
    inp = W.random_small(500 + i, lens, HQK, HV, dk, dv, dtype=dtype, s0=s0)
    d = to_device(inp)
    o, S = binding.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu"],
                           cu_seqlens_host=inp.cu_seqlens, S0=d["S0"], scale=inp.scale)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.run_inputs(inp)
    assert_parity(to_f64(o), to_f64(S), o_ref, S_ref, inp.as_f64("v"), dtype, f"random case {i}")


@pytest.mark.parametrize("case", _cases(8, 2026), ids=lambda c: f"case{c[0]}")
def test_random_decode(case):
    i, lens, HQK, HV, dk, dv, dtype, s0 = case
    N = max(1, len(lens))
    print(f"random decode {i}: N={N} HQK={HQK} HV={HV} dk={dk} dv={dv} {dtype}", flush=True)
    inp = W.make_inputs("dec", 600 + i, [1] * N, HQK, HV, dk, dv, dtype, 3.0, 1.0, 0.05)
    d = to_device(inp)
    S = d["S0"].clone()
    o = binding.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], S)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.run_inputs(inp)
    assert_parity(to_f64(o), to_f64(S), o_ref, S_ref, inp.as_f64("v"), dtype, f"random decode {i}")
