"""GPU parity at the measured workload sizes, through the C ABI.

The GPU runs every sequence and head; the float64 oracle checks a sample of
(sequence, V head) units element by element (the whole output row range and the
final table of each sampled unit), at the same tolerances as the small cases.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gated_deltanet_recurrence_rule_amd import binding, workloads as W
from gdn_testutil import assert_parity, oracle_units, to_device, to_f64

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    binding.load()


def _run_and_check(inp, groups, what):
    """Run the whole batch once; check each (sequences, heads) group against the oracle."""
    d = to_device(inp)
    o, S = binding.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu"],
                           cu_seqlens_host=inp.cu_seqlens, S0=d["S0"], scale=inp.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    for seqs, heads in groups:
        ref = oracle_units(inp, seqs, heads)
        for (n, h), (o_ref, S_ref) in ref.items():
            t0, t1 = int(inp.cu_seqlens[n]), int(inp.cu_seqlens[n + 1])
            v_ref = inp.as_f64_rows("v", t0, t1)[:, h]
            assert_parity(to_f64(o[t0:t1, h]), to_f64(S[n, h]), o_ref, S_ref, v_ref, inp.dtype,
                          f"{what} seq {n} head {h}")


def test_single_sequence_8192():
    """1 x 8192 tokens, 16 heads (no sharing), dk = dv = 128, bf16, empty start table."""
    _say("full size: single sequence T=8192 H=16")
    inp = W.prefill()
    _run_and_check(inp, [([0], range(16))], "T=8192")


def test_qwen3next_shape():
    """4 x 16384 tokens, 16 QK / 32 V heads, bf16, S0 ~ N(0, 0.05); sampled units."""
    _say("full size: 4 x 16384, 16 QK / 32 V heads")
    inp = W.qwen3next()
    _run_and_check(inp, [([0, 3], [0, 1, 17, 30])], "qwen3next")


def test_varlen_with_long_tail():
    """64 log-uniform lengths in [128, 32768] plus one 262144-token sequence."""
    _say("full size: varlen 64 sequences + 262144")
    inp = W.varlen()
    lens = np.diff(inp.cu_seqlens)
    short = [int(i) for i in np.argsort(lens)[:3]] + [int(np.argsort(lens)[32])]
    _run_and_check(inp, [(short, [0, 5, 31]), ([inp.N - 1], [2, 29])], "varlen")


def test_decode_large_batch():
    """1024 sequences x 32 V heads (16 QK), d = 128: 32768 tables, 2 GiB of state, so every
    workgroup of the capped decode grid walks 32 tables.  Sampled units against the oracle;
    then every table and read against the same step run in slices of 16 sequences (512
    tables, one workgroup each, no walk), which must agree bit for bit: a table skipped or
    stepped twice by the walk cannot."""
    _say("full size: decode 1024 sequences x 32 heads")
    inp = W.decode(seed=12, N=1024)
    d = to_device(inp)
    S = d["S0"].clone()
    o = binding.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], S)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    ref = oracle_units(inp, [0, 1, 511, 1000, 1023], [0, 7, 16, 31])
    for (n, h), (o_ref, S_ref) in ref.items():
        v_ref = inp.as_f64_rows("v", n, n + 1)[:, h]
        assert_parity(to_f64(o[n:n + 1, h]), to_f64(S[n, h]), o_ref, S_ref, v_ref, "bf16",
                      f"decode seq {n} head {h}")
    for a in range(0, 1024, 16):
        b = a + 16
        Sb = d["S0"][a:b].clone()
        ob = binding.decode_step(d["q"][a:b], d["k"][a:b], d["v"][a:b], d["g"][a:b], d["beta"][a:b], Sb)
        torch.cuda.synchronize()
        assert torch.equal(ob, o[a:b]), f"reads of sequences {a}..{b - 1} differ from the sliced step"
        assert torch.equal(Sb, S[a:b]), f"tables of sequences {a}..{b - 1} differ from the sliced step"
