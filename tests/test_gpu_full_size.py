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
