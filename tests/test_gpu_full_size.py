"""GPU parity at the measured workload sizes, through the C ABI.

The GPU runs every sequence and head in the launch configuration the benchmark times;
the float64 oracle then checks EVERY (sequence, V head) unit element by element: the
whole output row range and the final table of each unit, at the same tolerances as the
small cases.  The oracle runs in groups of sequences (and, for the 262144-token
sequence, of heads) so the float64 copies stay a few GB.

The batched prefill is also compared bit for bit with re-runs of slices of its
sequences.  A slice is padded with empty sequences so that it still fills the device, and
it is run without host lengths, so the sizes alone choose its plan: it runs unsplit on
64-column workgroups, as the batch runs every sequence but the longest of the packed
batch.  A workgroup that computed or wrote the wrong (sequence, head, columns) cannot
agree bit for bit with the re-run.  The packed batch's 262144-token sequence is cut into
segments in the batched call (its host lengths are given) and not in the re-run; the two
still agree bit for bit with these gates (log a about -0.2 per token on average): over a
segment of some 300 chunks each map's decay factor underflows to exactly zero in fp32, so
a segment starts from the previous segment's scan from a zero table, and a scan forgets
the bits of its start table within a few chunks.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gated_deltanet_recurrence_rule_amd import binding, workloads as W
from gdn_testutil import rows_f64, assert_parity, oracle_units, to_device, to_f64

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    binding.load()


def _run(inp, d):
    o, S = binding.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu"],
                           cu_seqlens_host=inp.cu_seqlens, S0=d["S0"], scale=inp.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    return o, S


def _check_all_units(inp, o, S, what, seq_groups, head_groups_for=None):
    """Oracle on every (sequence, V head) unit, in the given groups of sequences; a sequence
    listed in head_groups_for runs in those groups of heads instead of all heads at once."""
    o_host = o.cpu()  # one device-to-host copy; units are sliced on the host
    S_host = S.cpu()
    head_groups_for = head_groups_for or {}
    checked = 0
    for seqs in seq_groups:
        for n in seqs:
            groups = head_groups_for.get(n, [range(inp.HV)])
            for heads in groups:
                ref = oracle_units(inp, [n], heads)
                t0, t1 = int(inp.cu_seqlens[n]), int(inp.cu_seqlens[n + 1])
                for (n_, h), (o_ref, S_ref) in ref.items():
                    v_ref = rows_f64(inp.v[t0:t1, h])
                    assert_parity(to_f64(o_host[t0:t1, h]), to_f64(S_host[n_, h]), o_ref, S_ref, v_ref,
                                  inp.dtype, f"{what} seq {n_} head {h}")
                    checked += 1
    assert checked == inp.N * inp.HV
    return checked


def _padded_slice(inp, d, seqs, pad_to):
    """Re-run the sequences `seqs` (consecutive in the batch) as their own batch, followed by
    empty sequences up to pad_to sequences; returns (o of the slice's tokens, S_T of the slice)."""
    n0, n1 = seqs[0], seqs[-1] + 1
    t0, t1 = int(inp.cu_seqlens[n0]), int(inp.cu_seqlens[n1])
    lens = np.diff(inp.cu_seqlens[n0:n1 + 1]).astype(np.int64)
    npad = max(0, pad_to - len(seqs))
    cu = np.concatenate([[0], np.cumsum(lens), np.full(npad, t1 - t0)]).astype(np.int32)
    dev = d["q"].device
    sl = lambda x: x[t0:t1].contiguous()
    S0 = None
    if d["S0"] is not None:
        S0 = torch.zeros((len(cu) - 1,) + tuple(d["S0"].shape[1:]), dtype=torch.float32, device=dev)
        S0[:len(seqs)] = d["S0"][n0:n1]
    o, S = binding.prefill(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["g"]), sl(d["beta"]),
                           cu_seqlens=torch.from_numpy(cu).to(dev), S0=S0, scale=inp.scale)
    torch.cuda.synchronize()
    kname = binding.prefill_kernel_name(len(cu) - 1, t1 - t0, inp.HQK, inp.HV, inp.dk, inp.dv, torch.bfloat16)
    assert kname == "prefill_chunked", kname
    return o, S[:len(seqs)]


def _check_slices_bitwise(inp, d, o, S, slices, pad_to):
    for seqs in slices:
        t0, t1 = int(inp.cu_seqlens[seqs[0]]), int(inp.cu_seqlens[seqs[-1] + 1])
        os_, Ss = _padded_slice(inp, d, seqs, pad_to)
        assert torch.equal(os_, o[t0:t1]), f"reads of sequences {seqs} differ from the batched call"
        assert torch.equal(Ss, S[seqs[0]:seqs[-1] + 1]), f"tables of sequences {seqs} differ from the batched call"


def test_single_sequence_8192():
    """1 x 8192 tokens, 16 heads (no sharing), dk = dv = 128, bf16, empty start table (split path)."""
    _say("full size: single sequence T=8192 H=16")
    inp = W.prefill()
    d = to_device(inp)
    o, S = _run(inp, d)
    _check_all_units(inp, o, S, "T=8192", [[0]])


@pytest.mark.timeout(900)
def test_qwen3next_shape():
    """4 x 16384 tokens, 16 QK / 32 V heads, bf16, S0 ~ N(0, 0.05): all 128 units against the
    oracle, and each sequence re-run alone (padded with three empty sequences) bit for bit."""
    _say("full size: 4 x 16384, 16 QK / 32 V heads (all units)")
    inp = W.qwen3next()
    d = to_device(inp)
    o, S = _run(inp, d)
    assert binding.prefill_kernel_name(inp.N, inp.total_T, inp.HQK, inp.HV, 128, 128,
                                       torch.bfloat16) == "prefill_chunked"
    _say("  bit-identical per-sequence re-runs")
    _check_slices_bitwise(inp, d, o, S, [[n] for n in range(inp.N)], pad_to=4)
    _say("  oracle on all 128 units")
    _check_all_units(inp, o, S, "qwen3next", [[n] for n in range(inp.N)])


@pytest.mark.timeout(1200)
def test_varlen_with_long_tail():
    """64 log-uniform lengths in [128, 32768] plus one 262144-token sequence: every unit's reads
    and final table against the oracle; slices of 8 sequences (and the long one, padded)
    re-run bit for bit."""
    _say("full size: varlen 64 sequences + 262144 (all units)")
    inp = W.varlen()
    assert binding.prefill_kernel_name(inp.N, inp.total_T, inp.HQK, inp.HV, 128, 128, torch.bfloat16,
                                       cu_seqlens_host=inp.cu_seqlens) == "prefill_chunked_split"
    d = to_device(inp)
    o, S = _run(inp, d)
    N = inp.N
    _say("  bit-identical re-runs of sequence slices")
    slices = [list(range(a, min(a + 8, N - 1))) for a in range(0, N - 1, 8)] + [[N - 1]]
    _check_slices_bitwise(inp, d, o, S, slices, pad_to=4)
    _say("  oracle on all units")
    halves = [range(0, inp.HV // 2), range(inp.HV // 2, inp.HV)]
    _check_all_units(inp, o, S, "varlen", [list(range(N))], head_groups_for={N - 1: halves})


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


def test_decode_full_batch_all_units():
    """The 256-sequence decode batch the benchmark times: all 8192 tables and reads."""
    _say("full size: decode 256 sequences, all units")
    inp = W.decode()
    d = to_device(inp)
    S = d["S0"].clone()
    o = binding.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], S)
    torch.cuda.synchronize()
    ref = oracle_units(inp, range(inp.N), range(inp.HV))
    o_h, S_h = o.cpu(), S.cpu()
    for (n, h), (o_ref, S_ref) in ref.items():
        v_ref = rows_f64(inp.v[n:n + 1, h])
        assert_parity(to_f64(o_h[n:n + 1, h]), to_f64(S_h[n, h]), o_ref, S_ref, v_ref, "bf16",
                      f"decode B=256 seq {n} head {h}")
