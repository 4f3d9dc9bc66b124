"""The allocation-free prefill entry point (gdn_prefill_noalloc) against gdn_prefill_ex.

gdn_prefill_noalloc runs the same kernels with the library's static device scratch in
place of the caller's workspace, so on the same inputs its reads and final tables must
equal gdn_prefill_ex's bit for bit.  Two calls in a row on one device share that
scratch: the first needs most of it (a single sequence cut into segments, whose maps
and start tables live there), the second is smaller (a variable-length batch whose
longest-first launch order lives there).  A further call whose workspace would exceed
the scratch is rejected before anything runs.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
from gated_deltanet_recurrence_rule_amd import binding, workloads as W
from gdn_testutil import assert_parity, oracle_units, rows_f64, to_device, to_f64

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 24 << 20


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    binding.load()


def _both(inp, variant="gated_delta"):
    d = to_device(inp)
    kw = dict(cu_seqlens=d["cu"], cu_seqlens_host=inp.cu_seqlens, S0=d["S0"], scale=inp.scale, variant=variant)
    o_ref, S_ref = binding.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], **kw)
    o = torch.full_like(o_ref, float("nan"))
    S = torch.full_like(S_ref, float("nan"))
    binding.prefill_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], o=o, S_T=S, **kw)
    torch.cuda.synchronize()
    return o_ref, S_ref, o, S


def test_noalloc_equals_workspace_entry_on_two_calls():
    # first call: one 8192-token sequence, 16 heads: split into 9 segments, 22 MiB of maps
    # and start tables in the scratch
    big = W.prefill()
    need = binding.prefill_workspace_size(big.N, big.total_T, big.HQK, big.HV, big.dk, big.dv, torch.bfloat16)
    assert 16 << 20 < need <= SCRATCH_BYTES
    _say(f"noalloc call 1: 1 x 8192 tokens, 16 heads (workspace {need} bytes)")
    o_ref, S_ref, o, S = _both(big)
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
    ref = oracle_units(big, [0], [0, 15])
    for (n, h), (oo, ss) in ref.items():
        assert_parity(to_f64(o[:, h]), to_f64(S[n, h]), oo, ss, rows_f64(big.v[:, h]), "bf16", f"noalloc head {h}")

    # second call, smaller: unsorted lengths (the order kernel writes the scratch's first bytes)
    small = W.random_small(77, [70, 300, 5, 129], 2, 4, 128, 128, dtype="bf16")
    need2 = binding.prefill_workspace_size(small.N, small.total_T, small.HQK, small.HV, 128, 128, torch.bfloat16)
    assert 0 < need2 < need
    _say(f"noalloc call 2: 4 sequences (workspace {need2} bytes)")
    o_ref, S_ref, o, S = _both(small)
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)

    # a third, on the rule without the look-up and the token-serial kernel (fp32)
    f32 = W.random_small(78, [40, 3], 1, 2, 64, 64, dtype="f32")
    _say("noalloc call 3: fp32, token-serial kernel")
    o_ref, S_ref, o, S = _both(f32, variant="gated_linear")
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)


def test_noalloc_takes_the_lengths_plan():
    """A packed batch whose longest sequence outlasts the rest: given the host lengths, the
    allocation-free entry splits that sequence from its static scratch exactly as gdn_prefill_ex
    does with the workspace gdn_prefill_workspace_size_lens reports (shuffled lengths: the order
    kernel writes the scratch's first bytes, maps and start tables follow)."""
    lens = [64, 0, 6000, 100, 700, 300, 500]
    inp = W.random_small(80, lens, 8, 16, 128, 128, dtype="bf16")
    assert binding.prefill_kernel_name(inp.N, inp.total_T, 8, 16, 128, 128, torch.bfloat16,
                                       cu_seqlens_host=inp.cu_seqlens) == "prefill_chunked_split"
    need = binding.prefill_workspace_size(inp.N, inp.total_T, 8, 16, 128, 128, torch.bfloat16,
                                          cu_seqlens_host=inp.cu_seqlens)
    assert 16 << 20 < need <= SCRATCH_BYTES
    _say(f"noalloc, longest sequence split: {len(lens)} sequences (workspace {need} bytes)")
    o_ref, S_ref, o, S = _both(inp)
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
    o_or, S_or = oracle.run_inputs(inp)
    assert_parity(to_f64(o), to_f64(S), o_or, S_or, inp.as_f64("v"), "bf16", "noalloc longest split")


def test_noalloc_rejects_workspace_beyond_the_scratch():
    # a split batch (4096 tokens, 16 QK / 32 V heads of dv = 64) whose maps and start tables
    # need ~29 MiB
    T = 4096
    need = binding.prefill_workspace_size(1, T, 16, 32, 128, 64, torch.bfloat16)
    assert need > SCRATCH_BYTES
    inp = W.random_small(79, [T], 16, 32, 128, 64, dtype="bf16", s0=False)
    d = to_device(inp)
    o = torch.zeros((T, 32, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(binding.GdnError) as e:
        binding.prefill_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], N=1, o=o)
    assert e.value.status == -7 and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(o)) == 0  # nothing ran
