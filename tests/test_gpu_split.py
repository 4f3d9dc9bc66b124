"""GPU parity of split sequences: a batch too small to fill the GPU has each sequence cut
into segments.  The first is scanned from the start table while the affine maps of the middle
ones (S_out = M S_in + B, from the recurrence of the handbook page "7. Gated DeltaNet: the
token-by-token recurrence", section "The formula") are formed in parallel; the maps are
chained from the first segment's final table, and every later segment is then scanned from
its start table.  The result must match the float64 oracle's token loop to the same
tolerances as the unsplit path.
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


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    binding.load()


def _split_ws(inp):
    """Bytes of the split workspace part (the order part is at most 256 bytes per 64 sequences)."""
    return binding.prefill_workspace_size(inp.N, inp.total_T, inp.HQK, inp.HV, inp.dk, inp.dv, torch.bfloat16)


@pytest.mark.parametrize("lens,HQK,HV,s0,variant", [
    ([3000], 1, 2, True, "gated_delta"),          # one sequence, last segment partial
    ([5000, 700], 2, 4, True, "gated_delta"),      # the short sequence ends in empty segments
    ([2600, 2600], 1, 1, False, "gated_delta"),    # no start table
    ([4100], 2, 4, True, "linear"),                # no look-up, no decay
    ([3500], 1, 2, True, "delta"),                 # no decay
])
def test_split_prefill(lens, HQK, HV, s0, variant):
    _say(f"split prefill lens={lens} HQK={HQK} HV={HV} s0={s0} variant={variant}")
    inp = W.random_small(81, lens, HQK, HV, 128, 128, dtype="bf16", s0=s0)
    need = _split_ws(inp)
    assert need > 64 * 1024, "this batch is expected to take the split path"
    d = to_device(inp)
    gated = variant in ("gated_delta", "gated_linear")
    look = variant in ("gated_delta", "delta")
    o, S = binding.prefill(d["q"], d["k"], d["v"], d["g"] if gated else None, d["beta"] if look else None,
                           cu_seqlens=d["cu"], cu_seqlens_host=inp.cu_seqlens, S0=d["S0"], scale=inp.scale,
                           variant=variant)
    torch.cuda.synchronize()
    g = inp.as_f64("g") if gated else np.zeros_like(inp.g, dtype=np.float64)
    b = inp.as_f64("beta") if look else np.ones_like(inp.beta, dtype=np.float64)
    o_ref, S_ref = oracle.run(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"), g, b, inp.cu_seqlens,
                              inp.as_f64("S0"), scale=inp.scale, delta=look)
    assert_parity(to_f64(o), to_f64(S), o_ref, S_ref, inp.as_f64("v"), "bf16", f"split {lens} {variant}",
                  grows=not look)


def _split_plan_P(inp):
    """P of the library's split plan, from the workspace size (maps of P - 2 segments and start
    tables of P - 1, each part rounded to 256 bytes, after the launch order's 256 bytes)."""
    need = _split_ws(inp)
    order = 256 if 1 < inp.N <= 16384 else 0
    per_map = inp.N * inp.HV * inp.dk * (inp.dv + inp.dk) * 4
    per_start = inp.N * inp.HV * inp.dk * inp.dv * 4
    r = lambda x: (x + 255) // 256 * 256
    for P in range(3, 17):
        if need == order + r((P - 2) * per_map) + r((P - 1) * per_start):
            return P
    return 1


@pytest.mark.parametrize("lens,HQK,HV,P", [
    ([8192] * 16, 2, 4, 3),      # 128 workgroups: one middle segment, its maps two rounds beside segment 0
    ([8192], 16, 16, 9),         # the 8192-token workload's plan
])
def test_split_prefill_weak_decay(lens, HQK, HV, P):
    """Decay close to 1 (a = sigmoid(N(8, 1))): a segment's map M stays far from zero, so the start
    tables depend on how the chain applies it to segment 0's final table."""
    _say(f"split prefill, weak decay: lens={lens[0]} x {len(lens)} HQK={HQK} HV={HV}")
    inp = W.random_small(85, lens, HQK, HV, 128, 128, dtype="bf16", s0=True, g_mu=8.0, g_sd=1.0)
    assert _split_plan_P(inp) == P
    d = to_device(inp)
    o, S = binding.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu"],
                           cu_seqlens_host=inp.cu_seqlens, S0=d["S0"], scale=inp.scale)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.run(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"), inp.as_f64("g"),
                              inp.as_f64("beta"), inp.cu_seqlens, inp.as_f64("S0"), scale=inp.scale)
    assert_parity(to_f64(o), to_f64(S), o_ref, S_ref, inp.as_f64("v"), "bf16", f"split weak decay P={P}")


# One sequence, one head: the planner picks every segment count from 4 to 16 as the length
# grows (P = 3 is covered above), so each unrolled chain kernel (P - 2 steps) runs once.
_EVERY_P = [(4, 1024), (5, 1280), (6, 1152), (7, 1664), (8, 2048), (9, 2304), (10, 3200), (11, 4096),
            (12, 4608), (13, 4992), (14, 6272), (15, 7552), (16, 8192)]


@pytest.mark.parametrize("P,T", _EVERY_P, ids=lambda x: str(x))
def test_split_prefill_every_segment_count(P, T):
    """Weak decay (maps far from zero), one head: every chain length the planner can choose."""
    _say(f"split prefill, every segment count: P={P} T={T}")
    inp = W.random_small(86 + P, [T], 1, 1, 128, 128, dtype="bf16", s0=True, g_mu=8.0, g_sd=1.0)
    assert _split_plan_P(inp) == P
    d = to_device(inp)
    o, S = binding.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu"],
                           cu_seqlens_host=inp.cu_seqlens, S0=d["S0"], scale=inp.scale)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.run(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"), inp.as_f64("g"),
                              inp.as_f64("beta"), inp.cu_seqlens, inp.as_f64("S0"), scale=inp.scale)
    assert_parity(to_f64(o), to_f64(S), o_ref, S_ref, inp.as_f64("v"), "bf16", f"split every P={P}")


@pytest.mark.parametrize("lens,HQK,HV,P", [([2048, 2048], 1, 2, 8), ([1500, 1500], 1, 3, 6)],
                         ids=["2x2048_h1-2", "2x1500_h1-3"])
def test_split_prefill_weak_decay_dv64(lens, HQK, HV, P):
    """dv = 64 (four 16-column chain blocks of a 192-column map row), grouped heads, two split
    sequences, maps far from zero."""
    _say(f"split prefill, weak decay, dv=64: lens={lens} HQK={HQK} HV={HV}")
    inp = W.random_small(87, lens, HQK, HV, 128, 64, dtype="bf16", s0=True, g_mu=8.0, g_sd=1.0)
    assert _split_plan_P(inp) == P
    d = to_device(inp)
    o, S = binding.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu"],
                           cu_seqlens_host=inp.cu_seqlens, S0=d["S0"], scale=inp.scale)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.run(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"), inp.as_f64("g"),
                              inp.as_f64("beta"), inp.cu_seqlens, inp.as_f64("S0"), scale=inp.scale)
    assert_parity(to_f64(o), to_f64(S), o_ref, S_ref, inp.as_f64("v"), "bf16", f"split weak decay dv=64 P={P}")


def test_split_prefill_equal_lengths_in_place_raw_gates():
    """cu_seqlens NULL (equal lengths), the final table written over the start table, gates from
    raw projections: the split path reads S0 only before its segment pass."""
    _say("split prefill: equal lengths, in place, raw gates")
    lens = [2304, 2304]
    inp = W.random_small(82, lens, 1, 2, 128, 128, dtype="bf16", s0=True)
    bi = W.block_inputs(83, lens, 1, 2, 128, 128, "bf16")
    d = to_device(inp)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    S = d["S0"].clone()
    o, S2 = binding.prefill(d["q"], d["k"], d["v"], dev(bi.a), dev(bi.b), N=2, S0=S, S_T=S,
                            A_log=dev(bi.A_log), dt_bias=dev(bi.dt_bias), beta_logits=True)
    torch.cuda.synchronize()
    g, beta = shell.gates_np(bi.a, bi.b, bi.A_log, bi.dt_bias)
    o_ref, S_ref = oracle.run(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"), g, beta, inp.cu_seqlens,
                              inp.as_f64("S0"))
    assert S2.data_ptr() == S.data_ptr()
    assert_parity(to_f64(o), to_f64(S), o_ref, S_ref, inp.as_f64("v"), "bf16", "split in place")


def test_split_deterministic():
    """Two calls on a split batch give bit-identical reads and tables."""
    inp = W.random_small(84, [3000], 1, 2, 128, 128, dtype="bf16", s0=True)
    d = to_device(inp)
    kw = dict(cu_seqlens=d["cu"], cu_seqlens_host=inp.cu_seqlens, S0=d["S0"], scale=inp.scale)
    o1, S1 = binding.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], **kw)
    o2, S2 = binding.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
