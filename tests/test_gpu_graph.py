"""The C-ABI calls under HIP graph capture (torch.cuda.CUDAGraph), for serving loops that
replay a captured step instead of launching it.

Each call enqueues only kernels on the caller's stream (no allocation, no memset, no host
synchronisation), so it can be captured.  Each test replays the graph several times, with
eager work and synchronisations of the program in between, refills the captured input
buffers between replays, and checks every replay against the same call made eagerly.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gated_deltanet_recurrence_rule_amd import binding, workloads as W
from gdn_testutil import to_device

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    binding.load()


def test_decode_step_graph_replays():
    _say("graph: decode step, 3 replays")
    inputs = [to_device(W.make_inputs("dec", 90 + i, [1] * 16, 2, 4, 128, 128, "bf16", 3.0, 1.0, 0.05))
              for i in range(3)]
    static = {k: v.clone() for k, v in inputs[0].items() if k != "cu" and v is not None}
    S_static = static["S0"].clone()
    o_static = torch.empty((16, 4, 128), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):               # warm-up outside capture
        binding.decode_step(static["q"], static["k"], static["v"], static["g"], static["beta"],
                            S_static.clone(), o=o_static)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        binding.decode_step(static["q"], static["k"], static["v"], static["g"], static["beta"], S_static,
                            o=o_static)
    for i, d in enumerate(inputs):
        for k in ("q", "k", "v", "g", "beta"):
            static[k].copy_(d[k])
        S_static.copy_(d["S0"])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        S_eager = d["S0"].clone()
        o_eager = binding.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], S_eager)
        torch.cuda.synchronize()
        assert torch.equal(o_static, o_eager), f"replay {i}: reads differ from the eager call"
        assert torch.equal(S_static, S_eager), f"replay {i}: tables differ from the eager call"


def test_prefill_graph_replays():
    _say("graph: prefill with varlen order workspace, 3 replays")
    lens = [70, 200, 5]                          # increasing lengths: the order kernel runs
    inputs = [W.random_small(95 + i, lens, 2, 4, 128, 128, dtype="bf16", s0=True) for i in range(3)]
    devs = [to_device(x) for x in inputs]
    static = {k: v.clone() for k, v in devs[0].items() if v is not None}
    o_static = torch.empty_like(static["v"])
    ST_static = torch.empty_like(static["S0"])
    nws = binding.prefill_workspace_size(len(lens), sum(lens), 2, 4, 128, 128, torch.bfloat16)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")

    def call():
        binding.prefill(static["q"], static["k"], static["v"], static["g"], static["beta"],
                        cu_seqlens=static["cu"], S0=static["S0"], o=o_static, S_T=ST_static, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for i, (inp, d) in enumerate(zip(inputs, devs)):
        for k in ("q", "k", "v", "g", "beta", "S0"):
            static[k].copy_(d[k])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        o_e, S_e = binding.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu"],
                                   cu_seqlens_host=inp.cu_seqlens, S0=d["S0"])
        torch.cuda.synchronize()
        assert torch.equal(o_static, o_e), f"replay {i}: reads differ from the eager call"
        assert torch.equal(ST_static, S_e), f"replay {i}: tables differ from the eager call"
        # some eager work of the program between replays
        _ = (o_e.float() * 2).sum().item()


@pytest.mark.parametrize("lens,HQK,HV,host", [
    ([3000], 1, 2, False),                        # the sizes' plan splits every sequence
    ([64, 0, 6000, 100, 700, 300, 500], 8, 16, True),  # the host lengths split the longest
], ids=["split_by_sizes", "longest_split_by_lengths"])
def test_split_prefill_graph_replays(lens, HQK, HV, host):
    """Split sequences under capture: the segment-map pass, the chain and the segment pass (and,
    for the shuffled batch, the order kernel) in one graph, the maps and start tables in the
    caller's workspace."""
    _say(f"graph: split prefill {lens} HQK={HQK} HV={HV}, 3 replays")
    inputs = [W.random_small(130 + i, lens, HQK, HV, 128, 128, dtype="bf16", s0=True) for i in range(3)]
    devs = [to_device(x) for x in inputs]
    hl = inputs[0].cu_seqlens if host else None
    assert binding.prefill_kernel_name(len(lens), sum(lens), HQK, HV, 128, 128, torch.bfloat16,
                                       cu_seqlens_host=hl) == "prefill_chunked_split"
    static = {k: v.clone() for k, v in devs[0].items() if v is not None}
    o_static = torch.empty_like(static["v"])
    ST_static = torch.empty_like(static["S0"])
    nws = binding.prefill_workspace_size(len(lens), sum(lens), HQK, HV, 128, 128, torch.bfloat16,
                                         cu_seqlens_host=hl)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")

    def call():
        binding.prefill(static["q"], static["k"], static["v"], static["g"], static["beta"], cu_seqlens=static["cu"],
                        cu_seqlens_host=hl, S0=static["S0"], o=o_static, S_T=ST_static, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for i, (inp, d) in enumerate(zip(inputs, devs)):
        for k in ("q", "k", "v", "g", "beta", "S0"):
            static[k].copy_(d[k])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        o_e, S_e = binding.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu"],
                                   cu_seqlens_host=hl, S0=d["S0"])
        torch.cuda.synchronize()
        assert torch.equal(o_static, o_e), f"replay {i}: reads differ from the eager call"
        assert torch.equal(ST_static, S_e), f"replay {i}: tables differ from the eager call"
        _ = (o_e.float() * 2).sum().item()


def test_block_parts_graph_replays():
    """The causal convolution + SiLU (carried state in and out) and the gated RMS norm of its v
    channels, captured together."""
    _say("graph: conv + SiLU and gated norm, 3 replays")
    HQK, HV, d = 2, 4, 64
    lens = [40, 3, 90]
    T = sum(lens)

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda")
        return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")

    blocks = [W.block_inputs(120 + i, lens, HQK, HV, d, d) for i in range(3)]
    devs = [dict(x=up(b.x), w=up(b.conv_w), st=up(b.conv_state), z=up(b.z), nw=up(b.norm_w),
                 cu=up(b.cu_seqlens)) for b in blocks]
    static = {k: v.clone() for k, v in devs[0].items()}
    q = torch.empty((T, HQK, d), dtype=torch.bfloat16, device="cuda")
    k = torch.empty_like(q)
    v = torch.empty((T, HV, d), dtype=torch.bfloat16, device="cuda")
    st_out = torch.empty_like(static["st"])
    y = torch.empty_like(v)

    def call():
        binding.conv_silu(static["x"], static["w"], HQK=HQK, HV=HV, dk=d, dv=d, cu_seqlens=static["cu"],
                          state_in=static["st"], state_out=st_out, q=q, k=k, v=v)
        binding.gated_rmsnorm(v, static["z"], static["nw"], 1e-6, y=y)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for i, dv_ in enumerate(devs):
        for key in ("x", "w", "st", "z", "nw"):
            static[key].copy_(dv_[key])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        st_e = torch.empty_like(dv_["st"])
        qe, ke, ve = binding.conv_silu(dv_["x"], dv_["w"], HQK=HQK, HV=HV, dk=d, dv=d, cu_seqlens=dv_["cu"],
                                       state_in=dv_["st"], state_out=st_e)
        ye = binding.gated_rmsnorm(ve, dv_["z"], dv_["nw"], 1e-6)
        torch.cuda.synchronize()
        for got, want, what in ((q, qe, "q"), (k, ke, "k"), (v, ve, "v"), (st_out, st_e, "state"), (y, ye, "norm")):
            assert torch.equal(got, want), f"replay {i}: {what} differs from the eager call"
        _ = (ye.float() * 2).sum().item()
