#!/usr/bin/env python3
"""Throughput of the gated delta-rule scan on one MI355X.

One step = one pass of the whole hot path on synthetic inputs already resident
in HBM:
  * prefill of the Qwen3-Next-shaped batch: 4 sequences x 16384 tokens, 16 QK
    heads shared by 32 V heads, dk = dv = 128, bf16 q/k/v/o, fp32 S0 -> S_T;
  * one decode step of 256 sequences with the same head layout, fp32 state
    (512 MiB) updated in place.

`value` is the prefill throughput in Mtok/s (prefill tokens / prefill time);
the decode leg is reported beside it as state GB/s (2 |S| / time).  Beside the
step, "block" reports the parts of the GatedDeltaNet block around the scan on
the same prefill batch: the causal convolution + SiLU (gdn_conv_silu), the gated
RMS norm (gdn_gated_rmsnorm), the prefill and decode calls with the gates taken
from raw projections (and, for decode, the norm fused).  Kernel
times come from HIP events recorded on the stream the library launches on.
Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json

import numpy as np
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0     # dense bf16 MFMA
PEAK_FP32_VALU_TFLOPS = 157.3  # fp32 vector
CHUNK_REF = 64                # chunk length the algorithmic flop count is quoted at


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def prefill_alg(N, T, HQK, HV, dk, dv, e, with_s0):
    """Algorithmic bytes and flops of one prefill call (inputs read once, outputs written once)."""
    r = HV // HQK
    tok_head = N * T * HV
    bytes_ = tok_head * ((2 * dk * e) / r + 2 * dv * e + 8) + N * HV * dk * dv * 4 * (2 if with_s0 else 1)
    flops_chunk = tok_head * (10 * CHUNK_REF * dk + 6 * dk * dv)
    flops_rec = tok_head * 7 * dk * dv
    return int(bytes_), int(flops_chunk), int(flops_rec)


def decode_alg(N, HQK, HV, dk, dv, e):
    bytes_ = N * HV * 2 * dk * dv * 4 + N * HQK * 2 * dk * e + N * HV * 2 * dv * e + N * HV * 8
    return int(bytes_), int(N * HV * 7 * dk * dv), int(N * HV * 2 * dk * dv * 4)


def conv_alg(T, N, Ct, e):
    """x read once, q | k | v written once, the carried state read and written."""
    return int(2 * T * Ct * e + 2 * N * 3 * Ct * e + Ct * 16)


def norm_alg(rows, dv, e):
    return int(3 * rows * dv * e + dv * 4)


def recorded_traffic(kernel: str):
    """HBM bytes per dispatch measured with rocprofv3 counters (profiles/traffic.json),
    or None when the kernel's source has changed since the counters were taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))["kernels"][kernel]
        src = os.path.join(ROOT, "gated_deltanet_recurrence_rule_amd", "csrc", rec["source"])
        if hashlib.sha256(open(src, "rb").read()).hexdigest() != rec["sha256"]:
            return None
        return float(rec["bytes"])
    except (OSError, KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--cpu-sample-seqs", type=int, default=4,
                    help="prefill sequences (all V heads) the CPU oracle baseline runs on (default: all 4)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="before the warm-up steps, run steps for at least this long so the GPU "
                         "reaches its sustained clock (untimed; 0 disables)")
    ap.add_argument("--no-block", action="store_true", help="skip the block-parts leg")
    ap.add_argument("--no-varlen", action="store_true",
                    help="skip the packed variable-length batch with its 262144-token sequence (by default "
                         "it is timed under extra_configs with the tiny fp32 scan and the single "
                         "8192-token sequence; its inputs take about half a minute to draw)")
    ap.add_argument("--only", choices=["tiny_fp32", "single_8192", "varlen"], default=None,
                    help="time only this one of the extra configurations and print its record (for a "
                         "kernel trace of that workload alone; not the benchmark line)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after timing, run one 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}): "
              "the scan shards by (sequence, head) with no exchange, so there is nothing "
              "multi-GPU to time here.", file=sys.stderr)
        sys.exit(2)

    import torch

    from gated_deltanet_recurrence_rule_amd import binding, workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = binding.load()

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    if args.only:
        rec = extra_leg(args, binding, W, up, dev, legs=[args.only])
        print(json.dumps({"only": args.only, "steps": args.steps, **rec[args.only]}), flush=True)
        return

    t0 = time.time()
    pf = W.qwen3next()
    dc = W.decode()
    log(f"inputs generated in {time.time() - t0:.1f} s")
    P = dict(q=up(pf.q), k=up(pf.k), v=up(pf.v), g=up(pf.g), beta=up(pf.beta),
             cu=up(pf.cu_seqlens), S0=up(pf.S0))
    D = dict(q=up(dc.q), k=up(dc.k), v=up(dc.v), g=up(dc.g), beta=up(dc.beta), S=up(dc.S0))
    N, T = pf.N, pf.total_T // pf.N
    o_p = torch.empty((pf.total_T, pf.HV, pf.dv), dtype=torch.bfloat16, device=dev)
    S_T = torch.empty((pf.N, pf.HV, pf.dk, pf.dv), dtype=torch.float32, device=dev)
    o_d = torch.empty((dc.N, dc.HV, dc.dv), dtype=torch.bfloat16, device=dev)
    ws_bytes = binding.prefill_workspace_size(pf.N, pf.total_T, pf.HQK, pf.HV, pf.dk, pf.dv,
                                              torch.bfloat16, cu_seqlens_host=pf.cu_seqlens)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def prefill():
        binding.prefill(P["q"], P["k"], P["v"], P["g"], P["beta"], cu_seqlens=P["cu"], cu_seqlens_host=pf.cu_seqlens,
                        S0=P["S0"], o=o_p, S_T=S_T, workspace=ws)

    def decode():
        binding.decode_step(D["q"], D["k"], D["v"], D["g"], D["beta"], D["S"], o=o_d)

    # Clock settle (untimed): the first ~10 ms of load run ~20% slower than sustained.  It
    # repeats the timed region's pattern (K prefill calls, then K decode steps), so that a
    # kernel trace of the whole run averages calls made the way the timed ones are: a decode
    # step launched right after the MFMA-heavy prefill runs ~10% slower than one after
    # another decode step.
    if args.settle_ms > 0:
        t_set = time.perf_counter()
        while (time.perf_counter() - t_set) * 1e3 < args.settle_ms:
            for _ in range(args.steps):
                prefill()
            for _ in range(args.steps):
                decode()
            torch.cuda.synchronize()
    for _ in range(args.warmup):
        prefill()
    for _ in range(args.warmup):
        decode()
    torch.cuda.synchronize()

    # Timed region: K prefill calls back to back, then K decode steps back to back,
    # bracketed by HIP events on the stream the library launches on (an event between
    # calls gives the per-call times for the median and minimum).
    stream = torch.cuda.current_stream(dev)
    ev_p = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ev_d = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev_p[0].record(stream)
    for i in range(args.steps):
        prefill()
        ev_p[i + 1].record(stream)
    for i in range(args.steps):
        decode()
        ev_d[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    e0, e1, e2 = ev_p[0], ev_p[-1], ev_d[-1]
    pre_avg = e0.elapsed_time(e1) / args.steps
    dec_avg = e1.elapsed_time(e2) / args.steps
    step_ms = e0.elapsed_time(e2) / args.steps
    pre_calls = sorted(ev_p[i].elapsed_time(ev_p[i + 1]) for i in range(args.steps))
    dec_calls = sorted((ev_p[-1] if i == 0 else ev_d[i - 1]).elapsed_time(ev_d[i]) for i in range(args.steps))

    block = None
    if not args.no_block:
        block = block_leg(args, binding, W, P, D, pf, dc, o_p, S_T, o_d, ws, up, dev)

    extra = extra_leg(args, binding, W, up, dev, with_varlen=not args.no_varlen)

    # A plain 1 GiB device copy: the measured copy bandwidth reported beside the peaks, and
    # (one call, --copy-probe) the known-size dispatch that scales the HBM counters.
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    copy_gbps = None
    if args.copy_probe:
        dst.copy_(src)
        torch.cuda.synchronize()
    else:
        for _ in range(3):
            dst.copy_(src)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for _ in range(10):
            dst.copy_(src)
        c1.record(stream)
        torch.cuda.synchronize()
        copy_gbps = 2.0 * (1 << 30) / (c0.elapsed_time(c1) / 10 * 1e-3) / 1e9
    del src, dst

    e = 2  # bf16 bytes
    pb, pf_chunk, pf_rec = prefill_alg(N, T, pf.HQK, pf.HV, pf.dk, pf.dv, e, True)
    db, dflops, dstate = decode_alg(dc.N, dc.HQK, dc.HV, dc.dk, dc.dv, e)
    kname = binding.prefill_kernel_name(pf.N, pf.total_T, pf.HQK, pf.HV, pf.dk, pf.dv, torch.bfloat16,
                                        cu_seqlens_host=pf.cu_seqlens)
    pre_roof = prefill_roofline(pb, pf_chunk, pf_rec, pre_avg, kname)
    pre_roof["traffic"] = recorded_traffic("prefill_chunked") if "chunk" in kname else None
    dec_gbps = db / (dec_avg * 1e-3) / 1e9
    dec_roof = {"bound": "hbm", "achieved": dec_gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": dec_gbps / PEAK_HBM_GBPS, "traffic": recorded_traffic("decode"), "kernel": "decode"}
    pre_hbm_frac = pb / (pre_avg * 1e-3) / 1e9 / PEAK_HBM_GBPS
    value = N * T / (pre_avg * 1e-3) / 1e6
    state_gbps = dstate / (dec_avg * 1e-3) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        ns = max(1, min(args.cpu_sample_seqs, N))
        ts = ns * T
        f64 = {x: pf.as_f64_rows(x, 0, ts) for x in ("q", "k", "v")}
        f64.update({x: getattr(pf, x)[:ts].astype(np.float64) for x in ("g", "beta")})
        s0 = pf.S0[:ns].astype(np.float64)
        t0 = time.perf_counter()
        oracle.run(f64["q"], f64["k"], f64["v"], f64["g"], f64["beta"], pf.cu_seqlens[:ns + 1], s0)
        tc = time.perf_counter() - t0
        d64 = {x: dc.as_f64(x) for x in ("q", "k", "v", "g", "beta", "S0")}
        t1 = time.perf_counter()
        oracle.run(d64["q"], d64["k"], d64["v"], d64["g"], d64["beta"], dc.cu_seqlens, d64["S0"])
        td = time.perf_counter() - t1
        cpu = {"value": ts / tc / 1e6, "unit": "Mtok/s", "cores": oracle.threads(), "kind": "oracle",
               "sample": f"float64 token loop on the first {ns} of the {N} prefill sequences "
                         f"({ts} tokens, all {pf.HV} V heads, {tc:.2f} s); decode leg: the full "
                         f"256-sequence step "
                         f"({td:.2f} s)",
               "decode_state_GBps": dstate / td / 1e9}
        log(f"cpu oracle: {ts} tokens in {tc:.2f} s, decode step in {td:.2f} s")

    out = {
        "metric": "prefill Mtok/s + decode state GB/s on 1 GPU, as % of MFMA/HBM roofline",
        "value": value, "unit": "Mtok/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": step_ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Qwen3-Next-shaped prefill (4 x 16384 tokens, 16 QK / 32 V heads, "
                               "dk=dv=128, bf16, fp32 S0) + decode step (256 sequences, same heads, "
                               "512 MiB fp32 state)",
                   "prefill_tokens": N * T, "decode_sequences": dc.N, "parallelism": "none"},
        "prefill_ms": pre_avg, "prefill_ms_median": pre_calls[len(pre_calls) // 2],
        "prefill_ms_min": pre_calls[0], "prefill_hbm_frac": pre_hbm_frac,
        "prefill_mfma_frac": pre_roof.get("mfma_frac"),
        "prefill_roofline_frac": max(pf_chunk / (PEAK_BF16_TFLOPS * 1e12), pb / (PEAK_HBM_GBPS * 1e9)) / (pre_avg * 1e-3),
        "prefill_recurrence_TFLOPs": pf_rec / (pre_avg * 1e-3) / 1e12,
        "decode_us": dec_avg * 1e3, "decode_us_median": dec_calls[len(dec_calls) // 2] * 1e3,
        "decode_us_min": dec_calls[0] * 1e3, "decode_state_GBps": state_gbps,
        "copy_GBps": copy_gbps,
        "roofline": pre_roof if pre_avg >= dec_avg else dec_roof,
        "roofline_prefill": pre_roof, "roofline_decode": dec_roof,
        "cpu_baseline": cpu,
        "block": block,
        "extra_configs": extra,
        "host": {"cpu": host_cpu(), "cpu_count": os.cpu_count()},
        "wall_s_timed": wall,
    }
    print(json.dumps(out), flush=True)


def prefill_roofline(alg_bytes, flops_chunk, flops_rec, ms, kname):
    """Roofline of one prefill call.  Its algorithmic arithmetic intensity (flops_chunk /
    alg_bytes, ~230 flop/B at d = 128) lies below the bf16 ridge (2500 TFLOP/s / 8 TB/s =
    312 flop/B), so HBM is the binding roof: `frac` = algorithmic bytes / time / 8 TB/s.  The
    bf16 MFMA fraction (algorithmic chunk-form flops / time / 2500 TFLOP/s) is reported beside
    it.  The token-serial kernel (fp32 inputs) is bound by fp32 vector arithmetic instead:
    its recurrence flops (7 dk dv per token and head) against the fp32 vector peak."""
    t = ms * 1e-3
    hbm = alg_bytes / t / 1e9
    out = {"bound": "hbm", "achieved": hbm, "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": hbm / PEAK_HBM_GBPS,
           "alg_bytes": int(alg_bytes), "kernel": kname}
    if "chunk" in kname:
        out["mfma_achieved_TFLOPs"] = flops_chunk / t / 1e12
        out["mfma_frac"] = flops_chunk / t / 1e12 / PEAK_BF16_TFLOPS
        out["alg_flops"] = int(flops_chunk)
    else:
        alu = flops_rec / t / 1e12
        out.update({"bound": "alu", "achieved": alu, "peak": PEAK_FP32_VALU_TFLOPS, "unit": "TFLOP/s",
                    "frac": alu / PEAK_FP32_VALU_TFLOPS, "hbm_frac": hbm / PEAK_HBM_GBPS,
                    "alg_flops": int(flops_rec)})
    return out


def host_cpu():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def extra_leg(args, binding, W, up, dev, with_varlen=False, legs=None):
    """The other workloads, each timed over K calls between HIP events after a short settle
    (all of them, or only those named in `legs`)."""
    import torch

    out = {}
    stream = torch.cuda.current_stream(dev)
    makers = {"tiny_fp32": W.tiny, "single_8192": W.prefill, "varlen": W.varlen}
    if legs is None:
        legs = ["tiny_fp32", "single_8192"] + (["varlen"] if with_varlen else [])
    for name in legs:
        make = makers[name]
        t0 = time.time()
        inp = make()
        log(f"{name}: inputs generated in {time.time() - t0:.1f} s")
        d = {x: up(getattr(inp, x)) for x in ("q", "k", "v", "g", "beta")}
        cu = up(inp.cu_seqlens)
        S0 = None if inp.S0 is None else up(inp.S0)
        tdt = torch.bfloat16 if inp.dtype == "bf16" else torch.float32
        o = torch.empty((inp.total_T, inp.HV, inp.dv), dtype=tdt, device=dev)
        ST = torch.empty((inp.N, inp.HV, inp.dk, inp.dv), dtype=torch.float32, device=dev)
        nws = binding.prefill_workspace_size(inp.N, inp.total_T, inp.HQK, inp.HV, inp.dk, inp.dv, tdt,
                                             cu_seqlens_host=inp.cu_seqlens)
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)

        def call():
            binding.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=cu,
                            cu_seqlens_host=inp.cu_seqlens, S0=S0, o=o, S_T=ST, workspace=ws)

        t_set = time.perf_counter()
        while (time.perf_counter() - t_set) * 1e3 < max(args.settle_ms, 1.0):
            call()
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        e = 2 if inp.dtype == "bf16" else 4
        lens = np.diff(inp.cu_seqlens)
        ab = sum(prefill_alg(1, int(L), inp.HQK, inp.HV, inp.dk, inp.dv, e, inp.S0 is not None)[0] for L in lens)
        fl = sum(prefill_alg(1, int(L), inp.HQK, inp.HV, inp.dk, inp.dv, e, False)[1] for L in lens)
        fr = sum(prefill_alg(1, int(L), inp.HQK, inp.HV, inp.dk, inp.dv, e, False)[2] for L in lens)
        kname = binding.prefill_kernel_name(inp.N, inp.total_T, inp.HQK, inp.HV, inp.dk, inp.dv, tdt,
                                            cu_seqlens_host=inp.cu_seqlens)
        roof = prefill_roofline(ab, fl, fr, ms, kname)
        out[name] = {"sequences": inp.N, "tokens": inp.total_T, "heads": [inp.HQK, inp.HV], "d": [inp.dk, inp.dv],
                     "dtype": inp.dtype, "kernel": kname, "ms": ms, "Mtok_s": inp.total_T / (ms * 1e-3) / 1e6,
                     "mfma_frac": roof.get("mfma_frac"),
                     "hbm_frac": ab / (ms * 1e-3) / (PEAK_HBM_GBPS * 1e9), "roofline": roof}
        del d, o, ST, ws, S0, cu
        torch.cuda.empty_cache()
    return out


def block_leg(args, binding, W, P, D, pf, dc, o_p, S_T, o_d, ws, up, dev):
    """Time the block parts on the prefill batch (K calls each between HIP events)."""
    import torch

    t0 = time.time()
    bi = W.block_inputs(7, [pf.total_T // pf.N] * pf.N, pf.HQK, pf.HV, pf.dk, pf.dv)
    bd = W.block_inputs(8, [1] * dc.N, dc.HQK, dc.HV, dc.dk, dc.dv)
    log(f"block inputs generated in {time.time() - t0:.1f} s")
    x, w, st_in = up(bi.x), up(bi.conv_w), up(bi.conv_state)
    st_out = torch.empty_like(st_in)
    z, nw = up(bi.z), up(bi.norm_w)
    a, b, A_log, dt_bias = up(bi.a), up(bi.b), up(bi.A_log), up(bi.dt_bias)
    zd, ad, bd_, nwd = up(bd.z), up(bd.a), up(bd.b), up(bd.norm_w)
    Ad, dtd = up(bd.A_log), up(bd.dt_bias)
    q = torch.empty_like(P["q"])
    k = torch.empty_like(P["k"])
    v = torch.empty_like(P["v"])
    y = torch.empty_like(o_p)
    T, Ct = bi.x.shape

    def conv():
        binding.conv_silu(x, w, HQK=pf.HQK, HV=pf.HV, dk=pf.dk, dv=pf.dv, cu_seqlens=P["cu"],
                          state_in=st_in, state_out=st_out, q=q, k=k, v=v)

    def norm():
        binding.gated_rmsnorm(o_p, z, nw, 1e-6, y=y)

    def prefill_raw():
        binding.prefill(P["q"], P["k"], P["v"], a, b, cu_seqlens=P["cu"], cu_seqlens_host=pf.cu_seqlens,
                        S0=P["S0"], o=o_p, S_T=S_T, workspace=ws, A_log=A_log, dt_bias=dt_bias,
                        beta_logits=True)

    Sd = D["S"].clone()

    def decode_block():
        binding.decode_step(D["q"], D["k"], D["v"], ad, bd_, Sd, o=o_d, A_log=Ad, dt_bias=dtd,
                            beta_logits=True, z=zd, norm_w=nwd, norm_eps=1e-6)

    stream = torch.cuda.current_stream(dev)
    # the input generation above left the GPU idle: settle its clock again (untimed)
    if args.settle_ms > 0:
        t_set = time.perf_counter()
        while (time.perf_counter() - t_set) * 1e3 < args.settle_ms:
            conv()
            norm()
            prefill_raw()
            torch.cuda.synchronize()
    res = {}
    for name, f in (("conv", conv), ("norm", norm), ("prefill_raw_gates", prefill_raw),
                    ("decode_raw_gates_norm", decode_block)):
        for _ in range(max(1, args.warmup)):
            f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / args.steps
    cb = conv_alg(T, pf.N, Ct, 2)
    nb = norm_alg(pf.total_T * pf.HV, pf.dv, 2)

    def hbm(bytes_, ms, key):
        gbps = bytes_ / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": gbps / PEAK_HBM_GBPS, "traffic": recorded_traffic(key), "alg_bytes": bytes_}

    return {
        "workload": f"{pf.N} x {pf.total_T // pf.N} tokens, {Ct} conv channels (16 QK / 32 V heads, d 128), bf16",
        "conv_silu_us": res["conv"] * 1e3, "conv_silu_roofline": hbm(cb, res["conv"], "conv_silu"),
        "gated_rmsnorm_us": res["norm"] * 1e3, "gated_rmsnorm_roofline": hbm(nb, res["norm"], "gated_rmsnorm"),
        "prefill_raw_gates_ms": res["prefill_raw_gates"],
        "decode_raw_gates_norm_us": res["decode_raw_gates_norm"] * 1e3,
    }


if __name__ == "__main__":
    main()
