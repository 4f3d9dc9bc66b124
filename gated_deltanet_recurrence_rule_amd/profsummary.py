"""Summarise rocprofv3 runs of bench.py into the text records kept under profiles/.

Three runs feed it (each writes CSV files into its own directory):

  kernel times   rocprofv3 --kernel-trace --stats --output-format csv -d <KT> -o bench -- \
                     python3 bench.py --steps 5 --warmup 1 --no-cpu-baseline
  HBM reads      timeout -s KILL 180 rocprofv3 --pmc FETCH_SIZE --output-format csv -d <FETCH> -o bench -- \
                     python3 bench.py --steps 2 --warmup 1 --settle-ms 0 --no-cpu-baseline --copy-probe
  HBM writes     timeout -s KILL 180 rocprofv3 --pmc WRITE_SIZE --output-format csv -d <WRITE> -o bench -- \
                     python3 bench.py --steps 2 --warmup 1 --settle-ms 0 --no-cpu-baseline --copy-probe

and, for the MFMA evidence of the prefill kernel (optional),

  MFMA use       timeout -s KILL 180 rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 --output-format csv -d <MFMA> -o bench -- \
                     python3 bench.py --steps 2 --warmup 1 --settle-ms 0 --no-cpu-baseline --no-block

then

  python3 -m gated_deltanet_recurrence_rule_amd.profsummary <KT> <FETCH> <WRITE> [--mfma <MFMA>] [--out profiles]

writes one summary per kernel and traffic.json.  The counters are per dispatch, in KiB;
each is scaled by (1 GiB / what the same counter read for the plain 1 GiB device copy
that --copy-probe runs), so both are in bytes of HBM traffic.  traffic.json records the
sha256 of each kernel's source; bench.py reports the traffic only while it matches.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_deltanet_recurrence_rule_amd", "csrc")

KERNELS = {
    # key: (kernel-name fragment, source file, summary file, workload text)
    "prefill_chunked": ("prefill_chunked_kernel<true, false>", "prefill_chunked.hip", "prefill_chunked_qwen3next_4x16384.txt",
                        "prefill, 4 sequences x 16384 tokens, 16 QK / 32 V heads, dk = dv = 128, "
                        "bf16 q/k/v/o, fp32 S0 -> S_T"),
    "decode": ("decode_kernel<128, 128, unsigned short>", "decode.hip", "decode_b256_h32_d128.txt",
               "decode step, 256 sequences, 16 QK / 32 V heads, dk = dv = 128, bf16 q/k/v/o, "
               "fp32 state updated in place (512 MiB)"),
    "conv_silu": ("conv_silu_kernel", "block_ops.hip", "conv_silu_4x16384_c8192.txt",
                  "causal conv (width 4) + SiLU, 4 sequences x 16384 tokens, 8192 bf16 channels "
                  "(q | k | v of 16 QK / 32 V heads, d = 128), carried state in and out"),
    "gated_rmsnorm": ("gated_rmsnorm_kernel<128, unsigned short>", "block_ops.hip",
                      "gated_rmsnorm_4x16384_h32_d128.txt",
                      "gated RMS norm of 4 x 16384 tokens x 32 V heads (rows of 128 bf16), bf16 z"),
}

CMD_KT = ("rocprofv3 --kernel-trace --stats --output-format csv -d {kt} -o bench -- "
          "python3 bench.py --steps 5 --warmup 1 --no-cpu-baseline")
CMD_PMC = ("timeout -s KILL 180 rocprofv3 --pmc {ctr} --output-format csv -d {d} -o bench -- "
           "python3 bench.py --steps 2 --warmup 1 --settle-ms 0 --no-cpu-baseline --copy-probe")
CMD_MFMA = ("timeout -s KILL 180 rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 --output-format csv -d {d} -o bench -- "
            "python3 bench.py --steps 2 --warmup 1 --settle-ms 0 --no-cpu-baseline --no-block")
CMD_SUM = "python3 -m gated_deltanet_recurrence_rule_amd.profsummary {kt} {fetch} {write}{mfma}{sq} --out profiles"
CMD_SQ = ("timeout -s KILL 120 rocprofv3 --pmc {ctrs} --output-format csv -d {d} -o bench -- "
          "python3 bench.py --steps 2 --warmup 1 --settle-ms 0 --no-cpu-baseline --no-block")
# SQ counters that count in quad-cycles (4 clocks), per rocprofv3's counter descriptions
SQ_QUAD = {"SQ_WAVE_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_MISC",
           "SQ_INST_CYCLES_SALU", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY"}
SQ_FILE = "prefill_chunked_counters_4x16384.txt"


def sq_summary(dirs, frag: str, n_waves: int, n_chunks: int, sum_cmd: str) -> list:
    """Lines of the SQ-counter record of one kernel: for every counter of the given passes
    (one rocprofv3 --pmc run each), the mean over that kernel's dispatches, and per wave per
    chunk."""
    lines, table = [], []
    for d in dirs:
        with open(_one(d, "counter_collection.csv")) as f:
            rows = [r for r in csv.DictReader(f) if frag in r["Kernel_Name"]]
        names = list(dict.fromkeys(r["Counter_Name"] for r in rows))
        lines.append("  " + CMD_SQ.format(ctrs=" ".join(names), d=d))
        for n in names:
            v = [float(r["Counter_Value"]) for r in rows if r["Counter_Name"] == n]
            table.append((n, sum(v) / len(v), len(v)))
    out = [f"Kernel: {frag} ({n_waves} waves, {n_chunks} chunks of 64 tokens each).",
           "MI355X (gfx950), one GPU.  Per-dispatch SQ counters (summed over the shader engines by rocprofv3),",
           f"averaged over the kernel's dispatches in each pass and divided by {n_waves} waves x {n_chunks} chunks.",
           "Counters marked (q) count quad-cycles (4 clocks).",
           "Commands (run from the repository root on a machine with an MI355X; one pass per line):", *lines,
           f"  this summary: {sum_cmd}", "",
           f"{'counter':34s} {'per dispatch':>16s} {'per wave per chunk':>20s}  dispatches"]
    for n, mean, cnt in table:
        per = mean / (n_waves * n_chunks)
        clocks = f"   = {4 * per:.0f} clocks" if n in SQ_QUAD else ""
        out.append(f"{n + (' (q)' if n in SQ_QUAD else ''):34s} {mean:16.0f} {per:20.1f}  {cnt}{clocks}")
    return out


def _one(d: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return hits[0]


def kernel_stats(kt_dir: str) -> list:
    with open(_one(kt_dir, "kernel_stats.csv")) as f:
        return list(csv.DictReader(f))


def kernel_counter(d: str, name: str, frag: str) -> list:
    """Per-dispatch values of counter `name` for kernels whose name contains `frag`."""
    with open(_one(d, "counter_collection.csv")) as f:
        return [float(r["Counter_Value"]) for r in csv.DictReader(f)
                if r["Counter_Name"] == name and frag in r["Kernel_Name"]]


def counters(d: str, name: str):
    """(per-kernel list of values, copy-probe value) for counter `name`."""
    with open(_one(d, "counter_collection.csv")) as f:
        rows = [r for r in csv.DictReader(f) if r["Counter_Name"] == name]
    per = {}
    for key, (frag, *_rest) in KERNELS.items():
        per[key] = [float(r["Counter_Value"]) for r in rows if frag in r["Kernel_Name"]]
    copies = [float(r["Counter_Value"]) for r in rows
              if "copy" in r["Kernel_Name"].lower() or "elementwise" in r["Kernel_Name"].lower()]
    if not copies:
        raise ValueError(f"no copy-probe dispatch found for {name} in {d}")
    return per, max(copies)


def sha256(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("kt")
    ap.add_argument("fetch")
    ap.add_argument("write")
    ap.add_argument("--mfma", default=None, help="directory of the MfmaUtil / MfmaFlopsBF16 run")
    ap.add_argument("--sq", nargs="+", default=None,
                    help="directories of SQ counter passes of the prefill kernel (writes " + SQ_FILE + ")")
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    args = ap.parse_args(argv)

    sys.path.insert(0, ROOT)
    import bench  # the algorithmic byte counts

    stats = kernel_stats(args.kt)
    fetch, fetch_copy = counters(args.fetch, "FETCH_SIZE")
    write, write_copy = counters(args.write, "WRITE_SIZE")
    gib_kib = float(1 << 20)
    scale_f, scale_w = gib_kib / fetch_copy, gib_kib / write_copy
    alg = {
        "prefill_chunked": bench.prefill_alg(4, 16384, 16, 32, 128, 128, 2, True)[0],
        "decode": bench.decode_alg(256, 16, 32, 128, 128, 2)[0],
        "conv_silu": bench.conv_alg(4 * 16384, 4, 8192, 2),
        "gated_rmsnorm": bench.norm_alg(4 * 16384 * 32, 128, 2),
    }
    cmds = [CMD_KT.format(kt=args.kt), CMD_PMC.format(ctr="FETCH_SIZE", d=args.fetch),
            CMD_PMC.format(ctr="WRITE_SIZE", d=args.write),
            CMD_SUM.format(kt=args.kt, fetch=args.fetch, write=args.write,
                           mfma=f" --mfma {args.mfma}" if args.mfma else "",
                           sq=(" --sq " + " ".join(args.sq)) if args.sq else "")]
    mfma_lines = {}
    if args.mfma:
        frag = KERNELS["prefill_chunked"][0]
        util = kernel_counter(args.mfma, "MfmaUtil", frag)
        flops = kernel_counter(args.mfma, "MfmaFlopsBF16", frag)
        if util and flops:
            f_alg = bench.prefill_alg(4, 16384, 16, 32, 128, 128, 2, True)[1]
            fx = sum(flops) / len(flops)
            mfma_lines["prefill_chunked"] = [
                f"  MFMA use:      {CMD_MFMA.format(d=args.mfma)}",
                f"MFMA busy (MfmaUtil = MFMA-busy cycles / (GPU-active cycles x SIMDs)): "
                f"{sum(util) / len(util):.1f}% average over {len(util)} dispatches "
                f"(min {min(util):.1f}%, max {max(util):.1f}%)",
                f"bf16 MFMA flops executed per dispatch (MfmaFlopsBF16): {fx:.4e} = {fx / f_alg:.2f}x the "
                f"algorithmic {f_alg:.4e} (hi/lo operand splits, Grams recomputed per column slice)",
            ]
    traffic = {
        "note": "HBM bytes per dispatch from rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE (KiB), each "
                "scaled by 1 GiB / (the counter's reading for a plain 1 GiB device copy in the same run)",
        "copy_probe_kib": {"FETCH_SIZE": fetch_copy, "WRITE_SIZE": write_copy},
        "scale": {"FETCH_SIZE": scale_f, "WRITE_SIZE": scale_w},
        "kernels": {},
    }
    os.makedirs(args.out, exist_ok=True)
    for key, (frag, src, fname, workload) in KERNELS.items():
        st = [r for r in stats if frag in r["Name"]]
        if not st or not fetch[key] or not write[key]:
            print(f"skipping {key}: not found in every run", file=sys.stderr)
            continue
        st = st[0]
        f_kib = sum(fetch[key]) / len(fetch[key])
        w_kib = sum(write[key]) / len(write[key])
        nbytes = (f_kib * scale_f + w_kib * scale_w) * 1024.0
        digest = sha256(os.path.join(CSRC, src))
        traffic["kernels"][key] = {"source": src, "sha256": digest, "fetch_kib": f_kib, "write_kib": w_kib,
                                   "bytes": nbytes}
        others = [r for r in stats if frag not in r["Name"]]
        lines = [
            f"Workload: {workload}.",
            f"Algorithmic HBM bytes per call: {alg[key]:,} (every input read once, every output written once).",
            "MI355X (gfx950), one GPU.  Commands (run from the repository root on a machine with an MI355X):",
            f"  kernel times:  {cmds[0]}",
            f"  HBM fetch:     {cmds[1]}",
            f"  HBM write:     {cmds[2]}",
            f"  this summary:  {cmds[3]}",
            *mfma_lines.get(key, []),
            f"Counter calibration: a 1 GiB device copy (bench.py --copy-probe) read FETCH_SIZE = {fetch_copy:.0f} KiB "
            f"and WRITE_SIZE = {write_copy:.0f} KiB,",
            f"so FETCH_SIZE is scaled by {scale_f:.4f} and WRITE_SIZE by {scale_w:.4f}.",
            f"kernel: {st['Name'][:100]}",
            f"calls: {st['Calls']}   average: {float(st['AverageNs']) / 1e3:.1f} us   "
            f"min: {float(st['MinNs']) / 1e3:.1f} us   max: {float(st['MaxNs']) / 1e3:.1f} us",
            f"HBM per dispatch: FETCH_SIZE {f_kib:.0f} KiB x {scale_f:.4f} + WRITE_SIZE {w_kib:.0f} KiB x "
            f"{scale_w:.4f} = {nbytes / 1e9:.4f} GB ({nbytes / alg[key]:.2f}x the algorithmic bytes)",
            f"source sha256 at measurement: {digest}",
            "other kernels in the same run:",
        ]
        for r in others:
            lines.append(f"  {r['Name'][:80]}: {r['Calls']} calls, average {float(r['AverageNs']) / 1e3:.1f} us")
        with open(os.path.join(args.out, fname), "w") as f:
            f.write("\n".join(lines) + "\n")
        print("\n".join(lines))
    with open(os.path.join(args.out, "traffic.json"), "w") as f:
        json.dump(traffic, f, indent=1)
    if args.sq:
        # the 4 x 16384 workload: 256 workgroups of 8 waves, 256 chunks each
        sq = sq_summary(args.sq, KERNELS["prefill_chunked"][0], 256 * 8, 16384 // 64, cmds[3])
        sq = [f"Workload: {KERNELS['prefill_chunked'][3]}.", *sq]
        with open(os.path.join(args.out, SQ_FILE), "w") as f:
            f.write("\n".join(sq) + "\n")
        print("\n".join(sq))
    return 0


if __name__ == "__main__":
    sys.exit(main())
