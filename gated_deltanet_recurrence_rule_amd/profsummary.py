"""Summarise rocprofv3 runs of bench.py into the text records kept under profiles/.

Three runs feed it (each writes CSV files into its own directory):

  kernel times   rocprofv3 --kernel-trace --stats --output-format csv -d <KT> -o bench -- \
                     python3 bench.py --steps 5 --warmup 1 --no-cpu-baseline --no-varlen
  HBM reads      timeout -s KILL 180 rocprofv3 --pmc FETCH_SIZE --output-format csv -d <FETCH> -o bench -- \
                     python3 bench.py --steps 2 --warmup 1 --settle-ms 0 --no-cpu-baseline --no-varlen --copy-probe
  HBM writes     timeout -s KILL 180 rocprofv3 --pmc WRITE_SIZE --output-format csv -d <WRITE> -o bench -- \
                     python3 bench.py --steps 2 --warmup 1 --settle-ms 0 --no-cpu-baseline --no-varlen --copy-probe

and, for the MFMA evidence of the prefill kernel (optional),

  MFMA use       timeout -s KILL 180 rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 --output-format csv -d <MFMA> -o bench -- \
                     python3 bench.py --steps 2 --warmup 1 --settle-ms 0 --no-cpu-baseline --no-varlen --no-block

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
    # key: (kernel-name fragment, source file, summary file, workload text); GRID below
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
# Grid size (threads) of the prefill kernel's dispatch on its workload: 4 sequences x 32 V
# heads x 2 column slices, workgroups of 512 threads.  The same kernel can also run on the
# other configurations the benchmark times; the grid picks this workload's dispatches out of
# a trace.  The other kernels run on one workload only (None: every dispatch).
GRID = {"prefill_chunked": 4 * 32 * 2 * 512, "decode": None, "conv_silu": None, "gated_rmsnorm": None}


def _grid_ok(key: str, grid) -> bool:
    return GRID[key] is None or int(grid) == GRID[key]

CMD_KT = ("rocprofv3 --kernel-trace --stats --output-format csv -d {kt} -o bench -- "
          "python3 bench.py --steps 5 --warmup 1 --no-cpu-baseline --no-varlen")
CMD_PMC = ("timeout -s KILL 180 rocprofv3 --pmc {ctr} --output-format csv -d {d} -o bench -- "
           "python3 bench.py --steps 2 --warmup 1 --settle-ms 0 --no-cpu-baseline --no-varlen --copy-probe")
CMD_MFMA = ("timeout -s KILL 180 rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 --output-format csv -d {d} -o bench -- "
            "python3 bench.py --steps 2 --warmup 1 --settle-ms 0 --no-cpu-baseline --no-varlen --no-block")
CMD_SUM = "python3 -m gated_deltanet_recurrence_rule_amd.profsummary {kt} {fetch} {write}{mfma}{sq} --out profiles"
CMD_SQ = ("timeout -s KILL 120 rocprofv3 --pmc {ctrs} --output-format csv -d {d} -o bench -- "
          "python3 bench.py --steps 2 --warmup 1 --settle-ms 0 --no-cpu-baseline --no-varlen --no-block")
# SQ counters that count in quad-cycles (4 clocks), per rocprofv3's counter descriptions
SQ_QUAD = {"SQ_WAVE_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_MISC",
           "SQ_INST_CYCLES_SALU", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY"}
SQ_FILE = "prefill_chunked_counters_4x16384.txt"
VARLEN_FILE = "prefill_chunked_split_varlen_65seq.txt"
CMD_VARLEN = ("rocprofv3 --kernel-trace --stats --output-format csv -d {d} -o bench -- "
              "python3 bench.py --only varlen --steps 5 --warmup 1")


def sq_summary(dirs, frag: str, n_waves: int, n_chunks: int, sum_cmd: str) -> list:
    """Lines of the SQ-counter record of one kernel: for every counter of the given passes
    (one rocprofv3 --pmc run each), the mean over that kernel's dispatches, and per wave per
    chunk."""
    lines, table = [], []
    for d in dirs:
        with open(_one(d, "counter_collection.csv")) as f:
            rows = [r for r in csv.DictReader(f)
                    if frag in r["Kernel_Name"] and _grid_ok("prefill_chunked", r["Grid_Size"])]
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


def dispatches(kt_dir: str) -> list:
    """Every dispatch of the kernel trace: (start ns, end ns, kernel name, grid size), in start order."""
    with open(_one(kt_dir, "kernel_trace.csv")) as f:
        rows = [(int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"],
                 int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]))
                for r in csv.DictReader(f)]
    return sorted(rows)


def duration_stats(us: list) -> str:
    us = sorted(us)
    return (f"calls: {len(us)}   average: {sum(us) / len(us):.1f} us   median: {us[len(us) // 2]:.1f} us   "
            f"min: {us[0]:.1f} us   max: {us[-1]:.1f} us")


def short_name(name: str) -> str:
    base = name.split("(")[0] if not name.startswith("void") else name[5:].split("(")[0]
    return base.replace("gdn::(anonymous namespace)::", "")


def varlen_summary(kt_dir: str, only_cmd: str) -> list:
    """Kernel-trace record of the packed variable-length prefill (bench.py --only varlen).
    A call is either one chunked dispatch, or (split sequences) a chunked pass over the
    segment maps, their chain and a chunked pass over the segments; either may follow a
    longest-first ordering kernel when the lengths are not already sorted."""
    import bench
    from gated_deltanet_recurrence_rule_amd import workloads as W

    lens = W.varlen_lengths()
    disp = dispatches(kt_dir)
    calls, parts, grids = [], {}, set()
    i = 0
    while i < len(disp):
        b, e, name, grid = disp[i]
        first, j = disp[i], i
        if "rank_kernel" in name or "longest_first" in name:
            if i + 1 >= len(disp):
                break
            parts.setdefault("ordering", []).append((e - b) / 1e3)
            j = i + 1
        if "prefill_chunked_kernel" not in disp[j][2]:
            i = j + 1
            continue
        if j + 2 < len(disp) and "split_chain_kernel" in disp[j + 1][2]:
            maps, chain, seg = disp[j], disp[j + 1], disp[j + 2]
            parts.setdefault("chunked pass over the segment maps", []).append((maps[1] - maps[0]) / 1e3)
            parts.setdefault("segment chain", []).append((chain[1] - chain[0]) / 1e3)
            parts.setdefault("chunked pass over the segments", []).append((seg[1] - seg[0]) / 1e3)
            grids.add(("segment-map pass", maps[3] // 512))
            grids.add(("segment pass", seg[3] // 512))
            last, i = seg, j + 3
        else:
            last = disp[j]
            parts.setdefault("chunked prefill", []).append((last[1] - last[0]) / 1e3)
            grids.add(("chunked prefill", last[3] // 512))
            i = j + 1
        calls.append((last[1] - first[0]) / 1e3)
    if not calls:
        raise ValueError(f"no prefill call found in {kt_dir}")
    tot = sum(lens)
    ab = sum(bench.prefill_alg(1, int(L), 16, 32, 128, 128, 2, True)[0] for L in lens)
    span = sorted(calls)
    med = span[len(span) // 2]
    longest = max(lens)
    lines = [
        f"Workload: packed variable-length prefill, {len(lens)} sequences ({len(lens) - 1} of 128 .. 32768 "
        f"tokens, log-uniform, and one of {lens[-1]}), {tot} tokens, 16 QK / 32 V heads, dk = dv = 128, "
        "bf16 q/k/v/o, fp32 S0 -> S_T, 10% alpha = 1 and 10% beta = 1 tokens.",
        f"Algorithmic HBM bytes per call: {ab:,}.",
        "MI355X (gfx950), one GPU.  Commands (run from the repository root on a machine with an MI355X):",
        f"  kernel times:  {only_cmd}",
        f"  this summary:  python3 -m gated_deltanet_recurrence_rule_amd.profsummary --varlen {kt_dir} --out profiles",
        "grids (workgroups of 512 threads): " + ", ".join(f"{k} {v}" for k, v in sorted(grids)),
        f"whole call (first kernel start to last kernel end), {len(span)} calls (settle, warm-up and timed): "
        f"median {med:.1f} us, min {span[0]:.1f} us, max {span[-1]:.1f} us -> {tot / med:.1f} Mtok/s, "
        f"{ab / (med * 1e-6) / 1e9:.0f} GB/s algorithmic",
        f"the longest sequence is {longest} tokens = {(longest + 63) // 64} chunks: the median call takes "
        f"{med / ((longest + 63) // 64) * 1e3:.0f} ns per chunk of it",
    ]
    for name, us in parts.items():
        lines.append(f"{name}: {duration_stats(us)}")
    return lines


def kernel_counter(d: str, name: str, key: str) -> list:
    """Per-dispatch values of counter `name` for kernel `key` of KERNELS on its workload."""
    frag = KERNELS[key][0]
    with open(_one(d, "counter_collection.csv")) as f:
        return [float(r["Counter_Value"]) for r in csv.DictReader(f)
                if r["Counter_Name"] == name and frag in r["Kernel_Name"] and _grid_ok(key, r["Grid_Size"])]


def counters(d: str, name: str):
    """(per-kernel list of values, copy-probe value) for counter `name`."""
    with open(_one(d, "counter_collection.csv")) as f:
        rows = [r for r in csv.DictReader(f) if r["Counter_Name"] == name]
    per = {}
    for key, (frag, *_rest) in KERNELS.items():
        per[key] = [float(r["Counter_Value"]) for r in rows
                    if frag in r["Kernel_Name"] and _grid_ok(key, r["Grid_Size"])]
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
    ap.add_argument("kt", nargs="?")
    ap.add_argument("fetch", nargs="?")
    ap.add_argument("write", nargs="?")
    ap.add_argument("--varlen", default=None,
                    help="directory of a kernel trace of bench.py --only varlen (writes " + VARLEN_FILE + ")")
    ap.add_argument("--mfma", default=None, help="directory of the MfmaUtil / MfmaFlopsBF16 run")
    ap.add_argument("--sq", nargs="+", default=None,
                    help="directories of SQ counter passes of the prefill kernel (writes " + SQ_FILE + ")")
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    args = ap.parse_args(argv)

    sys.path.insert(0, ROOT)
    import bench  # the algorithmic byte counts

    if args.varlen:
        lines = varlen_summary(args.varlen, CMD_VARLEN.format(d=args.varlen))
        os.makedirs(args.out, exist_ok=True)
        with open(os.path.join(args.out, VARLEN_FILE), "w") as f:
            f.write("\n".join(lines) + "\n")
        print("\n".join(lines))
    if not args.kt:
        return 0
    if not (args.fetch and args.write):
        ap.error("the kernel-trace, fetch and write directories go together")

    stats = kernel_stats(args.kt)
    disp = dispatches(args.kt)
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
        util = kernel_counter(args.mfma, "MfmaUtil", "prefill_chunked")
        flops = kernel_counter(args.mfma, "MfmaFlopsBF16", "prefill_chunked")
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
        mine = [(e - b) / 1e3 for b, e, n, grid in disp if frag in n and _grid_ok(key, grid)]
        if not st or not mine or not fetch[key] or not write[key]:
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
            "dispatches on this workload" + (f" (grid of {GRID[key]} threads)" if GRID[key] else "")
            + ", settle, warm-up and timed calls:",
            f"  {duration_stats(mine)}",
            f"all dispatches of the kernel in the run: {st['Calls']}, average {float(st['AverageNs']) / 1e3:.1f} us",
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
