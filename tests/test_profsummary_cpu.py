"""profsummary on the CPU: it reads rocprofv3's CSV output, so small synthetic traces in the
same format check what it selects and how it reconstructs calls.

* the prefill kernel's dispatches are picked by grid size, so dispatches of the same kernel on
  other workloads in the run do not mix into its statistics;
* a packed variable-length call is rebuilt from consecutive dispatches: an optional ordering
  kernel, then either one chunked dispatch or the map pass, the chain and the segment pass.
"""
import csv
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from gated_deltanet_recurrence_rule_amd import profsummary as ps  # noqa: E402

TRACE_COLS = ["Kind", "Agent_Id", "Queue_Id", "Stream_Id", "Thread_Id", "Dispatch_Id", "Kernel_Id",
              "Kernel_Name", "Correlation_Id", "Start_Timestamp", "End_Timestamp", "LDS_Block_Size",
              "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Workgroup_Size_X",
              "Workgroup_Size_Y", "Workgroup_Size_Z", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]

CHUNKED = "void gdn::(anonymous namespace)::prefill_chunked_kernel<true, false>(unsigned short const*)"
SPLIT = "void gdn::(anonymous namespace)::prefill_chunked_kernel<true, true>(unsigned short const*)"
CHAIN = "gdn::(anonymous namespace)::split_chain_kernel(float const*, float const*)"
RANK = "gdn::(anonymous namespace)::rank_kernel(int const*, int, int*)"


def _write_trace(d, rows):
    """rows: (name, start_ns, end_ns, grid threads)"""
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "bench_kernel_trace.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=TRACE_COLS)
        w.writeheader()
        for i, (name, b, e, grid) in enumerate(rows):
            r = {c: 0 for c in TRACE_COLS}
            r.update(Kind="KERNEL_DISPATCH", Dispatch_Id=i + 1, Kernel_Name=name, Start_Timestamp=b,
                     End_Timestamp=e, Workgroup_Size_X=512, Workgroup_Size_Y=1, Workgroup_Size_Z=1,
                     Grid_Size_X=grid, Grid_Size_Y=1, Grid_Size_Z=1)
            w.writerow(r)


def test_dispatches_are_sorted_and_sized(tmp_path):
    d = str(tmp_path / "kt")
    _write_trace(d, [(CHUNKED, 5000, 6000, 131072), (CHUNKED, 1000, 1800, 229376)])
    rows = ps.dispatches(d)
    assert [r[0] for r in rows] == [1000, 5000]
    assert [r[3] for r in rows] == [229376, 131072]


def test_the_prefill_workload_is_selected_by_grid():
    assert ps.GRID["prefill_chunked"] == 4 * 32 * 2 * 512
    assert ps._grid_ok("prefill_chunked", 131072)
    assert not ps._grid_ok("prefill_chunked", 229376)
    assert ps._grid_ok("decode", 12345)  # kernels that run on one workload only: every dispatch


def test_duration_stats_text():
    txt = ps.duration_stats([3.0, 1.0, 2.0])
    assert "calls: 3" in txt and "average: 2.0 us" in txt and "median: 2.0 us" in txt
    assert "min: 1.0 us" in txt and "max: 3.0 us" in txt


def test_varlen_calls_unsplit_with_ordering(tmp_path):
    d = str(tmp_path / "kt")
    rows, t = [], 0
    for _ in range(3):  # three calls: ordering kernel, then one chunked dispatch of 10 ms
        rows.append((RANK, t, t + 5_000, 512))
        rows.append((CHUNKED, t + 6_000, t + 10_006_000, 4160 * 512))
        t += 20_000_000
    _write_trace(d, rows)
    lines = ps.varlen_summary(d, "cmd")
    text = "\n".join(lines)
    assert "3 calls" in text
    assert "median 10006.0 us" in text      # first kernel start to last kernel end
    assert "chunked prefill: calls: 3" in text
    assert "ordering: calls: 3" in text
    assert "chunked prefill 4160" in text


def test_varlen_calls_split(tmp_path):
    d = str(tmp_path / "kt")
    rows, t = [], 0
    for _ in range(2):  # map pass, chain, segment pass
        rows.append((SPLIT, t, t + 100_000, 448 * 512))
        rows.append((CHAIN, t + 101_000, t + 128_000, 128 * 256))
        rows.append((SPLIT, t + 129_000, t + 190_000, 256 * 512))
        t += 1_000_000
    _write_trace(d, rows)
    text = "\n".join(ps.varlen_summary(d, "cmd"))
    assert "2 calls" in text
    assert "median 190.0 us" in text
    assert "chunked pass over the segment maps: calls: 2" in text
    assert "segment chain: calls: 2" in text
    assert "chunked pass over the segments: calls: 2" in text
