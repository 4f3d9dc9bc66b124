"""bench.py on the CPU: its one-GPU contract, and the algorithmic counts its rooflines divide by.

The byte counts are re-derived here from the tensors each call must touch (every input read
once, every output written once), and the flop count from the products the chunked method is
quoted at: KK^T, QK^T, U, W and P Delta at 2 C d each, W S, Q S and K^T Delta at 2 d^2 each, per
token and V head, at C = 64.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def _tensor_bytes(*shapes_and_sizes):
    total = 0
    for shape, size in shapes_and_sizes:
        n = 1
        for x in shape:
            n *= x
        total += n * size
    return total


def test_prefill_counts_of_the_measured_workload():
    N, T, HQK, HV, d = 4, 16384, 16, 32, 128
    want = _tensor_bytes(((N * T, HQK, d), 2), ((N * T, HQK, d), 2),      # q, k (bf16)
                         ((N * T, HV, d), 2), ((N * T, HV, d), 2),        # v in, o out
                         ((N * T, HV), 4), ((N * T, HV), 4),              # g, beta (fp32)
                         ((N, HV, d, d), 4), ((N, HV, d, d), 4))          # S0 in, S_T out
    nbytes, flops, flops_rec = bench.prefill_alg(N, T, HQK, HV, d, d, 2, True)
    assert nbytes == want == 1_644_167_168
    per_token_head = 5 * (2 * 64 * d) + 3 * (2 * d * d)
    assert flops == N * T * HV * per_token_head
    assert abs(flops - 3.7796e11) / 3.7796e11 < 1e-4
    assert flops_rec == N * T * HV * 7 * d * d
    # without a start table, S_T alone
    assert bench.prefill_alg(N, T, HQK, HV, d, d, 2, False)[0] == want - N * HV * d * d * 4


def test_decode_counts_of_the_measured_workload():
    N, HQK, HV, d = 256, 16, 32, 128
    want = _tensor_bytes(((N, HV, d, d), 4), ((N, HV, d, d), 4),          # table read and written
                         ((N, HQK, d), 2), ((N, HQK, d), 2),              # q, k
                         ((N, HV, d), 2), ((N, HV, d), 2),                # v, o
                         ((N, HV), 4), ((N, HV), 4))                      # g, beta
    nbytes, flops, state_bytes = bench.decode_alg(N, HQK, HV, d, d, 2)
    assert nbytes == want == 1_080_098_816
    assert state_bytes == 2 * N * HV * d * d * 4 == 1 << 30
    assert flops == N * HV * 7 * d * d


def test_block_part_counts():
    T, N, Ct = 4 * 16384, 4, 2 * 16 * 128 + 32 * 128
    # x read, q | k | v written, the 3-token state read and written, the width-4 fp32 weights
    assert bench.conv_alg(T, N, Ct, 2) == _tensor_bytes(((T, Ct), 2), ((T, Ct), 2), ((N, 3, Ct), 2),
                                                        ((N, 3, Ct), 2), ((Ct, 4), 4)) == 2_148_007_936
    rows = T * 32
    # the read and z in, the normed read out, the fp32 weight of length dv
    assert bench.norm_alg(rows, 128, 2) == _tensor_bytes(((rows, 128), 2), ((rows, 128), 2),
                                                         ((rows, 128), 2), ((128,), 4)) == 1_610_613_248


def test_prefill_roofline_names_the_binding_roof():
    """The chunked prefill's algorithmic intensity (~230 flop/B) is below the bf16 ridge (312), so its
    headline roof is HBM, with the MFMA fraction beside it; the token-serial kernel is bound by
    fp32 vector arithmetic."""
    nbytes, flops, flops_rec = bench.prefill_alg(4, 16384, 16, 32, 128, 128, 2, True)
    assert flops / nbytes < bench.PEAK_BF16_TFLOPS * 1e12 / (bench.PEAK_HBM_GBPS * 1e9)
    r = bench.prefill_roofline(nbytes, flops, flops_rec, 1.0, "prefill_chunked")
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert abs(r["frac"] - nbytes / 1e-3 / 8e12) < 1e-12
    assert abs(r["mfma_frac"] - flops / 1e-3 / 2.5e15) < 1e-12
    t = bench.prefill_roofline(nbytes, flops, flops_rec, 2.0, "prefill_recurrent")
    assert t["bound"] == "alu" and "mfma_frac" not in t
    assert abs(t["frac"] - flops_rec / 2e-3 / 157.3e12) < 1e-12
