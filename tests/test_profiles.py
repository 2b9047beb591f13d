"""The committed rocprofv3 summaries agree with themselves and with what bench.py reads.

Runs on the CPU: it parses the text under profiles/, no profiler and no GPU.
"""
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROF = os.path.join(ROOT, "profiles")


def read(name):
    with open(os.path.join(PROF, name)) as f:
        return f.read()


def test_select_trace_mean_agrees_with_the_launch_events():
    # the kernel-trace mean of the benchmarked select launches and the bench's
    # own launch-recorded events, both quoted in the same summary
    text = read("kernels_qwen3_4b_batched.md")
    trace = float(re.search(r"Top-M select of the benchmarked workload[^:]*: \d+ calls, mean ([0-9.]+) us", text).group(1))
    events = float(re.search(r"HIP events that each launch records ([0-9.]+) us", text).group(1))
    assert abs(trace - events) / events < 0.05, (trace, events)


def test_select_traffic_line_is_consistent():
    text = read("topm_select_qwen3_4b_batched_pmc.md")
    shown = re.search(r"\): (\d+) bytes per launch against (\d+) algorithmic \(([0-9.]+)x\)", text)
    stored = re.search(r"topm_traffic_bytes=(\d+) source_sha256=[0-9a-f]{64}", text)
    assert shown and stored
    traffic, alg, ratio = int(shown.group(1)), int(shown.group(2)), float(shown.group(3))
    assert int(stored.group(1)) == traffic
    assert abs(traffic / alg - ratio) < 1e-3
    # B * L rows of V bf16 logits plus M (index, value) pairs written per row
    assert alg == 64 * 16 * (151936 * 2 + 64 * 8)
    # every logit is fetched once: no re-reads, no bytes missing
    assert 0.99 < ratio < 1.05


def test_every_summary_names_its_command():
    for name in os.listdir(PROF):
        text = read(name)
        assert "rocprofv3" in text and "bench.py" in text, name


def test_contraction_mfma_counters_match_the_kernel_structure():
    # SQ_INSTS_VALU_MFMA_MOPS_BF16 of the benchmarked contraction (64 unit
    # tiles x 4 K ranges, 8 waves: 4 on x chunks in one batch of 6 slots for
    # 5 chunks, 4 on h chunks, 2 each, the state as 3 bf16 parts), 4 row
    # blocks, 3 gates; one 16x16x32 MFMA is 16384 flops = 32 MOPs of 512
    text = read("gru_contraction_qwen3_4b_batched_mfma.md")
    m = re.search(r"gru_mfma_mops_bf16=(\d+) gru_mfma_busy_cycles=(\d+) source_sha256=[0-9a-f]{64}", text)
    assert m
    mops, busy = int(m.group(1)), int(m.group(2))
    tiles, ks, rb, gates = 64, 4, 4, 3
    x_mfma = tiles * ks * 4 * 6 * gates * rb
    h_mfma = tiles * ks * 4 * 2 * 3 * gates * rb
    assert mops == (x_mfma + h_mfma) * 32
    # 16 busy cycles per MFMA on each of the SIMDs that issue it
    assert busy == (x_mfma + h_mfma) * 16
    shown = re.search(r"(\d+) MOPs = ([0-9.]+) GFLOP issued per launch, against ([0-9.]+) GFLOP algorithmic", text)
    assert int(shown.group(1)) == mops
    assert abs(float(shown.group(2)) - 512 * mops / 1e9) < 1e-3
    assert abs(float(shown.group(3)) - 2 * 64 * 3 * 1024 * (2560 + 1024) / 1e9) < 1e-3


def test_fused_contraction_mfma_counters_match_the_kernel_structure():
    # SQ_INSTS_VALU_MFMA_MOPS_BF16 of the benchmarked fused launches (their
    # contraction workgroups): every (16-unit tile, 32-wide chunk) pair once,
    # 4 row blocks, 3 gates; the x part (E / 32 chunks) one MFMA per block and
    # gate, the h part (H / 32 chunks) three (the state's three bf16 parts)
    text = read("gru_contraction_qwen3_4b_batched_mfma.md")
    m = re.search(r"fused_mfma_mops_bf16=(\d+) fused_mfma_busy_cycles=(\d+) source_sha256=[0-9a-f]{64}", text)
    assert m
    mops, busy = int(m.group(1)), int(m.group(2))
    tiles, rb, gates = 1024 // 16, 4, 3
    x_mfma = tiles * (2560 // 32) * gates * rb
    h_mfma = tiles * (1024 // 32) * 3 * gates * rb
    assert mops == (x_mfma + h_mfma) * 32
    assert busy == (x_mfma + h_mfma) * 16
