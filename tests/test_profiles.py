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
    events = float(re.search(r"top-M select mean kernel time from the HIP events that each launch records ([0-9.]+) us",
                             text).group(1))
    assert abs(trace - events) / events < 0.05, (trace, events)


def test_persistent_trace_mean_agrees_with_the_launch_clock():
    # the kernel-trace mean of the persistent expansion launches and the
    # bench's own figure (the device-clock span each launch records)
    text = read("kernels_qwen3_4b_batched.md")
    trace = float(re.search(r"Persistent expansion of the benchmarked workload \(.*?\): \d+ launches, mean ([0-9.]+) us",
                            text).group(1))
    clock = float(re.search(r"persistent expansion mean kernel time from the device clock that each launch records "
                            r"([0-9.]+) us", text).group(1))
    assert abs(trace - clock) / clock < 0.05, (trace, clock)


def test_persistent_traffic_line_is_consistent():
    text = read("hbm_traffic_qwen3_4b_batched_pmc.md")
    shown = re.search(r"(\d+) bytes fetched and (\d+) written per launch, (\d+) in all, against (\d+) algorithmic "
                      r"\(([0-9.]+)x\)", text)
    stored = re.search(r"pers_traffic_bytes=(\d+) source_sha256=[0-9a-f]{64}", text)
    assert shown and stored
    fetched, written, total, alg = (int(shown.group(i)) for i in range(1, 5))
    ratio = float(shown.group(5))
    assert abs(fetched + written - total) <= 1 and int(stored.group(1)) == total
    assert abs(total / alg - ratio) < 1e-3
    # the weights once and, per expansion, the gathered correction rows and the embedding row
    B, L, E, H, M, n = 64, 16, 2560, 1024, 64, 16
    assert alg == (3 * H * (E + H) + n * B * (M * H + E)) * 2
    # the algorithmic bytes are all there; the rest is bounded (activations, sums, states)
    assert 1.0 < ratio < 3.0


def test_select_traffic_line_is_consistent():
    text = read("hbm_traffic_qwen3_4b_batched_pmc.md")
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


def test_persistent_contraction_mfma_counters_match_the_kernel_structure():
    # SQ_INSTS_VALU_MFMA_MOPS_BF16 of the benchmarked persistent launches
    # (their contraction workgroups): per contracting step every (16-unit
    # tile, 32-wide chunk) pair once, 4 row blocks, 3 gates; the x part
    # (E / 32 chunks) one MFMA per block and gate, the h part (H / 32 chunks)
    # three (the state's three bf16 parts).  Steps 1 .. n always contract,
    # step n + 1 only when some request waits in it.
    text = read("gru_contraction_qwen3_4b_batched_mfma.md")
    m = re.search(r"pers_mfma_mops_bf16=(\d+) pers_mfma_busy_cycles=(\d+) source_sha256=[0-9a-f]{64}", text)
    assert m
    mops, busy = int(m.group(1)), int(m.group(2))
    tiles, rb, gates, n = 1024 // 16, 4, 3, 16
    step = tiles * (2560 // 32) * gates * rb + tiles * (1024 // 32) * 3 * gates * rb
    assert mops % (step * 32) == 0 and mops // (step * 32) in (n, n + 1)
    assert busy * 2 == mops  # 16 busy cycles per 32-MOP MFMA
