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
