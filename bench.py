"""Benchmark of the conditional draft-tree builder on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config qwen3_4b_batched]

A step is one dt_build call: top-M select over the full vocabulary, the whole
best-first conditional expansion (n pops and their GRU updates) and the tree +
mask emit, for B independent requests on synthetic Zipf-shaped inputs already
resident in HBM.  dt_build runs its default expansion (the fused launches where
they apply); a second handle forced to the stepped expansion (contraction and
node step as separate kernels) gives the per-kernel figures.  Prints ONE JSON
line:

  value       tree builds per second (B * K / wall time of the K timed steps)
  roofline    the top-M select kernel (the dominant HBM stream): algorithmic
              bytes per launch / its mean kernel duration from the HIP events
              that each launch records on the library's stream (begin and end
              of the kernel itself) during the timed steps, against 8 TB/s
  cpu_baseline the CPU oracle on the same requests, on the host's cores (one
              single-threaded oracle call per request on a thread pool), and
              on one core on a bounded sample; host core count and CPU model
  parity      the timed trees compared with the oracle's, request by request
Extra keys: per-round time percentiles from per-call HIP events (a second
pass over the same steps), per-stage times (a pass with per-kernel events),
the fused expansion launch's roofline (the GRU contraction's flops and the
weights + gathers bytes per launch over its mean duration, with its MFMA
counters), the stepped expansion's GRU contraction (MFMA rate against the bf16
dense peak) and gathers, and latency figures.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16
MFMA_FP32_PEAK_TFS = 157.3


def committed_traffic(name, files):
    """HBM bytes per launch of a kernel (`name_traffic_bytes=`) from the
    committed counter summary, or None when the kernel's sources have changed
    since the counters were taken."""
    import hashlib
    import re
    try:
        text = open(os.path.join(ROOT, "profiles", "hbm_traffic_qwen3_4b_batched_pmc.md")).read()
    except OSError:
        return None
    m = re.search(name + r"_traffic_bytes=(\d+) source_sha256=([0-9a-f]{64})", text)
    if not m:
        return None
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "conditional_draft_tree_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return int(m.group(1)) if h.hexdigest() == m.group(2) else None


def mfma_counters(prefix, files):
    """(MFMA MOPs, MFMA busy SIMD-cycles) per benchmarked launch of a
    contraction from the committed counter summary (line `prefix_mfma_...`),
    or None when the kernel's sources have changed since they were taken."""
    import hashlib
    import re
    try:
        text = open(os.path.join(ROOT, "profiles", "gru_contraction_qwen3_4b_batched_mfma.md")).read()
    except OSError:
        return None
    m = re.search(prefix + r"_mfma_mops_bf16=(\d+) " + prefix +
                  r"_mfma_busy_cycles=(\d+) source_sha256=([0-9a-f]{64})", text)
    if not m:
        return None
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "conditional_draft_tree_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return (int(m.group(1)), int(m.group(2))) if h.hexdigest() == m.group(3) else None


# the sources each kernel is built from (the counters' hash)
GRU_SOURCES = ("gru.hip", "gate_tile.h", "dt_device.h", "dt_launch.h")
FUSED_SOURCES = ("expand.hip", "gate_tile.h", "dt_device.h", "dt_launch.h")
TOPM_SOURCES = ("topm.hip", "dt_device.h")


def counter_figures(c, mean_ms):
    if c is None or not mean_ms == mean_ms:
        return None
    mops, busy = c
    issued = 512.0 * mops / (mean_ms * 1e-3) / 1e12
    return {"mfma_mops_bf16_per_launch": mops, "issued_tflops": round(issued, 1),
            "issued_frac_of_peak": round(issued / MFMA_BF16_PEAK_TFS, 4),
            "mfma_busy_frac": round(busy / (mean_ms * 1e-3 * 2.4e9 * 1024), 4),
            "source": "profiles/gru_contraction_qwen3_4b_batched_mfma.md"}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def usable_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def percentile(xs, q):
    """Nearest-rank percentile of a non-empty list."""
    ys = sorted(xs)
    k = max(0, min(len(ys) - 1, int(-(-q * len(ys) // 100)) - 1))
    return ys[k]


def compare_trees(out_np, refs, tol=1e-4):
    """Timed trees against the oracle's, request by request: a request whose
    decisions all clear the near-tie threshold must match in topology (tokens,
    parents, depths, mask, count) bit for bit and in scores within tol; a
    request with a near tie must match in count and in the sorted scores."""
    import numpy as np
    exact = flagged = mismatched = 0
    err = 0.0
    for b, r in enumerate(refs):
        cnt = r["count"]
        ok = int(out_np["count"][b]) == cnt
        if r["flags"] == 0:
            ok = ok and all(np.array_equal(out_np[k][b], r[k]) for k in ("tokens", "parents", "depths", "mask"))
            e = float(np.abs(out_np["scores"][b][:cnt + 1] - r["scores"][:cnt + 1]).max())
        else:
            flagged += 1
            e = float(np.abs(np.sort(out_np["scores"][b][1:cnt + 1]) - np.sort(r["scores"][1:cnt + 1])).max()) \
                if ok and cnt else 0.0
        ok = ok and e <= tol
        err = max(err, e)
        if not ok:
            mismatched += 1
        elif r["flags"] == 0:
            exact += 1
    return {"requests": len(refs), "bit_exact_topology": exact, "near_tie_requests": flagged,
            "mismatched": mismatched, "max_score_error": err, "score_tolerance": tol}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--config", default="qwen3_4b_batched")
    p.add_argument("--cpu-requests", type=int, default=64,
                   help="requests in the CPU oracle sample (0 = skip)")
    p.add_argument("--cpu-threads", type=int, default=0, help="0 = min(16, usable cores)")
    p.add_argument("--cpu-single", type=int, default=8,
                   help="requests of the one-core oracle timing (0 = skip)")
    p.add_argument("--stage-steps", type=int, default=10, help="steps of the per-kernel timing pass")
    p.add_argument("--copy-calib", action="store_true",
                   help="also launch a plain 1 GiB device copy (counter calibration)")
    return p.parse_args()


def expansion_roofline(st, mode, B, L, E, H, M, n, esz, config, np):
    """The persistent expansion (one launch per call, every step of both
    roles; more than 64 requests: one launch per slice of 64).  Algorithmic
    bytes per call: the GRU weights once per launch, 3H (E + H) elements, and
    per expansion the gathered correction rows and the embedding row,
    n B (M H + E) elements; flops: the gate contraction of the T - 2 steps
    that contract, 2 B 3H (E + H) each.  Over the call's mean expansion time,
    which the launches record with the device clock (the first workgroup's
    start to the last one's end; the library's stage 8)."""
    if mode != "persistent" or not st["fused_each"]:
        return None
    T = n + 2
    nsl = -(-B // 64)
    ms = float(np.mean(st["fused_each"]))
    nbytes = (nsl * 3 * H * (E + H) + n * B * (M * H + E)) * esz
    flop = (T - 2) * 2.0 * B * 3 * H * (E + H)
    gbs = nbytes / (ms * 1e-3) / 1e9
    tfs = flop / (ms * 1e-3) / 1e12
    return {"kernel": "pers_kernel (the persistent expansion: every step of the call)",
            "bound": "hbm",
            "limited_by": "latency: a chain of n + 2 dependent steps, each a contraction and a node step "
                          "handing over through flag words",
            "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": committed_traffic("pers", FUSED_SOURCES) if config == "qwen3_4b_batched" else None,
            "algorithmic_bytes_per_launch": nbytes,
            "flop_per_launch": flop, "achieved_tflops": round(tfs, 2),
            "mfma_frac": round(tfs / MFMA_BF16_PEAK_TFS, 5),
            "mean_launch_ms": round(ms, 5), "launches": len(st["fused_each"]),
            "slices": nsl, "step_us": round(ms * 1e3 / (nsl * T), 2),
            "counters": counter_figures(mfma_counters("pers", FUSED_SOURCES), ms)
            if config == "qwen3_4b_batched" else None}


def fused_summary(st, sst, mode, n, stepped_us, stepped_same, per_step, np):
    """The expansion's share of a round: the default path's launches, the
    per-step fused launches and the stepped path on the same inputs."""
    d = {"mode": mode,
         "stepped_us_per_round": round(stepped_us, 1),
         "stepped_trees_equal_to_timed": stepped_same,
         "stepped_kernels_us_per_round": round(float(np.mean(sst["gru_gemm_total"]) + np.mean(sst["node_total"])) * 1e3, 1)
         if sst["gru_gemm_total"] and sst["node_total"] else None}
    if mode != "stepped" and st["fused_each"]:
        each = [x * 1e3 for x in st["fused_each"]]
        d.update({"launches_per_round": len(each) // max(len(st["fused_total"]), 1),
                  "kernels_us_per_round": round(float(np.mean(st["fused_total"])) * 1e3, 1),
                  "launch_us": {"mean": round(float(np.mean(each)), 2),
                                "p10": round(percentile(each, 10), 2),
                                "median": round(percentile(each, 50), 2),
                                "p90": round(percentile(each, 90), 2)}})
    if per_step is not None:
        d["per_step_launches"] = per_step
    return d


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the requests are independent: G GPUs would each take B/G of them, with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import conditional_draft_tree_amd as dtree
    import synthetic as S

    cfg = S.CONFIGS[args.config]
    B, V, L, E, H, M, n = (cfg[k] for k in ("B", "V", "L", "E", "H", "M", "n"))
    esz = 2 if cfg["dtype"] == "bf16" else 4
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    t0 = time.time()
    inp = S.make_inputs(cfg, seed=0)
    t = S.to_torch(inp, dev)
    print(f"[bench] inputs {args.config} ready in {time.time() - t0:.1f}s", file=sys.stderr,
          flush=True)

    bld = dtree.Builder(B, L, V, E, H, M, n, cfg["T"], cfg["dtype"], 1e-5, device=dev)
    fused = bld.fused
    stream = torch.cuda.current_stream()

    def step(out=None, b=bld):
        return b.build(t["base"], t["emb"], t["w_ih"], t["w_hh"], t["b_ih"], t["b_hh"], t["C"],
                       t["h0"], out=out)

    out = step()
    for _ in range(args.warmup):
        step(out)
    torch.cuda.synchronize()

    # ---- timed steps: no timing events (an event recorded after a kernel
    # delays the next one's start by a few microseconds)
    torch.cuda.synchronize()
    start = time.perf_counter()
    for _ in range(args.steps):
        step(out)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - start

    # ---- the same steps again with level-1 events (around the top-M kernels
    # and at the end of each call): per-round durations on the stream and the
    # select kernel's own time
    dtree.dt_timing_enable(bld.handle, 1, args.steps)
    for _ in range(args.steps):
        step(out)
    torch.cuda.synchronize()
    sel_ms = dtree.dt_timing_read(bld.handle, 0)
    merge_ms = dtree.dt_timing_read(bld.handle, 1)
    call_ms = dtree.dt_timing_read(bld.handle, 4)
    dtree.dt_timing_enable(bld.handle, 0, 0)

    mode = {dtree.DT_EXPAND_PERSISTENT: "persistent", dtree.DT_EXPAND_RESIDENT: "persistent",
            dtree.DT_EXPAND_FUSED: "fused", dtree.DT_EXPAND_STEPPED: "stepped"}[bld.expand_mode]
    launch = {dtree.DT_EXPAND_PERSISTENT: "cooperative", dtree.DT_EXPAND_RESIDENT: "plain"}.get(bld.expand_mode)
    ms_per_step = elapsed * 1e3 / args.steps
    value = B * args.steps / elapsed
    round_us = [m * 1e3 for m in call_ms]

    # ---- top-M roofline: per (request, position) row, V logits read and M
    # (index, value) pairs written
    rows = B * L
    topm_bytes = rows * (V * esz + M * 8)
    sel_mean = float(np.mean(sel_ms))
    achieved_gbs = topm_bytes / (sel_mean * 1e-3) / 1e9

    # ---- per-kernel pass (separate, untimed): every kernel bracketed by events
    dtree.dt_timing_enable(bld.handle, 2, args.stage_steps)
    for _ in range(args.stage_steps):
        step(out)
    torch.cuda.synchronize()
    st = {name: dtree.dt_timing_read(bld.handle, i) for i, name in
          ((0, "topm_select"), (1, "topm_merge"), (2, "gru_gemm_total"), (3, "node_total"),
           (4, "call"), (5, "gru_gemm_each"), (7, "fused_total"), (8, "fused_each"))}
    dtree.dt_timing_enable(bld.handle, 0, 0)

    # ---- the stepped expansion on the same inputs (its own handle): round
    # time, and per-kernel events of its contraction and node-step kernels
    sbld = dtree.Builder(B, L, V, E, H, M, n, cfg["T"], cfg["dtype"], 1e-5, device=dev,
                         expand=dtree.DT_EXPAND_STEPPED) if fused else bld
    sout = step(b=sbld) if fused else out
    for _ in range(3):
        step(sout, b=sbld)
    torch.cuda.synchronize()
    s0 = time.perf_counter()
    for _ in range(args.stage_steps):
        step(sout, b=sbld)
    torch.cuda.synchronize()
    stepped_us = (time.perf_counter() - s0) * 1e6 / max(args.stage_steps, 1)
    dtree.dt_timing_enable(sbld.handle, 2, args.stage_steps)
    for _ in range(args.stage_steps):
        step(sout, b=sbld)
    torch.cuda.synchronize()
    sst = {name: dtree.dt_timing_read(sbld.handle, i) for i, name in
           ((2, "gru_gemm_total"), (3, "node_total"), (5, "gru_gemm_each"))}
    dtree.dt_timing_enable(sbld.handle, 0, 0)
    stepped_same = bool(torch.equal(sout["tokens"], out["tokens"]) and torch.equal(sout["parents"], out["parents"]))
    if fused:
        sbld.close()
    # ---- the same pipeline as one launch per step (its own handle), where
    # the default runs it persistent: round time, per-launch time, trees
    per_step = None
    if mode == "persistent" and B <= 64:  # (one launch per step holds at most 64 requests)
        pbld = dtree.Builder(B, L, V, E, H, M, n, cfg["T"], cfg["dtype"], 1e-5, device=dev,
                             expand=dtree.DT_EXPAND_FUSED)
        pout = step(b=pbld)
        for _ in range(3):
            step(pout, b=pbld)
        torch.cuda.synchronize()
        p0 = time.perf_counter()
        for _ in range(args.stage_steps):
            step(pout, b=pbld)
        torch.cuda.synchronize()
        p_us = (time.perf_counter() - p0) * 1e6 / max(args.stage_steps, 1)
        dtree.dt_timing_enable(pbld.handle, 2, args.stage_steps)
        for _ in range(args.stage_steps):
            step(pout, b=pbld)
        torch.cuda.synchronize()
        p_each = dtree.dt_timing_read(pbld.handle, 8)
        dtree.dt_timing_enable(pbld.handle, 0, 0)
        per_step = {"us_per_round": round(p_us, 1),
                    "launch_us_mean": round(float(np.mean(p_each)) * 1e3, 2) if p_each else None,
                    "trees_equal_bit_for_bit": all(bool(torch.equal(pout[k], out[k])) for k in out)}
        pbld.close()
    # ---- the same persistent kernel as a cooperative launch (its own handle),
    # where the default launches it plainly: round time, trees
    coop_leg = None
    if launch == "plain":
        cbld = dtree.Builder(B, L, V, E, H, M, n, cfg["T"], cfg["dtype"], 1e-5, device=dev,
                             expand=dtree.DT_EXPAND_PERSISTENT)
        cout = step(b=cbld)
        for _ in range(3):
            step(cout, b=cbld)
        torch.cuda.synchronize()
        c0 = time.perf_counter()
        for _ in range(args.stage_steps):
            step(cout, b=cbld)
        torch.cuda.synchronize()
        coop_leg = {"us_per_round": round((time.perf_counter() - c0) * 1e6 / max(args.stage_steps, 1), 1),
                    "trees_equal_bit_for_bit": all(bool(torch.equal(cout[k], out[k])) for k in out)}
        cbld.close()
    gemm_each = float(np.mean(sst["gru_gemm_each"])) if sst["gru_gemm_each"] else float("nan")
    gemm_flop = 2.0 * B * 3 * H * (E + H)
    gemm_weight_bytes = 3 * H * (E + H) * esz
    peak_mfma = MFMA_BF16_PEAK_TFS if esz == 2 else MFMA_FP32_PEAK_TFS
    gemm_tfs = gemm_flop / (gemm_each * 1e-3) / 1e12

    # ---- the factorized (marginal) scoring mode on the same logits (extra key)
    mout = bld.build_marginal(t["base"])
    for _ in range(3):
        bld.build_marginal(t["base"], out=mout)
    torch.cuda.synchronize()
    m0 = time.perf_counter()
    for _ in range(args.stage_steps):
        bld.build_marginal(t["base"], out=mout)
    torch.cuda.synchronize()
    marg_us = (time.perf_counter() - m0) * 1e6 / max(args.stage_steps, 1)

    # ---- the full-vocabulary normalization mode (extra key): same inputs; the
    # top-M select also sums the tail mass; how many trees keep their shape
    fbld = dtree.Builder(B, L, V, E, H, M, n, cfg["T"], cfg["dtype"], 1e-5, device=dev, full_vocab=True)
    fout = fbld.build(t["base"], t["emb"], t["w_ih"], t["w_hh"], t["b_ih"], t["b_hh"], t["C"], t["h0"])
    for _ in range(3):
        fbld.build(t["base"], t["emb"], t["w_ih"], t["w_hh"], t["b_ih"], t["b_hh"], t["C"], t["h0"], out=fout)
    torch.cuda.synchronize()
    dtree.dt_timing_enable(fbld.handle, 1, args.stage_steps)
    f0 = time.perf_counter()
    for _ in range(args.stage_steps):
        fbld.build(t["base"], t["emb"], t["w_ih"], t["w_hh"], t["b_ih"], t["b_hh"], t["C"], t["h0"], out=fout)
    torch.cuda.synchronize()
    fv_us = (time.perf_counter() - f0) * 1e6 / max(args.stage_steps, 1)
    fv_sel = float(np.mean(dtree.dt_timing_read(fbld.handle, 0))) if args.stage_steps else float("nan")
    dtree.dt_timing_enable(fbld.handle, 0, 0)
    same_shape = float(((fout["tokens"] == out["tokens"]).all(dim=1) &
                        (fout["parents"] == out["parents"]).all(dim=1)).float().mean())
    fbld.close()

    # ---- the 256-wide correction head (extra key): the same logits and
    # embeddings, a 256-wide GRU state and C = W_2 [V, 256]
    c256 = S.with_config("qwen3_4b_head256") if args.config == "qwen3_4b_batched" else None
    h256 = None
    if c256 is not None:
        t256 = S.to_torch(S.make_inputs(c256, seed=0, skip=("base", "emb")), dev)
        hb = dtree.Builder(B, L, V, E, c256["H"], M, n, c256["T"], c256["dtype"], 1e-5, device=dev)
        hstep = lambda o=None: hb.build(t["base"], t["emb"], t256["w_ih"], t256["w_hh"], t256["b_ih"],
                                        t256["b_hh"], t256["C"], t256["h0"], out=o)
        hout = hstep()
        for _ in range(3):
            hstep(hout)
        torch.cuda.synchronize()
        h0t = time.perf_counter()
        for _ in range(args.stage_steps):
            hstep(hout)
        torch.cuda.synchronize()
        h_us = (time.perf_counter() - h0t) * 1e6 / max(args.stage_steps, 1)
        dtree.dt_timing_enable(hb.handle, 2, 3)
        for _ in range(3):
            hstep(hout)
        torch.cuda.synchronize()
        h256 = {"workload": "qwen3_4b_head256: H=256, C [V, 256], otherwise as the main workload",
                "us_per_round": round(h_us, 1), "tree_builds_per_s": round(B / (h_us * 1e-6), 1),
                "expansion": {dtree.DT_EXPAND_PERSISTENT: "persistent", dtree.DT_EXPAND_RESIDENT: "persistent",
                              dtree.DT_EXPAND_FUSED: "fused", dtree.DT_EXPAND_STEPPED: "stepped"}[hb.expand_mode]}
        if hb.fused:
            h256["expansion_launch_us"] = round(float(np.mean(dtree.dt_timing_read(hb.handle, 8))) * 1e3, 2)
        else:
            h256["gru_gemm_each_us"] = round(float(np.mean(dtree.dt_timing_read(hb.handle, 5))) * 1e3, 2)
            h256["node_step_each_us"] = round(float(np.mean(dtree.dt_timing_read(hb.handle, 3))) * 1e3 / n, 2)
        hb.close()
        del t256

    # ---- the folded input projection (extra key): the [V, 3H] table of
    # b_ih + W_ih . Emb[v] is computed once, then each step contracts W_hh . h only
    folded = None
    if esz == 2:
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        table = bld.fold_input(t["emb"], t["w_ih"], t["b_ih"])
        e1.record()
        torch.cuda.synchronize()
        fold_ms = e0.elapsed_time(e1)
        fstep = lambda o=None: bld.build_folded(t["base"], table, t["w_hh"], t["b_hh"], t["C"], t["h0"], out=o)
        fo = fstep()
        for _ in range(3):
            fstep(fo)
        torch.cuda.synchronize()
        f0 = time.perf_counter()
        for _ in range(args.stage_steps):
            fstep(fo)
        torch.cuda.synchronize()
        fo_us = (time.perf_counter() - f0) * 1e6 / max(args.stage_steps, 1)
        dtree.dt_timing_enable(bld.handle, 2, 3)
        for _ in range(3):
            fstep(fo)
        torch.cuda.synchronize()
        folded = {"us_per_round": round(fo_us, 1), "tree_builds_per_s": round(B / (fo_us * 1e-6), 1),
                  "fold_once_ms": round(fold_ms, 2), "table_bytes": V * 3 * H * 4,
                  "gru_gemm_each_us": round(float(np.mean(dtree.dt_timing_read(bld.handle, 5))) * 1e3, 2),
                  "node_step_each_us": round(float(np.mean(dtree.dt_timing_read(bld.handle, 3))) * 1e3 / n, 2),
                  "trees_equal_to_contracted": round(float(((fo["tokens"] == out["tokens"]).all(dim=1) &
                                                            (fo["parents"] == out["parents"]).all(dim=1))
                                                           .float().mean()), 4)}
        dtree.dt_timing_enable(bld.handle, 0, 0)
        del table

    # ---- the greedy acceptance walk on the timed trees (extra key): synthetic
    # greedy target tokens that follow one of a node's children with
    # probability 0.8
    tree_cpu = {k: out[k].cpu().numpy() for k in ("tokens", "parents", "count")}
    tgt = torch.from_numpy(S.make_greedy_targets(tree_cpu["tokens"], tree_cpu["parents"],
                                                 tree_cpu["count"], V, 0.8, seed=0)).to(dev)
    acc = bld.accept_greedy(out, tgt)
    torch.cuda.synchronize()
    dtree.dt_timing_enable(bld.handle, 1, args.stage_steps)
    for _ in range(args.stage_steps):
        bld.accept_greedy(out, tgt, out=acc)
    torch.cuda.synchronize()
    acc_us = float(np.mean(dtree.dt_timing_read(bld.handle, 6))) * 1e3 if args.stage_steps else float("nan")
    dtree.dt_timing_enable(bld.handle, 0, 0)
    tau = float((acc["accepted"].float() + 1).mean())

    if args.copy_calib:  # a plain copy of known size, for counter scaling
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    # ---- one request alone (extra key): request 0 of the same inputs built by
    # a B = 1 handle; the pages quote their per-round build time for one request
    # at n = 16, M = 64 (other hardware: context, not a target)
    single = None
    if args.config == "qwen3_4b_batched":
        sb = dtree.Builder(1, L, V, E, H, M, n, cfg["T"], cfg["dtype"], 1e-5, device=dev)
        s_base = t["base"][0:1].contiguous()
        s_h0 = t["h0"][0:1].contiguous() if t["h0"] is not None else None
        sstep = lambda o=None: sb.build(s_base, t["emb"], t["w_ih"], t["w_hh"], t["b_ih"], t["b_hh"], t["C"],
                                        s_h0, out=o)
        sout = sstep()
        for _ in range(3):
            sstep(sout)
        torch.cuda.synchronize()
        s0 = time.perf_counter()
        for _ in range(max(args.stage_steps, 1)):
            sstep(sout)
        torch.cuda.synchronize()
        s_us = (time.perf_counter() - s0) * 1e6 / max(args.stage_steps, 1)
        same = bool((sout["tokens"][0] == out["tokens"][0]).all() and (sout["parents"][0] == out["parents"][0]).all())
        sb.close()
        single = {"workload": "qwen3_4b_single: request 0 of the inputs above, B = 1",
                  "us_per_round": round(s_us, 1), "tree_equal_to_batched_request": same,
                  "pages_per_round_ms_other_hardware": {"python_builder": 3.67, "cuda_graph_builder": 2.31}}

    # ---- achievable HBM bandwidth on this machine: a plain device-to-device copy
    # (bytes read + bytes written per second), the select's second reference
    ca = torch.empty(1 << 29, dtype=torch.uint8, device=dev)
    cb = torch.empty_like(ca)
    for _ in range(3):
        cb.copy_(ca)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(10):
        cb.copy_(ca)
    c1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * ca.numel() * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del ca, cb

    cnt = out["count"].cpu().numpy()

    # ---- the gathers of the node step: per launch, M rows of C and one
    # embedding row per request; per round also the lower bound that reads
    # each (request, depth) slice of C once (slots 0 .. min(count, n-1) are
    # expanded, slot k from the slice of position depth(k))
    node_each = float(np.mean(sst["node_total"])) / n if sst["node_total"] else float("nan")
    gather_bytes = B * (M * H + E) * esz
    dep = out["depths"].cpu().numpy()
    uniq = sum(len(set(dep[b, :min(int(cnt[b]), n - 1) + 1].tolist())) for b in range(B))
    gather_gbs = gather_bytes / (node_each * 1e-3) / 1e9

    res = {
        "metric": "tree builds/sec and us/round at B, n=16, M=64; % HBM peak (topM) and % MFMA (GRU)",
        "value": round(value, 1),
        "unit": "tree builds/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "us_per_round": round(ms_per_step * 1e3, 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if esz == 2 else "f32",
        "data": "synthetic (seeded Zipf-shaped logits, random-init GRU/embedding/correction)",
        "config": {"workload": f"{args.config}: B={B} requests, V={V}, L={L}, E={E}, H={H}, "
                               f"M={M}, n={n}, T={cfg['T']}, Zipf alpha={cfg['alpha']}",
                   "B": B, "V": V, "L": L, "E": E, "H": H, "M": M, "n": n},
        "roofline_topm": {
            "kernel": "topm_partial_kernel (top-M select)",
            "bound": "hbm",
            "achieved": round(achieved_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
            "traffic": committed_traffic("topm", TOPM_SOURCES) if args.config == "qwen3_4b_batched" else None,
            "algorithmic_bytes_per_launch": topm_bytes,
            "mean_launch_ms": round(sel_mean, 5),
            "launches": len(sel_ms),
            "achievable_copy_gbs": round(copy_gbs, 1),
            "frac_of_copy": round(achieved_gbs / copy_gbs, 4),
        },
        "roofline_gather": {
            "kernel": "node_step_kernel (the gathers of one expansion step; stepped expansion)",
            "bound": "hbm",
            "limited_by": "latency: a dependent round trip for the candidate tokens, then 64 random "
                          "2 KiB rows per request",
            "achieved": round(gather_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gather_gbs / HBM_PEAK_GBS, 4),
            "algorithmic_bytes_per_launch": gather_bytes,
            "mean_launch_ms": round(node_each, 5),
            "round_bytes": gather_bytes * n,
            "round_bytes_unique_slices": uniq * M * H * esz + B * (n - 1) * E * esz,
        },
        "roofline_gru": {
            "kernel": "gru_gates_bf16_kernel (one expansion step; stepped expansion)",
            "bound": "hbm" if gemm_flop / gemm_weight_bytes < 312 else "mfma",
            "achieved_tflops": round(gemm_tfs, 2),
            "mfma_peak_tflops": peak_mfma,
            "mfma_frac": round(gemm_tfs / peak_mfma, 5),
            "weight_gbs": round(gemm_weight_bytes / (gemm_each * 1e-3) / 1e9, 1),
            "hbm_frac_weights": round(gemm_weight_bytes / (gemm_each * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "flop_per_launch": gemm_flop,
            "mean_launch_ms": round(gemm_each, 5),
            # from the committed rocprofv3 counters of the same launch shape:
            # MFMA ops actually issued (512 flops per MOP) and MFMA busy cycles
            # over the launch (1024 SIMDs at 2.4 GHz), at this run's mean time
            "counters": counter_figures(mfma_counters("gru", GRU_SOURCES), gemm_each)
            if args.config == "qwen3_4b_batched" else None,
        },
        "stages_ms_mean": {k: round(float(np.mean(v)), 5) for k, v in st.items() if v},
        "expansion": dict(fused_summary(st, sst, mode, n, stepped_us, stepped_same, per_step, np),
                          launch=launch, cooperative_launch=coop_leg),
        # (null: each row is one segment, so no merge kernel runs)
        "topm_merge_ms_mean": round(float(np.mean(merge_ms)), 5) if merge_ms else None,
        "call_ms_events_mean": round(float(np.mean(call_ms)), 5),
        # per-round durations from the events each call of the second pass
        # records on the library's stream (first kernel's begin to the call's end)
        "us_per_round_events": {"p10": round(percentile(round_us, 10), 1),
                                "median": round(percentile(round_us, 50), 1),
                                "p90": round(percentile(round_us, 90), 1),
                                "rounds": len(round_us)},
        "tree_builds_per_s_at_median_round": round(B / (percentile(round_us, 50) * 1e-6), 1),
        "latency_per_request_us": round(ms_per_step * 1e3, 1),
        "marginal_mode": {"us_per_round": round(marg_us, 1),
                          "tree_builds_per_s": round(B / (marg_us * 1e-6), 1)},
        "full_vocab_mode": {"us_per_round": round(fv_us, 1),
                            "tree_builds_per_s": round(B / (fv_us * 1e-6), 1),
                            "topm_select_with_tail_us": round(fv_sel * 1e3, 2),
                            "topm_select_with_tail_gbs": round(topm_bytes / (fv_sel * 1e-3) / 1e9, 1),
                            "trees_same_shape_as_top_m_softmax": round(same_shape, 4)},
        "head256_mode": h256,
        "folded_input_mode": folded,
        "single_request": single,
        "acceptance_walk": {"kernel_us": round(acc_us, 2), "requests": B,
                            "mean_tokens_per_round_synthetic_targets": round(tau, 3),
                            "target_follow_probability": 0.8},
    }

    # ---- the headline roofline: the kernel with the larger share of a round
    # (the persistent expansion launch, or the top-M select)
    exp_roof = expansion_roofline(st, mode, B, L, E, H, M, n, esz, args.config, np)
    if exp_roof is not None and exp_roof["mean_launch_ms"] > sel_mean:
        res["roofline"] = exp_roof
    else:
        res["roofline"] = res["roofline_topm"]
        if exp_roof is not None:
            res["roofline_expansion"] = exp_roof
    res = {k: res[k] for k in ["metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "us_per_round",
                               "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config", "roofline"]
           } | {k: v for k, v in res.items() if k != "roofline"}

    # ---- CPU baseline: the oracle as it stands, one request per thread on
    # the host's cores, and one request after another on one core; the
    # all-cores trees are also the reference the timed trees are checked
    # against (every one of those requests, bit for bit where no decision is
    # a near tie)
    if args.cpu_requests > 0:
        import oracle
        nproc = usable_cores()
        threads = args.cpu_threads or min(16, nproc)
        nreq = min(args.cpu_requests, B)
        sub = dict(inp)
        sub["base"] = inp["base"][:nreq]
        sub["h0"] = inp["h0"][:nreq]
        c0 = time.perf_counter()
        refs = oracle.build_batch(sub, M, n, cfg["T"], threads=threads)
        cpu_s = time.perf_counter() - c0
        single = None
        if args.cpu_single > 0:
            ns = min(args.cpu_single, nreq)
            s0 = time.perf_counter()
            oracle.build_batch(sub, M, n, cfg["T"], requests=range(ns), threads=1)
            single_s = time.perf_counter() - s0
            single = {"value": round(ns / single_s, 3), "unit": "tree builds/s", "cores": 1,
                      "sample": f"requests 0..{ns - 1}, one after another on one thread, {single_s:.1f} s wall"}
        res["cpu_baseline"] = {
            "value": round(nreq / cpu_s, 3),
            "unit": "tree builds/s",
            "cores": threads,
            "kind": "oracle",
            "sample": f"{nreq} requests of {args.config} (one single-threaded fp64 oracle call "
                      f"per request, {threads} threads), {cpu_s:.1f} s wall",
            "host_cores": nproc,
            "cpu_model": cpu_model(),
            "one_core": single,
        }
        out_np = {k: v.cpu().numpy() for k, v in out.items()}
        res["parity"] = compare_trees({k: v[:nreq] for k, v in out_np.items()}, refs)
        if res["parity"]["mismatched"]:
            print(json.dumps(res), flush=True)
            raise SystemExit(f"timed trees differ from the oracle's: {res['parity']}")
    print(json.dumps(res), flush=True)
    bld.close()


if __name__ == "__main__":
    main()
