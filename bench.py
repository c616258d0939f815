#!/usr/bin/env python
"""Benchmark of the chunked gated delta-rule forward on one MI355X.

One step is one complete forward pass (chunk table, gate prefix sums, A-build
+ solve, w/u products, state pass, output) over one batch of the long-context
GQA workload: T = 65536 tokens, 16 q/k heads, 32 value heads, dk = dv = 128,
bf16 q/k/v/beta, fp32 gates (g = logsigmoid(N(6, 1))) and state, S0 = 0,
seeded synthetic data. Inputs are resident in HBM before the timed region.

Prints one JSON line with the throughput (tokens/s), the roofline of the
dominant kernel (its average duration measured with the two HIP events that
each timed step records around it on the launch stream), the per-stage times
(from steps outside the timed region), and the CPU oracle timed on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from chunkwise_gated_delta_local_amd import api, synth  # noqa: E402

METRIC = "fwd tokens/s at Hv=32,dk=dv=128,T=64k bf16; % of MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0                   # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0          # MI355X dense bf16 / fp16 matrix cores, published
FP32_MFMA_PEAK_TFLOPS = 157.3
KERNEL_SOURCES = ("chunkwise_gated_delta_local_amd/csrc/gdr_kernels.hip",
                  "chunkwise_gated_delta_local_amd/csrc/gdr_fp16.hip",
                  "chunkwise_gated_delta_local_amd/csrc/gdr_recurrent.hip",
                  "chunkwise_gated_delta_local_amd/csrc/gdr_device.hpp")
STAGE_KERNELS = ("k_chunk_table", "k_gate_cumsum", "k_build_solve", "k_wu", "k_state", "k_output")
FP16_STAGE_KERNELS = ("k_chunk_table", "(none)", "k_prep", "(none)", "k_chunk16", "(none)")
FRAG16_BYTES = (4 * 512 + 2 * 256) * 2  # fp16 pair fragments per (chunk, value head), two of six halved: T or the score block
DECAY_ROW_BYTES = 2 * 64 * 4            # exp(G), exp(G_last - G) per (chunk, value head)


def method_bytes_per_token(w: synth.Workload, out_bytes: int) -> int:
    """Bytes the method itself must move per token (all heads): q, k, v, g and
    beta read once, o written once, in their stored types. The initial and
    final states are counted apart (per sequence, not per token)."""
    es = 2 if w.dtype == "bf16" else 4
    g_bytes = w.Nv * 4 if w.gated else 0
    return 2 * w.Nk * w.dk * es + w.Nv * w.dv * es + g_bytes + w.Nv * es + w.Nv * w.dv * out_bytes


def method_flops_per_token(w: synth.Workload, C: int = 64) -> float:
    """Floating-point operations of the chunk algorithm per token (all value
    heads, 2 per multiply-add, full chunks): 6 dk dv for the state products
    (W S, K^T V_new, Q S), 2C(3dk + 2dv) for the intra-chunk products (K K^T,
    Q K^T, W, and U, the score block times V_new) and (2/3) C^2 for the
    triangular solve."""
    return w.Nv * (6.0 * w.dk * w.dv + 2.0 * C * (3 * w.dk + 2 * w.dv) + (2.0 / 3.0) * C * C)


def stage_io_bytes(w: synth.Workload, Ttot: int, N: int, NT: int, out_bytes: int, s0: bool) -> dict:
    """Bytes each kernel moves by its own inputs and outputs (every tensor it
    reads read once, every tensor it writes written once, in its stored type),
    the pipeline's intermediates included (T and the score block as fp16
    fragments, the decay rows). Reported beside the method's bytes."""
    es = 2 if w.dtype == "bf16" else 4
    Nv, Nk, dk, dv = w.Nv, w.Nk, w.dk, w.dv
    tv = Ttot * Nv                      # token-heads (value heads)
    tk = Ttot * Nk                      # token-heads (q/k heads)
    beta_b = es
    state = N * Nv * dk * dv * 4
    if w.dtype == "bf16":               # fp16 path
        frag = NT * Nv * FRAG16_BYTES
        rows = NT * Nv * DECAY_ROW_BYTES
        return {
            "k_chunk_table": 4 * (N + 1) + 16 * NT,
            "k_prep": 2 * tk * dk * es + tv * (beta_b + 4) + 2 * frag + rows         # k, q, beta, g in; T, P, R out
                      + 2 * NT * Nk * 64 * dk * 2,                                      # fp16 K and Q tiles out
            "k_chunk16": 2 * NT * Nk * 64 * dk * 2 + tv * dv * es + rows + 2 * frag    # K16, Q16, v, R, T, P in
                         + tv * dv * out_bytes + state * (2 if s0 else 1),             # o, S_T out (S0 in)
            "(none)": 0,
        }
    return {
        "k_chunk_table": 4 * (N + 1) + 16 * NT,
        "k_gate_cumsum": tv * (4 + 4),                                        # g in, G out
        "k_build_solve": tk * dk * es + tv * (beta_b + 4) + tv * 64 * 4,       # k, beta, G in; A out
        "k_wu": tk * dk * es + tv * dv * es + tv * (beta_b + 4) + tv * 64 * 4  # k, v, beta, G, A in
                + tv * (dk + dv) * 4 + NT * Nk * 64 * dk * es,                # W, U, K^T out
        "k_state": tv * (dk + dv) * 4 + NT * Nk * 64 * dk * es + tv * 4       # W, U, K^T, G in
                   + NT * Nv * dk * dv * 4 + tv * dv * 4 + N * Nv * dk * dv * 4,  # H, V_new, S_T out
        "k_output": 2 * tk * dk * es + tv * 4 + NT * Nv * dk * dv * 4 + tv * dv * 4  # q, k, G, H, V_new in
                    + tv * dv * out_bytes,                                    # o out
    }


def measure_peaks(repeats: int = 5) -> dict:
    """The two roofline ceilings measured on this GPU with the library's probe
    kernels (include/gdr_peaks.h): a 1 GiB streaming copy (bytes read +
    written over time) and a loop of independent bf16 16x16x32 matrix-core
    products on every SIMD. Best of `repeats` timed launches after a warm-up."""
    lib = api.load_library()
    stream = torch.cuda.current_stream()
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def best(launch):
        launch()
        torch.cuda.synchronize()
        times = []
        for _ in range(repeats):
            ev[0].record()
            launch()
            ev[1].record()
            torch.cuda.synchronize()
            times.append(ev[0].elapsed_time(ev[1]))
        return min(times)

    copy_blocks = 256 * 8

    def copy():
        assert lib.gdr_peak_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                 ctypes.c_size_t(nbytes), copy_blocks, ctypes.c_void_p(stream.cuda_stream)) == 0
    t_copy = best(copy)
    if not torch.equal(dst[:1024], src[:1024]):
        raise RuntimeError("copy probe wrote wrong values")
    del src, dst
    mfma_blocks, iters = 256 * 4, 4096
    out = torch.empty(mfma_blocks * 256, dtype=torch.float32, device="cuda:0")

    def mfma():
        assert lib.gdr_peak_mfma(ctypes.c_void_p(out.data_ptr()), mfma_blocks, iters,
                                 ctypes.c_void_p(stream.cuda_stream)) == 0
    t_mfma = best(mfma)
    flops = lib.gdr_peak_mfma_flops(mfma_blocks, iters)
    return {"hbm_GBps": 2 * nbytes / (t_copy * 1e-3) / 1e9,
            "mfma_bf16_TFLOPs": flops / (t_mfma * 1e-3) / 1e12,
            "how": "gdr_peak_copy: 1 GiB read + 1 GiB written by %d workgroups (16-byte non-temporal accesses); "
                   "gdr_peak_mfma: %d workgroups x 4 wavefronts x %d x 8 independent "
                   "v_mfma_f32_16x16x32_bf16; best of %d" % (copy_blocks, mfma_blocks, iters, repeats)}


def source_digest() -> str:
    """Digest of the kernel sources' code: comments and blank lines are left out,
    so a counter summary stays valid across comment-only edits."""
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        lines = [re.sub(r"//.*$", "", l).rstrip() for l in text.splitlines()]
        h.update("\n".join(l for l in lines if l).encode())
    return h.hexdigest()[:16]


def counter_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, or None when there is none or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", "%s_%s_counters.txt" % (kernel, workload))
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                vals[key.strip()] = val.strip()
    if vals.get("source_digest") != source_digest():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(inp: dict, target_seconds: float, threads: int = 0) -> dict:
    """The fp64 token-recurrence oracle on the host cores over a bounded sample
    of the same workload: the first Ts tokens of every sequence (all heads),
    with Ts calibrated to about target_seconds (the whole workload when it
    fits). threads = 0: every core this process may run on."""
    from oracle import recurrence

    w = inp["workload"]
    threads = threads or len(os.sched_getaffinity(0))
    B, T = inp["q"].shape[:2]
    flat = lambda t: None if t is None else t.reshape((B * T,) + tuple(t.shape[2:]))
    q, k, v, beta, g = (flat(inp[n]) for n in ("q", "k", "v", "beta", "g"))
    if inp["cu_seqlens"] is not None:
        cu = inp["cu_seqlens"].numpy().astype(np.int64)
    else:
        cu = np.arange(B + 1, dtype=np.int64) * T
    lens = np.diff(cu)
    S0 = None if inp["S0"] is None else inp["S0"].double().numpy()

    def run(ts):
        take = np.minimum(lens, ts)
        idx = np.concatenate([np.arange(cu[n], cu[n] + take[n]) for n in range(len(lens))])
        sub = lambda t: None if t is None else t[torch.from_numpy(idx)].double().numpy()
        cs = np.concatenate([[0], np.cumsum(take)])
        args = (sub(q), sub(k), sub(v), sub(beta), sub(g))
        t0 = time.perf_counter()
        recurrence(*args, inp["scale"], S0, cs, threads=threads)
        return time.perf_counter() - t0, int(take.sum())

    longest = int(lens.max()) if len(lens) else 0
    probe = min(256, longest)
    dt, _ = run(probe)
    ts = int(min(longest, max(probe, probe * target_seconds / max(dt, 1e-6))))
    ts = max(64, (ts // 64) * 64) if ts < longest else longest
    dt, tokens = run(ts)
    return {
        "value": tokens / dt,
        "unit": "tokens/s",
        "cores": int(getattr(recurrence, "last_threads", threads)),
        "kind": "oracle",
        "sample": "the first %d tokens of each of the %d sequences (%d of %d tokens), all %d value heads; "
                  "fp64 C token recurrence, OpenMP over (sequence, head); %.1f s"
                  % (ts, len(lens), tokens, int(lens.sum()), w.Nv, dt),
    }


def copy_probe(mib: int) -> None:
    """A streaming elementwise kernel that reads and writes `mib` MiB each, three
    times: its FETCH_SIZE / WRITE_SIZE counter readings against the known byte
    counts give the scale factor applied to the kernels' counter readings."""
    n = mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4, "launches": 3}), flush=True)


def _counter_means(path: str, counter: str) -> dict:
    """Mean counter value per dispatch, by kernel name, from a rocprofv3 counter_collection.csv."""
    import csv
    sums, counts = {}, {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            name = row["Kernel_Name"]
            sums[name] = sums.get(name, 0.0) + float(row["Counter_Value"])
            counts[name] = counts.get(name, 0) + 1
    return {n: sums[n] / counts[n] for n in sums}


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_BUSY_CU_CYCLES")


def mfma_summary(src: str, out_dir: str) -> None:
    """Matrix-core utilisation of every gdr kernel from one rocprofv3 counter run
    (MFMA_COUNTERS, per dispatch): SQ_VALU_MFMA_BUSY_CYCLES (SIMD-cycles, summed
    over all SIMDs) over the kernel's SIMD-cycles, GRBM_GUI_ACTIVE / 8 (the
    counter is summed over the 8 XCDs) x 256 compute units x 4 SIMDs; and the
    issue-rate estimate SQ_INSTS_MFMA x 16 cycles (one v_mfma_f32_16x16x32_bf16
    on gfx950) over the same SIMD-cycles."""
    path = None
    for root, _, files in os.walk(src):
        for fn in files:
            if fn.endswith("counter_collection.csv"):
                path = os.path.join(root, fn)
    if path is None:
        raise FileNotFoundError(src)
    vals = {c: _counter_means(path, c) for c in MFMA_COUNTERS}
    cmd = ("rocprofv3 --pmc " + " ".join(MFMA_COUNTERS) +
           " -d <dir>/mfma -o run --output-format csv -- python3 bench.py --steps 3 --warmup 1 --cpu-seconds 0"
           " --no-peaks")
    lines = ["# Matrix-core utilisation per kernel, workload T65536_Nk16_Nv32_d128 (one forward per bench step)",
             "# command (run from the repository root):", "#   " + cmd,
             "#   python3 bench.py --mfma-summary <dir> --summary-out profiles",
             "# kernel cycles = GRBM_GUI_ACTIVE / 8 (the counter sums the 8 XCDs)",
             "# mfma_busy_frac = SQ_VALU_MFMA_BUSY_CYCLES / (kernel cycles * 256 CUs * 4 SIMDs)",
             "# mfma_issue_frac = SQ_INSTS_MFMA * 16 cycles / (kernel cycles * 256 * 4)",
             "# (counter values are means per dispatch)"]
    for name in sorted(vals["GRBM_GUI_ACTIVE"]):
        if "gdr" not in name:
            continue
        act = vals["GRBM_GUI_ACTIVE"][name]
        busy = vals["SQ_VALU_MFMA_BUSY_CYCLES"].get(name, float("nan"))
        insts = vals["SQ_INSTS_MFMA"].get(name, float("nan"))
        lines += ["", "kernel: %s" % name,
                  "grbm_gui_active: %.0f" % act,
                  "sq_valu_mfma_busy_cycles: %.0f" % busy,
                  "sq_insts_mfma: %.0f" % insts,
                  "sq_insts_valu: %.0f" % vals["SQ_INSTS_VALU"].get(name, float("nan")),
                  "sq_busy_cu_cycles: %.0f" % vals["SQ_BUSY_CU_CYCLES"].get(name, float("nan")),
                  "kernel_cycles: %.0f" % (act / 8),
                  "mfma_busy_frac: %.4f" % (busy / (act / 8 * 256 * 4)),
                  "mfma_issue_frac: %.4f" % (insts * 16 / (act / 8 * 256 * 4))]
    os.makedirs(out_dir, exist_ok=True)
    out = os.path.join(out_dir, "mfma_util_T65536_Nk16_Nv32_d128_counters.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)


def counter_summary(src: str, out_dir: str, workload: int) -> None:
    """HBM bytes per launch of every gdr kernel from FETCH_SIZE / WRITE_SIZE runs,
    each scaled by what the same counter reads for the copy probe of known size."""
    def csv_of(sub):
        for root, _, files in os.walk(os.path.join(src, sub)):
            for fn in files:
                if fn.endswith("counter_collection.csv"):
                    return os.path.join(root, fn)
        raise FileNotFoundError(os.path.join(src, sub))
    jobs = [("fetch", "write", "T65536_Nk16_Nv32_d128" if workload == 5 else "workload%d" % workload,
             "python3 bench.py --steps 3 --warmup 1 --cpu-seconds 0 --no-peaks")]
    if os.path.isdir(os.path.join(src, "rfetch")) and os.path.isdir(os.path.join(src, "rwrite")):
        jobs.append(("rfetch", "rwrite", "decode256_Nk16_Nv32_d128",
                     "python3 bench.py --mode recurrent --decode-seqs 256 --steps 3 --warmup 1"))
    for fdir, wdir, wl, cmd in jobs:
        _counter_summary_one(src, out_dir, csv_of, fdir, wdir, wl, cmd)


def _counter_summary_one(src, out_dir, csv_of, fdir, wdir, wl, cmd):
    fetch, write = _counter_means(csv_of(fdir), "FETCH_SIZE"), _counter_means(csv_of(wdir), "WRITE_SIZE")
    cfetch, cwrite = _counter_means(csv_of("cfetch"), "FETCH_SIZE"), _counter_means(csv_of("cwrite"), "WRITE_SIZE")
    probe = [n for n in cfetch if "neg_kernel" in n]
    if not probe:
        raise RuntimeError("copy-probe kernel not found in the calibration runs")
    probe_kib = 1024 * 1024.0                            # --copy-probe-mib 1024: 1 GiB read and 1 GiB written
    f_scale = probe_kib / cfetch[probe[0]]
    w_scale = probe_kib / cwrite[probe[0]]
    os.makedirs(out_dir, exist_ok=True)
    for name in sorted(fetch):
        short = next((k for k in sorted(STAGE_KERNELS + FP16_STAGE_KERNELS[:1] + ("k_prep", "k_chunk16", "k_recurrent"),
                                        key=len, reverse=True) if k in name), None)
        if short is None or name not in write:
            continue
        fb, wb = fetch[name] * f_scale * 1024.0, write[name] * w_scale * 1024.0
        path = os.path.join(out_dir, "%s_%s_counters.txt" % (short, wl))
        with open(path, "w") as f:
            f.write("# HBM traffic of %s, workload %s (one forward per bench step)\n" % (short, wl))
            f.write("# commands (run from the repository root):\n")
            f.write("#   rocprofv3 --pmc FETCH_SIZE -d <dir>/%s -o run --output-format csv -- %s\n" % (fdir, cmd))
            f.write("#   rocprofv3 --pmc WRITE_SIZE -d <dir>/%s -o run --output-format csv -- %s\n" % (wdir, cmd))
            f.write("#   rocprofv3 --pmc FETCH_SIZE -d <dir>/cfetch -o run --output-format csv -- "
                    "python3 bench.py --copy-probe-mib 1024\n")
            f.write("#   rocprofv3 --pmc WRITE_SIZE -d <dir>/cwrite -o run --output-format csv -- "
                    "python3 bench.py --copy-probe-mib 1024\n")
            f.write("#   python3 bench.py --counter-summary <dir> --summary-out profiles\n")
            f.write("# FETCH_SIZE / WRITE_SIZE are in KiB per dispatch; each is scaled by (known bytes of the\n")
            f.write("# copy probe) / (counter reading for the copy probe).\n")
            f.write("kernel: %s\n" % name)
            f.write("source_digest: %s\n" % source_digest())
            f.write("fetch_kib_per_dispatch_raw: %.1f\n" % fetch[name])
            f.write("write_kib_per_dispatch_raw: %.1f\n" % write[name])
            f.write("copy_probe_fetch_kib_raw: %.1f\n" % cfetch[probe[0]])
            f.write("copy_probe_write_kib_raw: %.1f\n" % cwrite[probe[0]])
            f.write("fetch_scale: %.4f\n" % f_scale)
            f.write("write_scale: %.4f\n" % w_scale)
            f.write("hbm_read_bytes_per_launch: %.0f\n" % fb)
            f.write("hbm_write_bytes_per_launch: %.0f\n" % wb)
            f.write("hbm_bytes_per_launch: %.0f\n" % (fb + wb))
        print(path)


def trace_summary(src: str, out_file: str, title: str, cmd: str) -> None:
    """Markdown table of a rocprofv3 --kernel-trace --stats run (run_kernel_stats.csv under src)."""
    import csv
    import re
    path = None
    for root, _, files in os.walk(src):
        for fn in files:
            if fn.endswith("kernel_stats.csv"):
                path = os.path.join(root, fn)
    if path is None:
        raise FileNotFoundError(src)
    rows = list(csv.DictReader(open(path)))
    total = sum(float(r["TotalDurationNs"]) for r in rows)

    def short(name):
        m = re.search(r"(k_[a-z0-9_]+)(?:I|E|<|\()", name)
        base = m.group(1) if m else name[:60]
        t = re.search(r"I(Li\d+E)+", name)
        if t:
            base += "<" + ", ".join(re.findall(r"Li(\d+)E", t.group(0))) + ">"
        return base
    lines = ["# Kernel trace: " + title, "", "Command (repository root):", "", "    " + cmd, "",
             "From `run_kernel_stats.csv` (durations in microseconds):", "",
             "| kernel | calls | average | min | max | share of GPU time |", "|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append("| %s | %s | %.1f | %.1f | %.1f | %.1f%% |" % (
            short(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, 100 * float(r["TotalDurationNs"]) / total))
    with open(out_file, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out_file)


def bench_recurrent(args) -> None:
    """One decode step per bench step: --decode-seqs sequences of one token each,
    16 q/k heads, 32 value heads, dk = dv = 128, bf16, from a random fp32 state,
    with the final state written. The step moves the state in and out of HBM;
    the roofline is the token-by-token kernel's bytes over its HIP-event time."""
    Nseq = args.decode_seqs
    w = synth.custom("decode-%dseq-Nk16-Nv32-d128" % Nseq, B=1, T=0, Nk=16, Nv=32, dk=128, dv=128, dtype="bf16",
                     g_mean=6.0, s0="randn", lengths=tuple([1] * Nseq))
    inp = synth.generate(w, seed=7)
    dev = torch.device("cuda:0")
    d = {k: (None if inp[k] is None else inp[k].to(dev)) for k in ("q", "k", "v", "beta", "g", "S0", "cu_seqlens")}
    run = lambda: api.recurrent_fwd(d["q"], d["k"], d["v"], d["beta"], g=d["g"], scale=inp["scale"],
                                    initial_state=d["S0"], output_final_state=True, cu_seqlens=d["cu_seqlens"],
                                    cu_seqlens_cpu=inp["cu_seqlens"])
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    K = args.steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(K):
        run()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / K
    state = Nseq * w.Nv * w.dk * w.dv * 4
    io = Nseq * (2 * w.Nk * w.dk * 2 + w.Nv * (w.dv * 2 + 2 + 4) + w.Nv * w.dv * 2)   # q, k, v, beta, g in; o out
    alg = 2 * state + io
    achieved = alg / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "decode tokens/s (token-by-token forward), %d sequences" % Nseq,
        "value": Nseq / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "seqs": Nseq, "Nk": w.Nk, "Nv": w.Nv, "dk": w.dk, "dv": w.dv, "seed": 7},
        "roofline": {"bound": "hbm", "kernel": "k_recurrent", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": counter_traffic("k_recurrent", "decode%d_Nk16_Nv32_d128" % Nseq),
                     "algorithmic_bytes": alg,
                     "avg_ms": ms},
        "cpu_baseline": None,
    }), flush=True)


def _stage_breakdown(fwd, K):
    """Mean ms of each forward stage (HIP events at every stage boundary)
    over K calls. Each recorded event adds a few microseconds between two
    launches, so these calls are kept out of the timed regions."""
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(api.NUM_STAGES + 1)] for _ in range(K)]
    for row in events:                     # create the HIP events before use
        for e in row:
            e.record()
    torch.cuda.synchronize()
    for s in range(K):
        fwd.timed(events[s])
    torch.cuda.synchronize()
    return np.array([[events[s][i].elapsed_time(events[s][i + 1]) for i in range(api.NUM_STAGES)]
                     for s in range(K)]).mean(axis=0)


def _time_forward(fwd, K, W):
    """Mean ms per forward over K timed calls (no events inside), and per
    stage from K more calls (None for a call that records no stage events)."""
    for _ in range(W):
        fwd()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(K):
        fwd()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / K, (_stage_breakdown(fwd, K) if fwd.stage_events else None)


def bench_chunk_sizes(args) -> None:
    """Chunk-size sensitivity on --workload: the five-kernel path at C = 16,
    32 and 64 (serial depth T/C of the state pass against the C x C solve and
    the C-wide intra-chunk products), each with its per-stage times, next to
    the fused C = 64 path that gdr_chunk_fwd runs for bf16. The five-kernel
    path at C = 64 is timed through gdr_chunk_fwd_debug with no intermediates
    requested (it then copies nothing; no per-stage times)."""
    w = synth.WORKLOADS[args.workload]
    inp = synth.generate(w, seed=args.workload)
    dev = torch.device("cuda:0")
    d = {k: (None if inp[k] is None else inp[k].to(dev)) for k in ("q", "k", "v", "beta", "g", "S0", "cu_seqlens")}
    K, W = args.steps, args.warmup
    B, T = inp["q"].shape[:2]
    Ttot = B * T
    rows = {}
    for C in (16, 32, 64):
        fwd = api.Forward(d["q"], d["k"], d["v"], d["beta"], g=d["g"], scale=inp["scale"], initial_state=d["S0"],
                          output_final_state=True, cu_seqlens=d["cu_seqlens"], cu_seqlens_cpu=inp["cu_seqlens"],
                          chunk_size=C, five_kernel=(C == 64))   # C < 64: gdr_chunk_fwd runs the five kernels
        ms, st = _time_forward(fwd, K, W)
        rows["five-kernel C=%d" % C] = {"ms_per_step": ms, "tokens_per_s": Ttot / (ms * 1e-3),
                                        "stage_ms": None if st is None else
                                        {api.STAGE_NAMES[i]: float(st[i]) for i in range(api.NUM_STAGES)}}
        del fwd
        torch.cuda.empty_cache()
    if w.dtype == "bf16":
        fwd = api.Forward(d["q"], d["k"], d["v"], d["beta"], g=d["g"], scale=inp["scale"], initial_state=d["S0"],
                          output_final_state=True, cu_seqlens=d["cu_seqlens"], cu_seqlens_cpu=inp["cu_seqlens"])
        ms, st = _time_forward(fwd, K, W)
        rows["fused C=64"] = {"ms_per_step": ms, "tokens_per_s": Ttot / (ms * 1e-3),
                              "stage_ms": {api.STAGE_NAMES[i]: float(st[i]) for i in range(api.NUM_STAGES)}}
    print(json.dumps({"metric": "fwd tokens/s by chunk size", "unit": "tokens/s", "n_gpus": 1, "steps": K,
                      "warmup": W, "dtype": w.dtype, "data": "synthetic",
                      "config": {"workload": w.name, "T": Ttot, "Nk": w.Nk, "Nv": w.Nv, "dk": w.dk, "dv": w.dv,
                                 "seed": args.workload},
                      "paths": rows}), flush=True)


FP32_VECTOR_PEAK_TFLOPS = 157.3


def backward_flops(w: synth.Workload, C: int, NT: int) -> dict:
    """Algorithmic flops (2 per multiply-add) of the backward kernels for NT
    chunks of C positions and Nv value heads: the matrix products each kernel
    forms, at full chunk length (the per-chunk pass: 16 products, listed in
    its source; the state pass: P^T dO over the lower triangle, K dS, Q^T dO
    and W^T dV_new per dv column; the preparation: Q K^T)."""
    dk, dv = w.dk, w.dv
    macs_chunk = (C * C * dv + C * dk * (dv + C) + C * dk * dv + C * dv * C + C * dk * C + C * C * (dv + dk)
                  + C * C * dk + 2 * C ** 3 + 3 * C * C * dk + C * dk * dv + C * dv * dk)
    macs_state = dv * (C * (C // 2 + dk) + 2 * dk * C)
    macs_prep = C * C * dk
    u = NT * w.Nv
    return {"k_bwd_chunk": 2 * macs_chunk * u, "k_bwd_state": 2 * macs_state * u, "k_bwd_prep": 2 * macs_prep * u}


def bench_backward(args) -> None:
    """The backward pass on --workload: dL/do and dL/dS_T are random, every
    gradient is written (dq, dk, dv, dbeta, dg, dh0), and the forward is
    recomputed inside the call (as a training step's backward would). Reports
    tokens/s of the whole backward, per-stage HIP-event times, the dominant
    kernel against the fp32 vector peak, and the oracle's backward on a bounded
    sample of one value head."""
    w = synth.WORKLOADS[args.workload]
    inp = synth.generate(w, seed=args.workload)
    dev = torch.device("cuda:0")
    d = {k: (None if inp[k] is None else inp[k].to(dev)) for k in ("q", "k", "v", "beta", "g", "S0", "cu_seqlens")}
    B, T = inp["q"].shape[:2]
    Ttot, N = B * T, inp["N"]
    rng = np.random.default_rng(11)
    do = torch.from_numpy(rng.standard_normal((B, T, w.Nv, w.dv)).astype(np.float32)).to(inp["q"].dtype).to(dev)
    dST = torch.from_numpy(rng.standard_normal((N, w.Nv, w.dk, w.dv)).astype(np.float32)).to(dev)
    bwd = api.Backward(d["q"], d["k"], d["v"], d["beta"], g=d["g"], scale=inp["scale"], initial_state=d["S0"],
                       cu_seqlens=d["cu_seqlens"], cu_seqlens_cpu=inp["cu_seqlens"], d_o=do, d_final_state=dST)
    K, W = args.steps, args.warmup
    for _ in range(W):
        bwd()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(api.BWD_NUM_STAGES + 1)] for _ in range(K)]
    for row in events:
        for e in row:
            e.record()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for s in range(K):
        bwd.timed(events[s])
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / K
    st = np.array([[events[s][i].elapsed_time(events[s][i + 1]) for i in range(api.BWD_NUM_STAGES)]
                   for s in range(K)]).mean(axis=0)
    NT = api.num_chunks(B, T, None if inp["cu_seqlens"] is None else inp["cu_seqlens"].to(torch.int32))
    flops = backward_flops(w, 64, NT)
    dom = int(np.argmax(st[1:])) + 1              # dominant backward kernel (the forward recompute aside)
    kname = api.BWD_STAGE_NAMES[dom]
    achieved = flops.get(kname, 0) / (st[dom] * 1e-3) / 1e12
    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_backward_baseline(inp, args.cpu_seconds)
    print(json.dumps({
        "metric": "bwd tokens/s (gradients of q, k, v, beta, g, h0; forward recomputed)",
        "value": Ttot / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "T": Ttot, "Nk": w.Nk, "Nv": w.Nv, "dk": w.dk, "dv": w.dv, "chunk": 64,
                   "io_dtype": w.dtype, "seed": args.workload},
        "stage_ms": {api.BWD_STAGE_NAMES[i]: float(st[i]) for i in range(api.BWD_NUM_STAGES)},
        "roofline": {"bound": "alu", "kernel": kname, "achieved": achieved, "peak": FP32_VECTOR_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / FP32_VECTOR_PEAK_TFLOPS, "traffic": None,
                     "algorithmic_flops": flops.get(kname, 0), "avg_ms": float(st[dom])},
        "cpu_baseline": cpu,
    }), flush=True)


def cpu_backward_baseline(inp: dict, target_seconds: float) -> dict:
    """The backward oracle (NumPy, fp64) on the first sequence of value head 0,
    over as many tokens as fit in about target_seconds (timed on a growing
    prefix), scaled to tokens/s of all value heads."""
    from oracle import recurrence_backward

    w = inp["workload"]
    kh = 0
    q = inp["q"].reshape(-1, w.Nk, w.dk)[:, kh:kh + 1].double().numpy()
    k = inp["k"].reshape(-1, w.Nk, w.dk)[:, kh:kh + 1].double().numpy()
    v = inp["v"].reshape(-1, w.Nv, w.dv)[:, :1].double().numpy()
    beta = inp["beta"].reshape(-1, w.Nv)[:, :1].double().numpy()
    g = None if inp["g"] is None else inp["g"].reshape(-1, w.Nv)[:, :1].double().numpy()
    rng = np.random.default_rng(0)
    n = 64
    while True:
        do = rng.standard_normal((n, 1, w.dv))
        t0 = time.perf_counter()
        recurrence_backward(q[:n], k[:n], v[:n], beta[:n], None if g is None else g[:n], inp["scale"], None,
                            None, do, None)
        dt = time.perf_counter() - t0
        if dt > target_seconds / 4 or n * 2 > q.shape[0]:
            break
        n *= 2
    rate = n / dt / w.Nv                          # tokens/s over all value heads
    return {"value": rate, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": "%d tokens of one value head (NumPy fp64 backward), scaled by 1/%d heads" % (n, w.Nv)}


def bench_segmented(args) -> None:
    """Segment-parallel state passing against the serial pass on one long
    sequence with few heads (64k tokens, 2 q/k heads, 4 value heads, dk = dv =
    128, bf16): the serial state pass has 4 x 8 = 32 workgroups for 256 compute
    units. Reports the segmented forward (--segment-chunks, 0 = the library's
    choice), the serial forward, a sweep of segment lengths, and the largest
    difference between the two outputs."""
    w = synth.custom("long-1seq-Nk2-Nv4-T65536-d128", B=1, T=65536, Nk=2, Nv=4, dk=128, dv=128, dtype="bf16",
                     g_mean=6.0, s0="zero")
    inp = synth.generate(w, seed=8)
    dev = torch.device("cuda:0")
    d = {k: (None if inp[k] is None else inp[k].to(dev)) for k in ("q", "k", "v", "beta", "g", "S0")}
    make = lambda sc: api.Forward(d["q"], d["k"], d["v"], d["beta"], g=d["g"], scale=inp["scale"],
                                  initial_state=d["S0"], output_final_state=True, segment_chunks=sc)
    K, W = args.steps, args.warmup
    serial = make(None)
    ms_serial, st_serial = _time_forward(serial, K, W)
    seg = make(args.segment_chunks)
    ms_seg, st_seg = _time_forward(seg, K, W)
    torch.cuda.synchronize()
    # the outputs are bf16: their difference is counted in bf16 steps (spacing at the larger
    # value) plus 1e-4 of the rms, as in the parity tests
    o_a, o_b = serial.o.float(), seg.o.float()
    mag = torch.maximum(o_a.abs(), o_b.abs())
    step = torch.where(mag > 0, torch.exp2(torch.floor(torch.log2(mag)) - 7), torch.zeros_like(mag))
    rms = float(o_a.pow(2).mean().sqrt())
    diff_o = float(((o_a - o_b).abs() / (step + 1e-4 * rms)).max())
    diff_s = float((serial.final_state - seg.final_state).abs().max()) / float(
        serial.final_state.pow(2).mean().sqrt())
    sweep = {}
    for sc in (16, 32, 64, 128, 256):
        f = make(sc)
        sweep[str(sc)] = _time_forward(f, max(5, K // 4), 2)[0]
        del f
    Ttot = w.T
    NT = Ttot // 64
    alg = method_bytes_per_token(w, 2) * Ttot
    achieved = alg / (st_seg[4] * 1e-3) / 1e9
    print(json.dumps({
        "metric": "fwd tokens/s, one 64k-token sequence with 4 value heads (segment-parallel state passing)",
        "value": Ttot / (ms_seg * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": ms_seg, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "T": Ttot, "Nk": w.Nk, "Nv": w.Nv, "dk": w.dk, "dv": w.dv, "chunk": 64,
                   "segment_chunks": args.segment_chunks, "seed": 8},
        "serial": {"ms_per_step": ms_serial, "value": Ttot / (ms_serial * 1e-3),
                   "state_stage_ms": float(st_serial[4])},
        "speedup_vs_serial": ms_serial / ms_seg,
        "state_stage_ms": float(st_seg[4]),
        "stage_ms": {("%d:%s" % (i, api.STAGE_NAMES[i])): float(st_seg[i]) for i in range(api.NUM_STAGES)},
        "sweep_ms_per_step": sweep,
        "diff_vs_serial": {"o_max_bf16_steps": diff_o, "S_T_max_over_rms": diff_s},
        "roofline": {"bound": "hbm", "kernel": "state stage (segment pass, scan, output pass)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": None, "algorithmic_bytes": alg, "avg_ms": float(st_seg[4])},
        "cpu_baseline": None,
    }), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=5, help="synth.WORKLOADS index (default 5)")
    ap.add_argument("--out-dtype", choices=("io", "f32"), default="io")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU-baseline budget; 0 skips it")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB three times (calibrates HBM byte counters)")
    ap.add_argument("--mode", choices=("chunk", "recurrent", "segmented", "chunk-sizes", "backward", "configs"),
                    default="chunk",
                    help="chunk: the chunked forward on --workload (default); recurrent: one decode step "
                         "(token-by-token kernel) for --decode-seqs sequences from a random state; segmented: "
                         "segment-parallel against serial state passing on one long sequence with few heads; "
                         "chunk-sizes: the five-kernel path at C = 16, 32, 64 and the fused path on --workload; "
                         "backward: the backward pass (forward recomputed) on --workload; "
                         "configs: every synthetic workload 1-5 with the oracle beside it")
    ap.add_argument("--segment-chunks", type=int, default=0,
                    help="chunks per segment in --mode segmented (0: the library's choice)")
    ap.add_argument("--decode-seqs", type=int, default=64)
    ap.add_argument("--counter-summary", metavar="DIR",
                    help="only summarise rocprofv3 counter runs found under DIR (fetch/, write/, cfetch/, cwrite/) "
                         "into one text file per kernel, written to --summary-out")
    ap.add_argument("--mfma-summary", metavar="DIR",
                    help="only summarise a rocprofv3 run of MFMA_COUNTERS found under DIR into profiles/")
    ap.add_argument("--summary-out", metavar="DIR", default="profiles")
    ap.add_argument("--trace-summary", nargs=4, metavar=("DIR", "OUT_FILE", "TITLE", "COMMAND"),
                    help="only write a markdown summary of a rocprofv3 --kernel-trace --stats run")
    ap.add_argument("--summary-file", metavar="FILE", help="--mode configs: also write a markdown table here")
    ap.add_argument("--no-peaks", dest="peaks", action="store_false",
                    help="skip measuring the HBM-copy and matrix-core peaks")
    args = ap.parse_args()
    if args.counter_summary:
        counter_summary(args.counter_summary, args.summary_out, args.workload)
        return
    if args.mfma_summary:
        mfma_summary(args.mfma_summary, args.summary_out)
        return
    if args.trace_summary:
        trace_summary(*args.trace_summary)
        return
    if args.gpus != 1:
        print("bench.py: this implementation runs on one GPU only; --gpus %d is not supported" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe_mib > 0:
        copy_probe(args.copy_probe_mib)
        return
    if args.mode == "recurrent":
        bench_recurrent(args)
        return
    if args.mode == "segmented":
        bench_segmented(args)
        return
    if args.mode == "chunk-sizes":
        bench_chunk_sizes(args)
        return
    if args.mode == "backward":
        bench_backward(args)
        return
    if args.mode == "configs":
        bench_configs(args)
        return

    w = synth.WORKLOADS[args.workload]
    inp = synth.generate(w, seed=args.workload)
    dev = torch.device("cuda:0")
    d = {k: (None if inp[k] is None else inp[k].to(dev)) for k in ("q", "k", "v", "beta", "g", "S0", "cu_seqlens")}
    out_dtype = torch.float32 if args.out_dtype == "f32" else None
    fwd = api.Forward(d["q"], d["k"], d["v"], d["beta"], g=d["g"], scale=inp["scale"], initial_state=d["S0"],
                      output_final_state=True, cu_seqlens=d["cu_seqlens"], cu_seqlens_cpu=inp["cu_seqlens"],
                      out_dtype=out_dtype)
    B, T = inp["q"].shape[:2]
    Ttot = B * T
    N = inp["N"]
    NT = api.num_chunks(B, T, None if inp["cu_seqlens"] is None else inp["cu_seqlens"].to(torch.int32))

    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()

    K = args.steps
    # per-stage times from K calls outside the timed region; they name the
    # dominant stage
    stage_ms = _stage_breakdown(fwd, K)
    dom = int(np.argmax(stage_ms))
    # timed region: K calls that record only the two events around the
    # dominant stage, whose launch time the roofline line divides by
    pairs = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in range(K)]
    for a, b in pairs:
        a.record()
        b.record()
    timed_events = [[None] * dom + [a, b] + [None] * (api.NUM_STAGES - dom - 1) for a, b in pairs]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for s in range(K):
        fwd.timed(timed_events[s])
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / K
    dom_ms = float(np.mean([a.elapsed_time(b) for a, b in pairs]))

    out_bytes = 4 if (args.out_dtype == "f32" or w.dtype == "f32") else 2
    io = stage_io_bytes(w, Ttot, N, NT, out_bytes, inp["S0"] is not None)
    names = FP16_STAGE_KERNELS if w.dtype == "bf16" else STAGE_KERNELS
    kname = names[dom]
    bpt = method_bytes_per_token(w, out_bytes)
    fpt = method_flops_per_token(w)
    alg_bytes = bpt * Ttot
    alg_flops = fpt * Ttot
    achieved = alg_bytes / (dom_ms * 1e-3) / 1e9
    traffic = counter_traffic(kname, "T65536_Nk16_Nv32_d128" if args.workload == 5 else "workload%d" % args.workload)
    mfma_peak = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_MFMA_PEAK_TFLOPS
    peaks = measure_peaks() if args.peaks else None

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(inp, args.cpu_seconds)

    step_s = ms_per_step * 1e-3
    e2e = {
        "bytes_per_token": bpt, "flop_per_token": fpt,
        "hbm_GBps": alg_bytes / step_s / 1e9, "hbm_frac": alg_bytes / step_s / 1e9 / HBM_PEAK_GBS,
        "mfma_TFLOPs": alg_flops / step_s / 1e12, "mfma_frac": alg_flops / step_s / 1e12 / mfma_peak,
        "mfma_peak": mfma_peak,
    }
    if peaks is not None:
        e2e["hbm_frac_measured_peak"] = e2e["hbm_GBps"] / peaks["hbm_GBps"]
        if w.dtype == "bf16":
            e2e["mfma_frac_measured_peak"] = e2e["mfma_TFLOPs"] / peaks["mfma_bf16_TFLOPs"]
    line = {
        "metric": METRIC,
        "value": Ttot * K / (total_ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "T": Ttot, "Nk": w.Nk, "Nv": w.Nv, "dk": w.dk, "dv": w.dv, "chunk": 64,
                   "gated": w.gated, "g": "logsigmoid(N(%g,1))" % w.g_mean, "S0": w.s0,
                   "out_dtype": "f32" if out_bytes == 4 else w.dtype, "seed": args.workload},
        # dominant kernel: the method's algorithmic bytes over its average launch time
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes": alg_bytes, "bytes_per_token": bpt, "avg_ms": dom_ms,
                     "kernel_io_bytes": io[kname],
                     "mfma_frac": alg_flops / (dom_ms * 1e-3) / 1e12 / mfma_peak},
        "end_to_end": e2e,
        "measured_peaks": peaks,
        "cpu_baseline": cpu,
        "stage_ms": {("%d:%s" % (i, names[i])): float(stage_ms[i]) for i in range(api.NUM_STAGES)},
    }
    print(json.dumps(line), flush=True)


def bench_configs(args) -> None:
    """Every synthetic workload (1-5): median and p90 of per-call HIP-event
    times over --steps calls after --warmup, tokens/s, and the end-to-end
    algorithmic fractions of HBM and matrix-core peaks; the oracle's token
    recurrence timed beside it on all host threads (bounded sample) and, for
    workloads 1-3, on one thread. One JSON line per workload; with
    --summary-file, also a markdown table there."""
    peaks = measure_peaks() if args.peaks else None
    rows = []
    for cfg in range(1, 6):
        w = synth.WORKLOADS[cfg]
        inp = synth.generate(w, seed=cfg)
        dev = torch.device("cuda:0")
        d = {k: (None if inp[k] is None else inp[k].to(dev)) for k in ("q", "k", "v", "beta", "g", "S0",
                                                                          "cu_seqlens")}
        fwd = api.Forward(d["q"], d["k"], d["v"], d["beta"], g=d["g"], scale=inp["scale"], initial_state=d["S0"],
                          output_final_state=True, cu_seqlens=d["cu_seqlens"], cu_seqlens_cpu=inp["cu_seqlens"])
        B, T = inp["q"].shape[:2]
        Ttot = B * T
        for _ in range(args.warmup):
            fwd()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for a, b in ev:
            a.record()
            fwd()
            b.record()
        torch.cuda.synchronize()
        t = np.array([a.elapsed_time(b) for a, b in ev])
        med, p90 = float(np.median(t)), float(np.percentile(t, 90))
        out_bytes = 2 if w.dtype == "bf16" else 4
        bpt, fpt = method_bytes_per_token(w, out_bytes), method_flops_per_token(w)
        mfma_peak = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_MFMA_PEAK_TFLOPS
        hbm = bpt * Ttot / (med * 1e-3) / 1e9
        tf = fpt * Ttot / (med * 1e-3) / 1e12
        row = {"workload": w.name, "cfg": cfg, "tokens": Ttot, "median_ms": med, "p90_ms": p90,
               "tokens_per_s": Ttot / (med * 1e-3), "hbm_GBps": hbm, "hbm_frac": hbm / HBM_PEAK_GBS,
               "mfma_TFLOPs": tf, "mfma_frac": tf / mfma_peak, "mfma_peak": mfma_peak}
        if peaks is not None:
            row["hbm_frac_measured_peak"] = hbm / peaks["hbm_GBps"]
            if w.dtype == "bf16":
                row["mfma_frac_measured_peak"] = tf / peaks["mfma_bf16_TFLOPs"]
        if args.cpu_seconds > 0:
            row["oracle"] = cpu_baseline(inp, args.cpu_seconds)
            if cfg <= 3:
                row["oracle_1thread"] = cpu_baseline(inp, args.cpu_seconds, threads=1)
        del fwd, d
        torch.cuda.empty_cache()
        rows.append(row)
        print(json.dumps(row), flush=True)
    if args.summary_file:
        lines = ["# Forward throughput on every synthetic workload", "",
                 "command: `python3 bench.py --mode configs --steps %d --warmup %d --cpu-seconds %g --summary-file "
                 "<file>`" % (args.steps, args.warmup, args.cpu_seconds), ""]
        if peaks is not None:
            lines += ["Measured peaks: HBM copy %.0f GB/s, bf16 matrix cores %.0f TFLOP/s (%s)." % (
                peaks["hbm_GBps"], peaks["mfma_bf16_TFLOPs"], peaks["how"]), ""]
        lines += ["| cfg | workload | tokens | median ms | p90 ms | tokens/s | HBM frac (spec / measured) "
                  "| MFMA frac (spec / measured) | oracle tokens/s (threads) | oracle 1 thread |",
                  "|---|---|---|---|---|---|---|---|---|---|"]
        for r in rows:
            o = r.get("oracle")
            o1 = r.get("oracle_1thread")
            lines.append("| %d | %s | %d | %.4f | %.4f | %.3g | %.4f / %s | %.4f / %s | %s | %s |" % (
                r["cfg"], r["workload"], r["tokens"], r["median_ms"], r["p90_ms"], r["tokens_per_s"],
                r["hbm_frac"], "%.4f" % r["hbm_frac_measured_peak"] if "hbm_frac_measured_peak" in r else "-",
                r["mfma_frac"], "%.4f" % r["mfma_frac_measured_peak"] if "mfma_frac_measured_peak" in r else "-",
                "%.3g (%d)" % (o["value"], o["cores"]) if o else "-",
                "%.3g" % o1["value"] if o1 else "-"))
        lines += ["", "Fractions are the method's algorithmic bytes (q, k, v, g, beta read once, o written once) "
                  "and flops (6 dk dv + 2C(3dk + 2dv) + (2/3)C^2 per token-head) over the median call time, "
                  "against the published peaks (HBM 8 TB/s; bf16 2.5 PFLOP/s, fp32 157.3 TFLOP/s for "
                  "workload 1) and the measured ones."]
        with open(args.summary_file, "w") as f:
            f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
