"""Benchmark of the exact-attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic inputs:
  1. fa_fwd on the GPT-2-medium-shaped prefill: B=64, H=16, N=Nk=1024,
     d=dv=64, bf16, causal (inputs 0.5*N(0,1));
  2. fa_decode_splitkv on the long-context decode: B=8, H=32, N=1,
     Nk=32768, d=dv=128, bf16, 64 splits (segment kernel + merge kernel);
  3. fa_fwd on the long-sequence prefill: B=2, H=32, N=Nk=8192, d=dv=128,
     bf16, causal (reported in its own sub-record).
In this order each prefill launch follows at least 0.5 GB of other traffic
(the decode streams 4.3 GB of K/V, the long prefill touches 0.5 GB), which
is larger than every cache (L2 4 MB per XCD, MALL 256 MB): that traffic is
the cache flush between prefill repetitions.

Inputs are drawn on the GPU with seeded generators before timing starts.
Every launch is bracketed by HIP events recorded on the stream the library
launches on (torch's current stream), so per-kernel times are live device
times.  ``value`` is the prefill throughput in TFLOP/s, crediting
4*N*Nk*d per head, halved for the causal mask (sum of credited FLOPs over
the timed steps / sum of the prefill launch times).  The decode figures
(HBM GB/s over K+V+Q+O+LSE bytes) are reported beside it.

The CPU baseline is the FP64 oracle (test infrastructure) timed on a bounded
sample of the prefill workload on the host cores, in the same run.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       python bench.py --summarize-pmc DIR   (turn rocprofv3 --pmc CSVs into
                                              the traffic summary under profiles/)
       python bench.py --summarize-trace DIR (kernel-trace statistics -> profiles/)
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import itertools
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn fwd TFLOP/s (% bf16 MFMA peak); split-KV decode HBM GB/s (% peak)"
PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_HBM_GBS = 8000.0          # HBM3E
PREFILL = "prefill_b64_h16_n1024_d64"
DECODE = "decode_b8_h32_nk32768_d128"
LONG = "prefill_b2_h32_n8192_d128"
# Kernel names (demangled template arguments) of the forward launches the
# default step makes: bf16, (d, dv) = (64, 64) and (128, 128), causal.
FWD_C3_NAME = "fwd_mfma32_kernelIDF16bLi64ELi64ELb1E"
FWD_C4_NAME = "fwd_mfma32_kernelIDF16bLi128ELi128ELb1E"
FWD_KERNEL_SRC = os.path.join(ROOT, "exact_tiled_attention_flashattention_amd", "csrc",
                              "fa_fwd_mfma_wide.hip")
DEC_KERNEL_SRC = os.path.join(ROOT, "exact_tiled_attention_flashattention_amd", "csrc",
                              "fa_decode.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.txt")
COPY_BYTES = 1 << 30           # plain copy used to calibrate the traffic counters


def credited_flops(s, causal: bool) -> float:
    per_head = 4.0 * s.N * s.Nk * s.d
    if causal:
        per_head /= 2
    return per_head * s.B * s.H


def decode_bytes(s) -> int:
    """Algorithmic bytes of one decode call: K and V once, Q, O (bf16), LSE (fp32)."""
    e = 2
    return (s.B * s.H * (2 * s.Nk * s.d * e + s.N * s.d * e + s.N * s.dv * e + s.N * 4))


def source_hash(path: str) -> str:
    """Hash of a kernel source together with the library headers it includes."""
    csrc = os.path.dirname(path)
    with open(path) as f:
        local = re.findall(r'^#include "([^"]+)"', f.read(), re.M)
    h = hashlib.sha256()
    for p in [path, *sorted(os.path.join(csrc, n) for n in local)]:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic():
    """Per-launch HBM traffic from the committed counter summary, or None per
    kernel if absent or if that kernel's source changed since it was taken."""
    out = {"fwd": None, "decode": None, "long": None}
    if not os.path.exists(TRAFFIC_FILE):
        return out
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                a, b = line.split(":", 1)
                kv[a.strip()] = b.strip()
    try:
        if kv.get("fwd_source_sha256_16") == source_hash(FWD_KERNEL_SRC):
            out["fwd"] = float(kv["fwd_bytes_per_launch"])
            if "long_bytes_per_launch" in kv:
                out["long"] = float(kv["long_bytes_per_launch"])
        if kv.get("decode_source_sha256_16") == source_hash(DEC_KERNEL_SRC):
            out["decode"] = float(kv["decode_bytes_per_launch"])
    except (KeyError, ValueError):
        pass
    return out


def cpu_baseline(q, k, v, s, causal, heads: int):
    """The FP64 oracle on the first ``heads`` heads of the prefill inputs."""
    import oracle
    import synth_inputs as si
    # The oracle runs on at most 16 threads: a one-GPU machine gives a job 16
    # CPU threads, whatever the affinity mask shows.
    available = len(os.sched_getaffinity(0))
    threads = max(1, min(16, available))
    qb = q.reshape(-1, s.N, s.d)[:heads]
    kb = k.reshape(-1, s.Nk, s.d)[:heads]
    vb = v.reshape(-1, s.Nk, s.dv)[:heads]
    qf, kf, vf = si.as_f64(qb), si.as_f64(kb), si.as_f64(vb)
    orc = oracle.default()
    t0 = time.perf_counter()
    orc.attention(qf, kf, vf, causal=causal, scale=1.0 / math.sqrt(s.d), nthreads=threads)
    dt = time.perf_counter() - t0
    flops = credited_flops(s, causal) * heads / (s.B * s.H)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
            "cores_in_affinity_mask": available, "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"{heads} of {s.B * s.H} heads of {PREFILL} (FP64 standard attention, "
                      f"{flops / 1e9:.1f} GFLOP credited, {dt:.2f} s wall on {threads} threads)"}


def sclk_files():
    """The DPM shader-clock tables of the amdgpu devices (sysfs pp_dpm_sclk)."""
    return sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))


def read_sclk(paths):
    """Current shader clock (MHz) of each DPM table: the level marked '*'."""
    out = []
    for p in paths:
        try:
            with open(p) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        mhz = line.split(":", 1)[1].strip().rstrip("*").strip()
                        out.append(float(mhz.lower().replace("mhz", "").strip()))
                        break
        except (OSError, ValueError, IndexError):
            pass
    return out


def cpu_model() -> str:
    """The host CPU's model name (first entry of /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def summarize_pmc(directory: str) -> None:
    """Build profiles/traffic_counters.txt from two rocprofv3 --pmc runs
    (FETCH_SIZE and WRITE_SIZE, KiB per dispatch) that include the 1 GiB
    calibration copy; the copy's counters give the KiB->byte scale."""
    import csv
    rows = []
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            rows += list(csv.DictReader(f))
    if not rows:
        raise SystemExit(f"no counter_collection.csv under {directory}")

    def values(counter, pred):
        return [float(r["Counter_Value"]) for r in rows
                if r["Counter_Name"] == counter and pred(r["Kernel_Name"])]

    def per_kernel(counter, pred):
        vals = values(counter, pred)
        return sum(vals) / len(vals) if vals else None

    is_fwd = lambda n: FWD_C3_NAME in n
    is_long = lambda n: FWD_C4_NAME in n
    is_seg = lambda n: "decode_segment_kernel" in n
    is_merge = lambda n: "decode_merge_kernel" in n
    # The 1 GiB calibration copy is a device-to-device memcpy; it is by far the
    # largest copyBuffer dispatch of the run, so take the largest reading.
    is_copy = lambda n: "copyBuffer" in n
    out = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        cps = values(counter, is_copy)
        if not cps:
            raise SystemExit(f"no calibration copy kernel found for {counter}")
        cp = max(cps)
        scale = COPY_BYTES / (cp * 1024.0)   # true bytes per counted byte
        out[counter] = {"copy_kib": cp, "scale": scale,
                        "fwd_kib": per_kernel(counter, is_fwd),
                        "long_kib": per_kernel(counter, is_long),
                        "seg_kib": per_kernel(counter, is_seg),
                        "merge_kib": per_kernel(counter, is_merge)}
    fetch, write = out["FETCH_SIZE"], out["WRITE_SIZE"]
    fwd_b = (fetch["fwd_kib"] * 1024 * fetch["scale"] + write["fwd_kib"] * 1024 * write["scale"])
    long_b = (fetch["long_kib"] * 1024 * fetch["scale"] + write["long_kib"] * 1024 * write["scale"]
              if fetch["long_kib"] is not None and write["long_kib"] is not None else None)
    dec_b = ((fetch["seg_kib"] + fetch["merge_kib"]) * 1024 * fetch["scale"]
             + (write["seg_kib"] + write["merge_kib"]) * 1024 * write["scale"])
    lines = [
        "# HBM traffic per launch from rocprofv3 --pmc (FETCH_SIZE and WRITE_SIZE, KiB per",
        "# dispatch, averaged over dispatches), each scaled so that a plain 1 GiB device copy",
        "# reads and writes exactly 1 GiB.  Made by: python bench.py --summarize-pmc <dir>,",
        "# <dir> holding the CSV output of (run from /tmp, repo at $R):",
        "#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/pmc_fetch -o run -- \\",
        "#       python $R/bench.py --no-cpu-baseline --steps 3 --warmup 1 --calibration-copy",
        "#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/pmc_write -o run -- \\",
        "#       python $R/bench.py --no-cpu-baseline --steps 3 --warmup 1 --calibration-copy",
        f"copy_fetch_kib: {fetch['copy_kib']:.1f}",
        f"copy_write_kib: {write['copy_kib']:.1f}",
        f"fetch_scale: {fetch['scale']:.6f}",
        f"write_scale: {write['scale']:.6f}",
        f"fwd_fetch_kib: {fetch['fwd_kib']:.1f}",
        f"fwd_write_kib: {write['fwd_kib']:.1f}",
        f"fwd_bytes_per_launch: {fwd_b:.0f}",
        f"fwd_source_sha256_16: {source_hash(FWD_KERNEL_SRC)}",
        *([f"long_fetch_kib: {fetch['long_kib']:.1f}",
           f"long_write_kib: {write['long_kib']:.1f}",
           f"long_bytes_per_launch: {long_b:.0f}"] if long_b is not None else []),
        f"decode_segment_fetch_kib: {fetch['seg_kib']:.1f}",
        f"decode_segment_write_kib: {write['seg_kib']:.1f}",
        f"decode_merge_fetch_kib: {fetch['merge_kib']:.1f}",
        f"decode_merge_write_kib: {write['merge_kib']:.1f}",
        f"decode_bytes_per_launch: {dec_b:.0f}",
        f"decode_source_sha256_16: {source_hash(DEC_KERNEL_SRC)}",
    ]
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_trace(directory: str) -> None:
    """Write the per-kernel rocprofv3 --kernel-trace --stats summaries of the
    library's kernels under profiles/, one file per entry point."""
    import csv
    paths = glob.glob(os.path.join(directory, "**", "*kernel_stats.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no kernel_stats.csv under {directory}")
    rows = list(csv.DictReader(open(paths[0])))
    default_cmd = ("rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/trace -o run -- "
                   "python $R/bench.py --no-cpu-baseline   (run from /tmp, repo at $R; 50 timed + "
                   "10 warm-up steps, each two fa_fwd calls and one fa_decode_splitkv call)")
    gqa_cmd = ("rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/trace_gqa -o run -- "
               "python $R/bench.py --only gqa   (run from /tmp, repo at $R; 50 timed + 10 warm-up "
               "fa_decode_splitkv_gqa calls)")
    bwd_cmd = ("rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/trace_bwd -o run -- "
               "python $R/bench.py --only bwd   (run from /tmp, repo at $R; 50 timed + 10 warm-up "
               "fa_bwd calls)")
    # file -> (kernel that must be in the trace, kernels listed, command)
    groups = {
        f"fwd_mfma32_kernel_{PREFILL}.txt": (FWD_C3_NAME, (FWD_C3_NAME,), default_cmd),
        f"fwd_mfma32_kernel_{LONG}.txt": (FWD_C4_NAME, (FWD_C4_NAME,), default_cmd),
        f"decode_splitkv_{DECODE}.txt": ("decode_segment_kernel",
                                         ("decode_segment_kernel", "decode_merge_kernel"),
                                         default_cmd),
        f"decode_splitkv_gqa_{GQA_WORKLOAD}.txt": ("decode_segment_mfma_kernel",
                                                   ("decode_segment_mfma_kernel",
                                                    "decode_merge_kernel"), gqa_cmd),
        f"bwd_mfma_{PREFILL}.txt": ("bwd_dq_mfma",
                                    ("bwd_dkdv_mfma", "bwd_dq_mfma", "bwd_dot_kernel"), bwd_cmd),
    }
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    for fname, (primary, keys, cmd) in groups.items():
        # Only the run that times this entry point (a run may launch others once).
        if not any(primary in r["Name"] and int(r["Calls"]) >= 10 for r in rows):
            continue
        lines = [f"# rocprofv3 kernel-trace statistics, {fname[:-4]}",
                 f"# command: {cmd}",
                 "# kernel | calls | average us | min us | max us | share of traced GPU time %"]
        for r in rows:
            if any(k in r["Name"] for k in keys):
                lines.append(f"{r['Name']} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                             f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                             f"{float(r['Percentage']):.2f}")
        with open(os.path.join(ROOT, "profiles", fname), "w") as f:
            f.write("\n".join(lines) + "\n")
        print("\n".join(lines))


GQA = dict(B=8, Hq=32, Hkv=8, Nk=32768, d=128, num_splits=0, seed_q=41, seed_kv=42)   # 0: automatic
GQA_WORKLOAD = "decode_gqa_b8_hq32_hkv8_nk32768_d128"


def bench_gqa(args, torch, fa, si, dev) -> int:
    """Grouped-query split-KV decode: 4 query heads per key/value head, the
    long-context decode size with 8 key/value heads, with the automatic split
    count (num_splits = 0).  Algorithmic bytes are K and V once per key/value
    head plus Q, O (bf16) and LSE (fp32)."""
    g = GQA
    q, _, _ = si.device_qkv(si.Shape(g["B"], g["Hq"], 1, 1, g["d"], g["d"]), g["seed_q"], "bf16", dev)
    _, k, v = si.device_qkv(si.Shape(g["B"], g["Hkv"], 1, g["Nk"], g["d"], g["d"]), g["seed_kv"],
                            "bf16", dev)
    o = torch.empty((g["B"], g["Hq"], 1, g["d"]), dtype=q.dtype, device=dev)
    lse = torch.empty((g["B"], g["Hq"], 1), dtype=torch.float32, device=dev)
    splits = g["num_splits"] or fa.decode_splitkv_auto_splits(g["B"], g["Hq"], g["Hkv"], 1, g["Nk"],
                                                               g["d"], g["d"], torch.bfloat16)
    ws = torch.empty(fa.decode_splitkv_workspace_size(g["B"], g["Hq"], 1, g["d"], splits),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def call():
        fa.decode_splitkv_gqa(q, k, v, num_splits=g["num_splits"], workspace=ws, out=o, lse=lse)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i].record(stream)
        call()
    ev[args.steps].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    avg_s = sum(ms) / len(ms) / 1e3
    e = 2
    nbytes = (g["B"] * g["Hkv"] * 2 * g["Nk"] * g["d"] * e
              + g["B"] * g["Hq"] * (2 * g["d"] * e + 4))
    gbs = nbytes / avg_s / 1e9
    print(json.dumps({
        "metric": "GQA split-KV decode HBM GB/s", "value": round(gbs, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded torch Philox draws on the GPU)",
        "config": {"workload": GQA_WORKLOAD, **{k2: v2 for k2, v2 in g.items()
                                                if not k2.startswith("seed")},
                   "splits_used": splits},
        "roofline": {"kernel": "decode_segment_mfma_kernel<bf16,128> + decode_merge_kernel",
                     "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "avg_launch_us": round(avg_s * 1e6, 2), "min_launch_us": round(min(ms) * 1e3, 2),
                     "algorithmic_bytes_per_launch": nbytes},
    }))
    return 0


SPLIT_CANDIDATES = (1, 2, 4, 8, 16, 32, 64, 128, 256)
SWEEP_FILE = os.path.join(ROOT, "profiles", "decode_split_sweep.txt")


def sweep_shapes():
    """Decode shapes (B, Hq, Hkv, N, Nk, d) of the split-count sweep: plain and
    grouped heads, one and several queries, short to long contexts; K and V
    stay under 4 GiB each."""
    out = []
    for B, Hq, Hkv in [(1, 8, 8), (1, 32, 32), (4, 32, 32), (16, 32, 32), (64, 32, 32),
                       (1, 32, 8), (8, 32, 8), (32, 32, 8), (1, 64, 8), (16, 64, 8), (4, 8, 1)]:
        for Nk in (1024, 4096, 16384, 65536, 262144):
            for N in (1, 4):
                if N == 4 and Hq != Hkv:
                    continue
                if B * Hkv * Nk * 128 * 2 > (4 << 30):
                    continue
                out.append((B, Hq, Hkv, N, Nk, 128))
    return out


def split_sweep(args, torch, fa) -> int:
    """Time decode at every candidate split count for each sweep shape (HIP
    events, median of args.steps launches after args.warmup) and write the
    table that the automatic split rule is checked against."""
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(7)
    big = torch.randn(1 << 31, generator=gen, device=dev, dtype=torch.bfloat16)   # 4 GiB
    bigv = torch.randn(1 << 31, generator=gen, device=dev, dtype=torch.bfloat16)
    ws = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    lines = ["# decode time (us, HIP events, median of %d launches after %d warm-up) per split "
             "count, bf16, d = 128, non-causal; 'auto' is the split count "
             "fa_decode_splitkv_auto_splits picks and its time relative to the best" % (
                 args.steps, args.warmup),
             "# command: python bench.py --split-sweep --steps %d --warmup %d" % (
                 args.steps, args.warmup),
             "# B Hq Hkv N Nk | " + " ".join(f"S={c}" for c in SPLIT_CANDIDATES) +
             " | best | auto (x best)"]
    for (B, Hq, Hkv, N, Nk, d) in sweep_shapes():
        q = torch.randn(B, Hq, N, d, generator=gen, device=dev).to(torch.bfloat16)
        k = big[:B * Hkv * Nk * d].view(B, Hkv, Nk, d)
        v = bigv[:B * Hkv * Nk * d].view(B, Hkv, Nk, d)
        o = torch.empty(B, Hq, N, d, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(B, Hq, N, dtype=torch.float32, device=dev)
        times = {}
        for S in SPLIT_CANDIDATES:
            if S > 1 and (S - 1) * 64 >= Nk:
                continue
            if fa.decode_splitkv_workspace_size(B, Hq, N, d, S) > ws.numel():
                continue

            def call():
                fa.decode_splitkv_gqa(q, k, v, num_splits=S, workspace=ws, out=o, lse=lse)
            for _ in range(args.warmup):
                call()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
            for i in range(args.steps):
                ev[i].record(stream)
                call()
            ev[args.steps].record(stream)
            torch.cuda.synchronize()
            ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
            times[S] = ms[len(ms) // 2] * 1e3
        best = min(times, key=times.get)
        auto = fa.decode_splitkv_auto_splits(B, Hq, Hkv, N, Nk, d, d, q.dtype)
        cells = " ".join(f"{times[c]:.1f}" if c in times else "-" for c in SPLIT_CANDIDATES)
        rel = times[auto] / times[best] if auto in times else float("nan")
        line = f"{B} {Hq} {Hkv} {N} {Nk} | {cells} | {best} | {auto} ({rel:.3f})"
        lines.append(line)
        print(line, flush=True)
    os.makedirs(os.path.dirname(SWEEP_FILE), exist_ok=True)
    with open(SWEEP_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    return 0


def bench_bwd(args, torch, fa, si, dev) -> int:
    """Backward (fa_bwd) at the B64 x H16 x 1024 causal prefill size: one step
    is one fa_bwd call (row dots, dK/dV kernel, dQ kernel) on the forward's o
    and lse.  Credited FLOPs are 2.5 times the forward's (five matrix
    products per tile instead of two; the lecture's count), causal-halved."""
    w = si.WORKLOADS[PREFILL]
    s = w.shapes[0]
    q, k, v = si.device_qkv(s, w.seed, w.dtype, dev, w.std)
    dout, _, _ = si.device_qkv(si.Shape(s.B, s.H, s.N, 1, s.dv, s.dv), w.seed + 100, w.dtype,
                               dev, 1.0)
    scale = 1.0 / math.sqrt(s.d)
    o, lse = fa.fwd(q, k, v, causal=True, scale=scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.bwd_workspace_size(s.B, s.H, s.N), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def call():
        fa.bwd(q, k, v, o, lse, dout, causal=True, scale=scale, workspace=ws, dq=dq, dk=dk, dv=dv)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i].record(stream)
        call()
    ev[args.steps].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    avg_s = sum(ms) / len(ms) / 1e3
    flop = 2.5 * 4.0 * s.N * s.Nk * s.d * s.B * s.H / 2
    tf = flop / avg_s / 1e12
    print(json.dumps({
        "metric": "attn bwd TFLOP/s (% bf16 MFMA peak)", "value": round(tf, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded torch Philox draws on the GPU)",
        "config": {"workload": PREFILL + " (fa_bwd)", "B": s.B, "H": s.H, "N": s.N, "Nk": s.Nk,
                   "d": s.d, "causal": True},
        "roofline": {"kernel": "bwd_dq_mfma32_kernel + bwd_dkdv_mfma32_kernel",
                     "bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "avg_launch_us": round(avg_s * 1e6, 2), "min_launch_us": round(min(ms) * 1e3, 2),
                     "credited_flop_per_launch": flop},
    }))
    return 0


def _time_call(torch, call, steps, warmup, stream):
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    for i in range(steps):
        ev[i].record(stream)
        call()
    ev[steps].record(stream)
    torch.cuda.synchronize()
    ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    return ms[len(ms) // 2] * 1e-3   # median seconds


def bench_dims(args, torch, fa, si, dev) -> int:
    """Head dimensions outside d = dv in {64, 128}: causal bf16 prefill
    (B16 x H16 x 2048), decode (B8 x H32 x 32768, 64 splits) and backward
    (B16 or B8 x H16 x 2048) for several (d, dv), next to d = dv = 128.  One
    JSON line with a case list; TFLOP/s credited as 2 N Nk (d + dv) per head,
    halved for causal (2.5 times that for the backward); decode GB/s over K,
    V once plus q, o, lse."""
    stream = torch.cuda.current_stream(dev)
    cases = []
    for d, dv in [(128, 128), (64, 128), (128, 64), (256, 256)]:
        B, H, N = 16, 16, 2048
        q, k, v = si.device_qkv(si.Shape(B, H, N, N, d, dv), 11, "bf16", dev, 1.0)
        sc = 1.0 / math.sqrt(d)
        t = _time_call(torch, lambda: fa.fwd(q, k, v, causal=True, scale=sc), args.steps,
                       args.warmup, stream)
        flop = 2.0 * N * N * (d + dv) * B * H / 2
        cases.append({"entry": "fa_fwd", "B": B, "H": H, "N": N, "d": d, "dv": dv,
                      "causal": True, "us": round(t * 1e6, 1),
                      "tflops": round(flop / t / 1e12, 1),
                      "frac_bf16_peak": round(flop / t / 1e12 / PEAK_BF16_TFLOPS, 4)})
        del q, k, v
    for d, dv in [(128, 128), (64, 128), (256, 256)]:
        B, H, Nk, S = 8, 32, 32768, 64
        q, k, v = si.device_qkv(si.Shape(B, H, 1, Nk, d, dv), 12, "bf16", dev, 1.0)
        ws = torch.empty(fa.decode_splitkv_workspace_size(B, H, 1, dv, S), dtype=torch.uint8,
                         device=dev)
        t = _time_call(torch, lambda: fa.decode_splitkv(q, k, v, num_splits=S, workspace=ws),
                       args.steps, args.warmup, stream)
        nbytes = B * H * (Nk * (d + dv) * 2 + d * 2 + dv * 2 + 4)
        cases.append({"entry": "fa_decode_splitkv", "B": B, "H": H, "Nk": Nk, "d": d, "dv": dv,
                      "splits": S, "us": round(t * 1e6, 1), "gbs": round(nbytes / t / 1e9, 1),
                      "frac_hbm_peak": round(nbytes / t / 1e9 / PEAK_HBM_GBS, 4)})
        del q, k, v
    # grouped-query decode, 4 query heads per key/value head, with 64 splits
    # and with the automatic split count (num_splits = 0)
    for (d, dv), S0 in itertools.product([(128, 128), (64, 64), (32, 32), (64, 128), (128, 64),
                                          (256, 256)],
                                         (64, 0)):
        B, Hq, Hkv, Nk = 8, 32, 8, 32768
        S = S0 if S0 > 0 else fa.decode_splitkv_auto_splits(B, Hq, Hkv, 1, Nk, d, dv, torch.bfloat16)
        q, _, _ = si.device_qkv(si.Shape(B, Hq, 1, 1, d, dv), 15, "bf16", dev, 1.0)
        _, k, v = si.device_qkv(si.Shape(B, Hkv, 1, Nk, d, dv), 16, "bf16", dev, 1.0)
        ws = torch.empty(fa.decode_splitkv_workspace_size(B, Hq, 1, dv, S), dtype=torch.uint8,
                         device=dev)
        t = _time_call(torch, lambda: fa.decode_splitkv_gqa(q, k, v, num_splits=S0, workspace=ws),
                       args.steps, args.warmup, stream)
        nbytes = B * Hkv * Nk * (d + dv) * 2 + B * Hq * ((d + dv) * 2 + 4)
        cases.append({"entry": "fa_decode_splitkv_gqa", "B": B, "Hq": Hq, "Hkv": Hkv, "Nk": Nk,
                      "d": d, "dv": dv, "splits": S if S0 > 0 else f"auto ({S})",
                      "us": round(t * 1e6, 1),
                      "gbs": round(nbytes / t / 1e9, 1),
                      "frac_hbm_peak": round(nbytes / t / 1e9 / PEAK_HBM_GBS, 4)})
        del q, k, v
    for (B, H, N, d, dv) in [(16, 16, 2048, 128, 128), (16, 16, 2048, 64, 128),
                             (8, 16, 2048, 256, 256), (8, 16, 2048, 32, 32)]:
        q, k, v = si.device_qkv(si.Shape(B, H, N, N, d, dv), 13, "bf16", dev, 0.5)
        dout, _, _ = si.device_qkv(si.Shape(B, H, N, 1, dv, dv), 14, "bf16", dev, 1.0)
        sc = 1.0 / math.sqrt(d)
        o, lse = fa.fwd(q, k, v, causal=True, scale=sc)
        ws = torch.empty(fa.bwd_workspace_size(B, H, N), dtype=torch.uint8, device=dev)
        dq, dk, dvv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        t = _time_call(torch, lambda: fa.bwd(q, k, v, o, lse, dout, causal=True, scale=sc,
                                             workspace=ws, dq=dq, dk=dk, dv=dvv),
                       args.steps, args.warmup, stream)
        flop = 2.5 * 2.0 * N * N * (d + dv) * B * H / 2
        cases.append({"entry": "fa_bwd", "B": B, "H": H, "N": N, "d": d, "dv": dv,
                      "causal": True, "us": round(t * 1e6, 1),
                      "tflops": round(flop / t / 1e12, 1),
                      "frac_bf16_peak": round(flop / t / 1e12 / PEAK_BF16_TFLOPS, 4)})
        del q, k, v, dout, o, lse, dq, dk, dvv
    print(json.dumps({"metric": "head-dimension coverage (median of HIP-event timings)",
                      "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "dtype": "bf16",
                      "data": "synthetic (seeded torch Philox draws on the GPU)",
                      "cases": cases}))
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=256,
                    help="prefill heads the CPU oracle is timed on")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="add one plain 1 GiB device copy per step (for counter calibration)")
    ap.add_argument("--only", choices=["prefill", "decode", "long", "gqa", "bwd", "dims"],
                    help="profile one entry point alone (the JSON line then omits the other); "
                         "'gqa' times the grouped-query decode, 'bwd' the backward, 'dims' "
                         "other head dimensions (none of these is part of the default line)")
    ap.add_argument("--split-sweep", action="store_true",
                    help="time decode at every candidate split count over a set of shapes "
                         "and write the table under profiles/")
    ap.add_argument("--summarize-pmc", metavar="DIR")
    ap.add_argument("--summarize-trace", metavar="DIR")
    args = ap.parse_args()

    if args.summarize_pmc or args.summarize_trace:
        if args.summarize_pmc:
            summarize_pmc(args.summarize_pmc)
        if args.summarize_trace:
            summarize_trace(args.summarize_trace)
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the attention path shards heads or key ranges with no collective on the hot "
              "path; this benchmark measures one GPU's share).", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    import torch

    import exact_tiled_attention_flashattention_amd as fa
    import synth_inputs as si

    fa.library()   # fail loudly here if the HIP library is missing
    dev = torch.device("cuda:0")
    if args.only == "gqa":
        return bench_gqa(args, torch, fa, si, dev)
    if args.only == "bwd":
        return bench_bwd(args, torch, fa, si, dev)
    if args.only == "dims":
        return bench_dims(args, torch, fa, si, dev)
    if args.split_sweep:
        return split_sweep(args, torch, fa)
    wp = si.WORKLOADS[PREFILL]
    wd = si.WORKLOADS[DECODE]
    wl = si.WORKLOADS[LONG]
    sp, sd, sl = wp.shapes[0], wd.shapes[0], wl.shapes[0]
    print(f"# drawing inputs: {wp.description}; {wd.description}; {wl.description}",
          file=sys.stderr, flush=True)
    run_p = args.only in (None, "prefill")
    run_d = args.only in (None, "decode")
    run_l = args.only in (None, "long")
    if not run_p:
        sp = si.Shape(1, 1, 1, 1, sp.d, sp.dv)
    if not run_d:
        sd = si.Shape(1, 1, 1, 1, sd.d, sd.dv)
    if not run_l:
        sl = si.Shape(1, 1, 1, 1, sl.d, sl.dv)
    qp, kp, vp = si.device_qkv(sp, wp.seed, wp.dtype, dev, wp.std)
    qd, kd, vd = si.device_qkv(sd, wd.seed, wd.dtype, dev, wd.std)
    ql, kl, vl = si.device_qkv(sl, wl.seed, wl.dtype, dev, wl.std)
    op = torch.empty((sp.B, sp.H, sp.N, sp.dv), dtype=qp.dtype, device=dev)
    lp = torch.empty((sp.B, sp.H, sp.N), dtype=torch.float32, device=dev)
    ol = torch.empty((sl.B, sl.H, sl.N, sl.dv), dtype=ql.dtype, device=dev)
    ll = torch.empty((sl.B, sl.H, sl.N), dtype=torch.float32, device=dev)
    od = torch.empty((sd.B, sd.H, sd.N, sd.dv), dtype=qd.dtype, device=dev)
    ld = torch.empty((sd.B, sd.H, sd.N), dtype=torch.float32, device=dev)
    ws = torch.empty(fa.decode_splitkv_workspace_size(sd.B, sd.H, sd.N, sd.dv, wd.num_splits),
                     dtype=torch.uint8, device=dev)
    copy_src = copy_dst = None
    if args.calibration_copy:
        copy_src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        copy_dst = torch.empty_like(copy_src)
    stream = torch.cuda.current_stream(dev)
    scale_p = 1.0 / math.sqrt(sp.d)
    scale_d = 1.0 / math.sqrt(sd.d)
    scale_l = 1.0 / math.sqrt(sl.d)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        if run_p:
            fa.fwd(qp, kp, vp, causal=True, scale=scale_p, out=op, lse=lp)
        if ev is not None:
            ev[1].record(stream)
        if run_d:
            fa.decode_splitkv(qd, kd, vd, causal=False, scale=scale_d, num_splits=wd.num_splits,
                              workspace=ws, out=od, lse=ld)
        if ev is not None:
            ev[2].record(stream)
        if run_l:
            fa.fwd(ql, kl, vl, causal=True, scale=scale_l, out=ol, lse=ll)
        if ev is not None:
            ev[3].record(stream)
        if copy_src is not None:
            copy_dst.copy_(copy_src)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    sclk_paths = sclk_files()
    sclk = []
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
        if i % 4 == 3:
            sclk += read_sclk(sclk_paths)   # while the queued steps run
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = [e[0].elapsed_time(e[1]) for e in events]
    dec_ms = [e[1].elapsed_time(e[2]) for e in events]
    long_ms = [e[2].elapsed_time(e[3]) for e in events]
    assert torch.isfinite(lp).all().item() and torch.isfinite(ld).all().item()
    assert torch.isfinite(ll).all().item()
    clock = ({"sclk_mhz_during_timed_steps": sclk, "source": "sysfs pp_dpm_sclk (level "
              "marked current), read by the host while the queued timed steps ran"}
             if sclk else None)

    flops = credited_flops(sp, True)
    fwd_avg_s = sum(fwd_ms) / len(fwd_ms) / 1e3
    dec_avg_s = sum(dec_ms) / len(dec_ms) / 1e3
    tflops = flops / fwd_avg_s / 1e12
    dbytes = decode_bytes(sd)
    dec_gbs = dbytes / dec_avg_s / 1e9
    traffic = read_traffic()
    lflops = credited_flops(sl, True)
    long_avg_s = sum(long_ms) / len(long_ms) / 1e3
    ltflops = lflops / long_avg_s / 1e12

    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded torch Philox draws on the GPU)",
        "config": {
            "workload": f"{PREFILL} (fa_fwd) + {DECODE} (fa_decode_splitkv)",
            "prefill": {"B": sp.B, "H": sp.H, "N": sp.N, "Nk": sp.Nk, "d": sp.d, "causal": True,
                        "input_std": wp.std},
            "decode": {"B": sd.B, "H": sd.H, "N": sd.N, "Nk": sd.Nk, "d": sd.d,
                       "num_splits": wd.num_splits},
            "long_prefill": {"B": sl.B, "H": sl.H, "N": sl.N, "Nk": sl.Nk, "d": sl.d,
                             "causal": True, "input_std": wl.std},
        },
        "gpu_clock": clock,
        "roofline": {
            "kernel": "fwd_mfma32_kernel<bf16,64,64,causal>",
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic["fwd"],
            "avg_launch_us": round(fwd_avg_s * 1e6, 2),
            "median_launch_us": round(sorted(fwd_ms)[len(fwd_ms) // 2] * 1e3, 2),
            "min_launch_us": round(min(fwd_ms) * 1e3, 2),
            "credited_flop_per_launch": flops,
        },
        "decode": {
            "metric": "split-KV decode HBM GB/s",
            "value": round(dec_gbs, 1),
            "unit": "GB/s",
            "roofline": {
                "kernel": "decode_segment_kernel<bf16,128,1> + decode_merge_kernel",
                "bound": "hbm",
                "achieved": round(dec_gbs, 1),
                "peak": PEAK_HBM_GBS,
                "unit": "GB/s",
                "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
                "traffic": traffic["decode"],
                "avg_launch_us": round(dec_avg_s * 1e6, 2),
                "median_launch_us": round(sorted(dec_ms)[len(dec_ms) // 2] * 1e3, 2),
                "min_launch_us": round(min(dec_ms) * 1e3, 2),
                "algorithmic_bytes_per_launch": dbytes,
            },
        },
        "long_prefill": {
            "metric": "attn fwd TFLOP/s (% bf16 MFMA peak), long causal prefill",
            "workload": f"{LONG} (fa_fwd)",
            "value": round(ltflops, 2),
            "unit": "TFLOP/s",
            "roofline": {
                "kernel": "fwd_mfma32_kernel<bf16,128,128,causal>",
                "bound": "mfma",
                "achieved": round(ltflops, 2),
                "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s",
                "frac": round(ltflops / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic["long"],
                "avg_launch_us": round(long_avg_s * 1e6, 2),
                "median_launch_us": round(sorted(long_ms)[len(long_ms) // 2] * 1e3, 2),
                "min_launch_us": round(min(long_ms) * 1e3, 2),
                "credited_flop_per_launch": lflops,
            },
        },
        "cpu_baseline": None,
    }
    if not run_p:
        result["value"] = None
        result["roofline"] = None
    if not run_d:
        result["decode"] = None
    if not run_l:
        result["long_prefill"] = None
    if not args.no_cpu_baseline and run_p:
        result["cpu_baseline"] = cpu_baseline(qp, kp, vp, sp, True, min(args.cpu_heads, sp.B * sp.H))
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
