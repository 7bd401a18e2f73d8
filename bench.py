"""Benchmark of the GDN-2 chunked prefill forward on one MI355X.

One step = one call of the fused forward (the whole hot path: decay cumsum,
decay-scaled K K^T with the erase gate, triangular inverse, w/u recompute,
sequential float32 state pass with intra + inter output, final state) over
one packed batch resident in HBM. The default workload is the H32/D128
varlen prefill: 8 sequences with lengths uniform in [256, 8192] (seed 2),
H = HV = 32, K = V = 128, bf16 inputs, float32 log-decay and state.

Prints ONE JSON line with the throughput (tokens/s), the HBM roofline of the
kernel (algorithmic bytes per launch / mean launch time from HIP events on
the launch stream) and the FP64 oracle timed on the host as a CPU baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload ID]
       python bench.py --mode bwd [--workload ID]   (the backward, its own JSON line)
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
METRIC = "GDN-2 chunk prefill tokens/s (H32 D128 bf16); % of MFMA/HBM roofline"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_varlen_h32_d128.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


FWD_KERNEL_SOURCES = ("gdn2_device.h", "gdn2_fwd.hip", "gdn2_internal.h")


def kernel_source_hash() -> str:
    """sha256 (first 16 hex) over the sources the forward kernel is built from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_attention_rnn_gdn2_amd", "csrc")
    for name in FWD_KERNEL_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(T, N, H, HV, K, V, has_init: bool, has_final: bool) -> int:
    """Bytes that must cross HBM once: q, k (bf16, per q/k head), v, w, out
    (bf16, per value head), beta (bf16) and g (float32) per value head and
    key channel, the initial state read and the final state written."""
    per_token = 2 * K * H * 2 + HV * (3 * 2 * V + 2 * K + 4 * K)
    state = N * HV * K * V * 4
    return T * per_token + (state if has_init else 0) + (state if has_final else 0)


def measured_traffic(src_hash: str, launches_per_profile: int = 1):
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    only if it was taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != src_hash:
        return None
    return rec.get("hbm_bytes_per_launch")


PROFILE_STEPS = {
    # name: (rocprofv3 options, bench.py options)
    "kt": ("--kernel-trace --stats", "--steps 10 --warmup 2 --no-cpu-baseline --no-peaks"),
    "pmc_fetch": ("--pmc FETCH_SIZE", "--steps 2 --warmup 1 --no-cpu-baseline --no-peaks"),
    "pmc_write": ("--pmc WRITE_SIZE", "--steps 2 --warmup 1 --no-cpu-baseline --no-peaks"),
    "cal_fetch": ("--pmc FETCH_SIZE", "--copy-probe-mib 1024"),
    "cal_write": ("--pmc WRITE_SIZE", "--copy-probe-mib 1024"),
    "bkt": ("--kernel-trace --stats", "--mode bwd --steps 5 --warmup 1"),
    "bpmc_fetch": ("--pmc FETCH_SIZE", "--mode bwd --steps 2 --warmup 1 --no-cpu-baseline --no-peaks"),
    "bpmc_write": ("--pmc WRITE_SIZE", "--mode bwd --steps 2 --warmup 1 --no-cpu-baseline --no-peaks"),
}
KERNEL_TAG = "chunk_fwd_kernel"


PROFILE_DIR = "profile_out"  # where the profile runs write their CSVs (git-ignored)


def profile_command(name: str) -> str:
    opts, bench_opts = PROFILE_STEPS[name]
    return (f"rocprofv3 {opts} -f csv -d {PROFILE_DIR}/{name} -o {name} -- "
            f"python -u bench.py {bench_opts}")


def _short(name: str, n: int = 110) -> str:
    return name if len(name) <= n else name[:n] + "..."


def _csv_rows(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _find(dirpath, suffix):
    for root, _, files in os.walk(dirpath):
        for fn in files:
            if fn.endswith(suffix):
                return os.path.join(root, fn)
    raise FileNotFoundError(f"no *{suffix} under {dirpath}")


def summarize_profiles(outdir: str, tag: str, dest: str | None = None):
    """Turn the rocprofv3 CSVs of the PROFILE_STEPS runs under ``outdir`` into
    the committed text summaries: the kernel-trace statistics, and the HBM
    bytes per launch of the forward kernel from FETCH_SIZE / WRITE_SIZE
    (KiB per dispatch), each scaled by the same counter's reading for a plain
    device copy of 1 GiB (so that bytes per KiB-unit are calibrated, not
    assumed). The summaries go to ``dest`` (default: profiles/)."""
    dest = dest or os.path.join(ROOT, "profiles")
    traffic_file = os.path.join(dest, os.path.basename(TRAFFIC_FILE))
    src_hash = kernel_source_hash()
    stats = _csv_rows(_find(os.path.join(outdir, "kt"), "_kernel_stats.csv"))
    lines = [f"# rocprofv3 kernel-trace statistics: GDN-2 forward, {tag}", "",
             f"kernel source hash (sha256 over csrc/{', '.join(FWD_KERNEL_SOURCES)}, first 16 hex): {src_hash}",
             "command (from the repository root):", "  " + profile_command("kt"), "",
             f"{'calls':>6} {'avg us':>10} {'min us':>10} {'max us':>10} {'share %':>8}  kernel"]
    for r in stats:
        lines.append(f"{int(r['Calls']):>6} {float(r['AverageNs'])/1e3:>10.1f} {float(r['MinNs'])/1e3:>10.1f} "
                     f"{float(r['MaxNs'])/1e3:>10.1f} {float(r['Percentage']):>8.2f}  {_short(r['Name'])}")

    def counter(name, want_kernel, value_min=0.0):
        rows = _csv_rows(_find(os.path.join(outdir, name), "_counter_collection.csv"))
        vals = [float(r["Counter_Value"]) for r in rows if want_kernel(r["Kernel_Name"])
                and float(r["Counter_Value"]) >= value_min]
        if not vals:
            raise ValueError(f"{name}: no matching dispatch")
        return vals

    fwd = lambda n: KERNEL_TAG in n
    copy = lambda n: "copyBuffer" in n
    copy_bytes = 1024 * (1 << 20)
    cal_f = max(counter("cal_fetch", copy))
    cal_w = max(counter("cal_write", copy))
    fetch_scale = copy_bytes / (cal_f * 1024)  # bytes per counted byte
    write_scale = copy_bytes / (cal_w * 1024)
    kf = counter("pmc_fetch", fwd)
    kw = counter("pmc_write", fwd)
    fetch = sum(kf) / len(kf) * 1024 * fetch_scale
    write = sum(kw) / len(kw) * 1024 * write_scale
    lines += ["", "## HBM traffic per launch (rocprofv3 --pmc, one counter per run)", "",
              "commands:", "  " + profile_command("pmc_fetch"), "  " + profile_command("pmc_write"),
              "  " + profile_command("cal_fetch"), "  " + profile_command("cal_write"), "",
              f"copy calibration: 1 GiB device copy reads FETCH_SIZE {cal_f:.1f} KiB, WRITE_SIZE {cal_w:.1f} KiB",
              f"  -> scale factors: fetch x{fetch_scale:.3f}, write x{write_scale:.3f}",
              f"forward kernel: FETCH_SIZE {sum(kf)/len(kf):.1f} KiB/dispatch ({len(kf)} dispatches), "
              f"WRITE_SIZE {sum(kw)/len(kw):.1f} KiB/dispatch ({len(kw)} dispatches)",
              f"  -> HBM read {fetch/1e6:.2f} MB, write {write/1e6:.2f} MB, total {(fetch+write)/1e6:.2f} MB per launch"]
    txt = os.path.join(dest, f"{KERNEL_TAG}_{tag}.txt")
    with open(txt, "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(traffic_file, "w") as f:
        json.dump({"kernel_source_hash": src_hash, "hbm_bytes_per_launch": fetch + write,
                   "hbm_read_bytes": fetch, "hbm_write_bytes": write,
                   "fetch_scale": fetch_scale, "write_scale": write_scale,
                   "commands": [profile_command(n) for n in ("pmc_fetch", "pmc_write", "cal_fetch", "cal_write")]},
                  f, indent=1)
        f.write("\n")
    log("\n".join(lines))
    bdir = os.path.join(outdir, "bkt")
    if os.path.isdir(bdir):
        rows = _csv_rows(_find(bdir, "_kernel_stats.csv"))
        bl = [f"# rocprofv3 kernel-trace statistics: GDN-2 backward (gdn2_chunk_bwd), {tag}", "",
              "command (from the repository root):", "  " + profile_command("bkt"), "",
              f"{'calls':>6} {'avg us':>10} {'min us':>10} {'max us':>10} {'share %':>8}  kernel"]
        for r in rows:
            bl.append(f"{int(r['Calls']):>6} {float(r['AverageNs'])/1e3:>10.1f} {float(r['MinNs'])/1e3:>10.1f} "
                      f"{float(r['MaxNs'])/1e3:>10.1f} {float(r['Percentage']):>8.2f}  {_short(r['Name'])}")
        if os.path.isdir(os.path.join(outdir, "bpmc_fetch")) and os.path.isdir(os.path.join(outdir, "bpmc_write")):
            bl += ["", "## HBM traffic per launch of each backward kernel (rocprofv3 --pmc, one counter per run)", "",
                   f"scaled by the 1 GiB copy calibration of the forward's runs: fetch x{fetch_scale:.3f}, "
                   f"write x{write_scale:.3f}", "",
                   "commands:", "  " + profile_command("bpmc_fetch"), "  " + profile_command("bpmc_write"), "",
                   f"{'read MB':>10} {'write MB':>10}  kernel"]
            ours = lambda n: "gdn2::" in n
            per = {}
            for name, key, scale in (("bpmc_fetch", 0, fetch_scale), ("bpmc_write", 1, write_scale)):
                rows = _csv_rows(_find(os.path.join(outdir, name), "_counter_collection.csv"))
                for r in rows:
                    if ours(r["Kernel_Name"]):
                        per.setdefault(r["Kernel_Name"], ([], []))[key].append(
                            float(r["Counter_Value"]) * 1024 * scale)
            total = 0.0
            for kname, (fv, wv) in sorted(per.items()):
                rd = sum(fv) / len(fv) if fv else 0.0
                wr = sum(wv) / len(wv) if wv else 0.0
                total += rd + wr
                bl.append(f"{rd/1e6:>10.1f} {wr/1e6:>10.1f}  {_short(kname)}")
            bl.append(f"sum over the kernels of one call: {total/1e6:.1f} MB")
        with open(os.path.join(dest, f"bwd_kernels_{tag}.txt"), "w") as f:
            f.write("\n".join(bl) + "\n")
        log("\n".join(bl))


BWD_METRIC = "GDN-2 chunk backward tokens/s (H32 D128 bf16); % of HBM roofline"


def bwd_algorithmic_bytes(T, N, H, HV, K, V, has_init: bool, has_final: bool) -> int:
    """Bytes the backward must move once: q, k, dq, dk (bf16, per q/k head),
    v, w, d_out, dv, dw (bf16), beta, dbeta (bf16) and g, dg (float32) per
    value head, the initial state and its gradient, the final state's
    gradient."""
    per_token = 4 * K * H * 2 + HV * (5 * 2 * V + 2 * 2 * K + 2 * 4 * K)
    state = N * HV * K * V * 4
    return T * per_token + (2 * state if has_init else state) + (state if has_final else 0)


def bwd_mfma_flop(T, N, HV, K) -> int:
    """Dense MFMA work of the backward's products per (64-token chunk, value
    head) at K = V = D, counted as issued (the forward recompute, which also
    writes each chunk's record, the state-gradient pass, and the gradient
    pass's products), times the chunk count (an upper bound of ceil(T / 64) +
    N chunks per head)."""
    D = K
    mm = lambda m, n, k: 2 * m * n * k
    fwd = 64 * (2 * (32 * (3 * D + 2 * D) + 3 * D * D))
    state = mm(64, D, 64) + 3 * mm(64, D, D)
    grads = (mm(64, D, 64) + mm(64, D, D) + mm(64, D, 64) + mm(64, D, D) + 2 * mm(64, D, D)
             + mm(64, D, D) + 10 * mm(16, 16, D) + 2 * mm(64, 64, D) + 2 * mm(64, D, 64)
             + 2 * mm(64, 64, 64) + 4 * mm(64, D, 64))
    return (T // 64 + N) * HV * (fwd + state + grads)


def measured_peaks(dev):
    """Context for the spec peaks, measured on this device after the timed
    region: a 1 GiB device-to-device copy (read + write bytes per second)
    and a 8192^3 bf16 GEMM through torch (the vendor library)."""
    import torch
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    a = torch.randn((8192, 8192), dtype=torch.bfloat16, device=dev)
    b = torch.randn((8192, 8192), dtype=torch.bfloat16, device=dev)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / reps

    t_copy = timed(lambda: dst.copy_(src), 5)
    t_mm = timed(lambda: torch.mm(a, b), 5)
    out = {"copy_GBps": 2 * n * 4 / t_copy / 1e9, "bf16_gemm_TFLOPs": 2 * 8192 ** 3 / t_mm / 1e12,
           "note": "measured on this device: 1 GiB copy (read + write), 8192^3 bf16 torch.mm"}
    del src, dst, a, b
    torch.cuda.empty_cache()
    return out


def bench_bwd(args, d, gdn2, dev):
    """Time gdn2.chunk_bwd (all of its launches, workspace included) over the
    workload and print one JSON line."""
    import torch
    from linear_attention_rnn_gdn2_amd.workloads import synth_cotangents
    wl = d["workload"]
    T, N = int(d["cu_seqlens"][-1]), len(d["lengths"])
    d_out, dht = synth_cotangents(T, N, wl.HV, wl.K, wl.V, args.workload)
    g = {n: d[n].to(dev) for n in ("q", "k", "v", "g", "beta", "w")}
    s0 = None if d["initial_state"] is None else d["initial_state"].to(dev)
    cu, do, dh = d["cu_seqlens"].to(dev), d_out.to(dev), dht.to(dev)
    grads = gdn2.chunk_bwd(g["q"], g["k"], g["v"], g["g"], g["beta"], g["w"], do, scale=d["scale"],
                           initial_state=s0, cu_seqlens=cu, d_final_state=dh)

    def step():
        gdn2.chunk_bwd(g["q"], g["k"], g["v"], g["g"], g["beta"], g["w"], do, scale=d["scale"],
                       initial_state=s0, cu_seqlens=cu, d_final_state=dh, grads=grads)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean_s = sum(a.elapsed_time(b) for a, b in ev) / len(ev) / 1e3
    algo = bwd_algorithmic_bytes(T, N, wl.H, wl.HV, wl.K, wl.V, s0 is not None, True)
    flop = bwd_mfma_flop(T, N, wl.HV, wl.K)
    achieved = algo / mean_s / 1e9
    rec = {"metric": BWD_METRIC, "value": T / (wall / args.steps), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall / args.steps * 1e3,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": f"{wl.name} backward: {N} sequences, {T} tokens, H={wl.H} HV={wl.HV} "
                                  f"K={wl.K} V={wl.V}, chunk 64, seed {args.workload}",
                      "global_batch": N, "seq_len": T, "parallelism": "single GPU"},
           "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": achieved / HBM_PEAK_GBS, "traffic": None, "algorithmic_bytes_per_call": algo,
                        "mean_call_ms": mean_s * 1e3, "mfma_tflops": flop / mean_s / 1e12,
                        "mfma_frac_of_2500": flop / mean_s / 2.5e15}}
    log(f"backward: mean call {mean_s*1e3:.3f} ms, {T / mean_s / 1e6:.2f} M tokens/s, {achieved:.0f} GB/s "
        f"algorithmic ({achieved / HBM_PEAK_GBS * 100:.1f}% of HBM peak), {flop / mean_s / 1e12:.1f} TFLOP/s MFMA")
    if not args.no_cpu_baseline:
        log("timing the FP64 backward oracle on the host")
        rec["cpu_baseline"] = cpu_baseline_bwd(d, wl, d_out, dht)
    print(json.dumps(rec), flush=True)


def cpu_baseline_bwd(d, workload, d_out, dht, min_seconds: float = 10.0):
    """The FP64 backward oracle on the host: whole passes over the same
    workload and incoming gradients, repeated until about ``min_seconds`` of
    wall time (at least one)."""
    from oracle.c_oracle import gdn2_recurrence_bwd_c, max_threads
    names = ("q", "k", "v", "g", "beta", "w")
    T = int(d["cu_seqlens"][-1])
    passes, t0 = 0, time.perf_counter()
    while True:
        gdn2_recurrence_bwd_c(*[d[n] for n in names], d["scale"], d["initial_state"], d["cu_seqlens"], d_out, dht)
        passes += 1
        wall = time.perf_counter() - t0
        if wall >= min_seconds:
            break
    return {"value": passes * T / wall, "unit": "tokens/s", "cores": max_threads(), "kind": "oracle",
            "sample": f"{passes} whole passes over the {workload.name} workload ({len(d['lengths'])} sequences, "
                      f"{T} tokens x {workload.HV} value heads each) and its incoming gradients, plain-C FP64 "
                      f"token-by-token backward oracle (forward with block checkpoints, then the reverse sweep), "
                      f"OpenMP over (sequence, head), wall {wall:.2f} s"}


def cpu_baseline(d, workload, min_seconds: float = 10.0):
    """The FP64 oracle on the host: whole passes over the same workload,
    repeated until about ``min_seconds`` of wall time (at least one)."""
    from oracle.c_oracle import gdn2_recurrence_c, max_threads
    names = ("q", "k", "v", "g", "beta", "w")
    T = int(d["cu_seqlens"][-1])
    passes, t0 = 0, time.perf_counter()
    while True:
        gdn2_recurrence_c(*[d[n] for n in names], d["scale"], d["initial_state"], d["cu_seqlens"])
        passes += 1
        wall = time.perf_counter() - t0
        if wall >= min_seconds:
            break
    return {"value": passes * T / wall, "unit": "tokens/s", "cores": max_threads(), "kind": "oracle",
            "sample": f"{passes} whole passes over the {workload.name} workload ({len(d['lengths'])} sequences, "
                      f"{T} tokens x {workload.HV} value heads each), plain-C FP64 token-by-token oracle, "
                      f"OpenMP over (sequence, head), wall {wall:.2f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured copy / GEMM context")
    ap.add_argument("--mode", choices=("fwd", "bwd"), default="fwd",
                    help="fwd: the chunked prefill forward (the headline); bwd: its backward "
                         "(gradients of every input and of the initial state)")
    ap.add_argument("--summarize-profiles", metavar="DIR", default=None,
                    help="host only: write the committed profile summaries from the rocprofv3 CSVs "
                         "of the runs printed by --print-profile-commands, found under DIR")
    ap.add_argument("--print-profile-commands", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB, twice (calibrates "
                         "the FETCH_SIZE / WRITE_SIZE counters against known bytes)")
    args = ap.parse_args()
    if args.print_profile_commands:
        for n in PROFILE_STEPS:
            print(profile_command(n))
        return
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles, "varlen_h32_d128")
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build measures one GPU only (every chain of the GDN-2 "
              "prefill is independent; multi-GPU sharding is not implemented). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from linear_attention_rnn_gdn2_amd import gdn2
    from linear_attention_rnn_gdn2_amd.workloads import make_inputs

    dev = torch.device("cuda:0")
    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {args.copy_probe_mib} MiB twice")
        return
    gdn2.load_library()
    log(f"drawing workload {args.workload}")
    d = make_inputs(args.workload)
    if args.mode == "bwd":
        bench_bwd(args, d, gdn2, dev)
        return
    wl = d["workload"]
    T = int(d["cu_seqlens"][-1])
    N = len(d["lengths"])
    names = ("q", "k", "v", "g", "beta", "w")
    gpu = {n: d[n].to(dev) for n in names}
    s0 = None if d["initial_state"] is None else d["initial_state"].to(dev)
    cu = d["cu_seqlens"].to(dev)
    out = torch.empty((T, wl.HV, wl.V), dtype=torch.bfloat16, device=dev)
    fin = torch.empty((N, wl.HV, wl.K, wl.V), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step():
        gdn2.chunk_fwd(**gpu, scale=d["scale"], initial_state=s0, cu_seqlens=cu, out=out, final_state=fin)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [a.elapsed_time(b) for a, b in ev]
    mean_launch_s = sum(launch_ms) / len(launch_ms) / 1e3
    ms_per_step = wall / args.steps * 1e3
    value = T / (ms_per_step / 1e3)

    algo = algorithmic_bytes(T, N, wl.H, wl.HV, wl.K, wl.V, s0 is not None, True)
    achieved = algo / mean_launch_s / 1e9
    src_hash = kernel_source_hash()
    traffic = measured_traffic(src_hash)
    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: {N} sequences, {T} tokens (lengths {d['lengths']}), "
                               f"H={wl.H} HV={wl.HV} K={wl.K} V={wl.V}, chunk 64, seed {args.workload}",
                   "global_batch": N, "seq_len": T, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": algo, "mean_launch_ms": mean_launch_s * 1e3,
                     "kernel_source_hash": src_hash},
    }
    log(f"mean launch {mean_launch_s*1e3:.3f} ms, wall/step {ms_per_step:.3f} ms, "
        f"{value/1e6:.2f} M tokens/s, {achieved:.0f} GB/s algorithmic ({achieved/HBM_PEAK_GBS*100:.1f}% of HBM peak)")
    if not args.no_peaks:
        rec["measured_peaks"] = measured_peaks(dev)
        log(f"measured on this device: copy {rec['measured_peaks']['copy_GBps']:.0f} GB/s, "
            f"bf16 GEMM {rec['measured_peaks']['bf16_gemm_TFLOPs']:.0f} TFLOP/s")
    if not args.no_cpu_baseline:
        log("timing the FP64 oracle on the host")
        rec["cpu_baseline"] = cpu_baseline(d, wl)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
