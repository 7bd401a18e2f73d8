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


# SQ counter passes (each within one run's hardware limits: at most 8 SQ,
# 2 TA and 2 GRBM counters; the derived ones are rocprofv3's own formulas:
# MfmaUtil = MFMA busy cycles / (GPU cycles x SIMDs), VALUBusy = VALU active
# cycles / (CUs x GPU cycles), LDSBankConflict = bank-conflict stall cycles /
# (GPU cycles x CUs), LdsUtil = indexed-LDS active cycles / (GPU cycles x CUs))
SQ_PASSES = {
    "sq1": "MfmaUtil VALUBusy SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_VALU_TRANS_F32",
    "sq2": "LDSBankConflict LdsUtil SQ_INSTS_LDS SQ_WAIT_INST_LDS SQ_VALU_MFMA_COEXEC_CYCLES",
    "sq3": "SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY SQ_WAVES SQ_INSTS_VMEM_RD TA_BUSY_avr TA_ADDR_STALLED_BY_TC_CYCLES_sum",
}
_Q = "--no-cpu-baseline --no-peaks --no-extra"
PROFILE_STEPS = {
    # name: (rocprofv3 options, bench.py options)
    "kt": ("--kernel-trace --stats", f"--steps 20 --warmup 2 {_Q}"),
    "pmc_fetch": ("--pmc FETCH_SIZE", f"--steps 2 --warmup 1 {_Q}"),
    "pmc_write": ("--pmc WRITE_SIZE", f"--steps 2 --warmup 1 {_Q}"),
    "cal_fetch": ("--pmc FETCH_SIZE", "--copy-probe-mib 1024"),
    "cal_write": ("--pmc WRITE_SIZE", "--copy-probe-mib 1024"),
    **{n: (f"--pmc {c}", f"--steps 2 --warmup 1 {_Q}") for n, c in SQ_PASSES.items()},
    "kt4": ("--kernel-trace --stats", f"--workload 4 --steps 5 --warmup 1 {_Q}"),
    **{n + "_4": (f"--pmc {c}", f"--workload 4 --steps 1 --warmup 1 {_Q}") for n, c in SQ_PASSES.items()},
    "bkt": ("--kernel-trace --stats", "--mode bwd --steps 5 --warmup 1"),
    "bpmc_fetch": ("--pmc FETCH_SIZE", f"--mode bwd --steps 2 --warmup 1 {_Q}"),
    "bpmc_write": ("--pmc WRITE_SIZE", f"--mode bwd --steps 2 --warmup 1 {_Q}"),
    **{"b" + n: (f"--pmc {c}", f"--mode bwd --steps 2 --warmup 1 {_Q}") for n, c in SQ_PASSES.items()},
}
KERNEL_TAG = "chunk_fwd_kernel"
CU_NUM, SIMD_NUM = 256, 1024  # MI355X


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


def _stats_lines(outdir, name):
    rows = _csv_rows(_find(os.path.join(outdir, name), "_kernel_stats.csv"))
    out = [f"{'calls':>6} {'avg us':>10} {'min us':>10} {'max us':>10} {'share %':>8}  kernel"]
    for r in rows:
        out.append(f"{int(r['Calls']):>6} {float(r['AverageNs'])/1e3:>10.1f} {float(r['MinNs'])/1e3:>10.1f} "
                   f"{float(r['MaxNs'])/1e3:>10.1f} {float(r['Percentage']):>8.2f}  {_short(r['Name'])}")
    return out


def _resource_lines(outdir, name, want):
    """Per-kernel resources from the kernel trace: VGPRs (arch + accumulation),
    SGPRs, LDS bytes per workgroup, scratch, workgroup and grid size."""
    try:
        rows = _csv_rows(_find(os.path.join(outdir, name), "_kernel_trace.csv"))
    except FileNotFoundError:
        return ["(no kernel trace CSV)"]
    cols = [("VGPR_Count", "VGPR"), ("Arch_VGPR_Count", "VGPR"), ("Accum_VGPR_Count", "AGPR"),
            ("SGPR_Count", "SGPR"), ("LDS_Block_Size", "LDS B"), ("Scratch_Size", "scratch"),
            ("Workgroup_Size_X", "WG"), ("Workgroup_Size", "WG"), ("Grid_Size_X", "grid"), ("Grid_Size", "grid")]
    have = [(c, h) for c, h in cols if rows and c in rows[0]]
    seen, out = set(), ["VGPR as rocprofv3 prints it: its granule count times 4; gfx950 allocates 8 VGPRs per "
                        "granule, so the allocation is twice this figure (the compiler's resource remark for the "
                        "forward kernel: 253 VGPRs, allocated 256)", "",
                        "  ".join(f"{h:>9}" for _, h in have) + "  kernel"]
    for r in rows:
        if not want(r["Kernel_Name"]) or r["Kernel_Name"] in seen:
            continue
        seen.add(r["Kernel_Name"])
        out.append("  ".join(f"{r[c]:>9}" for c, _ in have) + "  " + _short(r["Kernel_Name"]))
    return out


def _counter_means(outdir, names, want):
    """{(kernel, grid size): {counter: mean over its dispatches}} from the
    counter CSVs of the runs ``names``, and each one's mean duration (ns) in
    those runs."""
    vals, dur = {}, {}
    for name in names:
        d = os.path.join(outdir, name)
        if not os.path.isdir(d):
            continue
        for r in _csv_rows(_find(d, "_counter_collection.csv")):
            if not want(r["Kernel_Name"]):
                continue
            # one launch shape per key: a split run's transition pass (two
            # walks per segment) and output pass share the kernel
            k = (r["Kernel_Name"], int(r.get("Grid_Size") or 0))
            vals.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            if "End_Timestamp" in r and "Start_Timestamp" in r:
                dur.setdefault(k, {})[(name, r.get("Dispatch_Id"))] = \
                    float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    means = {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in vals.items()}
    durs = {k: sum(v.values()) / len(v) for k, v in dur.items()}
    return means, durs


def _bwd_calls(rows):
    """gdn2_chunk_bwd calls in a profiled run: one dispatch of the group
    ranking kernel per call that runs two groups of sequences, else one
    dispatch of the gradient kernel per call."""
    ids = lambda tag: {r.get("Dispatch_Id") for r in rows if tag in r["Kernel_Name"]}
    return len(ids("bwd_group_kernel")) or len(ids("bwd_chunk_kernel"))


def _sq_lines(outdir, prefix, suffix, want, chunk_heads, title, per_call=False):
    """The SQ counter passes of one workload, per kernel: rocprofv3's derived
    utilisations, and instruction counts per (64-token chunk, value head)
    summed over the workgroup's waves. per_call: a kernel dispatched more
    than once per call (the backward's two groups) has its counts summed
    over the call's dispatches."""
    names = [prefix + n + suffix for n in SQ_PASSES]
    if not all(os.path.isdir(os.path.join(outdir, n)) for n in names):
        return []
    means, durs = _counter_means(outdir, names, want)
    mult = {}
    if per_call:
        rows = _csv_rows(_find(os.path.join(outdir, names[0]), "_counter_collection.csv"))
        calls = max(_bwd_calls(rows), 1)
        for k in means:
            n = len({r.get("Dispatch_Id") for r in rows
                     if r["Kernel_Name"] == k[0] and int(r.get("Grid_Size") or 0) == k[1]})
            mult[k] = n / calls if n else 1.0
    cmds = [profile_command(n) for n in names]
    out = ["", f"## SQ counters per launch ({title}; rocprofv3 --pmc, three passes)", "", "commands:"]
    out += ["  " + c for c in cmds]
    out += ["", f"per chunk-head: divided by the {chunk_heads} (64-token chunk, value head) pairs of one call", ""]
    for k, c in sorted(means.items()):
        g = lambda n: c.get(n, float("nan"))
        m = mult.get(k, 1.0)
        ch = chunk_heads / m  # counts per dispatch, over the chunk-heads of a call's dispatches
        out.append(_short(k[0]) + (f"  [grid {k[1]} threads]" if k[1] else "")
                   + (f"  [{m:.0f} dispatches per call: counts summed over them]" if m != 1.0 else ""))
        dur = durs.get(k)
        if dur:
            out.append(f"  mean dispatch {dur/1e3:.1f} us in the counter runs")
        out.append(f"  MFMA busy (MfmaUtil) {g('MfmaUtil'):.1f} %   VALU busy (VALUBusy) {g('VALUBusy'):.1f} %   "
                   f"MFMA/VALU co-issue cycles {g('SQ_VALU_MFMA_COEXEC_CYCLES')/ch:.0f} per chunk-head")
        out.append(f"  LDS: bank-conflict stall (LDSBankConflict) {g('LDSBankConflict'):.2f} %, "
                   f"busy (LdsUtil) {g('LdsUtil'):.1f} %, wait for LDS issue {g('SQ_WAIT_INST_LDS')*4/ch:.0f} "
                   f"wave-cycles per chunk-head")
        out.append(f"  TA busy {g('TA_BUSY_avr'):.0f} cycles (mean over TA instances), address path stalled by "
                   f"TC {g('TA_ADDR_STALLED_BY_TC_CYCLES_sum'):.0f} cycles (sum)")
        out.append(f"  instructions per chunk-head: VALU {g('SQ_INSTS_VALU')/ch:.0f} (transcendental f32 "
                   f"{g('SQ_INSTS_VALU_TRANS_F32')/ch:.0f}), MFMA {g('SQ_INSTS_MFMA')/ch:.0f}, LDS "
                   f"{g('SQ_INSTS_LDS')/ch:.0f}, vector-memory reads {g('SQ_INSTS_VMEM_RD')/ch:.0f}")
        out.append(f"  waves {g('SQ_WAVES'):.0f}; wave-cycles waiting for issue {g('SQ_WAIT_INST_ANY')*4/ch:.0f}, "
                   f"active on any instruction {g('SQ_ACTIVE_INST_ANY')/ch:.0f} per chunk-head")
    return out


def _chunk_heads(config_id: int) -> int:
    from linear_attention_rnn_gdn2_amd.workloads import WORKLOADS, lengths_of
    return sum((n + 63) // 64 for n in lengths_of(config_id)) * WORKLOADS[config_id].HV


def summarize_profiles(outdir: str, dest: str | None = None):
    """Turn the rocprofv3 CSVs of the PROFILE_STEPS runs under ``outdir`` into
    the committed text summaries, each headed by the hash of the sources it
    was taken on: per forward workload the kernel-trace statistics, the
    kernel's resources and its SQ counters, plus (varlen) the HBM bytes per
    launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each scaled by the
    same counter's reading for a plain device copy of 1 GiB (so that bytes
    per KiB-unit are calibrated, not assumed); the same for every backward
    kernel. The summaries go to ``dest`` (default: profiles/)."""
    dest = dest or os.path.join(ROOT, "profiles")
    traffic_file = os.path.join(dest, os.path.basename(TRAFFIC_FILE))
    src_hash = kernel_source_hash()
    head = f"kernel source hash (sha256 over csrc/{', '.join(FWD_KERNEL_SOURCES)}, first 16 hex): {src_hash}"
    fwd = lambda n: KERNEL_TAG in n
    ours = lambda n: "gdn2::" in n

    def counter(name, want_kernel, value_min=0.0):
        rows = _csv_rows(_find(os.path.join(outdir, name), "_counter_collection.csv"))
        vals = [float(r["Counter_Value"]) for r in rows if want_kernel(r["Kernel_Name"])
                and float(r["Counter_Value"]) >= value_min]
        if not vals:
            raise ValueError(f"{name}: no matching dispatch")
        return vals

    copy = lambda n: "copyBuffer" in n
    copy_bytes = 1024 * (1 << 20)
    cal_f = max(counter("cal_fetch", copy))
    cal_w = max(counter("cal_write", copy))
    fetch_scale = copy_bytes / (cal_f * 1024)  # bytes per counted byte
    write_scale = copy_bytes / (cal_w * 1024)

    # forward, varlen H32 D128 (the headline workload)
    lines = [f"# rocprofv3 summary: GDN-2 forward (chunk_fwd_kernel), varlen H32 D128", "", head, "",
             "## kernel-trace statistics", "", "command (from the repository root):",
             "  " + profile_command("kt"), ""] + _stats_lines(outdir, "kt")
    lines += ["", "## resources (kernel trace)", ""] + _resource_lines(outdir, "kt", ours)
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
    lines += _sq_lines(outdir, "", "", fwd, _chunk_heads(2), "varlen")
    with open(os.path.join(dest, f"{KERNEL_TAG}_varlen_h32_d128.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(traffic_file, "w") as f:
        json.dump({"kernel_source_hash": src_hash, "hbm_bytes_per_launch": fetch + write,
                   "hbm_read_bytes": fetch, "hbm_write_bytes": write,
                   "fetch_scale": fetch_scale, "write_scale": write_scale,
                   "commands": [profile_command(n) for n in ("pmc_fetch", "pmc_write", "cal_fetch", "cal_write")]},
                  f, indent=1)
        f.write("\n")
    log("\n".join(lines))

    # forward, long_decay H16 D128 (strong decay: flagged channels in every chunk)
    if os.path.isdir(os.path.join(outdir, "kt4")):
        l4 = [f"# rocprofv3 summary: GDN-2 forward, long_decay H16 D128 (split walk)", "", head, "",
              "## kernel-trace statistics", "", "command (from the repository root):",
              "  " + profile_command("kt4"), ""] + _stats_lines(outdir, "kt4")
        l4 += ["", "## resources (kernel trace)", ""] + _resource_lines(outdir, "kt4", ours)
        l4 += _sq_lines(outdir, "", "_4", ours, _chunk_heads(4), "long_decay")
        with open(os.path.join(dest, f"{KERNEL_TAG}_long_decay_h16_d128.txt"), "w") as f:
            f.write("\n".join(l4) + "\n")
        log("\n".join(l4))

    # backward, varlen
    if os.path.isdir(os.path.join(outdir, "bkt")):
        bl = [f"# rocprofv3 summary: GDN-2 backward (gdn2_chunk_bwd), varlen H32 D128", "", head, "",
              "## kernel-trace statistics", "", "command (from the repository root):",
              "  " + profile_command("bkt"), ""] + _stats_lines(outdir, "bkt")
        try:
            tr = _csv_rows(_find(os.path.join(outdir, "bkt"), "_kernel_trace.csv"))
        except FileNotFoundError:
            tr = []
        ncall = _bwd_calls(tr)
        if ncall and any("bwd_group_kernel" in r["Kernel_Name"] for r in tr):
            tot = {}
            for r in tr:
                if ours(r["Kernel_Name"]):
                    t = tot.setdefault(r["Kernel_Name"], [0, 0.0])
                    t[0] += 1
                    t[1] += float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
            bl += ["", f"per call ({ncall} calls): each call runs its sequences as two groups (the longer half on "
                   f"the call's stream, the shorter half on a second stream, overlapping), so every pass is "
                   f"dispatched twice and the sums below exceed the call's wall time", "",
                   f"{'per call':>9} {'sum us':>10}  kernel"]
            for kname, (n, ns) in sorted(tot.items(), key=lambda x: -x[1][1]):
                bl.append(f"{n / ncall:>9.1f} {ns / ncall / 1e3:>10.1f}  {_short(kname)}")
        bl += ["", "## resources (kernel trace)", ""] + _resource_lines(outdir, "bkt", ours)
        if os.path.isdir(os.path.join(outdir, "bpmc_fetch")) and os.path.isdir(os.path.join(outdir, "bpmc_write")):
            bl += ["", "## HBM traffic per launch of each backward kernel (rocprofv3 --pmc, one counter per run)", "",
                   f"scaled by the 1 GiB copy calibration of the forward's runs: fetch x{fetch_scale:.3f}, "
                   f"write x{write_scale:.3f}", "",
                   "commands:", "  " + profile_command("bpmc_fetch"), "  " + profile_command("bpmc_write"), "",
                   f"per call: each kernel's bytes summed over its dispatches and divided by the number of "
                   f"gdn2_chunk_bwd calls in the run (a call that runs its sequences as two groups on two "
                   f"streams dispatches each pass twice, once per group; split runs dispatch some kernels "
                   f"more than once)", "",
                   f"{'read MB':>10} {'write MB':>10} {'per call':>9}  kernel"]
            per, calls = {}, {}
            for name, key, scale in (("bpmc_fetch", 0, fetch_scale), ("bpmc_write", 1, write_scale)):
                rows = _csv_rows(_find(os.path.join(outdir, name), "_counter_collection.csv"))
                calls[name] = _bwd_calls(rows)
                for r in rows:
                    if ours(r["Kernel_Name"]):
                        per.setdefault(r["Kernel_Name"], ([], []))[key].append(
                            float(r["Counter_Value"]) * 1024 * scale)
            nf, nw = max(calls["bpmc_fetch"], 1), max(calls["bpmc_write"], 1)
            total = 0.0
            for kname, (fv, wv) in sorted(per.items()):
                rd, wr = sum(fv) / nf, sum(wv) / nw
                total += rd + wr
                bl.append(f"{rd/1e6:>10.1f} {wr/1e6:>10.1f} {len(fv) / nf:>9.1f}  {_short(kname)}")
            bl.append(f"sum over the kernels of one call: {total/1e6:.1f} MB")
        bl += _sq_lines(outdir, "b", "", ours, _chunk_heads(2), "backward, varlen", per_call=True)
        with open(os.path.join(dest, f"bwd_kernels_varlen_h32_d128.txt"), "w") as f:
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


def _device_set(d, dev):
    import torch
    wl = d["workload"]
    T, N = int(d["cu_seqlens"][-1]), len(d["lengths"])
    x = {n: d[n].to(dev) for n in ("q", "k", "v", "g", "beta", "w")}
    x["initial_state"] = None if d["initial_state"] is None else d["initial_state"].to(dev)
    x["cu_seqlens"] = d["cu_seqlens"].to(dev)
    x["out"] = torch.empty((T, wl.HV, wl.V), dtype=torch.bfloat16, device=dev)
    x["final_state"] = torch.empty((N, wl.HV, wl.K, wl.V), dtype=torch.float32, device=dev)
    return x


def _set_bytes(x) -> int:
    return sum(t.numel() * t.element_size() for t in x.values() if t is not None)


def input_sets(config_id, seed, dev, cold: bool, cache_bytes: int = 512 << 20):
    """The device input sets a timed run rotates through: one, or with
    ``cold`` at least three whose total exceeds ``cache_bytes`` (more than the
    MI355X's 256 MB last-level cache, so that no launch finds its inputs
    there from the previous one). Set i is drawn with seed + 1000 i."""
    from linear_attention_rnn_gdn2_amd.workloads import make_inputs
    d = make_inputs(config_id, seed)
    sets = [_device_set(d, dev)]
    if cold:
        per = _set_bytes(sets[0])
        n = max(3, -(-(cache_bytes + 1) // per))
        for i in range(1, n):
            sets.append(_device_set(make_inputs(config_id, seed + 1000 * i), dev))
    return d, sets


def time_forward(gdn2, sets, scale, steps, warmup, dev):
    """Warm up, then time ``steps`` calls, call i on input set i mod len(sets):
    returns (per-call times in ms from HIP events on the launch stream, wall
    seconds of the whole timed region)."""
    import torch

    def call(x):
        gdn2.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["w"], scale=scale,
                       initial_state=x["initial_state"], cu_seqlens=x["cu_seqlens"],
                       out=x["out"], final_state=x["final_state"])

    for i in range(warmup):
        call(sets[i % len(sets)])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        call(sets[i % len(sets)])
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return [a.elapsed_time(b) for a, b in ev], wall


def other_workloads(gdn2, dev, ids, steps, seed_base):
    """Tokens/s and roofline fraction of further workloads (each its own
    seeded draw). single rotates cold input sets (each set is smaller than
    the last-level cache); gva and long_decay move several GB per call."""
    import torch
    from linear_attention_rnn_gdn2_amd.workloads import WORKLOADS
    res = []
    for c in ids:
        wl = WORKLOADS[c]
        cold = c == 1
        d, sets = input_sets(c, c if seed_base is None else seed_base, dev, cold)
        T, N = int(d["cu_seqlens"][-1]), len(d["lengths"])
        ms, wall = time_forward(gdn2, sets, d["scale"], steps, 2, dev)
        mean_s = sum(ms) / len(ms) / 1e3
        algo = algorithmic_bytes(T, N, wl.H, wl.HV, wl.K, wl.V, d["initial_state"] is not None, True)
        r = {"workload": f"{wl.name}: {N} x {T // N} tokens, H={wl.H} HV={wl.HV} K={wl.K} V={wl.V}",
             "tokens_per_s": T / mean_s, "mean_call_ms": mean_s * 1e3, "wall_ms_per_step": wall / steps * 1e3,
             "algorithmic_bytes_per_call": algo, "roofline_frac": algo / mean_s / 1e9 / HBM_PEAK_GBS,
             "input_sets": len(sets), "input_bytes_total": sum(_set_bytes(x) for x in sets)}
        log(f"{wl.name}: mean call {mean_s*1e3:.3f} ms, {T / mean_s / 1e6:.2f} M tokens/s, "
            f"{algo / mean_s / 1e9 / HBM_PEAK_GBS * 100:.1f}% of HBM peak ({len(sets)} input set(s))")
        res.append(r)
        del d, sets
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--seed", type=int, default=None,
                    help="seed of the synthetic inputs (default: the workload id)")
    ap.add_argument("--cold-cache", action="store_true",
                    help="rotate at least three input sets totalling more than 512 MB through the timed calls")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the single / gva / long_decay timings that follow the headline")
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
        summarize_profiles(args.summarize_profiles)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only (every chain of the GDN-2 "
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
    seed = args.workload if args.seed is None else args.seed
    log(f"drawing workload {args.workload} (seed {seed})")
    if args.mode == "bwd":
        bench_bwd(args, make_inputs(args.workload, seed), gdn2, dev)
        return
    d, sets = input_sets(args.workload, seed, dev, args.cold_cache)
    wl = d["workload"]
    T = int(d["cu_seqlens"][-1])
    N = len(d["lengths"])
    has_init = d["initial_state"] is not None
    launch_ms, wall = time_forward(gdn2, sets, d["scale"], args.steps, args.warmup, dev)
    mean_launch_s = sum(launch_ms) / len(launch_ms) / 1e3
    ms_per_step = wall / args.steps * 1e3
    value = T / (ms_per_step / 1e3)

    algo = algorithmic_bytes(T, N, wl.H, wl.HV, wl.K, wl.V, has_init, True)
    achieved = algo / mean_launch_s / 1e9
    src_hash = kernel_source_hash()
    traffic = measured_traffic(src_hash) if args.workload == 2 else None
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
                               f"H={wl.H} HV={wl.HV} K={wl.K} V={wl.V}, chunk 64, seed {seed}"
                               + (f", {len(sets)} input sets rotated" if len(sets) > 1 else ""),
                   "global_batch": N, "seq_len": T, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": algo, "mean_launch_ms": mean_launch_s * 1e3,
                     "kernel_source_hash": src_hash},
    }
    log(f"mean launch {mean_launch_s*1e3:.3f} ms, wall/step {ms_per_step:.3f} ms, "
        f"{value/1e6:.2f} M tokens/s, {achieved:.0f} GB/s algorithmic ({achieved/HBM_PEAK_GBS*100:.1f}% of HBM peak)")
    cpu_d = d
    del sets
    torch.cuda.empty_cache()
    if not args.no_extra:
        rec["other_workloads"] = other_workloads(gdn2, dev, [c for c in (1, 3, 4) if c != args.workload],
                                                 args.steps, args.seed)
    if not args.no_peaks:
        rec["measured_peaks"] = measured_peaks(dev)
        log(f"measured on this device: copy {rec['measured_peaks']['copy_GBps']:.0f} GB/s, "
            f"bf16 GEMM {rec['measured_peaks']['bf16_gemm_TFLOPs']:.0f} TFLOP/s")
    if not args.no_cpu_baseline:
        log("timing the FP64 oracle on the host")
        rec["cpu_baseline"] = cpu_baseline(cpu_d, wl)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
