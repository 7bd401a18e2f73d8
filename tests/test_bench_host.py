"""Host-side checks of the measurement code in bench.py (no GPU).

The roofline figures bench.py reports divide algorithmic bytes by a measured
time, and its HBM traffic comes from rocprofv3 counters scaled by a copy of
known size. These tests pin the byte counts to the totals worked out by hand
for the workloads (per (token, value head): 4K/m for q, k shared by m value
heads, 6V for v, w, out, 2K for beta, 4K for g; 64 KiB per state read or
written), run the counter summary on synthetic rocprofv3 CSVs whose answer is
known, and check that multi-GPU runs are refused before any device work.
"""

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_forward_bytes_per_token_head():
    # K = V = 128: 2,048 B per (token, value head) with m = 1, 1,706.7 B with m = 3
    assert bench.algorithmic_bytes(1, 1, 1, 1, 128, 128, False, False) == 2048
    assert bench.algorithmic_bytes(3, 1, 1, 3, 128, 128, False, False) == 3 * 5120  # 5,120 / 3 per head
    # K = V = 64: half
    assert bench.algorithmic_bytes(1, 1, 1, 1, 64, 64, False, False) == 1024


def test_forward_bytes_of_the_workloads():
    # varlen: 37,517 tokens, 32 heads, states in and out (8 sequences)
    assert bench.algorithmic_bytes(37517, 8, 32, 32, 128, 128, True, True) == 2_492_268_544
    # single: 4,096 tokens, 16 heads, states in and out
    assert bench.algorithmic_bytes(4096, 1, 16, 16, 128, 128, True, True) == 136_314_880
    # gva: 65,536 tokens, H = 16, HV = 48, final states only (4 sequences)
    assert bench.algorithmic_bytes(65536, 4, 16, 48, 128, 128, False, True) == 5_381_292_032
    # long_decay: 131,072 tokens, 16 heads, final states only (2 sequences)
    assert bench.algorithmic_bytes(131072, 2, 16, 16, 128, 128, False, True) == 4_297_064_448


def test_backward_bytes():
    # per (token, value head) at m = 1, K = V = 128: q, k, dq, dk 1,024 B;
    # v, w, d_out, dv, dw 1,280 B; beta, dbeta 512 B; g, dg 1,024 B; plus
    # per (sequence, head) the initial state's gradient (always written
    # by the bench's calls), the initial state when given, and the final
    # state's gradient when given
    s = 128 * 128 * 4
    assert bench.bwd_algorithmic_bytes(1, 1, 1, 1, 128, 128, False, False) == 1024 + 1280 + 512 + 1024 + s
    assert bench.bwd_algorithmic_bytes(0, 1, 1, 1, 128, 128, True, True) == 3 * s
    assert bench.bwd_algorithmic_bytes(0, 1, 1, 1, 128, 128, False, True) == 2 * s
    # varlen: 4.66 GB
    assert bench.bwd_algorithmic_bytes(37517, 8, 32, 32, 128, 128, True, True) == 37517 * 32 * 3840 + 8 * 32 * 3 * s


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_counter_summary_on_synthetic_profiles(tmp_path):
    """A 1 GiB copy that reads FETCH_SIZE 524,288 KiB and WRITE_SIZE
    1,048,576 KiB gives scale factors 2 and 1; a forward dispatch with
    FETCH_SIZE 1,000 KiB and WRITE_SIZE 500 KiB then moved 2,048,000 +
    512,000 bytes."""
    out = tmp_path / "prof_out"
    fwd = "void gdn2::(anonymous namespace)::chunk_fwd_kernel<128, 128, 0, false, false, false>(gdn2::FwdParams)"
    copy = "__amd_rocclr_copyBuffer"
    stats_hdr = ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"]
    _write_csv(str(out / "kt" / "kt_kernel_stats.csv"), stats_hdr,
               [[fwd, 12, 10_800_000, 900_000, 99.9, 880_000, 950_000], [copy, 1, 4_000, 4_000, 0.1, 4_000, 4_000]])
    _write_csv(str(out / "bkt" / "bkt_kernel_stats.csv"), stats_hdr, [[fwd, 7, 7_000_000, 1_000_000, 100.0, 1, 2]])
    ctr_hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    _write_csv(str(out / "cal_fetch" / "cal_fetch_counter_collection.csv"), ctr_hdr,
               [[1, copy, "FETCH_SIZE", 524288.0], [2, copy, "FETCH_SIZE", 524000.0]])
    _write_csv(str(out / "cal_write" / "cal_write_counter_collection.csv"), ctr_hdr,
               [[1, copy, "WRITE_SIZE", 1048576.0]])
    _write_csv(str(out / "pmc_fetch" / "pmc_fetch_counter_collection.csv"), ctr_hdr,
               [[1, copy, "FETCH_SIZE", 9.0], [2, fwd, "FETCH_SIZE", 1000.0], [3, fwd, "FETCH_SIZE", 1000.0]])
    _write_csv(str(out / "pmc_write" / "pmc_write_counter_collection.csv"), ctr_hdr,
               [[2, fwd, "WRITE_SIZE", 400.0], [3, fwd, "WRITE_SIZE", 600.0]])
    bwd_a = "void gdn2::(anonymous namespace)::bwd_chunk_kernel<128>(gdn2::BwdParams)"
    bwd_b = "void gdn2::(anonymous namespace)::bwd_state_kernel<128, false>(gdn2::BwdParams)"
    other = "void at::native::elementwise_kernel<128, 4>()"
    # two backward calls per run; the state kernel dispatched twice per call
    # (as in a split run)
    _write_csv(str(out / "bpmc_fetch" / "bpmc_fetch_counter_collection.csv"), ctr_hdr,
               [[1, other, "FETCH_SIZE", 5e6], [2, bwd_a, "FETCH_SIZE", 1000.0], [3, bwd_a, "FETCH_SIZE", 3000.0]]
               + [[4 + i, bwd_b, "FETCH_SIZE", 500.0] for i in range(4)])
    _write_csv(str(out / "bpmc_write" / "bpmc_write_counter_collection.csv"), ctr_hdr,
               [[2, bwd_a, "WRITE_SIZE", 250.0], [3, bwd_a, "WRITE_SIZE", 350.0]]
               + [[4 + i, bwd_b, "WRITE_SIZE", 100.0] for i in range(4)])
    # SQ passes: 1,000 VALU instructions per (chunk, value head) of the
    # varlen call and rocprofv3's derived utilisations passed through
    ch = bench._chunk_heads(2)
    _write_csv(str(out / "sq1" / "sq1_counter_collection.csv"), ctr_hdr,
               [[2, fwd, "MfmaUtil", 12.5], [2, fwd, "VALUBusy", 40.0], [2, fwd, "SQ_INSTS_VALU", 1000.0 * ch],
                [2, fwd, "SQ_INSTS_MFMA", 300.0 * ch], [2, fwd, "SQ_INSTS_VALU_TRANS_F32", 80.0 * ch],
                [3, copy, "SQ_INSTS_VALU", 1.0]])
    _write_csv(str(out / "sq2" / "sq2_counter_collection.csv"), ctr_hdr,
               [[2, fwd, "LDSBankConflict", 1.25], [2, fwd, "LdsUtil", 30.0], [2, fwd, "SQ_INSTS_LDS", 500.0 * ch],
                [2, fwd, "SQ_WAIT_INST_LDS", 10.0 * ch], [2, fwd, "SQ_VALU_MFMA_COEXEC_CYCLES", 7.0 * ch]])
    _write_csv(str(out / "sq3" / "sq3_counter_collection.csv"), ctr_hdr,
               [[2, fwd, "SQ_WAIT_INST_ANY", 5.0 * ch], [2, fwd, "SQ_ACTIVE_INST_ANY", 9.0 * ch],
                [2, fwd, "SQ_WAVES", 2048.0], [2, fwd, "SQ_INSTS_VMEM_RD", 20.0 * ch],
                [2, fwd, "TA_BUSY_avr", 123.0], [2, fwd, "TA_ADDR_STALLED_BY_TC_CYCLES_sum", 45.0]])
    dest = tmp_path / "profiles"
    dest.mkdir()
    bench.summarize_profiles(str(out), dest=str(dest))
    rec = json.load(open(dest / "hbm_traffic_varlen_h32_d128.json"))
    assert rec["fetch_scale"] == pytest.approx(2.0)
    assert rec["write_scale"] == pytest.approx(1.0)
    assert rec["hbm_read_bytes"] == pytest.approx(2_048_000)
    assert rec["hbm_write_bytes"] == pytest.approx(512_000)
    assert rec["kernel_source_hash"] == bench.kernel_source_hash()
    txt = open(dest / "chunk_fwd_kernel_varlen_h32_d128.txt").read()
    assert "900.0" in txt and "total 2.56 MB per launch" in txt
    assert bench.kernel_source_hash() in txt
    assert "MFMA busy (MfmaUtil) 12.5 %   VALU busy (VALUBusy) 40.0 %" in txt
    assert "VALU 1000 (transcendental f32 80), MFMA 300, LDS 500, vector-memory reads 20" in txt
    assert "bank-conflict stall (LDSBankConflict) 1.25 %" in txt and "wait for LDS issue 40 " in txt
    assert "copyBuffer" not in txt.split("## SQ counters")[1]
    # backward, per call (two calls): bwd_chunk reads 4,000 KiB x 2 / 2 and
    # writes 600 KiB / 2; bwd_state reads 2,000 KiB x 2 / 2 and writes
    # 400 KiB / 2 over two dispatches per call; torch's own kernels are left out
    btxt = open(dest / "bwd_kernels_varlen_h32_d128.txt").read()
    assert "       4.1        0.3       1.0  " + bwd_a in btxt
    assert "       2.0        0.2       2.0  " + bwd_b in btxt
    assert "sum over the kernels of one call: 6.7 MB" in btxt
    assert "elementwise" not in btxt


def test_traffic_is_null_for_another_source(tmp_path, monkeypatch):
    f = tmp_path / "t.json"
    f.write_text(json.dumps({"kernel_source_hash": "0" * 16, "hbm_bytes_per_launch": 1.0}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic(bench.kernel_source_hash()) is None
    f.write_text(json.dumps({"kernel_source_hash": bench.kernel_source_hash(), "hbm_bytes_per_launch": 5.0}))
    assert bench.measured_traffic(bench.kernel_source_hash()) == 5.0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_backward_summary_with_two_groups(tmp_path):
    """Two backward calls that each run two groups of sequences: one group
    ranking dispatch per call, every pass dispatched twice per call. Bytes
    and instruction counts are per call (summed over the call's dispatches),
    and the kernel trace gives each kernel's time summed per call."""
    out = tmp_path / "prof_out"
    fwd = "void gdn2::(anonymous namespace)::chunk_fwd_kernel<128, 128, 0, false, false, false>(gdn2::FwdParams)"
    copy = "__amd_rocclr_copyBuffer"
    stats_hdr = ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"]
    ctr_hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    _write_csv(str(out / "kt" / "kt_kernel_stats.csv"), stats_hdr, [[fwd, 1, 900_000, 900_000, 100.0, 1, 1]])
    _write_csv(str(out / "cal_fetch" / "cal_fetch_counter_collection.csv"), ctr_hdr, [[1, copy, "FETCH_SIZE", 524288.0]])
    _write_csv(str(out / "cal_write" / "cal_write_counter_collection.csv"), ctr_hdr, [[1, copy, "WRITE_SIZE", 1048576.0]])
    _write_csv(str(out / "pmc_fetch" / "pmc_fetch_counter_collection.csv"), ctr_hdr, [[2, fwd, "FETCH_SIZE", 1000.0]])
    _write_csv(str(out / "pmc_write" / "pmc_write_counter_collection.csv"), ctr_hdr, [[2, fwd, "WRITE_SIZE", 500.0]])
    grp = "gdn2::(anonymous namespace)::bwd_group_kernel(gdn2::BwdParams, int, int*)"
    bwd_a = "void gdn2::(anonymous namespace)::bwd_chunk_kernel<128>(gdn2::BwdParams)"
    # per call: the group kernel, then bwd_chunk for group 0 and group 1
    # (1,000 and 3,000 KiB read); two calls
    fetch, write, sq = [], [], []
    i = 1
    for call in range(2):
        fetch.append([i, grp, "FETCH_SIZE", 0.0]); write.append([i, grp, "WRITE_SIZE", 0.0]); i += 1
        for kib in (1000.0, 3000.0):
            fetch.append([i, bwd_a, "FETCH_SIZE", kib]); write.append([i, bwd_a, "WRITE_SIZE", kib / 10])
            i += 1
    _write_csv(str(out / "bpmc_fetch" / "bpmc_fetch_counter_collection.csv"), ctr_hdr, fetch)
    _write_csv(str(out / "bpmc_write" / "bpmc_write_counter_collection.csv"), ctr_hdr, write)
    # SQ passes: each of a call's two bwd_chunk dispatches issues 500 VALU
    # instructions per chunk-head of the call: 1,000 per chunk-head summed
    ch = bench._chunk_heads(2)
    for n, cs in bench.SQ_PASSES.items():
        rows, j = [], 1
        for call in range(2):
            rows.append([j, grp, "SQ_WAVES", 4.0]); j += 1
            for _ in range(2):
                rows += [[j, bwd_a, c, (500.0 * ch if c == "SQ_INSTS_VALU" else 7.0)] for c in cs.split()]
                j += 1
        _write_csv(str(out / ("b" + n) / f"b{n}_counter_collection.csv"), ctr_hdr + ["Grid_Size"],
                   [r + [9732096 if r[1] == bwd_a else 256] for r in rows])
    # kernel trace: per call the group kernel (5 us) and bwd_chunk at 1.0
    # and 2.0 ms
    tr_hdr = ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    tr, t, j = [], 0, 1
    for call in range(2):
        tr.append([j, grp, t, t + 5_000]); j += 1
        for dur in (1_000_000, 2_000_000):
            tr.append([j, bwd_a, t, t + dur]); j += 1
        t += 3_000_000
    _write_csv(str(out / "bkt" / "bkt_kernel_trace.csv"), tr_hdr, tr)
    _write_csv(str(out / "bkt" / "bkt_kernel_stats.csv"), stats_hdr, [[bwd_a, 4, 6_000_000, 1_500_000, 99.0, 1, 2]])
    dest = tmp_path / "profiles"
    dest.mkdir()
    bench.summarize_profiles(str(out), dest=str(dest))
    btxt = open(dest / "bwd_kernels_varlen_h32_d128.txt").read()
    # per call: (1,000 + 3,000) KiB x 2 read, 400 KiB written, two dispatches
    assert "       8.2        0.4       2.0  " + bwd_a in btxt
    assert "per call (2 calls)" in btxt
    assert "      2.0     3000.0  " + bwd_a in btxt
    assert "      1.0        5.0  " + grp in btxt
    assert "[2 dispatches per call: counts summed over them]" in btxt
    assert "instructions per chunk-head: VALU 1000 " in btxt
