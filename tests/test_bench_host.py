"""Host-side logic of bench.py: pair counting and the counter fold."""

import csv
import os

import numpy as np

import bench
import synth

HDR = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id",
       "Thread_Id", "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size",
       "LDS_Block_Size", "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count",
       "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp",
       "End_Timestamp"]


def _csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(HDR)
        for d, (name, kib) in enumerate(rows, 1):
            w.writerow([d, d, "Agent 1", 1, 1, 1, 64, 1, name, 64, 0, 0, 8, 0,
                        8, counter, kib, 0, 1])


def test_fold_traffic_scales_by_probe(tmp_path):
    mib = 64
    copy = mib << 20
    # the probe copy reads 10% more and writes 20% less than its size
    fetch = [("void ns::prefill_kernel<128, 8, 2>(P)", 1000.0),
             ("void ns::prefill_kernel<128, 8, 2>(P)", 1100.0),
             ("void ns::prefill_kernel<128, 8, 2>(P)", 1200.0),
             ("decode_split_kernel<128, 4>(P)", 500.0),
             ("decode_combine_kernel<128>(P)", 50.0),
             ("__amd_rocclr_copyBuffer", 1.1 * copy / 1024),
             ("__amd_rocclr_copyBuffer", 3.0)]  # a small host copy
    write = [("void ns::prefill_kernel<128, 8, 2>(P)", 400.0),
             ("decode_split_kernel<128, 4>(P)", 40.0),
             ("decode_combine_kernel<128>(P)", 4.0),
             ("__amd_rocclr_copyBuffer", 0.8 * copy / 1024)]
    fp, wp = tmp_path / "f.csv", tmp_path / "w.csv"
    _csv(fp, "FETCH_SIZE", fetch)
    _csv(wp, "WRITE_SIZE", write)
    rec = bench.fold_traffic(str(fp), str(wp), copy)
    sf, sw = 1 / 1.1, 1 / 0.8
    assert np.isclose(rec["copy_probe"]["scale_fetch"], sf)
    assert np.isclose(rec["copy_probe"]["scale_write"], sw)
    # median of the three prefill dispatches
    want = 1100 * 1024 * sf + 400 * 1024 * sw
    assert np.isclose(rec["prefill"]["hbm_bytes_per_launch"], want)
    want_d = (500 + 50) * 1024 * sf + (40 + 4) * 1024 * sw
    assert np.isclose(rec["decode"]["hbm_bytes_per_launch"], want_d)
    assert rec["prefill"]["source_sha256"] == bench.source_sha(
        bench.KERNEL_SOURCES["prefill"])


def test_allowed_pairs_matches_mask_count():
    from oracle import allowed_mask
    for w in (synth.Workload("t", 2, 2, 1, 37, 37, 64, "bf16", True,
                             window=5, len_lo=20, len_hi=37),
              synth.Workload("t", 3, 2, 2, 1, 50, 64, "bf16", True,
                             len_lo=1, len_hi=50),
              synth.Workload("t", 1, 1, 1, 16, 16, 64, "bf16", False),
              synth.Workload("t", 2, 1, 1, 40, 90, 64, "bf16", True,
                             window=9, sinks=5, len_lo=1, len_hi=90),
              synth.Workload("t", 2, 1, 1, 70, 70, 64, "bf16", False,
                             window=6, window_right=4, sinks=8, len_lo=3,
                             len_hi=70),
              synth.Workload("t", 1, 1, 1, 30, 60, 64, "bf16", False,
                             window_right=7, sinks=40),
              synth.Workload("t", 3, 1, 1, 1, 77, 64, "bf16", True,
                             window=10, sinks=12, len_lo=1, len_hi=77)):
        x = synth.make_inputs(w, 11)
        sl = x["seqlens"]
        total = 0
        for b in range(w.B):
            L = w.Nk if sl is None else int(sl[b])
            m = allowed_mask(w.Nq, w.Nk, L, w.causal, w.window,
                             window_right=w.window_right, sinks=w.sinks)
            total += int(m.sum())
        assert bench.allowed_pairs(w, sl) == total


def test_prefill_roofline_takes_the_longer_bound():
    """gpt2-small-causal-padded moves more bytes per FLOP than the ridge
    (2.5 PFLOP/s over 8 TB/s, 312 FLOP/B) allows: its bound is HBM.  The
    headline grouped-query prefill is MFMA-bound."""
    w = synth.by_name("gpt2-small-causal-padded")
    sl = synth.make_inputs(w, 2)["seqlens"]
    r = bench.prefill_roofline(w, sl, 1e-4)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["algorithmic_flop_per_launch"] / \
        r["algorithmic_bytes_per_launch"] < 312.5
    live = int(np.minimum(sl, 1024).sum())
    assert r["algorithmic_bytes_per_launch"] == \
        live * 12 * (2 * 64 * 2 + 4) + live * 12 * 2 * 64 * 2
    assert abs(r["achieved"] - r["algorithmic_bytes_per_launch"] / 1e-4 /
               1e9) < 0.1
    wp = synth.by_name("gqa-causal-prefill")
    rp = bench.prefill_roofline(wp, None, 1e-3)
    assert rp["bound"] == "mfma" and rp["unit"] == "TFLOP/s"
    assert rp["algorithmic_flop_per_launch"] == 4 * 128 * 28 * 4 * \
        (4096 * 4097 // 2)


def test_cpu_model_reads_proc_cpuinfo():
    m = bench.cpu_model()
    assert m is None or isinstance(m, str) and m
