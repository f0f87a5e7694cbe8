"""Benchmark of the attention hot path on one MI355X.

One step = one pass of the whole path on resident synthetic inputs:
  1. bf16 causal GQA prefill  B=4 Hq=28 Hkv=4 N=4096 d=128 (the headline),
  2. bf16 decode step         B=64 Hq=32 Hkv=8 d=128, cache lengths U[2048,8192],
  3. fp32 single-head case    B=1 H=1 N=128 d=64.
`value` is the prefill throughput in algorithmic TFLOP/s (4*d FLOPs per
allowed query/key pair, both matrix products, masked pairs not counted); the
decode step is reported in algorithmic HBM GB/s (valid K/V bytes + q + o +
lse).  Per-launch durations come from HIP events recorded on the stream the
kernels run on.  The fp64 CPU oracle is timed on a bounded sample of the
prefill workload as a reported baseline, with every core the process may use.

Besides the step it times, launch by launch with the latency protocol of the
SpAtten review (EVALUATION, latency: `--reps` repetitions, the largest and
smallest 15% dropped, the middle 70% averaged): the two other bf16 prefill
configurations (gpt2-small-causal-padded, sliding-window-causal), each against
its own roofline; the backward pass and the FP8 forward of the headline
prefill; and the 1 < Nq < Nk and local-window workloads (`--no-extra` skips
all of these).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--reps R]
                       [--no-cpu-baseline] [--no-extra] [--copy-probe MIB]
       python bench.py --only WORKLOAD [--seed S] [--reps R] [--warmup W]
       python bench.py --fold-traffic FETCH.csv WRITE.csv
       python bench.py --fold-counters COUNTERS.csv
Prints one JSON line.  `--only` runs one workload's forward call alone
(`backward` runs the headline's backward pass): the form used under
rocprofv3, so a profile holds that workload's kernels only.

HBM traffic: two rocprofv3 counter runs of a short bench with `--no-extra
--copy-probe 1024` (so that the only launches of the kernels are the step's;
one run with `--pmc FETCH_SIZE`, one with
`--pmc WRITE_SIZE`, each with `--output-format csv`) record the counters for
the attention kernels and for a plain device-to-device copy of known size;
`--fold-traffic` scales each kernel's counters by what the copy read and wrote
per byte and stores bytes per launch, with the kernel sources' hashes, in
profiles/traffic.json.  bench.py reports them only while the sources are
unchanged.
"""

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("attention fwd TFLOP/s (bf16 causal prefill) + decode HBM GB/s, "
          "% of roofline")
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E peak
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 matrix peak
PROFILES = os.path.join(ROOT, "profiles")
_CSRC = "transformer_self_attention_attn_amd/csrc/"
# each kernel's source and the local headers it is built from
KERNEL_SOURCES = {
    "prefill": tuple(_CSRC + f for f in (
        "prefill_bf16.hip", "kernels.h", "device_common.h", "lane_layout.h",
        "block_order.h", "fastdiv.h", "tail_queue.h")),
    "decode": tuple(_CSRC + f for f in (
        "decode_bf16.hip", "kernels.h", "device_common.h", "lane_layout.h",
        "fastdiv.h")),
}


def allowed_pairs(w, seqlens):
    """Number of allowed (query, key) pairs per head, summed over batch.

    Row at position pos: keys below hc (valid length; pos + 1 if causal),
    of those the window [lo, hw) and the sinks [0, sk); the count is the
    size of the union of the two ranges."""
    import numpy as np
    total = 0
    for b in range(w.B):
        L = w.Nk if seqlens is None else int(min(max(seqlens[b], 0), w.Nk))
        live = L if w.Nq == w.Nk else w.Nq
        i = np.arange(live, dtype=np.int64)
        pos = i + (L - live)
        hc = np.clip(pos + 1, 0, L) if w.causal else np.full_like(i, L)
        lo = np.maximum(0, pos - w.window + 1) if w.window > 0 else \
            np.zeros_like(i)
        hw = np.clip(pos + w.window_right, 0, hc) if w.window_right > 0 \
            else hc
        sk = np.minimum(w.sinks, hc)
        win = np.maximum(hw - lo, 0)
        both = np.maximum(np.minimum(hw, sk) - lo, 0)
        total += int((win + sk - both).sum())
    return total


def decode_bytes(w, seqlens):
    """Algorithmic bytes of a decode-shaped call: every K/V row some query
    row may see, read once for all the query heads and rows that share it
    (for one row, or a causal chunk without a window, the last row sees them
    all), plus q, o (bf16) and lse (fp32)."""
    assert w.Nq == 1 or (w.causal and not w.window and not w.window_right
                         and not w.sinks)
    keys = allowed_pairs(dataclasses.replace(w, Nq=1), seqlens)  # per b
    kv = keys * w.Hkv * w.d * 2 * 2
    q = w.B * w.Hq * w.Nq * w.d * 2
    o = w.B * w.Hq * w.Nq * w.d * 2
    lse = w.B * w.Hq * w.Nq * 4
    return kv + q + o + lse


def decode_shaped(w):
    """Calls the split-K decode kernel takes: one row, or a chunk whose
    query heads x rows fit its 16 columns."""
    return w.Nq == 1 or (w.Nq < w.Nk and (w.Hq // w.Hkv) * w.Nq <= 16)


def trimmed(ms):
    """SpAtten review, EVALUATION - latency protocol: drop the largest and
    the smallest 15% of the repetitions, average the middle 70%."""
    s = sorted(ms)
    n = len(s)
    cut = int(round(0.15 * n))
    mid = s[cut:n - cut] or s
    return dict(trimmed_mean_ms=sum(mid) / len(mid), p50_ms=s[n // 2],
                min_ms=s[0], reps=n)


def source_sha(rels):
    """sha256 over the files' bytes, in order."""
    h = hashlib.sha256()
    for rel in rels:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_for(kind):
    """HBM bytes per launch from committed rocprofv3 counter runs, only if
    they were taken on the kernel source as it is now."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kind)
    if not rec or rec.get("source_sha256") != source_sha(KERNEL_SOURCES[kind]):
        return None
    return rec.get("hbm_bytes_per_launch")


TRAFFIC_KERNELS = {
    "prefill": ("prefill_kernel",),
    "decode": ("decode_split_kernel", "decode_combine_kernel"),
}
COPY_KERNEL = "copyBuffer"


def read_counter_csv(path, counter):
    """{dispatch_id: (kernel_name, value)} for one counter of a rocprofv3
    counter_collection.csv (values summed over the rows of a dispatch)."""
    import csv
    out = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            d = int(row["Dispatch_Id"])
            name, v = out.get(d, (row["Kernel_Name"], 0.0))
            out[d] = (name, v + float(row["Counter_Value"]))
    return out


def fold_traffic(fetch_csv, write_csv, copy_bytes):
    """Per-launch HBM bytes of the attention kernels from FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled by copy_bytes over what the
    same counter read for the probe copy of copy_bytes bytes."""
    rec = {}
    scale = {}
    per = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        disp = read_counter_csv(path, counter)
        probe = [v for n, v in disp.values()
                 if COPY_KERNEL in n and 0.5 < v * 1024 / copy_bytes < 2.0]
        if not probe:
            raise SystemExit(f"no probe copy of ~{copy_bytes} B in {path}")
        kib = sorted(probe)[len(probe) // 2]
        scale[counter] = copy_bytes / (kib * 1024.0)
        per[counter] = disp
    for kind, names in TRAFFIC_KERNELS.items():
        total = 0.0
        parts = {}
        for nm in names:
            for counter in ("FETCH_SIZE", "WRITE_SIZE"):
                vals = sorted(v for n, v in per[counter].values() if nm in n)
                if not vals:
                    raise SystemExit(f"{nm} not found for {counter}")
                b = vals[len(vals) // 2] * 1024.0 * scale[counter]
                parts[f"{nm}:{counter}"] = b
                total += b
        rec[kind] = {"hbm_bytes_per_launch": total, "parts": parts,
                     "source_sha256": source_sha(KERNEL_SOURCES[kind])}
    rec["copy_probe"] = {"bytes": copy_bytes,
                         "scale_fetch": scale["FETCH_SIZE"],
                         "scale_write": scale["WRITE_SIZE"]}
    return rec


def fold_counters(csv_path, kernel_substr="", simds=1024, dies=8):
    """Per-kernel averages over the dispatches of a rocprofv3 counter CSV
    (rocprofv3 sums each counter over its hardware instances), with the
    derived ratios: MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES over (SIMDs x
    GRBM_GUI_ACTIVE per die; GRBM_GUI_ACTIVE is counted on each of the 8
    dies), and instructions per MFMA.  Returns {kernel: {counter: value}}."""
    import collections
    import csv
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    with open(csv_path, newline="") as f:
        for row in csv.DictReader(f):
            if kernel_substr not in row["Kernel_Name"]:
                continue
            d = int(row["Dispatch_Id"])
            per[d][row["Counter_Name"]] += float(row["Counter_Value"])
            names[d] = row["Kernel_Name"]
    out = {}
    for name in sorted(set(names.values())):
        ds = [d for d in per if names[d] == name]
        avg = {c: sum(per[d].get(c, 0.0) for d in ds) / len(ds)
               for c in sorted({c for d in ds for c in per[d]})}
        avg["dispatches"] = len(ds)
        if "SQ_VALU_MFMA_BUSY_CYCLES" in avg and "GRBM_GUI_ACTIVE" in avg:
            avg["mfma_busy_pct"] = 100.0 * avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (
                simds * avg["GRBM_GUI_ACTIVE"] / dies)
        if avg.get("SQ_INSTS_MFMA"):
            for c in ("SQ_INSTS_VALU", "SQ_INSTS_LDS"):
                if c in avg:
                    avg[c + "_per_mfma"] = avg[c] / avg["SQ_INSTS_MFMA"]
        out[name] = avg
    return out


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None if unreadable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, x, budget_s=20.0):
    """Times the fp64 oracle (as it stands) on whole (batch, head) slices of
    the prefill workload, in order, until about `budget_s` seconds of CPU
    work are done; reports algorithmic TFLOP/s of that sample.  Every core
    the process may use (its affinity set) runs the oracle's BLAS calls."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limiter = threadpool_limits(limits=cores, user_api="blas")
        threads = max([p.get("num_threads", 1) for p in threadpool_info()
                       if p.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        limiter, threads = None, None
    q32, k32, v32 = x["q32"], x["k32"], x["v32"]
    done = 0
    t_total = 0.0
    per_head_pairs = allowed_pairs(w.with_(B=1), None)
    g = w.Hq // w.Hkv
    try:
        while t_total < budget_s and done < w.B * w.Hq:
            b, h = divmod(done, w.Hq)
            hk = h // g
            t0 = time.perf_counter()
            oracle.attention(q32[b:b + 1, h:h + 1], k32[b:b + 1, hk:hk + 1],
                             v32[b:b + 1, hk:hk + 1], scale=w.scale,
                             causal=w.causal, window=w.window, seqlens=None)
            t_total += time.perf_counter() - t0
            done += 1
    finally:
        if limiter is not None:
            limiter.restore_original_limits()
    flops = 4.0 * w.d * per_head_pairs * done
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s",
            "cores": cores, "blas_threads": threads, "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": (f"{done} of {w.B * w.Hq} (batch, head) slices of "
                       f"{w.name}, all {w.Nq} query rows each, "
                       f"{t_total:.1f} s of fp64 NumPy"),
            "seconds": round(t_total, 2)}


def prefill_roofline(w, seqlens, sec):
    """Roofline record of a bf16 prefill-shaped call taking `sec` seconds:
    the bound is whichever of the MFMA time (algorithmic FLOPs at the dense
    bf16 peak) and the HBM time (compulsory bytes at the HBM peak) is
    longer; compulsory bytes are q and o of the live rows, k and v of the
    valid keys (bf16) and lse (fp32)."""
    pairs = allowed_pairs(w, seqlens) * w.Hq
    flops = 4.0 * w.d * pairs
    lens = [w.Nk] * w.B if seqlens is None else \
        [int(min(max(v, 0), w.Nk)) for v in seqlens]
    live_q = sum(L if w.Nq == w.Nk else w.Nq for L in lens)
    byts = float(live_q * w.Hq * (2 * w.d * 2 + 4)
                 + sum(lens) * w.Hkv * 2 * w.d * 2)
    t_mfma = flops / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = byts / (PEAK_HBM_GBS * 1e9)
    if t_hbm > t_mfma:
        ach = byts / sec / 1e9
        return {"bound": "hbm", "achieved": round(ach, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4),
                "algorithmic_bytes_per_launch": byts,
                "algorithmic_flop_per_launch": flops,
                "tflops": round(flops / sec / 1e12, 2)}
    ach = flops / sec / 1e12
    return {"bound": "mfma", "achieved": round(ach, 2),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach / PEAK_BF16_TFLOPS, 4),
            "algorithmic_flop_per_launch": flops,
            "algorithmic_bytes_per_launch": byts}


def shape_str(w):
    return (f"B={w.B} Hq={w.Hq} Hkv={w.Hkv} Nq={w.Nq} Nk={w.Nk} "
            f"d={w.d} causal={w.causal}"
            + (f" window={w.window}" if w.window else "")
            + (f" window_right={w.window_right}" if w.window_right else "")
            + (f" sinks={w.sinks}" if w.sinks else "")
            + (f" L~U[{w.len_lo},{w.len_hi}]" if w.padded else ""))


def run_only(args):
    """One workload's forward call (or the headline's backward pass) alone:
    warmup, then `reps` launches with HIP events around each; one JSON line
    with the trimmed mean.  Meant to run under rocprofv3."""
    import torch
    import synth
    import transformer_self_attention_attn_amd as mi
    mi.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    name = args.only
    bwd = name == "backward"
    f8 = name == "fp8"
    w = synth.by_name("gqa-causal-prefill" if bwd or f8 else name)
    seed = args.seed if args.seed is not None else SEEDS.get(w.name, 0)
    x = synth.make_inputs(w, seed)
    sl = None if x["seqlens"] is None else \
        torch.from_numpy(x["seqlens"]).to(dev)
    q, k, v = x["q"].to(dev), x["k"].to(dev), x["v"].to(dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)

    def fwd(i):
        mi.attn(q, k, v, causal=w.causal, window=w.window, seqlens=sl,
                out=o, lse=lse, window_right=w.window_right, sinks=w.sinks)
    fn = fwd
    if bwd:
        fwd(0)
        gout = synth.make_dout(w, seed)[0].to(dev)
        gq, gk, gv = (torch.empty_like(q), torch.empty_like(k),
                      torch.empty_like(v))

        def fn(i):
            rc = mi.attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                             o.data_ptr(), gout.data_ptr(), lse.data_ptr(),
                             gq.data_ptr(), gk.data_ptr(), gv.data_ptr(),
                             w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.scale,
                             int(w.causal), w.window, w.window_right,
                             w.sinks, 0 if sl is None else sl.data_ptr(),
                             stream.cuda_stream)
            assert rc == mi.MIATTN_OK, mi.attn_last_error()
    if f8:
        # quantize (block scales, Q and K rotated), then the forward on the
        # codes: one launch of each kernel per rep
        sg = torch.from_numpy(synth.make_signs(w.d, seed)).to(dev)

        def fn(i):
            z = mi.fp8_quantize(q, k, v, seqlens=sl, signs=sg)
            mi.attn_fp8(z, causal=w.causal, seqlens=sl, out=o, lse=lse)
    for i in range(args.warmup):
        fn(i)
    torch.cuda.synchronize()
    ev = []
    for i in range(args.reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn(i)
        b.record(stream)
        ev.append((a, b))
    torch.cuda.synchronize()
    prot = trimmed([a.elapsed_time(b) for a, b in ev])
    rec = {"only": name, "seed": seed, "shape": shape_str(w), **prot}
    if not bwd and not f8 and not decode_shaped(w):
        rec["roofline"] = prefill_roofline(w, x["seqlens"],
                                           prot["trimmed_mean_ms"] * 1e-3)
    print(json.dumps(rec), flush=True)


# seeds of the workloads' headline inputs (the first of each one's test seeds)
SEEDS = {"fp32-single-head": 1, "gpt2-small-causal-padded": 2,
         "gqa-causal-prefill": 3, "sliding-window-causal": 4,
         "decode-gqa": 5, "chunk32-gpt2-causal": 16,
         "chunked-prefill-gqa": 17, "cross-attention-padded": 18,
         "local-window-bidirectional": 19, "sliding-window-sinks": 20,
         "decode-window-sinks": 21, "decode-chunk4-gqa": 22}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--reps", type=int, default=1000,
                    help="repetitions of the trimmed-mean latency protocol")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="time the step only (no other configurations, "
                         "backward, FP8, chunks or local windows)")
    ap.add_argument("--only", metavar="WORKLOAD",
                    help="run one workload (or `backward`, or `fp8`: the FP8 "
                         "quantizer and forward on gqa-causal-prefill) alone "
                         "and exit")
    ap.add_argument("--seed", type=int, default=None,
                    help="input seed for --only (default: the workload's)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="after the timed region, copy MIB MiB device to "
                         "device three times (counter calibration)")
    ap.add_argument("--fold-traffic", nargs=2, metavar=("FETCH", "WRITE"),
                    help="fold two counter CSVs into profiles/traffic.json")
    ap.add_argument("--copy-mib", type=int, default=1024,
                    help="size of the probe copy the CSVs hold")
    ap.add_argument("--fold-counters", metavar="CSV",
                    help="print per-kernel counter averages of a rocprofv3 "
                         "counter_collection.csv as JSON")
    args = ap.parse_args()
    if args.fold_counters:
        print(json.dumps(fold_counters(args.fold_counters), indent=1))
        return
    if args.fold_traffic:
        rec = fold_traffic(*args.fold_traffic, args.copy_mib << 20)
        with open(os.path.join(PROFILES, "traffic.json"), "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus "
              f"{args.gpus}); the library has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    if args.only:
        run_only(args)
        return

    import torch
    import synth
    import transformer_self_attention_attn_amd as mi
    mi.load()

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    wp = synth.by_name("gqa-causal-prefill")
    wd = synth.by_name("decode-gqa")
    wf = synth.by_name("fp32-single-head")
    xp = synth.make_inputs(wp, SEEDS[wp.name])
    xd = synth.make_inputs(wd, SEEDS[wd.name])
    xf = synth.make_inputs(wf, SEEDS[wf.name])

    def dev_in(x):
        sl = None
        if x["seqlens"] is not None:
            sl = torch.from_numpy(x["seqlens"]).to(dev)
        return [x["q"].to(dev), x["k"].to(dev), x["v"].to(dev), sl]

    P = dev_in(xp)
    D0 = dev_in(xd)
    # a second copy of the decode cache: consecutive steps alternate between
    # them so a decode step never finds the previous step's K/V in cache
    D1 = [D0[0], D0[1].clone(), D0[2].clone(), D0[3]]
    F = dev_in(xf)
    po = torch.empty_like(P[0])
    pl = torch.empty(P[0].shape[:3], dtype=torch.float32, device=dev)
    do = torch.empty_like(D0[0])
    dl = torch.empty(D0[0].shape[:3], dtype=torch.float32, device=dev)
    fo = torch.empty_like(F[0])
    fl = torch.empty(F[0].shape[:3], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def prefill():
        mi.attn(P[0], P[1], P[2], causal=True, seqlens=P[3], out=po, lse=pl)

    def decode(i):
        Dx = D0 if i % 2 == 0 else D1
        mi.attn(Dx[0], Dx[1], Dx[2], causal=True, seqlens=Dx[3], out=do,
                lse=dl)

    def fp32():
        mi.attn(F[0], F[1], F[2], causal=False, seqlens=F[3], out=fo,
                lse=fl)

    for i in range(args.warmup):
        prefill()
        decode(i)
        fp32()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)]
          for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        e = ev[i]
        e[0].record(stream)
        prefill()
        e[1].record(stream)
        decode(i)
        e[2].record(stream)
        fp32()
        e[3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_ms = [e[0].elapsed_time(e[1]) for e in ev]
    dec_ms = [e[1].elapsed_time(e[2]) for e in ev]
    f32_ms = [e[2].elapsed_time(e[3]) for e in ev]

    flops = 4.0 * wp.d * allowed_pairs(wp, xp["seqlens"]) * wp.Hq
    dbytes = float(decode_bytes(wd, xd["seqlens"]))
    pre_avg = sum(pre_ms) / K
    dec_avg = sum(dec_ms) / K
    tflops = flops / (pre_avg * 1e-3) / 1e12
    gbs = dbytes / (dec_avg * 1e-3) / 1e9

    # latency protocol: R single-call repetitions each, trimmed mean
    def reps(fn):
        out = []
        for i in range(args.reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn(i)
            b.record(stream)
            out.append((a, b))
        torch.cuda.synchronize()
        return trimmed([a.elapsed_time(b) for a, b in out])

    proto_p = reps(lambda i: prefill())
    proto_d = reps(decode)

    # the two other bf16 prefill configurations, each against its roofline
    configs = {}
    if not args.no_extra:
        for name in ("gpt2-small-causal-padded", "sliding-window-causal"):
            w = synth.by_name(name)
            xw = synth.make_inputs(w, SEEDS[name])
            Xw = dev_in(xw)
            ow = torch.empty_like(Xw[0])
            lw = torch.empty(Xw[0].shape[:3], dtype=torch.float32,
                             device=dev)

            def run_c(i, w=w, Xw=Xw, ow=ow, lw=lw):
                mi.attn(Xw[0], Xw[1], Xw[2], causal=w.causal,
                        window=w.window, seqlens=Xw[3], out=ow, lse=lw)
            for i in range(args.warmup):
                run_c(i)
            prot = reps(run_c)
            rec = prefill_roofline(w, xw["seqlens"],
                                   prot["trimmed_mean_ms"] * 1e-3)
            rec.update(kernel=f"prefill_kernel<{w.d}>", seed=SEEDS[name],
                       shape=shape_str(w), latency_protocol=prot)
            configs[name] = rec
            del Xw, ow, lw

    # backward pass of the headline prefill: dQ, dK, dV from the forward's
    # o and lse and a seeded dO (all three kernels of one attn_bwd call);
    # algorithmic FLOPs 2.5x the forward's (10*d per allowed pair)
    bwd = None
    if not args.no_extra:
        prefill()
        gout = synth.make_dout(wp, SEEDS[wp.name])[0].to(dev)
        gq, gk, gv = (torch.empty_like(P[0]), torch.empty_like(P[1]),
                      torch.empty_like(P[2]))
        sptr = stream.cuda_stream

        def backward(i):
            rc = mi.attn_bwd(P[0].data_ptr(), P[1].data_ptr(),
                             P[2].data_ptr(), po.data_ptr(), gout.data_ptr(),
                             pl.data_ptr(), gq.data_ptr(), gk.data_ptr(),
                             gv.data_ptr(), wp.B, wp.Hq, wp.Hkv, wp.Nq,
                             wp.Nk, wp.d, wp.scale, 1, 0, 0, 0, 0, sptr)
            assert rc == mi.MIATTN_OK, mi.attn_last_error()
        for i in range(args.warmup):
            backward(i)
        protb = reps(backward)
        bfl = 2.5 * flops
        btf = bfl / (protb["trimmed_mean_ms"] * 1e-3) / 1e12
        bwd = {"value": round(btf, 2), "unit": "TFLOP/s",
               "frac": round(btf / PEAK_BF16_TFLOPS, 4),
               "algorithmic_flop_per_launch": bfl,
               "trimmed_mean_ms": round(protb["trimmed_mean_ms"], 5),
               "kernels": "bwd_pre_kernel + bwd_dkdv_kernel + bwd_dq_kernel",
               "workload": "gqa-causal-prefill, dO = N(0,1) seed [3, 1]"}
        del gout, gq, gk, gv

    # FP8 forward of the headline prefill: operands quantized once (block
    # scales, Q and K rotated), then the forward kernel on the codes alone;
    # algorithmic FLOPs as for bf16, against the dense FP8 peak
    fp8 = None
    if not args.no_extra:
        sg = torch.from_numpy(synth.make_signs(wp.d, 3)).to(dev)

        def quant(i):
            return mi.fp8_quantize(P[0], P[1], P[2], seqlens=P[3], signs=sg)
        z = quant(0)
        fo8 = torch.empty_like(P[0])
        fl8 = torch.empty(P[0].shape[:3], dtype=torch.float32, device=dev)

        def fwd8(i):
            mi.attn_fp8(z, causal=True, seqlens=P[3], out=fo8, lse=fl8)
        for i in range(args.warmup):
            fwd8(i)
        prot8 = reps(fwd8)
        protq = reps(quant)
        tf8 = flops / (prot8["trimmed_mean_ms"] * 1e-3) / 1e12
        fp8 = {"value": round(tf8, 2), "unit": "TFLOP/s",
               "frac": round(tf8 / PEAK_FP8_TFLOPS, 4),
               "peak": PEAK_FP8_TFLOPS,
               "algorithmic_flop_per_launch": flops,
               "trimmed_mean_ms": round(prot8["trimmed_mean_ms"], 5),
               "quantize_ms": round(protq["trimmed_mean_ms"], 5),
               "kernel": "attn_fp8_kernel<128, 4>",
               "workload": "gqa-causal-prefill, E4M3 codes with 64-row "
                           "block scales, Q and K rotated"}
        del z, fo8, fl8

    # Nq new rows against a longer key sequence, and the local-window
    # variants: each workload on its own, `reps` launches, HIP events around
    # each; decode shapes in GB/s, the others in TFLOP/s
    extra, masks = {}, {}
    if not args.no_extra:
        for name in ("decode-chunk4-gqa", "chunked-prefill-gqa",
                     "cross-attention-padded", "chunk32-gpt2-causal",
                     "local-window-bidirectional", "sliding-window-sinks",
                     "decode-window-sinks"):
            w = synth.by_name(name)
            xw = synth.make_inputs(w, SEEDS[name])
            Xw = dev_in(xw)
            ow = torch.empty_like(Xw[0])
            lw = torch.empty(Xw[0].shape[:3], dtype=torch.float32, device=dev)

            def run_w(i, w=w, Xw=Xw, ow=ow, lw=lw):
                mi.attn(Xw[0], Xw[1], Xw[2], causal=w.causal,
                        window=w.window, seqlens=Xw[3], out=ow, lse=lw,
                        window_right=w.window_right, sinks=w.sinks)
            for i in range(args.warmup):
                run_w(i)
            prot = reps(run_w)
            sec = prot["trimmed_mean_ms"] * 1e-3
            if decode_shaped(w):
                by = float(decode_bytes(w, xw["seqlens"]))
                rec = {"value": round(by / sec / 1e9, 1), "unit": "GB/s",
                       "frac": round(by / sec / 1e9 / PEAK_HBM_GBS, 4),
                       "algorithmic_bytes_per_launch": by}
            else:
                fl = 4.0 * w.d * allowed_pairs(w, xw["seqlens"]) * w.Hq
                rec = {"value": round(fl / sec / 1e12, 2), "unit": "TFLOP/s",
                       "frac": round(fl / sec / 1e12 / PEAK_BF16_TFLOPS, 4),
                       "algorithmic_flop_per_launch": fl}
            rec["trimmed_mean_ms"] = round(prot["trimmed_mean_ms"], 5)
            rec["shape"] = shape_str(w)
            local = w.window or w.window_right or w.sinks
            (masks if local else extra)[name] = rec
            del Xw, ow, lw

    if args.copy_probe:
        n = (args.copy_probe << 20) // 2
        src = torch.ones(n, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded normal draws; no dataset or weights)",
        "config": {
            "workload": ("gqa-causal-prefill: B=4 Hq=28 Hkv=4 N=4096 d=128 "
                         "bf16 causal, Q/K/V = 0.5*N(0,1), seed 3; the step "
                         "also runs decode-gqa (B=64 Hq=32 Hkv=8 d=128 bf16, "
                         "cache lengths U[2048,8192], seed 5) and "
                         "fp32-single-head (B=1 H=1 N=128 d=64)"),
            "global_batch": wp.B,
            "seq_len": wp.Nq,
            "parallelism": "none (one GPU)",
        },
        "device": {"name": props.name,
                   "arch": getattr(props, "gcnArchName", None),
                   "compute_units": props.multi_processor_count},
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic_for("prefill"),
            "kernel": "prefill_kernel<128>",
            "algorithmic_flop_per_launch": flops,
            "avg_launch_ms": round(pre_avg, 5),
        },
        "decode": {
            "value": round(gbs, 1),
            "unit": "GB/s",
            "roofline": {
                "bound": "hbm",
                "achieved": round(gbs, 1),
                "peak": PEAK_HBM_GBS,
                "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4),
                "traffic": traffic_for("decode"),
                "kernels": "decode_split_kernel<128> + "
                           "decode_combine_kernel<128>",
                "algorithmic_bytes_per_launch": dbytes,
                "avg_launch_ms": round(dec_avg, 5),
            },
        },
        "fp32_case_avg_ms": round(sum(f32_ms) / K, 5),
        "latency_protocol": {"prefill": proto_p, "decode": proto_d},
    }
    if configs:
        line["configs"] = configs
    if bwd:
        line["backward"] = bwd
    if fp8:
        line["fp8"] = fp8
    if extra:
        line["nq_lt_nk"] = extra
    if masks:
        line["local_windows"] = masks
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wp, xp)
        line["cpu_baseline"]["gpu_over_cpu"] = round(
            tflops / line["cpu_baseline"]["value"], 1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
