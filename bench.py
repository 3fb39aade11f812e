"""Benchmark of the KDA hot path on one MI355X.

One step = one chunked prefill over the prefill workload (chunk table,
intra-chunk kernel, scan kernel) followed by one fused decode step over the
decode workload — every stage of the path once.  Inputs are synthetic,
seeded, generated on the GPU and resident in HBM before timing starts.

Prints ONE JSON line:
  value        prefill tokens/s (tokens of the prefill workload, all heads)
               from HIP events around the library call, averaged over steps
  decode       decode sequence-steps/s over the 64-step decode trajectory run
               back to back (HIP events around the 64 calls); the figure for
               the decode step inside each timed step is reported beside it
  roofline     prefill: algorithmic HBM bytes / average call duration vs 8 TB/s,
               and vs what torch's plain 512 MiB device copy reaches in the same run
  prologue     the same prefill from raw pre-activations (softplus decay gate,
               sigmoid write gate and q/k L2 norm fused into the kernels)
  decode_multi 4 tokens per sequence per launch (multi-token decode), with
               and without the per-token states written for rollback
  short_conv   the width-4 causal convolution over a q-shaped prefill input
               and over one decode token per sequence (state rolled in place)
  backward     gradients over the T=4096, H=16 prefill shape: the prefill that
               writes the chunk checkpoints plus the chunked backward
  prefill_fp32 the same shape with fp32 inputs (1e-5 contract), chunk 64
  cpu_baseline the fp64 CPU oracle on a bounded sample of the same workload

  prefill_workloads  the T=4096, H=16 prefill and the packed 8-document
               prefill (H=32), each timed per call over >= 20 repetitions
               with a 512 MiB write between them (so their ~100 MB-2 GB
               working sets are not served from the 256 MB last-level cache)
  every per-call figure carries median, min, max and mean over its repetitions

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
                       [--workload long|prefill|packed] [--no-cpu-baseline]
       python bench.py --leg prefill_long|prefill_c2|prefill_c4|prefill_f32|decode|decode_multi|short_conv|backward
                       [--steps K] [--warmup W]
                       only that workload's calls (one rocprofv3 trace per workload)
       python bench.py --summarize DIR    per-kernel means of a rocprofv3 CSV run
       python bench.py --copy-calibration one 1 GiB device copy (counter scale)
       python bench.py --steps S --warmup W --record-traffic FETCH WRITE SQ CAL_FETCH CAL_WRITE MFMA
                        profiles/traffic.json from rocprofv3 --pmc result folders

`roofline.traffic` is filled from profiles/traffic.json (HBM bytes per call
measured with rocprofv3 FETCH_SIZE / WRITE_SIZE, scaled by the same counters
on a plain 1 GiB copy) while the sources of that call's kernels still hash to
the recorded value, else null.
"""
from __future__ import annotations

import argparse
import csv
import ctypes
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s + decode seq-steps/s @H=32,d=128; % MFMA / HBM peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP32_PEAK_TFLOPS = 157.3   # dense fp32 matrix cores
# Algorithmic bytes per (token, head): q, k, v, log_alpha in bf16 (4 x 256 B),
# beta (2 B), o in fp32 (512 B).
PREFILL_BYTES_PER_TOKEN_HEAD = 4 * 128 * 2 + 2 + 128 * 4
# Decode per (sequence, head, step): fp32 state read + write plus the same I/O.
DECODE_BYTES_PER_SEQ_HEAD = 2 * 128 * 128 * 4 + PREFILL_BYTES_PER_TOKEN_HEAD


def chunk_flops_per_token_head(C=64, d=128):
    """Useful flops of the chunked form per (token, head): Gram A and P
    (2 C d each, halved by triangularity counted as full here), W and U
    (2 C d each), and the state-side W S, (q e^G) S, P Delta, K^T Delta:
    10 C d + 6 d^2 in total."""
    return 10 * C * d + 6 * d * d


# Kernel sources behind each measured call: a recorded counter stays valid
# only while its group's sources (and the shared device headers) are unchanged.
SOURCE_GROUPS = {
    "prefill": ["kda_prefill_mfma.hip", "kda_prefill_table.hip", "kda_handoff.hpp"],
    "decode": ["kda_decode.hip"],
    "short_conv": ["kda_conv.hip"],
    "backward": ["kda_backward_chunked.hip", "kda_prefill_table.hip", "kda_chunk_block.hpp", "kda_chunk_prep.hpp"],
}
SHARED_HEADERS = ["kda_common.hpp", "kda_prefill_common.hpp", "kda_launch.hpp"]
# call key in profiles/traffic.json -> source group
CALL_GROUPS = {"prefill_long": "prefill", "decode": "decode", "decode_multi_m4": "decode",
               "short_conv_prefill": "short_conv", "short_conv_decode": "short_conv",
               "backward_T4096_H16": "backward"}
# kernels of each call key, as rocprofv3 names them (without namespace, spaces and arguments)
CALL_KERNELS = {
    "prefill_long": ["intra_kernel<64,128>", "scan_kernel<64,128,float,1>", "chunk_table_kernel"],
    "decode": ["decode1_kernel<128,128,unsignedshort,float>"],
    "decode_multi_m4": ["decodec_kernel<128,128,unsignedshort,float,4>"],
    "short_conv_prefill": ["short_conv_kernel<unsignedshort,unsignedshort,4,16>", "conv_state_kernel<unsignedshort,4>"],
    "short_conv_decode": ["conv_rows_kernel<unsignedshort,unsignedshort,4>"],
    "backward_T4096_H16": ["cb_prep_kernel<128,unsignedshort,false>", "cb_scan_kernel<128>",
                           "cb_grad_kernel<128,unsignedshort>"],
}
# call keys whose kernels each `--leg` runs
LEG_CALLS = {"prefill_long": ["prefill_long"], "decode": ["decode"], "decode_multi": ["decode_multi_m4"],
             "backward": ["backward_T4096_H16"], "short_conv": ["short_conv_prefill", "short_conv_decode"]}


def kernel_sources_sha(group: str) -> str:
    """sha256 over the HIP sources of one kernel group (what its counters were
    taken on)."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "gated_delta_rule_49_amd", "csrc")
    for f in sorted(SOURCE_GROUPS[group]) + SHARED_HEADERS:
        h.update(f.encode())
        h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()


def _traffic_record():
    try:
        return json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    except (OSError, ValueError):
        return None


def measured_traffic(key):
    """HBM bytes per call for `key` from profiles/traffic.json, or None if the
    record is missing or was taken on different kernel sources."""
    rec = _traffic_record()
    group = CALL_GROUPS.get(key)
    if rec is None or group is None or key not in rec.get("calls", {}):
        return None
    if rec.get("sources_sha", {}).get(group) != kernel_sources_sha(group):
        return None
    c = rec["calls"][key]
    return c["fetch_kib"] * 1024 * rec["fetch_scale"] + c["write_kib"] * 1024 * rec["write_scale"]


def measured_counter(kernel, counter, group="prefill"):
    """Per-dispatch value of a rocprofv3 counter for `kernel` recorded in
    profiles/traffic.json ("counters"), or None if missing or taken on
    different kernel sources."""
    rec = _traffic_record()
    if rec is None or rec.get("sources_sha", {}).get(group) != kernel_sources_sha(group):
        return None
    return rec.get("counters", {}).get(kernel, {}).get(counter)


def _counter_runs(dirs):
    """{(kernel, counter): [per-dispatch values in launch order]} over the
    rocprofv3 --pmc result folders `dirs`; kernel names without spaces, the
    namespace or the argument list."""
    acc = {}
    for root in dirs:
        for f in glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True):
            rows = list(csv.DictReader(open(f)))
            if rows and "Dispatch_Id" in rows[0]:
                rows.sort(key=lambda r: int(r["Dispatch_Id"]))
            for row in rows:
                name = row["Kernel_Name"].split("(")[0].replace("void ", "").replace("kda::", "")
                acc.setdefault((name.replace(" ", ""), row["Counter_Name"]), []).append(float(row["Counter_Value"]))
    return acc


# bytes a plain copy of 1 GiB (`--copy-calibration`) reads and writes
COPY_CAL_KIB = float(1 << 20)


def record_traffic(fetch_dir, write_dir, sq_dir, cal_fetch_dir, cal_write_dir, mfma_dir, calls):
    """Write profiles/traffic.json from rocprofv3 --pmc runs: FETCH_SIZE,
    WRITE_SIZE and SQ instruction counters of `bench.py --steps S --warmup W
    --no-cpu-baseline`, and FETCH_SIZE, WRITE_SIZE of `bench.py
    --copy-calibration` (which fix the counters' scale), and the matrix-core
    counters (SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_*,
    GRBM_GUI_ACTIVE) of the bench in `mfma_dir`.  `calls` = W + S
    plain prefill calls, which come first in launch order (the fused-prologue
    calls and the backward's checkpoint prefill follow and are left out)."""
    acc = _counter_runs([fetch_dir, write_dir, sq_dir, mfma_dir])
    cal = _counter_runs([cal_fetch_dir, cal_write_dir])

    def mean(table, kernel, counter, first=None):
        v = table.get((kernel, counter))
        if not v:
            raise SystemExit(f"no {counter} dispatches of {kernel} in the counter runs")
        v = v[:first] if first else v
        return sum(v) / len(v)

    fetch_scale = COPY_CAL_KIB / mean(cal, "__amd_rocclr_copyBuffer", "FETCH_SIZE")
    write_scale = COPY_CAL_KIB / mean(cal, "__amd_rocclr_copyBuffer", "WRITE_SIZE")
    groups = {key: [(k, calls if key == "prefill_long" else None) for k in ks]
              for key, ks in CALL_KERNELS.items()}
    out_calls = {}
    for key, ks in groups.items():
        per = {k: [mean(acc, k, "FETCH_SIZE", n), mean(acc, k, "WRITE_SIZE", n)] for k, n in ks}
        out_calls[key] = {"fetch_kib": sum(v[0] for v in per.values()),
                          "write_kib": sum(v[1] for v in per.values()), "kernels": per}
    counters = {}
    for k in ("intra_kernel<64,128>", "scan_kernel<64,128,float,1>"):
        counters[k] = {c: mean(acc, k, c, calls) for (kk, c) in acc
                       if kk == k and (c.startswith("SQ_") or c == "GRBM_GUI_ACTIVE")}
    rec = {"what": "HBM bytes per call = FETCH_SIZE KiB * 1024 * fetch_scale + WRITE_SIZE KiB * 1024 * "
                   "write_scale, means over dispatches of rocprofv3 --pmc runs of bench.py; the scales make "
                   "the counters read 1 GiB each way on a plain 1 GiB device copy. counters: per-dispatch SQ "
                   "counters of the plain prefill calls. A call is valid while its kernel group's sources "
                   "hash to sources_sha (bench.py SOURCE_GROUPS).",
           "sources_sha": {g: kernel_sources_sha(g) for g in SOURCE_GROUPS},
           "fetch_scale": fetch_scale, "write_scale": write_scale,
           "calls": out_calls, "counters": counters}
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps({"fetch_scale": fetch_scale, "write_scale": write_scale,
                      **{k: (v["fetch_kib"] * fetch_scale + v["write_kib"] * write_scale) * 1024 / 1e9
                         for k, v in out_calls.items()}}))


def record_prefill_traffic(fetch_dir, write_dir, sq_dir, mfma_dir, calls):
    """Refresh the long-prefill entry of profiles/traffic.json (its HBM bytes
    and the prefill kernels' SQ / matrix-core counters) from rocprofv3 --pmc
    runs of `bench.py --leg prefill_long --steps S --warmup W` (calls = W + S
    plain prefill calls), keeping the other entries and the copy calibration
    already recorded."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    rec = json.load(open(path))
    acc = _counter_runs([fetch_dir, write_dir, sq_dir, mfma_dir])

    def mean(kernel, counter):
        v = acc.get((kernel, counter))
        if not v:
            raise SystemExit(f"no {counter} dispatches of {kernel} in the counter runs")
        v = v[:calls]
        return sum(v) / len(v)

    ks = ["intra_kernel<64,128>", "scan_kernel<64,128,float,1>", "chunk_table_kernel"]
    per = {k: [mean(k, "FETCH_SIZE"), mean(k, "WRITE_SIZE")] for k in ks}
    rec["calls"]["prefill_long"] = {"fetch_kib": sum(v[0] for v in per.values()),
                                    "write_kib": sum(v[1] for v in per.values()), "kernels": per}
    rec["counters"] = {k: {c: mean(k, c) for (kk, c) in acc if kk == k and (c.startswith("SQ_") or
                                                                          c == "GRBM_GUI_ACTIVE")}
                       for k in ks[:2]}
    rec["sources_sha"]["prefill"] = kernel_sources_sha("prefill")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    v = rec["calls"]["prefill_long"]
    print(json.dumps({"prefill_long_gb": (v["fetch_kib"] * rec["fetch_scale"] + v["write_kib"] * rec["write_scale"])
                      * 1024 / 1e9}))


def record_leg_traffic(leg, fetch_dir, write_dir):
    """Refresh the entries of profiles/traffic.json for the calls that
    `bench.py --leg LEG` runs, from a FETCH_SIZE and a WRITE_SIZE rocprofv3
    --pmc run of that leg (every dispatch of the call's kernels averaged),
    keeping the other entries and the copy calibration already recorded."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    rec = json.load(open(path))
    acc = _counter_runs([fetch_dir, write_dir])

    def mean(kernel, counter):
        v = acc.get((kernel, counter))
        if not v:
            raise SystemExit(f"no {counter} dispatches of {kernel} in the counter runs")
        return sum(v) / len(v)

    res = {}
    for key in LEG_CALLS[leg]:
        per = {k: [mean(k, "FETCH_SIZE"), mean(k, "WRITE_SIZE")] for k in CALL_KERNELS[key]}
        rec["calls"][key] = {"fetch_kib": sum(v[0] for v in per.values()),
                             "write_kib": sum(v[1] for v in per.values()), "kernels": per}
        rec["sources_sha"][CALL_GROUPS[key]] = kernel_sources_sha(CALL_GROUPS[key])
        c = rec["calls"][key]
        res[key + "_gb"] = (c["fetch_kib"] * rec["fetch_scale"] + c["write_kib"] * rec["write_scale"]) * 1024 / 1e9
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(res))


# Vector-ALU issue peak of MI355X: 256 CUs x 4 SIMDs, one wave64 VALU
# instruction per SIMD every 4 cycles (16 lanes), at 2.4 GHz, counted in
# lane-operations (64 per wave instruction).
VALU_PEAK_TLANEOPS = 256 * 4 * 16 * 2.4e9 / 1e12


def summarize(root):
    """Per-kernel means of rocprofv3 --output-format csv results under root."""
    for f in glob.glob(os.path.join(root, "**", "*kernel_stats.csv"), recursive=True):
        print(f"# kernel stats ({os.path.basename(f)})")
        print("| kernel | calls | average | total |\n|---|---|---|---|")
        other = [0, 0.0]
        for row in csv.DictReader(open(f)):
            if "kda::" not in row["Name"]:  # input generation and copies
                other[0] += int(row["Calls"])
                other[1] += float(row["TotalDurationNs"])
                continue
            print(f"| {row['Name'].split('(')[0]} | {row['Calls']} | "
                  f"{float(row['AverageNs']) / 1e3:.1f} us | {float(row['TotalDurationNs']) / 1e6:.3f} ms |")
        print(f"| (other kernels: input generation, copies) | {other[0]} | | {other[1] / 1e6:.3f} ms |")
    # per-dispatch durations in launch order: the bench runs the plain prefill
    # (warmup + steps calls) before the fused-prologue prefill, and the
    # state-only multi-token decodes before those that write per-token states
    for f in glob.glob(os.path.join(root, "**", "*kernel_trace.csv"), recursive=True):
        per = {}
        for row in sorted(csv.DictReader(open(f)), key=lambda r: int(r["Start_Timestamp"])):
            if "kda::" in row["Kernel_Name"]:
                per.setdefault(row["Kernel_Name"].split("(")[0], []).append(
                    (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3)
        print("# dispatch durations in launch order (us)")
        for k, v in per.items():
            shown = " ".join(f"{x:.0f}" for x in v[:40]) + (" ..." if len(v) > 40 else "")
            print(f"- {k}: {shown}")
    acc = {}
    for f in glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True):
        rows = list(csv.DictReader(open(f)))
        key = "Dispatch_Id" if rows and "Dispatch_Id" in rows[0] else None
        if key:
            rows.sort(key=lambda r: int(r[key]))
        for row in rows:
            name = row["Kernel_Name"]
            if "kda::" not in name and "copyBuffer" not in name:
                continue
            acc.setdefault((name.split("(")[0], row["Counter_Name"]), []).append(float(row["Counter_Value"]))
    if acc:
        print("# counters (mean per dispatch)")
        print("| kernel | counter | dispatches | mean |\n|---|---|---|---|")
        for (k, c), v in sorted(acc.items()):
            print(f"| {k} | {c} | {len(v)} | {sum(v) / len(v):.6g} |")
        print("# counter values per dispatch in launch order (kda kernels, first 12)")
        for (k, c), v in sorted(acc.items()):
            if "kda::" in k:
                print(f"- {k} {c}: " + " ".join(f"{x:.6g}" for x in v[:12]))


def stats(xs):
    """median / min / max / mean of per-call durations (ms)."""
    ys = sorted(xs)
    n = len(ys)
    med = ys[n // 2] if n % 2 else 0.5 * (ys[n // 2 - 1] + ys[n // 2])
    return {"median": med, "min": ys[0], "max": ys[-1], "mean": sum(ys) / n, "n": n}


def host_cpu():
    """Model name of the host CPU and the number of cores this process may use."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"model": model, "cores_available": len(os.sched_getaffinity(0)),
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


class CacheFlush:
    """Writes a 512 MiB device buffer (twice the 256 MB last-level cache of an
    MI355X) so that the next call's inputs come from HBM."""

    def __init__(self, dev):
        import torch
        self.buf = torch.empty(1 << 27, dtype=torch.float32, device=dev)
        self.n = 0

    def __call__(self):
        self.n += 1
        self.buf.fill_(float(self.n))


def copy_calibration():
    import torch
    n = 1 << 28  # floats: 1 GiB
    a = torch.ones(n, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print("copied 3 x 1 GiB device to device")


class HipEvents:
    """Minimal ctypes access to hipEvent* so the library can record events on
    the stream its kernels run on."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            rc = self.lib.hipEventCreate(ctypes.byref(h))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed: {rc}")
            arr[i] = h
        return arr

    def ms(self, a, b):
        out = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(out), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(out.value)


def prefill_inputs(name, dev):
    import numpy as np
    import torch
    import synth
    if name == "long":
        ts = synth.long_tensors(5, 131072, 32, 128, 128, "bf16", True, dev)
        q, k, v, b, la = (t.to(torch.bfloat16) for t in ts)
        del ts
        return dict(workload="long_T131072_H32_d128_extreme", q=q, k=k, v=v, beta=b, log_alpha=la,
                    init=None, cu=None, cu_host=None, chunk=64)
    x = synth.workload(2 if name == "prefill" else 4, device=dev)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev, torch.bfloat16)  # noqa: E731
    init = None if x.initial_state is None else torch.from_numpy(x.initial_state).to(dev)
    cu = None if x.cu_seqlens is None else torch.from_numpy(x.cu_seqlens).to(dev)
    return dict(workload=x.name, q=t(x.q), k=t(x.k), v=t(x.v), beta=t(x.beta), log_alpha=t(x.log_alpha),
                init=init, cu=cu, cu_host=x.cu_seqlens, chunk=x.chunk_size)


def prefill_leg(kda, name, dev, reps, warmup, flush):
    """Per-call timing of one prefill workload: warmup calls, then ``reps``
    calls each preceded by a cache flush (untimed) and bracketed by HIP events
    on the stream the library launches on (torch's current stream)."""
    import torch
    P = prefill_inputs(name, dev)
    Bp, T, H, d = P["q"].shape
    N = Bp if P["cu"] is None else P["cu"].numel() - 1
    ws = torch.empty(kda.workspace_bytes(P["q"], P["k"], P["v"], P["beta"], P["log_alpha"], P["cu"],
                                         P["chunk"]), dtype=torch.uint8, device=dev)
    o = torch.empty((Bp, T, H, d), dtype=torch.float32, device=dev)
    fin = torch.empty((N, H, d, d), dtype=torch.float32, device=dev)
    # cu_seqlens validated once on the host; the timed calls do not synchronise
    kda.prefill(P["q"], P["k"], P["v"], P["beta"], P["log_alpha"], initial_state=P["init"],
                cu_seqlens=P["cu"], chunk_size=P["chunk"], workspace=ws, o=o, final_state=fin,
                check_seqlens=True)

    def call():
        kda.prefill(P["q"], P["k"], P["v"], P["beta"], P["log_alpha"], initial_state=P["init"],
                    cu_seqlens=P["cu"], chunk_size=P["chunk"], workspace=ws, o=o, final_state=fin,
                    check_seqlens=False)

    def timed():
        for _ in range(warmup):
            call()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a_, b_ in evs:
            if flush is not None:
                flush()
            a_.record()
            call()
            b_.record()
        torch.cuda.synchronize()
        return stats([a_.elapsed_time(b_) for a_, b_ in evs])
    st = timed()
    # one sequence with few heads runs both stages in one overlapped launch
    # (the library's own choice); the two-kernel launch is timed beside it
    overlapped = N == 1 and P["chunk"] == 64 and (H + 7) // 8 * (d // 16) <= 16
    two_kernel = None
    if overlapped:
        saved = os.environ.get("KDA_PREFILL_OVERLAP")
        os.environ["KDA_PREFILL_OVERLAP"] = "0"
        try:
            two_kernel = timed()
        finally:
            if saved is None:
                del os.environ["KDA_PREFILL_OVERLAP"]
            else:
                os.environ["KDA_PREFILL_OVERLAP"] = saved
    tokens = int(P["cu_host"][-1]) if P["cu_host"] is not None else Bp * T
    nbytes = tokens * H * PREFILL_BYTES_PER_TOKEN_HEAD + (2 * N * H * d * d * 4 if P["init"] is not None else 0)
    gbs = nbytes / (st["median"] * 1e-3) / 1e9
    useful_tf = tokens * H * chunk_flops_per_token_head(P["chunk"], d) / (st["median"] * 1e-3) / 1e12
    out = {"value": tokens / (st["median"] * 1e-3), "unit": "tokens/s", "workload": P["workload"],
           "tokens": tokens, "H": H, "num_seqs": N, "ms": st,
           "cache_flush": "512 MiB device write before every timed call" if flush is not None else None,
           "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes": nbytes,
                        "useful_mfma_frac": useful_tf / BF16_PEAK_TFLOPS,
                        "kernel": ("kda_prefill_chunked (chunk table + overlap_kernel: both stages in one launch)"
                                   if overlapped else
                                   "kda_prefill_chunked (chunk table + intra_kernel + scan_kernel)")}}
    if two_kernel is not None:
        out["two_kernel_launch_ms"] = two_kernel
    del P, ws, o, fin
    return out


def cpu_baseline_prefill(P, target_s=12.0):
    """The fp64 oracle on the first S tokens of every head of the prefill
    workload (S sized for ~target_s of CPU work)."""
    import numpy as np
    from oracle import native
    q, k, v, b, la = (P[n] for n in ("q", "k", "v", "beta", "log_alpha"))
    T, H = q.shape[1], q.shape[2]
    cu = P["cu_host"]

    def host(a, S):
        return a[:, :S].float().cpu().numpy()

    def run(S):
        arrs = [host(a, S) for a in (q, k, v, b, la)]
        init = None
        cus = None
        if cu is not None:  # the documents that lie inside the sample
            ends = [int(e) for e in cu[1:] if e <= S] or [S]
            S = ends[-1]
            arrs = [a[:, :S] for a in arrs]
            cus = np.array([0] + ends, np.int64)
            if P["init"] is not None:
                init = P["init"][:len(ends)].cpu().numpy()
        t = time.perf_counter()
        native.prefill(*arrs, cu_seqlens=cus, initial_state=init)
        return time.perf_counter() - t, S

    dt, S = run(min(T, 2048))
    S2 = int(min(T, max(2048, S * target_s / max(dt, 1e-3))))
    if S2 > S:
        dt, S = run(S2)
    # the same recurrence on one thread, first S1 tokens of all heads (~4 s)
    arrs1 = [host(a, 256) for a in (q, k, v, b, la)]
    t1 = time.perf_counter()
    native.prefill(*arrs1, nthreads=1)
    d1 = time.perf_counter() - t1
    S1 = int(min(T, max(256, 256 * 4.0 / max(d1, 1e-3))))
    arrs1 = [host(a, S1) for a in (q, k, v, b, la)]
    t1 = time.perf_counter()
    native.prefill(*arrs1, nthreads=1)
    d1 = time.perf_counter() - t1
    return dict(value=S / dt, unit="tokens/s", cores=native.max_threads(), kind="oracle",
                sample=f"first {S} of {T} tokens, all {H} heads, fp64 token-by-token recurrence "
                       f"({dt:.1f} s)",
                one_thread={"value": S1 / d1, "unit": "tokens/s", "cores": 1,
                            "sample": f"first {S1} of {T} tokens, all {H} heads ({d1:.1f} s)"},
                host_cpu=host_cpu())


def cpu_baseline_decode(D):
    from oracle import native
    import numpy as np
    B = D["q"].shape[1]
    args = [D[n][0].float().cpu().numpy()[None] for n in ("q", "k", "v", "beta", "log_alpha")]
    init = D["state0"].cpu().numpy()
    t = time.perf_counter()
    native.prefill(*args, cu_seqlens=np.arange(B + 1), initial_state=init)
    dt = time.perf_counter() - t
    return dict(value=B / dt, unit="seq-steps/s", cores=native.max_threads(), kind="oracle",
                sample=f"one step of all {B} sequences x {D['q'].shape[2]} heads ({dt:.2f} s)")


def intra_valu(intra_ms):
    """The intra-chunk kernel's own roofline: it is bound by vector-ALU issue.
    VALU wave-instructions per call (rocprofv3 SQ_INSTS_VALU, recorded in
    profiles/traffic.json) x 64 lanes / the live kernel time, against the
    issue peak; null when the record does not match the sources."""
    n = measured_counter("intra_kernel<64,128>", "SQ_INSTS_VALU")
    if n is None:
        return None
    achieved = n * 64 / (intra_ms * 1e-3) / 1e12
    return {"bound": "alu", "achieved": achieved, "peak": VALU_PEAK_TLANEOPS, "unit": "T lane-op/s",
            "frac": achieved / VALU_PEAK_TLANEOPS, "valu_wave_insts": n,
            "peak_basis": "256 CU x 4 SIMD x 16 lanes x 2.4 GHz (one wave64 instruction per 4 cycles)"}


def mfma_busy(kernel_ms):
    """rocprofv3 matrix-core utilisation of the prefill kernels: busy cycles
    of the MFMA units summed over the 1024 SIMDs (SQ_VALU_MFMA_BUSY_CYCLES)
    over 1024 x the active cycles of one XCD (GRBM_GUI_ACTIVE summed over the
    8 XCDs / 8), and the MFMA flops issued (SQ_INSTS_VALU_MFMA_MOPS_* x 512)
    per live kernel time; null when the record does not match the sources."""
    out = {}
    for name, key in (("intra_kernel", "intra_kernel<64,128>"), ("scan_kernel", "scan_kernel<64,128,float,1>")):
        busy = measured_counter(key, "SQ_VALU_MFMA_BUSY_CYCLES")
        active = measured_counter(key, "GRBM_GUI_ACTIVE")
        if busy is None or active is None:
            return None
        mops = sum(measured_counter(key, f"SQ_INSTS_VALU_MFMA_MOPS_{t}") or 0.0 for t in ("BF16", "F32"))
        out[name] = {"busy_frac": busy / (active / 8 * 1024),
                     "issued_tflops": mops * 512 / (kernel_ms[name] * 1e-3) / 1e12}
    out["source"] = ("rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 "
                     "SQ_INSTS_VALU_MFMA_MOPS_F32 GRBM_GUI_ACTIVE, plain prefill calls")
    return out


def _decode_into(kda, mt, state, om, tsb):
    """kda.decode writing the per-token states into a preallocated buffer
    (the binding allocates them otherwise)."""
    a = kda.DecodeArgs()
    B, m, H, d = mt["q"].shape
    a.B, a.H, a.d_k, a.d_v, a.n_tokens = B, H, d, d, m
    a.in_dtype, a.out_dtype, a.prologue = kda.KDA_BF16, kda.KDA_F32, 0
    a.q, a.k, a.v, a.beta, a.log_alpha = (ctypes.c_void_p(mt[n].data_ptr())
                                          for n in ("q", "k", "v", "beta", "log_alpha"))
    a.initial_state = a.final_state = ctypes.c_void_p(state.data_ptr())
    a.token_states = ctypes.c_void_p(tsb.data_ptr())
    a.o = ctypes.c_void_p(om.data_ptr())
    import torch
    st = kda.lib().kda_decode(ctypes.byref(a), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if st != 0:
        raise kda.KDAError(st, "kda_decode")


def run_leg(kda, args, dev):
    """One workload's calls only (warmup + steps), for a rocprofv3 trace whose
    per-kernel averages are per-call figures of that workload."""
    import torch
    from synth.kda_inputs import _draw_tokens, _gen, _state
    if args.leg in ("prefill_long", "prefill_c2", "prefill_c4"):
        name = {"prefill_long": "long", "prefill_c2": "prefill", "prefill_c4": "packed"}[args.leg]
        r = prefill_leg(kda, name, dev, reps=args.steps, warmup=args.warmup, flush=None)
        print(json.dumps({"leg": args.leg, "workload": r["workload"], "ms": r["ms"], "value": r["value"],
                          "unit": r["unit"], "kernel": r["roofline"]["kernel"],
                          "two_kernel_launch_ms": r.get("two_kernel_launch_ms")}), flush=True)
        return
    if args.leg == "decode":
        gg = _gen(3, dev)
        dq, dk_, dv_, db, dla = (t.to(torch.bfloat16) for t in _draw_tokens(gg, 64, 256, 32, 128, 128, 0.0,
                                                                               dev, True))
        state = _state(gg, (256, 32, 128, 128), 0.02, dev)
        od = torch.empty((256, 32, 128), dtype=torch.float32, device=dev)
        evs = []
        for i in range(args.warmup + args.steps):
            s_ = i % 64
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record()
            kda.decode_step(dq[s_], dk_[s_], dv_[s_], db[s_], dla[s_], state, o=od)
            b_.record()
            evs.append((a_, b_))
        torch.cuda.synchronize()
        st = stats([a_.elapsed_time(b_) for a_, b_ in evs[args.warmup:]])
        print(json.dumps({"leg": "decode", "workload": "decode_B256_H32_d128", "ms": st,
                          "value": 256 / (st["median"] * 1e-3), "unit": "seq-steps/s"}), flush=True)
        return
    if args.leg == "short_conv":   # width 4: the long prefill's q shape, then the decode rows (state in place)
        g = _gen(7, dev)
        cw = torch.randn((32 * 128, 4), generator=g, device=dev) / 2
        cx = torch.randn((1, 131072, 32 * 128), generator=g, device=dev).to(torch.bfloat16)
        cy = torch.empty_like(cx)
        cfin = torch.empty((1, 32 * 128, 3), dtype=torch.float32, device=dev)
        dx = torch.randn((256, 1, 32 * 128), generator=g, device=dev).to(torch.bfloat16)
        dy = torch.empty_like(dx)
        dst = torch.zeros((256, 32 * 128, 3), dtype=torch.float32, device=dev)
        evs = []
        for i in range(args.warmup + args.steps):
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record()
            kda.short_conv(cx, cw, final_state=cfin, y=cy)
            b_.record()
            kda.short_conv(dx, cw, initial_state=dst, update_state=True, y=dy)
            evs.append((a_, b_))
        torch.cuda.synchronize()
        st = stats([a_.elapsed_time(b_) for a_, b_ in evs[args.warmup:]])
        print(json.dumps({"leg": "short_conv", "workload": "[1, 131072, 4096] bf16, W=4 (+ [256, 1, 4096] rows)",
                          "ms": st, "value": 131072 / (st["median"] * 1e-3), "unit": "tokens/s"}), flush=True)
        return
    if args.leg == "decode_multi":   # 4 tokens per sequence per launch, no per-token states
        gg = _gen(3, dev)
        D = [t.to(torch.bfloat16) for t in _draw_tokens(gg, 64, 256, 32, 128, 128, 0.0, dev, True)]
        state = _state(gg, (256, 32, 128, 128), 0.02, dev)
        mt = [x[:4].transpose(0, 1).contiguous() for x in D]
        om = torch.empty((256, 4, 32, 128), dtype=torch.float32, device=dev)
        evs = []
        for i in range(args.warmup + args.steps):
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record()
            kda.decode(*mt, state, o=om)
            b_.record()
            evs.append((a_, b_))
        torch.cuda.synchronize()
        st = stats([a_.elapsed_time(b_) for a_, b_ in evs[args.warmup:]])
        print(json.dumps({"leg": "decode_multi", "workload": "decode_B256_H32_d128, 4 tokens per launch",
                          "ms": st, "value": 256 * 4 / (st["median"] * 1e-3), "unit": "seq-token-steps/s"}),
              flush=True)
        return
    import synth
    BX = synth.workload(2, device=dev)
    if args.leg == "prefill_f32":   # the T=4096, H=16 prefill shape with fp32 inputs, chunk 64
        ft = lambda a: torch.from_numpy(a).to(dev, torch.float32)  # noqa: E731
        fq, fk, fv, fb, fla = (ft(a) for a in (BX.q, BX.k, BX.v, BX.beta, BX.log_alpha))
        fo = torch.empty_like(fv)
        ffin = torch.empty((1, BX.H, 128, 128), dtype=torch.float32, device=dev)
        evs = []
        for i in range(args.warmup + args.steps):
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record()
            kda.prefill(fq, fk, fv, fb, fla, chunk_size=64, o=fo, final_state=ffin)
            b_.record()
            evs.append((a_, b_))
        torch.cuda.synchronize()
        st = stats([a_.elapsed_time(b_) for a_, b_ in evs[args.warmup:]])
        print(json.dumps({"leg": "prefill_f32", "workload": "prefill shape B=1 T=4096 H=16 d=128, fp32 inputs",
                          "ms": st, "value": BX.T / (st["median"] * 1e-3), "unit": "tokens/s"}), flush=True)
        return
    bt = lambda a: torch.from_numpy(a).to(dev, torch.bfloat16)  # noqa: E731
    bq, bk, bv, bb, bla = (bt(a) for a in (BX.q, BX.k, BX.v, BX.beta, BX.log_alpha))
    bdo = torch.randn(bv.shape, generator=_gen(9, dev), device=dev)
    _, _, ck = kda.prefill(bq, bk, bv, bb, bla, output_final_state=False, chunk_size=64, chunk_states=True)
    evs = []
    for i in range(args.warmup + args.steps):
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record()
        kda.backward(bq, bk, bv, bb, bla, bdo, checkpoints=ck, chunk_size=64)
        b_.record()
        evs.append((a_, b_))
    torch.cuda.synchronize()
    st = stats([a_.elapsed_time(b_) for a_, b_ in evs[args.warmup:]])
    print(json.dumps({"leg": "backward", "workload": "prefill shape B=1 T=4096 H=16 d=128 bf16", "ms": st,
                      "value": BX.T / (st["median"] * 1e-3), "unit": "tokens/s"}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long", choices=["long", "prefill", "packed"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill-workloads", action="store_true",
                    help="skip the per-call timing of the T=4096 and packed prefill workloads")
    ap.add_argument("--record-prefill-traffic", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "SQ_DIR", "MFMA_DIR"),
                    help="refresh the long-prefill entry of profiles/traffic.json from rocprofv3 --pmc runs of "
                         "`bench.py --leg prefill_long --steps S --warmup W` (give the same --steps/--warmup)")
    ap.add_argument("--record-leg-traffic", nargs=3, metavar=("LEG", "FETCH_DIR", "WRITE_DIR"),
                    help="refresh the traffic.json entries of one --leg's calls from a FETCH_SIZE and a "
                         "WRITE_SIZE rocprofv3 --pmc run of that leg")
    ap.add_argument("--leg", choices=["prefill_long", "prefill_c2", "prefill_c4", "prefill_f32", "decode",
                                      "decode_multi", "short_conv",
                                      "backward"],
                    help="run only this workload's calls (warmup + steps), for a per-workload profile")
    ap.add_argument("--summarize", metavar="DIR")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--record-traffic", nargs=6,
                    metavar=("FETCH_DIR", "WRITE_DIR", "SQ_DIR", "CAL_FETCH_DIR", "CAL_WRITE_DIR", "MFMA_DIR"),
                    help="write profiles/traffic.json from rocprofv3 --pmc runs of "
                         "`bench.py --steps S --warmup W --no-cpu-baseline` and `bench.py --copy-calibration` "
                         "(give the same --steps/--warmup)")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize)
        return
    if args.record_traffic:
        record_traffic(*args.record_traffic, calls=args.warmup + args.steps)
        return
    if args.record_prefill_traffic:
        record_prefill_traffic(*args.record_prefill_traffic, calls=args.warmup + args.steps)
        return
    if args.record_leg_traffic:
        record_leg_traffic(*args.record_leg_traffic)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1 "
                                   "(the recurrence shards by head or sequence with no exchange)"}))
        sys.exit(2)

    import torch
    import gated_delta_rule_49_amd as kda
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.leg:
        run_leg(kda, args, dev)
        return
    ev = HipEvents()
    print(f"[bench] generating {args.workload} prefill + decode inputs", file=sys.stderr, flush=True)
    P = prefill_inputs(args.workload, dev)
    Bp, T, H, d = P["q"].shape
    dw = synth.decode_workload(device=dev) if False else None  # host copy not needed
    g = torch.Generator(device=dev)
    # decode workload: B=256, H=32, d=128, 64 steps of fresh bf16 inputs
    from synth.kda_inputs import _draw_tokens, _gen, _state
    gg = _gen(3, dev)
    dq, dk_, dv_, db, dla = _draw_tokens(gg, 64, 256, 32, 128, 128, 0.0, dev, True)
    D = dict(q=dq.to(torch.bfloat16), k=dk_.to(torch.bfloat16), v=dv_.to(torch.bfloat16),
             beta=db.to(torch.bfloat16), log_alpha=dla.to(torch.bfloat16))
    D["state0"] = _state(gg, (256, 32, 128, 128), 0.02, dev)
    del dq, dk_, dv_, db, dla, g, dw
    state = D["state0"].clone()
    Bd = D["q"].shape[1]

    # preallocated outputs and workspace (nothing is allocated in the timed loop)
    ws = torch.empty(kda.workspace_bytes(P["q"], P["k"], P["v"], P["beta"], P["log_alpha"], P["cu"],
                                         P["chunk"]), dtype=torch.uint8, device=dev)
    o = torch.empty((Bp, T, H, d), dtype=torch.float32, device=dev)
    N = Bp if P["cu"] is None else P["cu"].numel() - 1
    fin = torch.empty((N, H, d, d), dtype=torch.float32, device=dev)
    od = torch.empty((Bd, 32, 128), dtype=torch.float32, device=dev)
    n_ev = args.warmup + args.steps
    pev = ev.create(3 * n_ev)
    dstart = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    dend = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]

    def step(i):
        kda.prefill(P["q"], P["k"], P["v"], P["beta"], P["log_alpha"], initial_state=P["init"],
                    cu_seqlens=P["cu"], chunk_size=P["chunk"], workspace=ws, o=o, final_state=fin,
                    check_seqlens=False, timing_events=ctypes.cast(ctypes.byref(pev, 3 * i * ctypes.sizeof(ctypes.c_void_p)),
                                              ctypes.c_void_p))
        s = i % 64
        dstart[i].record()
        kda.decode_step(D["q"][s], D["k"][s], D["v"][s], D["beta"][s], D["log_alpha"][s], state, o=od)
        dend[i].record()

    print("[bench] warmup", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    print("[bench] timed steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for i in range(args.warmup, n_ev):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # Decode throughput as a serving loop sees it: the 64-step trajectory of the
    # decode workload back to back (after one untimed pass), one event pair.
    dec_a = torch.cuda.Event(enable_timing=True)
    dec_b = torch.cuda.Event(enable_timing=True)
    for s_ in range(64):
        kda.decode_step(D["q"][s_], D["k"][s_], D["v"][s_], D["beta"][s_], D["log_alpha"][s_], state, o=od)
    dec_a.record()
    for s_ in range(64):
        kda.decode_step(D["q"][s_], D["k"][s_], D["v"][s_], D["beta"][s_], D["log_alpha"][s_], state, o=od)
    dec_b.record()
    torch.cuda.synchronize()
    dec_loop = dec_a.elapsed_time(dec_b) / 64

    # A reference rate for this box right now: torch's plain 512 MiB device
    # copy (read + write, the traffic of one decode step), best of 3 x 10.
    # It is not the ceiling: copies with non-temporal accesses and small
    # per-workgroup tiles move ~6.2-6.8 TB/s on MI355X.
    csrc = torch.empty(1 << 27, dtype=torch.float32, device=dev).fill_(1.0)
    cdst = torch.empty_like(csrc)
    copy_gbs = 0.0
    for _ in range(3):
        ca = torch.cuda.Event(enable_timing=True)
        cb = torch.cuda.Event(enable_timing=True)
        ca.record()
        for _ in range(10):
            cdst.copy_(csrc)
        cb.record()
        torch.cuda.synchronize()
        copy_gbs = max(copy_gbs, 2 * csrc.numel() * 4 / (ca.elapsed_time(cb) / 10 * 1e-3) / 1e9)
    del csrc, cdst

    # Prefill from pre-activations: the same shapes, q, k, v, beta_raw,
    # gate_raw ~ N(0, 1) (bf16), every prologue stage fused.
    print("[bench] fused prologue", file=sys.stderr, flush=True)
    pro = None
    if Bp == 1 and P["cu"] is None:
        from synth.kda_inputs import preact_tensors
        xq, xk, xv, xb, xg = preact_tensors(_gen(5, dev), 1, T, H, d, d, "bf16", dev)
        pro_ms = []
        for i in range(1 + args.warmup):
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record()
            kda.prefill(xq, xk, xv, xb, xg, chunk_size=P["chunk"], workspace=ws, o=o, final_state=fin,
                        prologue=kda.PROLOGUE_ALL)
            b_.record()
            torch.cuda.synchronize()
            pro_ms.append(a_.elapsed_time(b_))
        del xq, xk, xv, xb, xg
        pro = min(pro_ms[1:]) if len(pro_ms) > 1 else pro_ms[0]

    # Multi-token decode: 4 tokens per sequence per launch over the decode
    # workload's shapes (B=256, H=32, d=128), 16 launches back to back.
    print("[bench] multi-token decode", file=sys.stderr, flush=True)
    M_TOK = 4
    mt = {n: D[n][:M_TOK].transpose(0, 1).contiguous() for n in ("q", "k", "v", "beta", "log_alpha")}
    om = torch.empty((Bd, M_TOK, 32, 128), dtype=torch.float32, device=dev)
    tsb = torch.empty((Bd, M_TOK, 32, 128, 128), dtype=torch.float32, device=dev)
    multi = {}
    for with_states in (False, True):
        def launch():
            kda.decode(mt["q"], mt["k"], mt["v"], mt["beta"], mt["log_alpha"], state, o=om,
                       token_states=False) if not with_states else \
                _decode_into(kda, mt, state, om, tsb)
        launch()
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record()
        for _ in range(16):
            launch()
        b_.record()
        torch.cuda.synchronize()
        ms = a_.elapsed_time(b_) / 16
        nbytes = Bd * 32 * (2 * 128 * 128 * 4 + M_TOK * PREFILL_BYTES_PER_TOKEN_HEAD)
        if with_states:
            nbytes += Bd * 32 * M_TOK * 128 * 128 * 4
        gbs = nbytes / (ms * 1e-3) / 1e9
        multi["with_token_states" if with_states else "state_only"] = {
            "value": Bd * M_TOK / (ms * 1e-3), "unit": "seq-token-steps/s", "avg_ms": ms,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "frac_of_torch_copy": None, "algorithmic_bytes": nbytes,
                         "traffic": None if with_states else measured_traffic("decode_multi_m4"),
                         "kernel": ("decodem_kernel (m = 4, persistent)" if with_states
                                    else "decodec_kernel (m = 4 as one chunk, persistent)")}}
    del tsb, om, mt

    # Short causal convolution (width 4) over a q-shaped input of the prefill
    # workload, [B, T, H * d] bf16 -> bf16, and over one decode token per
    # sequence with the rolling state updated in place.
    print("[bench] short convolution", file=sys.stderr, flush=True)
    CW = 4
    cx = P["q"].reshape(Bp, T, H * d)
    cw = torch.randn((H * d, CW), generator=_gen(7, dev), device=dev) / 2
    cy = torch.empty_like(cx)
    cfin = torch.empty((Bp, H * d, CW - 1), dtype=torch.float32, device=dev)
    conv = {}
    for _ in range(2):
        kda.short_conv(cx, cw, final_state=cfin, y=cy)
    a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a_.record()
    for _ in range(10):
        kda.short_conv(cx, cw, final_state=cfin, y=cy)
    b_.record()
    torch.cuda.synchronize()
    ms = a_.elapsed_time(b_) / 10
    nbytes = 2 * cx.numel() * 2 + cw.numel() * 4 + cfin.numel() * 4
    conv["prefill"] = {"value": Bp * T / (ms * 1e-3), "unit": "tokens/s", "avg_ms": ms,
                       "shape": f"[{Bp}, {T}, {H * d}] bf16 -> bf16, W={CW}",
                       "roofline": {"bound": "hbm", "achieved": nbytes / (ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                                    "unit": "GB/s", "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                    "frac_of_torch_copy": None, "algorithmic_bytes": nbytes,
                                    "kernel": "short_conv_kernel<bf16,bf16,4> + conv_state_kernel",
                                    # recorded on the long workload's shape
                                    "traffic": (measured_traffic("short_conv_prefill")
                                                if args.workload == "long" else None)}}
    del cx, cy, cfin
    dx = D["q"][0].reshape(Bd, 1, 32 * 128)
    dst = torch.zeros((Bd, 32 * 128, CW - 1), dtype=torch.float32, device=dev)
    dy = torch.empty_like(dx)
    if cw.shape[0] != 32 * 128:  # the prefill workload has another channel count
        cw = torch.randn((32 * 128, CW), generator=_gen(7, dev), device=dev) / 2
    for _ in range(2):
        kda.short_conv(dx, cw, initial_state=dst, update_state=True, y=dy)
    a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a_.record()
    for _ in range(64):
        kda.short_conv(dx, cw, initial_state=dst, update_state=True, y=dy)
    b_.record()
    torch.cuda.synchronize()
    ms = a_.elapsed_time(b_) / 64
    nbytes = 2 * dst.numel() * 4 + 2 * dx.numel() * 2 + cw.numel() * 4
    conv["decode"] = {"value": Bd / (ms * 1e-3), "unit": "seq-steps/s", "avg_ms": ms,
                      "shape": f"[{Bd}, 1, {32 * 128}] bf16, state [{Bd}, {32 * 128}, {CW - 1}] in place",
                      "roofline": {"bound": "hbm", "achieved": nbytes / (ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                                   "unit": "GB/s", "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                   "algorithmic_bytes": nbytes}}
    del dx, dst, dy, cw

    # Backward over the prefill workload's shape (B=1, T=4096, H=16, d=128,
    # bf16): the chunked prefill writing the chunk checkpoints (chunk 64),
    # then the chunked backward (prep, reverse state-gradient scan, per-chunk
    # gradients); d_o ~ N(0, 1) fp32.
    print("[bench] backward", file=sys.stderr, flush=True)
    BX = synth.workload(2, device=dev)
    bt = lambda a: torch.from_numpy(a).to(dev, torch.bfloat16)  # noqa: E731
    bq, bk, bv, bb, bla = (bt(a) for a in (BX.q, BX.k, BX.v, BX.beta, BX.log_alpha))
    bdo = torch.randn(bv.shape, generator=_gen(9, dev), device=dev)
    for _ in range(2):
        _, _, ck = kda.prefill(bq, bk, bv, bb, bla, output_final_state=False, chunk_size=64, chunk_states=True)
        kda.backward(bq, bk, bv, bb, bla, bdo, checkpoints=ck, chunk_size=64)
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    e0.record()
    _, _, ck = kda.prefill(bq, bk, bv, bb, bla, output_final_state=False, chunk_size=64, chunk_states=True)
    e1.record()
    kda.backward(bq, bk, bv, bb, bla, bdo, checkpoints=ck, chunk_size=64)
    e2.record()
    torch.cuda.synchronize()
    fwd_ms, bwd_ms = e0.elapsed_time(e1), e1.elapsed_time(e2)
    bT, bH = BX.T, BX.H
    # algorithmic bytes of the backward per token-head: q, k, v, log alpha
    # (bf16) + beta + d_o (fp32) read, dq, dk, dv, dlog alpha (fp32) and dbeta
    # written, plus the chunk checkpoints read once (d^2 * 4 / 64)
    bwd_unit = 4 * 128 * 2 + 2 + 128 * 4 + 4 * 128 * 4 + 4 + 128 * 128 * 4 // 64
    bwd_bytes = bT * bH * bwd_unit
    backward = {"value": bT / ((fwd_ms + bwd_ms) * 1e-3), "unit": "tokens/s",
                "workload": f"prefill shape B=1 T={bT} H={bH} d=128 bf16",
                "checkpoint_prefill_ms": fwd_ms, "backward_ms": bwd_ms,
                "roofline": {"bound": "hbm", "achieved": bwd_bytes / (bwd_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": bwd_bytes / (bwd_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                             "algorithmic_bytes": bwd_bytes,
                             "kernel": "cb_prep_kernel + cb_scan_kernel + cb_grad_kernel (d=128, bf16)",
                             "traffic": measured_traffic("backward_T4096_H16")}}
    del bq, bk, bv, bb, bla, bdo, ck

    # fp32 inputs (the 1e-5 contract) over the same shape, chunk 64: the
    # chunk prep and the scan on fp32 matrix cores.  Bound: fp32 MFMA.
    print("[bench] fp32 prefill", file=sys.stderr, flush=True)
    ft = lambda a: torch.from_numpy(a).to(dev, torch.float32)  # noqa: E731
    fq, fk, fv, fb, fla = (ft(a) for a in (BX.q, BX.k, BX.v, BX.beta, BX.log_alpha))
    fo = torch.empty_like(fv)
    ffin = torch.empty((1, bH, 128, 128), dtype=torch.float32, device=dev)
    def f32_avg_ms():
        for _ in range(2):
            kda.prefill(fq, fk, fv, fb, fla, chunk_size=64, o=fo, final_state=ffin)
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        f0.record()
        for _ in range(5):
            kda.prefill(fq, fk, fv, fb, fla, chunk_size=64, o=fo, final_state=ffin)
        f1.record()
        torch.cuda.synchronize()
        return f0.elapsed_time(f1) / 5
    f_ms = f32_avg_ms()
    # one sequence, 16 heads: the library overlaps the two stages in one
    # launch; the two-kernel launch is timed beside it
    saved = os.environ.get("KDA_PREFILL_OVERLAP")
    os.environ["KDA_PREFILL_OVERLAP"] = "0"
    try:
        f_two_ms = f32_avg_ms()
    finally:
        if saved is None:
            del os.environ["KDA_PREFILL_OVERLAP"]
        else:
            os.environ["KDA_PREFILL_OVERLAP"] = saved
    f_tf = bT * bH * chunk_flops_per_token_head(64, 128) / (f_ms * 1e-3) / 1e12
    prefill_f32 = {"value": bT / (f_ms * 1e-3), "unit": "tokens/s", "avg_ms": f_ms,
                   "two_kernel_launch_avg_ms": f_two_ms,
                   "workload": f"prefill shape B=1 T={bT} H={bH} d=128, fp32 inputs, chunk 64",
                   "roofline": {"bound": "mfma", "achieved": f_tf, "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                                "frac": f_tf / FP32_PEAK_TFLOPS,
                                "basis": "useful chunked-form flops (10 C d + 6 d^2 per token-head) against "
                                         "the fp32 matrix-core peak",
                                "kernel": "chunk table + f32mm_overlap_kernel (chunk prep and fp32 scan in one "
                                          "launch; two-kernel launch: cb_prep_kernel + f32mm_scan_kernel)"}}
    del fq, fk, fv, fb, fla, fo, ffin, BX

    rng = range(args.warmup, n_ev)
    pre_ms = [ev.ms(pev[3 * i], pev[3 * i + 2]) for i in rng]
    intra_ms = [ev.ms(pev[3 * i], pev[3 * i + 1]) for i in rng]
    scan_ms = [ev.ms(pev[3 * i + 1], pev[3 * i + 2]) for i in rng]
    dec_ms = [dstart[i].elapsed_time(dend[i]) for i in rng]
    pre_st, intra_st, scan_st, dec_st = stats(pre_ms), stats(intra_ms), stats(scan_ms), stats(dec_ms)
    pre, intra, scan, dec_in_step = pre_st["median"], intra_st["median"], scan_st["median"], dec_st["median"]
    dec = dec_loop

    tokens = Bp * T
    value = tokens / (pre * 1e-3)
    pbytes = tokens * H * PREFILL_BYTES_PER_TOKEN_HEAD
    if P["init"] is not None:
        pbytes += 2 * N * H * d * d * 4
    p_gbs = pbytes / (pre * 1e-3) / 1e9
    useful_tf = tokens * H * chunk_flops_per_token_head(P["chunk"], d) / (pre * 1e-3) / 1e12
    dbytes = Bd * 32 * DECODE_BYTES_PER_SEQ_HEAD
    d_gbs = dbytes / (dec * 1e-3) / 1e9

    out = {
        "metric": METRIC,
        "value_basis": "prefill tokens / median per-call time over the timed steps",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": P["workload"], "B": Bp, "T": T, "H": H, "d_k": d, "d_v": d,
                   "chunk": P["chunk"], "num_seqs": N,
                   "decode_workload": "decode_B256_H32_d128", "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": p_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": p_gbs / HBM_PEAK_GBS, "traffic": measured_traffic(f"prefill_{args.workload}"),
                     "torch_copy_gbs": copy_gbs, "frac_of_torch_copy": p_gbs / copy_gbs,
                     "kernel": "kda_prefill_chunked (chunk table + intra_kernel + scan_kernel)",
                     "algorithmic_bytes": pbytes, "avg_ms": pre_st["mean"], "median_ms": pre,
                     "call_ms": pre_st,
                     "kernels_ms": {"intra_kernel": intra, "scan_kernel": scan},
                     "kernels_ms_stats": {"intra_kernel": intra_st, "scan_kernel": scan_st},
                     "useful_mfma_tflops": useful_tf,
                     "useful_mfma_frac": useful_tf / BF16_PEAK_TFLOPS,
                     # counters recorded on the long workload's calls
                     "intra_valu": intra_valu(intra) if args.workload == "long" else None,
                     "mfma_busy": (mfma_busy({"intra_kernel": intra, "scan_kernel": scan})
                                   if args.workload == "long" else None)},
        "decode": {"value": Bd / (dec * 1e-3), "unit": "seq-steps/s", "avg_ms": dec,
                   "timing": "64 consecutive steps of the decode trajectory, one HIP event pair",
                   "avg_ms_right_after_prefill": dec_in_step,
                   "right_after_prefill_ms": dec_st,
                   "roofline": {"bound": "hbm", "achieved": d_gbs, "peak": HBM_PEAK_GBS,
                                "unit": "GB/s", "frac": d_gbs / HBM_PEAK_GBS,
                                "torch_copy_gbs": copy_gbs, "frac_of_torch_copy": d_gbs / copy_gbs,
                                "traffic": measured_traffic("decode"),
                                "kernel": "decode1_kernel (m = 1, persistent)", "algorithmic_bytes": dbytes}},
        "prefill_ms": pre,
    }
    if pro is not None:
        pro_bytes = tokens * H * PREFILL_BYTES_PER_TOKEN_HEAD
        out["prologue"] = {"value": tokens / (pro * 1e-3), "unit": "tokens/s", "avg_ms": pro,
                           "overhead_vs_plain": pro / pre - 1.0,
                           "stages": "log alpha = -softplus(x), beta = sigmoid(x), q/k L2 norm",
                           "inputs": "q, k, v, beta_raw, gate_raw ~ N(0,1) bf16, same shapes",
                           "roofline": {"bound": "hbm", "achieved": pro_bytes / (pro * 1e-3) / 1e9,
                                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                        "frac": pro_bytes / (pro * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                        "algorithmic_bytes": pro_bytes}}
    for v_ in multi.values():
        v_["roofline"]["frac_of_torch_copy"] = v_["roofline"]["achieved"] / copy_gbs
    out["decode_multi"] = dict(tokens_per_launch=M_TOK, **multi)
    conv["prefill"]["roofline"]["frac_of_torch_copy"] = conv["prefill"]["roofline"]["achieved"] / copy_gbs
    out["short_conv"] = conv
    out["backward"] = backward
    out["prefill_fp32"] = prefill_f32
    if not args.no_prefill_workloads:
        print("[bench] prefill workloads (T=4096 H=16; packed 8 documents H=32)", file=sys.stderr, flush=True)
        flush = CacheFlush(dev)
        out["prefill_workloads"] = {
            "prefill_T4096_H16": prefill_leg(kda, "prefill", dev, reps=max(20, args.steps), warmup=3, flush=flush),
            "packed_8docs_H32": prefill_leg(kda, "packed", dev, reps=max(20, args.steps), warmup=3, flush=flush)}
        del flush
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline_prefill(P)
        out["decode"]["cpu_baseline"] = cpu_baseline_decode(D)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
