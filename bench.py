"""Benchmark of the K-grouped weight-gradient GEMM (libkgwgrad) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--fast]

A step is one kg_wgrad call over one batch of synthetic inputs (the whole hot
path: device scan of the expert sizes, schedule, grouped contraction with the
block rescale, epilogue with C, empty-expert fill). Inputs are resident in HBM
before the timed region. Prints one JSON line.

Default workload: one GPU's local expert share, G = 8 experts, M = 7168, N = 4096,
262144 tokens with per-expert counts ~N(32768, 8192), fp8 e4m3 with fp32 scales per
128 tokens, D accumulated onto C; the default (precise) mode, which meets the
1e-5 tolerance. The other workloads (worked, bf16, zipf_fp8, ue8m0_many, and the
six non-grouped shapes single_m{m}_n{n}_k{k} of the issue page's 1D1D table) are
selectable with --workload; --fast selects the fp8-MFMA mode.

Untimed steps run before the timed ones: the --warmup steps asked for, then more
until about one second has passed (--settle-s), so that the clocks have settled.
After the timed region, `cold` times launches that each follow a 1 GiB write (L2
and the 256 MB MALL hold none of the inputs), and `worked_shape` gives the worked
shape's microseconds per call (launch-latency bound).

    python bench.py --dgrad NAME [--fast] [--fp32-out]

times the M-grouped data-gradient GEMM (kg_dgrad) on dgrad_local_share or
dgrad_ue8m0_many_down (bf16 output unless --fp32-out), with its roofline and the
CPU oracle timed on a row sample.

    python bench.py --requant NAME [--steps K] [--warmup W]

times the requantiser (kg_requant) that produces a workload's fp8 operand instead:
local_share_A (262144 x 7168 bf16 activations -> e4m3 + fp32 scales per 128 tokens),
local_share_A_fp8 (the same activations stored as e4m3 with 1x128 per-token scales),
ue8m0_many_B (131072 x 7168 bf16 gradients -> e4m3 + UE8M0 per 32 tokens). Its line
reports GB/s of algorithmic traffic (source read, codes and scales written) against
8 TB/s of HBM.

The JSON line carries:
  value / ms_per_step     TFLOP/s of useful work 2*sum(K_g)*M*N over the timed steps
  roofline                the kernel's average launch time (HIP events on its
                          stream at the two ends of the back-to-back timed steps)
                          against its bound: MFMA peak for its dtype or 8 TB/s of
                          HBM, whichever the algorithmic work hits first; the
                          precise fp8 mode also reports its fraction of the bf16
                          MFMA peak it contracts at (bf16_mfma_ceiling_frac), and
                          mfma_counters the stored rocprofv3 MFMA-busy record;
                          `traffic` is the measured HBM bytes per launch from
                          rocprofv3 counters (profiles/*.json) if those were taken
                          for the current kernel source, else null
  cpu_baseline            the CPU oracle (fp64, all host cores) timed on a bounded
                          sample of the same workload, scaled to TFLOP/s
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"bf16": 2500.0, "fp8": 5000.0}  # dense MFMA TFLOP/s, MI355X
HBM_GBS = 8000.0
METRIC = "K-grouped wgrad TFLOP/s (2*sum(K)*M*N) + % of FP8 MFMA / HBM roofline, 1 GPU"

DESCR = {
    "worked": "worked shape: G=3, ks=[32,45,27], M=64, N=128, fp8 e4m3 + fp32 scales per 128 tokens, no C",
    "bf16": "bf16: G=4, M=1024, N=2048, 16384 tokens uniform over 3 experts (1 empty), D += C",
    "zipf_fp8": "zipf fp8: G=32, M=7168, N=4096, 65536 tokens Zipf(1.2), fp8 e4m3 + fp32 scales per 128, D += C",
    "ue8m0_many": "many experts UE8M0: G=256 (51 empty), M=2048, N=7168, 131072 tokens top-8, fp8 e4m3 + E8M0 per 32, no C",
    "local_share": "local expert share: G=8, M=7168, N=4096, 262144 tokens ~N(32768,8192), fp8 e4m3 + fp32 scales per 128, D += C",
}
for _m, _n, _k in ((4096, 2112, 7168), (4096, 24576, 1536), (4096, 32768, 512),
                   (4096, 7168, 16384), (4096, 4096, 7168), (4096, 7168, 2048)):
    DESCR[f"single_m{_m}_n{_n}_k{_k}"] = (
        f"non-grouped 1D1D shape of the issue page's table: G=1, M={_m}, N={_n}, {_k} tokens, "
        f"fp8 e4m3 + fp32 scales per 128, no C")


# The sources each kernel is built from (kgwgrad.hip includes the other two headers
# at its end; the GEMM kernels do not use them).
KERNEL_SOURCES = {
    "kg_wgrad": ("kgwgrad.hip", "kg_device.h", "kg_sched.h"),
    "kg_dgrad": ("kg_dgrad.h", "kgwgrad.hip", "kg_device.h", "kg_sched.h"),
    "kg_requant": ("kg_requant.h", "kg_device.h", "kg_sched.h"),
}


def kernel_source_hash(kernel="kg_wgrad"):
    """Hash of the kernel's sources with comments and whitespace removed (a comment
    edit does not change the kernels, so it does not invalidate stored counters)."""
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fp8_grouped_gemm_tn_amd", "csrc")
    for name in sorted(KERNEL_SOURCES[kernel]):
        with open(os.path.join(csrc, name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(name.encode() + " ".join(text.split()).encode())
    return h.hexdigest()[:16]


def counters_for(workload, fast, bf16_out=False, kernel="kg_wgrad", nt=False):
    """HBM bytes per launch measured with rocprofv3 counters for this kernel source."""
    name = f"{workload}{'_nt' if nt else ''}{'_fast' if fast else ''}{'_bf16out' if bf16_out else ''}"
    path = os.path.join(ROOT, "profiles", f"{kernel}_{name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source") != kernel_source_hash(kernel):
        return None
    return rec.get("traffic_bytes")


COPY_BYTES = 1 << 30


def _counter_rows(path):
    """(kernel name, counter name, value) per dispatch from a rocprofv3 counter CSV."""
    import csv
    out = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            key = (row.get("Dispatch_Id") or row.get("Correlation_Id"), row["Kernel_Name"])
            rec = out.setdefault(key, {})
            rec[row["Counter_Name"]] = float(row["Counter_Value"])
            if row.get("Start_Timestamp") and row.get("End_Timestamp"):
                rec["duration_ns"] = float(int(row["End_Timestamp"]) - int(row["Start_Timestamp"]))
    return out


def ingest_counters(fetch_csv, write_csv, name, out_dir=None):
    """HBM bytes per launch of a kernel from FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for the 1 GiB plain copy
    recorded in the same CSV (run the profiled bench.py with --copy-calib). `name` is
    the record's name, prefixed "dgrad:" or "requant:" for those kernels (kg_wgrad
    otherwise)."""
    kern = "kg_wgrad"
    for prefix in ("dgrad", "requant"):
        if name.startswith(prefix + ":"):
            kern, name = "kg_" + prefix, name[len(prefix) + 1:]
    res = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _counter_rows(path)
        mine = [v[counter] for (d, k), v in rows.items() if kern + "_kernel" in k]
        # the calibration copy is the run's first copy dispatch (bench.py issues it
        # before it generates any input, which may copy too)
        copies = sorted((int(d), v[counter]) for (d, k), v in rows.items()
                        if "copy" in k.lower() and "kg_" not in k)
        copy = [copies[0][1]] if copies and \
            COPY_BYTES / 1024 / 4 < copies[0][1] < COPY_BYTES / 1024 * 4 else []
        assert mine, f"no {kern} dispatch in {path}"
        assert copy, f"no 1 GiB copy dispatch in {path}"
        factor = (COPY_BYTES / 1024) / max(copy)   # true KiB per counted KiB
        per_launch = sorted(mine)[len(mine) // 2] * factor * 1024
        res[counter] = {"raw_kib_median": sorted(mine)[len(mine) // 2], "copy_kib": max(copy),
                        "scale": factor, "bytes_per_launch": per_launch}
    rec = {"workload": name, "kernel_source": kernel_source_hash(kern),
           "traffic_bytes": int(res["FETCH_SIZE"]["bytes_per_launch"] +
                                res["WRITE_SIZE"]["bytes_per_launch"]),
           "counters": res}
    path = os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"{kern}_{name}_traffic.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                 "SQ_INSTS_VALU_MFMA_MOPS_F8", "SQ_ACTIVE_INST_VALU", "SQ_LDS_BANK_CONFLICT",
                 "SQ_LDS_IDX_ACTIVE", "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE",
                 "GRBM_COUNT")
SIMDS = 4 * 256  # MI355X: 256 compute units of 4 SIMDs
XCDS = 8  # GRBM counters come summed over the 8 XCDs' GRBMs


def ingest_mfma(csv_path, name, command, out_dir=None):
    """MFMA utilisation of a kernel from one rocprofv3 --pmc pass over MFMA_COUNTERS
    (CSV): per dispatch (median over the kernel's dispatches) the MFMA-busy fraction
    SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / XCDS x SIMDs) (rocprofv3's MfmaUtil,
    which takes the largest of the XCDs' GUI-active counts; the CSV holds their sum);
    the busy pipe runs at the bf16 rate for bf16 MFMAs and at the fp8 rate for fp8
    ones. Also the MFMA work it counted (MOPS x 512 flops) and the rate that gives over
    the dispatch's duration, the shader clock (GUI-active cycles per second), LDS
    bank-conflict cycles per LDS-active cycle, and the raw counters. `name` as for
    ingest_counters."""
    kern = "kg_wgrad"
    for prefix in ("dgrad", "requant"):
        if name.startswith(prefix + ":"):
            kern, name = "kg_" + prefix, name[len(prefix) + 1:]
    rows = _counter_rows(csv_path)
    mine = [v for (d, k), v in rows.items() if kern + "_kernel" in k]
    assert mine, f"no {kern} dispatch in {csv_path}"
    med = lambda c: sorted(v.get(c, float("nan")) for v in mine)[len(mine) // 2]
    raw = {c: med(c) for c in MFMA_COUNTERS + ("duration_ns",)}
    busy = raw["SQ_VALU_MFMA_BUSY_CYCLES"] / (raw["GRBM_GUI_ACTIVE"] / XCDS * SIMDS)
    flops = (raw["SQ_INSTS_VALU_MFMA_MOPS_BF16"] + raw["SQ_INSTS_VALU_MFMA_MOPS_F8"]) * 512
    rec = {"workload": name, "kernel_source": kernel_source_hash(kern), "command": command,
           "dispatches": len(mine),
           "mfma_busy_frac": round(busy, 4),
           "duration_ms_median": round(raw["duration_ns"] / 1e6, 4),
           "shader_clock_ghz": round(raw["GRBM_GUI_ACTIVE"] / XCDS / raw["duration_ns"], 3),
           "mfma_tflops_counted": round(flops / raw["duration_ns"] / 1e3, 1),
           "mfma_flops_counted": (raw["SQ_INSTS_VALU_MFMA_MOPS_BF16"] +
                                  raw["SQ_INSTS_VALU_MFMA_MOPS_F8"]) * 512,
           "mfma_flops_bf16": raw["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512,
           "mfma_flops_f8": raw["SQ_INSTS_VALU_MFMA_MOPS_F8"] * 512,
           "lds_bank_conflict_per_active": round(raw["SQ_LDS_BANK_CONFLICT"] /
                                                 max(raw["SQ_LDS_IDX_ACTIVE"], 1.0), 4),
           # SQ_ACTIVE_INST_VALU counts, summed over waves, the 4-cycle units in which a
           # wave issues VALU instructions (MFMA issue included): per SIMD cycle
           "valu_issue_frac": round(4 * raw["SQ_ACTIVE_INST_VALU"] /
                                    (raw["GRBM_GUI_ACTIVE"] / XCDS * SIMDS), 4),
           "counters_median": raw}
    path = os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"{kern}_{name}_mfma.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def mfma_counters_for(name, kernel="kg_wgrad"):
    """Stored MFMA counters of this kernel source and workload, or None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{name}_mfma.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source") != kernel_source_hash(kernel):
        return None
    return {"mfma_busy_frac": rec["mfma_busy_frac"],
            "mfma_flops_counted": rec["mfma_flops_counted"],
            "shader_clock_ghz": rec["shader_clock_ghz"],
            "lds_bank_conflict_per_active": rec["lds_bank_conflict_per_active"],
            "valu_issue_frac": rec.get("valu_issue_frac"),
            "source": os.path.relpath(path, ROOT)}


def copy_calibration(args, dev):
    """With --copy-calib: one plain 1 GiB device copy (untimed), so that a counter run
    sees it beside the kernel (HBM counter calibration)."""
    if not args.copy_calib:
        return
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


# Every LAUNCH_SAMPLE-th timed step is bracketed by its own pair of events (the
# roofline's per-launch duration); the others run back to back. An event record
# between two launches costs the GPU several microseconds (measured ~7 us per step
# on the default problem), so only a sample of the launches carries them.
LAUNCH_SAMPLE = 8


def timed_steps(step, steps, stream):
    """Time exactly `steps` calls of `step` on `stream`, synchronised before and after.
    Returns (ms_per_step, avg_launch_ms, wall_s, sampled): ms_per_step from events at
    the region's two ends, avg_launch_ms the mean of the sampled launches' own events."""
    import torch
    def sampled(k):
        return k % LAUNCH_SAMPLE == LAUNCH_SAMPLE // 2 or (steps <= LAUNCH_SAMPLE // 2 and
                                                          k == steps - 1)
    n = sum(sampled(k) for k in range(steps))
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(n)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_start.record(stream)
    i = 0
    for k in range(steps):
        if sampled(k):
            pairs[i][0].record(stream)
            step()
            pairs[i][1].record(stream)
            i += 1
        else:
            step()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = t_start.elapsed_time(t_end) / steps
    avg_launch_ms = sum(a.elapsed_time(b) for a, b in pairs) / n
    return ms_per_step, avg_launch_ms, wall, n


def warm_up(step, warmup, seconds=1.0):
    """Run `warmup` untimed steps (10 if None), then more untimed steps until about
    `seconds` have passed in all: with only a few warm-up calls the first timed calls
    run at lower clocks (the default line read 8-10% low). Returns (steps asked for,
    steps run in all, seconds)."""
    import torch
    asked = 10 if warmup is None else warmup
    t0 = time.perf_counter()
    for _ in range(asked):
        step()
    torch.cuda.synchronize()
    n = asked
    while time.perf_counter() - t0 < seconds:
        for _ in range(5):
            step()
        n += 5
        torch.cuda.synchronize()
    return asked, n, time.perf_counter() - t0


# Bytes written between cold-cache launches: four times the 256 MB Infinity Cache
# (MALL) and far more than the L2s, so that a launch finds none of its inputs cached.
FLUSH_BYTES = 1 << 30


def cold_launches(step, n, stream):
    """Median duration (ms) of `n` launches of `step`, each preceded by a write of
    FLUSH_BYTES to a scratch buffer outside its events (cold L2 and MALL)."""
    import torch
    scratch = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    times = []
    for i in range(n):
        scratch.fill_(float(i))
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        b.synchronize()
        times.append(a.elapsed_time(b))
    del scratch
    times.sort()
    return times[len(times) // 2]


def cpu_baseline(case, budget_s=12.0):
    """The oracle as it is, on a bounded sample of the workload's rows."""
    from oracle import kgref
    h = case.host()
    G, M, N = case.G, case.M, case.N
    live = [g for g in range(G) if case.ks[g] > 0]
    g_lo, g_hi = min(live), max(live) + 1
    tokens = int(case.ks[g_lo:g_hi].astype("int64").sum())

    def run(rows):
        t0 = time.perf_counter()
        rc, _, _ = kgref.wgrad(h["A"], h["sa"], h["B"], h["sb"], h["C"], h["ks"], M, N,
                               case.gran_k, case.dtype, g_range=(g_lo, g_hi), m_range=(0, rows))
        assert rc == kgref.OK
        return time.perf_counter() - t0

    # grow the sample towards budget_s of oracle time (the whole workload when that
    # takes less)
    rows = 8
    t = run(rows)
    if t < budget_s / 4:
        rows = int(min(M, max(rows, rows * budget_s / max(t, 1e-3))))
        rows = M if rows >= M else max(8, rows - rows % 8)
        t = run(rows)
    flops = 2.0 * tokens * rows * N
    return {"value": round(flops / t / 1e12, 6), "unit": "TFLOP/s", "cores": kgref.last_threads(),
            "kind": "oracle",
            "sample": f"experts {g_lo}..{g_hi - 1}, rows 0..{rows - 1} of M={M}, all N={N}: "
                      f"{flops / 1e9:.2f} GFLOP in {t:.2f} s (fp64)"}


REQUANT = {
    # name: (routing workload, H, gran_k, scale kind, source, description)
    "local_share_A": ("local_share", 7168, 128, 0, 0,
                      "requantise local-share activations: 262144 x 7168 bf16 -> e4m3 + fp32 "
                      "scales per 128 tokens of 8 experts ~N(32768,8192)"),
    "local_share_A_fp8": ("local_share", 7168, 128, 0, 1,
                          "requantise local-share activations stored as e4m3 with 1x128 per-token "
                          "scales: 262144 x 7168 -> e4m3 + fp32 scales per 128 tokens"),
    "ue8m0_many_B": ("ue8m0_many", 7168, 32, 1, 0,
                     "requantise many-expert gradients: 131072 x 7168 bf16 -> e4m3 + UE8M0 "
                     "scales per 32 tokens of 256 experts (51 empty)"),
}


def requant_main(args):
    """Time kg_requant on one workload's operand; print one JSON line."""
    import numpy as np
    import torch
    import fp8_grouped_gemm_tn_amd as kg
    from fp8_grouped_gemm_tn_amd import inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    wl, H, gran, kind, src, descr = REQUANT[args.requant]
    assert inputs.REQUANT_WORKLOADS[args.requant] == (wl, H, gran, kind, src)
    dev = torch.device("cuda:0")
    copy_calibration(args, dev)
    X, xs, ks = inputs.requant_source(args.requant, device=dev, seed=args.seed)
    K = int(ks.astype(np.int64).sum())
    nblk = int(sum((int(k) + gran - 1) // gran for k in ks))
    ksd = torch.from_numpy(ks).to(dev)
    Q = torch.empty((K, H), dtype=torch.uint8, device=dev)
    S = torch.empty((nblk, H), dtype=torch.float32 if kind == kg.KG_E4M3_F32SCALE else torch.uint8,
                    device=dev)

    def step():
        rc = kg.kg_requant_raw(X, xs, ksd, ks.size, H, K, gran, src, kind, Q, S)
        assert rc == kg.KG_OK, rc

    args.warmup, settle_steps, settle_s = warm_up(step, args.warmup, args.settle_s)
    assert kg.kg_status() == kg.KG_OK
    stream = torch.cuda.current_stream()
    ms_per_step, avg_ms, _, nsampled = timed_steps(step, args.steps, stream)
    assert kg.kg_status() == kg.KG_OK
    nbytes = (K * H * (2 if src == kg.KG_SRC_BF16 else 1) + (0 if xs is None else xs.numel() * 4)
              + K * H + nblk * H * (4 if kind == kg.KG_E4M3_F32SCALE else 1))
    achieved = nbytes / (ms_per_step / 1e3) / 1e9
    line = {
        "metric": "requantiser GB/s of algorithmic HBM traffic (source read + codes and scales "
                  "written) + % of HBM roofline, 1 GPU",
        "value": round(nbytes / (ms_per_step / 1e3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32 arithmetic, bf16/e4m3 in, e4m3 out",
        "data": "synthetic (seeded N(0,1) values, the workload's seeded routing)",
        "config": {"workload": descr, "tokens": K, "H": H, "G": int(ks.size), "gran_k": gran},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_GBS, 4),
                     "traffic": counters_for(args.requant, False, False, "kg_requant"),
                     "algorithmic_bytes": nbytes, "launch_ms": round(ms_per_step, 5),
                     "launch_ms_sampled_events": round(avg_ms, 5),
                     "launches_timed": args.steps},
    }
    if not args.no_cpu:
        from oracle import kgref
        # the oracle on the leading experts whose tokens fit in 32768 rows (all
        # channels; at least the first expert's first 4 blocks): several seconds of CPU
        ks64 = ks.astype(np.int64)
        ne = 1
        while ne < ks.size and ks64[:ne + 1].sum() <= 32768:
            ne += 1
        ks_sub = [int(k) for k in ks[:ne]]
        g0 = 0
        rows = int(sum(ks_sub))
        if rows > 32768 or ne == 1:
            rows = min(int(ks[0]), 32768)
            ks_sub = [rows]
        t0 = 0
        Xr = X[t0:t0 + rows]
        Xs = np.ascontiguousarray((Xr.view(torch.int16) if src == kg.KG_SRC_BF16 else Xr).cpu().numpy())
        if src == kg.KG_SRC_BF16:
            Xs = Xs.view(np.uint16)
        sub = lambda a: None if a is None else np.ascontiguousarray(a[t0:t0 + rows].cpu().numpy())
        tt = time.perf_counter()
        rc, _, _ = kgref.requant(Xs, sub(xs), ks_sub, H, gran,
                                 kgref.SRC_BF16 if src == kg.KG_SRC_BF16 else kgref.SRC_E4M3_1X128,
                                 kgref.SCALE_F32 if kind == kg.KG_E4M3_F32SCALE else kgref.SCALE_UE8M0)
        dt = time.perf_counter() - tt
        assert rc == kgref.OK
        sb = rows * H * (2 if src == kg.KG_SRC_BF16 else 1) + rows * H
        line["cpu_baseline"] = {"value": round(sb / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
                                "kind": "oracle",
                                "sample": f"experts 0..{len(ks_sub) - 1} (token rows 0..{rows - 1}), "
                                          f"all {H} channels: {sb / 1e6:.1f} MB in {dt:.2f} s"}
    print(json.dumps(line), flush=True)


def dgrad_main(args):
    """Time kg_dgrad on one dgrad workload; print one JSON line."""
    import numpy as np
    import torch
    import fp8_grouped_gemm_tn_amd as kg
    from fp8_grouped_gemm_tn_amd import inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    copy_calibration(args, dev)
    c = inputs.dgrad_workload(args.dgrad, device="cuda", seed=args.seed)
    ms = torch.from_numpy(c.ms).to(dev)
    out = torch.float32 if args.fp32_out else torch.bfloat16
    D = torch.empty((c.M_total, c.N), dtype=out, device=dev)
    flags = kg.KG_FLAG_FP8_MFMA if args.fast else 0

    def step():
        kg.kg_dgrad(c.A, c.sa, c.W, c.sw, D, ms, flags)

    args.warmup, settle_steps, settle_s = warm_up(step, args.warmup, args.settle_s)
    assert kg.kg_status() == kg.KG_OK
    stream = torch.cuda.current_stream()
    ms_per_step, avg_ms, wall, nsampled = timed_steps(step, args.steps, stream)
    assert kg.kg_status() == kg.KG_OK
    flops = c.flops
    nbytes = c.algorithmic_bytes(4 if args.fp32_out else 2)
    mfma_peak = PEAK["fp8"]
    t_mfma, t_hbm = flops / (mfma_peak * 1e12), nbytes / (HBM_GBS * 1e9)
    secs = ms_per_step / 1e3
    if t_mfma >= t_hbm:
        roof = {"bound": "mfma", "achieved": round(flops / secs / 1e12, 3), "peak": mfma_peak,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(nbytes / secs / 1e9, 3), "peak": HBM_GBS,
                "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = counters_for(args.dgrad[len("dgrad_"):], bool(args.fast), not args.fp32_out,
                                   "kg_dgrad")
    roof["algorithmic_bytes"] = nbytes
    roof["algorithmic_flops"] = flops
    roof["launch_ms"] = round(ms_per_step, 5)
    roof["launch_ms_sampled_events"] = round(avg_ms, 5)
    roof["launches_timed"] = args.steps
    line = {
        "metric": "M-grouped dgrad TFLOP/s (2*M_total*N*K) + % of FP8 MFMA / HBM roofline, 1 GPU",
        "value": round(flops / (ms_per_step / 1e3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 e4m3 (fp8 MFMA)" if args.fast else "fp8 e4m3 (bf16 MFMA)",
        "data": "synthetic (seeded N(0,1), 1x128 activation and 128x128 weight quantisation)",
        "config": {"workload": DGRAD_DESCR[args.dgrad], "G": c.G, "N": c.N, "K": c.K,
                   "tokens": c.M_total, "fp8_mfma": bool(args.fast),
                   "d_dtype": "fp32" if args.fp32_out else "bf16"},
        "roofline": roof,
        "wall_s": round(wall, 4),
    }
    if not args.no_cpu:
        from oracle import kgref
        h = {k: v.cpu().numpy() for k, v in dict(A=c.A, sa=c.sa, W=c.W, sw=c.sw).items()}
        rows = 16
        while True:
            tt = time.perf_counter()
            rc, _, _ = kgref.dgrad(h["A"], h["sa"], h["W"], h["sw"], c.ms, c.N, c.K, rows=(0, rows))
            dt = time.perf_counter() - tt
            assert rc == kgref.OK
            if dt > 3.0 or rows >= 4096:
                break
            rows = min(4096, int(rows * max(2.0, 10.0 / max(dt, 1e-3))))
        f = 2.0 * rows * c.N * c.K
        line["cpu_baseline"] = {"value": round(f / dt / 1e12, 6), "unit": "TFLOP/s",
                                "cores": kgref.last_threads(), "kind": "oracle",
                                "sample": f"token rows 0..{rows - 1}, all {c.N} columns: "
                                          f"{f / 1e9:.2f} GFLOP in {dt:.2f} s (fp64)"}
    print(json.dumps(line), flush=True)


DGRAD_DESCR = {
    "dgrad_local_share": "dgrad paired with the local-share wgrad: G=8, 262144 tokens ~N(32768,8192), "
                         "dx [262144, 7168] = dy [262144, 4096] . w, fp8 e4m3 1x128 / 128x128 scales",
    "dgrad_ue8m0_many_down": "dgrad of the many-expert down projection: G=256 (51 empty), 131072 "
                             "tokens top-8, dx [131072, 2048] = dy [131072, 7168] . w, fp8 e4m3 "
                             "1x128 / 128x128 scales",
}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps before the timed ones (default: as many as fit in "
                         "about one second, so that the GPU clocks have settled)")
    ap.add_argument("--workload", default="local_share", choices=list(DESCR))
    ap.add_argument("--fast", action="store_true", help="fp8 kinds: contract with the fp8 MFMA")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache launches (each after a 1 GiB write)")
    ap.add_argument("--no-worked", action="store_true",
                    help="skip the worked-shape (launch-latency) timing")
    ap.add_argument("--gran-k", type=int, default=None, choices=[32, 128],
                    help="replace an fp8 workload's scale granularity (tokens per scale)")
    ap.add_argument("--bf16-out", action="store_true",
                    help="the bf16-output variant: C and D in bf16 (KG_FLAG_D_BF16)")
    ap.add_argument("--nt", action="store_true",
                    help="K-major (NT) operands: A [M, tokens] and B [N, tokens], kg_wgrad_nt")
    ap.add_argument("--no-workspace", action="store_true",
                    help="call kg_wgrad without a workspace (no stream-K split of small problems)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--copy-calib", action="store_true",
                    help="first run one plain 1 GiB device copy (untimed), so that a counter "
                         "run sees it beside the kernel (HBM counter calibration)")
    ap.add_argument("--ingest-mfma", nargs=3, metavar=("CSV", "NAME", "COMMAND"),
                    help="turn one rocprofv3 --pmc CSV over the MFMA counters into "
                         "profiles/kg_wgrad_NAME_mfma.json (COMMAND: the profiled command)")
    ap.add_argument("--settle-s", type=float, default=1.0,
                    help="seconds of untimed steps before the timed ones (clock settling)")
    ap.add_argument("--ingest-counters", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "NAME"),
                    help="turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, WRITE_SIZE) into "
                         "profiles/kg_wgrad_NAME_traffic.json")
    ap.add_argument("--requant", choices=list(REQUANT),
                    help="time the requantiser on this operand instead of the GEMM")
    ap.add_argument("--dgrad", choices=list(DGRAD_DESCR),
                    help="time the M-grouped dgrad GEMM (kg_dgrad, bf16 output) instead")
    ap.add_argument("--fp32-out", action="store_true", help="--dgrad: fp32 output")
    args = ap.parse_args()
    if args.dgrad:
        if args.gpus != 1:
            print("bench.py measures one GPU; run with --gpus 1.", file=sys.stderr)
            sys.exit(2)
        dgrad_main(args)
        return
    if args.requant:
        if args.gpus != 1:
            print("bench.py measures one GPU; run with --gpus 1.", file=sys.stderr)
            sys.exit(2)
        requant_main(args)
        return
    if args.ingest_counters:
        ingest_counters(*args.ingest_counters)
        return
    if args.ingest_mfma:
        ingest_mfma(*args.ingest_mfma)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for "
              f"--gpus {args.gpus}); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import fp8_grouped_gemm_tn_amd as kg
    from fp8_grouped_gemm_tn_amd import inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    copy_calibration(args, dev)
    case = inputs.workload(args.workload, device="cuda", seed=args.seed, gran_k=args.gran_k)
    A, B = case.A, case.B
    sa, sb, C = case.sa, case.sb, case.C
    out_dtype = torch.bfloat16 if args.bf16_out else torch.float32
    if C is not None and args.bf16_out:
        C = C.to(torch.bfloat16)
    ks = torch.from_numpy(case.ks).to(dev)
    D = torch.empty((case.G, case.M, case.N), dtype=out_dtype, device=dev)
    flags = kg.KG_FLAG_FP8_MFMA if (args.fast and case.dtype != kg.KG_BF16) else 0
    dtype = case.dtype | flags
    # the library's workspace (zeroed once, left zeroed by every call), allocated
    # before the timed region; it lets small bf16 problems spread over every CU
    ws = None if args.no_workspace else kg.new_workspace(dev)
    if args.nt:
        # K-major copies of the operands, made before the timed region
        At, Bt = inputs.k_major(A), inputs.k_major(B)
        assert torch.equal(At, A.t()) and torch.equal(Bt, B.t())

        def step():
            kg.kg_wgrad_nt(At, sa, Bt, sb, C, D, ks, case.gran_k, dtype, workspace=ws)
    else:
        def step():
            kg.kg_wgrad(A, sa, B, sb, C, D, ks, case.gran_k, dtype, K_total=case.K_total,
                        workspace=ws)

    args.warmup, settle_steps, settle_s = warm_up(step, args.warmup, args.settle_s)
    assert kg.kg_status() == kg.KG_OK
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ms_per_step, avg_launch_ms, wall, nsampled = timed_steps(step, args.steps, stream)
    assert kg.kg_status() == kg.KG_OK

    flops = case.flops
    nbytes = case.algorithmic_bytes(2 if args.bf16_out else 4)
    is_bf16 = case.dtype == kg.KG_BF16
    mfma_peak = PEAK["bf16"] if is_bf16 else PEAK["fp8"]
    t_mfma = flops / (mfma_peak * 1e12)
    t_hbm = nbytes / (HBM_GBS * 1e9)
    bound = "mfma" if t_mfma >= t_hbm else "hbm"

    def roof_of(ms):
        secs = ms / 1e3
        if bound == "mfma":
            r = {"bound": "mfma", "achieved": round(flops / secs / 1e12, 3), "peak": mfma_peak,
                 "unit": "TFLOP/s"}
        else:
            r = {"bound": "hbm", "achieved": round(nbytes / secs / 1e9, 3), "peak": HBM_GBS,
                 "unit": "GB/s"}
        r["frac"] = round(r["achieved"] / r["peak"], 4)
        return r

    # the roofline's launch duration: every timed launch (events at the two ends of the
    # back-to-back region on the launch stream); the sampled per-launch events are kept
    # beside it (they carry a few microseconds of event overhead each)
    roof = roof_of(ms_per_step)
    name = args.workload + ("_nt" if args.nt else "") + ("_fast" if flags else "") + \
        ("_bf16out" if args.bf16_out else "")
    roof["traffic"] = (counters_for(args.workload, bool(flags), args.bf16_out, nt=args.nt)
                       if args.gran_k is None else None)
    roof["algorithmic_bytes"] = nbytes
    roof["algorithmic_flops"] = flops
    roof["roofline_ms"] = round(max(t_mfma, t_hbm) * 1e3, 4)
    roof["launch_ms"] = round(ms_per_step, 5)
    roof["launch_ms_sampled_events"] = round(avg_launch_ms, 5)
    roof["launches_timed"] = args.steps
    if not is_bf16 and not flags:
        # the precise fp8 path contracts exactly widened values with the bf16 MFMA
        roof["bf16_mfma_ceiling_frac"] = round(flops / (ms_per_step / 1e3) / 1e12 / PEAK["bf16"], 4)
    if args.gran_k is None:
        roof["mfma_counters"] = mfma_counters_for(name)

    value = flops / (ms_per_step / 1e3) / 1e12
    dname = "bf16" if is_bf16 else ("fp8 e4m3 (fp8 MFMA)" if flags else "fp8 e4m3 (bf16 MFMA)")
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dname,
        "data": "synthetic (seeded generators, fp8 values quantised per 128/32-token block)",
        "config": {"workload": DESCR[args.workload] + (f" (scales per {args.gran_k} tokens)"
                                                        if args.gran_k else ""),
                   "G": case.G, "M": case.M, "N": case.N,
                   "tokens": case.K_total, "gran_k": case.gran_k if not is_bf16 else None,
                   "fp8_mfma": bool(flags), "workspace": ws is not None,
                   "layout": "K-major (NT)" if args.nt else "token-major (TN)",
                   "d_dtype": "bf16" if args.bf16_out else "fp32"},
        "roofline": roof,
        "pct_fp8_peak": round(100.0 * value / PEAK["fp8"], 2),
        "hbm_gbs": round(nbytes / (ms_per_step / 1e3) / 1e9, 1),
        "settle": {"steps": settle_steps, "s": round(settle_s, 3),
                   "note": "untimed steps run in all before the timed region (at least the "
                           "warmup steps asked for, and about one second so the clocks settle)"},
        "wall_s": round(wall, 4),
    }
    if not args.no_cold:
        cold_ms = cold_launches(step, min(args.steps, 20), stream)
        assert kg.kg_status() == kg.KG_OK
        cold = roof_of(cold_ms)
        line["cold"] = {"launch_ms": round(cold_ms, 5), "value": round(flops / cold_ms / 1e9, 3),
                        "unit": "TFLOP/s", "frac": cold["frac"], "bound": bound,
                        "note": f"median of {min(args.steps, 20)} launches, each after a "
                                f"{FLUSH_BYTES >> 20} MiB write outside its events (L2 and MALL cold)"}
    del A, B, sa, sb, C, D
    if args.workload != "worked" and not args.no_worked:
        line["worked_shape"] = worked_shape_timing(kg, inputs)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(case)
    print(json.dumps(line), flush=True)


def worked_shape_timing(kg, inputs, calls=400):
    """The how-to page's worked shape (3 experts of 32, 45 and 27 tokens, 64 x 128, fp8
    with fp32 scales per 128 tokens): microseconds per call, launch-latency bound."""
    import torch
    c = inputs.workload("worked", device="cuda")
    ks = torch.from_numpy(c.ks).cuda()
    D = torch.empty((c.G, c.M, c.N), dtype=torch.float32, device="cuda")

    def step():
        kg.kg_wgrad(c.A, c.sa, c.B, c.sb, None, D, ks, c.gran_k, c.dtype, K_total=c.K_total)

    warm_up(step, 50, seconds=0.2)
    stream = torch.cuda.current_stream()
    ms, _, _, _ = timed_steps(step, calls, stream)
    # one call on its own, events around it
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    singles = []
    for _ in range(20):
        torch.cuda.synchronize()
        a.record(stream)
        step()
        b.record(stream)
        b.synchronize()
        singles.append(a.elapsed_time(b))
    assert kg.kg_status() == kg.KG_OK
    singles.sort()
    # 20 calls captured in a HIP graph and replayed: the device-side time per call
    # without the Python binding's per-call work
    per_graph, replays = 20, 25
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        for _ in range(per_graph):
            step()
    graph.replay()
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(replays):
        graph.replay()
    b.record(stream)
    b.synchronize()
    us_graph = a.elapsed_time(b) * 1e3 / (replays * per_graph)
    assert kg.kg_status() == kg.KG_OK
    return {"workload": DESCR["worked"], "us_per_call_back_to_back": round(ms * 1e3, 2),
            "us_single_call_events": round(singles[len(singles) // 2] * 1e3, 2),
            "us_per_call_graph_replay": round(us_graph, 2),
            "flops": c.flops, "bound": "launch latency"}


if __name__ == "__main__":
    main()
