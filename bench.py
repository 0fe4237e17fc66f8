#!/usr/bin/env python3
"""Benchmark: causal GQA attention fwd+bwd (with the QK-norm + RoPE prologue) on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input: RoPE cache and
QK-norm + RoPE on K (one launch), attention forward (for bf16 io with QK-norm + RoPE of Q inside it),
attention backward with the group sum and the prologue backward (for bf16 io applied inside
the dq and dk/dv kernels' stores), and the dgamma reductions (libxattn kernels only,
preallocated buffers, one stream).  The workload is the long-context Qwen3-shaped GQA
configuration (B=1, S=4096, 32 query heads, 8 KV heads, head_dim 128, bf16 in / fp32
accumulate).

value = algorithmic attention FLOP per step (12 * hd per causal pair per query head:
4 * hd forward, 8 * hd backward; recompute not counted) / measured step time, in TFLOP/s.
The step time includes the prologue kernels, which do no counted FLOP.

Before the W untimed warmup steps the step runs for --settle-ms (default 200 ms) of wall
time: from idle the GPU runs at a low clock and needs tens of milliseconds of continuous
load to reach its sustained clock (measured on workload 5: 0.99 ms for the first 20 steps,
0.66 ms from about the 60th on).  The timed region is then K whole steps as usual.

Prints ONE JSON line on stdout; progress goes to stderr.
  python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms 200] [--workload 5]
  python bench.py --copy-calibration   # plain device copy of known size, for PMC scaling
  python bench.py --workload K --counter-summary SQ_DIR FETCH_DIR WRITE_DIR COPY_FETCH_DIR \
      COPY_WRITE_DIR   # writes profiles/counters_<workload>.json/.md from five
                       # `rocprofv3 --pmc` output folders (no GPU use)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal GQA attn fwd+bwd TFLOP/s (bf16) and % of MI355X MFMA peak"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # MI355X published dense MFMA peaks
PEAK_HBM_GBS = 8000.0
CSRC = os.path.join(ROOT, "causal_gqa_attention_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
# sources whose text decides the attention kernels' code (the build script holds their
# compile flags): counter summaries taken on other text are stale and not reported
KERNEL_SOURCES = ["attn.hip", "attn_bf16.hip", "prologue.hip", "lds_copy.h", "xattn_device.h",
                  os.path.join("..", "build.py")]
# counters of one rocprofv3 --pmc pass (8 SQ counters and one GRBM counter fit one pass)
SQ_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_MFMA",
               "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_VALU",
               "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE"]
# library kernel name (the xattn_profile names) <- substring of the compiled kernel's name
KERNEL_MATCH = [("attn_bwd_dkdv", "dkdv"), ("attn_bwd_dq", "dq_kernel"),
                ("qknorm_rope_fwd", "qknorm_rope_fwd"), ("dgamma_reduce", "dgamma_reduce"),
                ("attn_fwd", "fwd_kernel")]
SIMDS, XCDS = 1024, 8  # MI355X: 256 CUs x 4 SIMDs, 8 XCDs


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--settle-ms", type=float, default=200.0,
                   help="before the warmup steps, run the step until the GPU has been busy "
                        "this long (it leaves its idle clock state only after tens of ms "
                        "of load); 0 disables")
    p.add_argument("--workload", type=int, default=5, help="index of the workload shape")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a plain device copy of 1 GiB (for HBM counter scaling)")
    p.add_argument("--stats-summary", nargs=3, default=None,
                   metavar=("OUT_NAME", "DIR", "BENCH_ARGS"),
                   help="write profiles/OUT_NAME.md from the kernel statistics CSV of a "
                        "`rocprofv3 --kernel-trace --stats -f csv -d DIR -o kt -- python3 "
                        "bench.py BENCH_ARGS` run; no GPU use")
    p.add_argument("--counter-summary", nargs=5, default=None,
                   metavar=("SQ_DIR", "FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR",
                            "COPY_WRITE_DIR"),
                   help="write the per-kernel counter summary of the workload from the CSVs "
                        "of five rocprofv3 --pmc runs (the SQ pass, FETCH_SIZE and WRITE_SIZE "
                        "of the bench, then FETCH_SIZE and WRITE_SIZE of --copy-calibration); "
                        "no GPU use")
    p.add_argument("--docs", type=str, default=None,
                   help="comma-separated document lengths packed along the sequence "
                        "(block-causal mask); must sum to the workload's seq_len")
    p.add_argument("--proj", action="store_true",
                   help="measure the projections around attention instead (QKV and output "
                        "GEMMs, forward and backward)")
    p.add_argument("--model-dim", type=int, default=4096)
    p.add_argument("--decode", action="store_true",
                   help="measure the KV-cache decode step instead (xattn_decode)")
    p.add_argument("--decode-batch", type=int, default=8)
    p.add_argument("--decode-cache", type=int, default=4096,
                   help="cache capacity; the step decodes one token at position capacity-1")
    return p.parse_args()


# dense MFMA flop per clock per CU (gfx950, 4 SIMDs): bf16 32x32x16 in 32 clocks, fp32
# 32x32x2 in 64 clocks (the published 2.5 PFLOP/s and 157.3 TFLOP/s at 2.4 GHz)
MFMA_FLOP_PER_CLK_CU = {"bf16": 4 * 32 * 32 * 16 * 2 // 32, "f32": 4 * 32 * 32 * 2 * 2 // 64}


def device_peak(dtype):
    """The MFMA peak re-derived on this device: CU count (device properties) x dense MFMA
    flop per clock per CU x the device's peak clock (hipDeviceAttributeClockRate)."""
    import ctypes

    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    khz = ctypes.c_int(0)
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        if hip.hipDeviceGetAttribute(ctypes.byref(khz), 5, 0) != 0:  # 5: ClockRate (kHz)
            return None
    except OSError:
        return None
    tflops = cus * MFMA_FLOP_PER_CLK_CU[dtype] * khz.value * 1e3 / 1e12
    return {"cus": cus, "clock_mhz": khz.value / 1e3, "tflops": tflops}


def settle(step, min_ms):
    """Run `step` (synchronised each time) until min_ms of wall time have passed.  From
    idle the GPU starts at a low clock and reaches its sustained clock only after tens of
    milliseconds of continuous load; a training or serving loop runs in that sustained
    state, so the timed steps should too.  Untimed, like the warmup steps."""
    import torch
    n, t0 = 0, time.perf_counter()
    while n == 0 or (time.perf_counter() - t0) * 1e3 < min_ms:
        step()
        torch.cuda.synchronize()
        n += 1
    ms = (time.perf_counter() - t0) * 1e3
    log(f"settle: {n} steps in {ms:.0f} ms")
    return {"ms": round(ms, 1), "steps": n}


def doc_pairs(w, docs):
    """Visible (query, key) pairs per query head: S(S+1)/2 for plain causal attention, the
    sum of L(L+1)/2 over the documents with the block-causal mask."""
    if not docs:
        return w.causal_pairs()
    return sum(n * (n + 1) // 2 for n in docs)


def kernel_units(w, docs=None):
    """Algorithmic work per launch of each kernel of the step (flops for MFMA kernels,
    HBM bytes for the memory-bound prologue), and the bound that applies."""
    pairs = doc_pairs(w, docs) * w.bh
    hd = w.head_dim
    io = 2 if w.dtype == "bf16" else 4
    rows_q, rows_k = w.bh * w.seq_len, w.bkv * w.seq_len
    return {
        "attn_fwd": ("mfma", 4 * hd * pairs, "QK^T and PV: 4*hd per causal pair"),
        "attn_bwd_dkdv": ("mfma", 6 * hd * pairs, "dP, dV, dK: 6*hd per causal pair"),
        "attn_bwd_dq": ("mfma", 2 * hd * pairs, "dQ: 2*hd per causal pair"),
        # prologue forward: K alone (the Q side runs inside attn_fwd)
        "qknorm_rope_fwd": ("hbm", rows_k * (hd * 2 * io + 4),
                            "read x, write y (io dtype), write rstd"),
        # standalone prologue backward (fp32 io, and bf16 shapes whose dk/dv launch splits
        # the group's query heads; bf16 io otherwise fuses it into attn_bwd_dq / dkdv): one
        # launch for Q and K together
        "qknorm_rope_bwd": ("hbm", (rows_q + rows_k) * (hd * (4 + 2 * io) + 4),
                            "read fp32 dy, read x, write dx (io dtype), read rstd"),
    }


def executed_work(w, docs=None):
    """Flops of the products each MFMA kernel executes, recomputation included: not the
    metric, but the matrix units' own rate, reported next to the algorithmic one."""
    pairs = doc_pairs(w, docs) * w.bh
    hd = w.head_dim
    return {"attn_fwd": (4 * hd * pairs, "QK^T, PV"),
            "attn_bwd_dkdv": (8 * hd * pairs, "S recompute, dP, dV, dK"),
            "attn_bwd_dq": (6 * hd * pairs, "S and dP recompute, dQ")}


def sources_sha():
    h = hashlib.sha256()
    for src in KERNEL_SOURCES:
        with open(os.path.join(CSRC, src), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counters_file(name):
    return os.path.join(PROFILES, f"counters_{name}.json")


def counters_for(kernel, name):
    """The committed counter summary of `kernel` on workload `name` (HBM bytes per launch,
    MFMA busy fraction, counter-derived TFLOP/s, ...), if it was taken on the current
    kernel sources; else None."""
    try:
        with open(counters_file(name)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != sources_sha():
        return None
    return t["kernels"].get(kernel)


def cpu_baseline(w, x, budget_s=10.0, docs=None, min_s=2.0):
    """The CPU oracle on a bounded sample of the workload: whole KV-head groups (a KV
    head with its query heads: prologue + attention forward + backward), taken in order
    until about `budget_s` seconds of CPU work or the whole workload is done; a workload
    that takes less than `min_s` is repeated whole until it has taken that long."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        blas = ",".join(sorted({i.get("internal_api", "?") for i in info}))
    except Exception:  # threadpoolctl missing: report the affinity set
        threads, blas = len(os.sched_getaffinity(0)), "unknown"
    g = w.group
    sub = w.replace(batch=1, num_heads=g, num_kv_heads=1)
    done, dt_f, dt_b = 0, 0.0, 0.0
    while True:
        kv = done % w.bkv
        b, kvh = divmod(kv, w.num_kv_heads)
        qs = [b * w.num_heads + kvh * g + r for r in range(g)]
        xq, xk, v, do = x.xq[qs], x.xk[[kv]], x.v[[kv]], x.dout[qs]
        t0 = time.perf_counter()
        oracle.forward(xq, xk, v, x.gamma_q, x.gamma_k, g, 1, w.eps, w.theta, segments=docs)
        t1 = time.perf_counter()
        oracle.backward(xq, xk, v, x.gamma_q, x.gamma_k, do, g, 1, w.eps, w.theta,
                        segments=docs)
        dt_f += t1 - t0
        dt_b += time.perf_counter() - t1
        done += 1
        dt = dt_f + dt_b
        if dt >= budget_s or (done >= w.bkv and dt >= min_s):
            break
    unit = w.head_dim * doc_pairs(w, docs) * sub.bh * done
    flops = 12 * unit
    what = (f"{done} of {w.bkv} KV-head groups" if done <= w.bkv else
            f"{done} KV-head groups ({done / w.bkv:.1f} passes over the workload's {w.bkv})")
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": (f"{what} (each a KV head with its {g} query heads, S={w.seq_len}): "
                       f"float64 numpy oracle, prologue + attention fwd + bwd, {dt:.1f} s, "
                       f"{flops / 1e9:.1f} GFLOP algorithmic"),
            "seconds": dt, "fwd_seconds": dt_f, "bwd_seconds": dt_b,
            "fwd_value": 4 * unit / dt_f / 1e12, "bwd_value": 8 * unit / dt_b / 1e12,
            "blas": blas, "affinity_cpus": len(os.sched_getaffinity(0))}


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for i in range(5):
        b.copy_(a)
        torch.cuda.synchronize()
        log(f"copy {i}: {n} bytes read, {n} bytes written")
    print(json.dumps({"copy_calibration_bytes": n, "dispatches": 5}))


def pmc_rows(folder):
    """Per-dispatch counter values from the counter-collection CSVs rocprofv3 wrote under
    `folder`: {(file, dispatch): {"kernel": name, "ns": duration, counter: value}}."""
    import csv
    import glob
    out = {}
    for fn in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(fn, newline="") as f:
            for row in csv.DictReader(f):
                d = out.setdefault((fn, row["Dispatch_Id"]), {
                    "kernel": row["Kernel_Name"],
                    "ns": int(row["End_Timestamp"]) - int(row["Start_Timestamp"])})
                d[row["Counter_Name"]] = d.get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
    return out


def library_kernel(compiled_name):
    low = compiled_name.lower()
    for name, part in KERNEL_MATCH:
        if part in low:
            return name
    return "copy" if "copy" in low else None


def pmc_means(folder):
    """Mean of every counter (and of the duration) per dispatch, per library kernel."""
    acc = {}
    for d in pmc_rows(folder).values():
        k = library_kernel(d["kernel"])
        if k is None:
            continue
        a = acc.setdefault(k, {"dispatches": 0})
        a["dispatches"] += 1
        for c, v in d.items():
            if c != "kernel":
                a[c] = a.get(c, 0.0) + v
    return {k: {c: (v / a["dispatches"] if c != "dispatches" else v) for c, v in a.items()}
            for k, a in acc.items()}


def min_traffic(w):
    """Least HBM bytes of attention fwd + bwd, each tensor read or written once: the forward
    reads q, k, v and writes out and lse (fp32); the backward reads q, k, v, out, dO, lse and
    D and writes dq, dk, dv."""
    esz = 2 if w.dtype == "bf16" else 4
    q_el, kv_el = w.bh * w.seq_len * w.head_dim, w.bkv * w.seq_len * w.head_dim
    rows = w.bh * w.seq_len
    fwd = esz * (2 * q_el + 2 * kv_el) + 4 * rows
    bwd = esz * (4 * q_el + 4 * kv_el) + 8 * rows
    return fwd + bwd


def attainable(flop, min_bytes, value, peak):
    """Roofline bound of the step from its least HBM traffic: intensity = FLOP / bytes, the
    bound min(peak, intensity x HBM peak) in TFLOP/s, and the measured rate's share of it."""
    ai = flop / min_bytes
    bound = min(peak, ai * PEAK_HBM_GBS / 1e3)
    return {"min_bytes": min_bytes, "flop_per_byte": ai, "tflops": bound,
            "pct": 100.0 * value / bound}


def stats_summary(out_name, folder, bench_args):
    """profiles/<out_name>.md: the kernel statistics rocprofv3 wrote (calls, total, average,
    min and max duration per kernel) as a table, with the command that made them."""
    import csv
    import glob
    files = glob.glob(os.path.join(folder, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {folder}")
    with open(files[0], newline="") as f:
        rows = list(csv.DictReader(f))

    def col(row, *keys):
        for k in row:
            if any(k.lower() == key.lower() for key in keys):
                return row[k]
        raise KeyError(keys)

    cmd = (f"cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -f csv "
           f"-d $REPO/{folder} -o kt -- python3 $REPO/bench.py {bench_args}")
    lines = [f"# Kernel statistics: `bench.py {bench_args}`", "",
             "Command (one MI355X; `REPO` = the repository root; raw output stays in "
             "gpurun_out/):", "", f"    {cmd}", "",
             "| kernel | calls | total us | avg us | min us | max us | % |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    for r in rows:
        us = lambda *k: float(col(r, *k)) / 1e3
        lines.append(f"| `{col(r, 'Name', 'KERNEL_NAME')}` | {col(r, 'Calls')} | "
                     f"{us('TotalDurationNs'):.1f} | {us('AverageNs'):.1f} | "
                     f"{us('MinNs'):.1f} | {us('MaxNs'):.1f} | "
                     f"{float(col(r, 'Percentage')):.1f} |")
    with open(os.path.join(PROFILES, out_name + ".md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    log(f"wrote profiles/{out_name}.md")


def counter_summary(dirs, w):
    """Write profiles/counters_<workload>.json and .md: per library kernel of the step, the
    SQ counters of one pass (MFMA busy cycles and bf16 MFMA ops, LDS instructions and bank
    conflicts, GRBM active cycles) and the HBM bytes of a FETCH_SIZE and a WRITE_SIZE pass,
    each scaled by what the same counter reads for a plain 1 GiB device copy; tagged with the
    hash of the kernel sources they were taken on."""
    sq_dir, fetch_dir, write_dir, cfetch_dir, cwrite_dir = dirs
    sq, fe, wr = pmc_means(sq_dir), pmc_means(fetch_dir), pmc_means(write_dir)
    kib = (1 << 30) / 1024.0
    scale = {"fetch": pmc_means(cfetch_dir)["copy"]["FETCH_SIZE"] / kib,
             "write": pmc_means(cwrite_dir)["copy"]["WRITE_SIZE"] / kib}
    units = kernel_units(w)
    kernels = {}
    for k, c in sq.items():
        if k == "copy":
            continue
        e = {"dispatches": int(c["dispatches"]), "pmc_pass_us": c["ns"] / 1e3}
        grbm = c["GRBM_GUI_ACTIVE"] / XCDS          # active cycles of one XCD
        e["grbm_clock_ghz"] = grbm / c["ns"]
        e["mfma_busy"] = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (grbm * SIMDS)
        e["mfma_tflops_counter"] = c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / (c["ns"] * 1e-9) / 1e12
        e["mfma_insts"] = c["SQ_INSTS_MFMA"]
        e["lds_insts"] = c["SQ_INSTS_LDS"]
        e["lds_insts_per_mfma"] = c["SQ_INSTS_LDS"] / c["SQ_INSTS_MFMA"] if c["SQ_INSTS_MFMA"] else None
        e["valu_insts_per_mfma"] = c["SQ_INSTS_VALU"] / c["SQ_INSTS_MFMA"] if c["SQ_INSTS_MFMA"] else None
        e["lds_bank_conflict_rate"] = (c["SQ_LDS_BANK_CONFLICT"] /
                                       max(c["SQ_LDS_IDX_ACTIVE"] - c["SQ_LDS_BANK_CONFLICT"], 1.0))
        if k in fe and k in wr:
            e["hbm_fetch_bytes"] = fe[k]["FETCH_SIZE"] / scale["fetch"] * 1024.0
            e["hbm_write_bytes"] = wr[k]["WRITE_SIZE"] / scale["write"] * 1024.0
            e["hbm_bytes"] = e["hbm_fetch_bytes"] + e["hbm_write_bytes"]
            e["hbm_gbs_counter"] = e["hbm_bytes"] / (fe[k]["ns"] * 1e-9) / 1e9
        if k in units:
            e["bound"], e["algorithmic_work"], e["work_basis"] = units[k]
        kernels[k] = e
    pre = "cd /tmp && export TMPDIR=/tmp && "
    run = f"-- python3 $REPO/bench.py --workload {w.index} --steps 3 --warmup 1 --settle-ms 0 --no-cpu-baseline"
    copy = "-- python3 $REPO/bench.py --copy-calibration"
    t = {"workload": w.name, "source_sha256": sources_sha(), "source_files": KERNEL_SOURCES,
         "copy_scale": scale, "kernels": kernels,
         "notes": {"mfma_busy": "SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE of one XCD x 1024 "
                                "SIMDs): the MFMA-busy fraction of the active cycles, i.e. the "
                                "fraction of the MFMA peak at the measured clock",
                   "grbm_clock_ghz": "GRBM_GUI_ACTIVE of one XCD / dispatch duration",
                   "mfma_tflops_counter": "SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 / dispatch "
                                          "duration (executed MFMA work, recompute included)",
                   "hbm_bytes": "FETCH_SIZE / copy_scale.fetch + WRITE_SIZE / copy_scale.write, "
                                "KiB -> bytes, per dispatch",
                   "pmc_pass_us": "dispatch duration inside the counter pass (counter "
                                  "collection serialises kernels; the kernel-trace stats give "
                                  "the timing)"},
         "commands": [
             pre + f"timeout -s KILL 120 rocprofv3 --pmc {' '.join(SQ_COUNTERS)} -d $REPO/{sq_dir} -o pmc -f csv " + run,
             pre + f"timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE -d $REPO/{fetch_dir} -o pmc -f csv " + run,
             pre + f"timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE -d $REPO/{write_dir} -o pmc -f csv " + run,
             pre + f"timeout -s KILL 90 rocprofv3 --pmc FETCH_SIZE -d $REPO/{cfetch_dir} -o copy -f csv " + copy,
             pre + f"timeout -s KILL 90 rocprofv3 --pmc WRITE_SIZE -d $REPO/{cwrite_dir} -o copy -f csv " + copy,
             f"python3 bench.py --workload {w.index} --counter-summary {' '.join(dirs)}"]}
    with open(counters_file(w.name), "w") as f:
        json.dump(t, f, indent=1)
    lines = [f"# Counters: {w.name}", "",
             f"Per dispatch, means over the dispatches of `bench.py --workload {w.index}` under "
             "rocprofv3 (three steps). Commands:", ""]
    lines += [f"    {c}" for c in t["commands"]]
    lines += ["", "| kernel | dispatches | MFMA busy | counter TFLOP/s | GRBM GHz | LDS inst / MFMA "
              "| VALU inst / MFMA | LDS bank conflict | HBM MB (fetch + write) | HBM GB/s |",
              "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    f2 = lambda v, fmt: "—" if v is None else format(v, fmt)
    for k, e in kernels.items():
        hb = e.get("hbm_bytes")
        lines.append(
            f"| {k} | {e['dispatches']} | {100 * e['mfma_busy']:.1f} % | "
            f"{e['mfma_tflops_counter']:.0f} | {e['grbm_clock_ghz']:.2f} | "
            f"{f2(e['lds_insts_per_mfma'], '.2f')} | {f2(e['valu_insts_per_mfma'], '.2f')} | "
            f"{100 * e['lds_bank_conflict_rate']:.2f} % | "
            f"{'—' if hb is None else format(hb / 1e6, '.1f')} | "
            f"{'—' if hb is None else format(e['hbm_gbs_counter'], '.0f')} |")
    lines += ["", "Copy calibration (counter KiB per KiB copied): "
              f"FETCH_SIZE {scale['fetch']:.3f}, WRITE_SIZE {scale['write']:.3f}.",
              f"Kernel sources hash: `{t['source_sha256'][:16]}`."]
    with open(counters_file(w.name)[:-5] + ".md", "w") as f:
        f.write("\n".join(lines) + "\n")
    log(f"wrote {counters_file(w.name)} and .md")


PROJ_METRIC = "attention-block projections fwd+bwd TFLOP/s (bf16 GEMMs, fp32 accumulate)"


def proj_bench(args):
    """One projection step = the QKV projection and the output projection, forward and
    backward (weight and bias gradients included), on the workload's heads with model
    dimension --model-dim; inputs seeded, synthetic, resident in HBM."""
    import numpy as np
    import torch

    import causal_gqa_attention_amd as X
    import workloads as W

    w = W.WORKLOADS[args.workload]
    B, S, H, Hkv, hd, d = w.batch, w.seq_len, w.num_heads, w.num_kv_heads, w.head_dim, args.model_dim
    M, nq, nk = B * S, H * hd, Hkv * hd
    name = f"{w.name}_proj_d{d}"
    log(f"projection workload {name}: tokens {M}, d={d}, q {nq}, k/v {nk}, {w.dtype}")
    torch.cuda.set_device(0)
    g = torch.Generator(device="cpu").manual_seed(77)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    rnd = lambda *shape, scale=1.0: (torch.randn(*shape, generator=g) * scale).to(dt).to("cuda")
    x = rnd(M, d)
    wq, wk, wv = rnd(d, nq, scale=d ** -0.5), rnd(d, nk, scale=d ** -0.5), rnd(d, nk, scale=d ** -0.5)
    wo = rnd(nq, d, scale=nq ** -0.5)
    bias = [(0.1 * torch.randn(n, generator=g)).to("cuda") for n in (nq, nk, nk, d)]
    pr = X.Projection(B, S, H, Hkv, hd, wq, wk, wv, wo, *bias)
    out, dy = rnd(B * H, S, hd), rnd(M, d)
    gq, gk, gv = rnd(B * H, S, hd), rnd(B * Hkv, S, hd), rnd(B * Hkv, S, hd)

    def step():
        pr.qkv_fwd(x)
        pr.out_fwd(out)
        pr.out_bwd(out, dy)
        pr.qkv_bwd(x, gq, gk, gv)

    flops = 2 * M * d * (nq + 2 * nk) + 2 * M * nq * d      # forward: QKV, output
    flops += 2 * (2 * M * d * nq)                             # output backward: dO, dWo
    flops += 2 * (2 * M * d * (nq + 2 * nk))                  # QKV backward: dx, dW
    settled = settle(step, args.settle_ms) if args.settle_ms > 0 else None
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    value = flops / (ms * 1e-3) / 1e12
    log(f"timed {args.steps} projection steps: {ms:.3f} ms/step, {value:.1f} TFLOP/s")
    X.xattn_profile_start()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof = X.xattn_profile_stop()
    kernels = {n: {"launches_per_step": c / args.steps, "avg_ms": t / max(c, 1),
                   "ms_per_step": t / args.steps} for n, (c, t) in prof.items()}
    log("kernels: " + ", ".join(f"{n} {k['avg_ms'] * 1e3:.1f} us x{k['launches_per_step']:.0f}"
                                for n, k in kernels.items()))
    k = kernels["proj_gemm"]
    achieved = flops / (k["ms_per_step"] * 1e-3) / 1e12  # all GEMM flops over all GEMM time
    roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_TFLOPS[w.dtype],
                "unit": "TFLOP/s", "frac": achieved / PEAK_TFLOPS[w.dtype], "traffic": None,
                "kernel": "proj_gemm (gemm_bf16_kernel)", "work_per_launch": flops / k["launches_per_step"],
                "work_basis": "2*M*N*K of the step's 10 GEMMs, averaged per launch"}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        import os as _os
        log("timing the CPU oracle on a bounded sample ...")
        try:
            from threadpoolctl import threadpool_info
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:
            threads = len(_os.sched_getaffinity(0))
        rows = min(S, 256)  # the first `rows` tokens of batch row 0, every head
        xs = x[:rows].float().cpu().numpy()
        wn = [t.float().cpu().numpy() for t in (wq, wk, wv, wo)]
        bn = [t.cpu().numpy() for t in bias]
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < 10.0:
            q_, k_, v_ = oracle.qkv_proj(xs, *wn[:3], *bn[:3], 1, rows, H, Hkv, hd)
            oracle.out_proj(q_, wn[3], bn[3], 1, rows, H, hd)
            oracle.out_proj_bwd(q_, wn[3], xs, 1, rows, H, hd)
            oracle.qkv_proj_bwd(xs, *wn[:3], q_, k_, v_, 1, rows, H, Hkv, hd)
            reps += 1
        dtc = time.perf_counter() - t0
        cpu = {"value": flops * rows / M * reps / dtc / 1e12, "unit": "TFLOP/s",
               "cores": int(threads), "kind": "oracle",
               "sample": f"{reps} x the step on the first {rows} of {M} token rows: float64 "
                         f"numpy oracle projections fwd + bwd, {dtc:.1f} s"}
    print(json.dumps({
        "metric": PROJ_METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "settle": settled, "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": name, "tokens": M, "model_dim": d, "num_heads": H,
                   "num_kv_heads": Hkv, "head_dim": hd, "io_dtype": w.dtype,
                   "parallelism": "none (1 GPU)"},
        "pct_of_peak": 100.0 * value / PEAK_TFLOPS[w.dtype], "roofline": roofline,
        "cpu_baseline": cpu, "kernels": kernels, "flop_per_step": flops}))


DECODE_METRIC = "KV-cache decode step: cache bytes streamed per second (HBM GB/s)"


def decode_ranges(bkv, rows):
    """Key ranges per KV head of the library's decode plan: ranges of at least 64 keys, at
    most 1024 // bkv of them, each a whole number of 16-key tiles."""
    cap_splits = 1 if bkv >= 1024 else 1024 // bkv
    n = max(1, min(-(-rows // 64), cap_splits))
    ks = -(-(-(-rows // n)) // 16) * 16
    return -(-rows // ks)


def decode_bench(args):
    """One decode step = xattn_decode of one new token per sequence against a full cache
    (Qwen3-shaped heads: 32 query heads, 8 KV heads, head_dim 128, bf16, theta 1e6), the
    cache and the new token's inputs seeded and synthetic, resident in HBM.  value = the
    step's algorithmic HBM bytes (K and V cache rows read, new rows written, q / k / v read,
    out written) / step time."""
    import numpy as np
    import torch

    import causal_gqa_attention_amd as X
    import workloads as W

    base = W.WORKLOADS[5]
    B, cap, q_len = args.decode_batch, args.decode_cache, 1
    H, Hkv, hd = base.num_heads, base.num_kv_heads, base.head_dim
    pos = cap - q_len
    name = f"qwen3_decode_b{B}_cache{cap}_bf16"
    log(f"decode workload {name}: B={B} H={H} Hkv={Hkv} hd={hd} cache_len={pos} q_len={q_len}")
    rng = np.random.default_rng(55)
    f32 = np.float32
    kc_h = W.bf16_round(rng.standard_normal((B * Hkv, cap, hd), dtype=f32))
    vc_h = W.bf16_round(rng.standard_normal((B * Hkv, cap, hd), dtype=f32))
    xq_h = W.bf16_round(rng.standard_normal((B * H, q_len, hd), dtype=f32))
    xk_h = W.bf16_round(rng.standard_normal((B * Hkv, q_len, hd), dtype=f32))
    v_h = W.bf16_round(rng.standard_normal((B * Hkv, q_len, hd), dtype=f32))
    g_h = (1.0 + 0.1 * rng.standard_normal((2, hd), dtype=f32)).astype(f32)
    torch.cuda.set_device(0)
    d = lambda a, dt=torch.bfloat16: torch.from_numpy(a).to("cuda").to(dt)
    kc, vc, xq, xk, v = d(kc_h), d(vc_h), d(xq_h), d(xk_h), d(v_h)
    gq, gk = d(g_h[0], torch.float32), d(g_h[1], torch.float32)
    cos, sin = X.rope_cache(cap, hd, base.theta)
    dims = X.make_decode_dims(xq, kc, H, Hkv, pos)
    ws = torch.empty(X.xattn_decode_workspace_bytes(dims), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(xq)
    lse = torch.empty(B * H * q_len, dtype=torch.float32, device="cuda")

    def step():
        X.xattn_decode(dims, xq, xk, v, gq, gk, cos, sin, base.eps, kc, vc, out, lse, ws)

    settled = settle(step, args.settle_ms) if args.settle_ms > 0 else None
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    Lk = pos + q_len
    cache_read = 2 * B * Hkv * Lk * hd * 2          # every visible K and V row, bf16
    small = (B * H + 2 * B * Hkv) * q_len * hd * 2 + 2 * B * Hkv * q_len * hd * 2 \
        + B * H * q_len * (hd * 2 + 4)              # new q/k/v in, new rows, out + lse
    total = cache_read + small
    value = total / (ms * 1e-3) / 1e9
    log(f"timed {args.steps} decode steps: {ms * 1e3:.1f} us/step, {value:.0f} GB/s, "
        f"{B * q_len / (ms * 1e-3):.0f} tokens/s")

    X.xattn_profile_start()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof = X.xattn_profile_stop()
    kernels = {n: {"launches_per_step": c / args.steps, "avg_ms": t / max(c, 1),
                   "ms_per_step": t / args.steps} for n, (c, t) in prof.items()}
    log("kernels: " + ", ".join(f"{n} {k['avg_ms'] * 1e3:.1f} us" for n, k in kernels.items()))
    # dominant kernel: the split attention; its algorithmic bytes are the cache rows it
    # streams plus the rotated queries it reads and the partials it writes
    ranges = decode_ranges(B * Hkv, Lk)
    split_bytes = (cache_read + B * H * q_len * hd * 2
                   + B * Hkv * ranges * (H // Hkv) * q_len * (hd + 2) * 4)
    k = kernels["decode_split"]
    achieved = split_bytes / (k["avg_ms"] * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": None, "kernel": "decode_split",
                "work_per_launch": split_bytes,
                "work_basis": "K and V cache rows read (bf16) + rotated q read + fp32 range "
                              "partials written"}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        log("timing the CPU oracle on a bounded sample ...")
        try:
            from threadpoolctl import threadpool_info
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:
            threads = len(os.sched_getaffinity(0))
        g = H // Hkv
        # KV-head groups in order, the whole step repeated until about 2 s of CPU work (one
        # pass over all groups takes well under a second)
        done, dt = 0, 0.0
        while dt < 2.0:
            kv = done % (B * Hkv)
            b, kvh = divmod(kv, Hkv)
            qs = [b * H + kvh * g + r for r in range(g)]
            t0 = time.perf_counter()
            oracle.decode(xq_h[qs], xk_h[[kv]], v_h[[kv]], g_h[0], g_h[1], kc_h[[kv]],
                          vc_h[[kv]], pos, g, 1, base.eps, base.theta)
            dt += time.perf_counter() - t0
            done += 1
            if done >= 64 * B * Hkv:
                break
        per_group = total / (B * Hkv)
        cpu = {"value": done * per_group / dt / 1e9, "unit": "GB/s", "cores": int(threads),
               "kind": "oracle",
               "sample": f"{done} KV-head groups ({done / (B * Hkv):.1f} passes over the "
                         f"step's {B * Hkv}; each a KV head's {Lk} cached rows with its {g} "
                         f"query heads): float64 numpy oracle.decode, {dt * 1e3:.0f} ms",
               "seconds": dt}
    line = {
        "metric": DECODE_METRIC, "value": value, "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "settle": settled, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "batch": B, "cache_len": pos, "q_len": q_len,
                   "num_heads": H, "num_kv_heads": Hkv, "head_dim": hd, "io_dtype": "bf16",
                   "parallelism": "none (1 GPU)"},
        "tokens_per_s": B * q_len / (ms * 1e-3),
        "pct_of_hbm_peak": 100.0 * value / PEAK_HBM_GBS,
        "roofline": roofline, "cpu_baseline": cpu, "kernels": kernels,
        "bytes_per_step": total,
    }
    print(json.dumps(line))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): this path shards by "
              "KV-head groups with no exchange besides a 2*hd-float dgamma all-reduce, and "
              "no multi-GPU figure is produced.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.stats_summary:
        stats_summary(*args.stats_summary)
        return
    if args.counter_summary:
        import workloads as W
        counter_summary(args.counter_summary, W.WORKLOADS[args.workload])
        return
    if args.decode:
        decode_bench(args)
        return
    if args.proj:
        proj_bench(args)
        return

    import numpy as np
    import torch

    import causal_gqa_attention_amd as X
    import workloads as W
    from causal_gqa_attention_amd.step import AttentionStep

    w = W.WORKLOADS[args.workload]
    docs = [int(n) for n in args.docs.split(",")] if args.docs else None
    if docs and sum(docs) != w.seq_len:
        print(f"--docs must sum to seq_len {w.seq_len}", file=sys.stderr)
        sys.exit(2)
    wname = w.name if not docs else f"{w.name}_docs{len(docs)}"
    log(f"workload {w}" + (f", documents {docs}" if docs else ""))
    x = W.make_inputs(w)
    torch.cuda.set_device(0)
    step = AttentionStep(w.batch, w.seq_len, w.num_heads, w.num_kv_heads, w.head_dim, w.dtype,
                         w.eps, w.theta, doc_lengths=docs).load(x.xq, x.xk, x.v, x.dout,
                                                                x.gamma_q, x.gamma_k)
    stream = torch.cuda.current_stream()
    units_per_head = doc_pairs(w, docs) * w.bh
    flops = {"fwd": 4 * w.head_dim * units_per_head, "bwd": 8 * w.head_dim * units_per_head,
             "total": 12 * w.head_dim * units_per_head}
    min_bytes = min_traffic(w)

    settled = settle(step.run, args.settle_ms) if args.settle_ms > 0 else None
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    # timed region: K steps, bracketed by a synchronisation on both sides; an event between
    # consecutive steps (recording one does not wait) gives each step's own time
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        step.run()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = evs[0].elapsed_time(evs[-1]) / args.steps
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    ms_median = per_step[len(per_step) // 2] if len(per_step) % 2 else \
        0.5 * (per_step[len(per_step) // 2 - 1] + per_step[len(per_step) // 2])
    value = flops["total"] / (ms * 1e-3) / 1e12
    log(f"timed {args.steps} steps: {ms:.3f} ms/step (median {ms_median:.3f}, min "
        f"{per_step[0]:.3f}; wall {wall * 1e3 / args.steps:.3f}), {value:.1f} TFLOP/s")

    # per-kernel durations: the same K steps again with library HIP events around every
    # launch (recorded on the launch stream)
    X.xattn_profile_start()
    tp0 = time.perf_counter()
    for _ in range(args.steps):
        step.run()
    torch.cuda.synchronize()
    prof = X.xattn_profile_stop()
    prof_ms = (time.perf_counter() - tp0) * 1e3 / args.steps
    units = kernel_units(w, docs)
    executed = executed_work(w, docs)
    kernels = {}
    for name, (n, tot) in prof.items():
        avg = tot / max(n, 1)
        k = {"launches_per_step": n / args.steps, "avg_ms": avg,
             "ms_per_step": tot / args.steps}
        if name in units:
            bound, work, _ = units[name]
            if bound == "mfma":
                k["tflops"] = work / (avg * 1e-3) / 1e12
                ex, basis = executed[name]
                k["executed_tflops"] = ex / (avg * 1e-3) / 1e12
                k["executed_basis"] = basis
            else:
                k["gbs"] = work / (avg * 1e-3) / 1e9
        kernels[name] = k
    dom = max((n for n in kernels if n in units), key=lambda n: kernels[n]["ms_per_step"])
    bound, work, what = units[dom]
    avg_s = kernels[dom]["avg_ms"] * 1e-3
    if bound == "mfma":
        achieved, peak, unit = work / avg_s / 1e12, PEAK_TFLOPS[w.dtype], "TFLOP/s"
    else:
        achieved, peak, unit = work / avg_s / 1e9, PEAK_HBM_GBS, "GB/s"
    cnt = counters_for(dom, wname)
    traffic = cnt.get("hbm_bytes") if cnt else None
    roofline = {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                "frac": achieved / peak, "traffic": traffic, "kernel": dom,
                "work_per_launch": work, "work_basis": what}
    peak_dev = device_peak(w.dtype) if bound == "mfma" else None
    if peak_dev:
        roofline["peak_rederived"] = peak_dev
        roofline["frac_rederived"] = achieved / peak_dev["tflops"]
    if cnt and bound == "mfma":
        # the same kernel's counters (committed summary, current sources): MFMA-busy fraction
        # of the active cycles = fraction of the MFMA peak at the measured clock
        roofline["frac_measured_clock"] = cnt["mfma_busy"]
        roofline["measured_clock_ghz"] = cnt["grbm_clock_ghz"]
    log(f"kernels: " + ", ".join(f"{n} {k['avg_ms']:.3f} ms x{k['launches_per_step']:.0f}"
                                  for n, k in kernels.items()))
    attn_ms = sum(kernels[n]["ms_per_step"] for n in ("attn_fwd", "attn_bwd_dq", "attn_bwd_dkdv")
                  if n in kernels)

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(w, x, docs=docs)
        log(f"cpu baseline {cpu['value'] * 1e3:.2f} GFLOP/s in {cpu['seconds']:.1f} s")

    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "settle": settled, "ms_per_step": ms,
        "ms_per_step_median": ms_median, "ms_per_step_min": per_step[0],
        "tflops_at_median": flops["total"] / (ms_median * 1e-3) / 1e12,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": wname, "batch": w.batch, "seq_len": w.seq_len,
                   "num_heads": w.num_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "io_dtype": w.dtype, "parallelism": "none (1 GPU)",
                   **({"documents": docs} if docs else {})},
        "pct_of_peak": 100.0 * value / PEAK_TFLOPS[w.dtype],
        "attention_kernels_tflops": flops["total"] / (attn_ms * 1e-3) / 1e12 if attn_ms else None,
        # the same step counted the FlashAttention way (backward = 2.5 x forward: 14 hd per
        # pair), for comparison with figures quoted in that convention
        "fa_convention_tflops": 14 * w.head_dim * units_per_head / (ms * 1e-3) / 1e12,
        # attainable bound min(MFMA peak, intensity x HBM peak) over the least traffic
        "attainable": attainable(flops["total"], min_bytes, value, PEAK_TFLOPS[w.dtype]),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "profiled_ms_per_step": prof_ms,
        "flop_per_step": flops["total"],
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
