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
  python bench.py --traffic-summary FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR
      # writes the dk/dv traffic summary from four `rocprofv3 --pmc` output folders
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_attn_bwd_dkdv_qwen3_long_gqa_bf16.json")
CSRC = os.path.join(ROOT, "causal_gqa_attention_amd", "csrc")


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
    p.add_argument("--traffic-summary", nargs=4, default=None,
                   metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                   help="write the HBM traffic summary of the dk/dv kernel from the counter "
                        "CSVs of four rocprofv3 --pmc runs (FETCH_SIZE and WRITE_SIZE of the "
                        "bench, then of --copy-calibration); no GPU use")
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
    fused_q = w.dtype == "bf16" and hd in (64, 128)
    return {
        "attn_fwd": ("mfma", 4 * hd * pairs, "QK^T and PV: 4*hd per causal pair"),
        "attn_bwd_dkdv": ("mfma", 6 * hd * pairs, "dP, dV, dK: 6*hd per causal pair"),
        "attn_bwd_dq": ("mfma", 2 * hd * pairs, "dQ: 2*hd per causal pair"),
        # prologue forward: K alone when the Q side runs inside attn_fwd (bf16, hd 64/128),
        # else the per-launch average over the Q launch and the K launch
        "qknorm_rope_fwd": ("hbm", (rows_k if fused_q else (rows_q + rows_k) / 2)
                            * (hd * 2 * io + 4), "read x, write y (io dtype), write rstd"),
        # standalone prologue backward (fp32 io; bf16 io fuses it into attn_bwd_dq / dkdv):
        # one launch for Q and K together
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


def traffic_for(kernel, name):
    """HBM bytes per launch from the committed counter summary, if it was taken on the
    current kernel source for this workload; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        h = hashlib.sha256()
        for src in t["source_files"]:
            with open(os.path.join(CSRC, src), "rb") as f:
                h.update(f.read())
        sha = h.hexdigest()
    except (OSError, ValueError, KeyError):
        return None
    if t.get("kernel") != kernel or t.get("workload") != name or t.get("source_sha256") != sha:
        return None
    scale = t["copy_scale"]
    return (t["fetch_kib_per_dispatch"] / scale["fetch"] +
            t["write_kib_per_dispatch"] / scale["write"]) * 1024.0


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
    done, dt = 0, 0.0
    while True:
        kv = done % w.bkv
        b, kvh = divmod(kv, w.num_kv_heads)
        qs = [b * w.num_heads + kvh * g + r for r in range(g)]
        xq, xk, v, do = x.xq[qs], x.xk[[kv]], x.v[[kv]], x.dout[qs]
        t0 = time.perf_counter()
        oracle.forward(xq, xk, v, x.gamma_q, x.gamma_k, g, 1, w.eps, w.theta, segments=docs)
        oracle.backward(xq, xk, v, x.gamma_q, x.gamma_k, do, g, 1, w.eps, w.theta,
                        segments=docs)
        dt += time.perf_counter() - t0
        done += 1
        if dt >= budget_s or (done >= w.bkv and dt >= min_s):
            break
    flops = 12 * w.head_dim * doc_pairs(w, docs) * sub.bh * done
    what = (f"{done} of {w.bkv} KV-head groups" if done <= w.bkv else
            f"{done} KV-head groups ({done / w.bkv:.1f} passes over the workload's {w.bkv})")
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": (f"{what} (each a KV head with its {g} query heads, S={w.seq_len}): "
                       f"float64 numpy oracle, prologue + attention fwd + bwd, {dt:.1f} s, "
                       f"{flops / 1e9:.1f} GFLOP algorithmic"),
            "seconds": dt, "blas": blas, "affinity_cpus": len(os.sched_getaffinity(0))}


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


def pmc_per_dispatch(folder, counter, name_part):
    """Average of `counter` per dispatch over the dispatches whose kernel name contains
    `name_part`, from the counter-collection CSVs rocprofv3 wrote under `folder`."""
    import csv
    import glob
    per = {}
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    for fn in files:
        with open(fn, newline="") as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                if name_part.lower() not in row.get("Kernel_Name", "").lower():
                    continue
                key = (fn, row.get("Dispatch_Id"))
                per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} rows for kernels matching '{name_part}' under {folder}")
    return sum(per.values()) / len(per), len(per)


def traffic_summary(dirs, workload_name):
    """Write the committed traffic summary of the dk/dv kernel: FETCH_SIZE and WRITE_SIZE
    (KiB per dispatch) and the same counters per KiB of a plain 1 GiB device copy, with the
    hash of the kernel sources they were taken on (the bench reports `traffic` only while
    that hash still matches)."""
    fetch_dir, write_dir, cfetch_dir, cwrite_dir = dirs
    fetch, n_f = pmc_per_dispatch(fetch_dir, "FETCH_SIZE", "dkdv")
    write, n_w = pmc_per_dispatch(write_dir, "WRITE_SIZE", "dkdv")
    cfetch, _ = pmc_per_dispatch(cfetch_dir, "FETCH_SIZE", "copy")
    cwrite, _ = pmc_per_dispatch(cwrite_dir, "WRITE_SIZE", "copy")
    kib = (1 << 30) / 1024.0
    files = ["attn.hip", "attn_bf16.hip", "xattn_device.h"]
    h = hashlib.sha256()
    for src in files:
        with open(os.path.join(CSRC, src), "rb") as f:
            h.update(f.read())
    scale = {"fetch": cfetch / kib, "write": cwrite / kib,
             "note": "FETCH_SIZE / WRITE_SIZE (KiB) of one 1 GiB device copy divided by "
                     "1 GiB in KiB"}
    pre = "cd /tmp && export TMPDIR=/tmp && "
    bench_cmd = "-- python3 $REPO/bench.py --steps 3 --warmup 1 --settle-ms 0 --no-cpu-baseline"
    t = {"kernel": "attn_bwd_dkdv", "workload": workload_name,
         "source_sha256": h.hexdigest(), "source_files": files,
         "fetch_kib_per_dispatch": fetch, "write_kib_per_dispatch": write,
         "dispatches": min(n_f, n_w), "copy_scale": scale,
         "commands": [
             pre + f"timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE --kernel-include-regex dkdv "
             f"-d $REPO/{fetch_dir} -o dkdv -f csv " + bench_cmd,
             pre + f"timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE --kernel-include-regex dkdv "
             f"-d $REPO/{write_dir} -o dkdv -f csv " + bench_cmd,
             pre + f"timeout -s KILL 90 rocprofv3 --pmc FETCH_SIZE -d $REPO/{cfetch_dir} -o copy "
             "-f csv -- python3 $REPO/bench.py --copy-calibration",
             pre + f"timeout -s KILL 90 rocprofv3 --pmc WRITE_SIZE -d $REPO/{cwrite_dir} -o copy "
             "-f csv -- python3 $REPO/bench.py --copy-calibration",
             f"python3 bench.py --traffic-summary {fetch_dir} {write_dir} {cfetch_dir} {cwrite_dir}"],
         "hbm_bytes_per_dispatch": (fetch / scale["fetch"] + write / scale["write"]) * 1024.0}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(t, f, indent=1)
    log(f"wrote {TRAFFIC_FILE}: {t['hbm_bytes_per_dispatch'] / 1e6:.1f} MB per dispatch")


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
                "kernel": "proj_gemm (hipBLASLt)", "work_per_launch": flops / k["launches_per_step"],
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
    most ceil(2048 / bkv) of them, equal length."""
    cap_splits = 1 if bkv >= 2048 else -(-2048 // bkv)
    n = max(1, min(-(-rows // 64), cap_splits))
    ks = -(-rows // n)
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
    if args.traffic_summary:
        import workloads as W
        traffic_summary(args.traffic_summary, W.WORKLOADS[args.workload].name)
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

    settled = settle(step.run, args.settle_ms) if args.settle_ms > 0 else None
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    # timed region: K steps, bracketed by a synchronisation on both sides
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step.run()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    value = flops["total"] / (ms * 1e-3) / 1e12
    log(f"timed {args.steps} steps: {ms:.3f} ms/step (wall {wall * 1e3 / args.steps:.3f}), "
        f"{value:.1f} TFLOP/s")

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
    traffic = traffic_for(dom, wname)
    roofline = {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                "frac": achieved / peak, "traffic": traffic, "kernel": dom,
                "work_per_launch": work, "work_basis": what}
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
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": wname, "batch": w.batch, "seq_len": w.seq_len,
                   "num_heads": w.num_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "io_dtype": w.dtype, "parallelism": "none (1 GPU)",
                   **({"documents": docs} if docs else {})},
        "pct_of_peak": 100.0 * value / PEAK_TFLOPS[w.dtype],
        "attention_kernels_tflops": flops["total"] / (attn_ms * 1e-3) / 1e12 if attn_ms else None,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "profiled_ms_per_step": prof_ms,
        "flop_per_step": flops["total"],
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
