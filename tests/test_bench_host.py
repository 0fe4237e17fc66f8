"""Host logic of bench.py (no GPU): the rocprofv3 counter-CSV reader, the per-kernel counter
summary written from it (HBM bytes scaled by a plain copy, MFMA busy fraction, counter
TFLOP/s), and the guard that reports counters only for the kernel sources they were taken
on."""
import csv
import importlib.util
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def write_csv(folder, rows):
    """rows: (dispatch id, kernel name, counter, value[, duration ns]) in rocprofv3's counter
    CSV layout, one row per dimension instance as the tool writes them."""
    os.makedirs(os.path.join(folder, "host"), exist_ok=True)
    path = os.path.join(folder, "host", "1234_counter_collection.csv")
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for r in rows:
            d, k, c, v = r[:4]
            ns = r[4] if len(r) > 4 else 1000
            w.writerow({"Dispatch_Id": d, "Kernel_Name": k, "Counter_Name": c,
                        "Counter_Value": v, "Start_Timestamp": 5000, "End_Timestamp": 5000 + ns})


def test_pmc_means_sum_instances_and_average_dispatches(bench, tmp_path):
    d = str(tmp_path / "f")
    write_csv(d, [(1, "void x::dkdv_pipe_kernel<128>", "FETCH_SIZE", 100.0),
                  (1, "void x::dkdv_pipe_kernel<128>", "FETCH_SIZE", 50.0),  # 2nd instance
                  (2, "void x::dkdv_pipe_kernel<128>", "FETCH_SIZE", 170.0),
                  (3, "void x::dq_kernel<128>", "FETCH_SIZE", 1e9),
                  (4, "void x::fwd_kernel<64, true>", "FETCH_SIZE", 8.0),
                  (5, "void x::qknorm_rope_fwd_table_kernel<1>", "FETCH_SIZE", 4.0),
                  (6, "some_other_kernel", "FETCH_SIZE", 1.0)])
    m = bench.pmc_means(d)
    assert m["attn_bwd_dkdv"]["dispatches"] == 2
    assert m["attn_bwd_dkdv"]["FETCH_SIZE"] == pytest.approx(160.0)
    assert m["attn_bwd_dq"]["FETCH_SIZE"] == 1e9
    assert m["attn_fwd"]["FETCH_SIZE"] == 8.0 and m["qknorm_rope_fwd"]["FETCH_SIZE"] == 4.0
    assert set(m) == {"attn_bwd_dkdv", "attn_bwd_dq", "attn_fwd", "qknorm_rope_fwd"}


def test_counter_summary_scales_by_the_copy_and_guards_the_source(bench, tmp_path,
                                                                 monkeypatch):
    import workloads as W
    w = W.WORKLOADS[5]
    kib = float(1 << 20)  # 1 GiB in KiB
    dirs = [str(tmp_path / n) for n in ("sq", "f", "w", "cf", "cw")]
    k = "void x::dkdv_pipe_kernel<128, true>"
    ns = 300_000
    # one XCD active for 600k cycles in 300 us (2 GHz); MFMAs busy 40 % of 1024 SIMDs
    sq = {"GRBM_GUI_ACTIVE": 8 * 600_000, "SQ_VALU_MFMA_BUSY_CYCLES": 0.4 * 600_000 * 1024,
          "SQ_INSTS_VALU_MFMA_MOPS_BF16": 2e8, "SQ_INSTS_MFMA": 1e6, "SQ_INSTS_LDS": 2e6,
          "SQ_LDS_BANK_CONFLICT": 10.0, "SQ_LDS_IDX_ACTIVE": 1010.0, "SQ_INSTS_VALU": 5e6,
          "SQ_BUSY_CU_CYCLES": 1.0}
    write_csv(dirs[0], [(1, k, c, v, ns) for c, v in sq.items()])
    write_csv(dirs[1], [(1, k, "FETCH_SIZE", 1000.0, ns)])
    write_csv(dirs[2], [(1, k, "WRITE_SIZE", 300.0, ns)])
    # the plain 1 GiB copy reads half its bytes in FETCH_SIZE KiB, all in WRITE_SIZE
    write_csv(dirs[3], [(7, "__amd_rocclr_copyBuffer", "FETCH_SIZE", kib / 2)])
    write_csv(dirs[4], [(7, "__amd_rocclr_copyBuffer", "WRITE_SIZE", kib)])
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    bench.counter_summary(dirs, w)
    t = json.load(open(bench.counters_file(w.name)))
    assert os.path.exists(bench.counters_file(w.name)[:-5] + ".md")
    e = t["kernels"]["attn_bwd_dkdv"]
    assert t["copy_scale"]["fetch"] == pytest.approx(0.5)
    assert t["copy_scale"]["write"] == pytest.approx(1.0)
    assert e["hbm_bytes"] == pytest.approx((1000.0 / 0.5 + 300.0) * 1024.0)
    assert e["mfma_busy"] == pytest.approx(0.4)
    assert e["grbm_clock_ghz"] == pytest.approx(2.0)
    assert e["mfma_tflops_counter"] == pytest.approx(2e8 * 512 / 300e-6 / 1e12)
    assert e["lds_insts_per_mfma"] == pytest.approx(2.0)
    assert e["lds_bank_conflict_rate"] == pytest.approx(0.01)
    # reported for the same kernel, workload and sources only
    assert bench.counters_for("attn_bwd_dkdv", w.name)["hbm_bytes"] == pytest.approx(e["hbm_bytes"])
    assert bench.counters_for("attn_bwd_dkdv", "other_workload") is None
    assert bench.counters_for("attn_fwd", w.name) is None
    t["source_sha256"] = "0" * 64
    json.dump(t, open(bench.counters_file(w.name), "w"))
    assert bench.counters_for("attn_bwd_dkdv", w.name) is None


def test_gpus_above_one_exits_with_a_message(bench, monkeypatch, capsys):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().err


def test_executed_work_counts_the_recomputation(bench):
    import workloads as W
    w = W.WORKLOADS[5]
    alg, ex = bench.kernel_units(w), bench.executed_work(w)
    assert ex["attn_fwd"][0] == alg["attn_fwd"][1]
    assert ex["attn_bwd_dq"][0] == 3 * alg["attn_bwd_dq"][1]
    assert 3 * ex["attn_bwd_dkdv"][0] == 4 * alg["attn_bwd_dkdv"][1]
    # the step's headline counts 12 * hd per causal pair: forward + dk/dv + dq algorithmic
    total = sum(alg[k][1] for k in ("attn_fwd", "attn_bwd_dkdv", "attn_bwd_dq"))
    assert total == 12 * w.head_dim * w.causal_pairs() * w.bh


def test_attainable_bound_from_the_least_traffic(bench):
    """The least-traffic bytes and the attainable bound of the dim768 MHA shape: 202.9 MB
    forward + 405.8 MB backward, 254 FLOP per byte, min(2500, 254 x 8 TB/s) = 2.03 PFLOP/s
    (below the bf16 ridge); the Qwen3 shape (84.4 + 168.8 MB) is bound by the MFMA peak."""
    import workloads as W
    w3, w5 = W.WORKLOADS[3], W.WORKLOADS[5]
    assert bench.min_traffic(w3) == pytest.approx(608.7e6, rel=2e-4)
    assert bench.min_traffic(w5) == pytest.approx(253.2e6, rel=2e-4)
    flop3 = 12 * w3.head_dim * w3.causal_pairs() * w3.bh
    a = bench.attainable(flop3, bench.min_traffic(w3), 500.0, 2500.0)
    assert a["flop_per_byte"] == pytest.approx(254.26, rel=1e-3)
    assert a["tflops"] == pytest.approx(2034.1, rel=1e-3)
    assert a["pct"] == pytest.approx(100.0 * 500.0 / a["tflops"])
    flop5 = 12 * w5.head_dim * w5.causal_pairs() * w5.bh
    assert bench.attainable(flop5, bench.min_traffic(w5), 1.0, 2500.0)["tflops"] == 2500.0
