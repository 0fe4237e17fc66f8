"""Host logic of bench.py (no GPU): the rocprofv3 counter-CSV reader, the HBM traffic
summary written from it, and the guard that reports traffic only for the kernel source
the counters were taken on."""
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
    """rows: (dispatch id, kernel name, counter, value) in rocprofv3's counter CSV layout,
    one row per dimension instance as the tool writes them."""
    os.makedirs(os.path.join(folder, "host"), exist_ok=True)
    path = os.path.join(folder, "host", "1234_counter_collection.csv")
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for d, k, c, v in rows:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": k, "Counter_Name": c,
                        "Counter_Value": v})


def test_pmc_per_dispatch_sums_instances_and_averages_dispatches(bench, tmp_path):
    d = str(tmp_path / "f")
    write_csv(d, [(1, "dkdv_pipe_kernel<128>", "FETCH_SIZE", 100.0),
                  (1, "dkdv_pipe_kernel<128>", "FETCH_SIZE", 50.0),   # second XCC instance
                  (2, "dkdv_pipe_kernel<128>", "FETCH_SIZE", 170.0),
                  (3, "dq_kernel<128>", "FETCH_SIZE", 1e9),            # other kernel
                  (2, "dkdv_pipe_kernel<128>", "WRITE_SIZE", 5.0)])    # other counter
    avg, n = bench.pmc_per_dispatch(d, "FETCH_SIZE", "dkdv")
    assert n == 2 and avg == pytest.approx(160.0)
    with pytest.raises(SystemExit):
        bench.pmc_per_dispatch(d, "FETCH_SIZE", "no_such_kernel")


def test_traffic_summary_scales_by_the_copy_and_guards_the_source(bench, tmp_path,
                                                                 monkeypatch):
    kib = float(1 << 20)  # 1 GiB in KiB
    dirs = [str(tmp_path / n) for n in ("f", "w", "cf", "cw")]
    write_csv(dirs[0], [(1, "dkdv", "FETCH_SIZE", 1000.0)])
    write_csv(dirs[1], [(1, "dkdv", "WRITE_SIZE", 300.0)])
    # the plain 1 GiB copy reads half its bytes in FETCH_SIZE KiB, all in WRITE_SIZE
    write_csv(dirs[2], [(7, "__amd_rocclr_copyBuffer", "FETCH_SIZE", kib / 2)])
    write_csv(dirs[3], [(7, "__amd_rocclr_copyBuffer", "WRITE_SIZE", kib)])
    out = str(tmp_path / "traffic.json")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", out)
    bench.traffic_summary(dirs, "some_workload")
    t = json.load(open(out))
    assert t["copy_scale"]["fetch"] == pytest.approx(0.5)
    assert t["copy_scale"]["write"] == pytest.approx(1.0)
    assert t["hbm_bytes_per_dispatch"] == pytest.approx((1000.0 / 0.5 + 300.0) * 1024.0)
    # reported for the same kernel, workload and sources only
    assert bench.traffic_for("attn_bwd_dkdv", "some_workload") == \
        pytest.approx(t["hbm_bytes_per_dispatch"])
    assert bench.traffic_for("attn_bwd_dkdv", "other_workload") is None
    assert bench.traffic_for("attn_fwd", "some_workload") is None
    t["source_sha256"] = "0" * 64
    json.dump(t, open(out, "w"))
    assert bench.traffic_for("attn_bwd_dkdv", "some_workload") is None


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
