"""Host logic of the bench (CPU only): the HBM-traffic ingestion from
rocprofv3 counter output and the source-hash gate on its use, the
kernel-trace summary set against the bench line, and the CPU baseline's
oracle legs on a small workload."""
import json
import sqlite3

import bench

GIB_KIB = float(1 << 20)


def _counter_db(path, rows):
    con = sqlite3.connect(path)
    con.execute("create table counters_collection (counter_name text, kernel_name text, grid_size integer, "
                "dispatch_id integer, value real)")
    con.executemany("insert into counters_collection values (?, ?, ?, ?, ?)", rows)
    con.commit()
    con.close()


def _rows(counter, copy_kib, attn_kib, gather_kib):
    # a 1 GiB calibration copy (plus a small clone), the active and the dense
    # attention launch, one gather launch; one row per (dispatch, XCD) as the
    # counters come, summed per dispatch by the ingestion
    r = []
    for x in range(8):
        r.append((counter, "__amd_rocclr_copyBuffer", 131072, 1, copy_kib / 8))
        r.append((counter, "__amd_rocclr_copyBuffer", 512, 2, 1.0))
        r.append((counter, "jano::(anonymous namespace)::attn_fwd_d128_kernel(a, b)", 1003520, 3, attn_kib / 8))
        r.append((counter, "jano::(anonymous namespace)::attn_fwd_d128_kernel(a, b)", 4034560, 4, 4 * attn_kib / 8))
        r.append((counter, "jano::(anonymous namespace)::gather_rows_v16(a)", 11819520, 5, gather_kib / 8))
    return r


def test_ingest_scales_by_the_copy_and_splits_attention_grids(tmp_path):
    f_db, w_db, out = str(tmp_path / "f.db"), str(tmp_path / "w.db"), str(tmp_path / "traffic.json")
    # FETCH_SIZE reads the 1 GiB copy as half its bytes; WRITE_SIZE as all of them
    _counter_db(f_db, _rows("FETCH_SIZE", GIB_KIB / 2, 1000.0, 300.0))
    _counter_db(w_db, _rows("WRITE_SIZE", GIB_KIB, 50.0, 100.0))
    got = bench.ingest_counters(f_db, w_db, "wl", out_path=out)
    assert got["calibration"]["fetch_factor"] == 2.0 and got["calibration"]["write_factor"] == 1.0
    assert got["attention"]["grid_threads"] == 1003520
    assert got["attention_dense"]["grid_threads"] == 4034560
    assert got["attention"]["fetch_bytes"] == round(1000.0 * 1024 * 2)
    assert got["attention"]["write_bytes"] == round(50.0 * 1024)
    assert got["attention_dense"]["fetch_bytes"] == round(4000.0 * 1024 * 2)
    assert got["gather"]["hbm_bytes_per_launch"] == round(300.0 * 1024 * 2 + 100.0 * 1024)
    assert "scatter" not in got
    with open(out) as f:
        assert json.load(f)["wl"] == got


def test_traffic_used_only_for_the_profiled_source(tmp_path):
    out = str(tmp_path / "traffic.json")
    src = "attention.hip"
    entry = {"source": src, "source_sha256_16": bench.kernel_source_hash(src), "hbm_bytes_per_launch": 123}
    with open(out, "w") as f:
        json.dump({"wl": {"attention": entry, "gather": dict(entry, source="rows.hip",
                                                             source_sha256_16="0" * 16)}}, f)
    assert bench.load_traffic("attention", "wl", path=out) == 123
    assert bench.load_traffic("gather", "wl", path=out) is None      # source changed since
    assert bench.load_traffic("scatter", "wl", path=out) is None     # never profiled
    assert bench.load_traffic("attention", "other", path=out) is None


def test_trace_summary_sets_the_profile_against_the_line(tmp_path):
    # a kernel trace whose headline attention launches take 20, 10, 10 ms
    # (the first is the cold one) and a bench line with frac for 10 ms
    import csv
    trace = tmp_path / "t.csv"
    n_act, N, H, d = 18468, 75600, 40, 128
    grid = (44 + 7) * H * 512
    with open(trace, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Grid_Size_Y",
                    "Workgroup_Size_X"])
        t = 0
        for dur in (20e6, 10e6, 10e6):
            w.writerow(["jano::(anonymous namespace)::attn_fwd_d128_kernel(x)", t, t + int(dur),
                        grid, 1, 512])
            t += int(dur) + 1000
        w.writerow(["gather_rows_v16(x)", t, t + 60000, 11819520, 1, 640])
    flops = 4.0 * n_act * N * H * d
    achieved = flops / 10e-3 / 1e12
    line = {"metric": "m", "value": 1.0, "ms_per_step": 10.5, "config": {"workload": "w", "n_act": n_act,
            "tokens": N, "heads": H, "head_dim": d},
            "roofline": {"achieved": achieved, "frac": achieved / 2500.0, "tiles_per_head_384_256": [44, 7]}}
    log = tmp_path / "b.log"
    log.write_text("bench: noise\n" + json.dumps(line) + "\n")
    out = tmp_path / "s.md"
    bench.summarize_trace(str(trace), str(log), str(out), "rocprofv3 ... -- python bench.py")
    text = out.read_text()
    assert "2 dispatches after the first, average 10.000 ms" in text
    assert "(ratio 1.0000)" in text
    assert "| 3 | 13333.33 | 10000.00 |" in text          # calls, mean, mean without the first


def test_cpu_baseline_runs_every_leg_on_a_small_workload():
    from token_sparse_attention_block_amd import configs, synth
    cfg = configs.TINY
    Qb, Kb, Vb = synth.qkv_bits(cfg)
    sc = cfg.schedule
    got = bench.cpu_baseline(cfg, synth, Qb, Kb, Vb, 450, 300, sc.W + 1, seconds_hint=0.2)
    assert got["kind"] == "oracle" and got["unit"] == "TFLOP/s" and got["value"] > 0
    assert set(got["oracle_ms"]) == {"analyze_scores", "levels", "schedule", "gather", "scatter"}
    assert got["oracle_step_ms_extrapolated"] >= got["oracle_attention_ms_extrapolated"]
    assert got["cores"] >= 1


def test_more_than_one_gpu_exits_with_a_message():
    # the path runs on one GPU; asking for more exits before touching a device
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
