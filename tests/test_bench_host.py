"""Host logic of the bench (CPU only): the HBM-traffic ingestion from
rocprofv3 counter output and the source-hash gate on its use."""
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
