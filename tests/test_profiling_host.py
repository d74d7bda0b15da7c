"""Host-side checks of the rocprofv3 summary helpers used by bench.py."""
import csv
import json
import os

from token_sampling_scaled_amd import profiling

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _counter_csv(path, rows):
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(cols, r)))


def test_source_digest_is_stable():
    a = profiling.source_digest()
    assert a == profiling.source_digest() and len(a) == 64


def test_per_dispatch_sums_instances(tmp_path):
    p = tmp_path / "c.csv"
    _counter_csv(p, [(1, "k", "FETCH_SIZE", 1.5), (1, "k", "FETCH_SIZE", 2.5),
                     (2, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 7.0)])
    d = profiling.per_dispatch(str(p))
    assert d[1] == ("k", {"FETCH_SIZE": 4.0})
    assert d[2][1]["FETCH_SIZE"] == 7.0


def test_traffic_record_scales_by_copy(tmp_path, capsys):
    f = tmp_path / "f.csv"
    w = tmp_path / "w.csv"
    # copy of 1 MiB: FETCH_SIZE reads half of it, WRITE_SIZE all of it
    _counter_csv(f, [(1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 512.0),
                     (2, "my_kernel<1>", "FETCH_SIZE", 100.0), (3, "my_kernel<1>", "FETCH_SIZE", 300.0)])
    _counter_csv(w, [(1, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 1024.0),
                     (2, "my_kernel<1>", "WRITE_SIZE", 4.0)])
    profiling.main(["traffic", "--fetch", str(f), "--write", str(w), "--copy-mib", "1",
                    "--kernel", "my_kernel", "--workload", "wl", "--command-fetch", "a",
                    "--command-write", "b"])
    out = capsys.readouterr().out
    (tmp_path / "summary.md").write_text(out)
    recs = profiling.read_records(str(tmp_path))
    assert len(recs) == 1
    rec = recs[0]
    assert rec["fetch_bytes"] == 200.0 * 2 * 1024
    assert rec["write_bytes"] == 4.0 * 1024
    assert rec["source_sha256"] == profiling.source_digest()


def test_committed_records_parse():
    for rec in profiling.read_records(os.path.join(ROOT, "profiles")):
        json.dumps(rec)
        assert rec["bytes_per_launch"] > 0 and len(rec["source_sha256"]) == 64
