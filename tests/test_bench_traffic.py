"""bench.py's recorded HBM traffic: a record counts only for the operation and
workload it was taken for, and only while its kernel source is unchanged."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_records_are_per_operation_and_source(tmp_path, monkeypatch):
    path = tmp_path / "traffic.json"
    recs = {
        "wl": {"kernel_source_sha256": bench.kernel_source_hash("prefill"), "hbm_bytes_per_launch": 1.0},
        "quantize_append:wl": {"kernel_source_sha256": bench.kernel_source_hash("quantize_append"),
                               "hbm_bytes_per_launch": 2.0},
        "decode:wl": {"kernel_source_sha256": "0" * 64, "hbm_bytes_per_launch": 3.0},
    }
    path.write_text(json.dumps(recs))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.recorded_traffic("wl") == 1.0
    assert bench.recorded_traffic("wl", "quantize_append") == 2.0
    assert bench.recorded_traffic("wl", "decode") is None        # taken for another source
    assert bench.recorded_traffic("other") is None
    assert bench.recorded_traffic("other", "quantize_append") is None


def test_committed_records_are_well_formed():
    # every committed record names a known operation and holds a source hash and
    # positive byte counts (a record whose source changed since is reported as
    # null by the bench, not used)
    recs = json.load(open(bench.TRAFFIC_FILE))
    for key, rec in recs.items():
        op = key.split(":")[0] if ":" in key else "prefill"
        assert op in bench.KERNELS, key
        assert len(rec["kernel_source_sha256"]) == 64, key
        assert rec["hbm_bytes_per_launch"] > 0 and rec["fetch_kib_per_launch"] > 0, key
