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
        assert len(rec["kernel_source_sha256"]) == 64, key
        if key.startswith("clock:"):
            # shader clock of the prefill: plausible for an MI355X (at most 2.4 GHz)
            _, wl, qk = key.split(":")
            assert qk in ("f16", "fp8", "fp8split"), key
            assert 0.5 < rec["clock_ghz_min"] <= rec["clock_ghz_mean"] <= rec["clock_ghz_max"] <= 2.5, key
            assert rec["num_xcc"] == 8 and rec["dispatches"] > 0, key
            continue
        op = key.split(":")[0] if ":" in key else "prefill"
        assert op in bench.KERNELS, key
        assert rec["hbm_bytes_per_launch"] > 0 and rec["fetch_kib_per_launch"] > 0, key


def test_clock_record_is_per_path_and_source(tmp_path, monkeypatch):
    path = tmp_path / "traffic.json"
    good = {"kernel_source_sha256": bench.kernel_source_hash("prefill"), "clock_ghz_mean": 1.9}
    recs = {f"clock:wl:{bench.DEFAULT_QK}": good, "clock:wl:fp8": dict(good, kernel_source_sha256="0" * 64)}
    path.write_text(json.dumps(recs))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.clock_record("wl", "default")["clock_ghz_mean"] == 1.9   # the library's default path
    assert bench.clock_record("wl", bench.DEFAULT_QK)["clock_ghz_mean"] == 1.9
    assert bench.clock_record("wl", "fp8") is None                       # taken for another source
    assert bench.clock_record("other", "default") is None


def test_mix_ceiling():
    # Q.K^T and P.V carry equal FLOP; f16 products run at half the FP8 rate
    assert abs(bench.qk_ceiling_tflops("default") - 10000.0 / 3.0) < 1e-6
    assert abs(bench.qk_ceiling_tflops("f16") - 10000.0 / 3.0) < 1e-6
    assert bench.qk_ceiling_tflops("fp8") == 5000.0
    # two FP8 products per K operand: Q.K^T at half the FP8 rate, like f16
    assert abs(bench.qk_ceiling_tflops("fp8split") - 10000.0 / 3.0) < 1e-6
