"""The traffic record's arithmetic on synthetic counter files (no GPU): the
copy calibrates each counter, the select's median is scaled by it, and the
record carries the current source's digest (which bench.py checks)."""
import csv
import hashlib
import json

from stable_top_selection_amd import traffic_record as T


def _csv(path, counter, select_values, copy_values):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for v in copy_values:
            w.writerow({"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": counter, "Counter_Value": v})
        for v in select_values:
            w.writerow({"Kernel_Name": "void dcptopk::stable_topk_kernel<512, 2, 16, true, G, P>(G, P, int)",
                        "Counter_Name": counter, "Counter_Value": v})


def test_record_from_counters(tmp_path, monkeypatch):
    monkeypatch.setattr(T, "RECORD", str(tmp_path / "rec.json"))
    _csv(tmp_path / "f.csv", "FETCH_SIZE", [8000.0, 8192.0, 9000.0], [262144.0, 262144.0, 300000.0])
    _csv(tmp_path / "w.csv", "WRITE_SIZE", [4096.0, 4096.0], [524288.0])
    rec = T.main(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0  # copy medians 262144 and 524288 KiB
    assert rec["fetch_bytes_per_launch"] == 8192 * 1024 * 2
    assert rec["write_bytes_per_launch"] == 4096 * 1024
    assert rec["bytes_per_launch"] == 16 * 2**20 + 4 * 2**20 == T.ALGORITHMIC
    with open(T.SOURCE, "rb") as f:
        assert rec["select_source_sha256"] == hashlib.sha256(f.read()).hexdigest()
    assert json.load(open(tmp_path / "rec.json")) == rec
