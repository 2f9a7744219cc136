"""Host-side logic of bench.py: the committed traffic records are used only
for the kernel sources they were measured on, and the recorded figures are
consistent with their own calibration.  No GPU."""

import json
import os

import pytest

import bench


def _fake_tree(tmp_path, src_text):
    csrc = tmp_path / "mxfp4_moe_expert_route_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_text(src_text)
    (tmp_path / "profiles").mkdir()
    return csrc


def test_traffic_record_follows_the_source(tmp_path, monkeypatch):
    csrc = _fake_tree(tmp_path, "// kernel v1\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    rec = {"sources": ["k.hip"], "source_hash": bench.kernel_source_hash(["k.hip"]),
           "bytes_per_launch": 123}
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps({"moe_x@w": rec}))
    assert bench.measured_traffic("moe_x", "w") == 123
    assert bench.measured_traffic("moe_x", "other") is None
    (csrc / "k.hip").write_text("// kernel v2\n")              # any edit invalidates it
    assert bench.measured_traffic("moe_x", "w") is None


def test_traffic_missing_file_or_sources(tmp_path, monkeypatch):
    _fake_tree(tmp_path, "x")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("moe_x", "w") is None
    (tmp_path / "profiles" / "traffic.json").write_text(
        json.dumps({"moe_x@w": {"bytes_per_launch": 5}}))
    assert bench.measured_traffic("moe_x", "w") is None


def test_committed_traffic_records_are_self_consistent():
    path = os.path.join(bench.ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        pytest.skip("no traffic records committed")
    with open(path) as f:
        db = json.load(f)
    for key, rec in db.items():
        entry, workload = key.split("@")
        assert entry in bench.ENTRY_KERNELS, key
        assert rec["bytes_per_launch"] == rec["fetch_bytes"] + rec["write_bytes"], key
        # the calibrated counters can only exceed what the kernels must move
        # by re-reads; they cannot fall far below it
        assert rec["bytes_per_launch"] >= 0.99 * rec["algorithmic_bytes"], key
        for f in rec["sources"]:
            assert os.path.exists(os.path.join(bench.ROOT, "mxfp4_moe_expert_route_amd",
                                               "csrc", f)), (key, f)
