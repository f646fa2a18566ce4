"""Host-side logic of bench.py (no GPU): the one-GPU contract, the traffic record's source check, the host
description and the oracle-wall helper."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_world_size_above_one_exits_too():
    env = dict(os.environ, WORLD_SIZE="2")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], capture_output=True, text=True,
                       timeout=120, env=env)
    assert r.returncode == 2 and "WORLD_SIZE 2" in r.stderr


def test_source_hash_ignores_comments_and_blank_lines(tmp_path, monkeypatch):
    src = tmp_path / "attention.hip"
    src.write_text("int a;\n// a comment\n\nint b; // trailing\n")
    monkeypatch.setattr(bench, "ATTN_SRC", str(src))
    h1 = bench.attention_source_hash()
    src.write_text("int a;\n\n\n// another comment\nint b;\n")
    assert bench.attention_source_hash() == h1
    src.write_text("int a;\nint c;\n")
    assert bench.attention_source_hash() != h1
    assert len(h1) == 16 and int(h1, 16) >= 0


def test_traffic_record_is_used_only_for_the_source_it_was_taken_on(tmp_path, monkeypatch):
    rec = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    assert bench.measured_traffic() is None                 # no record
    rec.write_text(json.dumps({"attention_source_sha256_16": bench.attention_source_hash(),
                               "hbm_bytes_per_launch": 123456}))
    assert bench.measured_traffic() == 123456
    rec.write_text(json.dumps({"attention_source_sha256_16": "0" * 16, "hbm_bytes_per_launch": 123456}))
    assert bench.measured_traffic() is None                 # taken on another kernel
    rec.write_text("not json")
    assert bench.measured_traffic() is None


def test_committed_traffic_record_is_well_formed():
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    assert t["hbm_bytes_per_launch"] == t["fetch_bytes_per_launch"] + t["write_bytes_per_launch"]
    assert len(t["attention_source_sha256_16"]) == 16
    assert all("rocprofv3" in c for c in t["commands"])


def test_host_description_fields():
    h = bench.host_description()
    assert h["cpu_count"] == os.cpu_count()
    assert isinstance(h["cpu_model"], str) and isinstance(h["blas"], str)
    assert h["blas_threads"] >= 1


def test_oracle_wall_scales_the_sample():
    seen = []
    wall, est = bench.oracle_wall(seen.append, [3, 5], 10)
    assert seen == [3, 5]
    assert wall >= 0.0 and est == pytest.approx(wall / 2 * 10, rel=1e-6, abs=1e-3)
