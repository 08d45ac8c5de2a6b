"""Host-side contract of bench.py that needs no GPU: the one-GPU limit and
the staleness rule of the stored HBM-traffic records."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_exits_with_a_message(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""


def test_traffic_record_is_used_only_while_its_sources_are_unchanged(tmp_path, monkeypatch):
    import bench
    srcs = ["common.hpp", "kernels.hpp"]
    rec = {"k": {"source_sha": bench.src_sha(*srcs), "bytes_per_launch": 1234.0}}
    (tmp_path / "pmc_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.traffic_from_profile("k", srcs, None) == 1234.0
    # another source set (a stand-in for an edited kernel) has another hash
    assert bench.traffic_from_profile("k", srcs + ["decode.hip"], None) is None
    assert bench.traffic_from_profile("missing", srcs, None) is None


def test_stored_traffic_records_name_their_sources():
    with open(os.path.join(ROOT, "profiles", "pmc_traffic.json")) as f:
        recs = json.load(f)
    assert recs
    for key, r in recs.items():
        assert r["source_files"], key
        assert r["bytes_per_launch"] > 0, key
        for n in r["source_files"]:
            assert os.path.exists(os.path.join(ROOT, "bit_expert_ffn_router_amd", "csrc", n)), (key, n)
