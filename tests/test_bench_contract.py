"""CPU checks of bench.py's host side: the one-GPU refusal, and the stored
rocprofv3 byte counts it reports as `traffic` being tied to the kernel
sources as they are now."""
import glob
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_stored_traffic_matches_the_current_kernel_sources():
    """The headline workload's score, attention and combine counters were
    taken on the sources in the tree (else `traffic` would be null)."""
    import bench
    w = "qwen3_8b_layer_b32_t32k_bf16"
    for k in ("oasis_score", "oasis_sparse_attn", "oasis_sparse_attn_hbm", "oasis_combine"):
        v = bench.stored_traffic(k, w)
        assert v is not None and v > 0, k


def test_stored_traffic_is_null_for_other_sources_or_workloads(tmp_path, monkeypatch):
    import bench
    assert bench.stored_traffic("oasis_score", "no_such_workload") is None
    data = json.load(open(os.path.join(ROOT, "profiles", "hbm_traffic.json")))
    e = data["workloads"]["qwen3_8b_layer_b32_t32k_bf16"]["oasis_score"]
    e["source_sha256"] = "0" * 64
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "hbm_traffic.json").write_text(json.dumps(data))
    sha = {k: bench.kernel_source_sha(k) for k in bench.KERNEL_SOURCES}
    monkeypatch.setattr(bench, "kernel_source_sha", lambda k: sha[k])
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.stored_traffic("oasis_score", "qwen3_8b_layer_b32_t32k_bf16") is None
    assert bench.stored_traffic("oasis_combine", "qwen3_8b_layer_b32_t32k_bf16") is not None


@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))))
def test_profile_summaries_give_their_commands(path):
    text = open(path).read()
    assert "rocprofv3" in text and "bench.py" in text, os.path.basename(path)
