"""Host-side checks of bench.py's contract (no GPU): the one-GPU refusal, the
oracle sample it reports as the CPU baseline, and the guard that reports HBM
traffic only for kernel sources the counters were taken on."""
import json
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
sys.path.insert(0, str(ROOT))

import bench  # noqa: E402
from dense_fp32_gemm_f32_amd import inputs  # noqa: E402


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", n],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""   # no JSON line for an unsupported run


def test_cpu_baseline_reports_the_oracle_sample():
    w = inputs.WORKLOADS["square_512"]
    rec = bench.cpu_baseline(w, target_s=0.05)
    assert rec["kind"] == "oracle" and rec["unit"] == "GFLOP/s"
    assert rec["value"] > 0 and rec["cores"] >= 1
    assert "of 512 rows of A" in rec["sample"]


def test_traffic_is_reported_only_for_matching_sources(tmp_path, monkeypatch):
    from dense_fp32_gemm_f32_amd.prof_summary import source_hash
    rec = json.loads((ROOT / "profiles" / "traffic.json").read_text())
    assert rec, "no traffic figures recorded"
    name, entry = next(iter(rec.items()))
    # a figure is reported exactly when its recorded hash matches the sources
    for k, v in rec.items():
        want = v["hbm_bytes_per_launch"] if v["source_sha256"] == source_hash(k) else None
        assert bench.traffic_for(k, v["workload"]) == want
        # nor is a figure reported for another workload of the same kernel
        assert bench.traffic_for(k, v["workload"] + "_other") is None
    # a figure taken on other sources is not reported
    fake = tmp_path / "profiles"
    fake.mkdir()
    (fake / "traffic.json").write_text(json.dumps({name: dict(entry, source_sha256="0" * 64)}))
    monkeypatch.setattr(bench, "ROOT", tmp_path)
    assert bench.traffic_for(name, entry["workload"]) is None
    assert bench.traffic_for("no_such_kernel", entry["workload"]) is None


@pytest.mark.parametrize("name", list(inputs.SHARDS))
def test_shard_is_one_share_of_its_workload(name):
    """Each shard workload is the full product cut 8 ways along one of M, N
    or K, with the full workload's distributions (B's scale depends on K,
    which no split of M or N changes)."""
    s, w = inputs.SHARDS[name], inputs.WORKLOADS[inputs.SHARD_OF[name]]
    ways = inputs.SHARD_WAYS
    cuts = [(s.M * ways, s.N, s.K), (s.M, s.N * ways, s.K), (s.M, s.N, s.K * ways)]
    assert sum(c == (w.M, w.N, w.K) for c in cuts) == 1
    assert (s.dist_a, s.dist_b) == (w.dist_a, w.dist_b)
    if w.dist_b == "u_inv_sqrt_k":
        assert s.K == w.K
    assert s.flops * ways == w.flops


def test_every_traffic_record_has_its_summary():
    """Each recorded traffic figure belongs to a committed profile summary of
    the same kernel on the same workload (no record outlives its summary)."""
    rec = json.loads((ROOT / "profiles" / "traffic.json").read_text())
    for kernel, v in rec.items():
        summary = ROOT / "profiles" / v["summary"]
        assert summary.exists(), (kernel, v["summary"])
        first = summary.read_text().splitlines()[0]
        assert first == f"# {kernel} on {v['workload']}", (kernel, first)
