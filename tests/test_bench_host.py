"""Host-side parts of the benchmark script (no GPU): the one-GPU refusal, the
oracle baseline leg and the lookup of committed traffic counters."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import nm_inputs  # noqa: E402


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line for a configuration that was not measured


def test_cpu_baseline_fields():
    wl = nm_inputs.WORKLOADS[1]
    out = bench.cpu_baseline(wl, 2, 4, wl.Ts[0], reps=1)
    assert out["kind"] == "oracle" and out["unit"] == "TFLOP/s"
    assert out["value"] > 0 and out["cores"] >= 1
    assert out["prune_pack_s"] > 0 and out["decompress_gemm_s"] > 0
    assert f"{wl.R}x{wl.K}x{wl.Ts[0]}" in out["sample"]


def test_cpu_baseline_fp8_and_int8():
    # the 8-bit legs: fp8 times the whole workload's fp64 product, int8 a row sample
    f8 = bench.cpu_baseline(nm_inputs.WORKLOADS[7], 2, 4, 256, reps=1)
    assert f8["unit"] == "TFLOP/s" and f8["value"] > 0 and "4096x4096x256" in f8["sample"]
    i8 = bench.cpu_baseline(nm_inputs.WORKLOADS[6], 2, 4, 64, reps=1)
    assert i8["unit"] == "TOP/s" and i8["value"] > 0 and "first 512 rows" in i8["sample"]


def test_source_hash_is_stable_and_content_based(tmp_path):
    a, b = tmp_path / "a.hip", tmp_path / "b.hip"
    a.write_text("x")
    b.write_text("y")
    h1 = bench.source_hash([str(a), str(b)])
    assert h1 == bench.source_hash([str(a), str(b)]) and len(h1) == 16
    b.write_text("z")
    assert bench.source_hash([str(a), str(b)]) != h1


def test_traffic_lookup_requires_matching_source(monkeypatch, tmp_path):
    (tmp_path / "profiles").mkdir()
    entry = {"source_hash": "0123456789abcdef", "hbm_bytes_per_launch": 3000,
             "read_bytes": 1000, "write_bytes": 2000}
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps({"k": entry}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_from_profile("k", "0123456789abcdef") == 3000
    assert bench.traffic_from_profile("k", "ffffffffffffffff") is None  # stale counters
    assert bench.traffic_from_profile("other", "0123456789abcdef") is None


def test_committed_traffic_entries_are_well_formed():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        d = json.load(f)
    assert d, "no traffic entries committed"
    for key, e in d.items():
        assert len(e["source_hash"]) == 16
        assert e["read_bytes"] > 0 and e["write_bytes"] > 0, key
        # each part is rounded to whole bytes on its own
        assert abs(e["hbm_bytes_per_launch"] - e["read_bytes"] - e["write_bytes"]) <= 1, key
        assert os.path.exists(os.path.join(ROOT, e["profile"])), key


def test_cpu_baseline_train_and_hosts():
    # the training products and the block / diagonal legs, on a few tokens
    tr = bench.cpu_baseline_train(nm_inputs.WORKLOADS[9], 64, reps=1)
    assert tr["kind"] == "oracle" and tr["value"] > 0 and "4096x4096x64" in tr["sample"]
    for wid, kind in ((10, "block"), (11, "diag")):
        h = bench.cpu_baseline_host(nm_inputs.WORKLOADS[wid], 64, reps=1)
        assert h["kind"] == "oracle" and h["value"] > 0 and kind in h["sample"] and "3072x768x64" in h["sample"]


def test_host_workload_inputs():
    # workload 10 keeps about a tenth of its 32 x 32 blocks, workload 11 has 77
    # distinct offsets in [0, 768)
    mask = nm_inputs.WORKLOADS[10].block_mask()
    assert mask.shape == (96, 24) and 0.07 < mask.mean() < 0.13
    offs = nm_inputs.WORKLOADS[11].diag_offsets()
    assert len(offs) == 77 and len(set(offs.tolist())) == 77 and offs.min() >= 0 and offs.max() < 768


def test_kernel_source_hash_covers_one_family(monkeypatch, tmp_path):
    """A family's hash changes with its own sources and the shared ones, not with
    another family's translation unit."""
    csrc = tmp_path / "csrc"
    csrc.mkdir()
    (tmp_path / "include").mkdir()
    (tmp_path / "include" / "nmsparse.h").write_text("h")
    names = {n for fam in bench.KERNEL_SOURCES.values() for n in fam} | set(bench.SHARED_SOURCES)
    for n in names:
        (csrc / n).write_text(n)
    monkeypatch.setattr(bench, "CSRC", str(csrc))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    before = {f: bench.kernel_source_hash(f) for f in bench.KERNEL_SOURCES}
    (csrc / "nm_hosts.hip").write_text("changed")
    after = {f: bench.kernel_source_hash(f) for f in bench.KERNEL_SOURCES}
    assert after["host"] != before["host"]
    assert all(after[f] == before[f] for f in bench.KERNEL_SOURCES if f != "host")
    (csrc / "nm_device.h").write_text("changed")
    assert all(bench.kernel_source_hash(f) != after[f] for f in bench.KERNEL_SOURCES)


def test_every_kernel_source_belongs_to_a_family():
    """A new source file cannot escape the hashes that counter summaries are
    filed under (the prune / pack kernels have no counter summary of their own)."""
    names = {n for n in os.listdir(bench.CSRC) if n.endswith((".hip", ".cpp", ".h"))}
    covered = {n for fam in bench.KERNEL_SOURCES.values() for n in fam} | set(bench.SHARED_SOURCES)
    assert names - covered == {"nm_prune_pack.hip"}
    assert covered <= names
