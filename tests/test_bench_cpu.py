"""bench.py's host-side contract, without a GPU: more than one GPU is
refused before anything touches a device; the roofline's traffic comes from
a committed PMC summary only while the kernel's source is the one it was
measured on; the oracle's thread count stays within one GPU's share of the
host."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _run(args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, env=e, timeout=120)


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], None), (["--gpus", "8"], None),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(args, env):
    r = _run(args, env)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("kernel,workload", [("thc_ring_kernel", "shard"),
                                             ("thc_ring_lane_kernel", "vgg16"),
                                             ("ring_fused_vec_kernel", "shard"),
                                             ("fusion_ring_kernel", "fusion")])
def test_traffic_only_for_the_measured_source(kernel, workload, monkeypatch):
    with open(os.path.join(ROOT, "profiles", bench.PMC_FILE[kernel].format(workload))) as f:
        d = json.load(f)
    assert d["workload"] == workload
    got = bench.traffic_from_profile(workload, kernel)
    if d["ring_src_sha256_16"] == bench.source_hash(kernel):
        assert got == d["hbm_bytes_per_launch"] and got > 0
    else:
        assert got is None
    # another source, or another workload: no figure
    monkeypatch.setattr(bench, "source_hash", lambda k: "0" * 16)
    assert bench.traffic_from_profile(workload, kernel) is None
    monkeypatch.undo()
    assert bench.traffic_from_profile("small", kernel) is None


def test_committed_profiles_match_the_current_sources():
    """Every committed PMC summary of a dominant kernel was taken on the
    source the kernel has now (bench.py reports its traffic)."""
    for kernel, pattern in bench.PMC_FILE.items():
        for name in os.listdir(os.path.join(ROOT, "profiles")):
            prefix, suffix = pattern.split("{}")
            if not (name.startswith(prefix) and name.endswith(suffix)):
                continue
            workload = name[len(prefix):-len(suffix)]
            if workload not in bench.DESCRIPTIONS:
                continue
            with open(os.path.join(ROOT, "profiles", name)) as f:
                d = json.load(f)
            assert d["ring_src_sha256_16"] == bench.source_hash(kernel), name


def test_host_threads_bounds(monkeypatch):
    monkeypatch.setattr(os, "sched_getaffinity", lambda pid: set(range(64)))
    monkeypatch.delenv("OMP_NUM_THREADS", raising=False)
    assert bench.host_threads() == 16
    monkeypatch.setenv("OMP_NUM_THREADS", "4")
    assert bench.host_threads() == 4
    monkeypatch.setenv("OMP_NUM_THREADS", "junk")
    assert bench.host_threads() == 16
    monkeypatch.setattr(os, "sched_getaffinity", lambda pid: {0})
    assert bench.host_threads() == 1
