"""Host-side logic of bench.py (no GPU): the one-GPU contract, the counter summaries it reads, the
roofline it picks."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("flops,nbytes,bound", [
    (51.5e9, 3.38e9, "hbm"),        # decode T=128 gate/up: 15 FLOP per byte
    (103e9, 1.13e9, "hbm"),         # skewed decode T=256: 91 FLOP per byte
    (3.30e12, 4.02e9, "mfma"),      # prefill T=8192: 821 FLOP per byte
    (624.0, 1.0, "hbm"), (626.0, 1.0, "mfma"),   # either side of the ridge point, 625
])
def test_roofline_bound(flops, nbytes, bound):
    assert bench.roofline_bound(flops, nbytes) == bound


def test_traffic_only_on_matching_sources(tmp_path):
    f = tmp_path / "k_pmc.txt"
    f.write_text("# summary\n\n    rocprofv3 --pmc FETCH_SIZE ...\n\nkernel_sources_hash: abc123\n"
                 "hbm_bytes_per_launch: 3403699277\n")
    assert bench.load_traffic(str(f), "abc123") == 3403699277
    assert bench.load_traffic(str(f), "def456") is None          # counters taken on other sources
    assert bench.load_traffic(str(tmp_path / "missing.txt"), "abc123") is None


def test_committed_summaries_name_their_kernel_hash():
    # every HBM-counter summary names the sources it was taken on (bench.py ignores it once they change)
    prof = os.path.join(ROOT, "profiles")
    names = [n for n in os.listdir(prof) if n.endswith("_pmc.txt") and not n.endswith("_sq_pmc.txt")]
    assert names
    for name in names:
        text = open(os.path.join(prof, name)).read()
        assert "kernel_sources_hash: " in text and "hbm_bytes_per_launch: " in text, name
        assert "rocprofv3 --pmc FETCH_SIZE" in text and "rocprofv3 --pmc WRITE_SIZE" in text, name


def test_workload_tags_are_distinct():
    from quantized_grouped_gemm_token_amd import workloads
    tags = [bench.workload_tag(s) for s in workloads.WORKLOADS] + [bench.workload_tag(workloads.SKEWED_DECODE)]
    assert len(set(tags)) == len(tags)
