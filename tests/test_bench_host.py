"""Host-side logic of bench.py (no GPU): percentiles, the reading of the
committed rocprofv3 counter summaries, and the refusal of several GPUs."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

# summary file -> kernel source it was measured on
SUMMARIES = {
    "scatter_apply_long_counters.txt": "scatter.hip",
    "gather_long_counters.txt": "gather.hip",
    "conv_fwd_ple_counters.txt": "ple.hip",
    "conv_bwd_ple_counters.txt": "ple.hip",
    "norm_fwd_ple_counters.txt": "ple.hip",
    "norm_bwd_ple_counters.txt": "ple.hip",
    "pack_values_route_counters.txt": "route.hip",
    "unpack_values_route_counters.txt": "route.hip",
    "unpermute_values_route_counters.txt": "route.hip",
}


def test_percentiles_nearest_rank():
    ms = [float(v) for v in range(1, 12)]          # 1 .. 11
    assert bench.percentiles(ms) == [2.0, 6.0, 10.0]
    assert bench.percentiles([5.0]) == [5.0, 5.0, 5.0]


def fields(path):
    out = {}
    for line in open(path):
        parts = line.split()
        if len(parts) == 2 and not line.startswith("#"):
            out[parts[0]] = parts[1]
    return out


@pytest.mark.parametrize("name", sorted(SUMMARIES))
def test_committed_summaries_are_current_and_plausible(name):
    """Every counter summary names the kernel source it was taken on; that source
    is the committed one, and the measured HBM bytes are at least the algorithmic
    bytes less 5% (a summary below that would mean a counter or scale slip)."""
    path = os.path.join(bench.PROFILES, name)
    f = fields(path)
    assert f["source_sha256_16"] == bench.source_sha(SUMMARIES[name]), \
        "%s was taken on another %s: retake the counters" % (name, SUMMARIES[name])
    hbm = float(f["hbm_bytes_per_launch"])
    alg = float(f["algorithmic_bytes_per_launch"])
    assert hbm == pytest.approx(float(f["fetch_bytes_per_launch"]) + float(f["write_bytes_per_launch"]), abs=2)  # each printed rounded
    assert hbm >= 0.95 * alg
    assert hbm <= 2.0 * alg
    assert bench.counter_traffic(SUMMARIES[name], name) == pytest.approx(hbm)
    text = open(path).read()
    assert "rocprofv3 --pmc FETCH_SIZE" in text and "rocprofv3 --pmc WRITE_SIZE" in text


def test_counter_traffic_refuses_other_sources(tmp_path, monkeypatch):
    (tmp_path / "k.hip").write_bytes(b"kernel v1\n")
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    sha = bench.source_sha("k.hip")
    (tmp_path / "x_counters.txt").write_text("# header 1 2\nsource_sha256_16 %s\nhbm_bytes_per_launch 1200\n" % sha)
    assert bench.counter_traffic("k.hip", "x_counters.txt") == 1200.0
    assert bench.counter_traffic("k.hip", "x_counters.txt", launches_per_step=4) == 300.0
    (tmp_path / "k.hip").write_bytes(b"kernel v2\n")
    assert bench.counter_traffic("k.hip", "x_counters.txt") is None
    assert bench.counter_traffic("k.hip", "missing.txt") is None


def test_kernel_trace_summaries_name_their_command():
    for name in ("kernel_trace_long_context.md", "kernel_trace_ple.md", "kernel_trace_route.md"):
        text = open(os.path.join(bench.PROFILES, name)).read()
        assert re.search(r"rocprofv3 --kernel-trace --stats .* -- python3 \$REPO/bench.py", text), name


def test_several_gpus_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_source_sha_covers_included_headers(tmp_path, monkeypatch):
    (tmp_path / "k.hip").write_text('#include "a.h"\nkernel\n')
    (tmp_path / "a.h").write_text('#include "b.h"\nheader a\n')
    (tmp_path / "b.h").write_text("header b v1\n")
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    first = bench.source_sha("k.hip")
    (tmp_path / "b.h").write_text("header b v2\n")
    assert bench.source_sha("k.hip") != first
