"""Host-side logic of bench.py (no GPU): percentiles, the reading of the
committed rocprofv3 counter summaries, and the refusal of several GPUs."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench
import hashed_gram_embedding_engram_amd as E  # noqa: E402

# summary file -> kernel source it was measured on
SUMMARIES = {
    "scatter_apply_long_counters.txt": "scatter.hip",
    "gather_long_counters.txt": "lookup.hip",
    "gather_full-sft_counters.txt": "lookup.hip",
    "gather_owner_counters.txt": "gather.hip",
    "scatter_apply_owner_counters.txt": "scatter.hip",
    "scatter_plan_long_counters.txt": "scatter.hip",
    "scatter_plan_owner_counters.txt": "scatter.hip",
    "conv_fwd_ple_counters.txt": "ple.hip",
    "conv_bwd_ple_counters.txt": "ple.hip",
    "norm_fwd_ple_counters.txt": "ple.hip",
    "norm_bwd_ple_counters.txt": "ple.hip",
    "pack_values_route_counters.txt": "route.hip",
    "unpack_unpermute_values_route_counters.txt": "route.hip",
    "backward_send_route_counters.txt": "route.hip",
    "owner_response_owner_counters.txt": "route.hip",
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
    """Every counter summary names the kernel source it was taken on.  A summary
    taken on another source is never used (the bench line's traffic is null
    for it).  A current one's measured HBM bytes are at least the compulsory
    bytes (each distinct row moved once; for kernels without row reuse, the
    algorithmic bytes) less 5%: below that would mean a counter or scale slip."""
    path = os.path.join(bench.PROFILES, name)
    f = fields(path)
    text = open(path).read()
    assert "rocprofv3 --pmc FETCH_SIZE" in text and "rocprofv3 --pmc WRITE_SIZE" in text
    if f["source_sha256_16"] != bench.source_sha(SUMMARIES[name]):
        assert bench.counter_traffic(SUMMARIES[name], name) is None
        pytest.skip("%s was taken on another %s: the bench reports its traffic as null" % (name, SUMMARIES[name]))
    hbm = float(f["hbm_bytes_per_launch"])
    alg = float(f["algorithmic_bytes_per_launch"])
    assert hbm == pytest.approx(float(f["fetch_bytes_per_launch"]) + float(f["write_bytes_per_launch"]), abs=2)  # each printed rounded
    comp = float(f.get("compulsory_bytes_per_launch", alg))
    assert comp <= alg
    assert hbm >= 0.95 * comp
    assert hbm <= 2.0 * alg
    assert bench.counter_traffic(SUMMARIES[name], name) == pytest.approx(hbm)


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
    for name in ("kernel_trace_long_context.md", "kernel_trace_full_sft.md", "kernel_trace_owner.md",
                 "kernel_trace_ple.md", "kernel_trace_route.md"):
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


def test_sort_nominal_bytes():
    """The plan's traffic model: 29-bit keys take four passes, 23-bit keys three."""
    n, u = 1000, 600
    assert bench.sort_nominal_bytes(n, 320_001_536, u) == 92 * n + 8 * u
    assert bench.sort_nominal_bytes(n, 5_000_024) == 68 * n
    assert bench.sort_nominal_bytes(n, (1 << 24) - 1) == 68 * n   # the sentinel fits 24 bits
    assert bench.sort_nominal_bytes(n, 1 << 24) == 88 * n           # it needs a 25th
    assert bench.sort_nominal_bytes(n, 320_001_536, u, from_tokens=True) == 92 * n + 8 * u - 8 * n + n // 2
    # from tokens with the released heads the sort runs per head in three passes: one 20-B pass less
    p = bench.plan_passes(320_001_536, True, E.QWEN3_8_FLASH_NEXT_NGRAM_HEAD_VOCAB_SIZES,
                          E.QWEN3_8_FLASH_NEXT_NGRAM_HEAD_OFFSETS)
    assert p == 3
    assert bench.sort_nominal_bytes(n, 320_001_536, u, True, p) == 72 * n + 8 * u - 8 * n + n // 2


def test_plan_passes_split_rule():
    """Per-head passes only when the head ranges are disjoint, ascending and inside the shard."""
    mods = [60_000] * 16
    offs = [60_000 * h for h in range(16)]
    assert bench.plan_passes(960_000, False, mods, offs) == 3           # rows: the whole sort
    assert bench.plan_passes(960_000, True, mods, offs) == 2            # 16-bit heads, 20-bit table
    assert bench.plan_passes(960_000, True, mods, offs[::-1]) == 3      # descending ranges
    assert bench.plan_passes(959_999, True, mods, offs) == 3            # last head past the shard
    assert bench.plan_passes(1_700_000, True, [100_000] * 16, [100_000 * h for h in range(16)]) == 2  # 8 + 9 bits
    # the sentinel 65,536 needs a 17th bit: three passes whole, two per head
    assert bench.plan_passes(65_536, False, [4_096] * 16, [4_096 * h for h in range(16)]) == 3
    assert bench.plan_passes(65_536, True, [4_096] * 16, [4_096 * h for h in range(16)]) == 2


def test_route_cpu_baseline_runs_on_tiny_inputs():
    """The routing line's oracle baseline (pack, unpack and unpermute through the
    routing oracle) on CPU tensors of a tiny world."""
    import numpy as np
    import torch
    rng = np.random.default_rng(3)
    ids = torch.from_numpy(rng.integers(0, 1000, size=64).astype(np.int64))
    vals = torch.from_numpy(rng.standard_normal((64, 8)).astype(np.float32))
    counts = np.bincount(ids.numpy() // 250, minlength=4)
    wl = {"world": 4, "num_embeddings": 1000, "rots": [{"ids": ids, "vals": vals, "cap": int(counts.max())}]}
    out = bench.route_cpu_baseline(wl, target_seconds=0.01)
    assert out["value"] > 0 and out["unit"] == "lookups/s" and out["kind"] == "oracle"


def test_ple_cpu_baseline_runs_on_tiny_inputs():
    import torch
    g = torch.Generator().manual_seed(4)
    B, S, C = 2, 16, 32
    rot = {"x": torch.randn((B, S, C), generator=g), "dy": torch.randn((B, S, C), generator=g),
           "halo": torch.randn((B, 9, C), generator=g), "conv_w": torch.randn((C, 4), generator=g),
           "conv_b": torch.randn(C, generator=g), "norm_w": torch.randn(C, generator=g)}
    wl = {"rots": [rot], "batch": B, "seq": S, "channels": C, "group": 8}
    out = bench.ple_cpu_baseline(wl, sample_rows=1, target_seconds=0.01)
    assert out["value"] > 0 and out["unit"] == "tokens/s" and out["kind"] == "oracle"
