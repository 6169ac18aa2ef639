"""Benchmark of the Engram n-gram embedding hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long]

A step is one pass of the whole path over one batch of synthetic tokens:
engram_hash (raw IDs -> 16 head rows) -> engram_gather (rows -> table values)
-> engram_scatter_add (output gradients -> per-row gradient sums).  Inputs are
resident in HBM before the timed region starts; W untimed steps, then exactly
K timed steps between two device synchronisations.  Four independent token
streams, gradients and output buffers rotate so caches cannot replay a step.

Default workload ("long"): one packed 262,144-token THD stream (log-uniform
document lengths in [64, 16,384], each ending in EOS, Zipf(1.1) tokens) against
the full 320,001,536 x 160 bf16 table (102.4 GB) held whole on the GPU, forward
plus backward with the compact (distinct rows + sums) gradient output:
4,194,304 (token x head) lookups per step.

Workload "ple" times the step after the lookup instead: the PLE causal short
convolution (kernel 4, dilation 3) followed by the grouped RMSNorm over the
four 2,560-wide HyperConnection branches, forward and backward, on a batch of
8 x 4,096 tokens x 10,240 bf16 channels; its line reports tokens/s.

Workload "route" times the single-GPU half of the row-owner exchange for one
request rank of a world-64 owner group (8 x 4,096 Zipf(1.2) tokens, 524,288
lookups): group by owner, validate the segments, pack the IDs to the agreed
capacity, the owner's unpack of them, the owner's pack of the 320-B value rows,
the requester's unpack and its return to request order.  The all-to-all
itself needs several GPUs and is not timed; the exchange is the identity.

Printed: one JSON line with lookups/s, the roofline of the dominant kernel
(timed with HIP events on the stream the kernels run on) and the oracle's CPU
throughput on the same stream (rank 0, N = 1).  After the timed steps the
gather, the plan and the apply also run one at a time, untimed by the step
clock (phases_alone_ms_p50, gather_alone, backward_plan_then_apply).
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Engram (token x head) lookups/sec fwd+bwd and achieved HBM GB/s vs peak"
HBM_PEAK_GBPS = 8000.0
EVENT_STRIDE = 4  # timed steps per step that carries the dominant phase's events
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "hashed_gram_embedding_engram_amd", "csrc")


def log(msg):
    """A progress line on stderr (the JSON result is the only line on stdout)."""
    print("[bench %7.1fs] %s" % (time.perf_counter() - _T0, msg), file=sys.stderr, flush=True)


_T0 = time.perf_counter()


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long", choices=["long", "full-sft", "owner", "sft", "ple", "route"])
    ap.add_argument("--rotations", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one plain 1 GiB device copy first (reference for HBM byte counters)")
    ap.add_argument("--no-alone", action="store_true",
                    help="skip the phases-one-at-a-time launches after the timed steps (profiler runs)")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the HBM ceiling probes")
    ap.add_argument("--no-extra-configs", action="store_true",
                    help="long workload: skip the full-table SFT forward and owner-shard lines after the headline")
    return ap.parse_args()


def source_sha(name):
    """SHA-256 prefix of a kernel source together with the local headers it
    includes (recursively, in include order), so that a header edit marks
    the counter summaries of every kernel built from it as stale."""
    h = hashlib.sha256()
    seen = set()

    def add(fname):
        if fname in seen or not os.path.exists(os.path.join(CSRC, fname)):
            return
        seen.add(fname)
        with open(os.path.join(CSRC, fname), "rb") as f:
            data = f.read()
        h.update(data)
        for line in data.decode(errors="replace").splitlines():
            line = line.strip()
            if line.startswith('#include "') and line.endswith('"'):
                add(line[len('#include "'):-1])

    add(name)
    return h.hexdigest()[:16]


def counter_traffic(kernel_file, summary_name, launches_per_step=1):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None when
    the summary is missing or was taken on a different kernel source."""
    path = os.path.join(PROFILES, summary_name)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        parts = line.strip().split()
        if len(parts) == 2 and not line.startswith("#"):
            fields[parts[0]] = parts[1]
    if fields.get("source_sha256_16") != source_sha(kernel_file):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"]) / launches_per_step
    except (KeyError, ValueError):
        return None


def build_workload(name, rotations, dev, table=None):
    import numpy as np
    import torch

    import hashed_gram_embedding_engram_amd as E
    import workloads as W

    spec = E.qwen3_8_flash_next_spec()
    if name in ("long", "full-sft"):
        table_rows, row_begin = W.FULL_ROWS, 0
    elif name == "owner":
        table_rows, row_begin = W.OWNER_ROWS, 0
    else:
        ws = W.sft_spec()
        spec = E.make_hash_spec(3, 8, ws["eos"], E.QWEN3_8_FLASH_NEXT_LAYER_MULTIPLIERS, ws["vocab_sizes"],
                                ws["offsets"])
        table_rows, row_begin = ws["num_rows"], 0
    if table is None or tuple(table.shape) != (table_rows, W.DIM):
        table = torch.empty((table_rows, W.DIM), dtype=torch.bfloat16, device=dev)
        W.fill_normal_(table, seed=1234)

    batches = []
    for r in range(rotations):
        if name == "long":
            ids, _ = W.long_context_stream(seed=r)
        elif name == "owner":
            ids = W.owner_token_batches(seeds=range(100 + 64 * r, 164 + 64 * r)).reshape(-1, 4096)
        else:
            ids, _ = W.sft_batch(seed=r)
        tokens = torch.from_numpy(ids).to(dev)
        rows = torch.empty(tuple(tokens.shape) + (spec.num_heads,), dtype=torch.int64, device=dev)
        if name == "owner":
            # The owner receives only its own rows: emulated here by the request
            # ranks' hash followed by a filter (input preparation, not timed).
            all_rows = E.engram_hash(tokens, spec).reshape(-1)
            owner_rows = all_rows[all_rows < W.OWNER_ROWS].contiguous()
            tokens, rows = None, owner_rows
            # The same rows as the exchange delivers them: each request rank's
            # segment in its own block of the agreed capacity.
            recv_counts = (all_rows.view(64, -1) < W.OWNER_ROWS).sum(1).to(torch.int64).contiguous()
            cap = int(recv_counts.max().item())
            recv = {"counts": recv_counts, "capacity": cap,
                    "ids": E.engram_pack_fixed_capacity(owner_rows, recv_counts, 64, cap, fill=-1),
                    "vals": torch.empty((64, cap, W.DIM), dtype=torch.bfloat16, device=dev)}
            del all_rows
        n = rows.numel()
        g = torch.Generator(device=dev)
        g.manual_seed(1000 + r)
        b = {"ids": ids, "tokens": tokens, "rows": rows, "n": n,
             "out": torch.empty((n, W.DIM), dtype=torch.bfloat16, device=dev),
             "status": torch.empty((), dtype=torch.int64, device=dev),
             "plan_status": torch.empty((), dtype=torch.int64, device=dev)}
        if name in ("long", "owner"):
            b["dy"] = torch.randn((n, W.DIM), generator=g, device=dev).to(torch.bfloat16)
        if name == "owner":
            # the output gradients as the exchange returns them to the owner
            recv["dy"] = E.engram_pack_fixed_capacity(b["dy"], recv["counts"], 64, recv["capacity"], fill=0)
            b["recv"] = recv
        if name == "long":
            b["compact"] = (torch.empty(n, dtype=torch.int64, device=dev),
                            torch.empty((n, W.DIM), dtype=torch.float32, device=dev),
                            torch.empty((), dtype=torch.int64, device=dev))
        batches.append(b)
    grad_dense = None
    if name == "owner":
        grad_dense = torch.zeros((table_rows, W.DIM), dtype=torch.float32, device=dev)
    n_max = max(b["n"] for b in batches)
    workspace = None
    if name in ("long", "owner"):
        workspace = torch.empty(E.engram_scatter_add_workspace(n_max, table_rows, W.DIM), dtype=torch.uint8,
                                device=dev)
    return {"side": torch.cuda.Stream(device=dev), "name": name, "spec": spec, "table": table, "row_begin": row_begin, "table_rows": table_rows, "batches": batches,
            "grad_dense": grad_dense, "workspace": workspace, "backward": name in ("long", "owner")}


def run_step(wl, b, ev=None):
    """One step.  From tokens (long, sft, full-sft): the fused hash-and-gather
    forward on the main stream; with a backward, the plan (sort by row) from
    the same tokens, which hashes the rows itself, on a side stream beside it;
    the apply once both are done.  No rows array is written or read.  From
    rows (the owner shard, which receives its rows): the plan, a chain of
    short launches and the longer of the two there, on the main stream, and
    the gather beside it on the side stream, then the apply.  A stream that
    waits on the other starts some microseconds late, so the longer chain goes
    on the main stream.  ev: events (step start, unused, forward end, plan
    start, plan end, apply start, apply end); an entry may be None, and only
    the events given are recorded."""
    import torch

    import hashed_gram_embedding_engram_amd as E
    main = torch.cuda.current_stream()
    side = wl["side"]

    def mark(k, stream):
        if ev and ev[k] is not None:
            ev[k].record(stream)

    compact = b.get("compact")

    def plan(stream):
        args = dict(workspace=wl["workspace"], uniq_rows=compact[0] if compact else None,
                    num_uniq=compact[2] if compact else None, status=b["plan_status"], stream=stream)
        if b["tokens"] is not None:   # the rows hashed inside the plan
            E.engram_scatter_add_plan_from_tokens(b["tokens"], wl["spec"], wl["table_rows"], b["dy"].shape[-1],
                                                  wl["row_begin"], **args)
        else:
            E.engram_scatter_add_plan(b["rows"], wl["table_rows"], b["dy"].shape[-1], wl["row_begin"], **args)

    mark(0, main)
    if wl["backward"] and b["tokens"] is None:
        side.wait_stream(main)        # the gather starts once the previous step is done
        mark(3, main)
        plan(main)
        mark(4, main)
        E.engram_gather(wl["table"], b["rows"], wl["row_begin"], out=b["out"], status=b["status"], validate=False,
                        stream=side)
        mark(2, side)
    else:
        if wl["backward"]:
            side.wait_stream(main)
            mark(3, side)
            plan(side)
            mark(4, side)
        if b["tokens"] is not None:
            E.engram_hash_gather(b["tokens"], wl["spec"], wl["table"], wl["row_begin"], out=b["out"],
                                 status=b["status"], validate=False)
        else:
            E.engram_gather(wl["table"], b["rows"], wl["row_begin"], out=b["out"], status=b["status"],
                            validate=False)
        mark(2, main)
    if wl["backward"]:
        main.wait_stream(side)
        mark(5, main)
        E.engram_scatter_add_apply(b["dy"], b["n"], wl["table_rows"], wl["workspace"], wl["row_begin"],
                                   grad_dense=wl["grad_dense"], uniq_grad=compact[1] if compact else None)
        mark(6, main)


def phases_alone(wl, k):
    """Median ms of the forward gather and the plan (each from tokens when the
    workload starts from them, with the hash inside) and the apply, each run by
    itself on the main stream with nothing beside it, over k launches rotating
    through the input sets (outside the timed steps)."""
    import torch

    import hashed_gram_embedding_engram_amd as E
    R = len(wl["batches"])
    ev = lambda: torch.cuda.Event(enable_timing=True)
    ms = {"gather": [], "scatter_plan": [], "scatter_apply": []}
    events = []
    for i in range(k + 2):  # queued back to back, as in the steps
        b = wl["batches"][i % R]
        e = [ev() for _ in range(6)]
        events.append(e)
        e[0].record()
        if b["tokens"] is not None:  # the forward as the steps run it: fused hash and gather
            E.engram_hash_gather(b["tokens"], wl["spec"], wl["table"], wl["row_begin"], out=b["out"],
                                 status=b["status"], validate=False)
        else:
            E.engram_gather(wl["table"], b["rows"], wl["row_begin"], out=b["out"], status=b["status"],
                            validate=False)
        e[1].record()
        if wl["backward"]:
            compact = b.get("compact")
            args = dict(workspace=wl["workspace"], uniq_rows=compact[0] if compact else None,
                        num_uniq=compact[2] if compact else None, status=b["plan_status"])
            e[2].record()
            if b["tokens"] is not None:   # as the steps run it: the rows hashed inside the plan
                E.engram_scatter_add_plan_from_tokens(b["tokens"], wl["spec"], wl["table_rows"], b["dy"].shape[-1],
                                                      wl["row_begin"], **args)
            else:
                E.engram_scatter_add_plan(b["rows"], wl["table_rows"], b["dy"].shape[-1], wl["row_begin"], **args)
            e[3].record()
            e[4].record()
            E.engram_scatter_add_apply(b["dy"], b["n"], wl["table_rows"], wl["workspace"], wl["row_begin"],
                                       grad_dense=wl["grad_dense"], uniq_grad=compact[1] if compact else None)
            e[5].record()
    torch.cuda.synchronize()
    for e in events[2:]:  # the first two are warm-up
        ms["gather"].append(e[0].elapsed_time(e[1]))
        if wl["backward"]:
            ms["scatter_plan"].append(e[2].elapsed_time(e[3]))
            ms["scatter_apply"].append(e[4].elapsed_time(e[5]))
    return {key: round(sorted(v)[len(v) // 2], 4) for key, v in ms.items() if v}


def percentiles(ms):
    """p10, p50 and p90 of a list of times (nearest rank), rounded to 0.1 us."""
    v = sorted(ms)
    at = lambda q: v[min(len(v) - 1, int(q * (len(v) - 1) + 0.5))]
    return [round(at(0.1), 4), round(at(0.5), 4), round(at(0.9), 4)]


def host_info():
    """The CPUs this process may run on, their model name and the host memory."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    info = {"cpus_available": len(os.sched_getaffinity(0)), "cpu_model": model}
    try:
        import psutil
        vm = psutil.virtual_memory()
        info.update({"mem_total_gb": round(vm.total / 1e9, 1), "mem_available_gb": round(vm.available / 1e9, 1)})
    except Exception:
        pass
    return info


def host_table(wl, margin=64e9):
    """The table as the oracle reads it: a host copy of the whole table when host
    memory holds it with `margin` to spare (copied from the GPU in 1 GiB
    chunks), else None."""
    import numpy as np
    import torch
    table = wl["table"]
    need = table.numel() * table.element_size()
    try:
        import psutil
        if psutil.virtual_memory().available < need + margin:
            return None
    except Exception:
        return None
    host = np.empty(tuple(table.shape), dtype=np.uint16)
    step = max(1, (1 << 30) // (table.shape[1] * table.element_size()))
    for r0 in range(0, table.shape[0], step):
        r1 = min(table.shape[0], r0 + step)
        torch.from_numpy(host[r0:r1].view(np.int16)).copy_(table[r0:r1].view(torch.int16))
    return host


def cpu_baseline(wl, target_seconds=10.0, mt_seconds=5.0):
    """The oracle on the same streams as the timed steps, twice: the plain
    single-threaded C oracle, rotation after rotation until at least
    `target_seconds` of its work has been timed, then its OpenMP twin (same
    bits, every host core the process may use) until at least `mt_seconds`.
    Each pass is hash, gather, compact scatter-add.  The gather reads a host
    copy of the whole table when host memory holds one, else a host copy of
    exactly the rows the stream reads (renumbered)."""
    import numpy as np
    import torch

    import workloads as W
    from oracle import c_oracle, constants as C

    if wl["name"] == "sft":
        ws = W.sft_spec()
        mods, offs = ws["vocab_sizes"], ws["offsets"]
    else:
        mods, offs = C.head_vocab_sizes(), C.head_offsets()
    if any(b["tokens"] is None for b in wl["batches"]):
        return None
    log("cpu baseline: host copy of the table")
    full = host_table(wl)
    log("cpu baseline: %s" % ("whole table on the host" if full is not None else "distinct rows only"))
    prep = []
    for b in wl["batches"]:
        ids = b["ids"]
        n = ids.size * 16
        dy = b["dy"][:n].cpu().view(torch.int16).numpy().view(np.uint16) if "dy" in b else None
        if full is not None:
            prep.append((ids, full, None, dy, wl["row_begin"]))
            continue
        # no room for the whole table: the rows this stream reads, renumbered (untimed)
        rows_prep = c_oracle.hash_input_ids(ids, 3, 8, C.EOS_TOKEN_ID, 0, C.LAYER_MULTIPLIERS, mods, offs).reshape(-1)
        uniq, inv = np.unique(rows_prep, return_inverse=True)
        sub = wl["table"][torch.from_numpy(uniq).to(wl["table"].device)].cpu().view(torch.int16).numpy() \
            .view(np.uint16)
        prep.append((ids, sub, inv.astype(np.int64), dy, 0))

    def run(mt, budget):
        hash_fn = c_oracle.hash_input_ids_mt if mt else c_oracle.hash_input_ids
        gather_fn = c_oracle.gather_mt if mt else c_oracle.gather
        scatter_fn = c_oracle.scatter_add_compact_mt if mt else c_oracle.scatter_add_compact
        secs = {"hash": 0.0, "gather": 0.0, "scatter_add": 0.0}
        lookups, passes = 0, 0
        while sum(secs.values()) < budget and passes < 64:
            ids, tab, remap, dy, row_begin = prep[passes % len(prep)]
            t0 = time.perf_counter()
            rows = hash_fn(ids, 3, 8, C.EOS_TOKEN_ID, 0, C.LAYER_MULTIPLIERS, mods, offs).reshape(-1)
            t1 = time.perf_counter()
            out, bad = gather_fn(tab, rows if remap is None else remap, row_begin)
            t2 = time.perf_counter()
            if dy is not None:
                scatter_fn(rows, dy, wl["table_rows"], wl["row_begin"])
            t3 = time.perf_counter()
            assert bad == -1
            del out
            secs["hash"] += t1 - t0
            secs["gather"] += t2 - t1
            secs["scatter_add"] += t3 - t2
            lookups += rows.size
            passes += 1
        return lookups, passes, secs

    l1, p1, s1 = run(False, target_seconds)
    log("cpu baseline: single-threaded oracle done")
    lm, pm, sm = run(True, mt_seconds)
    log("cpu baseline: OpenMP oracle done")
    threads = c_oracle.mt_threads()
    what = "hash, gather, compact scatter-add" if prep[0][3] is not None else "hash, gather"
    table_note = ("a host copy of the whole %d-row table" % wl["table_rows"] if full is not None else
                  "a host copy of only the rows each stream reads (host memory cannot hold the whole table)")
    return {"value": lm / sum(sm.values()), "unit": "lookups/s", "cores": threads, "kind": "oracle",
            "host": host_info(),
            "sample": "OpenMP oracle on %d threads: %d passes over the %d rotations in turn (%d lookups in all): "
                      "%s; the gather reads %s" % (threads, pm, len(prep), lm, what, table_note),
            "seconds": {k: round(v, 3) for k, v in sm.items()},
            "single_thread": {"value": l1 / sum(s1.values()), "cores": 1,
                              "sample": "plain single-threaded C oracle: %d passes (%d lookups)" % (p1, l1),
                              "seconds": {k: round(v, 3) for k, v in s1.items()}}}


# ---------------------------------------------------------------- PLE conv + norm

PLE_METRIC = "PLE short-conv + grouped-RMSNorm tokens/sec fwd+bwd and achieved HBM GB/s vs peak"


def ple_build(rotations, dev, batch=8, seq=4096):
    import torch

    import hashed_gram_embedding_engram_amd as E
    import workloads as W
    from hashed_gram_embedding_engram_amd import engram as EB

    lib = EB._ple_lib()
    C = W.HC_COUNT * W.HC_WIDTH
    rots = []
    for r in range(rotations):
        t = W.ple_tensors(dev, 2000 + r, batch, seq, C)
        t["c"] = torch.empty_like(t["x"])        # conv output = norm input
        t["z"] = torch.empty_like(t["x"])        # norm output
        t["dc"] = torch.empty_like(t["x"])       # norm input gradient = conv output gradient
        t["dx"] = torch.empty_like(t["x"])
        t["dhalo"] = torch.empty_like(t["halo"])
        t["dconv_w"] = torch.empty_like(t["conv_w"])
        t["dconv_b"] = torch.empty_like(t["conv_b"])
        t["dnorm_w"] = torch.empty_like(t["norm_w"])
        rots.append(t)
    ws_conv = torch.empty(max(lib.engram_short_conv_workspace(batch, seq, C, 4), 256), dtype=torch.uint8, device=dev)
    ws_norm = torch.empty(max(lib.engram_grouped_rms_norm_workspace(batch * seq, C), 256), dtype=torch.uint8,
                          device=dev)
    return {"rots": rots, "ws_conv": ws_conv, "ws_norm": ws_norm, "batch": batch, "seq": seq, "channels": C,
            "group": W.HC_WIDTH}


def ple_step(wl, t, ev=None):
    """conv forward -> grouped norm forward -> norm backward -> conv backward."""
    import hashed_gram_embedding_engram_amd as E
    rows, C, G = wl["batch"] * wl["seq"], wl["channels"], wl["group"]
    if ev and ev[0] is not None:
        ev[0].record()
    E.engram_short_conv(t["x"], t["conv_w"], t["conv_b"], 3, t["halo"], out=t["c"])
    if ev and ev[1] is not None:
        ev[1].record()
    E.engram_grouped_rms_norm(t["c"].view(rows, C), t["norm_w"], G, 1e-6, out=t["z"].view(rows, C))
    if ev and ev[2] is not None:
        ev[2].record()
    E.engram_grouped_rms_norm_backward(t["c"].view(rows, C), t["dy"].view(rows, C), t["norm_w"], G, 1e-6,
                                       workspace=wl["ws_norm"], out=(t["dc"].view(rows, C), t["dnorm_w"]))
    if ev and ev[3] is not None:
        ev[3].record()
    E.engram_short_conv_backward(t["x"], t["dc"], t["conv_w"], 3, t["halo"], workspace=wl["ws_conv"],
                                 out=(t["dx"], t["dconv_w"], t["dconv_b"], t["dhalo"]))
    if ev and ev[4] is not None:
        ev[4].record()


def timed_phases(step, rots, nphases, steps):
    """Run `steps` timed steps of a multi-phase pipeline.  Each recorded event
    costs the step a few microseconds, so a first pass of up to 20 steps with
    events around every phase finds the dominant phase, and every
    EVENT_STRIDE-th timed step then carries only that phase's two events.
    Returns (seconds, phase ms means, phase percentiles, index of the
    dominant phase); the dominant phase's figures come from the timed steps."""
    import torch

    R = len(rots)
    mk = lambda: torch.cuda.Event(enable_timing=True)
    kb = min(steps, 20)
    bevs = [[mk() for _ in range(nphases + 1)] for _ in range(kb)]
    for i in range(kb):
        step(rots[i % R], bevs[i])
    torch.cuda.synchronize()
    mean = [sum(e[k].elapsed_time(e[k + 1]) for e in bevs) / kb for k in range(nphases)]
    pct = [percentiles([e[k].elapsed_time(e[k + 1]) for e in bevs]) for k in range(nphases)]
    dom = max(range(nphases), key=lambda k: mean[k])
    tevs = [[mk() if j in (dom, dom + 1) else None for j in range(nphases + 1)] if i % EVENT_STRIDE == 0 else None
            for i in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(rots[i % R], tevs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    dom_ms = [e[dom].elapsed_time(e[dom + 1]) for e in tevs if e]
    mean[dom] = sum(dom_ms) / len(dom_ms)
    pct[dom] = percentiles(dom_ms)
    return t1 - t0, mean, pct, dom


def ple_cpu_baseline(wl, sample_rows=2, target_seconds=10.0):
    """The fp64 numpy oracle on successive groups of ``sample_rows`` batch rows
    (rotation 0 first, then the next rotations) until at least
    `target_seconds` of oracle work has been timed."""
    from oracle import ple_ref as P
    G = wl["group"]
    spent, tokens, groups = 0.0, 0, 0
    for t in wl["rots"]:
        cw, cb, nw = (t[k].double().cpu().numpy() for k in ("conv_w", "conv_b", "norm_w"))
        for r0 in range(0, wl["batch"], sample_rows):
            r1 = min(wl["batch"], r0 + sample_rows)
            x = t["x"][r0:r1].double().cpu().numpy()
            dy = t["dy"][r0:r1].double().cpu().numpy()
            halo = t["halo"][r0:r1].double().cpu().numpy()
            t0 = time.perf_counter()
            c = P.short_conv(x, cw, cb, 3, halo)
            P.grouped_rms_norm(c, nw, G)
            dc, _ = P.grouped_rms_norm_backward(c, dy, nw, G)
            P.short_conv_backward(x, dc, cw, 3, halo)
            spent += time.perf_counter() - t0
            tokens += (r1 - r0) * wl["seq"]
            groups += 1
            del x, dy, halo, c, dc
            if spent >= target_seconds:
                break
        if spent >= target_seconds:
            break
    return {"value": tokens / spent, "unit": "tokens/s", "cores": 1, "kind": "oracle", "host": host_info(),
            "sample": "%d groups of %d batch rows (%d tokens x %d channels in all), rotation 0 first: conv, norm, "
                      "their backwards in fp64 numpy, single-threaded" % (groups, sample_rows, tokens,
                                                                          wl["channels"]),
            "seconds": round(spent, 3)}


def ple_main(args, dev):
    import torch

    wl = ple_build(args.rotations, dev)
    torch.cuda.synchronize()
    R = len(wl["rots"])
    for i in range(args.warmup):
        ple_step(wl, wl["rots"][i % R])
    torch.cuda.synchronize()
    names = ["conv_fwd", "norm_fwd", "norm_bwd", "conv_bwd"]
    elapsed, mean, pct, di = timed_phases(lambda t, ev: ple_step(wl, t, ev), wl["rots"], len(names), args.steps)
    tokens = wl["batch"] * wl["seq"]
    C = wl["channels"]
    phase = dict(zip(names, mean))
    phase_pct = dict(zip(names, pct))
    # Algorithmic bytes per launch (bf16 activations, 2 B per element): forward
    # passes read x and write y (4 B per element); backward passes read x and
    # dy and write dx (6 B per element).  Weights, halos and the weight
    # gradients are under 0.1 %; the fp64 partial sums are scratch.
    elems = float(tokens * C)
    alg = {"conv_fwd": 4 * elems, "norm_fwd": 4 * elems, "norm_bwd": 6 * elems, "conv_bwd": 6 * elems}
    kname = {"conv_fwd": ("short_conv_fwd_d3_kernel<bf16,4>", "ple.hip"),
             "norm_fwd": ("rms_norm_fwd_kernel<bf16,5>", "ple.hip"),
             "norm_bwd": ("rms_norm_bwd_kernel<bf16,5> + column_sum_kernel", "ple.hip"),
             "conv_bwd": ("short_conv_bwd_d3_kernel<bf16,4> + column_sum_kernel", "ple.hip")}
    dom = names[di]
    achieved = alg[dom] / (phase[dom] / 1e3) / 1e9
    result = {
        "metric": PLE_METRIC,
        "value": tokens * args.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "PLE causal short conv (kernel 4, dilation 3, 9-token halo) + grouped RMSNorm "
                               "(4 branches x 2,560), fwd+bwd", "batch": wl["batch"], "seq_len": wl["seq"],
                   "channels": C, "rotations": R},
        "phases_ms": {k: round(v, 4) for k, v in phase.items()},
        "phases_ms_p10_p50_p90": phase_pct,
        "phases_from": "%s: HIP events in every %dth timed step; other phases: %d earlier steps with events "
                       "around every phase" % (dom, EVENT_STRIDE, min(args.steps, 20)),
        "roofline": {"kernel": kname[dom][0], "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": counter_traffic(kname[dom][1], "%s_ple_counters.txt" % dom),
                     "algorithmic_bytes_per_launch": alg[dom], "avg_launch_ms": phase[dom]},
        "phase_gbps_algorithmic": {k: round(alg[k] / (phase[k] / 1e3) / 1e9, 1) for k in names},
        "phase_algorithmic_bytes": alg,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = ple_cpu_baseline(wl)
    print(json.dumps(result), flush=True)


# ---------------------------------------------------------------- owner routing

ROUTE_METRIC = "Owner-routing (token x head) lookups/sec, request + owner side of one exchange, and HBM GB/s vs peak"


def route_build(rotations, dev, world=64):
    import torch

    import hashed_gram_embedding_engram_amd as E
    import workloads as W
    from hashed_gram_embedding_engram_amd import engram as EB

    lib = EB._route_lib()
    spec = E.qwen3_8_flash_next_spec()
    rots = []
    for r in range(rotations):
        ids = W.owner_token_batches(seeds=[100 + r])[0]
        gids = E.engram_hash(torch.from_numpy(ids).to(dev), spec).reshape(-1).contiguous()
        n = gids.numel()
        t = {"ids": gids, "n": n,
             "sorted": torch.empty(n, dtype=torch.int64, device=dev),
             "order": torch.empty(n, dtype=torch.int64, device=dev),
             "counts": torch.empty(world, dtype=torch.int64, device=dev),
             "status": torch.empty((), dtype=torch.int64, device=dev),
             "ws": torch.empty(max(int(lib.engram_route_workspace(n)), 256), dtype=torch.uint8, device=dev)}
        E.engram_route_plan(gids, W.FULL_ROWS, world, out=(t["sorted"], t["order"], t["counts"]), workspace=t["ws"])
        cap = int(t["counts"].max().item())
        g = torch.Generator(device=dev)
        g.manual_seed(3000 + r)
        t["cap"] = cap
        t["ids_packed"] = torch.empty((world, cap), dtype=torch.int64, device=dev)
        t["ids_recv"] = torch.empty(n, dtype=torch.int64, device=dev)
        # the owner's looked-up values, in the received (grouped) order
        t["vals"] = torch.randn((n, W.DIM), generator=g, device=dev).to(torch.bfloat16)
        t["vals_packed"] = torch.empty((world, cap, W.DIM), dtype=torch.bfloat16, device=dev)
        t["vals_out"] = torch.empty((n, W.DIM), dtype=torch.bfloat16, device=dev)
        t["grads_grouped"] = torch.empty((n, W.DIM), dtype=torch.bfloat16, device=dev)  # two-call comparison only
        rots.append(t)
    return {"rots": rots, "world": world, "num_embeddings": W.FULL_ROWS}


def route_step(wl, t, ev=None):
    import hashed_gram_embedding_engram_amd as E
    W_, NE = wl["world"], wl["num_embeddings"]
    k = 0

    def mark():
        nonlocal k
        if ev and ev[k] is not None:
            ev[k].record()
        k += 1
    mark()
    E.engram_route_plan(t["ids"], NE, W_, status=t["status"], workspace=t["ws"],
                        out=(t["sorted"], t["order"], t["counts"]))
    mark()
    E.engram_route_validate(t["sorted"], t["counts"], NE, W_)
    mark()
    E.engram_pack_fixed_capacity(t["sorted"], t["counts"], W_, t["cap"], fill=-1, out=t["ids_packed"])
    mark()
    E.engram_unpack_fixed_capacity(t["ids_packed"], t["counts"], t["n"], out=t["ids_recv"])
    mark()
    E.engram_pack_fixed_capacity(t["vals"], t["counts"], W_, t["cap"], fill=0, out=t["vals_packed"])
    mark()
    E.engram_unpack_unpermute_rows(t["vals_packed"], t["counts"], t["order"], out=t["vals_out"])
    mark()


def route_cpu_baseline(wl, target_seconds=10.0):
    """The routing oracle on whole rotations, cycling through them, until at
    least `target_seconds` of oracle work has been timed."""
    import numpy as np

    from oracle import route_ref as RR
    W_, NE = wl["world"], wl["num_embeddings"]
    host = [(t["ids"].cpu().numpy(), t["vals"].float().cpu().numpy(), t["cap"]) for t in wl["rots"]]
    spent, lookups, passes = 0.0, 0, 0
    while spent < target_seconds:
        ids, vals, cap = host[passes % len(host)]
        t0 = time.perf_counter()
        s, order, counts, _ = RR.route_plan(ids, NE, W_)
        RR.validate(s, counts, NE, W_)
        packed_ids, _ = RR.pack(s, counts, W_, cap, -1)
        RR.unpack(packed_ids, counts, ids.size)
        packed, _ = RR.pack(vals, counts, W_, cap, 0.0)
        grouped, _ = RR.unpack(packed, counts, ids.size)
        out = np.empty_like(grouped)
        out[order] = grouped
        spent += time.perf_counter() - t0
        lookups += ids.size
        passes += 1
    return {"value": lookups / spent, "unit": "lookups/s", "cores": 1, "kind": "oracle", "host": host_info(),
            "sample": "%d passes over the %d rotations in turn (%d lookups in all, world %d), plain Python loops "
                      "over segments with numpy arrays, single-threaded" % (passes, len(host), lookups, W_),
            "seconds": round(spent, 3)}


def owner_response(wl, k, compare, distinct):
    """The owner's forward response, timed after the steps and outside their
    clock: its lookup straight from the received padded ID blocks into padded
    value blocks (engram_gather_padded); with `compare`, also the three calls it
    replaces (unpack of the IDs, gather, pack of the values).  Median of k
    launches, HIP events on the stream they run on."""
    import torch

    import hashed_gram_embedding_engram_amd as E
    import workloads as W
    R = len(wl["batches"])

    def median_ms(fn):
        ms = []
        for i in range(k + 2):
            b = wl["batches"][i % R]
            a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn(b, b["recv"])
            e.record()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(e))
        ms = sorted(ms[2:])
        return ms[len(ms) // 2]

    fused = median_ms(lambda b, r: E.engram_gather_padded(wl["table"], r["ids"], r["counts"], wl["row_begin"],
                                                          out=r["vals"], status=b["status"], validate=False))
    n = sum(b["n"] for b in wl["batches"]) / R
    padded = sum(64 * b["recv"]["capacity"] for b in wl["batches"]) / R
    # the padded IDs read, a table row per ID, every padded value row written;
    # compulsory: each distinct table row read once (rotation 0's count)
    alg = 8.0 * padded + 320.0 * n + 320.0 * padded
    comp = 8.0 * padded + 320.0 * distinct + 320.0 * padded
    out = {"kernel": "gather_padded_kernel<20,16,true>", "ms": round(fused, 4),
           "gbps_algorithmic": round(alg / (fused / 1e3) / 1e9, 1), "algorithmic_bytes_per_launch": alg,
           "gbps_compulsory": round(comp / (fused / 1e3) / 1e9, 1), "compulsory_bytes_per_launch": comp,
           "padded_rows": int(padded), "lookups": int(n),
           "traffic": counter_traffic("route.hip", "owner_response_owner_counters.txt"),
           "from": "median of %d launches with HIP events, after the timed steps" % k}
    if compare:
        def three(b, r):
            ids = E.engram_unpack_fixed_capacity(r["ids"], r["counts"], b["n"], out=b["rows_recv"])
            E.engram_gather(wl["table"], ids, wl["row_begin"], out=b["out"], status=b["status"], validate=False)
            E.engram_pack_fixed_capacity(b["out"], r["counts"], 64, r["capacity"], fill=0, out=r["vals"])
        for b in wl["batches"]:
            b.setdefault("rows_recv", torch.empty_like(b["rows"]))
        out["three_calls_ms"] = round(median_ms(three), 4)
    return out


def owner_backward_from_exchange(wl, k, compare):
    """The owner's backward on what the exchange delivers, timed after the steps
    and outside their clock: the plan over the received padded ID blocks and the
    apply reading the received padded gradient blocks directly
    (engram_scatter_add_plan_padded), one after the other on one stream; with
    `compare`, the same after unpacking the IDs and the gradients first.
    Median of k runs, HIP events."""
    import torch

    import hashed_gram_embedding_engram_amd as E
    import workloads as W
    R = len(wl["batches"])

    def median_ms(fn):
        ms = []
        for i in range(k + 2):
            b = wl["batches"][i % R]
            a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn(b, b["recv"])
            e.record()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(e))
        ms = sorted(ms[2:])
        return ms[len(ms) // 2]

    def padded(b, r):
        m = 64 * r["capacity"]
        E.engram_scatter_add_plan_padded(r["ids"], r["counts"], wl["table_rows"], W.DIM, wl["row_begin"],
                                         workspace=wl["workspace_padded"], status=b["plan_status"])
        E.engram_scatter_add_apply(r["dy"].view(m, W.DIM), m, wl["table_rows"], wl["workspace_padded"],
                                   wl["row_begin"], grad_dense=wl["grad_dense"])

    m_max = max(64 * b["recv"]["capacity"] for b in wl["batches"])
    wl.setdefault("workspace_padded", torch.empty(E.engram_scatter_add_workspace(m_max, wl["table_rows"], W.DIM),
                                                  dtype=torch.uint8, device=wl["table"].device))
    out = {"plan_then_apply_ms": round(median_ms(padded), 4),
           "from": "median of %d runs with HIP events, after the timed steps" % k}
    if compare:
        def unpacked(b, r):
            E.engram_unpack_fixed_capacity(r["ids"], r["counts"], b["n"], out=b["rows_recv"])
            E.engram_unpack_fixed_capacity(r["dy"], r["counts"], b["n"], out=b["dy_recv"])
            E.engram_scatter_add_plan(b["rows_recv"], wl["table_rows"], W.DIM, wl["row_begin"],
                                      workspace=wl["workspace"], status=b["plan_status"])
            E.engram_scatter_add_apply(b["dy_recv"], b["n"], wl["table_rows"], wl["workspace"], wl["row_begin"],
                                       grad_dense=wl["grad_dense"])
        for b in wl["batches"]:
            b.setdefault("rows_recv", torch.empty_like(b["rows"]))
            b.setdefault("dy_recv", torch.empty_like(b["dy"]))
        out["unpack_then_plan_then_apply_ms"] = round(median_ms(unpacked), 4)
    return out


def route_backward_send(wl, k, compare):
    """The backward's send, timed after the steps and outside their clock: the
    gradient rows (request order; the returned values stand in for them) taken
    into grouped order and packed to the capacity in one pass
    (engram_permute_pack_rows); with `compare`, also the two calls it replaces.
    Median of k launches, HIP events on the stream they run on."""
    import torch

    import hashed_gram_embedding_engram_amd as E
    import workloads as W
    R, W_ = len(wl["rots"]), wl["world"]

    def median_ms(fn):
        ms = []
        for i in range(k + 2):
            t = wl["rots"][i % R]
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn(t)
            b.record()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        ms = sorted(ms[2:])
        return ms[len(ms) // 2]

    fused = median_ms(lambda t: E.engram_permute_pack_rows(t["vals_out"], t["order"], t["counts"], W_, t["cap"],
                                                           fill=0, out=t["vals_packed"]))
    n = sum(t["n"] for t in wl["rots"]) / R
    cap = sum(t["cap"] for t in wl["rots"]) / R
    row = 2.0 * W.DIM
    alg = row * n + 8.0 * n + row * W_ * cap   # rows and positions read, the padded blocks written
    out = {"kernel": "permute_pack_kernel<u32x4,uint32_t,2>", "ms": round(fused, 4),
           "gbps_algorithmic": round(alg / (fused / 1e3) / 1e9, 1), "algorithmic_bytes_per_launch": alg,
           "traffic": counter_traffic("route.hip", "backward_send_route_counters.txt"),
           "from": "median of %d launches with HIP events, after the timed steps" % k}
    if compare:
        def two(t):
            E.engram_permute_rows(t["vals_out"], t["order"], out=t["grads_grouped"])
            E.engram_pack_fixed_capacity(t["grads_grouped"], t["counts"], W_, t["cap"], fill=0, out=t["vals_packed"])
        out["two_calls_ms"] = round(median_ms(two), 4)
    return out


def route_main(args, dev):
    import torch

    import workloads as W
    wl = route_build(args.rotations, dev)
    torch.cuda.synchronize()
    R = len(wl["rots"])
    for i in range(args.warmup):
        route_step(wl, wl["rots"][i % R])
    torch.cuda.synchronize()
    names = ["plan", "validate", "pack_ids", "unpack_ids", "pack_values", "unpack_unpermute_values"]
    elapsed, mean, pct, di = timed_phases(lambda t, ev: route_step(wl, t, ev), wl["rots"], len(names), args.steps)
    phase = dict(zip(names, mean))
    phase_pct = dict(zip(names, pct))
    n = sum(wl["rots"][i % R]["n"] for i in range(args.steps)) / args.steps
    cap = sum(wl["rots"][i % R]["cap"] for i in range(args.steps)) / args.steps
    Wd, row = wl["world"], 2.0 * W.DIM
    # Algorithmic bytes per launch: the plan reads the 8-B IDs and writes the
    # sorted IDs and their 8-B request positions; validation reads the sorted
    # IDs; a pack reads the compact rows and writes the whole padded
    # [world][capacity] block; the IDs' unpack reads the valid rows and writes
    # them compact; the values' unpack into request order reads every valid
    # row and its 8-B request position and writes the row there.
    alg = {"plan": 24.0 * n, "validate": 8.0 * n, "pack_ids": 8.0 * n + 8.0 * Wd * cap,
           "unpack_ids": 16.0 * n, "pack_values": row * n + row * Wd * cap,
           "unpack_unpermute_values": (2 * row + 8.0) * n}
    dom = names[di]
    kname = {"plan": "route_keys_kernel + radix pass writing the grouped output", "validate": "route_validate_kernel",
             "pack_ids": "pack_kernel<uint32_t,uint32_t,4>", "unpack_ids": "unpack_kernel<uint32_t,uint32_t,4>",
             "pack_values": "pack_kernel<u32x4,uint32_t,2>",
             "unpack_unpermute_values": "unpack_unpermute_kernel<u32x4,uint32_t,2>"}
    achieved = alg[dom] / (phase[dom] / 1e3) / 1e9
    result = {
        "metric": ROUTE_METRIC,
        "value": n * args.steps / elapsed,
        "unit": "lookups/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "owner routing, one request rank of world 64: 8x4096 Zipf(1.2) tokens, "
                               "full-table row IDs, 320-B bf16 value rows; exchange = identity",
                   "lookups_per_step": int(n), "world": Wd, "capacity": int(cap), "rotations": R},
        "phases_ms": {k: round(v, 4) for k, v in phase.items()},
        "phases_ms_p10_p50_p90": phase_pct,
        "phases_from": "%s: HIP events in every %dth timed step; other phases: %d earlier steps with events "
                       "around every phase" % (dom, EVENT_STRIDE, min(args.steps, 20)),
        "roofline": {"kernel": kname[dom], "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": counter_traffic("route.hip", "%s_route_counters.txt" % dom),
                     "algorithmic_bytes_per_launch": alg[dom], "avg_launch_ms": phase[dom]},
        "phase_gbps_algorithmic": {k: round(alg[k] / (phase[k] / 1e3) / 1e9, 1) for k in names},
        "phase_algorithmic_bytes": alg,
        "cpu_baseline": None,
    }
    result["backward_send"] = route_backward_send(wl, min(args.steps, 20), compare=not args.no_alone)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = route_cpu_baseline(wl)
    print(json.dumps(result), flush=True)


def lookup_line(name, args, dev, table=None):
    """Warm-up, timed steps, phase breakdown and phases one at a time of one
    lookup workload; returns (the JSON line's dict without the CPU baseline,
    the workload)."""
    import torch

    import workloads as W

    log("building the %s workload" % name)
    wl = build_workload(name, args.rotations, dev, table=table)
    torch.cuda.synchronize()
    log("workload resident")

    R = len(wl["batches"])
    for i in range(args.warmup):
        run_step(wl, wl["batches"][i % R])
    torch.cuda.synchronize()

    # Each recorded event costs the step a few microseconds (the two around
    # the apply add about 9 us to a 1.29 ms step), so only every
    # EVENT_STRIDE-th timed step carries events, and only the two around the
    # dominant phase (the apply, or the gather of a forward-only workload); a
    # second pass with events around every phase gives the breakdown.
    fused = wl["batches"][0]["tokens"] is not None
    dom = "scatter_apply" if wl["backward"] else "gather"
    dom_span = (5, 6) if wl["backward"] else (0, 2)
    mk = lambda: torch.cuda.Event(enable_timing=True)
    tevs = [[mk() if k in dom_span else None for k in range(7)] if i % EVENT_STRIDE == 0 else None
            for i in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run_step(wl, wl["batches"][i % R], tevs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    log("timed steps done")
    lookups = sum(wl["batches"][i % R]["n"] for i in range(args.steps))
    elapsed = t1 - t0
    dom_ms = [e[dom_span[0]].elapsed_time(e[dom_span[1]]) for e in tevs if e]

    kb = min(args.steps, 20)
    evs = [[mk() for _ in range(7)] for _ in range(kb)]
    for i in range(kb):
        run_step(wl, wl["batches"][i % R], evs[i])
    torch.cuda.synchronize()
    alone = None if args.no_alone else phases_alone(wl, min(args.steps, 20))
    # From tokens the forward is one fused kernel ("gather") and the plan
    # hashes its rows itself; from rows there is no hash.
    spans = {"gather": (0, 2)}
    if wl["backward"] and fused:
        spans.update({"scatter_plan (side stream)": (3, 4), "wait_for_plan": (2, 5), "scatter_apply": (5, 6)})
    elif wl["backward"]:
        spans.update({"scatter_plan": (3, 4), "wait_for_gather": (4, 5), "scatter_apply": (5, 6)})
    phase = {k: sum(e[a].elapsed_time(e[b]) for e in evs) / kb for k, (a, b) in spans.items()}
    phase_pct = {k: percentiles([e[a].elapsed_time(e[b]) for e in evs]) for k, (a, b) in spans.items()}
    phase[dom] = sum(dom_ms) / len(dom_ms)        # the dominant phase from the timed steps themselves
    phase_pct[dom] = percentiles(dom_ms)
    n_avg = lookups / args.steps
    U = None
    b0 = wl["batches"][0]
    if "compact" in b0:
        U = int(b0["compact"][2].item())

    # Algorithmic bytes (what the method must move, per launch):
    #   gather: per lookup one 320 B table row read, one 320 B output row
    #           written and one 8 B row id read -> 648 B; fused with the hash
    #           (from tokens), 640 B per lookup and one 8 B token per position;
    #   apply (segment reduce + carry fix-up): per lookup one 320 B bf16
    #           gradient row read and its 8 B sorted (key, index) pair; per
    #           distinct row one 640 B fp32 sum written (compact) or a 640 B
    #           read + 640 B write (dense).
    positions = int(b0["ids"].size)
    gather_bytes = 640.0 * n_avg + 8.0 * positions if fused else 648.0 * n_avg
    if wl["backward"]:
        u_rows = sum(int(b["compact"][2].item()) for b in wl["batches"]) / R if "compact" in b0 else None
        if u_rows is None:  # dense: distinct rows counted from the plan of rotation 0
            import numpy as np
            u_rows = float(np.unique(b0["rows"].cpu().numpy()).size)
            apply_bytes = 328.0 * n_avg + 1280.0 * u_rows
        else:
            apply_bytes = 328.0 * n_avg + 640.0 * u_rows
    kern = {"gather": (gather_bytes, phase["gather"],
                       "hash_gather_kernel<true,false> (hash and gather fused)" if fused
                       else "gather_rows_kernel<20,16,true>", PROFILED[name]["gather"][0])}
    # The plan and the gather run side by side; apply is timed from after the
    # main stream's wait for both.
    if wl["backward"]:
        kern["scatter_apply"] = (apply_bytes, phase["scatter_apply"],
                                 "segment_reduce_kernel<20,bf16> + carry_fixup_kernel + long_run_kernel", "scatter.hip")
    dbytes, dms, dname, dsrc = kern[dom]
    achieved = dbytes / (dms / 1e3) / 1e9
    traffic = counter_traffic(dsrc, "%s_%s_counters.txt" % (dom, name))

    # Three GB/s figures per kernel: per-lookup bytes (above); compulsory
    # bytes, which count each distinct table row's read once (the gather reads
    # (U/L) * 320 + 328 B per lookup); and the HBM bytes the committed
    # rocprofv3 counters measured for that kernel (null when they were taken
    # on other kernel sources).
    import hashed_gram_embedding_engram_amd as E
    rows0 = E.engram_hash(b0["tokens"], wl["spec"]) if fused else b0["rows"]   # outside the timed steps
    u_fwd = int(torch.unique(rows0.reshape(-1)).numel())
    del rows0
    compulsory = {"gather": 320.0 * u_fwd + (320.0 * n_avg + 8.0 * positions if fused else 328.0 * n_avg)}
    if wl["backward"]:
        compulsory["scatter_apply"] = apply_bytes   # every gradient row is read once already
    gbps = {}
    for k, (byts, ms, _, src) in kern.items():
        hbm = counter_traffic(src, "%s_%s_counters.txt" % (k, name))
        gbps[k] = {"per_lookup": round(byts / (ms / 1e3) / 1e9, 1),
                   "compulsory": round(compulsory[k] / (ms / 1e3) / 1e9, 1),
                   "counters": None if hbm is None else round(hbm / (ms / 1e3) / 1e9, 1)}
    # Step time distribution from the events (first to last event of a step).
    last = 6 if wl["backward"] else 2
    step_ms = sorted(e[0].elapsed_time(e[last]) for e in evs)
    pct = lambda q: step_ms[min(len(step_ms) - 1, int(q * (len(step_ms) - 1) + 0.5))]
    fwd_ms = phase["gather"]
    result = {
        "metric": METRIC,
        "value": lookups / elapsed,
        "unit": "lookups/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": WORKLOAD_NAMES[name],
            "tokens": int(b0["ids"].size), "lookups_per_step": int(n_avg), "table_rows": wl["table_rows"],
            "dim": W.DIM, "table_dtype": "bf16", "grad_dtype": "bf16" if wl["backward"] else None,
            "distinct_rows_rotation0": U, "rotations": R,
        },
        "phases_ms": {k: round(v, 4) for k, v in phase.items()},
        "phases_ms_p10_p50_p90": phase_pct,
        "phases_from": "%s: HIP events in %d of the timed steps (every %dth); other phases and step_ms_events: "
                       "%d more steps with events around every phase" % (dom, len(dom_ms), EVENT_STRIDE, kb),
        "roofline": {"kernel": dname, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": dbytes, "avg_launch_ms": dms},
        "phase_gbps_algorithmic": {k: round(v[0] / (v[1] / 1e3) / 1e9, 1) for k, v in kern.items()},
        "phase_gbps": gbps,
        "distinct_rows_forward_rotation0": u_fwd,
        "step_ms_events": {"p10": round(pct(0.1), 4), "p50": round(pct(0.5), 4), "p90": round(pct(0.9), 4)},
        "forward_lookups_per_s": n_avg / (fwd_ms / 1e3),
        "phases_alone_ms_p50": alone,
        "cpu_baseline": None,
    }
    # The same phases one at a time (measured after the timed steps): the
    # gather without the plan beside it, and the backward as plan then apply.
    if alone:
        ga = alone["gather"]
        result["gather_alone"] = {"gbps_algorithmic": round(gather_bytes / (ga / 1e3) / 1e9, 1),
                                  "gbps_compulsory": round(compulsory["gather"] / (ga / 1e3) / 1e9, 1),
                                  "frac": round(gather_bytes / (ga / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
                                  "frac_compulsory": round(compulsory["gather"] / (ga / 1e3) / 1e9 / HBM_PEAK_GBPS, 4)}
    # HBM bytes of every phase of the step from the committed counter
    # summaries, against the step time (only when all are current).
    counted = ["gather"] + (["scatter_plan", "scatter_apply"] if wl["backward"] else [])
    per = {ph: counter_traffic(PROFILED[name][ph][0], "%s_%s_counters.txt" % (ph, name)) for ph in counted}
    if all(v is not None for v in per.values()):
        total = sum(per.values())
        result["step_traffic"] = {"bytes_per_step": total, "gbps": round(total / (result["ms_per_step"] / 1e3) / 1e9, 1),
                                  "phases_gb": {k: round(v / 1e9, 4) for k, v in per.items()},
                                  "from": "FETCH_SIZE + WRITE_SIZE per launch in the committed rocprofv3 summaries of "
                                          "every phase of the step, over ms_per_step"}
    if name == "owner":
        result["owner_response"] = owner_response(wl, min(args.steps, 20), compare=not args.no_alone,
                                                  distinct=u_fwd)
        if not args.no_alone:   # its plan and apply kernels would mix with the step's in a profile
            result["owner_backward_from_exchange"] = owner_backward_from_exchange(wl, min(args.steps, 20),
                                                                                  compare=True)
    if wl["backward"]:
        # What the step pays for the backward: the plan runs beside the
        # forward, so only what follows the forward's end counts (the wait for
        # the plan, if it ends later, and the apply).
        after_forward = sum(e[2].elapsed_time(e[5]) for e in evs) / kb
        bw = after_forward + phase["scatter_apply"]
        result["backward_in_step"] = {"ms": round(bw, 4), "gbps_algorithmic": round(apply_bytes / (bw / 1e3) / 1e9, 1),
                                      "frac": round(apply_bytes / (bw / 1e3) / 1e9 / HBM_PEAK_GBPS, 4)}
    if alone and wl["backward"]:
        bs = alone["scatter_plan"] + alone["scatter_apply"]
        result["backward_plan_then_apply"] = {"ms": round(bs, 4),
                                              "gbps_algorithmic": round(apply_bytes / (bs / 1e3) / 1e9, 1),
                                              "frac": round(apply_bytes / (bs / 1e3) / 1e9 / HBM_PEAK_GBPS, 4)}
    return result, wl


WORKLOAD_NAMES = {"long": "long-context packed THD stream, full table, fwd+bwd (compact grad)",
                  "full-sft": "SFT batch 8x4096, full table, fwd",
                  "owner": "owner shard 1/64 of a world-64 step, fwd+bwd (dense grad)",
                  "sft": "SFT batch 8x4096, 10M-row table, fwd"}
LOOKUP_WORKLOADS = tuple(WORKLOAD_NAMES)

# The ceiling a kernel's traffic is compared with: the probe with the same
# mix and access distribution.  The backward's sums read a random permutation
# of the gradient rows, as row_expand does; the gather's Zipf-skewed rows hit
# in cache more often than row_gather's uniform ones, so it has no such probe.
CEILING_OF = {"scatter_apply": "row_expand", "scatter_apply_dense": "row_rmw"}

# Fields of the other configurations' lines kept in the default line.
EXTRA_KEYS = ("value", "unit", "ms_per_step", "config", "phases_ms", "roofline", "phase_gbps", "gather_alone",
              "backward_in_step", "backward_plan_then_apply", "phases_alone_ms_p50", "distinct_rows_forward_rotation0", "step_traffic",
              "owner_response", "owner_backward_from_exchange")


def add_ceiling_fracs(result, ceilings):
    """The dominant kernel's achieved rate against the probe with its traffic mix."""
    if not ceilings:
        return
    dom = "scatter_apply" if "scatter_apply" in result["phase_gbps"] else "gather"
    if dom == "scatter_apply" and result["config"].get("distinct_rows_rotation0") is None:
        dom = "scatter_apply_dense"   # the dense gradient's read-modify-write
    c = ceilings.get(CEILING_OF.get(dom))
    if c:
        result["roofline"]["measured_ceiling"] = {"probe": CEILING_OF[dom], "gbps": c,
                                                  "frac": round(result["roofline"]["achieved"] / c, 4)}


# ---------------------------------------------------------------- profile summaries

# Kernels of each phase, as rocprofv3 names them (regular expressions over the
# name without its argument list), and the source each phase's kernels are
# built from.  A kernel that matches several phases of a workload (the column
# sum shared by both PLE backwards) is charged to the phase of the dispatch
# before it.
LOOKUP_PHASES = {
    "hash": ("hash.hip", [r"\bhash_kernel"]),
    "gather": ("gather.hip", [r"\bgather_rows_kernel"]),
    # a plan starts with its init kernel, or, split by head into short
    # segments, with the keys kernel that does the init's work itself
    "scatter_plan": ("scatter.hip", [r"\bscatter_init_kernel|\bhead_keys_kernel<\d+, true\b", r"\bkeys_kernel",
                                     r"\bhead_keys_kernel", r"\bupsweep_kernel",
                                     r"\bdownsweep_kernel", r"\brun_count_kernel", r"\bblock_scan_kernel",
                                     r"\buniq_rows_kernel"]),
    "scatter_apply": ("scatter.hip", [r"\bsegment_reduce_kernel", r"\bcarry_fixup_kernel", r"\blong_run_kernel"]),
}
# Workloads that start from tokens run the fused hash-and-gather forward.
FUSED_PHASES = dict(LOOKUP_PHASES, gather=("lookup.hip", [r"\bhash_gather_kernel"]))
PROFILED = {
    "long": FUSED_PHASES, "full-sft": FUSED_PHASES, "sft": FUSED_PHASES,
    "owner": dict(LOOKUP_PHASES, owner_response=("route.hip", [r"\bgather_padded_kernel"])),
    "ple": {"conv_fwd": ("ple.hip", [r"\bshort_conv_fwd"]), "norm_fwd": ("ple.hip", [r"\brms_norm_fwd"]),
            "norm_bwd": ("ple.hip", [r"\brms_norm_bwd", r"\bcolumn_sum_kernel"]),
            "conv_bwd": ("ple.hip", [r"\bshort_conv_bwd", r"\bcolumn_sum_kernel"])},
    "route": {"plan": ("route.hip", [r"\broute_init_kernel", r"\broute_keys_kernel", r"\bupsweep_kernel",
                                     r"\bdownsweep_kernel"]),
              "validate": ("route.hip", [r"\broute_validate_kernel"]),
              "pack_ids": ("route.hip", [r"\bpack_kernel<unsigned int,"]),
              "unpack_ids": ("route.hip", [r"\bunpack_kernel<unsigned int,"]),
              "pack_values": ("route.hip", [r"\bpack_kernel<u32x4"]),
              "unpack_unpermute_values": ("route.hip", [r"\bunpack_unpermute_kernel<u32x4"]),
              "backward_send": ("route.hip", [r"\bpermute_pack_kernel<u32x4"])},
}
# Phases whose counter summaries are written (the ones a bench line can name
# as its dominant kernel).
COUNTED = {"long": ["gather", "scatter_plan", "scatter_apply"], "full-sft": ["gather"],
           "owner": ["gather", "scatter_plan", "scatter_apply", "owner_response"],
           "ple": ["conv_fwd", "norm_fwd", "norm_bwd", "conv_bwd"],
           "route": ["pack_values", "unpack_unpermute_values", "backward_send"]}
PROFILE_FLAGS = "--steps 5 --warmup 2 --no-cpu-baseline --no-alone --no-ceilings --no-extra-configs --calibrate-copy"
TRACE_FILE = {"long": "kernel_trace_long_context.md", "full-sft": "kernel_trace_full_sft.md",
              "owner": "kernel_trace_owner.md", "ple": "kernel_trace_ple.md", "route": "kernel_trace_route.md"}
WORKLOAD_TEXT = {
    "ple": "activations [8, 4,096, 10,240] bf16 (four 2,560-wide branches); per step the causal depthwise conv "
           "(kernel 4, dilation 3, 9-token halo), the grouped RMSNorm (groups of 2,560), the norm backward and "
           "the conv backward, each backward followed by a column sum of its weight-gradient partials",
    "route": "one request rank of a world-64 owner group: 8 x 4,096 Zipf(1.2) tokens hashed into 524,288 "
             "full-table row IDs; per step: group by owner (route keys, then one radix digit pass that writes the grouped IDs, positions and counts), "
             "segment validation, pack of the IDs to the step's capacity, the owner's unpack, the owner's pack "
             "of 320-B bf16 value rows, and the requester's unpack straight into request order (one pass); after the "
             "steps, the backward's send (gradient rows into grouped order and packed, one pass) timed on its own",
}


def plan_passes(num_rows, from_tokens=False, moduli=None, offsets=None, row_begin=0):
    """Digit passes of the backward plan's sort: 8-bit digits over the bits of
    num_rows (the out-of-range sentinel num_rows sorts last); from tokens, when
    every head's range [offset, offset + modulus) lies in the shard and the
    ranges are disjoint and ascending in head order, the sort runs per head over
    the bits of the largest modulus (the last pass taking 9 bits where that
    saves a pass), if that needs fewer passes."""
    bits = 0
    while bits < 32 and (num_rows >> bits) != 0:
        bits += 1
    passes = (bits + 7) // 8
    if not from_tokens or moduli is None:
        return passes
    prev_end = 0
    for off, mod in zip(offsets, moduli):
        lo = off - row_begin
        if lo < 0 or lo > num_rows or mod > num_rows - lo or lo < prev_end:
            return passes
        prev_end = lo + mod
    head_bits = (max(moduli) - 1).bit_length()
    split = 1 if head_bits <= 8 else max(2, (head_bits - 1 + 7) // 8)
    return min(passes, split)


def sort_nominal_bytes(n, num_rows, uniq=None, from_tokens=False, passes=None):
    """HBM bytes the backward plan's own traffic model gives for n lookups:
    keys (8 B row read, or 8 B per token when the plan hashes the rows itself,
    and 4 B key written), the first pass (4 B read, 8 B written), each later
    pass (16 B) with its histogram (4 B), the run count's read (4 B) and, in
    the compact form, the distinct rows' pass (4 B read, 8 B per distinct row
    written).  `passes` defaults to the whole sort's (plan_passes)."""
    if passes is None:
        passes = plan_passes(num_rows)
    total = (n // 2 if from_tokens else 8 * n) + 16 * n + (passes - 1) * 20 * n + 4 * n
    if uniq is not None:
        total += 4 * n + 8 * uniq
    return float(total)


def profile_commands(name):
    """The three rocprofv3 runs behind a workload's summaries (REPO = repository root)."""
    pre = "cd /tmp && export TMPDIR=/tmp && "
    run = "-- python3 $REPO/bench.py --workload %s %s" % (name, PROFILE_FLAGS)
    pats = []
    for _, ks in PROFILED[name].values():
        for alt in ks:
            for k in alt.split("|"):
                k = k.replace(r"\b", "").split("<")[0]
                if k not in pats:
                    pats.append(k)
    regex = "|".join(pats) + "|copyBuffer"
    out = "$REPO/gpurun_out/prof/%s" % name
    return {
        "trace": pre + "timeout -k 10 300 rocprofv3 --kernel-trace --stats -f csv -d %s_kt -o kt %s > %s_line.json"
                       % (out, run, out),
        "fetch": pre + 'timeout -s KILL 300 rocprofv3 --pmc FETCH_SIZE -f csv --kernel-include-regex "%s" -d %s_fetch '
                       "-o f %s" % (regex, out, run),
        "write": pre + 'timeout -s KILL 300 rocprofv3 --pmc WRITE_SIZE -f csv --kernel-include-regex "%s" -d %s_write '
                       "-o w %s" % (regex, out, run),
    }


def _short_kernel(name):
    """A kernel's name without its argument list and anonymous namespaces,
    with the 16-byte vector type spelled u32x4."""
    name = name.replace("(anonymous namespace)::", "").replace("unsigned int __vector(4)", "u32x4")
    if name.startswith("void "):
        name = name[5:]
    depth = 0
    for i, c in enumerate(name):   # the argument list opens outside every template bracket
        depth += (c == "<") - (c == ">")
        if c == "(" and depth == 0:
            return name[:i]
    return name


def _phases_of(kernel, phases):
    return [p for p, (_, ks) in phases.items() if any(re.search(x, kernel) for x in ks)]


def _charge(dispatches, phases):
    """[(kernel, value)] in dispatch order -> {phase: [value per launch]}: a
    dispatch of a phase's first kernel starts a launch of that phase; a kernel
    matching several phases goes to the phase of the dispatch before it."""
    per, prev = {}, None
    for kernel, value in dispatches:
        ps = _phases_of(kernel, phases)
        p = ps[0] if len(ps) == 1 else (prev if prev in ps else None)
        prev = p
        if p is None:
            continue
        if re.search(phases[p][1][0], kernel) or p not in per:
            per.setdefault(p, []).append(0.0)
        per[p][-1] += value
    return per


def summarize_profiles(name, raw):
    """Write profiles/<trace file> and <phase>_<workload>_counters.txt from the
    rocprofv3 output of profile_commands(name) under `raw`."""
    import csv
    phases = PROFILED[name]
    cmds = profile_commands(name)
    line = json.loads(open(os.path.join(raw, "%s_line.json" % name)).read().strip().splitlines()[-1])
    stats = list(csv.DictReader(open(os.path.join(raw, "%s_kt" % name, "kt_kernel_stats.csv"))))
    avg_us = {_short_kernel(r["Name"]): float(r["AverageNs"]) / 1e3 for r in stats}
    calls = {_short_kernel(r["Name"]): int(r["Calls"]) for r in stats}
    trace = sorted(csv.DictReader(open(os.path.join(raw, "%s_kt" % name, "kt_kernel_trace.csv"))),
                   key=lambda r: int(r["Dispatch_Id"]))
    t_us = _charge([(_short_kernel(r["Kernel_Name"]),
                     (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3) for r in trace], phases)

    def counters(kind, cname):
        rows = [r for r in csv.DictReader(open(os.path.join(raw, "%s_%s" % (name, kind),
                                                            "%s_counter_collection.csv" % kind[0])))
                if r["Counter_Name"] == cname]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        disp = [(_short_kernel(r["Kernel_Name"]), float(r["Counter_Value"])) for r in rows]
        per_kernel = {}
        for k, v in disp:
            per_kernel.setdefault(k, []).append(v)
        # the 1 GiB calibration copy is the largest device copy of the run
        calib = max(v for k, v in disp if "copyBuffer" in k)
        return _charge(disp, phases), per_kernel, calib
    fetch, fetch_k, f_copy = counters("fetch", "FETCH_SIZE")
    write, write_k, w_copy = counters("write", "WRITE_SIZE")
    f_scale, w_scale = 1048576.0 / f_copy, 1048576.0 / w_copy
    mean = lambda v: sum(v) / len(v)

    # trace summary
    if name in WORKLOAD_TEXT:
        desc = "%s; 2 warm-up steps, 5 steps with events around every phase, then 5 timed steps, over 4 " \
               "rotating input sets." % WORKLOAD_TEXT[name]
    else:
        desc = "%s; %d (token x head) lookups per step; 2 warm-up steps, 5 timed steps, then 5 steps with events " \
               "around every phase; 4 rotating input sets.  In the step the plan (sort) and the gather run on two " \
               "streams side by side, so the two share HBM." % (WORKLOAD_NAMES[name],
                                                                line["config"]["lookups_per_step"])
        if "owner_response" in line:
            desc += "  After the steps, the owner's lookup from the received padded ID blocks into padded value " \
                    "blocks (owner_response) is launched on its own."
    title = WORKLOAD_NAMES.get(name) or line["config"]["workload"]
    lines = ["# Kernel trace: %s, one MI355X" % title, "",
             "Command (REPO = repository root on the MI355X machine):", "", "    " + cmds["trace"], "",
             "Workload: " + desc, "",
             "Step from the same run: %.4f ms (%.4g %s); phases (ms): %s." % (
                 line["ms_per_step"], line["value"], line["unit"],
                 ", ".join("%s %.4f" % kv for kv in line["phases_ms"].items())), "",
             "| kernel | calls | avg us | phase |", "|---|---:|---:|---|"]
    for k in sorted(avg_us, key=lambda k: -avg_us[k] * calls[k]):
        lines.append("| `%s` | %d | %.1f | %s |" % (k, calls[k], avg_us[k], ", ".join(_phases_of(k, phases)) or "setup"))
    lines += ["", "Phase time per launch (sum of its kernels' durations, averaged over its launches): " +
              ", ".join("%s %.1f us" % (p, mean(t_us[p])) for p in phases if p in t_us) + ".",
              "Kernels of no phase (input generation, the 1 GiB calibration copy%s) are setup."
              % (", the distinct-row count" if name in LOOKUP_WORKLOADS else "")]
    with open(os.path.join(PROFILES, TRACE_FILE[name]), "w") as f:
        f.write("\n".join(lines) + "\n")

    # counter summaries of the phases whose algorithmic bytes the line states
    alg = dict(line.get("phase_algorithmic_bytes") or {})
    if "backward_send" in line:   # the routing line's extra measurement
        alg["backward_send"] = line["backward_send"]["algorithmic_bytes_per_launch"]
    comp = dict(alg)
    if name in LOOKUP_WORKLOADS:
        cfg = line["config"]
        n = cfg["lookups_per_step"]
        fused = phases["gather"][0] == "lookup.hip"   # the forward hashes inside the gather
        per_lookup = 640.0 * n + 8.0 * cfg["tokens"] if fused else 648.0 * n
        alg = {"gather": per_lookup, "hash": 8.0 * cfg["tokens"] + 8.0 * n}
        # compulsory bytes read each distinct table row once (rotation 0's count)
        comp = {"gather": 320.0 * line["distinct_rows_forward_rotation0"] + per_lookup - 320.0 * n,
                "hash": alg["hash"]}
        if "owner_response" in line:   # the owner line's extra measurement
            alg["owner_response"] = line["owner_response"]["algorithmic_bytes_per_launch"]
            comp["owner_response"] = line["owner_response"].get("compulsory_bytes_per_launch", alg["owner_response"])
        if "scatter_apply" in line["phase_gbps"]:
            alg["scatter_apply"] = comp["scatter_apply"] = line["roofline"]["algorithmic_bytes_per_launch"]
            # the full table's workloads hash with the released head layout
            import hashed_gram_embedding_engram_amd as E
            released = cfg["table_rows"] == E.QWEN3_8_FLASH_NEXT_NGRAM_PADDED_ROWS
            passes = plan_passes(cfg["table_rows"], fused, E.QWEN3_8_FLASH_NEXT_NGRAM_HEAD_VOCAB_SIZES,
                                 E.QWEN3_8_FLASH_NEXT_NGRAM_HEAD_OFFSETS) if released else None
            alg["scatter_plan"] = comp["scatter_plan"] = sort_nominal_bytes(n, cfg["table_rows"],
                                                                            cfg["distinct_rows_rotation0"], fused,
                                                                            passes)
    for phase in COUNTED[name]:
        if phase not in alg or phase not in fetch:
            continue
        ks = [k for k in fetch_k if phase in _phases_of(k, phases)]
        fb = mean(fetch[phase]) * 1024 * f_scale
        wb = mean(write[phase]) * 1024 * w_scale
        tp = mean(t_us[phase])
        out = ["# HBM traffic of one launch of the %s phase, %s, MI355X, rocprofv3 counters." % (phase, title),
               "# Commands (REPO = repository root on the MI355X machine):", "#   " + cmds["fetch"],
               "#   " + cmds["write"], "#   " + cmds["trace"],
               "# Counters are KiB per dispatch; a launch sums its dispatches, averaged over the %d launches of the "
               "run." % len(fetch[phase]),
               "# Scale: the 1 GiB device copy that --calibrate-copy runs first reads FETCH_SIZE %.0f KiB and "
               "WRITE_SIZE %.0f KiB" % (f_copy, w_copy),
               "#   for 1,048,576 KiB each way, so FETCH_SIZE is scaled x%.3f and WRITE_SIZE x%.3f." % (f_scale, w_scale),
               "# Kernels of the phase (KiB per dispatch, unscaled; a kernel shared with another phase shows its "
               "mean over both):"]
        for k in ks:
            out.append("#   %-55s FETCH %11.1f KiB  WRITE %11.1f KiB  avg %8.1f us" % (
                k, mean(fetch_k[k]), mean(write_k.get(k, [0.0])), avg_us.get(k, 0.0)))
        out += ["# Algorithmic bytes per launch: %.0f; compulsory bytes (each distinct table row moved once): %.0f"
                % (alg[phase], comp[phase]),
                "# Average time per launch (kernel-trace run): %.1f us" % tp,
                "# source_sha256_16: SHA-256 prefix of the kernel source and the local headers it includes",
                "source_sha256_16 %s" % source_sha(phases[phase][0]),
                "fetch_bytes_per_launch %.0f" % fb, "write_bytes_per_launch %.0f" % wb,
                "hbm_bytes_per_launch %.0f" % (fb + wb), "algorithmic_bytes_per_launch %.0f" % alg[phase],
                "compulsory_bytes_per_launch %.0f" % comp[phase],
                "kernel_time_us_per_launch %.1f" % tp]
        with open(os.path.join(PROFILES, "%s_%s_counters.txt" % (phase, name)), "w") as f:
            f.write("\n".join(out) + "\n")


def main():
    if len(sys.argv) >= 2 and sys.argv[1] == "--profile-commands":
        for c in profile_commands(sys.argv[2]).values():
            print(c)
        return
    if len(sys.argv) >= 2 and sys.argv[1] == "--summarize-profiles":
        summarize_profiles(sys.argv[2], sys.argv[3] if len(sys.argv) > 3 else os.path.join(ROOT, "gpurun_out", "prof"))
        return
    args = parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the Engram path here is built and timed on a single MI355X; "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch

    import hashed_gram_embedding_engram_amd as E

    E.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        src = torch.empty(1 << 29, dtype=torch.int16, device=dev).fill_(1)   # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.workload == "ple":
        ple_main(args, dev)
        return
    if args.workload == "route":
        route_main(args, dev)
        return
    ceilings = None
    if not args.no_ceilings:
        from hashed_gram_embedding_engram_amd import probe
        log("HBM ceilings")
        ceilings = probe.measure_ceilings(dev)
    result, wl = lookup_line(args.workload, args, dev)
    if ceilings:
        result["ceilings_gbps"] = ceilings
        result["ceilings_from"] = ("libengram_probe.so: streaming 16-byte reads and writes of 4 GiB; row_gather "
                                   "reads 4,194,304 uniform-random 320-B rows of a 25 M-row bf16 table and writes "
                                   "them in order; row_expand reads 3,163,052 distinct random 320-B bf16 rows and "
                                   "writes them as 640-B fp32 rows; row_rmw adds 4 random 320-B bf16 rows into each "
                                   "of 156,202 distinct random 640-B fp32 rows of a 5,000,024-row array (read, add, "
                                   "write back); the row probes launch one 16-row tile per wave; GB/s = bytes moved / median of 10 "
                                   "launches")
        add_ceiling_fracs(result, ceilings)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl)
    if args.workload == "long" and not args.no_extra_configs:
        # The other full-table and owner-shard configurations, measured after
        # the headline in the same run: the SFT batch's forward against the
        # same 102.4 GB table, then the owner shard's forward and dense backward.
        table = wl["table"]
        del wl
        extra = {}
        line, wl = lookup_line("full-sft", args, dev, table=table)
        add_ceiling_fracs(line, ceilings)
        extra["full_table_sft_forward"] = {k: line[k] for k in EXTRA_KEYS if k in line}
        del wl, table
        torch.cuda.empty_cache()
        line, wl = lookup_line("owner", args, dev)
        add_ceiling_fracs(line, ceilings)
        extra["owner_shard_step"] = {k: line[k] for k in EXTRA_KEYS if k in line}
        del wl
        result["other_configs"] = extra
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
