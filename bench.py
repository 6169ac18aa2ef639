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


def build_workload(name, rotations, dev):
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
        n = rows.numel()
        g = torch.Generator(device=dev)
        g.manual_seed(1000 + r)
        b = {"ids": ids, "tokens": tokens, "rows": rows, "n": n,
             "out": torch.empty((n, W.DIM), dtype=torch.bfloat16, device=dev),
             "status": torch.empty((), dtype=torch.int64, device=dev),
             "plan_status": torch.empty((), dtype=torch.int64, device=dev)}
        if name in ("long", "owner"):
            b["dy"] = torch.randn((n, W.DIM), generator=g, device=dev).to(torch.bfloat16)
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
    """hash -> gather, with the backward plan (sort by row) on a side stream
    concurrently with the gather, then apply once both are done.  ev: events
    (hash start, hash end, gather end, plan start, plan end, apply start, apply
    end); an entry may be None, and only the events given are recorded."""
    import torch

    import hashed_gram_embedding_engram_amd as E
    main = torch.cuda.current_stream()
    side = wl["side"]

    def mark(k, stream):
        if ev and ev[k] is not None:
            ev[k].record(stream)

    mark(0, main)
    if b["tokens"] is not None:
        E.engram_hash(b["tokens"], wl["spec"], rows_out=b["rows"])
    mark(1, main)
    if wl["backward"]:
        side.wait_stream(main)
        compact = b.get("compact")
        mark(3, side)
        E.engram_scatter_add_plan(b["rows"], wl["table_rows"], b["dy"].shape[-1], wl["row_begin"],
                                  workspace=wl["workspace"], uniq_rows=compact[0] if compact else None,
                                  num_uniq=compact[2] if compact else None, status=b["plan_status"], stream=side)
        mark(4, side)
    E.engram_gather(wl["table"], b["rows"], wl["row_begin"], out=b["out"], status=b["status"], validate=False)
    mark(2, main)
    if wl["backward"]:
        main.wait_stream(side)
        mark(5, main)
        E.engram_scatter_add_apply(b["dy"], b["n"], wl["table_rows"], wl["workspace"], wl["row_begin"],
                                   grad_dense=wl["grad_dense"], uniq_grad=compact[1] if compact else None)
        mark(6, main)


def phases_alone(wl, k):
    """Median ms of the gather, the plan and the apply, each run by itself on
    the main stream with nothing beside it, over k launches rotating through
    the input sets (outside the timed steps)."""
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
        E.engram_gather(wl["table"], b["rows"], wl["row_begin"], out=b["out"], status=b["status"], validate=False)
        e[1].record()
        if wl["backward"]:
            compact = b.get("compact")
            e[2].record()
            E.engram_scatter_add_plan(b["rows"], wl["table_rows"], b["dy"].shape[-1], wl["row_begin"],
                                      workspace=wl["workspace"], uniq_rows=compact[0] if compact else None,
                                      num_uniq=compact[2] if compact else None, status=b["plan_status"])
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
    """The CPUs this process may run on and their model name (the baseline uses one)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpus_available": len(os.sched_getaffinity(0)), "cpu_model": model}


def cpu_baseline(wl, max_tokens=None, target_seconds=10.0):
    """The oracle (plain single-threaded C) on the same streams as the timed
    steps: rotation after rotation until at least `target_seconds` of oracle
    work (or every rotation) has been timed."""
    import numpy as np
    import torch

    import workloads as W
    from oracle import c_oracle, constants as C

    if wl["name"] == "sft":
        ws = W.sft_spec()
        mods, offs = ws["vocab_sizes"], ws["offsets"]
    else:
        mods, offs = C.head_vocab_sizes(), C.head_offsets()
    secs = {"hash": 0.0, "gather": 0.0, "scatter_add": 0.0}
    lookups, tokens, rotations, distinct = 0, 0, 0, []
    for b in wl["batches"]:
        if b["tokens"] is None:
            return None
        ids = b["ids"]
        if max_tokens is not None and ids.shape[1] > max_tokens:
            ids = ids[:, :max_tokens]
        # Sample preparation (untimed): the oracle gathers from a host copy of exactly
        # the table rows this stream reads, renumbered; the 102.4 GB table stays on the GPU.
        rows_prep = c_oracle.hash_input_ids(ids, 3, 8, C.EOS_TOKEN_ID, 0, C.LAYER_MULTIPLIERS, mods,
                                            offs).reshape(-1)
        uniq, inv = np.unique(rows_prep, return_inverse=True)
        sub = wl["table"][torch.from_numpy(uniq).to(wl["table"].device)].cpu().view(torch.int16).numpy() \
            .view(np.uint16)
        inv = inv.astype(np.int64)
        n = rows_prep.size
        dy = b["dy"][:n].cpu().view(torch.int16).numpy().view(np.uint16) if "dy" in b else None
        t0 = time.perf_counter()
        rows = c_oracle.hash_input_ids(ids, 3, 8, C.EOS_TOKEN_ID, 0, C.LAYER_MULTIPLIERS, mods, offs).reshape(-1)
        t1 = time.perf_counter()
        out, _ = c_oracle.gather(sub, inv)
        t2 = time.perf_counter()
        if dy is not None:
            c_oracle.scatter_add_compact(rows, dy, wl["table_rows"], wl["row_begin"])
        t3 = time.perf_counter()
        del out, sub
        secs["hash"] += t1 - t0
        secs["gather"] += t2 - t1
        secs["scatter_add"] += t3 - t2
        lookups += n
        tokens += ids.size
        rotations += 1
        distinct.append(int(uniq.size))
        if sum(secs.values()) >= target_seconds:
            break
    total = sum(secs.values())
    return {"value": lookups / total, "unit": "lookups/s", "cores": 1, "kind": "oracle", "host": host_info(),
            "sample": "%d rotation(s), %d tokens (%d lookups) in all: hash, gather from a host copy of each "
                      "rotation's distinct rows (%s), compact scatter-add; single-threaded C"
                      % (rotations, tokens, lookups, ", ".join(str(u) for u in distinct)),
            "seconds": {k: round(v, 3) for k, v in secs.items()}}


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
        t["vals_grouped"] = torch.empty((n, W.DIM), dtype=torch.bfloat16, device=dev)
        t["vals_out"] = torch.empty((n, W.DIM), dtype=torch.bfloat16, device=dev)
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
    E.engram_unpack_fixed_capacity(t["vals_packed"], t["counts"], t["n"], out=t["vals_grouped"])
    mark()
    E.engram_unpermute_rows(t["vals_grouped"], t["order"], out=t["vals_out"])
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
        grouped = RR.unpack(packed, counts, ids.size)
        out = np.empty_like(grouped)
        out[order] = grouped
        spent += time.perf_counter() - t0
        lookups += ids.size
        passes += 1
    return {"value": lookups / spent, "unit": "lookups/s", "cores": 1, "kind": "oracle", "host": host_info(),
            "sample": "%d passes over the %d rotations in turn (%d lookups in all, world %d), plain Python loops "
                      "over segments with numpy arrays, single-threaded" % (passes, len(host), lookups, W_),
            "seconds": round(spent, 3)}


def route_main(args, dev):
    import torch

    import workloads as W
    wl = route_build(args.rotations, dev)
    torch.cuda.synchronize()
    R = len(wl["rots"])
    for i in range(args.warmup):
        route_step(wl, wl["rots"][i % R])
    torch.cuda.synchronize()
    names = ["plan", "validate", "pack_ids", "unpack_ids", "pack_values", "unpack_values", "unpermute_values"]
    elapsed, mean, pct, di = timed_phases(lambda t, ev: route_step(wl, t, ev), wl["rots"], len(names), args.steps)
    phase = dict(zip(names, mean))
    phase_pct = dict(zip(names, pct))
    n = sum(wl["rots"][i % R]["n"] for i in range(args.steps)) / args.steps
    cap = sum(wl["rots"][i % R]["cap"] for i in range(args.steps)) / args.steps
    Wd, row = wl["world"], 2.0 * W.DIM
    # Algorithmic bytes per launch: the plan reads the 8-B IDs and writes the
    # sorted IDs and their 8-B request positions; validation reads the sorted
    # IDs; a pack reads the compact rows and writes the whole padded
    # [world][capacity] block; an unpack reads the valid rows and writes them
    # compact; the unpermute reads and writes every row plus its 8-B position.
    alg = {"plan": 24.0 * n, "validate": 8.0 * n, "pack_ids": 8.0 * n + 8.0 * Wd * cap,
           "unpack_ids": 16.0 * n, "pack_values": row * n + row * Wd * cap, "unpack_values": 2 * row * n,
           "unpermute_values": (2 * row + 8.0) * n}
    dom = names[di]
    kname = {"plan": "route_keys_kernel + radix pass + route_output_kernel", "validate": "route_validate_kernel",
             "pack_ids": "pack_kernel<uint32_t,uint32_t,4>", "unpack_ids": "unpack_kernel<uint32_t,uint32_t,4>",
             "pack_values": "pack_kernel<u32x4,uint32_t,2>", "unpack_values": "unpack_kernel<u32x4,uint32_t,4>",
             "unpermute_values": "permute_kernel<u32x4,false,1>"}
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
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = route_cpu_baseline(wl)
    print(json.dumps(result), flush=True)


def main():
    args = parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the Engram path here is built and timed on a single MI355X; "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch

    import hashed_gram_embedding_engram_amd as E
    import workloads as W

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
    wl = build_workload(args.workload, args.rotations, dev)
    torch.cuda.synchronize()

    R = len(wl["batches"])
    for i in range(args.warmup):
        run_step(wl, wl["batches"][i % R])
    torch.cuda.synchronize()

    # Each recorded event costs the step a few microseconds (the two around
    # the apply add about 9 us to a 1.29 ms step), so only every
    # EVENT_STRIDE-th timed step carries events, and only the two around the
    # dominant phase (the apply, or the gather of a forward-only workload); a
    # second pass with events around every phase gives the breakdown.
    dom = "scatter_apply" if wl["backward"] else "gather"
    dom_span = (5, 6) if wl["backward"] else (1, 2)
    mk = lambda: torch.cuda.Event(enable_timing=True)
    tevs = [[mk() if k in dom_span else None for k in range(7)] if i % EVENT_STRIDE == 0 else None
            for i in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run_step(wl, wl["batches"][i % R], tevs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    lookups = sum(wl["batches"][i % R]["n"] for i in range(args.steps))
    elapsed = t1 - t0
    dom_ms = [e[dom_span[0]].elapsed_time(e[dom_span[1]]) for e in tevs if e]

    kb = min(args.steps, 20)
    evs = [[mk() for _ in range(7)] for _ in range(kb)]
    for i in range(kb):
        run_step(wl, wl["batches"][i % R], evs[i])
    torch.cuda.synchronize()
    alone = None if args.no_alone else phases_alone(wl, min(args.steps, 20))
    spans = {"hash": (0, 1), "gather": (1, 2)}
    if wl["backward"]:
        spans.update({"scatter_plan (side stream)": (3, 4), "wait_for_plan": (2, 5), "scatter_apply": (5, 6)})
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
    #           written and one 8 B row id read -> 648 B;
    #   apply (segment reduce + carry fix-up): per lookup one 320 B bf16
    #           gradient row read and its 8 B sorted (key, index) pair; per
    #           distinct row one 640 B fp32 sum written (compact) or a 640 B
    #           read + 640 B write (dense).
    gather_bytes = 648.0 * n_avg
    if wl["backward"]:
        u_rows = sum(int(b["compact"][2].item()) for b in wl["batches"]) / R if "compact" in b0 else None
        if u_rows is None:  # dense: distinct rows counted from the plan of rotation 0
            import numpy as np
            u_rows = float(np.unique(b0["rows"].cpu().numpy()).size)
            apply_bytes = 328.0 * n_avg + 1280.0 * u_rows
        else:
            apply_bytes = 328.0 * n_avg + 640.0 * u_rows
    kern = {"gather": (gather_bytes, phase["gather"], "gather_rows_kernel<20,16,true>", "gather.hip")}
    # The plan runs on a side stream during the gather; apply is timed from
    # after the main stream's wait for it.
    if wl["backward"]:
        kern["scatter_apply"] = (apply_bytes, phase["scatter_apply"],
                                 "segment_reduce_kernel<20,bf16> + carry_fixup_kernel + long_run_kernel", "scatter.hip")
    dbytes, dms, dname, dsrc = kern[dom]
    achieved = dbytes / (dms / 1e3) / 1e9
    traffic = counter_traffic(dsrc, "%s_%s_counters.txt" % (dom, args.workload))

    # Three GB/s figures per kernel: per-lookup bytes (above); compulsory
    # bytes, which count each distinct table row's read once (the gather reads
    # (U/L) * 320 + 328 B per lookup); and the HBM bytes the committed
    # rocprofv3 counters measured for that kernel (null when they were taken
    # on other kernel sources).
    import torch as _t
    u_fwd = int(_t.unique(b0["rows"].reshape(-1)).numel())
    compulsory = {"gather": 320.0 * u_fwd + 328.0 * n_avg}
    if wl["backward"]:
        compulsory["scatter_apply"] = apply_bytes   # every gradient row is read once already
    gbps = {}
    for k, (byts, ms, _, src) in kern.items():
        hbm = counter_traffic(src, "%s_%s_counters.txt" % (k, args.workload))
        gbps[k] = {"per_lookup": round(byts / (ms / 1e3) / 1e9, 1),
                   "compulsory": round(compulsory[k] / (ms / 1e3) / 1e9, 1),
                   "counters": None if hbm is None else round(hbm / (ms / 1e3) / 1e9, 1)}
    # Step time distribution from the events (first to last event of a step).
    last = 6 if wl["backward"] else 2
    step_ms = sorted(e[0].elapsed_time(e[last]) for e in evs)
    pct = lambda q: step_ms[min(len(step_ms) - 1, int(q * (len(step_ms) - 1) + 0.5))]
    fwd_ms = phase["hash"] + phase["gather"]
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
            "workload": {"long": "long-context packed THD stream, full table, fwd+bwd (compact grad)",
                         "full-sft": "SFT batch 8x4096, full table, fwd",
                         "owner": "owner shard 1/64 of a world-64 step, fwd+bwd (dense grad)",
                         "sft": "SFT batch 8x4096, 10M-row table, fwd"}[args.workload],
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
                                  "frac": round(gather_bytes / (ga / 1e3) / 1e9 / HBM_PEAK_GBPS, 4)}
    if alone and wl["backward"]:
        bs = alone["scatter_plan"] + alone["scatter_apply"]
        result["backward_plan_then_apply"] = {"ms": round(bs, 4),
                                              "gbps_algorithmic": round(apply_bytes / (bs / 1e3) / 1e9, 1),
                                              "frac": round(apply_bytes / (bs / 1e3) / 1e9 / HBM_PEAK_GBPS, 4)}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
