"""HBM ceilings of this machine, from the kernels of libengram_probe.so
(csrc/hbm_probe.hip): what plain streaming reads and writes, and plain
kernels with the traffic of the forward gather and of the backward's sums,
reach.  The benchmark reports them beside the lookup kernels' rates."""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB_PATH = os.path.join(_PKG, "libengram_probe.so")
_lib = None


def load_probe():
    global _lib
    if _lib is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise RuntimeError("libengram_probe.so not found at %s: run the package build" % PROBE_LIB_PATH)
        lib = ctypes.CDLL(PROBE_LIB_PATH)
        lib.engram_probe.restype = ctypes.c_int
        lib.engram_probe.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                     ctypes.c_int, ctypes.c_void_p]
        _lib = lib
    return _lib


def run_probe(kind, src, idx, count, dst, grid, stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    rc = load_probe().engram_probe(kind, ctypes.c_void_p(src.data_ptr()) if src is not None else None,
                                   ctypes.c_void_p(idx.data_ptr()) if idx is not None else None, count,
                                   ctypes.c_void_p(dst.data_ptr()), grid, ctypes.c_void_p(s.cuda_stream))
    if rc != 0:
        raise RuntimeError("engram_probe(%d) failed: hipError %d" % (kind, rc))


def _median_ms(fn, reps):
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ms = []
    for _ in range(reps):
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    return sorted(ms)[len(ms) // 2]


RMW_READS = 4  # bf16 rows the rmw probe adds into each fp32 row


def _tiles(rows):
    """Blocks for one 16-row tile per wave (4 waves per block)."""
    return max(1, (rows + 63) // 64)


def measure_ceilings(dev, reps=10, stream_bytes=4 << 30, table_rows=25_000_000, lookups=4_194_304,
                     distinct=3_163_052, grid=8192, seed=0, dense_rows=5_000_024, dense_distinct=156_202,
                     dense_lookups=562_578):
    """GB/s of each probe (bytes the kernel must move / median time).  The
    streaming probes stride over their buffer with `grid` blocks; the row probes
    launch one 16-row tile per wave (their fastest launch shape, as the lookup
    kernels launch one unit of work per wave).  The gather
    reads `lookups` uniform-random 320-byte rows of a `table_rows`-row bf16 table;
    the expand reads `distinct` distinct rows of a `lookups`-row bf16 array in
    random order and writes them as fp32; the rmw adds RMW_READS random rows
    of a `dense_lookups`-row bf16 array into each of `dense_distinct` distinct
    random fp32 rows of a `dense_rows`-row array (the owner shard's sizes)."""
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    out = {}
    buf = torch.empty(stream_bytes // 2, dtype=torch.int16, device=dev).fill_(1)
    sink = torch.empty((grid, 4), dtype=torch.int32, device=dev)
    out["read"] = stream_bytes / _median_ms(lambda: run_probe(0, buf, None, stream_bytes, sink, grid), reps) / 1e6
    out["write"] = stream_bytes / _median_ms(lambda: run_probe(1, None, None, stream_bytes, buf, grid), reps) / 1e6
    del buf, sink
    table = torch.empty((table_rows, 160), dtype=torch.bfloat16, device=dev).fill_(1.0)
    idx = torch.randint(0, table_rows, (lookups,), generator=g, device=dev, dtype=torch.int64).to(torch.int32)
    dst = torch.empty((lookups, 160), dtype=torch.bfloat16, device=dev)
    ms = _median_ms(lambda: run_probe(2, table, idx, lookups, dst, _tiles(lookups)), reps)
    out["row_gather"] = lookups * (320 + 320 + 4) / ms / 1e6
    del table, idx, dst
    src = torch.empty((lookups, 160), dtype=torch.bfloat16, device=dev).fill_(1.0)
    idx = torch.randperm(lookups, generator=g, device=dev)[:distinct].to(torch.int32).contiguous()
    dst = torch.empty((distinct, 160), dtype=torch.float32, device=dev)
    ms = _median_ms(lambda: run_probe(3, src, idx, distinct, dst, _tiles(distinct)), reps)
    out["row_expand"] = distinct * (320 + 640 + 4) / ms / 1e6
    del src, idx, dst
    src = torch.empty((dense_lookups, 160), dtype=torch.bfloat16, device=dev).fill_(1.0)
    reads = torch.randint(0, dense_lookups, (dense_distinct * RMW_READS,), generator=g, device=dev,
                          dtype=torch.int64)
    rows = torch.randperm(dense_rows, generator=g, device=dev)[:dense_distinct]
    idx = torch.cat([reads, rows]).to(torch.int32).contiguous()
    dst = torch.zeros((dense_rows, 160), dtype=torch.float32, device=dev)
    ms = _median_ms(lambda: run_probe(4, src, idx, dense_distinct, dst, _tiles(dense_distinct)), reps)
    out["row_rmw"] = dense_distinct * (RMW_READS * (320 + 4) + 640 + 640 + 4) / ms / 1e6
    del src, reads, rows, idx, dst
    torch.cuda.empty_cache()
    return {k: round(v, 1) for k, v in out.items()}
