"""The whole path captured in a HIP graph (torch.cuda.CUDAGraph records the
library's launches on the capture stream).  Every reset the library makes
(status words, counters, count totals) is a kernel, never a memset, so a
replay must equal the eager calls bit for bit.

The graph holds the step in both forms: hash and gather on the capture
stream with the backward plan on a forked stream joined before the apply; and
as the benchmark runs it, the fused hash-and-gather forward on the capture
stream while the forked stream plans from the same tokens (no rows array), also
with a head layout where that plan sorts per head.  Each
replay gets fresh inputs copied into the captured buffers and poisoned
outputs, with eager calls and synchronisations between replays."""
import numpy as np
import pytest
import torch

import hashed_gram_embedding_engram_amd as E
import workloads as W
from tests.gpu_common import head_layout, product_spec_from, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


@pytest.mark.parametrize("fused,split", [(False, False), (True, False), (True, True)])
def test_step_graph_replays_equal_eager(fused, split):
    """split: a head layout (16-bit heads in a 20-bit table) where the plan from
    tokens sorts per head and its keys kernel also does the plan's resets."""
    dev = torch.device("cuda")
    ws = head_layout(60_000) if split else W.sft_spec()
    R, D = ws["num_rows"], 160
    table = torch.empty((R, D), dtype=torch.bfloat16, device=dev)
    W.fill_normal_(table, seed=5)
    spec = product_spec_from(ws)
    B, T = 2, 4059                      # 129,888 lookups: 32 sort tiles, the last one ragged
    n = B * T * 16
    ids = torch.empty((B, T), dtype=torch.int64, device=dev)
    dy = torch.empty((n, D), dtype=torch.bfloat16, device=dev)
    rows = torch.empty((B, T, 16), dtype=torch.int64, device=dev)
    out = torch.empty((B, T, 16, D), dtype=torch.bfloat16, device=dev)
    status = torch.empty((), dtype=torch.int64, device=dev)
    plan_status = torch.empty((), dtype=torch.int64, device=dev)
    workspace = torch.empty(E.engram_scatter_add_workspace(n, R, D), dtype=torch.uint8, device=dev)
    uniq_rows = torch.empty(n, dtype=torch.int64, device=dev)
    uniq_grad = torch.empty((n, D), dtype=torch.float32, device=dev)
    num_uniq = torch.empty((), dtype=torch.int64, device=dev)
    side = torch.cuda.Stream()

    def load_inputs(seed):
        tokens, _ = W.sft_batch(seed, batch=B, seq=T)
        ids.copy_(torch.from_numpy(tokens))
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        dy.copy_(torch.randn((n, D), generator=g, device=dev).to(torch.bfloat16))

    def step():
        main = torch.cuda.current_stream()
        if fused:
            side.wait_stream(main)
            with torch.cuda.stream(side):
                E.engram_scatter_add_plan_from_tokens(ids, spec, R, D, workspace=workspace, uniq_rows=uniq_rows,
                                                      num_uniq=num_uniq, status=plan_status)
            E.engram_hash_gather(ids, spec, table, out=out, status=status, validate=False)
        else:
            E.engram_hash(ids, spec, rows_out=rows)
            side.wait_stream(main)
            with torch.cuda.stream(side):
                E.engram_scatter_add_plan(rows, R, D, workspace=workspace, uniq_rows=uniq_rows, num_uniq=num_uniq,
                                          status=plan_status)
            E.engram_gather(table, rows, out=out, status=status, validate=False)
        main.wait_stream(side)
        E.engram_scatter_add_apply(dy, n, R, workspace, uniq_grad=uniq_grad)

    load_inputs(100)
    warm = torch.cuda.Stream()
    warm.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(warm):
        step()
    torch.cuda.current_stream().wait_stream(warm)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for seed in (101, 102, 101, 103):
        load_inputs(seed)
        # eager reference into buffers of its own
        ref_rows = E.engram_hash(ids, spec)
        ref_out = E.engram_gather(table, ref_rows)
        ref_ur, ref_ug = E.engram_scatter_add(ref_rows, dy, R)
        torch.cuda.synchronize()
        # poison everything the graph writes, so a replay that skips a write fails
        rows.fill_(-1)
        out.fill_(1.0)
        uniq_rows.fill_(-7)
        uniq_grad.fill_(float("nan"))
        num_uniq.fill_(-1)
        status.fill_(-5)
        plan_status.fill_(-5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        u = int(num_uniq.item())
        assert u == ref_ur.numel()
        if not fused:   # the fused step writes no rows array
            assert torch.equal(rows, ref_rows)
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
        assert torch.equal(uniq_rows[:u], ref_ur)
        assert np.array_equal(uniq_grad[:u].cpu().numpy().view(np.uint32), ref_ug.cpu().numpy().view(np.uint32))
        assert int(status.item()) == -1 and int(plan_status.item()) == -1
