"""Parity at full size, in the launch configuration the benchmark times:
the 320,001,536 x 160 bf16 table (102.4 GB) held whole on one GPU, the SFT and
long-context streams, and the owner shard of a world-64 step.  Everything is
compared in full: the hash, the backward, and every lookup of the forward
gather.  For the gather the table streams to the host in contiguous chunks of
at most 1 GiB (plain copies, no device-side indexing), the oracle gathers each
chunk's lookups with row_begin at the chunk start, and host memory never holds
more than one chunk of the table."""
import numpy as np
import pytest
import torch

import hashed_gram_embedding_engram_amd as E
import workloads as W
from oracle import c_oracle
from tests.gpu_common import assert_close_to_fp64, full_oracle_spec, oracle_hash, requires_gpu, to_host

pytestmark = [pytest.mark.gpu, requires_gpu]


@pytest.fixture(scope="module")
def full_table():
    free, _ = torch.cuda.mem_get_info()
    need = W.FULL_ROWS * W.DIM * 2
    if free < need + (24 << 30):
        pytest.skip("needs %.1f GB free on the GPU" % (need / 1e9))
    t = torch.empty((W.FULL_ROWS, W.DIM), dtype=torch.bfloat16, device="cuda")
    W.fill_normal_(t, seed=1234)
    yield t
    del t
    torch.cuda.empty_cache()


CHUNK_BYTES = 1 << 30


def streamed_gather_check(table, outs, rows_ref, row_begin=0):
    """Every lookup's output row, in each of `outs` (one output or several), equals
    the oracle's gather of the table row it names.  The lookups are ordered by row
    on the host; for each chunk of table rows holding at least one of them, the
    chunk is copied to the host and the C oracle gathers exactly those lookups
    from it."""
    rows_ref = np.ascontiguousarray(rows_ref, dtype=np.int64).reshape(-1)
    num_rows, dim = table.shape
    outs = outs if isinstance(outs, (list, tuple)) else [outs]
    got = [to_host(o.reshape(-1, dim)) for o in outs]
    assert all(g.shape[0] == rows_ref.size for g in got)
    order = np.argsort(rows_ref, kind="stable")
    srt = rows_ref[order]
    assert srt[0] >= row_begin and srt[-1] < row_begin + num_rows     # every row lies in the table
    chunk_rows = max(1, CHUNK_BYTES // (dim * table.element_size()))
    host = torch.empty((chunk_rows, dim), dtype=table.dtype, pin_memory=True)
    checked = 0
    for c0 in range(0, num_rows, chunk_rows):
        c1 = min(num_rows, c0 + chunk_rows)
        lo, hi = np.searchsorted(srt, [row_begin + c0, row_begin + c1])
        if lo == hi:
            continue
        host[:c1 - c0].copy_(table[c0:c1])
        chunk = to_host(host[:c1 - c0])
        sel = order[lo:hi]
        ref, bad = c_oracle.gather(chunk, rows_ref[sel], row_begin=row_begin + c0)
        assert bad == -1
        for k, got_all in enumerate(got):
            if not np.array_equal(got_all[sel], ref):
                i = int(np.argwhere((got_all[sel] != ref).any(axis=1))[0][0])
                raise AssertionError("output %d: lookup %d (row %d) differs from the oracle"
                                     % (k, sel[i], rows_ref[sel[i]]))
        checked += hi - lo
    assert checked == rows_ref.size


def test_full_table_sft_forward(full_table):
    """Hash then gather, and the fused forward (with and without its rows), on
    the SFT batch: every lookup of both outputs against the oracle."""
    ids, _ = W.sft_batch(0)
    tokens = torch.from_numpy(ids).cuda()
    spec = E.qwen3_8_flash_next_spec()
    rows = E.engram_hash(tokens, spec)
    out = E.engram_gather(full_table, rows)
    fused_rows = torch.empty_like(rows)
    fused = E.engram_hash_gather(tokens, spec, full_table, rows_out=fused_rows)
    fused_bare = E.engram_hash_gather(tokens, spec, full_table)
    rows_ref = oracle_hash(ids, full_oracle_spec())
    assert np.array_equal(rows.cpu().numpy(), rows_ref)
    assert np.array_equal(fused_rows.cpu().numpy(), rows_ref)
    assert out.shape == fused.shape == (8, 4096, 16, 160)
    assert torch.equal(fused.view(torch.int16), fused_bare.view(torch.int16))
    del fused_bare
    streamed_gather_check(full_table, [out, fused], rows_ref)


def test_full_table_long_context_step(full_table):
    """Hash + gather + compact backward on the 262,144-token packed stream."""
    ids, _ = W.long_context_stream(0)
    tokens = torch.from_numpy(ids).cuda()
    rows = E.engram_hash(tokens, E.qwen3_8_flash_next_spec())
    out = E.engram_gather(full_table, rows)
    fused = E.engram_hash_gather(tokens, E.qwen3_8_flash_next_spec(), full_table)   # the benchmark's forward
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    dy = torch.randn(out.shape, generator=g, device="cuda").to(torch.bfloat16)
    ur, ug = E.engram_scatter_add(rows, dy, W.FULL_ROWS)
    rows_ref = oracle_hash(ids, full_oracle_spec())
    assert np.array_equal(rows.cpu().numpy(), rows_ref)
    streamed_gather_check(full_table, [out, fused], rows_ref)
    dy_host = to_host(dy).reshape(-1, 160)
    del out, fused, dy
    rur, rug, bad = c_oracle.scatter_add_compact(rows_ref.reshape(-1), dy_host, W.FULL_ROWS)
    assert bad == -1
    assert np.array_equal(ur.cpu().numpy(), rur)
    assert_close_to_fp64(ug.cpu().numpy(), rug, "long-context compact backward")


def test_owner_shard_step():
    """Owner 0 of a world-64 table: the lookups of 64 request ranks that fall in
    rows [0, 5,000,024), gathered from the shard and scattered into a dense fp32
    gradient, both from the compact rows and from the padded [64][capacity]
    blocks the exchange delivers."""
    ids = W.owner_token_batches().reshape(-1, 4096)
    spec = E.qwen3_8_flash_next_spec()
    rows_all = E.engram_hash(torch.from_numpy(ids).cuda(), spec).reshape(-1)
    owner = rows_all[rows_all < W.OWNER_ROWS].contiguous()          # what the owner receives
    rows_ref_all = oracle_hash(ids, full_oracle_spec()).reshape(-1)
    rows_ref = rows_ref_all[rows_ref_all < W.OWNER_ROWS]
    assert np.array_equal(owner.cpu().numpy(), rows_ref)
    shard = torch.empty((W.OWNER_ROWS, W.DIM), dtype=torch.bfloat16, device="cuda")
    W.fill_normal_(shard, seed=99)
    out = E.engram_gather(shard, owner)
    streamed_gather_check(shard, out, rows_ref)
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    dy = torch.randn(out.shape, generator=g, device="cuda").to(torch.bfloat16)
    grad = torch.zeros((W.OWNER_ROWS, W.DIM), dtype=torch.float32, device="cuda")
    E.engram_scatter_add(owner, dy, W.OWNER_ROWS, grad_dense=grad)
    rur, rug, bad = c_oracle.scatter_add_compact(rows_ref, to_host(dy), W.OWNER_ROWS)
    assert bad == -1
    counts = np.bincount(rows_ref, minlength=W.OWNER_ROWS)
    assert counts.max() > 10000                                        # hot rows are present
    assert_close_to_fp64(grad[torch.from_numpy(rur).cuda()].cpu().numpy(), rug, "owner dense backward")
    touched = torch.zeros(W.OWNER_ROWS, dtype=torch.bool, device="cuda")
    touched[torch.from_numpy(rur).cuda()] = True
    assert int((grad[~touched] != 0).sum().item()) == 0

    # The same lookups as the exchange delivers them to the owner: request rank
    # w's rows in block w of the agreed capacity (the largest count), padding
    # after them; the owner's response and backward read these blocks directly.
    counts_np = (rows_ref_all.reshape(64, -1) < W.OWNER_ROWS).sum(1).astype(np.int64)
    cap = int(counts_np.max())
    counts = torch.from_numpy(counts_np).cuda()
    real = torch.from_numpy(np.arange(cap)[None, :] < counts_np[:, None]).cuda().reshape(-1)
    ids_pad = E.engram_pack_fixed_capacity(owner, counts, 64, cap, fill=-1)
    vals = E.engram_gather_padded(shard, ids_pad, counts).reshape(-1, W.DIM)
    streamed_gather_check(shard, vals[real], rows_ref)         # real entries, in rank order
    assert int((vals[~real] != 0).sum().item()) == 0             # padding rows are zero
    del vals
    dy_pad = E.engram_pack_fixed_capacity(dy, counts, 64, cap, fill=0)
    m = 64 * cap
    grad_pad = torch.zeros_like(grad)
    ws = E.engram_scatter_add_plan_padded(ids_pad, counts, W.OWNER_ROWS, W.DIM)
    E.engram_scatter_add_apply(dy_pad.view(m, W.DIM), m, W.OWNER_ROWS, ws, grad_dense=grad_pad)
    assert_close_to_fp64(grad_pad[torch.from_numpy(rur).cuda()].cpu().numpy(), rug, "owner backward from blocks")
    assert int((grad_pad[~touched] != 0).sum().item()) == 0
    # Padding sorts after every row and the rows keep their relative order, so
    # the sums are those of the compact form bit for bit.
    assert torch.equal(grad_pad, grad)
