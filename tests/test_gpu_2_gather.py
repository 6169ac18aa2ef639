"""Row-gather kernel parity: bit-exact against the oracle's gather."""
import numpy as np
import pytest
import torch

import hashed_gram_embedding_engram_amd as E
import workloads as W
from oracle import c_oracle
from tests.gpu_common import oracle_hash, product_spec_from, requires_gpu, to_host

pytestmark = [pytest.mark.gpu, requires_gpu]


def check_gather(table_gpu, rows_np, row_begin=0, expect_bad=-1):
    rows = torch.from_numpy(np.ascontiguousarray(rows_np, dtype=np.int64)).cuda()
    status = torch.empty((), dtype=torch.int64, device="cuda")
    out = E.engram_gather(table_gpu, rows, row_begin, status=status, validate=False)
    torch.cuda.synchronize()
    ref, bad = c_oracle.gather(to_host(table_gpu), rows_np, row_begin)
    got = to_host(out)
    assert got.shape == ref.shape
    assert np.array_equal(got.view(np.uint8), ref.view(np.uint8))
    assert int(status.item()) == bad == expect_bad
    return out


def test_tiny_case_fp32():
    ws = W.tiny_spec()
    table = torch.from_numpy(W.tiny_table(ws["num_rows"])).cuda()
    rows = oracle_hash(W.tiny_tokens(), ws)
    check_gather(table, rows)


def test_tiny_product_rows():
    """The whole forward on the GPU (hash then gather) equals the oracle's."""
    ws = W.tiny_spec()
    table = torch.from_numpy(W.tiny_table(ws["num_rows"])).cuda()
    ids = W.tiny_tokens()
    rows = E.engram_hash(torch.from_numpy(ids).cuda(), product_spec_from(ws))
    out = E.engram_gather(table, rows)
    ref, _ = c_oracle.gather(W.tiny_table(ws["num_rows"]), oracle_hash(ids, ws))
    assert out.shape == (1, 256, 16, 160)
    assert np.array_equal(to_host(out).view(np.uint32), ref.view(np.uint32))
    # viewed as the concatenated [batch, seq, heads * dim] embedding
    assert out.reshape(1, 256, 16 * 160).is_contiguous()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("n", [1, 2, 15, 16, 17, 63, 64, 65, 1000, 4099])
def test_ragged_counts(dtype, n):
    g = torch.Generator(device="cuda")
    g.manual_seed(n)
    table = torch.randn((3000, 160), generator=g, device="cuda").to(dtype)
    rows = np.random.default_rng(n).integers(0, 3000, size=n).astype(np.int64)
    check_gather(table, rows)


def test_empty():
    table = torch.zeros((10, 160), dtype=torch.bfloat16, device="cuda")
    out = E.engram_gather(table, torch.empty(0, dtype=torch.int64, device="cuda"))
    assert out.shape == (0, 160)


@pytest.mark.parametrize("dtype,dim", [(torch.bfloat16, 8), (torch.bfloat16, 64), (torch.bfloat16, 512),
                                       (torch.float32, 4), (torch.float32, 12), (torch.float32, 256)])
def test_other_widths(dtype, dim):
    g = torch.Generator(device="cuda")
    g.manual_seed(dim)
    table = torch.randn((777, dim), generator=g, device="cuda").to(dtype)
    rows = np.random.default_rng(dim).integers(0, 777, size=1234).astype(np.int64)
    check_gather(table, rows)


def test_owner_window_and_bad_rows():
    """Shard [row_begin, row_begin + num_rows): rows outside give zero rows and the
    lowest offending lookup index in status; nothing outside the shard is read."""
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    rb, R = 1_000_000, 5000
    table = torch.randn((R, 160), generator=g, device="cuda").to(torch.bfloat16)
    rng = np.random.default_rng(3)
    rows = rng.integers(rb, rb + R, size=5000).astype(np.int64)
    check_gather(table, rows, rb)
    bad = rows.copy()
    bad[[4000, 777, 4999]] = [rb - 1, rb + R, -(1 << 63)]
    check_gather(table, bad, rb, expect_bad=777)
    bad[[3]] = (1 << 63) - 1
    check_gather(table, bad, rb, expect_bad=3)
    with pytest.raises(E.EngramError, match="outside the owned range"):
        E.engram_gather(table, torch.from_numpy(bad).cuda(), rb)


def test_sft_table_full_parity():
    """SFT shape: [8, 4096] Zipf(1.1) tokens over a 10,000,000-row bf16 table, every lookup."""
    ws = W.sft_spec()
    table = torch.empty((ws["num_rows"], 160), dtype=torch.bfloat16, device="cuda")
    W.fill_normal_(table, seed=11)
    ids, _ = W.sft_batch(0)
    rows_gpu = E.engram_hash(torch.from_numpy(ids).cuda(), product_spec_from(ws))
    out = E.engram_gather(table, rows_gpu)
    rows_ref = oracle_hash(ids, ws)
    ref, bad = c_oracle.gather(to_host(table), rows_ref)
    assert bad == -1
    assert np.array_equal(to_host(out), ref)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_wide_shard_row_ids(dtype):
    """A shard declared with 2^32 + 5 rows takes the 64-bit row-id path.  Only rows
    inside the allocated 4,000-row prefix are looked up (plus rows outside the
    declared shard, which are never read), so every access stays in the table."""
    g = torch.Generator(device="cuda")
    g.manual_seed(17)
    rb, R, declared = 7, 4000, (1 << 32) + 5
    table = torch.randn((R, 160), generator=g, device="cuda").to(dtype)
    rng = np.random.default_rng(17)
    rows = rng.integers(rb, rb + R, size=3001).astype(np.int64)
    rows[[100, 2500]] = [rb + declared, rb - 1]
    out = torch.empty((rows.size, 160), dtype=dtype, device="cuda")
    status = torch.empty((), dtype=torch.int64, device="cuda")
    rows_gpu = torch.from_numpy(rows).cuda()
    lib = E.load_library()
    rc = lib.engram_gather(table.data_ptr(), 1 if dtype == torch.bfloat16 else 0, rb, declared, 160,
                           rows_gpu.data_ptr(), rows.size, out.data_ptr(), status.data_ptr(), None)
    assert rc == 0
    torch.cuda.synchronize()
    in_table = (rows >= rb) & (rows < rb + R)
    ref, _ = c_oracle.gather(to_host(table), np.where(in_table, rows, rb), rb)
    ref[~in_table] = 0
    assert np.array_equal(to_host(out).view(np.uint8), ref.view(np.uint8))
    assert int(status.item()) == 100


@pytest.mark.parametrize("dtype,dim", [(torch.bfloat16, 160), (torch.float32, 160), (torch.bfloat16, 64)])
def test_empty_shard(dtype, dim):
    """An owner with no rows: every lookup is out of range, so every output row is
    zero and the status names lookup 0; the (empty) table is never read."""
    table = torch.empty((0, dim), dtype=dtype, device="cuda")
    rows = torch.arange(37, dtype=torch.int64, device="cuda") * 1000
    status = torch.empty((), dtype=torch.int64, device="cuda")
    out = torch.full((37, dim), 7, dtype=dtype, device="cuda")
    E.engram_gather(table, rows, 0, out=out, status=status, validate=False)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(out, torch.zeros_like(out))
    with pytest.raises(E.EngramError, match="outside the owned range"):
        E.engram_gather(table, rows)
