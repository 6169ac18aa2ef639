"""The largest lookup count the scatter-add accepts (n = 2^31 - 1) and the same
count through the gather, with 16-byte rows (8 bf16 values) so that everything
fits in HBM (about 92 GB for the scatter-add, 52 GB for the gather);
gathers whose work passes what one launch can hold (2^32 work-items), up to
172 GB of output; and the plan from tokens at its largest batch, where its sort
runs per head.

The oracle cannot run at this size, so both checks use properties that hold at
any size.  Lookup i reads row (i * 7919) mod R with R = 1,000,003 (prime, and
7919 is invertible mod R), so row r is hit by the lookups i = i0(r) + k R with
i0(r) = r * 7919^-1 mod R: count(r) = (n - 1 - i0(r)) // R + 1.  With every
gradient value 1, the fp64 sum of row r is exactly count(r) (below 2^24, so
exact in fp32 too).  The gather is compared bit for bit with index_select,
in chunks of 2^22 rows."""
import pytest
import torch

import hashed_gram_embedding_engram_amd as E
from tests.gpu_common import requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]

N_MAX = (1 << 31) - 1
R = 1_000_003
MULT = 7919
DIM = 8
CHUNK = 1 << 27
REF_CHUNK = 1 << 22  # torch's index_select rejects the launch for a 2^27-row index


def strided_rows(n, dev):
    rows = torch.empty(n, dtype=torch.int64, device=dev)
    for a in range(0, n, CHUNK):
        b = min(n, a + CHUNK)
        rows[a:b] = torch.arange(a, b, dtype=torch.int64, device=dev).mul_(MULT).remainder_(R)
    return rows


def expected_counts(n, dev):
    inv = pow(MULT, -1, R)
    i0 = torch.arange(R, dtype=torch.int64, device=dev).mul_(inv).remainder_(R)
    return torch.where(i0 < n, (n - 1 - i0) // R + 1, torch.zeros_like(i0))


def test_scatter_add_at_max_lookups():
    dev = torch.device("cuda")
    torch.cuda.empty_cache()
    rows = strided_rows(N_MAX, dev)
    dy = torch.ones((N_MAX, DIM), dtype=torch.bfloat16, device=dev)
    grad = torch.zeros((R, DIM), dtype=torch.float32, device=dev)
    grad[:, 0] = 0.5                      # the dense form adds to what is there
    E.engram_scatter_add(rows, dy, R, grad_dense=grad)   # validates: raises on any out-of-range row
    torch.cuda.synchronize()
    counts = expected_counts(N_MAX, dev)
    assert int(counts.sum().item()) == N_MAX
    want = counts.to(torch.float32)
    assert torch.equal(grad[:, 1:], want[:, None].expand(R, DIM - 1))
    assert torch.equal(grad[:, 0], want + 0.5)
    del rows, dy, grad
    torch.cuda.empty_cache()


def test_gather_at_max_lookups():
    dev = torch.device("cuda")
    torch.cuda.empty_cache()
    g = torch.Generator(device=dev)
    g.manual_seed(31)
    table = torch.randn((R, DIM), generator=g, device=dev).to(torch.bfloat16)
    rows = strided_rows(N_MAX, dev)
    out = E.engram_gather(table, rows)   # validates: raises on any out-of-range row
    torch.cuda.synchronize()
    assert out.shape == (N_MAX, DIM)
    gather_matches_index_select(table, rows, out)
    del rows, out, table
    torch.cuda.empty_cache()


def gather_matches_index_select(table, rows, out):
    n = rows.numel()
    for a in range(0, n, REF_CHUNK):
        b = min(n, a + REF_CHUNK)
        ref = torch.index_select(table, 0, rows[a:b])
        assert torch.equal(out[a:b].view(torch.int16), ref.view(torch.int16)), (a, b)


@pytest.mark.parametrize("dim,n", [
    (256, (1 << 27) + 5),    # generic kernel: n * 32 chunks > 2^32 work-items, 69 GB of output
    (160, (1 << 29) + 3),    # the 160-wide kernel's grid would pass 2^31 work-items: generic kernel, 172 GB
])
def test_gather_past_one_launch_of_work_items(dim, n):
    dev = torch.device("cuda")
    torch.cuda.empty_cache()
    g = torch.Generator(device=dev)
    g.manual_seed(dim)
    table = torch.randn((R, dim), generator=g, device=dev).to(torch.bfloat16)
    rows = strided_rows(n, dev)
    out = E.engram_gather(table, rows)   # validates: raises on any out-of-range row
    torch.cuda.synchronize()
    gather_matches_index_select(table, rows, out)
    del rows, out, table
    torch.cuda.empty_cache()


def test_plan_from_tokens_split_at_max_lookups():
    """The largest token batch the plan from tokens accepts (2^27 - 1 positions, so
    n = 2^31 - 16 lookups) with the released heads over the full row range, where the
    sort runs per head with a last pass of 9 bits: its dense sums equal those of the
    whole sort from engram_hash's rows bit for bit.  Every gradient value is 1, so each
    row's sum is its exact hit count, and the counts add up to n."""
    dev = torch.device("cuda")
    torch.cuda.empty_cache()
    positions = (1 << 27) - 1
    g = torch.Generator(device=dev)
    g.manual_seed(37)
    tokens = torch.randint(0, 248_320, (1, positions), generator=g, device=dev, dtype=torch.int64)
    n = positions * 16
    spec = E.qwen3_8_flash_next_spec()
    rows_total = E.QWEN3_8_FLASH_NEXT_NGRAM_PADDED_ROWS
    dy = torch.ones((n, DIM), dtype=torch.bfloat16, device=dev)
    whole = torch.zeros((rows_total, DIM), dtype=torch.float32, device=dev)
    rows = E.engram_hash(tokens, spec).view(-1)
    E.engram_scatter_add(rows, dy, rows_total, grad_dense=whole)   # validates: raises on any out-of-range row
    torch.cuda.synchronize()
    del rows
    torch.cuda.empty_cache()
    split = torch.zeros_like(whole)
    ws = E.engram_scatter_add_plan_from_tokens(tokens, spec, rows_total, DIM)
    E.engram_scatter_add_apply(dy, n, rows_total, ws, grad_dense=split)
    torch.cuda.synchronize()
    assert torch.equal(split, whole)
    assert int(split[:, 0].double().sum().item()) == n
    del tokens, dy, whole, split, ws
    torch.cuda.empty_cache()
