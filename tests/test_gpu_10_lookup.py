"""The path from tokens without a rows array.  Fused forward (engram_hash_gather):
bit-exact against the oracle's hash followed by the oracle's gather; the released
head layout (3-gram, 8 heads per order) with a 160-wide bf16 table takes the
one-kernel path, other layouts and fp32 tables the hash-then-gather path through
rows_out.  The backward's plan from tokens (engram_scatter_add_plan_from_tokens):
plan + apply against the oracle's scatter-add of the oracle's rows, for the whole
sort and for the sort split by head."""
import ctypes

import numpy as np
import pytest
import torch

import hashed_gram_embedding_engram_amd as E
import workloads as W
from oracle import c_oracle, constants as C
from tests.gpu_common import (assert_close_to_fp64, full_oracle_spec, head_layout, oracle_hash, product_spec_from,
                               requires_gpu, to_host)

pytestmark = [pytest.mark.gpu, requires_gpu]

INT64_MAX, INT64_MIN = (1 << 63) - 1, -(1 << 63)


def bf16_table(num_rows, seed, dtype=torch.bfloat16):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn((num_rows, 160), generator=g, device="cuda").to(dtype)


def check(ids, ws, table, row_begin=0, fill=None, with_rows=True, spec=None):
    """Run the fused forward and compare out, status and rows_out with the oracle."""
    spec = spec if spec is not None else product_spec_from(ws, fill)
    ids = np.ascontiguousarray(ids, dtype=np.int64)
    batch, seq = ids.shape
    heads = spec.num_heads
    tokens = torch.from_numpy(ids).cuda()
    status = torch.empty((), dtype=torch.int64, device="cuda")
    rows_out = torch.full((batch, seq, heads), -7, dtype=torch.int64, device="cuda") if with_rows else None
    out = E.engram_hash_gather(tokens, spec, table, row_begin, rows_out=rows_out, status=status, validate=False)
    torch.cuda.synchronize()
    ref_rows = oracle_hash(ids, ws, fill=fill)
    ref, bad = c_oracle.gather(to_host(table), ref_rows.reshape(-1), row_begin)
    assert out.shape == (batch, seq, heads, table.shape[1])
    assert np.array_equal(to_host(out).reshape(ref.shape).view(np.uint8), ref.view(np.uint8))
    assert int(status.item()) == bad
    if with_rows:
        assert np.array_equal(rows_out.cpu().numpy(), ref_rows)
    return bad


def uniform_ids(shape, seed, eos, p_eos=1.0 / 16, vocab=1000):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, vocab, size=shape, dtype=np.int64)
    ids[rng.random(shape) < p_eos] = eos
    return ids


@pytest.mark.parametrize("with_rows", [True, False])
def test_tiny_tokens_fused(with_rows):
    ws = W.tiny_spec()
    assert check(W.tiny_tokens(), ws, bf16_table(ws["num_rows"], 1), with_rows=with_rows) == -1


@pytest.mark.parametrize("shape", [(1, 1), (1, 2), (1, 3), (3, 5), (2, 63), (2, 64), (2, 65), (4, 1000), (7, 333)])
def test_ragged_shapes(shape):
    """Batch rows of every short length (history before the row start is the fill)
    and shapes whose positions end in a partial block."""
    ws = W.tiny_spec()
    ids = uniform_ids(shape, sum(shape), ws["eos"])
    check(ids, ws, bf16_table(ws["num_rows"], 2), with_rows=shape[0] % 2 == 1)


@pytest.mark.parametrize("fill", [0, -1, INT64_MAX, INT64_MIN, 998])
def test_fill_values(fill):
    ws = W.tiny_spec()
    ids = uniform_ids((3, 200), 7, ws["eos"], p_eos=0.2)
    check(ids, ws, bf16_table(ws["num_rows"], 3), fill=fill)


def test_eos_runs_and_extreme_tokens():
    """Runs of EOS, EOS at the first and last positions, and int64 extremes as tokens."""
    ws = W.tiny_spec()
    e = ws["eos"]
    ids = np.array([[e, e, 5, e, e, e, 6, 7, 8, e, 9, e],
                    [1, 2, 3, 4, e, 1, 2, e, e, 3, 4, 5],
                    [INT64_MAX, INT64_MIN, -1, 0, e, INT64_MIN, INT64_MAX, 1 << 40, -(1 << 40), e, 2, 3]],
                   dtype=np.int64)
    check(ids, ws, bf16_table(ws["num_rows"], 4))


def test_rows_outside_the_shard():
    """A shard in the middle of the table: rows outside it give zero output rows and
    the lowest such lookup index in status."""
    ws = W.tiny_spec()
    row_begin, num_rows = 20_000, 30_000
    ids = uniform_ids((5, 300), 11, ws["eos"])
    bad = check(ids, ws, bf16_table(num_rows, 5), row_begin=row_begin)
    assert bad >= 0


def test_released_constants_on_the_owner_shard():
    """The released spec (moduli above 20,000,000, Barrett reduction) on owner 0's
    5,000,024-row shard, with an SFT batch: most rows fall outside the shard."""
    ws = full_oracle_spec()
    ids, _ = W.sft_batch(seed=3)
    table = bf16_table(W.OWNER_ROWS, 6)
    check(ids, ws, table, spec=E.qwen3_8_flash_next_spec())


def test_sft_batch_on_its_table():
    """The SFT configuration's spec and 10,000,000-row table, all 524,288 lookups."""
    ws = W.sft_spec()
    ids, _ = W.sft_batch(seed=0)
    check(ids, ws, bf16_table(ws["num_rows"], 7))


def test_two_kernel_path():
    """fp32 table and a 2-gram layout: the forward runs the hash into rows_out and
    the gather from it; without rows_out such a call is refused."""
    ws = W.tiny_spec()
    ids = uniform_ids((2, 100), 13, ws["eos"])
    check(ids, ws, bf16_table(ws["num_rows"], 8, torch.float32))
    with pytest.raises(E.EngramError):
        E.engram_hash_gather(torch.from_numpy(ids).cuda(), product_spec_from(ws),
                             bf16_table(ws["num_rows"], 8, torch.float32))
    two = dict(ws, ngram_size=2, vocab_sizes=ws["vocab_sizes"][:8], offsets=ws["offsets"][:8])
    check(ids, two, bf16_table(ws["num_rows"], 9))


def test_validate_raises_on_rows_outside_the_shard():
    ws = W.tiny_spec()
    ids = uniform_ids((1, 64), 17, ws["eos"])
    with pytest.raises(E.EngramError, match="outside the owned range"):
        E.engram_hash_gather(torch.from_numpy(ids).cuda(), product_spec_from(ws), bf16_table(10, 10), 0)


# ---- The backward's plan from tokens (engram_scatter_add_plan_from_tokens): the
# rows are hashed inside the plan's first kernel; plan + apply must equal the
# oracle's scatter-add of the oracle's rows, compact and dense.

def grads(n, seed, dim=160):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn((n, dim), generator=g, device="cuda").to(torch.bfloat16)


def check_plan_from_tokens(ids, ws, num_rows, row_begin=0, fill=None, dim=160, dense=False, seed=0):
    spec = product_spec_from(ws, fill)
    ids = np.ascontiguousarray(ids, dtype=np.int64)
    tokens = torch.from_numpy(ids).cuda()
    n = ids.size * 16
    dy = grads(n, seed, dim)
    status = torch.empty((), dtype=torch.int64, device="cuda")
    ur = torch.full((n,), -7, dtype=torch.int64, device="cuda")
    nu = torch.empty((), dtype=torch.int64, device="cuda")
    ws_t = E.engram_scatter_add_plan_from_tokens(tokens, spec, num_rows, dim, row_begin, uniq_rows=ur, num_uniq=nu,
                                                 status=status)
    rows_ref = oracle_hash(ids, ws, fill=fill).reshape(-1)
    dy_host = to_host(dy)
    if dense:
        g = torch.zeros((num_rows, dim), dtype=torch.float32, device="cuda")
        E.engram_scatter_add_apply(dy, n, num_rows, ws_t, row_begin, grad_dense=g)
        ref, rbad = c_oracle.scatter_add_dense(rows_ref, dy_host, num_rows, row_begin)
        torch.cuda.synchronize()
        assert int(status.item()) == rbad
        assert_close_to_fp64(g.cpu().numpy(), ref, "dense sums from tokens")
        return rbad
    ug = torch.empty((n, dim), dtype=torch.float32, device="cuda")
    E.engram_scatter_add_apply(dy, n, num_rows, ws_t, row_begin, uniq_grad=ug)
    torch.cuda.synchronize()
    rur, rug, rbad = c_oracle.scatter_add_compact(rows_ref, dy_host, num_rows, row_begin)
    u = int(nu.item())
    assert int(status.item()) == rbad
    assert u == rur.size and np.array_equal(ur[:u].cpu().numpy(), rur)
    assert_close_to_fp64(ug[:u].cpu().numpy(), rug, "compact sums from tokens")
    return rbad


@pytest.mark.parametrize("shape", [(1, 1), (1, 2), (1, 3), (3, 5), (2, 63), (4, 1000), (7, 333), (1, 4099)])
def test_plan_from_tokens_ragged(shape):
    ws = W.tiny_spec()
    check_plan_from_tokens(uniform_ids(shape, sum(shape) + 1, ws["eos"]), ws, ws["num_rows"], seed=sum(shape))


@pytest.mark.parametrize("fill", [0, -1, INT64_MAX, INT64_MIN])
def test_plan_from_tokens_fill_values(fill):
    ws = W.tiny_spec()
    check_plan_from_tokens(uniform_ids((3, 300), 19, ws["eos"], p_eos=0.2), ws, ws["num_rows"], fill=fill,
                           dense=fill == -1)


def test_plan_from_tokens_outside_the_shard():
    ws = W.tiny_spec()
    bad = check_plan_from_tokens(uniform_ids((5, 300), 23, ws["eos"]), ws, 30_000, row_begin=20_000, dim=8)
    assert bad >= 0


@pytest.mark.parametrize("seq", [1 << 16, (1 << 16) + 3, (1 << 17) + 5, 1 << 18])
def test_plan_from_tokens_every_tile_size(seq):
    """One long row: 2^20, 2^20 + 48, 2^21 + 80 and 2^22 lookups take the three tile
    sizes of the plan's sort, each with its own stretch of positions per tile."""
    ws = W.tiny_spec()
    check_plan_from_tokens(uniform_ids((1, seq), seq % 97, ws["eos"], p_eos=1 / 64), ws, ws["num_rows"], dim=8,
                           seed=seq % 89)


def test_plan_from_tokens_sft_batch():
    ws = W.sft_spec()
    ids, _ = W.sft_batch(seed=2)
    check_plan_from_tokens(ids, ws, ws["num_rows"], dim=8, seed=5)


def test_plan_from_tokens_equals_plan_from_rows_long_context():
    """The long-context stream with the released constants over the full row range:
    the plan from tokens and the plan from engram_hash's rows give the same distinct
    rows and the same sums bit for bit (the rows path is checked against the oracle
    in the full-table tests)."""
    ids, _ = W.long_context_stream(1)
    tokens = torch.from_numpy(ids).cuda()
    spec = E.qwen3_8_flash_next_spec()
    n = ids.size * 16
    dy = grads(n, 31)
    ur_a, ug_a = E.engram_scatter_add(E.engram_hash(tokens, spec), dy, W.FULL_ROWS)
    ur_b = torch.empty(n, dtype=torch.int64, device="cuda")
    nu_b = torch.empty((), dtype=torch.int64, device="cuda")
    ug_b = torch.empty((n, 160), dtype=torch.float32, device="cuda")
    wsb = E.engram_scatter_add_plan_from_tokens(tokens, spec, W.FULL_ROWS, 160, uniq_rows=ur_b, num_uniq=nu_b)
    E.engram_scatter_add_apply(dy, n, W.FULL_ROWS, wsb, uniq_grad=ug_b)
    torch.cuda.synchronize()
    u = int(nu_b.item())
    assert u == ur_a.numel()
    assert torch.equal(ur_b[:u], ur_a)
    assert torch.equal(ug_b[:u].view(torch.int32), ug_a.view(torch.int32))


# ---- The plan from tokens split by head.  When every head's row range lies in the
# shard and the ranges are disjoint and ascending in head order, the sort runs per
# head over the bits of the head's modulus, in fewer passes than num_rows needs.
# The layouts below take it with two 8-bit passes (moduli below 2^16 in a 20-bit
# table), with an 8-bit and a 9-bit pass (moduli below 2^17 in a 21-bit table), with
# gaps between the ranges and a shard that starts before the first one, and not at
# all (ranges in descending head order, or one head outside the shard).  Each must
# equal the oracle, and the plan from engram_hash's rows (never split) bit for bit.

def check_split_plan(ids, ws, num_rows, row_begin=0, dim=8, seed=0, dense=False):
    check_plan_from_tokens(ids, ws, num_rows, row_begin=row_begin, dim=dim, dense=dense, seed=seed)
    spec = product_spec_from(ws)
    tokens = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int64)).cuda()
    n = ids.size * 16
    dy = grads(n, seed + 1, dim)
    ur_a, ug_a = E.engram_scatter_add(E.engram_hash(tokens, spec), dy, num_rows, row_begin)
    ur_b = torch.empty(n, dtype=torch.int64, device="cuda")
    nu_b = torch.empty((), dtype=torch.int64, device="cuda")
    ug_b = torch.empty((n, dim), dtype=torch.float32, device="cuda")
    wsb = E.engram_scatter_add_plan_from_tokens(tokens, spec, num_rows, dim, row_begin, uniq_rows=ur_b,
                                                num_uniq=nu_b)
    E.engram_scatter_add_apply(dy, n, num_rows, wsb, row_begin, uniq_grad=ug_b)
    torch.cuda.synchronize()
    u = int(nu_b.item())
    assert u == ur_a.numel()
    assert torch.equal(ur_b[:u], ur_a)
    assert torch.equal(ug_b[:u].view(torch.int32), ug_a.view(torch.int32))


SPLIT_SHAPES = [(1, 1), (1, 2), (2, 63), (3, 5000), (1, (1 << 16) + 3), (1, (1 << 17) + 5)]


@pytest.mark.parametrize("shape", SPLIT_SHAPES)
def test_split_plan_two_8_bit_passes(shape):
    ws = head_layout(60_000)
    check_split_plan(uniform_ids(shape, sum(shape) + 3, ws["eos"]), ws, ws["num_rows"], seed=sum(shape) % 13)


@pytest.mark.parametrize("shape", SPLIT_SHAPES)
def test_split_plan_8_and_9_bit_passes(shape):
    ws = head_layout(100_000)
    check_split_plan(uniform_ids(shape, sum(shape) + 5, ws["eos"]), ws, ws["num_rows"], seed=sum(shape) % 11)


@pytest.mark.parametrize("fill", [-1, INT64_MAX, INT64_MIN])
def test_split_plan_fill_values_and_eos_runs(fill):
    """Missing context takes the fill value, and EOS runs (one token in three) reset
    the context often: the per-head sort must still see exactly the oracle's rows."""
    ws = dict(head_layout(100_000), fill=fill)
    ids = uniform_ids((5, 777), 59, ws["eos"], p_eos=1 / 3)
    check_plan_from_tokens(ids, ws, ws["num_rows"], fill=fill, dim=8, seed=9)


def test_split_plan_one_pass():
    """Heads below 256 rows in a 12-bit table: the per-head sort is one 8-bit pass."""
    ws = head_layout(100)
    check_split_plan(uniform_ids((3, 2000), 61, ws["eos"]), ws, ws["num_rows"], seed=10)


def test_split_plan_long_segments():
    """400,000 positions: 66 sort tiles per head, past the 64 a first pass can count
    from the tile histograms alone, so the plan clears its counts in a kernel of its
    own and the first pass reads chunk and group totals (8- and 9-bit passes)."""
    ws = head_layout(100_000)
    check_split_plan(uniform_ids((1, 400_000), 67, ws["eos"], p_eos=1 / 500), ws, ws["num_rows"], seed=11)


def test_split_plan_gaps_and_shard_start():
    ws = head_layout(100_000, gap=777, start=12_345)
    ids = uniform_ids((4, 20_000), 41, ws["eos"], p_eos=1 / 32)
    check_split_plan(ids, ws, ws["num_rows"] - 12_000 + 500, row_begin=12_000, seed=3)


def test_split_plan_dense():
    ws = head_layout(60_000)
    check_split_plan(uniform_ids((2, 30_000), 43, ws["eos"]), ws, ws["num_rows"], seed=4, dense=True)


def test_split_plan_released_heads_on_long_rows():
    """The released moduli (25 bits) on the full row range: three passes, the last of 9 bits."""
    ids = uniform_ids((2, 70_000), 47, C.EOS_TOKEN_ID, p_eos=1 / 128, vocab=5000)
    check_split_plan(ids, full_oracle_spec(), C.padded_rows(), seed=6)


@pytest.mark.parametrize("case", ["descending", "head_outside"])
def test_whole_sort_when_not_split(case):
    if case == "descending":
        ws = head_layout(60_000, descending=True)
        num_rows = ws["num_rows"]
    else:
        ws = head_layout(60_000)
        num_rows = ws["num_rows"] - 1  # the last head's last row is outside the shard
    ids = uniform_ids((3, 9_000), 53, ws["eos"])
    bad = check_plan_from_tokens(ids, ws, num_rows, dim=8, seed=7)  # status checked against the oracle's
    if case == "descending":
        assert bad < 0


# ---- The plan from a context-parallel slice (engram_scatter_add_plan_from_tokens_slice):
# columns [a, b) of every batch row, the columns before a read as history.  Plan and
# apply must equal the oracle's scatter-add of columns [a, b) of the oracle's hash of
# the whole rows, for the whole sort and the sort split by head, at cuts inside EOS
# runs and at the row ends.

def check_slice_plan(ids, ws, a, b, num_rows, dim=8, seed=0, dense=False):
    spec = product_spec_from(ws)
    ids = np.ascontiguousarray(ids, dtype=np.int64)
    tokens = torch.from_numpy(ids).cuda()
    n = ids.shape[0] * (b - a) * 16
    rows_ref = oracle_hash(ids, ws)[:, a:b].reshape(-1)
    status = torch.empty((), dtype=torch.int64, device="cuda")
    nu = torch.empty((), dtype=torch.int64, device="cuda")
    ur = torch.full((max(n, 1),), -7, dtype=torch.int64, device="cuda")
    wsp = E.engram_scatter_add_plan_from_tokens_slice(tokens, spec, a, b, num_rows, dim, uniq_rows=ur, num_uniq=nu,
                                                      status=status)
    if n == 0:
        torch.cuda.synchronize()
        assert int(nu.item()) == 0 and int(status.item()) == -1
        return
    dy = grads(n, seed, dim)
    dy_host = to_host(dy)
    if dense:
        g = torch.zeros((num_rows, dim), dtype=torch.float32, device="cuda")
        E.engram_scatter_add_apply(dy, n, num_rows, wsp, grad_dense=g)
        ref, rbad = c_oracle.scatter_add_dense(rows_ref, dy_host, num_rows, 0)
        torch.cuda.synchronize()
        assert int(status.item()) == rbad
        assert_close_to_fp64(g.cpu().numpy(), ref, "dense sums from a token slice")
        return
    ug = torch.empty((n, dim), dtype=torch.float32, device="cuda")
    E.engram_scatter_add_apply(dy, n, num_rows, wsp, uniq_grad=ug)
    torch.cuda.synchronize()
    rur, rug, rbad = c_oracle.scatter_add_compact(rows_ref, dy_host, num_rows, 0)
    u = int(nu.item())
    assert int(status.item()) == rbad
    assert u == rur.size and np.array_equal(ur[:u].cpu().numpy(), rur)
    assert_close_to_fp64(ug[:u].cpu().numpy(), rug, "compact sums from a token slice")


SLICE_CUTS = [(0, 300), (1, 2), (2, 301), (37, 41), (150, 300), (299, 300), (64, 192), (120, 120)]


@pytest.mark.parametrize("layout", ["whole", "split"])
@pytest.mark.parametrize("cut", SLICE_CUTS)
def test_plan_from_token_slice(layout, cut):
    ws = W.tiny_spec() if layout == "whole" else head_layout(100_000)
    ids = uniform_ids((3, 301), 71, ws["eos"], p_eos=1 / 8)
    ids[1, 36:40] = ws["eos"]   # a cut inside an EOS run
    check_slice_plan(ids, ws, cut[0], cut[1], ws["num_rows"], seed=cut[0] % 7)


@pytest.mark.parametrize("layout", ["whole", "split"])
def test_plan_from_token_slice_every_tile_size(layout):
    """One long row cut at 1,000 and 1,000 + 2^16 + 3 or + 2^17 + 5 positions: the
    16- and 24-key tiles, 1 M and 2 M lookups; the dense form once."""
    ws = W.tiny_spec() if layout == "whole" else head_layout(100_000)
    ids = uniform_ids((1, 140_000), 73, ws["eos"], p_eos=1 / 64)
    check_slice_plan(ids, ws, 1000, 1000 + (1 << 16) + 3, ws["num_rows"], seed=2, dense=layout == "split")
    check_slice_plan(ids, ws, 1000, 1000 + (1 << 17) + 5, ws["num_rows"], seed=3)


def test_plan_from_token_slice_released_heads():
    """The released moduli over the full row range (per-head sort, 9-bit last pass):
    an eighth of a context-parallel world's sequence, cut at 3/8 of it."""
    ids = uniform_ids((2, 40_000), 79, C.EOS_TOKEN_ID, p_eos=1 / 256, vocab=5000)
    check_slice_plan(ids, full_oracle_spec(), 15_000, 20_000, C.padded_rows(), seed=4)


def test_plan_from_token_slice_refused():
    ws = W.tiny_spec()
    t = torch.zeros((2, 8), dtype=torch.int64, device="cuda")
    for a, b in [(-1, 3), (4, 3), (0, 9)]:
        with pytest.raises(ValueError):
            E.engram_scatter_add_plan_from_tokens_slice(t, product_spec_from(ws), a, b, ws["num_rows"], 8)


def test_plan_from_tokens_refuses_other_layouts():
    ws = W.tiny_spec()
    two = dict(ws, ngram_size=2, vocab_sizes=ws["vocab_sizes"][:8], offsets=ws["offsets"][:8])
    with pytest.raises(E.EngramError):
        E.engram_scatter_add_plan_from_tokens(torch.zeros((1, 8), dtype=torch.int64, device="cuda"),
                                              product_spec_from(two), ws["num_rows"], 160)


def test_fused_wide_shard_row_ids():
    """The fused kernel's 64-bit row-id path: a shard declared with 2^32 + 5 rows
    from row_begin 100, of which the allocated table holds the tiny layout's rows;
    rows below row_begin fall outside the shard (zero output, status)."""
    ws = W.tiny_spec()
    rb, declared = 100, (1 << 32) + 5
    table = bf16_table(ws["num_rows"], 21)
    ids = uniform_ids((3, 500), 21, ws["eos"])
    spec = product_spec_from(ws)
    tokens = torch.from_numpy(ids).cuda()
    out = torch.empty((3, 500, 16, 160), dtype=torch.bfloat16, device="cuda")
    status = torch.empty((), dtype=torch.int64, device="cuda")
    lib = E.load_library()
    rc = lib.engram_hash_gather(tokens.data_ptr(), 3, 500, ctypes.byref(spec), table.data_ptr(), E.ENGRAM_BF16, rb,
                                declared, 160, out.data_ptr(), None, status.data_ptr(), None)
    assert rc == 0
    torch.cuda.synchronize()
    rows = oracle_hash(ids, ws).reshape(-1)
    assert rows.max() < rb + ws["num_rows"]          # every in-shard row lies in the allocated table
    inside = rows >= rb
    ref, _ = c_oracle.gather(to_host(table), np.where(inside, rows, rb), rb)
    ref[~inside] = 0
    assert np.array_equal(to_host(out).reshape(ref.shape), ref)
    assert int(status.item()) == int(np.argmax(~inside)) and not inside.all()


def test_fused_empty_shard_and_empty_batches():
    """An owner with no rows: every output row is zero and the status names lookup 0
    (the empty table is never read).  Empty token batches write nothing and report
    no bad row."""
    ws = W.tiny_spec()
    spec = product_spec_from(ws)
    ids = torch.from_numpy(uniform_ids((2, 40), 29, ws["eos"])).cuda()
    empty = torch.empty((0, 160), dtype=torch.bfloat16, device="cuda")
    status = torch.empty((), dtype=torch.int64, device="cuda")
    out = E.engram_hash_gather(ids, spec, empty, 5, status=status, validate=False)
    torch.cuda.synchronize()
    assert out.shape == (2, 40, 16, 160) and not out.view(torch.int16).any()
    assert int(status.item()) == 0
    table = bf16_table(ws["num_rows"], 30)
    for shape in ((0, 7), (3, 0)):
        status.fill_(-5)
        out = E.engram_hash_gather(torch.empty(shape, dtype=torch.int64, device="cuda"), spec, table, status=status,
                                   validate=False)
        torch.cuda.synchronize()
        assert out.numel() == 0 and int(status.item()) == -1


def check_slice(ids, ws, table, a, b, row_begin=0, with_rows=True, spec=None):
    """The fused forward of columns [a, b): against the oracle's hash of the whole
    sequence (its columns a..b-1) and the oracle's gather, and against
    engram_hash_slice followed by engram_gather."""
    spec = spec if spec is not None else product_spec_from(ws)
    ids = np.ascontiguousarray(ids, dtype=np.int64)
    batch, seq = ids.shape
    heads = spec.num_heads
    tokens = torch.from_numpy(ids).cuda()
    status = torch.empty((), dtype=torch.int64, device="cuda")
    rows_out = torch.full((batch, b - a, heads), -7, dtype=torch.int64, device="cuda") if with_rows else None
    out = E.engram_hash_gather_slice(tokens, spec, table, a, b, row_begin, rows_out=rows_out, status=status,
                                     validate=False)
    torch.cuda.synchronize()
    ref_rows = np.ascontiguousarray(oracle_hash(ids, ws)[:, a:b])
    ref, bad = c_oracle.gather(to_host(table), ref_rows.reshape(-1), row_begin)
    assert out.shape == (batch, b - a, heads, table.shape[1])
    assert np.array_equal(to_host(out).reshape(ref.shape).view(np.uint8), ref.view(np.uint8))
    assert int(status.item()) == bad
    if with_rows:
        assert np.array_equal(rows_out.cpu().numpy(), ref_rows)
    two = E.engram_gather(table, E.engram_hash_slice(tokens, a, b, spec), row_begin, validate=False)
    assert np.array_equal(to_host(two).view(np.uint8), to_host(out).view(np.uint8))


def test_slice_forward_cuts():
    """Slices of a sequence with EOS runs: cuts at, just after and just before
    EOS positions, at the ends, one column, and the whole row."""
    ws = W.tiny_spec()
    ids = uniform_ids((3, 500), 17, ws["eos"], p_eos=1.0 / 8)
    table = bf16_table(ws["num_rows"], 10)
    eos_at = [int(t) for t in np.nonzero(ids[0] == ws["eos"])[0][:3]]
    cuts = [(0, 500), (0, 1), (499, 500), (1, 2), (2, 3), (250, 251), (100, 357)]
    for t in eos_at:
        cuts += [(t, min(t + 40, 500)), (min(t + 1, 499), min(t + 60, 500)), (max(t - 1, 0), min(t + 7, 500))]
    for k, (a, b) in enumerate(cuts):
        check_slice(ids, ws, table, a, b, with_rows=k % 2 == 0)


def test_slice_forward_released_constants():
    """A context-parallel rank's slice of a long-context stream with the released
    constants on owner 0's shard (most rows outside it: zero rows, status)."""
    ws = full_oracle_spec()
    ids, _ = W.long_context_stream(seed=5, total=20_000)
    check_slice(ids, ws, bf16_table(W.OWNER_ROWS, 11), 7_123, 12_345, spec=E.qwen3_8_flash_next_spec())


def test_slice_forward_empty_and_refused():
    ws = W.tiny_spec()
    ids = uniform_ids((2, 50), 19, ws["eos"])
    tokens = torch.from_numpy(ids).cuda()
    table = bf16_table(ws["num_rows"], 12)
    spec = product_spec_from(ws)
    assert E.engram_hash_gather_slice(tokens, spec, table, 20, 20).shape == (2, 0, 16, 160)
    with pytest.raises(E.EngramError):
        E.engram_hash_gather_slice(tokens, spec, table, 30, 20)      # seq_begin > seq_end
    with pytest.raises(E.EngramError):
        E.engram_hash_gather_slice(tokens, spec, table, 0, 51)       # past the row
    fp32 = bf16_table(ws["num_rows"], 13, torch.float32)             # two-kernel path: rows_out required
    with pytest.raises(E.EngramError):
        E.engram_hash_gather_slice(tokens, spec, fp32, 5, 25)
    rows = torch.empty((2, 20, 16), dtype=torch.int64, device="cuda")
    out = E.engram_hash_gather_slice(tokens, spec, fp32, 5, 25, rows_out=rows)
    assert torch.equal(out, E.engram_gather(fp32, E.engram_hash_slice(tokens, 5, 25, spec)))
