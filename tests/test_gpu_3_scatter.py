"""Gradient scatter-add parity: fp32 results within 1e-5 relative / 1e-6 absolute
of the fp64 oracle; bit-exact where the sums are exact; deterministic."""
import numpy as np
import pytest
import torch

import hashed_gram_embedding_engram_amd as E
import workloads as W
from oracle import c_oracle
from tests.gpu_common import assert_close_to_fp64, oracle_hash, requires_gpu, to_host

pytestmark = [pytest.mark.gpu, requires_gpu]


def run_compact(rows_np, dy_gpu, num_rows, row_begin=0):
    rows = torch.from_numpy(np.ascontiguousarray(rows_np, dtype=np.int64).reshape(-1)).cuda()
    status = torch.empty((), dtype=torch.int64, device="cuda")
    ur, ug, nu = E.engram_scatter_add(rows, dy_gpu, num_rows, row_begin, status=status, validate=False,
                                      compact=(torch.full((max(rows.numel(), 1),), -7, dtype=torch.int64, device="cuda"),
                                               torch.empty((max(rows.numel(), 1), dy_gpu.shape[-1]),
                                                           dtype=torch.float32, device="cuda"),
                                               torch.empty((), dtype=torch.int64, device="cuda")))
    torch.cuda.synchronize()
    u = int(nu.item())
    return ur[:u].cpu().numpy(), ug[:u].cpu().numpy(), int(status.item()), ur.cpu().numpy()


def run_dense(rows_np, dy_gpu, num_rows, row_begin=0, grad_in=None):
    rows = torch.from_numpy(np.ascontiguousarray(rows_np, dtype=np.int64).reshape(-1)).cuda()
    status = torch.empty((), dtype=torch.int64, device="cuda")
    g = torch.zeros((num_rows, dy_gpu.shape[-1]), dtype=torch.float32, device="cuda") if grad_in is None \
        else torch.from_numpy(grad_in).cuda()
    E.engram_scatter_add(rows, dy_gpu, num_rows, row_begin, grad_dense=g, status=status, validate=False)
    torch.cuda.synchronize()
    return g.cpu().numpy(), int(status.item())


def check_compact(rows_np, dy_gpu, num_rows, row_begin=0, exact=False):
    ur, ug, bad, _ = run_compact(rows_np, dy_gpu, num_rows, row_begin)
    rur, rug, rbad = c_oracle.scatter_add_compact(rows_np, to_host(dy_gpu), num_rows, row_begin)
    assert bad == rbad
    assert np.array_equal(ur, rur)
    if exact:
        assert np.array_equal(ug.astype(np.float64), rug)
    else:
        assert_close_to_fp64(ug, rug, "compact sums")
    return ur, ug


def grads(n, dim=160, dtype=torch.bfloat16, seed=0):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn((n, dim), generator=g, device="cuda").to(dtype)


def test_tiny_case():
    """Tiny: fp32 table and grad_out, compact and dense, against the oracle."""
    ws = W.tiny_spec()
    rows = oracle_hash(W.tiny_tokens(), ws).reshape(-1)
    dy = torch.from_numpy(W.tiny_grad(rows.size)).cuda()
    check_compact(rows, dy, ws["num_rows"])
    gin = np.random.default_rng(4).standard_normal((ws["num_rows"], 160)).astype(np.float32)
    got, bad = run_dense(rows, dy, ws["num_rows"], grad_in=gin)
    ref, rbad = c_oracle.scatter_add_dense(rows, W.tiny_grad(rows.size), ws["num_rows"], 0, gin)
    assert bad == rbad == -1
    assert_close_to_fp64(got, ref, "dense tiny")


@pytest.mark.parametrize("n", [1, 2, 255, 256, 257, 4095, 4096, 4097, 3 * 4096 + 17, 70001])
def test_ragged_counts(n):
    rng = np.random.default_rng(n)
    rows = (rng.zipf(1.2, size=n) % 5000).astype(np.int64)
    check_compact(rows, grads(n, seed=n), 5000)


@pytest.mark.parametrize("num_rows", [1, 2, 255, 256, 257, 65536, 65537, 5_000_024, (1 << 31) + 5, 0xFFFFFFFE])
def test_key_widths(num_rows):
    """Sort passes follow the bit length of the shard (1 to 32 bits)."""
    rng = np.random.default_rng(num_rows % 1000)
    n = 20000
    hot = rng.integers(0, num_rows, size=50)
    rows = np.where(rng.random(n) < 0.5, hot[rng.integers(0, 50, size=n)], rng.integers(0, num_rows, size=n))
    check_compact(rows.astype(np.int64), grads(n, seed=7), num_rows)


def test_ones_give_histogram():
    rng = np.random.default_rng(2)
    rows = rng.integers(100, 400, size=300000).astype(np.int64)
    dy = torch.ones((rows.size, 160), dtype=torch.bfloat16, device="cuda")
    ur, ug, _, _ = run_compact(rows, dy, 300, row_begin=100)
    counts = np.bincount(rows - 100, minlength=300)
    assert np.array_equal(ur, np.nonzero(counts)[0] + 100)
    assert np.array_equal(ug, np.repeat(counts[ur - 100][:, None], 160, axis=1).astype(np.float32))


def test_integer_grads_exact():
    """Small-integer gradients: every sum is exact in fp64 and fp32, so bit-exact."""
    rng = np.random.default_rng(3)
    rows = (rng.zipf(1.3, size=200000) % 10000).astype(np.int64)
    dy = torch.from_numpy(rng.integers(-8, 9, size=(rows.size, 160)).astype(np.float32)).cuda().to(torch.bfloat16)
    check_compact(rows, dy, 10000, exact=True)
    got, _ = run_dense(rows, dy, 10000)
    ref, _ = c_oracle.scatter_add_dense(rows, to_host(dy), 10000)
    assert np.array_equal(got.astype(np.float64), ref)


def test_hot_row_stress():
    """One row taking 300,000 hits spans ~1,200 reduce slices: carried partials."""
    rng = np.random.default_rng(4)
    n = 400000
    rows = rng.integers(0, 100000, size=n).astype(np.int64)
    rows[rng.random(n) < 0.75] = 31337
    assert (rows == 31337).sum() >= 100000
    dy = grads(n, seed=4)
    check_compact(rows, dy, 100000)
    got, _ = run_dense(rows, dy, 100000)
    ref, _ = c_oracle.scatter_add_dense(rows, to_host(dy), 100000)
    assert_close_to_fp64(got, ref, "dense hot row")


@pytest.mark.parametrize("dtype,dim", [(torch.float32, 160), (torch.float32, 12), (torch.bfloat16, 64)])
def test_hot_row_other_widths(dtype, dim):
    """A row with 40,000 hits (625 reduce slices: a run summed in chunks) and one
    with 3,000 (under the chunked size) among uniform rows, in both output forms,
    for fp32 gradients and other row widths."""
    rng = np.random.default_rng(dim + 3)
    n = 120000
    rows = rng.integers(0, 50000, size=n).astype(np.int64)
    idx = rng.permutation(n)
    rows[idx[:40000]] = 4242
    rows[idx[40000:43000]] = 17
    dy = grads(n, dim=dim, dtype=dtype, seed=dim)
    check_compact(rows, dy, 50000)
    got, _ = run_dense(rows, dy, 50000)
    ref, _ = c_oracle.scatter_add_dense(rows, to_host(dy), 50000)
    assert_close_to_fp64(got, ref, "dense hot rows, width %d" % dim)


def test_all_same_row_and_sorted_input():
    n = 100000
    dy = grads(n, seed=5)
    check_compact(np.full(n, 7, dtype=np.int64), dy, 10)
    check_compact(np.arange(n, dtype=np.int64) // 3, dy, n)
    check_compact(np.arange(n, dtype=np.int64)[::-1].copy() // 300, dy, n)


def test_deterministic():
    rng = np.random.default_rng(6)
    rows = (rng.zipf(1.1, size=300000) % 200000).astype(np.int64)
    dy = grads(rows.size, seed=6)
    a = run_compact(rows, dy, 200000)
    b = run_compact(rows, dy, 200000)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    da, _ = run_dense(rows, dy, 200000)
    db, _ = run_dense(rows, dy, 200000)
    assert np.array_equal(da.view(np.uint32), db.view(np.uint32))
    # dense from zero and compact agree bit for bit on the touched rows; untouched rows stay zero
    assert np.array_equal(da[a[0]].view(np.uint32), a[1].view(np.uint32))
    mask = np.ones(200000, bool)
    mask[a[0]] = False
    assert not da[mask].any()


def test_out_of_range_dropped():
    rng = np.random.default_rng(8)
    rb, R = 5000, 3000
    rows = rng.integers(rb, rb + R, size=50000).astype(np.int64)
    rows[[40000, 1234, 49999]] = [rb - 1, rb + R, -(1 << 63)]
    dy = grads(rows.size, seed=8)
    ur, ug, bad, full_ur = run_compact(rows, dy, R, rb)
    rur, rug, rbad = c_oracle.scatter_add_compact(rows, to_host(dy), R, rb)
    assert bad == rbad == 1234
    assert np.array_equal(ur, rur)
    assert_close_to_fp64(ug, rug, "compact with bad rows")
    assert (full_ur[ur.size:] == -7).all()          # entries past U untouched
    got, bad = run_dense(rows, dy, R, rb)
    ref, _ = c_oracle.scatter_add_dense(rows, to_host(dy), R, rb)
    assert bad == 1234
    assert_close_to_fp64(got, ref, "dense with bad rows")
    with pytest.raises(E.EngramError, match="outside the owned range"):
        E.engram_scatter_add(torch.from_numpy(rows).cuda(), dy, R, rb)


def test_empty_and_all_invalid():
    dy = grads(3, seed=9)
    ur, ug, bad, _ = run_compact(np.zeros(0, dtype=np.int64), dy[:0], 100)
    assert ur.size == 0 and bad == -1
    ur, ug, bad, _ = run_compact(np.array([100, 101, -1], dtype=np.int64), dy, 100)
    assert ur.size == 0 and bad == 0
    got, bad = run_dense(np.array([100, 101, -1], dtype=np.int64), dy, 100)
    assert bad == 0 and not got.any()
    ur, _, bad, _ = run_compact(np.array([0, 0, 0], dtype=np.int64), dy, 0)   # an empty shard
    assert ur.size == 0 and bad == 0


@pytest.mark.parametrize("dtype,dim", [(torch.bfloat16, 8), (torch.bfloat16, 64), (torch.bfloat16, 512),
                                       (torch.float32, 4), (torch.float32, 12), (torch.float32, 160),
                                       (torch.float32, 256)])
def test_other_widths(dtype, dim):
    rng = np.random.default_rng(dim)
    rows = (rng.zipf(1.2, size=30000) % 2000).astype(np.int64)
    dy = grads(rows.size, dim=dim, dtype=dtype, seed=dim)
    check_compact(rows, dy, 2000)
    got, _ = run_dense(rows, dy, 2000)
    ref, _ = c_oracle.scatter_add_dense(rows, to_host(dy), 2000)
    assert_close_to_fp64(got, ref, "dense width %d" % dim)


def test_sft_shape_backward():
    """SFT-shaped lookups (524,288) into the 10,000,000-row table, bf16 grad_out."""
    ws = W.sft_spec()
    ids, _ = W.sft_batch(0)
    rows = oracle_hash(ids, ws).reshape(-1)
    check_compact(rows, grads(rows.size, seed=10), ws["num_rows"])


def test_plan_apply_reuse():
    """One plan, several gradients: each apply equals a full scatter-add bit for bit,
    in both output forms."""
    rng = np.random.default_rng(12)
    R = 50000
    rows_np = (rng.zipf(1.2, size=150000) % R).astype(np.int64)
    rows = torch.from_numpy(rows_np).cuda()
    n = rows.numel()
    ur = torch.empty(n, dtype=torch.int64, device="cuda")
    nu = torch.empty((), dtype=torch.int64, device="cuda")
    ws = E.engram_scatter_add_plan(rows, R, 160, uniq_rows=ur, num_uniq=nu)
    for seed in (1, 2):
        dy = grads(n, seed=seed)
        ug = torch.empty((n, 160), dtype=torch.float32, device="cuda")
        E.engram_scatter_add_apply(dy, n, R, ws, uniq_grad=ug)
        g = torch.zeros((R, 160), dtype=torch.float32, device="cuda")
        E.engram_scatter_add_apply(dy, n, R, ws, grad_dense=g)
        ref_r, ref_g = E.engram_scatter_add(rows, dy, R)
        u = int(nu.item())
        assert u == ref_r.numel()
        assert torch.equal(ur[:u], ref_r)
        assert torch.equal(ug[:u].view(torch.int32), ref_g.view(torch.int32))
        assert torch.equal(g[ref_r].view(torch.int32), ref_g.view(torch.int32))
        rur, rug, _ = c_oracle.scatter_add_compact(rows_np, to_host(dy), R)
        assert_close_to_fp64(ug[:u].cpu().numpy(), rug, "apply seed %d" % seed)


def test_plan_without_outputs():
    """A plan needs neither uniq_rows nor num_uniq; apply still writes the compact sums."""
    rng = np.random.default_rng(13)
    rows_np = rng.integers(0, 1000, size=20000).astype(np.int64)
    rows = torch.from_numpy(rows_np).cuda()
    ws = E.engram_scatter_add_plan(rows, 1000, 160)
    dy = grads(rows.numel(), seed=13)
    ug = torch.empty((rows.numel(), 160), dtype=torch.float32, device="cuda")
    E.engram_scatter_add_apply(dy, rows.numel(), 1000, ws, uniq_grad=ug)
    rur, rug, _ = c_oracle.scatter_add_compact(rows_np, to_host(dy), 1000)
    assert_close_to_fp64(ug[:rur.size].cpu().numpy(), rug, "apply without plan outputs")


def test_many_long_runs():
    """Dozens of rows with thousands of hits each (several slices per run), shuffled
    among singletons, in both output forms."""
    rng = np.random.default_rng(14)
    hot = rng.choice(200000, size=40, replace=False)
    rows = np.concatenate([np.repeat(hot, rng.integers(2000, 20000, size=40)),
                           rng.integers(0, 200000, size=100000)]).astype(np.int64)
    rng.shuffle(rows)
    dy = grads(rows.size, seed=14)
    check_compact(rows, dy, 200000)
    got, _ = run_dense(rows, dy, 200000)
    ref, _ = c_oracle.scatter_add_dense(rows, to_host(dy), 200000)
    assert_close_to_fp64(got, ref, "dense many long runs")


# ---- Over a million lookups: 256 or more sort tiles, wide key ranges, rows
# repeated hundreds of thousands of times next to uniform ones.  Narrow rows
# (dim 8) keep the oracle's work small; the sort does not depend on the width.
LARGE_N = (1 << 20) + 4097


@pytest.mark.parametrize("num_rows", [1000, 70001, 5_000_024, 320_001_536, 0xFFFFFFFE])
def test_large_key_widths(num_rows):
    rng = np.random.default_rng(num_rows % 977)
    n = LARGE_N
    hot = rng.integers(0, num_rows, size=64)
    rows = np.where(rng.random(n) < 0.3, hot[rng.integers(0, 64, size=n)], rng.integers(0, num_rows, size=n))
    check_compact(rows.astype(np.int64), grads(n, dim=8, seed=21), num_rows)


def test_large_hot_rows():
    """One row repeated 300,000 times, one 25,000 times and 60,000 rows packed
    into one 2^20-row range, among uniform rows; out-of-range rows too."""
    rng = np.random.default_rng(22)
    R = 320_001_536
    n = LARGE_N + 200_000
    rows = rng.integers(0, R, size=n).astype(np.int64)
    idx = rng.permutation(n)
    rows[idx[:300_000]] = 123_456_789
    rows[idx[300_000:325_000]] = 5
    narrow = rng.integers(7 << 20, (7 << 20) + (1 << 20), size=60_000)   # 60,000 rows within 2^20 of each other
    rows[idx[325_000:385_000]] = narrow
    rows[idx[385_000:385_010]] = [-1, R, R + 5, 1 << 40, -(1 << 62), R, R, -3, R + 1, 2 * R]
    first_bad = int(np.sort(idx[385_000:385_010])[0])
    dy = grads(n, dim=8, seed=22)
    ur, ug, bad, _ = run_compact(rows, dy, R)
    rur, rug, rbad = c_oracle.scatter_add_compact(rows, to_host(dy), R, 0)
    assert bad == rbad == first_bad
    assert np.array_equal(ur, rur)
    assert_close_to_fp64(ug, rug, "large n, hot rows")


def test_large_dense_and_deterministic():
    rng = np.random.default_rng(23)
    R = 150_000
    n = LARGE_N
    rows = (rng.zipf(1.1, size=n) % R).astype(np.int64)
    dy = grads(n, dim=160, seed=23)
    a = run_compact(rows, dy, R)
    b = run_compact(rows, dy, R)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    rur, rug, _ = c_oracle.scatter_add_compact(rows, to_host(dy), R, 0)
    assert np.array_equal(a[0], rur)
    assert_close_to_fp64(a[1], rug, "large n, dim 160")
    got, bad = run_dense(rows, dy, R)
    assert bad == -1
    assert np.array_equal(got[a[0]].view(np.uint32), a[1].view(np.uint32))   # the two forms agree bit for bit


def test_sort_beyond_one_shot_counts():
    """6,291,456 + 12,305 lookups (1,027 sort tiles of 6,144 keys): beyond
    1,024 tiles the scatter pass sums its tiles' digit counts in loops
    instead of loading them in one go."""
    rng = np.random.default_rng(25)
    R = 320_001_536
    n = 1024 * 6144 + 2 * 6144 + 17
    hot = rng.integers(0, R, size=32)
    rows = np.where(rng.random(n) < 0.2, hot[rng.integers(0, 32, size=n)], rng.integers(0, R, size=n))
    check_compact(rows.astype(np.int64), grads(n, dim=8, seed=25), R)


def test_large_all_one_row():
    """Every lookup on one row: every sort pass leaves the order as it is."""
    n = LARGE_N
    dy = grads(n, dim=8, seed=24)
    check_compact(np.full(n, 99_999, dtype=np.int64), dy, 320_001_536)


@pytest.mark.parametrize("n", [(1 << 20) - 1, 1 << 20, (1 << 20) + 1, (1 << 21) - 1, 1 << 21, (1 << 21) + 1])
def test_sort_tile_size_boundaries(n):
    """The plan's sort tiles hold 8 keys per thread up to 2^20 lookups, 16
    below 2^21 and 24 from 2^21: both sides of each change, compact and dense,
    with hot rows and a 29-bit key range."""
    rng = np.random.default_rng(n % 1009)
    R = 320_001_536
    hot = rng.integers(0, R, size=48)
    rows = np.where(rng.random(n) < 0.25, hot[rng.integers(0, 48, size=n)], rng.integers(0, R, size=n))
    rows = rows.astype(np.int64)
    dy = grads(n, dim=8, seed=n % 101)
    ur, ug = check_compact(rows, dy, R)
    R2 = 3_000_017
    rows2 = rows % R2
    got, bad = run_dense(rows2, dy, R2)
    ref, rbad = c_oracle.scatter_add_dense(rows2, to_host(dy), R2)
    assert bad == rbad == -1
    assert_close_to_fp64(got, ref, "dense, n = %d" % n)


def padded_case(rng, world, capacity, num_rows, row_begin, dim=160, bad_at=()):
    """Received padded ID and gradient blocks: counts (one negative, one above the
    capacity), garbage in the padding, IDs outside the shard at the given
    (block, entry) places; returns the padded tensors and their compact forms."""
    counts = rng.integers(0, capacity + 1, size=world).astype(np.int64)
    if world > 2:
        counts[1] = -3
        counts[2] = capacity + 7
    ids = rng.integers(-10**9, 10**9, size=(world, capacity)).astype(np.int64)   # padding: never read as IDs
    kept = np.clip(counts, 0, capacity)
    for w in range(world):
        ids[w, :kept[w]] = rng.integers(row_begin, row_begin + num_rows, size=kept[w])
    for w, r in bad_at:
        ids[w, r] = row_begin + num_rows + 5
    dy = grads(world * capacity, dim, seed=world).reshape(world, capacity, dim)
    compact_ids = np.concatenate([ids[w, :kept[w]] for w in range(world)])
    dy_h = to_host(dy)
    compact_dy = np.concatenate([dy_h[w, :kept[w]] for w in range(world)])
    return counts, ids, dy, compact_ids, compact_dy


@pytest.mark.parametrize("world,capacity", [(1, 700), (8, 333), (64, 97), (255, 3), (4, 1)])
def test_plan_padded_dense_and_compact(world, capacity):
    """The plan over received padded blocks, applied to the padded gradient
    blocks, equals the fp64 oracle's scatter-add of the compact IDs and
    gradients (dense and compact outputs); padding is never read as an ID."""
    rng = np.random.default_rng(world)
    num_rows, row_begin = 30_000, 1_000
    counts, ids, dy, cids, cdy = padded_case(rng, world, capacity, num_rows, row_begin)
    c = torch.from_numpy(counts).cuda()
    ids_g = torch.from_numpy(ids).cuda()
    n = world * capacity
    status = torch.empty((), dtype=torch.int64, device="cuda")
    g = torch.zeros((num_rows, 160), dtype=torch.float32, device="cuda")
    ws = E.engram_scatter_add_plan_padded(ids_g, c, num_rows, 160, row_begin, status=status)
    E.engram_scatter_add_apply(dy.reshape(n, 160), n, num_rows, ws, row_begin, grad_dense=g)
    assert int(status.item()) == -1
    ref, rbad = c_oracle.scatter_add_dense(cids, cdy, num_rows, row_begin)
    assert rbad == -1
    assert_close_to_fp64(g.cpu().numpy(), ref, "dense from padded blocks")
    ur = torch.empty(n, dtype=torch.int64, device="cuda")
    ug = torch.empty((n, 160), dtype=torch.float32, device="cuda")
    nu = torch.empty((), dtype=torch.int64, device="cuda")
    ws = E.engram_scatter_add_plan_padded(ids_g, c, num_rows, 160, row_begin, workspace=ws, uniq_rows=ur,
                                          num_uniq=nu)
    E.engram_scatter_add_apply(dy.reshape(n, 160), n, num_rows, ws, row_begin, uniq_grad=ug)
    u = int(nu.item())
    rur, rug, _ = c_oracle.scatter_add_compact(cids, cdy, num_rows, row_begin)
    assert np.array_equal(ur[:u].cpu().numpy(), rur)
    assert_close_to_fp64(ug[:u].cpu().numpy(), rug, "compact from padded blocks")


def test_plan_padded_bad_ids():
    """Received IDs outside the shard: dropped, and the lowest padded index
    reported (an ID in the padding is not one)."""
    rng = np.random.default_rng(77)
    world, capacity, num_rows, row_begin = 8, 120, 5_000, 0
    counts, ids, dy, cids, cdy = padded_case(rng, world, capacity, num_rows, row_begin,
                                             bad_at=[(4, 3), (6, 0)])
    ids[0, capacity - 1] = -1 if counts[0] < capacity else ids[0, capacity - 1]   # padding or real, as it falls
    kept = np.clip(counts, 0, capacity)
    bad_real = [w * capacity + r for w in range(world) for r in range(kept[w])
                if not (row_begin <= ids[w, r] < row_begin + num_rows)]
    status = torch.empty((), dtype=torch.int64, device="cuda")
    n = world * capacity
    g = torch.zeros((num_rows, 160), dtype=torch.float32, device="cuda")
    ws = E.engram_scatter_add_plan_padded(torch.from_numpy(ids).cuda(), torch.from_numpy(counts).cuda(), num_rows,
                                          160, row_begin, status=status)
    E.engram_scatter_add_apply(dy.reshape(n, 160), n, num_rows, ws, row_begin, grad_dense=g)
    assert int(status.item()) == min(bad_real)
    cids = np.concatenate([ids[w, :kept[w]] for w in range(world)])
    ref, _ = c_oracle.scatter_add_dense(cids, cdy, num_rows, row_begin)
    assert_close_to_fp64(g.cpu().numpy(), ref, "dense from padded blocks with bad IDs")
