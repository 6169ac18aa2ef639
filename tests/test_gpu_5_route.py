"""Owner routing on the GPU: bit-exact against the routing oracle, and a loopback
world of virtual ranks whose routed lookup and backward equal the direct ones."""
import numpy as np
import pytest
import torch

import hashed_gram_embedding_engram_amd as E
import workloads as W
from oracle import c_oracle, route_ref as RR
from tests.gpu_common import assert_close_to_fp64, requires_gpu, to_host

pytestmark = [pytest.mark.gpu, requires_gpu]


def ids_for(rng, n, num_embeddings, bad=0.0):
    ids = rng.integers(0, num_embeddings, size=n).astype(np.int64)
    ids[rng.random(n) < bad] = -3
    return ids


# 2^22 IDs are the most whose sort tiles' counts are each loaded in one go;
# 2^22 + 12,305 IDs (1,028 tiles) take the looped sums.
@pytest.mark.parametrize("world,n", [(1, 1000), (8, 1), (8, 4095), (8, 50000), (64, 70001), (255, 100000),
                                     (64, 1 << 22), (64, (1 << 22) + 3 * 4096 + 17)])
def test_route_plan_parity(world, n):
    rng = np.random.default_rng(world * 7 + n)
    num_embeddings = world * 12345
    ids = ids_for(rng, n, num_embeddings, bad=0.002)
    ids[n // 2] = num_embeddings      # one past the end
    status = torch.empty((), dtype=torch.int64, device="cuda")
    s, o, c = E.engram_route_plan(torch.from_numpy(ids).cuda(), num_embeddings, world, status=status)
    rs, ro, rc, rbad = RR.route_plan(ids, num_embeddings, world)
    assert np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(o.cpu().numpy(), ro)
    assert np.array_equal(c.cpu().numpy(), rc)
    assert int(status.item()) == rbad
    assert int(E.engram_route_validate(s, c, num_embeddings, world).item()) == -1


def test_route_plan_empty():
    s, o, c = E.engram_route_plan(torch.empty(0, dtype=torch.int64, device="cuda"), 800, 8)
    assert s.numel() == 0 and c.cpu().tolist() == [0] * 8


def test_validate_detects_misrouted_and_bad_counts():
    rng = np.random.default_rng(5)
    ids = ids_for(rng, 20000, 8 * 1000)
    s, o, c = E.engram_route_plan(torch.from_numpy(ids).cuda(), 8000, 8)
    cc = c.cpu().numpy()
    bad = s.clone()
    j = int(cc[:3].sum()) + 7
    bad[j] = 0
    assert int(E.engram_route_validate(bad, c, 8000, 8).item()) == j == RR.validate(bad.cpu().numpy(), cc, 8000, 8)
    c2 = c.clone()
    c2[4] = -1
    assert int(E.engram_route_validate(s, c2, 8000, 8).item()) == 20000
    c3 = c.clone()
    c3[0] += 1
    assert int(E.engram_route_validate(s, c3, 8000, 8).item()) == 20000


@pytest.mark.parametrize("dtype,row,fill", [(torch.int64, (), -1), (torch.bfloat16, (160,), 0.0),
                                            (torch.float32, (3,), 2.5), (torch.int16, (2, 4), 7)])
def test_pack_unpack_parity(dtype, row, fill):
    rng = np.random.default_rng(len(row))
    world, capacity = 9, 300
    counts = rng.integers(0, capacity + 1, size=world).astype(np.int64)
    counts[3] = 0
    m = int(counts.sum())
    src = torch.from_numpy(rng.standard_normal((m,) + row) * 100).to(dtype).cuda()
    c = torch.from_numpy(counts).cuda()
    status = torch.empty((), dtype=torch.int64, device="cuda")
    packed = E.engram_pack_fixed_capacity(src, c, world, capacity, fill=fill, status=status)
    src_h = src.cpu()
    ref, rbad = RR.pack(src_h.numpy() if dtype != torch.bfloat16 else src_h.view(torch.int16).numpy(), counts,
                        world, capacity,
                        fill if dtype != torch.bfloat16 else int(torch.tensor([fill], dtype=dtype).view(torch.int16)))
    got = packed.cpu()
    got = got.view(torch.int16).numpy() if dtype == torch.bfloat16 else got.numpy()
    assert np.array_equal(got, ref) and int(status.item()) == rbad == -1
    back = E.engram_unpack_fixed_capacity(packed, c, m, status=status)
    assert torch.equal(back.cpu().view(torch.int16) if dtype == torch.bfloat16 else back.cpu(),
                       src_h.view(torch.int16) if dtype == torch.bfloat16 else src_h)
    assert int(status.item()) == -1


def test_pack_capacity_overflow_reported():
    counts = torch.tensor([2, 7, 1], dtype=torch.int64, device="cuda")
    src = torch.arange(10, dtype=torch.int64, device="cuda")
    status = torch.empty((), dtype=torch.int64, device="cuda")
    packed = E.engram_pack_fixed_capacity(src, counts, 3, 5, fill=-1, status=status)
    assert int(status.item()) == 1
    assert packed.cpu().tolist() == [[0, 1, -1, -1, -1], [2, 3, 4, 5, 6], [9, -1, -1, -1, -1]]
    out = E.engram_unpack_fixed_capacity(packed, torch.tensor([2, 3, 1], device="cuda"), 5, status=status)
    assert int(status.item()) == 3          # 6 compact rows do not fit 5
    assert out.cpu().tolist() == [0, 1, 2, 3, 4]


def test_pack_unpack_bad_counts_match_oracle():
    """A negative count and a count above capacity: both are reported (lowest
    rank), and the rows written equal the oracle's."""
    rng = np.random.default_rng(11)
    world, capacity = 6, 40
    counts = np.array([12, -3, 55, 0, 40, 7], dtype=np.int64)
    m = int(np.maximum(counts, 0).sum())
    src = torch.from_numpy(rng.integers(-1000, 1000, size=(m, 3)).astype(np.int64)).cuda()
    c = torch.from_numpy(counts).cuda()
    status = torch.empty((), dtype=torch.int64, device="cuda")
    packed = E.engram_pack_fixed_capacity(src, c, world, capacity, fill=-9, status=status)
    ref, rbad = RR.pack(src.cpu().numpy(), counts, world, capacity, -9)
    assert np.array_equal(packed.cpu().numpy(), ref) and int(status.item()) == rbad == 1
    kept = int(np.clip(counts, 0, capacity).sum())
    back = E.engram_unpack_fixed_capacity(packed, c, kept, status=status)
    ref_back, ubad = RR.unpack(ref, counts, kept)
    assert int(status.item()) == ubad == 1
    assert np.array_equal(back.cpu().numpy(), ref_back)
    short = E.engram_unpack_fixed_capacity(packed, c, kept - 5, status=status)
    ref_short, ubad = RR.unpack(ref, counts, kept - 5)
    assert int(status.item()) == ubad == 1          # rank errors come before the overflow (world)
    assert np.array_equal(short.cpu().numpy(), ref_short)


@pytest.mark.parametrize("dtype,row", [(torch.int64, ()), (torch.bfloat16, (160,)), (torch.int32, (3,))])
def test_pack_never_reads_past_the_source(dtype, row):
    """Counts that reach past the source rows: those block rows take the fill
    and the status reports rank `world` (or a lower bad rank), as in the oracle;
    the source tensor is exactly src_rows long, so any read past it would be
    out of bounds."""
    rng = np.random.default_rng(17)
    world, capacity = 5, 30
    # (counts, source rows, expected status): world = 5 when only the source runs out
    for counts, src_rows, want in (([10, 25, 3, 0, 12], 33, 5), ([10, 45, 3, 0, 12], 50, 1), ([8, 8, 8, 8, 8], 0, 5),
                                   ([4, -2, 30, 6, 1], 20, 1)):
        counts = np.array(counts, dtype=np.int64)
        host = rng.integers(-1000, 1000, size=(src_rows,) + row).astype(np.int64)
        src = torch.from_numpy(host).to(dtype).cuda()
        status = torch.empty((), dtype=torch.int64, device="cuda")
        packed = E.engram_pack_fixed_capacity(src, torch.from_numpy(counts).cuda(), world, capacity, fill=-7,
                                              status=status)
        ref, rbad = RR.pack(src.cpu().numpy() if dtype != torch.bfloat16 else src.cpu().view(torch.int16).numpy(),
                            counts, world, capacity,
                            -7 if dtype != torch.bfloat16 else int(torch.tensor([-7], dtype=dtype).view(torch.int16)),
                            src_rows=src_rows)
        got = packed.cpu()
        got = got.view(torch.int16).numpy() if dtype == torch.bfloat16 else got.numpy()
        assert np.array_equal(got, ref), counts
        assert int(status.item()) == rbad == want, counts


def test_pack_zero_capacity_reports_counts():
    status = torch.empty((), dtype=torch.int64, device="cuda")
    src = torch.arange(4, dtype=torch.int64, device="cuda")
    out = E.engram_pack_fixed_capacity(src, torch.tensor([0, 3, 1], device="cuda"), 3, 0, fill=0, status=status)
    assert out.shape == (3, 0) and int(status.item()) == 1


def test_permute_unpermute():
    rng = np.random.default_rng(6)
    x = torch.from_numpy(rng.standard_normal((777, 5)).astype(np.float32)).cuda()
    order = torch.from_numpy(rng.permutation(777)).cuda()
    p = E.engram_permute_rows(x, order)
    assert torch.equal(p, x[order])
    assert torch.equal(E.engram_unpermute_rows(p, order), x)
    y = torch.from_numpy(rng.standard_normal((100, 160))).to(torch.bfloat16).cuda()
    o2 = torch.from_numpy(rng.permutation(100)).cuda()
    assert torch.equal(E.engram_unpermute_rows(E.engram_permute_rows(y, o2), o2), y)


def loopback(blocks):
    """The exchange of a world of virtual ranks (transport, not part of the library):
    rank d receives block d of every rank's [world, capacity, ...] send buffer."""
    world = len(blocks)
    return [torch.stack([blocks[s][d] for s in range(world)]) for d in range(world)]


def test_loopback_world_forward_and_backward():
    """Eight owners of the SFT-shaped 10,000,000-row table, eight request ranks with
    their own token batches.  Routed forward and backward equal the direct ones."""
    world = 8
    ws = W.sft_spec()
    R = ws["num_rows"]
    local = R // world
    spec = E.make_hash_spec(3, 8, ws["eos"], E.QWEN3_8_FLASH_NEXT_LAYER_MULTIPLIERS, ws["vocab_sizes"], ws["offsets"])
    table = torch.empty((R, 160), dtype=torch.bfloat16, device="cuda")
    W.fill_normal_(table, seed=21)
    rows = [E.engram_hash(torch.from_numpy(W.sft_batch(seed=r)[0]).cuda(), spec).reshape(-1) for r in range(world)]
    plans = [E.engram_route_plan(r, R, world) for r in rows]
    capacity = int(torch.stack([c for _, _, c in plans]).max().item())      # the agreed capacity (a collective)
    for s, _, c in plans:
        assert int(E.engram_route_validate(s, c, R, world).item()) == -1
    recv = loopback([E.engram_pack_fixed_capacity(s, c, world, capacity, fill=-1) for s, _, c in plans])
    recv_counts = [torch.stack([plans[s][2][d] for s in range(world)]) for d in range(world)]
    owner_ids, owner_vals = [], []
    for d in range(world):
        got = E.engram_unpack_fixed_capacity(recv[d], recv_counts[d], int(recv_counts[d].sum().item()))
        shard = table[d * local:(d + 1) * local]
        owner_ids.append(got)
        owner_vals.append(E.engram_gather(shard, got, row_begin=d * local))      # raises on a misrouted ID
    back = loopback([E.engram_pack_fixed_capacity(v, recv_counts[d], world, capacity, fill=0.0)
                     for d, v in enumerate(owner_vals)])
    dys = []
    for r in range(world):
        s, order, c = plans[r]
        vals = E.engram_unpack_fixed_capacity(back[r], c, int(c.sum().item()))
        out = E.engram_unpermute_rows(vals, order)
        assert torch.equal(out.view(torch.int16), E.engram_gather(table, rows[r]).view(torch.int16))
        g = torch.Generator(device="cuda")
        g.manual_seed(100 + r)
        dys.append(torch.randn((rows[r].numel(), 160), generator=g, device="cuda").to(torch.bfloat16))
    # backward: gradients take the reverse route and each owner scatter-adds into its shard
    grads_sorted = [E.engram_permute_rows(dys[r], plans[r][1]) for r in range(world)]
    recv_g = loopback([E.engram_pack_fixed_capacity(gs, plans[r][2], world, capacity, fill=0.0)
                       for r, gs in enumerate(grads_sorted)])
    all_rows = torch.cat(rows)
    all_dy = torch.cat(dys)
    rur, rug, _ = c_oracle.scatter_add_compact(all_rows.cpu().numpy(), to_host(all_dy), R)
    for d in range(world):
        gd = E.engram_unpack_fixed_capacity(recv_g[d], recv_counts[d], int(recv_counts[d].sum().item()))
        shard_grad = torch.zeros((local, 160), dtype=torch.float32, device="cuda")
        E.engram_scatter_add(owner_ids[d], gd, local, row_begin=d * local, grad_dense=shard_grad)
        mine = (rur >= d * local) & (rur < (d + 1) * local)
        got = shard_grad[torch.from_numpy(rur[mine] - d * local).cuda()].cpu().numpy()
        assert_close_to_fp64(got, rug[mine], "owner %d gradient" % d)


def test_route_bench_shape():
    """The benchmarked exchange half: one request rank of world 64 (8 x 4,096
    Zipf tokens hashed into 524,288 full-table IDs), capacity the largest
    count, 320-byte bf16 value rows; the same calls the benchmark times, the
    backward's one-pass send included."""
    world = 64
    ids = W.owner_token_batches(seeds=[100])[0]
    gids = E.engram_hash(torch.from_numpy(ids).cuda(), E.qwen3_8_flash_next_spec()).reshape(-1).contiguous()
    n = gids.numel()
    s, order, c = E.engram_route_plan(gids, W.FULL_ROWS, world)
    ids_h = gids.cpu().numpy()
    rs, ro, rc, rbad = RR.route_plan(ids_h, W.FULL_ROWS, world)
    assert rbad == -1
    assert np.array_equal(s.cpu().numpy(), rs) and np.array_equal(order.cpu().numpy(), ro)
    assert np.array_equal(c.cpu().numpy(), rc)
    assert int(E.engram_route_validate(s, c, W.FULL_ROWS, world).item()) == -1
    cap = int(rc.max())
    status = torch.empty((), dtype=torch.int64, device="cuda")
    packed_ids = E.engram_pack_fixed_capacity(s, c, world, cap, fill=-1, status=status)
    ref_ids, _ = RR.pack(rs, rc, world, cap, -1)
    assert np.array_equal(packed_ids.cpu().numpy(), ref_ids) and int(status.item()) == -1
    assert torch.equal(E.engram_unpack_fixed_capacity(packed_ids, c, n, status=status), s)
    g = torch.Generator(device="cuda")
    g.manual_seed(3000)
    vals = torch.randn((n, 160), generator=g, device="cuda").to(torch.bfloat16)
    packed = E.engram_pack_fixed_capacity(vals, c, world, cap, fill=0.0, status=status)
    vals_h = vals.cpu().view(torch.int16).numpy()
    ref_packed, _ = RR.pack(vals_h, rc, world, cap, 0)
    assert np.array_equal(packed.cpu().view(torch.int16).numpy(), ref_packed)
    back = E.engram_unpack_fixed_capacity(packed, c, n, status=status)
    assert np.array_equal(back.cpu().view(torch.int16).numpy(), RR.unpack(ref_packed, rc, n)[0])
    out = E.engram_unpermute_rows(back, order)
    ref_out = np.empty_like(vals_h)
    ref_out[ro] = vals_h
    assert np.array_equal(out.cpu().view(torch.int16).numpy(), ref_out)
    fused = E.engram_unpack_unpermute_rows(packed, c, order, status=status)   # the two calls in one pass
    assert int(status.item()) == -1
    assert np.array_equal(fused.cpu().view(torch.int16).numpy(), ref_out)
    # the backward's send: gradient rows in request order, grouped and packed in one pass
    dy = torch.randn((n, 160), generator=g, device="cuda").to(torch.bfloat16)
    send = E.engram_permute_pack_rows(dy, order, c, world, cap, fill=0.0, status=status)
    assert int(status.item()) == -1
    ref_send, _ = RR.pack(dy.cpu().view(torch.int16).numpy()[ro], rc, world, cap, 0)
    assert np.array_equal(send.cpu().view(torch.int16).numpy(), ref_send)


def unpack_unpermute_ref(packed, counts, order, before):
    """The oracle's unpack into n rows, then each compact row k that exists moved
    to row order[k] of `before` (rows without a compact row keep their values)."""
    n = order.size
    compact, bad = RR.unpack(packed, counts, n)
    world, capacity = packed.shape[:2]
    total = int(sum(max(0, min(int(c), capacity)) for c in counts))
    out = before.copy()
    for k in range(min(total, n)):
        if 0 <= order[k] < n:
            out[order[k]] = compact[k]
    return out, bad


@pytest.mark.parametrize("dtype,row,world", [(torch.int64, (), 8), (torch.bfloat16, (160,), 64),
                                             (torch.int32, (3,), 5), (torch.bfloat16, (160,), 1),
                                             (torch.int16, (2, 4), 255)])
def test_unpack_unpermute_parity(dtype, row, world):
    """The fused return path equals the oracle's unpack followed by the move to
    request order, and the two library calls it replaces, bit for bit (16-byte
    and 4-byte row units, one to 255 ranks)."""
    rng = np.random.default_rng(world)
    capacity = 97
    counts = rng.integers(1, capacity + 1, size=world).astype(np.int64)
    if world > 1:
        counts[world // 2] = 0
    n = int(counts.sum())
    packed = torch.from_numpy(rng.standard_normal((world, capacity) + row) * 100).to(dtype).cuda()
    order = torch.from_numpy(rng.permutation(n).astype(np.int64)).cuda()
    c = torch.from_numpy(counts).cuda()
    status = torch.empty((), dtype=torch.int64, device="cuda")
    fused = E.engram_unpack_unpermute_rows(packed, c, order, status=status)
    assert int(status.item()) == -1
    two = E.engram_unpermute_rows(E.engram_unpack_fixed_capacity(packed, c, n), order)
    view = (lambda t: t.cpu().view(torch.int16).numpy()) if dtype == torch.bfloat16 else (lambda t: t.cpu().numpy())
    assert np.array_equal(view(fused), view(two))
    ref, bad = unpack_unpermute_ref(view(packed), counts, order.cpu().numpy(), view(fused))
    assert bad == -1 and np.array_equal(view(fused), ref)


def test_unpack_unpermute_bad_counts_and_orders():
    """Counts that are negative, above the capacity, or sum past n, and order
    entries outside [0, n): the status is the unpack's, compact rows at or past
    n are dropped, bad order entries are skipped, and rows without a compact
    row keep what they held."""
    rng = np.random.default_rng(21)
    world, capacity = 6, 40
    packed_h = rng.integers(-1000, 1000, size=(world, capacity, 3)).astype(np.int64)
    packed = torch.from_numpy(packed_h).cuda()
    status = torch.empty((), dtype=torch.int64, device="cuda")
    cases = [(np.array([12, -3, 55, 0, 40, 7]), 90),     # negative (rank 1) and above capacity (rank 2)
             (np.array([12, 3, 30, 0, 40, 7]), 80),      # 92 compact rows for 80: dropped past n, status world
             (np.array([12, 3, 30, 0, 20, 7]), 90)]      # 72 compact rows for 90: 18 rows keep their values
    for counts, n in cases:
        order_h = rng.permutation(n).astype(np.int64)
        order_h[rng.random(n) < 0.05] = n + 3             # skipped
        order_h[0] = -1
        before = np.full((n, 3), -77, dtype=np.int64)
        out = torch.from_numpy(before).cuda()
        E.engram_unpack_unpermute_rows(packed, torch.from_numpy(counts).cuda(), torch.from_numpy(order_h).cuda(),
                                       status=status, out=out)
        ref, bad = unpack_unpermute_ref(packed_h, counts, order_h, before)
        assert int(status.item()) == bad
        assert np.array_equal(out.cpu().numpy(), ref)


def test_unpack_unpermute_empty():
    """No rows at all (zero capacity, or counts all zero), and the two calls it
    replaces on empty inputs."""
    status = torch.empty((), dtype=torch.int64, device="cuda")
    none = torch.zeros(0, dtype=torch.int64, device="cuda")
    zeros = torch.zeros(4, dtype=torch.int64, device="cuda")
    for cap in (0, 5):
        packed = torch.zeros((4, cap, 160), dtype=torch.bfloat16, device="cuda")
        out = E.engram_unpack_unpermute_rows(packed, zeros, none, status=status)
        assert out.shape == (0, 160) and int(status.item()) == -1
        assert E.engram_unpermute_rows(E.engram_unpack_fixed_capacity(packed, zeros, 0), none).shape == (0, 160)


def permute_pack_ref(src, order, counts, world, capacity, fill):
    """The move into grouped order (grouped row k = src[order[k]], order entries
    outside [0, n) leaving the fill), then the oracle's pack of the n grouped rows."""
    n = order.size
    grouped = np.empty((n,) + src.shape[1:], dtype=src.dtype)
    grouped[...] = fill
    ok = (order >= 0) & (order < n)
    grouped[ok] = src[order[ok]]
    return RR.pack(grouped, counts, world, capacity, fill)


@pytest.mark.parametrize("dtype,row,world", [(torch.int64, (), 8), (torch.bfloat16, (160,), 64),
                                             (torch.int32, (3,), 5), (torch.float32, (160,), 1),
                                             (torch.int16, (2, 4), 255)])
def test_permute_pack_parity(dtype, row, world):
    """The backward's send in one pass equals the move into grouped order and the
    pack (the oracle's, and the two library calls), bit for bit."""
    rng = np.random.default_rng(100 + world)
    capacity = 97
    counts = rng.integers(1, capacity + 1, size=world).astype(np.int64)
    if world > 1:
        counts[world // 2] = 0
    n = int(counts.sum())
    src = torch.from_numpy(rng.standard_normal((n,) + row) * 100).to(dtype).cuda()
    order = torch.from_numpy(rng.permutation(n).astype(np.int64)).cuda()
    c = torch.from_numpy(counts).cuda()
    status = torch.empty((), dtype=torch.int64, device="cuda")
    fill = 7 if dtype != torch.float32 else -2.5
    fused = E.engram_permute_pack_rows(src, order, c, world, capacity, fill=fill, status=status)
    assert int(status.item()) == -1
    two = E.engram_pack_fixed_capacity(E.engram_permute_rows(src, order), c, world, capacity, fill=fill)
    view = (lambda t: t.cpu().view(torch.int16).numpy()) if dtype == torch.bfloat16 else (lambda t: t.cpu().numpy())
    assert np.array_equal(view(fused), view(two))
    fill_ref = fill if dtype != torch.bfloat16 else int(torch.tensor([fill], dtype=dtype).view(torch.int16))
    ref, bad = permute_pack_ref(view(src), order.cpu().numpy(), counts, world, capacity, fill_ref)
    assert bad == -1 and np.array_equal(view(fused), ref)


def test_permute_pack_bad_counts_and_orders():
    """Counts that are negative, above the capacity or past n, and order entries
    outside [0, n): the status is the pack's, and those block rows take the fill."""
    rng = np.random.default_rng(31)
    world, capacity = 6, 40
    status = torch.empty((), dtype=torch.int64, device="cuda")
    for counts, n in [(np.array([12, -3, 55, 0, 40, 7]), 90), (np.array([12, 3, 30, 0, 40, 7]), 80),
                      (np.array([12, 3, 30, 0, 20, 7]), 90)]:
        src_h = rng.integers(-1000, 1000, size=(n, 3)).astype(np.int64)
        order_h = rng.permutation(n).astype(np.int64)
        order_h[rng.random(n) < 0.05] = n + 3
        order_h[0] = -1
        got = E.engram_permute_pack_rows(torch.from_numpy(src_h).cuda(), torch.from_numpy(order_h).cuda(),
                                         torch.from_numpy(counts).cuda(), world, capacity, fill=-9, status=status)
        ref, bad = permute_pack_ref(src_h, order_h, counts, world, capacity, -9)
        assert int(status.item()) == bad
        assert np.array_equal(got.cpu().numpy(), ref)


def test_permute_pack_round_trip():
    """The backward's send and the owner's unpack, then the forward's return path
    packed by the owner: every row comes back to its request position."""
    rng = np.random.default_rng(41)
    world = 16
    ids = torch.from_numpy(rng.integers(0, 16_000, size=20_000).astype(np.int64)).cuda()
    s, order, c = E.engram_route_plan(ids, 16_000, world)
    cap = int(c.max().item())
    g = torch.from_numpy(rng.standard_normal((20_000, 160)).astype(np.float32)).cuda()
    sent = E.engram_permute_pack_rows(g, order, c, world, cap)
    grouped = E.engram_unpack_fixed_capacity(sent, c, 20_000)
    assert torch.equal(grouped, g[order])
    back = E.engram_unpack_unpermute_rows(E.engram_pack_fixed_capacity(grouped, c, world, cap), c, order)
    assert torch.equal(back, g)


@pytest.mark.parametrize("dtype,dim,world,row_begin,capacity", [(torch.bfloat16, 160, 64, 0, 300),
                                                                (torch.float32, 160, 8, 5000, 300),
                                                                (torch.bfloat16, 64, 5, 123, 300),
                                                                (torch.float32, 8, 1, 0, 300),
                                                                (torch.bfloat16, 160, 255, 7, 1),
                                                                (torch.bfloat16, 160, 3, 0, 17)])
def test_gather_padded_parity(dtype, dim, world, row_begin, capacity):
    """The owner's lookup on padded ID blocks equals the unpack of the IDs, the
    oracle's gather and the pack of the values with a zero fill, bit for bit
    (the 16-row and 8-row wave kernels and the generic one)."""
    rng = np.random.default_rng(world + dim + capacity)
    num_rows = 20_000
    table = torch.from_numpy(rng.standard_normal((num_rows, dim)).astype(np.float32)).to(dtype).cuda()
    counts = rng.integers(1, capacity + 1, size=world).astype(np.int64)
    if world > 1:
        counts[world // 2] = 0
    n = int(counts.sum())
    compact = rng.integers(row_begin, row_begin + num_rows, size=n).astype(np.int64)
    ids_packed, _ = RR.pack(compact, counts, world, capacity, -1)
    ids = torch.from_numpy(ids_packed).cuda()
    c = torch.from_numpy(counts).cuda()
    got = E.engram_gather_padded(table, ids, c, row_begin=row_begin)
    view = (lambda t: t.cpu().view(torch.int16).numpy()) if dtype == torch.bfloat16 else (lambda t: t.cpu().numpy())
    three = E.engram_pack_fixed_capacity(E.engram_gather(table, E.engram_unpack_fixed_capacity(ids, c, n),
                                                         row_begin=row_begin), c, world, capacity, fill=0)
    assert np.array_equal(view(got), view(three))
    vals, gbad = c_oracle.gather(to_host(table), compact, row_begin)
    ref, bad = RR.pack(vals, counts, world, capacity, 0)
    assert gbad == -1 and bad == -1 and np.array_equal(to_host(got), ref)


def test_gather_padded_bad_ids_and_counts():
    """IDs outside the shard give zero rows and the lowest padded index; a
    negative count has no IDs, a count above the capacity fills its block;
    padding entries are never checked."""
    rng = np.random.default_rng(5)
    world, capacity, num_rows, row_begin = 4, 50, 1000, 300
    table = torch.from_numpy(rng.standard_normal((num_rows, 160)).astype(np.float32)).cuda()
    ids_h = rng.integers(row_begin, row_begin + num_rows, size=(world, capacity)).astype(np.int64)
    counts = np.array([10, -2, 70, 25], dtype=np.int64)
    ids_h[0, 40] = 5                      # padding of block 0: never checked
    ids_h[2, 33] = row_begin + num_rows   # outside the shard
    ids_h[3, 7] = -1                      # outside the shard, later block
    status = torch.empty((), dtype=torch.int64, device="cuda")
    got = E.engram_gather_padded(table, torch.from_numpy(ids_h).cuda(), torch.from_numpy(counts).cuda(),
                                 row_begin=row_begin, status=status, validate=False).cpu().numpy()
    assert int(status.item()) == 2 * capacity + 33
    tab = table.cpu().numpy()
    for w in range(world):
        real = max(0, min(int(counts[w]), capacity))
        for r in range(capacity):
            i = ids_h[w, r] - row_begin
            want = tab[i] if r < real and 0 <= i < num_rows else np.zeros(160, np.float32)
            assert np.array_equal(got[w, r], want), (w, r)
    with pytest.raises(E.EngramError):
        E.engram_gather_padded(table, torch.from_numpy(ids_h).cuda(), torch.from_numpy(counts).cuda(),
                               row_begin=row_begin)
