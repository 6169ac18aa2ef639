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
    assert int(status.item()) == 1
    assert np.array_equal(back.cpu().numpy(), RR.unpack(ref, counts, kept))
    short = E.engram_unpack_fixed_capacity(packed, c, kept - 5, status=status)
    assert int(status.item()) == 1          # rank errors come before the overflow (world)
    assert np.array_equal(short.cpu().numpy(), RR.unpack(ref, counts, kept - 5))


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
    count, 320-byte bf16 value rows; the same calls the benchmark times."""
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
    assert np.array_equal(back.cpu().view(torch.int16).numpy(), RR.unpack(ref_packed, rc, n))
    out = E.engram_unpermute_rows(back, order)
    ref_out = np.empty_like(vals_h)
    ref_out[ro] = vals_h
    assert np.array_equal(out.cpu().view(torch.int16).numpy(), ref_out)
