"""Pins of the routing oracle — no GPU.

Grouping is pinned to numpy's stable argsort by owner (textbook routine);
pack/unpack to being inverse; and the whole routed lookup of a loopback world
of virtual ranks to the direct lookup it replaces."""
import numpy as np
import pytest

from oracle import route_ref as RR


def random_ids(rng, n, num_embeddings, bad=0.0):
    ids = rng.integers(0, num_embeddings, size=n).astype(np.int64)
    ids[rng.random(n) < bad] = num_embeddings + 5
    return ids


@pytest.mark.parametrize("world", [1, 3, 8, 64])
def test_plan_is_stable_grouping(world):
    rng = np.random.default_rng(world)
    E = world * 1000
    ids = random_ids(rng, 5000, E, bad=0.01)
    sorted_ids, order, counts, bad = RR.route_plan(ids, E, world)
    key = np.where((ids >= 0) & (ids < E), ids // (E // world), world)
    assert np.array_equal(order, np.argsort(key, kind="stable"))
    assert np.array_equal(sorted_ids, ids[order])
    assert np.array_equal(counts, np.bincount(key, minlength=world + 1)[:world])
    assert bad == int(np.nonzero(key == world)[0][0])
    assert RR.validate(sorted_ids, counts, E, world) == -1


def test_validate_finds_misrouted():
    rng = np.random.default_rng(1)
    ids = random_ids(rng, 1000, 8000)
    s, o, c, _ = RR.route_plan(ids, 8000, 8)
    s2 = s.copy()
    s2[int(c[0]) + 3] = 0          # an owner-0 ID in owner 1's segment
    assert RR.validate(s2, c, 8000, 8) == int(c[0]) + 3
    s3 = s.copy()
    s3[5] = 1000                   # owner 1's first row at the end of owner 0's range
    assert RR.validate(s3, c, 8000, 8) == 5
    s3[5] = 999                    # owner 0's last row is fine
    assert RR.validate(s3, c, 8000, 8) == -1
    assert RR.validate(s, c + np.eye(8, dtype=np.int64)[2] * 5000, 8000, 8) == 1000


def test_pack_unpack_inverse():
    rng = np.random.default_rng(2)
    counts = np.array([3, 0, 5, 1], dtype=np.int64)
    rows = rng.standard_normal((9, 6)).astype(np.float32)
    packed, bad = RR.pack(rows, counts, 4, 5, -7.0)
    assert bad == -1 and packed.shape == (4, 5, 6)
    assert (packed[1] == -7.0).all() and (packed[0, 3:] == -7.0).all()
    back, ubad = RR.unpack(packed, counts, 9)
    assert ubad == -1 and np.array_equal(back, rows)
    _, bad = RR.pack(rows, np.array([3, 0, 6, 0]), 4, 5, 0.0)
    assert bad == 2


def test_loopback_world_equals_direct_lookup():
    """Route -> pack -> exchange -> unpack -> owner lookup -> pack -> exchange ->
    unpack -> back to request order gives every rank the rows a direct lookup of
    the whole table gives."""
    rng = np.random.default_rng(3)
    world, E, dim = 6, 6 * 500, 4
    table = rng.standard_normal((E, dim))
    requests = [random_ids(rng, int(rng.integers(50, 400)), E) for _ in range(world)]
    plans = [RR.route_plan(ids, E, world) for ids in requests]
    capacity = max(int(c) for _, _, counts, _ in plans for c in counts)
    sent = RR.all_to_all([RR.pack(s, counts, world, capacity, -1)[0] for s, _, counts, _ in plans])
    recv_counts = [np.array([plans[src][2][dst] for src in range(world)]) for dst in range(world)]
    values_back = []
    for dst in range(world):
        got_ids, _ = RR.unpack(sent[dst], recv_counts[dst], int(recv_counts[dst].sum()))
        local = got_ids - dst * (E // world)
        assert ((local >= 0) & (local < E // world)).all()
        vals = table[dst * (E // world):(dst + 1) * (E // world)][local]
        values_back.append(RR.pack(vals, recv_counts[dst], world, capacity, 0.0)[0])
    returned = RR.all_to_all(values_back)
    for r in range(world):
        s, order, counts, _ = plans[r]
        vals_sorted, _ = RR.unpack(returned[r], counts, int(counts.sum()))
        out = np.empty_like(vals_sorted)
        out[order] = vals_sorted
        assert np.array_equal(out, table[requests[r]])


# ---- Error branches, against arrays worked out by hand.  F is the fill.
# Source row k holds the value k, so every expected entry names the row it came from.

F = -1


def test_pack_count_above_capacity_consumes_its_rows():
    """Counts [2, 7, 1] at capacity 5: rank 1 keeps rows 2..6 and is cut at the
    capacity, but its segment still spans rows 2..8, so rank 2 starts at row 9."""
    rows = np.arange(10, dtype=np.int64)
    packed, bad = RR.pack(rows, np.array([2, 7, 1]), 3, 5, F)
    assert packed.tolist() == [[0, 1, F, F, F], [2, 3, 4, 5, 6], [9, F, F, F, F]]
    assert bad == 1


def test_pack_negative_count_is_empty_and_consumes_nothing():
    rows = np.arange(6, dtype=np.int64)
    packed, bad = RR.pack(rows, np.array([2, -3, 2]), 3, 4, F)
    assert packed.tolist() == [[0, 1, F, F], [F, F, F, F], [2, 3, F, F]]
    assert bad == 1
    packed, bad = RR.pack(rows, np.array([1, 2, -1]), 3, 2, F)   # the first bad rank is reported
    assert packed.tolist() == [[0, F], [1, 2], [F, F]] and bad == 2


def test_pack_rows_past_the_source_take_the_fill():
    """Only src_rows source rows exist: block rows whose source lies past them
    are filled and reported as rank `world`, unless a bad count comes first."""
    rows = np.arange(10, dtype=np.int64)
    packed, bad = RR.pack(rows, np.array([3, 3]), 2, 4, F, src_rows=5)
    assert packed.tolist() == [[0, 1, 2, F], [3, 4, F, F]] and bad == 2
    packed, bad = RR.pack(rows, np.array([2, 7, 1]), 3, 5, F, src_rows=8)
    assert packed.tolist() == [[0, 1, F, F, F], [2, 3, 4, 5, 6], [F, F, F, F, F]] and bad == 1
    packed, bad = RR.pack(rows, np.array([7, 0]), 2, 5, F, src_rows=5)   # the cut rows need not exist
    assert packed.tolist() == [[0, 1, 2, 3, 4], [F, F, F, F, F]] and bad == 0


def test_unpack_caps_each_segment_at_capacity():
    """Counts [1, 3, 2] at capacity 2: rank 1 contributes its block's 2 rows,
    never a row of the next block."""
    packed = np.array([[10, 11], [20, 21], [30, 31]], dtype=np.int64)
    out, bad = RR.unpack(packed, np.array([1, 3, 2]), 5)
    assert out.tolist() == [10, 20, 21, 30, 31] and bad == 1
    out, bad = RR.unpack(packed, np.array([2, -1, 1]), 4)
    assert out.tolist() == [10, 11, 30, 0] and bad == 1


def test_unpack_short_destination_keeps_what_fits():
    """Counts [2, 1, 2] into 4 rows: the last segment's first row still fits
    and is kept; its second is dropped, reported as rank `world`."""
    packed = np.array([[10, 11], [20, 21], [30, 31]], dtype=np.int64)
    out, bad = RR.unpack(packed, np.array([2, 1, 2]), 4)
    assert out.tolist() == [10, 11, 20, 30] and bad == 3
    out, bad = RR.unpack(packed, np.array([2, 1, 2]), 3)
    assert out.tolist() == [10, 11, 20] and bad == 3
    out, bad = RR.unpack(packed, np.array([2, 1, 2]), 6)
    assert out.tolist() == [10, 11, 20, 30, 31, 0] and bad == -1
