"""Oracle of the owner routing steps — test infrastructure.

Engram API page ("nemo_automodel.components.models.qwen3_8_flash_next.engram"),
Qwen3_8_FlashNextOwnerShardedEmbedding: rank r owns rows
[r * local_rows, (r + 1) * local_rows).  Before the first All-to-All
(_exchange_ids) a request rank groups its global IDs by owner;
_validate_sorted_send_ids checks each destination segment;
_fixed_capacity_all_to_all pads every peer segment to one agreed capacity with
a fill value and restores the compact, source-ordered result.  Plain loops
over segments; numpy only holds the arrays.
"""
import numpy as np


def route_plan(ids, num_embeddings, world):
    """Returns (sorted_ids, order, send_counts, first_bad).  Segments in owner
    order, request order inside a segment; IDs outside the table go last."""
    local = num_embeddings // world
    segments = [[] for _ in range(world)]
    outside = []
    for pos, g in enumerate(int(x) for x in ids):
        if 0 <= g < num_embeddings:
            segments[g // local].append(pos)
        else:
            outside.append(pos)
    order = [p for seg in segments for p in seg] + outside
    ids = np.asarray(ids, dtype=np.int64)
    return (ids[order] if order else ids[:0].copy(), np.asarray(order, dtype=np.int64),
            np.asarray([len(s) for s in segments], dtype=np.int64), outside[0] if outside else -1)


def validate(sorted_ids, send_counts, num_embeddings, world):
    """Lowest sorted index whose ID is not owned by its segment's rank; n when a
    count is negative or the counts exceed n; else -1."""
    n = len(sorted_ids)
    if any(c < 0 for c in send_counts) or sum(int(c) for c in send_counts) > n:
        return n
    local = num_embeddings // world
    i = 0
    for w, c in enumerate(int(c) for c in send_counts):
        for _ in range(c):
            g = int(sorted_ids[i])
            if not (w * local <= g < (w + 1) * local):
                return i
            i += 1
    return -1


def pack(rows, split_sizes, world, capacity, fill, src_rows=None):
    """Compact rows -> [world, capacity, ...]; returns (packed, status).

    Segment w is the next max(count_w, 0) source rows, in rank order; block w
    holds its first min(count_w, capacity) rows and the fill after them.  A
    count above the capacity still consumes all its source rows (the rows past
    the capacity are the ones cut), and a negative count is an empty segment
    that consumes none.  Only the first `src_rows` source rows exist (default:
    all of them); a block row whose source lies past them takes the fill.
    status: the lowest rank whose count is negative or above the capacity,
    else `world` when some segment reaches past src_rows, else -1."""
    rows = np.asarray(rows)
    if src_rows is None:
        src_rows = rows.shape[0]
    out = np.full((world, capacity) + rows.shape[1:], fill, dtype=rows.dtype)
    bad = -1
    past_end = False
    start = 0
    for w in range(world):
        c = int(split_sizes[w])
        if (c < 0 or c > capacity) and bad < 0:
            bad = w
        for s in range(max(0, min(c, capacity))):
            if start + s < src_rows:
                out[w, s] = rows[start + s]
            else:
                past_end = True
        start += max(c, 0)
    if bad < 0 and past_end:
        bad = world
    return out, bad


def unpack(packed, split_sizes, dst_rows):
    """[world, capacity, ...] -> (compact [dst_rows, ...], status).

    The first min(count_w, capacity) rows of block w (none for a negative
    count) are appended in rank order; rows that would land at or past
    dst_rows are dropped, and the output rows after the last appended one are
    zero.  status: the lowest rank whose count is negative or above the
    capacity, else `world` when the appended rows exceed dst_rows, else -1."""
    packed = np.asarray(packed)
    world, capacity = packed.shape[:2]
    out = np.zeros((dst_rows,) + packed.shape[2:], dtype=packed.dtype)
    bad = -1
    i = 0
    for w in range(world):
        c = int(split_sizes[w])
        if (c < 0 or c > capacity) and bad < 0:
            bad = w
        for s in range(max(0, min(c, capacity))):
            if i < dst_rows:
                out[i] = packed[w, s]
            i += 1
    if bad < 0 and i > dst_rows:
        bad = world
    return out, bad


def all_to_all(blocks):
    """Loopback exchange of virtual ranks: blocks[src] is [world, capacity, ...];
    rank dst receives blocks[src][dst] from every src, stacked by src."""
    world = len(blocks)
    return [np.stack([blocks[s][d] for s in range(world)]) for d in range(world)]
