"""Planted mistakes in the routing and PLE oracles must each fail at least one
of their pins (tests/test_oracle_route.py, tests/test_oracle_ple.py).

Each mutant replaces one oracle function for the duration of a test (on the
CPU) and runs every pin of that oracle; a pin set that let a plausible slip
through would not pin the oracle."""
import numpy as np
import pytest

from oracle import ple_ref, route_ref
from tests import test_oracle_ple as PP
from tests import test_oracle_route as RP

_orig_conv = ple_ref.short_conv
_orig_conv_bwd = ple_ref.short_conv_backward
_orig_norm = ple_ref.grouped_rms_norm
_orig_norm_bwd = ple_ref.grouped_rms_norm_backward


def ple_pins():
    """Every PLE pin; returns the names of those that fail."""
    checks = [("library", lambda: [PP.test_conv_equals_library(K, d) for K, d in [(4, 3), (4, 1), (2, 5), (1, 3)]]),
              ("shift", PP.test_one_hot_kernel_is_a_shift), ("bias", PP.test_zero_start_gives_bias),
              ("halo", PP.test_halo_reproduces_full_sequence),
              ("conv_bwd", PP.test_conv_backward_finite_differences_and_autograd),
              ("norm", PP.test_norm_invariants), ("norm_bwd", PP.test_norm_backward_finite_differences)]
    failed = []
    for name, fn in checks:
        try:
            fn()
        except AssertionError:
            failed.append(name)
    return failed


def route_pins():
    checks = [("plan", lambda: [RP.test_plan_is_stable_grouping(w) for w in (1, 3, 8, 64)]),
              ("validate", RP.test_validate_finds_misrouted), ("pack", RP.test_pack_unpack_inverse),
              ("loopback", RP.test_loopback_world_equals_direct_lookup),
              ("pack_over_capacity", RP.test_pack_count_above_capacity_consumes_its_rows),
              ("pack_negative", RP.test_pack_negative_count_is_empty_and_consumes_nothing),
              ("pack_past_source", RP.test_pack_rows_past_the_source_take_the_fill),
              ("unpack_capacity", RP.test_unpack_caps_each_segment_at_capacity),
              ("unpack_short", RP.test_unpack_short_destination_keeps_what_fits)]
    failed = []
    for name, fn in checks:
        try:
            fn()
        except (AssertionError, IndexError, ValueError):
            failed.append(name)
    return failed


def test_real_oracles_pass_their_pins():
    assert ple_pins() == []
    assert route_pins() == []


# ---- PLE mutants

def conv_taps_reversed(x, weight, bias=None, dilation=3, halo=None):
    return _orig_conv(x, np.asarray(weight)[:, ::-1], bias, dilation, halo)


def conv_dilation_ignored(x, weight, bias=None, dilation=3, halo=None):
    h = None if halo is None else np.asarray(halo)[:, -(np.asarray(weight).shape[1] - 1):]
    return _orig_conv(x, weight, bias, 1, h)


def conv_halo_shifted(x, weight, bias=None, dilation=3, halo=None):
    if halo is not None:
        halo = np.roll(np.asarray(halo, dtype=np.float64), 1, axis=1)
    return _orig_conv(x, weight, bias, dilation, halo)


def conv_bias_dropped(x, weight, bias=None, dilation=3, halo=None):
    return _orig_conv(x, weight, None, dilation, halo)


def conv_bwd_no_halo_in_dw(x, dy, weight, dilation=3, halo=None):
    dx, dw, db, dh = _orig_conv_bwd(x, dy, weight, dilation, None)
    _, _, _, dh2 = _orig_conv_bwd(x, dy, weight, dilation, halo)
    return dx, dw, db, dh2


def conv_bwd_taps_forward(x, dy, weight, dilation=3, halo=None):
    dx, dw, db, dh = _orig_conv_bwd(x, dy, np.asarray(weight)[:, ::-1], dilation, halo)
    return dx, dw[:, ::-1], db, dh


def norm_whole_row(x, weight, group_size, eps=1e-6):
    return _orig_norm(x, weight, np.asarray(x).shape[-1], eps)


def norm_plain_weight(x, weight, group_size, eps=1e-6):
    return _orig_norm(x, np.asarray(weight, dtype=np.float64) - 1.0, group_size, eps)


def norm_eps_outside(x, weight, group_size, eps=1e-6):
    x = np.asarray(x, dtype=np.float64)
    g = x.reshape(-1, x.shape[-1] // group_size, group_size)
    y = g / (np.sqrt((g * g).mean(axis=-1, keepdims=True)) + eps)
    return (y.reshape(-1, x.shape[-1]) * (1.0 + np.asarray(weight))).reshape(x.shape)


def norm_bwd_no_projection(x, dy, weight, group_size, eps=1e-6):
    x = np.asarray(x, dtype=np.float64)
    g = x.reshape(-1, x.shape[-1] // group_size, group_size)
    inv = 1.0 / np.sqrt((g * g).mean(axis=-1, keepdims=True) + eps)
    dn = (np.asarray(dy).reshape(-1, x.shape[-1]) * (1.0 + np.asarray(weight))).reshape(g.shape)
    _, dw = _orig_norm_bwd(x, dy, weight, group_size, eps)
    return (inv * dn).reshape(x.shape), dw


@pytest.mark.parametrize("attr,mutant", [
    ("short_conv", conv_taps_reversed), ("short_conv", conv_dilation_ignored), ("short_conv", conv_halo_shifted),
    ("short_conv", conv_bias_dropped), ("short_conv_backward", conv_bwd_no_halo_in_dw),
    ("short_conv_backward", conv_bwd_taps_forward), ("grouped_rms_norm", norm_whole_row),
    ("grouped_rms_norm", norm_plain_weight), ("grouped_rms_norm", norm_eps_outside),
    ("grouped_rms_norm_backward", norm_bwd_no_projection)], ids=lambda v: getattr(v, "__name__", v))
def test_ple_mutant_is_caught(monkeypatch, attr, mutant):
    monkeypatch.setattr(ple_ref, attr, mutant)
    assert ple_pins(), "mutant %s passed every PLE pin" % mutant.__name__


# ---- routing mutants

_orig_plan = route_ref.route_plan
_orig_pack = route_ref.pack
_orig_unpack = route_ref.unpack
_orig_validate = route_ref.validate


def plan_reversed_inside_segment(ids, num_embeddings, world):
    s, order, counts, bad = _orig_plan(ids, num_embeddings, world)
    order = order.copy()
    start = 0
    for c in counts:
        order[start:start + c] = order[start:start + c][::-1]
        start += int(c)
    return np.asarray(ids)[order], order, counts, bad


def plan_counts_outside(ids, num_embeddings, world):
    s, order, counts, bad = _orig_plan(ids, num_embeddings, world)
    counts = counts.copy()
    counts[-1] += int((np.asarray(ids) >= num_embeddings).sum() + (np.asarray(ids) < 0).sum())
    return s, order, counts, bad


def pack_no_fill(rows, split_sizes, world, capacity, fill, src_rows=None):
    return _orig_pack(rows, split_sizes, world, capacity, 0, src_rows)


def pack_advances_by_kept_rows(rows, split_sizes, world, capacity, fill, src_rows=None):
    """The source advances by the rows kept (min(count, capacity)) instead of
    the whole segment, so the rank after a cut one starts too early."""
    rows = np.asarray(rows)
    src_rows = rows.shape[0] if src_rows is None else src_rows
    out = np.full((world, capacity) + rows.shape[1:], fill, dtype=rows.dtype)
    bad, past, start = -1, False, 0
    for w in range(world):
        c = int(split_sizes[w])
        if (c < 0 or c > capacity) and bad < 0:
            bad = w
        k = max(0, min(c, capacity))
        for s in range(k):
            if start + s < src_rows:
                out[w, s] = rows[start + s]
            else:
                past = True
        start += k
    return out, (world if bad < 0 and past else bad)


def pack_negative_advances(rows, split_sizes, world, capacity, fill, src_rows=None):
    """A negative count moves the source back (start += count)."""
    rows = np.asarray(rows)
    src_rows = rows.shape[0] if src_rows is None else src_rows
    out = np.full((world, capacity) + rows.shape[1:], fill, dtype=rows.dtype)
    bad, past, start = -1, False, 0
    for w in range(world):
        c = int(split_sizes[w])
        if (c < 0 or c > capacity) and bad < 0:
            bad = w
        for s in range(max(0, min(c, capacity))):
            if 0 <= start + s < src_rows:
                out[w, s] = rows[start + s]
            else:
                past = True
        start += c
    return out, (world if bad < 0 and past else bad)


def pack_reads_past_source(rows, split_sizes, world, capacity, fill, src_rows=None):
    """src_rows ignored: every segment row is read from the array as given."""
    return _orig_pack(rows, split_sizes, world, capacity, fill, None)


def unpack_unclamped(packed, split_sizes, dst_rows):
    """No per-segment capacity cap: a count above the capacity reads on into
    the next rank's block (rows of the flattened [world * capacity] array)."""
    packed = np.asarray(packed)
    world, capacity = packed.shape[:2]
    flat = packed.reshape((world * capacity,) + packed.shape[2:])
    out = np.zeros((dst_rows,) + packed.shape[2:], dtype=packed.dtype)
    bad, i = -1, 0
    for w in range(world):
        c = int(split_sizes[w])
        if (c < 0 or c > capacity) and bad < 0:
            bad = w
        for s in range(max(0, c)):
            if i < dst_rows and w * capacity + s < flat.shape[0]:
                out[i] = flat[w * capacity + s]
            i += 1
    return out, (world if bad < 0 and i > dst_rows else bad)


def unpack_drops_partial_segment(packed, split_sizes, dst_rows):
    """A segment that does not fit whole is dropped whole."""
    packed = np.asarray(packed)
    world, capacity = packed.shape[:2]
    out = np.zeros((dst_rows,) + packed.shape[2:], dtype=packed.dtype)
    bad, i = -1, 0
    for w in range(world):
        c = int(split_sizes[w])
        if (c < 0 or c > capacity) and bad < 0:
            bad = w
        k = max(0, min(c, capacity))
        if i + k <= dst_rows:
            out[i:i + k] = packed[w, :k]
        i += k
    return out, (world if bad < 0 and i > dst_rows else bad)


def unpack_segments_reversed(packed, split_sizes, dst_rows):
    """Each rank's count applied to the mirrored rank's block."""
    return _orig_unpack(packed, np.asarray(split_sizes)[::-1], dst_rows)


def validate_off_by_one(sorted_ids, send_counts, num_embeddings, world):
    n = len(sorted_ids)
    if any(c < 0 for c in send_counts) or sum(int(c) for c in send_counts) > n:
        return n
    local = num_embeddings // world
    i = 0
    for w, c in enumerate(int(c) for c in send_counts):
        for _ in range(c):
            g = int(sorted_ids[i])
            if not (w * local <= g <= (w + 1) * local):  # inclusive upper bound: the slip
                return i
            i += 1
    return -1


@pytest.mark.parametrize("attr,mutant", [
    ("route_plan", plan_reversed_inside_segment), ("route_plan", plan_counts_outside), ("pack", pack_no_fill),
    ("pack", pack_advances_by_kept_rows), ("pack", pack_negative_advances), ("pack", pack_reads_past_source),
    ("unpack", unpack_unclamped), ("unpack", unpack_drops_partial_segment), ("unpack", unpack_segments_reversed),
    ("validate", validate_off_by_one)], ids=lambda v: getattr(v, "__name__", v))
def test_route_mutant_is_caught(monkeypatch, attr, mutant):
    monkeypatch.setattr(route_ref, attr, mutant)
    assert route_pins(), "mutant %s passed every routing pin" % mutant.__name__
