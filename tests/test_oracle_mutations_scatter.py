"""Planted mistakes in the C oracle's gather and scatter-add must each fail at
least one of their pins (tests/test_oracle_gather_scatter.py).

Each mutant wraps the oracle's own function and changes its result the way a
plausible slip in the C code would: a missing or shifted owner offset,
clamping instead of rejecting, the last offending index instead of the first,
a dropped prior gradient, fp32 accumulation, a lookup lost at the end, rows
left in first-seen order or reported shard-local.  Mutants live only in this
test, on the CPU."""
import numpy as np
import pytest

from oracle import c_oracle
from tests import test_oracle_gather_scatter as T

ORIG = {"gather": c_oracle.gather, "dense": c_oracle.scatter_add_dense, "compact": c_oracle.scatter_add_compact}


def run_pins():
    """Number of pins that fail (an exception counts as a failure)."""
    pins = [lambda: T.test_gather_equals_index_select("f32"), lambda: T.test_gather_equals_index_select("bf16"),
            T.test_gather_out_of_range,
            lambda: T.test_scatter_equals_one_hot("f32"), lambda: T.test_scatter_equals_one_hot("bf16"),
            T.test_scatter_ones_is_histogram, T.test_scatter_integer_grads_exact,
            T.test_scatter_empty_and_all_invalid]
    failed = 0
    for pin in pins:
        try:
            pin()
        except Exception:
            failed += 1
    return failed


def as_f32(dy):
    dy = np.asarray(dy)
    if dy.dtype == np.uint16:
        return (dy.astype(np.uint32) << 16).view(np.float32)
    return dy.astype(np.float32)


def last_bad(rows, row_begin, num_rows):
    local = np.asarray(rows, dtype=np.int64).reshape(-1) - row_begin
    bad = np.nonzero((local < 0) | (local >= num_rows))[0]
    return int(bad[-1]) if bad.size else -1


# ---- gather mutants
def gather_ignores_row_begin(table, rows, row_begin=0):
    return ORIG["gather"](table, rows, 0)


def gather_reads_next_row(table, rows, row_begin=0):
    return ORIG["gather"](table, rows, row_begin - 1)


def gather_clamps(table, rows, row_begin=0):
    num_rows = np.shape(table)[0]
    clamped = np.clip(np.asarray(rows, dtype=np.int64) - row_begin, 0, num_rows - 1) + row_begin
    out, _ = ORIG["gather"](table, clamped, row_begin)
    return out, -1


def gather_reports_last_bad(table, rows, row_begin=0):
    out, _ = ORIG["gather"](table, rows, row_begin)
    return out, last_bad(rows, row_begin, np.shape(table)[0])


# ---- dense scatter-add mutants
def dense_drops_prior(rows, dy, num_rows, row_begin=0, grad_in=None):
    out, bad = ORIG["dense"](rows, dy, num_rows, row_begin, grad_in)
    if grad_in is not None:
        out = out - np.asarray(grad_in, dtype=np.float64)
    return out, bad


def dense_fp32_accumulate(rows, dy, num_rows, row_begin=0, grad_in=None):
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    d = as_f32(dy).reshape(rows.size, -1)
    acc = np.zeros((num_rows, d.shape[1]), dtype=np.float32) if grad_in is None else \
        np.array(grad_in, dtype=np.float32)
    ok = (rows >= row_begin) & (rows < row_begin + num_rows)
    np.add.at(acc, rows[ok] - row_begin, d[ok])
    bad = np.nonzero(~ok)[0]
    return acc.astype(np.float64), int(bad[0]) if bad.size else -1


def dense_clamps_rows(rows, dy, num_rows, row_begin=0, grad_in=None):
    r = np.clip(np.asarray(rows, dtype=np.int64) - row_begin, 0, num_rows - 1) + row_begin
    return ORIG["dense"](r, dy, num_rows, row_begin, grad_in)


def dense_drops_last_lookup(rows, dy, num_rows, row_begin=0, grad_in=None):
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    d = np.asarray(dy).reshape(rows.size, -1)
    if rows.size == 0:
        return ORIG["dense"](rows, d, num_rows, row_begin, grad_in)
    return ORIG["dense"](rows[:-1], d[:-1], num_rows, row_begin, grad_in)


# ---- compact scatter-add mutants
def compact_first_seen_order(rows, dy, num_rows, row_begin=0):
    ur, ug, bad = ORIG["compact"](rows, dy, num_rows, row_begin)
    flat = np.asarray(rows, dtype=np.int64).reshape(-1)
    first = {}
    for i, r in enumerate(flat):
        first.setdefault(int(r), i)
    order = np.argsort([first[int(r)] for r in ur], kind="stable")
    return ur[order], ug[order], bad


def compact_local_rows(rows, dy, num_rows, row_begin=0):
    ur, ug, bad = ORIG["compact"](rows, dy, num_rows, row_begin)
    return ur - row_begin, ug, bad


def compact_reports_last_bad(rows, dy, num_rows, row_begin=0):
    ur, ug, _ = ORIG["compact"](rows, dy, num_rows, row_begin)
    return ur, ug, last_bad(rows, row_begin, num_rows)


def compact_drops_last_lookup(rows, dy, num_rows, row_begin=0):
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    d = np.asarray(dy).reshape(rows.size, -1)
    if rows.size == 0:
        return ORIG["compact"](rows, d, num_rows, row_begin)
    return ORIG["compact"](rows[:-1], d[:-1], num_rows, row_begin)


MUTANTS = {
    "gather_ignores_row_begin": ("gather", gather_ignores_row_begin),
    "gather_reads_next_row": ("gather", gather_reads_next_row),
    "gather_clamps": ("gather", gather_clamps),
    "gather_reports_last_bad": ("gather", gather_reports_last_bad),
    "dense_drops_prior": ("scatter_add_dense", dense_drops_prior),
    "dense_fp32_accumulate": ("scatter_add_dense", dense_fp32_accumulate),
    "dense_clamps_rows": ("scatter_add_dense", dense_clamps_rows),
    "dense_drops_last_lookup": ("scatter_add_dense", dense_drops_last_lookup),
    "compact_first_seen_order": ("scatter_add_compact", compact_first_seen_order),
    "compact_local_rows": ("scatter_add_compact", compact_local_rows),
    "compact_reports_last_bad": ("scatter_add_compact", compact_reports_last_bad),
    "compact_drops_last_lookup": ("scatter_add_compact", compact_drops_last_lookup),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_caught(monkeypatch, name):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(c_oracle, attr, fn)
    assert run_pins() > 0, "mutant %s passed every pin" % name


def test_unmutated_passes():
    assert run_pins() == 0
