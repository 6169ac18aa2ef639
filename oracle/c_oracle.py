"""ctypes wrapper of the plain-C oracle (``engram_oracle.c``) — test infrastructure.

numpy arrays in, numpy arrays out; no GPU, no torch.  ``build()`` compiles the
C file with gcc into ``oracle/libengram_oracle.so``; ``load()`` builds it when
it is missing.  The ``*_mt`` functions call the OpenMP twins in
``engram_oracle_mt.c`` (``oracle/libengram_oracle_mt.so``), which spread the
same computation over every host core for the CPU baseline and give the same
bits.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "engram_oracle.c")
_SRC_MT = os.path.join(_HERE, "engram_oracle_mt.c")
# ENGRAM_ORACLE_LIBDIR points at another build of the two libraries (the
# sanitizer test builds them with AddressSanitizer and UBSan there).
_LIBDIR = os.environ.get("ENGRAM_ORACLE_LIBDIR", _HERE)
_LIB = os.path.join(_LIBDIR, "libengram_oracle.so")
_LIB_MT = os.path.join(_LIBDIR, "libengram_oracle_mt.so")
_lib = None
_lib_mt = None

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32


def build():
    """Compile the oracle (plain -O2 C, single-threaded) and its OpenMP twin."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", tmp, _SRC])
    os.replace(tmp, _LIB)
    tmp = _LIB_MT + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=gnu11", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC_MT])
    os.replace(tmp, _LIB_MT)
    return _LIB


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    lib.oracle_hash.restype = ctypes.c_int
    lib.oracle_hash.argtypes = [_p, _i64, _i64, _i32, _i32, _i64, _i64, _p, _p, _p, _p]
    lib.oracle_gather.restype = _i64
    lib.oracle_gather.argtypes = [_p, _i32, _i32, _i64, _i64, _p, _i64, _p]
    lib.oracle_scatter_add_dense.restype = _i64
    lib.oracle_scatter_add_dense.argtypes = [_p, _i64, _p, _i32, _i32, _i64, _i64, _p, _p]
    lib.oracle_scatter_add_compact.restype = _i64
    lib.oracle_scatter_add_compact.argtypes = [_p, _i64, _p, _i32, _i32, _i64, _i64, _p, _p, _p]
    _lib = lib
    return lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def hash_input_ids(ids, ngram_size, heads_per_ngram, eos, fill, multipliers, vocab_sizes, offsets):
    """ids: int64 [batch, seq] -> int64 [batch, seq, heads]."""
    lib = load()
    ids = np.ascontiguousarray(ids, dtype=np.int64)
    assert ids.ndim == 2
    batch, seq = ids.shape
    heads = (ngram_size - 1) * heads_per_ngram
    mult = np.ascontiguousarray(multipliers, dtype=np.int64)
    mods = np.ascontiguousarray(vocab_sizes, dtype=np.int64)
    offs = np.ascontiguousarray(offsets, dtype=np.int64)
    assert mult.size >= ngram_size and mods.size == heads and offs.size == heads
    rows = np.empty((batch, seq, heads), dtype=np.int64)
    rc = lib.oracle_hash(_ptr(ids), batch, seq, ngram_size, heads_per_ngram, int(eos), int(fill),
                         _ptr(mult), _ptr(mods), _ptr(offs), _ptr(rows))
    if rc != 0:
        raise ValueError("oracle_hash rejected the configuration")
    return rows


def _elem(table_or_grad):
    """Element size and bf16 flag for float32 arrays or uint16 arrays holding bf16 bits."""
    if table_or_grad.dtype == np.float32:
        return 4, 0
    if table_or_grad.dtype == np.uint16:
        return 2, 1
    raise TypeError("expected float32 or uint16 (bf16 bits), got %s" % table_or_grad.dtype)


def gather(table, rows, row_begin=0):
    """table: [num_rows, dim] float32 or uint16 (bf16 bits); rows: int64 [...].

    Returns (out [..., dim] same dtype, first_bad index or -1)."""
    lib = load()
    table = np.ascontiguousarray(table)
    rows_flat = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1)
    num_rows, dim = table.shape
    esize, _ = _elem(table)
    out = np.empty((rows_flat.size, dim), dtype=table.dtype)
    bad = lib.oracle_gather(_ptr(table), esize, dim, int(row_begin), num_rows, _ptr(rows_flat),
                            rows_flat.size, _ptr(out))
    return out.reshape(tuple(np.shape(rows)) + (dim,)), int(bad)


def scatter_add_dense(rows, dy, num_rows, row_begin=0, grad_in=None):
    """Returns (grad fp64 [num_rows, dim], first_bad)."""
    lib = load()
    rows_flat = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1)
    dy = np.ascontiguousarray(dy)
    dy = dy.reshape(rows_flat.size, dy.shape[-1])
    dim = dy.shape[1]
    _, is_bf16 = _elem(dy)
    if grad_in is None:
        grad_in = np.zeros((num_rows, dim), dtype=np.float32)
    grad_in = np.ascontiguousarray(grad_in, dtype=np.float32)
    assert grad_in.shape == (num_rows, dim)
    out = np.empty((num_rows, dim), dtype=np.float64)
    bad = lib.oracle_scatter_add_dense(_ptr(rows_flat), rows_flat.size, _ptr(dy), is_bf16, dim,
                                       int(row_begin), num_rows, _ptr(grad_in), _ptr(out))
    return out, int(bad)


def scatter_add_compact(rows, dy, num_rows, row_begin=0):
    """Returns (uniq_rows int64 [U], uniq_grad fp64 [U, dim], first_bad)."""
    lib = load()
    rows_flat = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1)
    n = rows_flat.size
    dy = np.ascontiguousarray(dy)
    dy = dy.reshape(n, dy.shape[-1])
    dim = dy.shape[1]
    _, is_bf16 = _elem(dy)
    uniq_rows = np.empty(max(n, 1), dtype=np.int64)
    uniq_grad = np.empty((max(n, 1), dim), dtype=np.float64)
    nu = np.zeros(1, dtype=np.int64)
    bad = lib.oracle_scatter_add_compact(_ptr(rows_flat), n, _ptr(dy), is_bf16, dim, int(row_begin),
                                         num_rows, _ptr(uniq_rows), _ptr(uniq_grad), _ptr(nu))
    u = int(nu[0])
    return uniq_rows[:u].copy(), uniq_grad[:u].copy(), int(bad)


# ---- the OpenMP twins (same results, every host core)

def load_mt():
    global _lib_mt
    if _lib_mt is not None:
        return _lib_mt
    if not os.path.exists(_LIB_MT) or os.path.getmtime(_LIB_MT) < os.path.getmtime(_SRC_MT):
        build()
    lib = ctypes.CDLL(_LIB_MT)
    lib.oracle_mt_threads.restype = ctypes.c_int
    lib.oracle_mt_threads.argtypes = []
    lib.oracle_mt_hash.restype = ctypes.c_int
    lib.oracle_mt_hash.argtypes = [_p, _i64, _i64, _i32, _i32, _i64, _i64, _p, _p, _p, _p]
    lib.oracle_mt_gather.restype = _i64
    lib.oracle_mt_gather.argtypes = [_p, _i32, _i32, _i64, _i64, _p, _i64, _p]
    lib.oracle_mt_scatter_add_compact.restype = _i64
    lib.oracle_mt_scatter_add_compact.argtypes = [_p, _i64, _p, _i32, _i32, _i64, _i64, _p, _p, _p]
    _lib_mt = lib
    return lib


def mt_threads():
    """OpenMP threads the *_mt functions run on."""
    return int(load_mt().oracle_mt_threads())


def hash_input_ids_mt(ids, ngram_size, heads_per_ngram, eos, fill, multipliers, vocab_sizes, offsets):
    lib = load_mt()
    ids = np.ascontiguousarray(ids, dtype=np.int64)
    assert ids.ndim == 2
    batch, seq = ids.shape
    heads = (ngram_size - 1) * heads_per_ngram
    mult = np.ascontiguousarray(multipliers, dtype=np.int64)
    mods = np.ascontiguousarray(vocab_sizes, dtype=np.int64)
    offs = np.ascontiguousarray(offsets, dtype=np.int64)
    assert mult.size >= ngram_size and mods.size == heads and offs.size == heads
    rows = np.empty((batch, seq, heads), dtype=np.int64)
    rc = lib.oracle_mt_hash(_ptr(ids), batch, seq, ngram_size, heads_per_ngram, int(eos), int(fill),
                            _ptr(mult), _ptr(mods), _ptr(offs), _ptr(rows))
    if rc != 0:
        raise ValueError("oracle_mt_hash rejected the configuration")
    return rows


def gather_mt(table, rows, row_begin=0):
    lib = load_mt()
    table = np.ascontiguousarray(table)
    rows_flat = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1)
    num_rows, dim = table.shape
    esize, _ = _elem(table)
    out = np.empty((rows_flat.size, dim), dtype=table.dtype)
    bad = lib.oracle_mt_gather(_ptr(table), esize, dim, int(row_begin), num_rows, _ptr(rows_flat), rows_flat.size,
                               _ptr(out))
    return out.reshape(tuple(np.shape(rows)) + (dim,)), int(bad)


def scatter_add_compact_mt(rows, dy, num_rows, row_begin=0):
    lib = load_mt()
    rows_flat = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1)
    n = rows_flat.size
    dy = np.ascontiguousarray(dy)
    dy = dy.reshape(n, dy.shape[-1])
    dim = dy.shape[1]
    _, is_bf16 = _elem(dy)
    uniq_rows = np.empty(max(n, 1), dtype=np.int64)
    uniq_grad = np.empty((max(n, 1), dim), dtype=np.float64)
    nu = np.zeros(1, dtype=np.int64)
    bad = lib.oracle_mt_scatter_add_compact(_ptr(rows_flat), n, _ptr(dy), is_bf16, dim, int(row_begin), num_rows,
                                            _ptr(uniq_rows), _ptr(uniq_grad), _ptr(nu))
    u = int(nu[0])
    return uniq_rows[:u].copy(), uniq_grad[:u].copy(), int(bad)
