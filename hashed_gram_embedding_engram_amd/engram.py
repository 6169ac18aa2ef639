"""Thin Python binding of libengram (include/engram.h): argument marshalling only.

Every step of the path runs in the library's HIP kernels.  torch supplies
device memory and the current HIP stream; nothing here computes on tensors.
If the library is missing, loading fails with an error — there is no CPU or
PyTorch fallback.

The functions keep the names of the C ABI (``engram_hash``, ``engram_hash_slice``,
``engram_gather``, ``engram_hash_gather``, ``engram_scatter_add``, ...) and take
torch tensors in place of raw pointers.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libengram.so")

ENGRAM_OK, ENGRAM_EINVAL, ENGRAM_EDTYPE, ENGRAM_EWORKSPACE, ENGRAM_ELAUNCH, ENGRAM_ESPEC = 0, -1, -2, -3, -4, -5
ENGRAM_F32, ENGRAM_BF16 = 0, 1
MAX_NGRAM, MAX_HEADS = 8, 64

# Released Qwen3.8-Flash-Next configuration (engram API page,
# "nemo_automodel.components.models.qwen3_8_flash_next.engram": module data and
# the Qwen3_8_FlashNextNGramEmbedding signature).  The page prints the first
# eight head moduli and offsets before cutting the tuples off; the remaining
# eight moduli continue the run of consecutive primes above 20,000,000 that the
# printed ones start, and every offset is the running total of the moduli
# before it.  Their sum, rounded up to a multiple of 128, is the printed
# padded row count.
QWEN3_8_FLASH_NEXT_LAYER_MULTIPLIERS = (23703573157769, 20109073645365, 8052911324071)
QWEN3_8_FLASH_NEXT_NGRAM_HEAD_VOCAB_SIZES = (
    20000003, 20000023, 20000033, 20000047, 20000059, 20000063, 20000069, 20000077,
    20000081, 20000093, 20000107, 20000147, 20000153, 20000159, 20000161, 20000171)
QWEN3_8_FLASH_NEXT_NGRAM_HEAD_OFFSETS = (
    0, 20000003, 40000026, 60000059, 80000106, 100000165, 120000228, 140000297,
    160000374, 180000455, 200000548, 220000655, 240000802, 260000955, 280001114, 300001275)
QWEN3_8_FLASH_NEXT_NGRAM_PADDED_ROWS = 320001536
QWEN3_8_FLASH_NEXT_EOS_TOKEN_ID = 248044
QWEN3_8_FLASH_NEXT_EMBEDDING_DIM = 160


class EngramHashSpec(ctypes.Structure):
    """Mirror of ``engram_hash_spec``."""
    _fields_ = [("ngram_size", ctypes.c_int32), ("heads_per_ngram", ctypes.c_int32),
                ("eos_id", ctypes.c_int64), ("fill_id", ctypes.c_int64),
                ("multipliers", ctypes.c_int64 * MAX_NGRAM), ("head_mod", ctypes.c_int64 * MAX_HEADS),
                ("head_offset", ctypes.c_int64 * MAX_HEADS)]

    @property
    def num_heads(self):
        return (self.ngram_size - 1) * self.heads_per_ngram


def make_hash_spec(ngram_size, heads_per_ngram, eos_id, multipliers, head_mod, head_offset, fill_id=0):
    s = EngramHashSpec()
    s.ngram_size, s.heads_per_ngram = int(ngram_size), int(heads_per_ngram)
    s.eos_id, s.fill_id = int(eos_id), int(fill_id)
    if len(multipliers) > MAX_NGRAM or len(head_mod) > MAX_HEADS or len(head_offset) != len(head_mod):
        raise ValueError("hash spec arrays too long or mismatched")
    for k, m in enumerate(multipliers):
        s.multipliers[k] = int(m)
    for h, (m, o) in enumerate(zip(head_mod, head_offset)):
        s.head_mod[h], s.head_offset[h] = int(m), int(o)
    return s


def qwen3_8_flash_next_spec(fill_id=0):
    """The released hash configuration: 3-gram, 8 heads per order, EOS 248044."""
    return make_hash_spec(3, 8, QWEN3_8_FLASH_NEXT_EOS_TOKEN_ID, QWEN3_8_FLASH_NEXT_LAYER_MULTIPLIERS,
                          QWEN3_8_FLASH_NEXT_NGRAM_HEAD_VOCAB_SIZES, QWEN3_8_FLASH_NEXT_NGRAM_HEAD_OFFSETS,
                          fill_id)


_lib = None


def load_library(path=LIB_PATH):
    """Load libengram.so; raises if it has not been built (no fallback path exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libengram.so not found at %s: build it with "
                           "`python -m hashed_gram_embedding_engram_amd.build`" % path)
    lib = ctypes.CDLL(path)
    p, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    lib.engram_hash.restype = ctypes.c_int
    lib.engram_hash.argtypes = [p, i64, i64, ctypes.POINTER(EngramHashSpec), p, p]
    lib.engram_hash_slice.restype = ctypes.c_int
    lib.engram_hash_slice.argtypes = [p, i64, i64, i64, i64, ctypes.POINTER(EngramHashSpec), p, p]
    lib.engram_gather.restype = ctypes.c_int
    lib.engram_gather.argtypes = [p, i32, i64, i64, i32, p, i64, p, p, p]
    lib.engram_hash_gather.restype = ctypes.c_int
    lib.engram_hash_gather.argtypes = [p, i64, i64, ctypes.POINTER(EngramHashSpec), p, i32, i64, i64, i32, p, p, p, p]
    lib.engram_hash_gather_slice.restype = ctypes.c_int
    lib.engram_hash_gather_slice.argtypes = [p, i64, i64, i64, i64, ctypes.POINTER(EngramHashSpec), p, i32, i64, i64,
                                             i32, p, p, p, p]
    lib.engram_scatter_add_workspace.restype = sz
    lib.engram_scatter_add_workspace.argtypes = [i64, i64, i32]
    lib.engram_scatter_add.restype = ctypes.c_int
    lib.engram_scatter_add.argtypes = [p, i64, p, i32, i32, i64, i64, p, p, p, p, p, sz, p, p]
    lib.engram_scatter_add_plan.restype = ctypes.c_int
    lib.engram_scatter_add_plan.argtypes = [p, i64, i64, i64, i32, p, p, p, sz, p, p]
    lib.engram_scatter_add_plan_padded.restype = ctypes.c_int
    lib.engram_scatter_add_plan_padded.argtypes = [p, p, i32, i64, i64, i64, i32, p, p, p, sz, p, p]
    lib.engram_scatter_add_plan_from_tokens.restype = ctypes.c_int
    lib.engram_scatter_add_plan_from_tokens.argtypes = [p, i64, i64, ctypes.POINTER(EngramHashSpec), i64, i64, i32, p,
                                                        p, p, sz, p, p]
    lib.engram_scatter_add_plan_from_tokens_slice.restype = ctypes.c_int
    lib.engram_scatter_add_plan_from_tokens_slice.argtypes = [p, i64, i64, i64, i64, ctypes.POINTER(EngramHashSpec),
                                                              i64, i64, i32, p, p, p, sz, p, p]
    lib.engram_scatter_add_apply.restype = ctypes.c_int
    lib.engram_scatter_add_apply.argtypes = [p, i32, i32, i64, i64, i64, p, p, p, sz, p]
    lib.engram_scatter_add_noalloc.restype = ctypes.c_int
    lib.engram_scatter_add_noalloc.argtypes = [p, i64, p, i32, i32, i64, i64, p, p, p, p, p, p]
    lib.engram_strerror.restype = ctypes.c_char_p
    lib.engram_strerror.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


class EngramError(RuntimeError):
    pass


def _check(rc, what):
    if rc != ENGRAM_OK:
        raise EngramError("%s: %s (%d)" % (what, load_library().engram_strerror(rc).decode(), rc))


def _stream_handle(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev_ptr(t, name, dtype=None, numel=None, min_numel=None, shape=None):
    """Device address of a contiguous GPU tensor, after checking what the C call
    will assume of it: dtype, exact element count or shape, or a lower bound on
    the element count (a buffer the kernels fill only in part).  A mismatch
    raises ValueError before anything is enqueued: an undersized buffer would
    otherwise become an out-of-bounds device access."""
    if t is None:
        return None
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if numel is not None and t.numel() != numel:
        raise ValueError("%s must hold %d elements, got %d" % (name, numel, t.numel()))
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError("%s must hold at least %d elements, got %d" % (name, min_numel, t.numel()))
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return ctypes.c_void_p(t.data_ptr())


def _status_ptr(status):
    return _dev_ptr(status, "status", torch.int64, numel=1)


def _dtype_code(t):
    if t.dtype == torch.float32:
        return ENGRAM_F32
    if t.dtype == torch.bfloat16:
        return ENGRAM_BF16
    raise ValueError("table and gradients must be float32 or bfloat16, got %s" % t.dtype)


def _raise_on_status(status, what, rows):
    bad = int(status.item())
    if bad >= 0:
        raise EngramError("%s: row id %d at lookup %d is outside the owned range" %
                          (what, int(rows.reshape(-1)[bad].item()), bad))


def engram_hash(tokens, spec, rows_out=None, stream=None):
    """tokens: int64 [batch, seq] on the GPU -> int64 [batch, seq, H] global rows."""
    lib = load_library()
    if tokens.dim() != 2:
        raise ValueError("tokens must be [batch, seq]")
    batch, seq = tokens.shape
    if rows_out is None:
        rows_out = torch.empty((batch, seq, spec.num_heads), dtype=torch.int64, device=tokens.device)
    _check(lib.engram_hash(_dev_ptr(tokens, "tokens", torch.int64), batch, seq, ctypes.byref(spec),
                           _dev_ptr(rows_out, "rows_out", torch.int64, numel=batch * seq * spec.num_heads),
                           _stream_handle(stream)), "engram_hash")
    return rows_out


def engram_hash_slice(tokens, seq_begin, seq_end, spec, rows_out=None, stream=None):
    """Rows of positions [seq_begin, seq_end) of every batch row, hashed with the full history."""
    lib = load_library()
    if tokens.dim() != 2:
        raise ValueError("tokens must be [batch, seq]")
    batch, seq = tokens.shape
    if rows_out is None:
        rows_out = torch.empty((batch, max(seq_end - seq_begin, 0), spec.num_heads), dtype=torch.int64,
                               device=tokens.device)
    width = max(seq_end - seq_begin, 0)
    _check(lib.engram_hash_slice(_dev_ptr(tokens, "tokens", torch.int64), batch, seq, seq_begin, seq_end,
                                 ctypes.byref(spec),
                                 _dev_ptr(rows_out, "rows_out", torch.int64, numel=batch * width * spec.num_heads),
                                 _stream_handle(stream)), "engram_hash_slice")
    return rows_out


def engram_gather(table, rows, row_begin=0, out=None, status=None, validate=True, stream=None):
    """table: [num_rows, dim] (fp32/bf16) holding global rows [row_begin, row_begin+num_rows);
    rows: int64 [...] -> out [..., dim].  With ``validate`` the call synchronises and
    raises on an out-of-range row (the output row is zero in any case)."""
    lib = load_library()
    if table.dim() != 2:
        raise ValueError("table must be [num_rows, dim]")
    num_rows, dim = table.shape
    n = rows.numel()
    if out is None:
        out = torch.empty(tuple(rows.shape) + (dim,), dtype=table.dtype, device=table.device)
    if validate and status is None:
        status = torch.empty((), dtype=torch.int64, device=table.device)
    _check(lib.engram_gather(_dev_ptr(table, "table", table.dtype), _dtype_code(table), row_begin, num_rows, dim,
                             _dev_ptr(rows, "rows", torch.int64), n, _dev_ptr(out, "out", table.dtype, numel=n * dim),
                             _status_ptr(status), _stream_handle(stream)), "engram_gather")
    if validate:
        _raise_on_status(status, "engram_gather", rows)
    return out


def engram_hash_gather(tokens, spec, table, row_begin=0, out=None, rows_out=None, status=None, validate=True,
                       stream=None):
    """Forward in one call: engram_hash of tokens int64 [batch, seq] then engram_gather
    of every position's H rows -> out [batch, seq, H, dim].  ``rows_out`` (int64
    [batch, seq, H]) also receives the hashed rows; it may be None for the released
    layout with a 160-wide bf16 table, where one kernel does both.  With
    ``validate`` the call synchronises and raises on a row outside the table's shard."""
    lib = load_library()
    if tokens.dim() != 2:
        raise ValueError("tokens must be [batch, seq]")
    if table.dim() != 2:
        raise ValueError("table must be [num_rows, dim]")
    batch, seq = tokens.shape
    num_rows, dim = table.shape
    heads = spec.num_heads
    if out is None:
        out = torch.empty((batch, seq, heads, dim), dtype=table.dtype, device=table.device)
    if validate and status is None:
        status = torch.empty((), dtype=torch.int64, device=table.device)
    _check(lib.engram_hash_gather(_dev_ptr(tokens, "tokens", torch.int64), batch, seq, ctypes.byref(spec),
                                  _dev_ptr(table, "table", table.dtype), _dtype_code(table), row_begin, num_rows, dim,
                                  _dev_ptr(out, "out", table.dtype, numel=batch * seq * heads * dim),
                                  _dev_ptr(rows_out, "rows_out", torch.int64, numel=batch * seq * heads),
                                  _status_ptr(status), _stream_handle(stream)), "engram_hash_gather")
    if validate:
        bad = int(status.item())
        if bad >= 0:
            raise EngramError("engram_hash_gather: the row of lookup %d (position %d, head %d) is outside the owned "
                              "range" % (bad, bad // heads, bad % heads))
    return out


def engram_hash_gather_slice(tokens, spec, table, seq_begin, seq_end, row_begin=0, out=None, rows_out=None,
                             status=None, validate=True, stream=None):
    """engram_hash_gather for columns [seq_begin, seq_end) of tokens int64 [batch, seq],
    hashed with the tokens before them -> out [batch, seq_end - seq_begin, H, dim]."""
    lib = load_library()
    if tokens.dim() != 2 or table.dim() != 2:
        raise ValueError("tokens must be [batch, seq] and table [num_rows, dim]")
    batch, seq = tokens.shape
    num_rows, dim = table.shape
    heads = spec.num_heads
    width = max(0, seq_end - seq_begin)
    if out is None:
        out = torch.empty((batch, width, heads, dim), dtype=table.dtype, device=table.device)
    if validate and status is None:
        status = torch.empty((), dtype=torch.int64, device=table.device)
    _check(lib.engram_hash_gather_slice(_dev_ptr(tokens, "tokens", torch.int64), batch, seq, seq_begin, seq_end,
                                        ctypes.byref(spec), _dev_ptr(table, "table", table.dtype), _dtype_code(table),
                                        row_begin, num_rows, dim,
                                        _dev_ptr(out, "out", table.dtype, numel=batch * width * heads * dim),
                                        _dev_ptr(rows_out, "rows_out", torch.int64, numel=batch * width * heads),
                                        _status_ptr(status), _stream_handle(stream)), "engram_hash_gather_slice")
    if validate:
        bad = int(status.item())
        if bad >= 0:
            raise EngramError("engram_hash_gather_slice: the row of lookup %d (slice position %d, head %d) is "
                              "outside the owned range" % (bad, bad // heads, bad % heads))
    return out


def engram_scatter_add_workspace(n, num_rows, dim):
    return int(load_library().engram_scatter_add_workspace(n, num_rows, dim))


def engram_scatter_add(rows, grad_out, num_rows, row_begin=0, grad_dense=None, compact=None, workspace=None,
                       status=None, validate=True, stream=None):
    """Backward of engram_gather.

    Dense form: pass ``grad_dense`` fp32 [num_rows, dim]; it is updated in place and returned.
    Compact form (default): returns (uniq_rows int64 [U], uniq_grad fp32 [U, dim]); pass
    ``compact=(uniq_rows [n], uniq_grad [n, dim], num_uniq [])`` to reuse buffers, in which
    case the full buffers and the device count are returned without synchronising."""
    lib = load_library()
    dim = grad_out.shape[-1]
    n = rows.numel()
    dev = grad_out.device
    if grad_out.numel() != n * dim:
        raise ValueError("grad_out must hold one row per lookup")
    if workspace is None:
        workspace = torch.empty(engram_scatter_add_workspace(n, num_rows, dim), dtype=torch.uint8, device=dev)
    if validate and status is None:
        status = torch.empty((), dtype=torch.int64, device=dev)
    own_compact = grad_dense is None and compact is None
    if own_compact:
        compact = (torch.empty(max(n, 1), dtype=torch.int64, device=dev),
                   torch.empty((max(n, 1), dim), dtype=torch.float32, device=dev),
                   torch.empty((), dtype=torch.int64, device=dev))
    ur, ug, nu = compact if compact is not None else (None, None, None)
    rc = lib.engram_scatter_add(_dev_ptr(rows, "rows", torch.int64), n, _dev_ptr(grad_out, "grad_out"),
                                _dtype_code(grad_out), dim, row_begin, num_rows,
                                _dev_ptr(grad_dense, "grad_dense", torch.float32, shape=(num_rows, dim)),
                                _dev_ptr(ur, "uniq_rows", torch.int64, min_numel=n),
                                _dev_ptr(ug, "uniq_grad", torch.float32, min_numel=n * dim),
                                _dev_ptr(nu, "num_uniq", torch.int64, numel=1), _dev_ptr(workspace, "workspace"),
                                workspace.numel() * workspace.element_size(), _status_ptr(status),
                                _stream_handle(stream))
    _check(rc, "engram_scatter_add")
    if validate:
        _raise_on_status(status, "engram_scatter_add", rows)
    if grad_dense is not None:
        return grad_dense
    if own_compact:
        u = int(nu.item())
        return ur[:u], ug[:u]
    return ur, ug, nu


NOALLOC_SCRATCH_BYTES = 64 << 20


def engram_scatter_add_noalloc(rows, grad_out, num_rows, row_begin=0, grad_dense=None, compact=None, status=None,
                               stream=None):
    """engram_scatter_add on the library's fixed scratch array: allocates nothing.
    Exactly one output form: ``grad_dense`` fp32 [num_rows, dim] (updated in place),
    or ``compact=(uniq_rows [>= n], uniq_grad [>= n, dim], num_uniq [])``; both are
    returned as given.  Raises EngramError when n lookups need more than the 64 MiB
    scratch.  Calls that overlap on one GPU race."""
    lib = load_library()
    dim = grad_out.shape[-1]
    n = rows.numel()
    if grad_out.numel() != n * dim:
        raise ValueError("grad_out must hold one row per lookup")
    ur, ug, nu = compact if compact is not None else (None, None, None)
    _check(lib.engram_scatter_add_noalloc(_dev_ptr(rows, "rows", torch.int64), n, _dev_ptr(grad_out, "grad_out"),
                                          _dtype_code(grad_out), dim, row_begin, num_rows,
                                          _dev_ptr(grad_dense, "grad_dense", torch.float32, shape=(num_rows, dim)),
                                          _dev_ptr(ur, "uniq_rows", torch.int64, min_numel=n),
                                          _dev_ptr(ug, "uniq_grad", torch.float32, min_numel=n * dim),
                                          _dev_ptr(nu, "num_uniq", torch.int64, numel=1), _status_ptr(status),
                                          _stream_handle(stream)), "engram_scatter_add_noalloc")
    return grad_dense if grad_dense is not None else compact


def engram_scatter_add_plan(rows, num_rows, dim, row_begin=0, workspace=None, uniq_rows=None, num_uniq=None,
                            status=None, stream=None):
    """Phase 1 of engram_scatter_add: sort the lookups by row into ``workspace``.
    Returns the workspace (allocated when not given)."""
    lib = load_library()
    n = rows.numel()
    if workspace is None:
        workspace = torch.empty(engram_scatter_add_workspace(n, num_rows, dim), dtype=torch.uint8, device=rows.device)
    _check(lib.engram_scatter_add_plan(_dev_ptr(rows, "rows", torch.int64), n, row_begin, num_rows, dim,
                                       _dev_ptr(uniq_rows, "uniq_rows", torch.int64, min_numel=n),
                                       _dev_ptr(num_uniq, "num_uniq", torch.int64, numel=1),
                                       _dev_ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                                       _status_ptr(status), _stream_handle(stream)),
           "engram_scatter_add_plan")
    # What the plan in this workspace was made for; apply refuses other sizes.
    workspace._engram_plan = (n, num_rows, dim, row_begin)
    return workspace


def engram_scatter_add_plan_padded(ids, split_sizes, num_rows, dim, row_begin=0, workspace=None, uniq_rows=None,
                                   num_uniq=None, status=None, stream=None):
    """engram_scatter_add_plan for received padded ID blocks ids int64 [world, capacity]
    (block w's first split_sizes[w] entries are IDs, the rest padding).  Returns the
    workspace; apply with n = world * capacity and the padded gradient blocks."""
    lib = load_library()
    if ids.dim() != 2:
        raise ValueError("ids must be [world, capacity]")
    world, capacity = ids.shape
    n = world * capacity
    if workspace is None:
        workspace = torch.empty(engram_scatter_add_workspace(n, num_rows, dim), dtype=torch.uint8, device=ids.device)
    _check(lib.engram_scatter_add_plan_padded(_dev_ptr(ids, "ids", torch.int64),
                                              _dev_ptr(split_sizes, "split_sizes", torch.int64, numel=world), world,
                                              capacity, row_begin, num_rows, dim,
                                              _dev_ptr(uniq_rows, "uniq_rows", torch.int64, min_numel=n),
                                              _dev_ptr(num_uniq, "num_uniq", torch.int64, numel=1),
                                              _dev_ptr(workspace, "workspace"),
                                              workspace.numel() * workspace.element_size(), _status_ptr(status),
                                              _stream_handle(stream)),
           "engram_scatter_add_plan_padded")
    workspace._engram_plan = (n, num_rows, dim, row_begin)
    return workspace


def engram_scatter_add_plan_from_tokens(tokens, spec, num_rows, dim, row_begin=0, workspace=None, uniq_rows=None,
                                        num_uniq=None, status=None, stream=None):
    """engram_scatter_add_plan for the rows engram_hash(tokens, spec) would give,
    hashed inside the plan (released head layout only: 16 rows per position).
    Returns the workspace; apply with n = tokens.numel() * 16."""
    lib = load_library()
    if tokens.dim() != 2:
        raise ValueError("tokens must be [batch, seq]")
    batch, seq = tokens.shape
    n = batch * seq * spec.num_heads
    if workspace is None:
        workspace = torch.empty(engram_scatter_add_workspace(n, num_rows, dim), dtype=torch.uint8,
                                device=tokens.device)
    _check(lib.engram_scatter_add_plan_from_tokens(_dev_ptr(tokens, "tokens", torch.int64), batch, seq,
                                                   ctypes.byref(spec), row_begin, num_rows, dim,
                                                   _dev_ptr(uniq_rows, "uniq_rows", torch.int64, min_numel=n),
                                                   _dev_ptr(num_uniq, "num_uniq", torch.int64, numel=1),
                                                   _dev_ptr(workspace, "workspace"),
                                                   workspace.numel() * workspace.element_size(), _status_ptr(status),
                                                   _stream_handle(stream)),
           "engram_scatter_add_plan_from_tokens")
    workspace._engram_plan = (n, num_rows, dim, row_begin)
    return workspace


def engram_scatter_add_plan_from_tokens_slice(tokens, spec, seq_begin, seq_end, num_rows, dim, row_begin=0,
                                              workspace=None, uniq_rows=None, num_uniq=None, status=None,
                                              stream=None):
    """engram_scatter_add_plan_from_tokens for columns [seq_begin, seq_end) of every
    batch row, the columns before seq_begin read as history: the rows
    engram_hash_slice would give.  Returns the workspace; apply with
    n = batch * (seq_end - seq_begin) * 16."""
    lib = load_library()
    if tokens.dim() != 2:
        raise ValueError("tokens must be [batch, seq]")
    batch, seq = tokens.shape
    if not 0 <= seq_begin <= seq_end <= seq:
        raise ValueError("need 0 <= seq_begin <= seq_end <= seq_len")
    n = batch * (seq_end - seq_begin) * spec.num_heads
    if workspace is None:
        workspace = torch.empty(engram_scatter_add_workspace(n, num_rows, dim), dtype=torch.uint8,
                                device=tokens.device)
    _check(lib.engram_scatter_add_plan_from_tokens_slice(_dev_ptr(tokens, "tokens", torch.int64), batch, seq,
                                                         seq_begin, seq_end, ctypes.byref(spec), row_begin,
                                                         num_rows, dim,
                                                         _dev_ptr(uniq_rows, "uniq_rows", torch.int64, min_numel=n),
                                                         _dev_ptr(num_uniq, "num_uniq", torch.int64, numel=1),
                                                         _dev_ptr(workspace, "workspace"),
                                                         workspace.numel() * workspace.element_size(),
                                                         _status_ptr(status), _stream_handle(stream)),
           "engram_scatter_add_plan_from_tokens_slice")
    workspace._engram_plan = (n, num_rows, dim, row_begin)
    return workspace


def engram_scatter_add_apply(grad_out, n, num_rows, workspace, row_begin=0, grad_dense=None, uniq_grad=None,
                             stream=None):
    """Phase 2: per-row sums of ``grad_out`` along the plan in ``workspace`` (dense or compact)."""
    lib = load_library()
    dim = grad_out.shape[-1]
    made_for = getattr(workspace, "_engram_plan", None)
    if made_for is not None and made_for != (n, num_rows, dim, row_begin):
        raise ValueError("workspace holds a plan for (n, num_rows, dim, row_begin) = %s, not %s"
                         % (made_for, (n, num_rows, dim, row_begin)))
    _check(lib.engram_scatter_add_apply(_dev_ptr(grad_out, "grad_out", numel=n * dim), _dtype_code(grad_out), dim, n,
                                        row_begin, num_rows,
                                        _dev_ptr(grad_dense, "grad_dense", torch.float32, shape=(num_rows, dim)),
                                        _dev_ptr(uniq_grad, "uniq_grad", torch.float32, min_numel=n * dim),
                                        _dev_ptr(workspace, "workspace"),
                                        workspace.numel() * workspace.element_size(), _stream_handle(stream)),
           "engram_scatter_add_apply")
    return grad_dense if grad_dense is not None else uniq_grad


# ---------------------------------------------------------------- owner routing

def _bind_route(lib):
    if getattr(lib, "_route_bound", False):
        return
    p, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    lib.engram_route_workspace.restype = sz
    lib.engram_route_workspace.argtypes = [i64]
    lib.engram_route_plan.restype = ctypes.c_int
    lib.engram_route_plan.argtypes = [p, i64, i64, i32, p, p, p, p, sz, p, p]
    lib.engram_route_validate.restype = ctypes.c_int
    lib.engram_route_validate.argtypes = [p, i64, p, i32, i64, p, p]
    lib.engram_pack_fixed_capacity.restype = ctypes.c_int
    lib.engram_pack_fixed_capacity.argtypes = [p, i64, i64, p, i32, i64, p, i32, p, p, p]
    lib.engram_unpack_fixed_capacity.restype = ctypes.c_int
    lib.engram_unpack_fixed_capacity.argtypes = [p, i64, p, i32, i64, p, i64, p, p]
    lib.engram_permute_rows.restype = ctypes.c_int
    lib.engram_permute_rows.argtypes = [p, i64, p, i64, p, p]
    lib.engram_unpermute_rows.restype = ctypes.c_int
    lib.engram_unpermute_rows.argtypes = [p, i64, p, i64, p, p]
    lib.engram_unpack_unpermute_rows.restype = ctypes.c_int
    lib.engram_unpack_unpermute_rows.argtypes = [p, i64, p, i32, i64, p, i64, p, p, p]
    lib.engram_permute_pack_rows.restype = ctypes.c_int
    lib.engram_permute_pack_rows.argtypes = [p, i64, p, i64, p, i32, i64, p, i32, p, p, p]
    lib.engram_gather_padded.restype = ctypes.c_int
    lib.engram_gather_padded.argtypes = [p, i32, i64, i64, i32, p, p, i32, i64, p, p, p]
    lib._route_bound = True


def _route_lib():
    lib = load_library()
    _bind_route(lib)
    return lib


def _row_bytes(t):
    return (t.numel() // max(t.shape[0], 1)) * t.element_size() if t.dim() > 1 else t.element_size()


def engram_route_plan(global_ids, num_embeddings, world, status=None, workspace=None, out=None, stream=None):
    """Group global row IDs by owner.  Returns (sorted_ids [n], order [n], send_counts [world]);
    ``out`` may supply those three buffers."""
    lib = _route_lib()
    ids = global_ids.reshape(-1)
    n = ids.numel()
    dev = ids.device
    if out is not None:
        sorted_ids, order, counts = out
    else:
        sorted_ids = torch.empty(n, dtype=torch.int64, device=dev)
        order = torch.empty(n, dtype=torch.int64, device=dev)
        counts = torch.empty(world, dtype=torch.int64, device=dev)
    ws = workspace if workspace is not None else \
        torch.empty(max(int(lib.engram_route_workspace(n)), 256), dtype=torch.uint8, device=dev)
    _check(lib.engram_route_plan(_dev_ptr(ids, "global_ids", torch.int64), n, num_embeddings, world,
                                 _dev_ptr(sorted_ids, "sorted_ids", torch.int64, numel=n),
                                 _dev_ptr(order, "order", torch.int64, numel=n),
                                 _dev_ptr(counts, "send_counts", torch.int64, numel=world),
                                 _dev_ptr(ws, "workspace"), ws.numel() * ws.element_size(), _status_ptr(status),
                                 _stream_handle(stream)), "engram_route_plan")
    return sorted_ids, order, counts


def engram_route_validate(sorted_ids, send_counts, num_embeddings, world, stream=None):
    """Returns the device status word (lowest offending sorted index, n for bad counts, or -1)."""
    lib = _route_lib()
    status = torch.empty((), dtype=torch.int64, device=sorted_ids.device)
    _check(lib.engram_route_validate(_dev_ptr(sorted_ids, "sorted_ids", torch.int64), sorted_ids.numel(),
                                     _dev_ptr(send_counts, "send_counts", torch.int64, numel=world), world,
                                     num_embeddings,
                                     _dev_ptr(status, "status"), _stream_handle(stream)), "engram_route_validate")
    return status


def engram_pack_fixed_capacity(src, split_sizes, world, capacity, fill=0, status=None, out=None, stream=None):
    """Compact rows src [src_rows, ...] -> [world, capacity, ...] padded with ``fill``;
    segment rows past src's src_rows = src.shape[0] rows are never read (fill, status world)."""
    lib = _route_lib()
    row_shape = tuple(src.shape[1:])
    esize = src.element_size()
    row_bytes = esize * int(torch.Size(row_shape).numel()) if row_shape else esize
    dst = torch.empty((world, capacity) + row_shape, dtype=src.dtype, device=src.device) if out is None else out
    fill_t = torch.tensor([fill], dtype=src.dtype)
    fill_bytes = (ctypes.c_ubyte * esize).from_buffer_copy(fill_t.view(torch.uint8).numpy().tobytes())
    _check(lib.engram_pack_fixed_capacity(_dev_ptr(src, "src"), src.shape[0] if src.dim() else 0, row_bytes,
                                          _dev_ptr(split_sizes, "split_sizes", torch.int64, numel=world), world,
                                          capacity, ctypes.cast(fill_bytes, ctypes.c_void_p), esize,
                                          _dev_ptr(dst, "dst", src.dtype, shape=(world, capacity) + row_shape),
                                          _status_ptr(status), _stream_handle(stream)),
           "engram_pack_fixed_capacity")
    return dst


def engram_unpack_fixed_capacity(src, split_sizes, dst_rows, status=None, out=None, stream=None):
    """[world, capacity, ...] -> compact [dst_rows, ...] (rank order; rows past the counts untouched)."""
    lib = _route_lib()
    world, capacity = src.shape[0], src.shape[1]
    row_shape = tuple(src.shape[2:])
    esize = src.element_size()
    row_bytes = esize * int(torch.Size(row_shape).numel()) if row_shape else esize
    dst = torch.empty((dst_rows,) + row_shape, dtype=src.dtype, device=src.device) if out is None else out
    _check(lib.engram_unpack_fixed_capacity(_dev_ptr(src, "src"), row_bytes,
                                            _dev_ptr(split_sizes, "split_sizes", torch.int64, numel=world), world,
                                            capacity,
                                            _dev_ptr(dst, "dst", src.dtype, min_numel=dst_rows * (row_bytes // esize)),
                                            dst_rows, _status_ptr(status), _stream_handle(stream)),
           "engram_unpack_fixed_capacity")
    return dst


def engram_gather_padded(table, ids, split_sizes, row_begin=0, out=None, status=None, validate=True, stream=None):
    """The owner's lookup on received padded ID blocks ids int64 [world, capacity]
    (block w's first split_sizes[w] entries are IDs) -> values [world, capacity, dim],
    padding rows zero.  With ``validate`` the call synchronises and raises on an ID
    outside the table's rows."""
    lib = _route_lib()
    if table.dim() != 2 or ids.dim() != 2:
        raise ValueError("table must be [num_rows, dim] and ids [world, capacity]")
    num_rows, dim = table.shape
    world, capacity = ids.shape
    if out is None:
        out = torch.empty((world, capacity, dim), dtype=table.dtype, device=table.device)
    if validate and status is None:
        status = torch.empty((), dtype=torch.int64, device=table.device)
    _check(lib.engram_gather_padded(_dev_ptr(table, "table", table.dtype), _dtype_code(table), row_begin, num_rows,
                                    dim, _dev_ptr(ids, "ids", torch.int64),
                                    _dev_ptr(split_sizes, "split_sizes", torch.int64, numel=world), world, capacity,
                                    _dev_ptr(out, "out", table.dtype, shape=(world, capacity, dim)),
                                    _status_ptr(status), _stream_handle(stream)), "engram_gather_padded")
    if validate:
        _raise_on_status(status, "engram_gather_padded", ids)
    return out


def engram_permute_pack_rows(src, order, split_sizes, world, capacity, fill=0, status=None, out=None, stream=None):
    """Rows src [n, ...] in request order -> [world, capacity, ...]: grouped row k is
    src[order[k]], packed as engram_pack_fixed_capacity packs; n = order.numel()."""
    lib = _route_lib()
    row_shape = tuple(src.shape[1:])
    esize = src.element_size()
    row_elems = int(torch.Size(row_shape).numel()) if row_shape else 1
    row_bytes = esize * row_elems
    n = order.numel()
    dst = torch.empty((world, capacity) + row_shape, dtype=src.dtype, device=src.device) if out is None else out
    fill_t = torch.tensor([fill], dtype=src.dtype)
    fill_bytes = (ctypes.c_ubyte * esize).from_buffer_copy(fill_t.view(torch.uint8).numpy().tobytes())
    _check(lib.engram_permute_pack_rows(_dev_ptr(src, "src", min_numel=n * row_elems), row_bytes,
                                        _dev_ptr(order, "order", torch.int64), n,
                                        _dev_ptr(split_sizes, "split_sizes", torch.int64, numel=world), world,
                                        capacity, ctypes.cast(fill_bytes, ctypes.c_void_p), esize,
                                        _dev_ptr(dst, "dst", src.dtype, shape=(world, capacity) + row_shape),
                                        _status_ptr(status), _stream_handle(stream)),
           "engram_permute_pack_rows")
    return dst


def engram_unpack_unpermute_rows(src, split_sizes, order, status=None, out=None, stream=None):
    """[world, capacity, ...] -> [n, ...] in request order: compact row k (rank
    order, as engram_unpack_fixed_capacity) lands in row order[k]; n = order.numel()."""
    lib = _route_lib()
    world, capacity = src.shape[0], src.shape[1]
    row_shape = tuple(src.shape[2:])
    esize = src.element_size()
    row_bytes = esize * int(torch.Size(row_shape).numel()) if row_shape else esize
    n = order.numel()
    dst = torch.empty((n,) + row_shape, dtype=src.dtype, device=src.device) if out is None else out
    _check(lib.engram_unpack_unpermute_rows(_dev_ptr(src, "src"), row_bytes,
                                            _dev_ptr(split_sizes, "split_sizes", torch.int64, numel=world), world,
                                            capacity, _dev_ptr(order, "order", torch.int64), n,
                                            _dev_ptr(dst, "dst", src.dtype, min_numel=n * (row_bytes // esize)),
                                            _status_ptr(status), _stream_handle(stream)),
           "engram_unpack_unpermute_rows")
    return dst


def _permute(src, order, gather, stream, out=None):
    lib = _route_lib()
    n = order.numel()
    row_elems = int(torch.Size(src.shape[1:]).numel()) if src.dim() > 1 else 1
    row_bytes = row_elems * src.element_size()
    dst = torch.empty_like(src) if out is None else out
    fn = lib.engram_permute_rows if gather else lib.engram_unpermute_rows
    # order indexes n rows of src and n rows of dst
    _check(fn(_dev_ptr(src, "src", min_numel=n * row_elems), row_bytes, _dev_ptr(order, "order", torch.int64), n,
              _dev_ptr(dst, "dst", src.dtype, min_numel=n * row_elems), _stream_handle(stream)),
           "engram_permute_rows" if gather else "engram_unpermute_rows")
    return dst


def engram_permute_rows(src, order, out=None, stream=None):
    """dst[i] = src[order[i]]."""
    return _permute(src, order, True, stream, out)


def engram_unpermute_rows(src, order, out=None, stream=None):
    """dst[order[i]] = src[i]."""
    return _permute(src, order, False, stream, out)


# ---- PLE short convolution and grouped RMSNorm --------------------------------

def _bind_ple(lib):
    if getattr(lib, "_ple_bound", False):
        return
    p, i64, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    lib.engram_short_conv_workspace.restype = sz
    lib.engram_short_conv_workspace.argtypes = [i64, i64, i64, i32]
    lib.engram_short_conv.restype = ctypes.c_int
    lib.engram_short_conv.argtypes = [p, i32, i64, i64, i64, p, p, i32, i32, p, p, p]
    lib.engram_short_conv_backward.restype = ctypes.c_int
    lib.engram_short_conv_backward.argtypes = [p, p, i32, i64, i64, i64, p, i32, i32, p, p, p, p, p, p, sz, p]
    lib.engram_grouped_rms_norm_workspace.restype = sz
    lib.engram_grouped_rms_norm_workspace.argtypes = [i64, i64]
    lib.engram_grouped_rms_norm.restype = ctypes.c_int
    lib.engram_grouped_rms_norm.argtypes = [p, i32, i64, i64, i64, p, f32, p, p]
    lib.engram_grouped_rms_norm_backward.restype = ctypes.c_int
    lib.engram_grouped_rms_norm_backward.argtypes = [p, p, i32, i64, i64, i64, p, f32, p, p, p, sz, p]
    lib._ple_bound = True


def _ple_lib():
    lib = load_library()
    _bind_ple(lib)
    return lib


def _workspace(nbytes, device):
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def engram_short_conv(x, weight, bias=None, dilation=3, halo=None, out=None, stream=None):
    """Causal depthwise convolution of x [batch, seq, channels]; weight fp32 [channels, K]."""
    lib = _ple_lib()
    B, S, C = x.shape
    if weight.dim() != 2 or weight.shape[0] != C:
        raise ValueError("weight must be [channels, K]")
    K = weight.shape[1]
    y = torch.empty_like(x) if out is None else out
    _check(lib.engram_short_conv(_dev_ptr(x, "x"), _dtype_code(x), B, S, C,
                                 _dev_ptr(weight, "weight", torch.float32),
                                 _dev_ptr(bias, "bias", torch.float32, shape=(C,)), K, dilation,
                                 _dev_ptr(halo, "halo", x.dtype, shape=(B, (K - 1) * dilation, C)),
                                 _dev_ptr(y, "y", x.dtype, shape=(B, S, C)), _stream_handle(stream)),
           "engram_short_conv")
    return y


def engram_short_conv_backward(x, dy, weight, dilation=3, halo=None, want_bias=True, want_halo=False,
                               workspace=None, out=None, stream=None):
    """Returns (dx, dweight, dbias or None, dhalo or None); ``out`` may supply
    that tuple's buffers (then want_bias / want_halo follow its entries)."""
    lib = _ple_lib()
    B, S, C = x.shape
    if weight.dim() != 2 or weight.shape[0] != C:
        raise ValueError("weight must be [channels, K]")
    K = weight.shape[1]
    dev = x.device
    if out is not None:
        dx, dw, db, dhalo = out
    else:
        dx = torch.empty_like(x)
        dw = torch.empty((C, K), dtype=torch.float32, device=dev)
        db = torch.empty(C, dtype=torch.float32, device=dev) if want_bias else None
        dhalo = torch.empty((B, (K - 1) * dilation, C), dtype=x.dtype, device=dev) if want_halo else None
    if workspace is None:
        workspace = _workspace(lib.engram_short_conv_workspace(B, S, C, K), dev)
    hshape = (B, (K - 1) * dilation, C)
    _check(lib.engram_short_conv_backward(_dev_ptr(x, "x"), _dev_ptr(dy, "dy", x.dtype, shape=(B, S, C)),
                                          _dtype_code(x), B, S, C, _dev_ptr(weight, "weight", torch.float32), K,
                                          dilation, _dev_ptr(halo, "halo", x.dtype, shape=hshape),
                                          _dev_ptr(dx, "dx", x.dtype, shape=(B, S, C)),
                                          _dev_ptr(dw, "dw", torch.float32, shape=(C, K)),
                                          _dev_ptr(db, "db", torch.float32, shape=(C,)),
                                          _dev_ptr(dhalo, "dhalo", x.dtype, shape=hshape),
                                          _dev_ptr(workspace, "workspace"), workspace.numel(),
                                          _stream_handle(stream)), "engram_short_conv_backward")
    return dx, dw, db, dhalo


def engram_grouped_rms_norm(x, weight, group_size, eps=1e-6, out=None, stream=None):
    """Grouped Gemma RMSNorm over the last dim of x; weight fp32 [hidden]."""
    lib = _ple_lib()
    hidden = x.shape[-1]
    rows = x.numel() // hidden if hidden else 0
    y = torch.empty_like(x) if out is None else out
    _check(lib.engram_grouped_rms_norm(_dev_ptr(x, "x"), _dtype_code(x), rows, hidden, group_size,
                                       _dev_ptr(weight, "weight", torch.float32, shape=(hidden,)), eps,
                                       _dev_ptr(y, "y", x.dtype, shape=tuple(x.shape)), _stream_handle(stream)),
           "engram_grouped_rms_norm")
    return y


def engram_grouped_rms_norm_backward(x, dy, weight, group_size, eps=1e-6, workspace=None, out=None, stream=None):
    """Returns (dx, dweight); ``out`` may supply those two buffers."""
    lib = _ple_lib()
    hidden = x.shape[-1]
    rows = x.numel() // hidden if hidden else 0
    if out is not None:
        dx, dw = out
    else:
        dx = torch.empty_like(x)
        dw = torch.empty(hidden, dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = _workspace(lib.engram_grouped_rms_norm_workspace(rows, hidden), x.device)
    _check(lib.engram_grouped_rms_norm_backward(_dev_ptr(x, "x"), _dev_ptr(dy, "dy", x.dtype, shape=tuple(x.shape)),
                                                _dtype_code(x), rows, hidden, group_size,
                                                _dev_ptr(weight, "weight", torch.float32, shape=(hidden,)), eps,
                                                _dev_ptr(dx, "dx", x.dtype, shape=tuple(x.shape)),
                                                _dev_ptr(dw, "dw", torch.float32, shape=(hidden,)),
                                                _dev_ptr(workspace, "workspace"), workspace.numel(),
                                                _stream_handle(stream)), "engram_grouped_rms_norm_backward")
    return dx, dw
