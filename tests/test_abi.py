"""The C-ABI library: it loads, exports every function include/engram.h declares,
and rejects bad host arguments before enqueuing anything.  No GPU is touched:
every call here fails host validation and returns before any HIP call."""
import ctypes
import os
import re

import pytest

import hashed_gram_embedding_engram_amd as E
from hashed_gram_embedding_engram_amd import engram as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from hashed_gram_embedding_engram_amd import build
        build.build()
    return B.load_library()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "engram.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(engram_[a-z_]+)\s*\(", text, re.M)))


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert {"engram_hash", "engram_hash_slice", "engram_gather", "engram_scatter_add",
            "engram_scatter_add_workspace", "engram_strerror"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_codes_match_header(lib):
    text = open(os.path.join(ROOT, "include", "engram.h")).read()
    for name, val in re.findall(r"(ENGRAM_E?[A-Z]+)\s*=\s*(-?\d+)", text):
        if hasattr(B, name):
            assert getattr(B, name) == int(val), name
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.engram_strerror(code) and lib.engram_strerror(code) != b"unknown engram status"
    assert lib.engram_strerror(-99) == b"unknown engram status"


def test_spec_struct_layout():
    # int32, int32, int64 x2, int64[8], int64[64], int64[64]
    assert ctypes.sizeof(B.EngramHashSpec) == 8 + 16 + 8 * 8 + 2 * 64 * 8


def test_hash_rejects_bad_spec(lib):
    s = E.qwen3_8_flash_next_spec()
    fake = ctypes.c_void_p(0x1000)       # never dereferenced: validation fails first
    for field, value, code in (("ngram_size", 1, B.ENGRAM_ESPEC), ("ngram_size", 9, B.ENGRAM_ESPEC),
                               ("heads_per_ngram", 0, B.ENGRAM_ESPEC), ("heads_per_ngram", 65, B.ENGRAM_ESPEC)):
        t = E.qwen3_8_flash_next_spec()
        setattr(t, field, value)
        assert lib.engram_hash(fake, 1, 4, ctypes.byref(t), fake, None) == code
    for h, m in ((3, 1), (0, 0), (15, -7), (2, (1 << 62) + 1)):
        t = E.qwen3_8_flash_next_spec()
        t.head_mod[h] = m
        assert lib.engram_hash(fake, 1, 4, ctypes.byref(t), fake, None) == B.ENGRAM_ESPEC
    t = E.qwen3_8_flash_next_spec()
    t.head_offset[5] = -1
    assert lib.engram_hash(fake, 1, 4, ctypes.byref(t), fake, None) == B.ENGRAM_ESPEC
    t = E.qwen3_8_flash_next_spec()
    t.head_offset[5] = (1 << 63) - 5
    assert lib.engram_hash(fake, 1, 4, ctypes.byref(t), fake, None) == B.ENGRAM_ESPEC
    assert lib.engram_hash(None, 1, 4, ctypes.byref(s), fake, None) == B.ENGRAM_EINVAL
    assert lib.engram_hash(fake, 1, 4, ctypes.byref(s), None, None) == B.ENGRAM_EINVAL
    assert lib.engram_hash(fake, -1, 4, ctypes.byref(s), fake, None) == B.ENGRAM_EINVAL
    assert lib.engram_hash(fake, 1, 4, None, fake, None) == B.ENGRAM_EINVAL
    assert lib.engram_hash_slice(fake, 1, 4, 3, 2, ctypes.byref(s), fake, None) == B.ENGRAM_EINVAL
    assert lib.engram_hash_slice(fake, 1, 4, 0, 5, ctypes.byref(s), fake, None) == B.ENGRAM_EINVAL
    assert lib.engram_hash_slice(fake, 1, 4, -1, 2, ctypes.byref(s), fake, None) == B.ENGRAM_EINVAL
    # empty work is a successful no-op, with or without pointers
    assert lib.engram_hash(None, 0, 4, ctypes.byref(s), None, None) == B.ENGRAM_OK
    assert lib.engram_hash_slice(None, 2, 4, 2, 2, ctypes.byref(s), None, None) == B.ENGRAM_OK


def test_gather_rejects_bad_arguments(lib):
    f = ctypes.c_void_p(0x1000)
    assert lib.engram_gather(f, 7, 0, 10, 160, f, 4, f, None, None) == B.ENGRAM_EDTYPE
    for dim in (0, -8, 100, 12, 1024):               # bytes not a multiple of 16, or above 1024
        assert lib.engram_gather(f, B.ENGRAM_BF16, 0, 10, dim, f, 4, f, None, None) == B.ENGRAM_EINVAL
    assert lib.engram_gather(f, B.ENGRAM_F32, 0, 10, 257, f, 4, f, None, None) == B.ENGRAM_EINVAL
    assert lib.engram_gather(None, B.ENGRAM_BF16, 0, 10, 160, f, 4, f, None, None) == B.ENGRAM_EINVAL
    assert lib.engram_gather(f, B.ENGRAM_BF16, 0, 10, 160, None, 4, f, None, None) == B.ENGRAM_EINVAL
    assert lib.engram_gather(f, B.ENGRAM_BF16, 0, 10, 160, f, 4, None, None, None) == B.ENGRAM_EINVAL
    assert lib.engram_gather(f, B.ENGRAM_BF16, -1, 10, 160, f, 4, f, None, None) == B.ENGRAM_EINVAL
    assert lib.engram_gather(f, B.ENGRAM_BF16, 0, -10, 160, f, 4, f, None, None) == B.ENGRAM_EINVAL
    assert lib.engram_gather(f, B.ENGRAM_BF16, 0, 10, 160, f, -4, f, None, None) == B.ENGRAM_EINVAL


def test_scatter_rejects_bad_arguments(lib):
    f = ctypes.c_void_p(0x1000)
    ws_ok = ctypes.c_void_p(0x100000)                # 256-aligned, never dereferenced
    n, R, D = 1000, 5000, 160
    need = lib.engram_scatter_add_workspace(n, R, D)
    assert need > 0

    def call(rows=f, nn=n, g=f, dt=B.ENGRAM_BF16, dim=D, rb=0, nr=R, dense=None, ur=f, ug=f, nu=f,
             ws=ws_ok, wsb=need):
        return lib.engram_scatter_add(rows, nn, g, dt, dim, rb, nr, dense, ur, ug, nu, ws, wsb, None, None)

    assert call(dt=3) == B.ENGRAM_EDTYPE
    assert call(dim=100) == B.ENGRAM_EINVAL
    assert call(nn=-1) == B.ENGRAM_EINVAL
    assert call(nn=1 << 31) == B.ENGRAM_EINVAL
    assert call(nr=0xFFFFFFFF) == B.ENGRAM_EINVAL
    assert call(rb=-1) == B.ENGRAM_EINVAL
    assert call(dense=f) == B.ENGRAM_EINVAL                       # both output forms
    assert call(ur=None, ug=None, nu=None) == B.ENGRAM_EINVAL     # neither
    assert call(nu=None) == B.ENGRAM_EINVAL                       # incomplete compact form
    assert call(rows=None) == B.ENGRAM_EINVAL
    assert call(g=None) == B.ENGRAM_EINVAL
    assert call(ws=None) == B.ENGRAM_EWORKSPACE
    assert call(wsb=need - 1) == B.ENGRAM_EWORKSPACE
    assert call(ws=ctypes.c_void_p(0x100010)) == B.ENGRAM_EWORKSPACE


def test_workspace_grows_with_n(lib):
    a = lib.engram_scatter_add_workspace(1 << 16, 320001536, 160)
    b = lib.engram_scatter_add_workspace(1 << 20, 320001536, 160)
    assert 0 < a < b
    # four 32-bit key/index arrays dominate: at least 16 bytes per lookup
    assert b >= 16 * (1 << 20)
    assert lib.engram_scatter_add_workspace(-1, 10, 160) == 0


def test_product_constants_match_oracle_derivation():
    """The binding's literal Qwen3.8-Flash-Next constants equal the oracle's derived ones."""
    from oracle import constants as C
    assert E.QWEN3_8_FLASH_NEXT_NGRAM_HEAD_VOCAB_SIZES == C.head_vocab_sizes()
    assert E.QWEN3_8_FLASH_NEXT_NGRAM_HEAD_OFFSETS == C.head_offsets()
    assert E.QWEN3_8_FLASH_NEXT_NGRAM_PADDED_ROWS == C.padded_rows()
    assert E.QWEN3_8_FLASH_NEXT_LAYER_MULTIPLIERS == C.LAYER_MULTIPLIERS
    assert E.QWEN3_8_FLASH_NEXT_EOS_TOKEN_ID == C.EOS_TOKEN_ID


def test_plan_apply_reject_bad_arguments(lib):
    f = ctypes.c_void_p(0x1000)
    ws = ctypes.c_void_p(0x100000)
    n, R, D = 1000, 5000, 160
    need = lib.engram_scatter_add_workspace(n, R, D)
    plan = lambda rows=f, nn=n, rb=0, nr=R, dim=D, w=ws, wb=need: lib.engram_scatter_add_plan(
        rows, nn, rb, nr, dim, None, None, w, wb, None, None)
    assert plan(rows=None) == B.ENGRAM_EINVAL
    assert plan(nn=-5) == B.ENGRAM_EINVAL
    assert plan(dim=6) == B.ENGRAM_EINVAL               # valid for neither element type
    assert plan(nr=-1) == B.ENGRAM_EINVAL
    assert plan(w=None) == B.ENGRAM_EWORKSPACE
    assert plan(wb=need - 1) == B.ENGRAM_EWORKSPACE
    apply = lambda g=f, dt=B.ENGRAM_BF16, dim=D, nn=n, dense=None, ug=f, w=ws, wb=need: lib.engram_scatter_add_apply(
        g, dt, dim, nn, 0, R, dense, ug, w, wb, None)
    assert apply(dt=9) == B.ENGRAM_EDTYPE
    assert apply(g=None) == B.ENGRAM_EINVAL
    assert apply(dense=f) == B.ENGRAM_EINVAL          # both forms
    assert apply(ug=None) == B.ENGRAM_EINVAL          # neither form
    assert apply(w=ctypes.c_void_p(0x100008)) == B.ENGRAM_EWORKSPACE


def test_route_entry_points_reject_bad_arguments(lib):
    from hashed_gram_embedding_engram_amd import engram as EB
    EB._bind_route(lib)
    f = ctypes.c_void_p(0x1000)
    ws = ctypes.c_void_p(0x100000)
    need = lib.engram_route_workspace(1000)
    plan = lambda E=8000, W=8, n=1000, w=ws, wb=need, ids=f: lib.engram_route_plan(
        ids, n, E, W, f, f, f, w, wb, None, None)
    assert plan(E=8001) == B.ENGRAM_EINVAL          # rows do not divide by the owner count
    assert plan(W=0) == B.ENGRAM_EINVAL
    assert plan(W=256, E=256000) == B.ENGRAM_EINVAL
    assert plan(n=-1) == B.ENGRAM_EINVAL
    assert plan(ids=None) == B.ENGRAM_EINVAL
    assert plan(w=None) == B.ENGRAM_EWORKSPACE
    assert plan(wb=need - 1) == B.ENGRAM_EWORKSPACE
    assert lib.engram_route_validate(f, 10, f, 8, 8000, None, None) == B.ENGRAM_EINVAL   # status required
    one = (ctypes.c_ubyte * 8)()
    pack = lambda rb=320, cap=16, fb=2, W=8, fill=ctypes.cast(one, ctypes.c_void_p), sr=100: \
        lib.engram_pack_fixed_capacity(f, sr, rb, f, W, cap, fill, fb, f, None, None)
    assert pack(rb=10) == B.ENGRAM_EINVAL            # rows are whole 4-byte words
    assert pack(fb=3) == B.ENGRAM_EINVAL
    assert pack(fb=8, rb=12) == B.ENGRAM_EINVAL       # the fill element must tile the row
    assert pack(cap=-1) == B.ENGRAM_EINVAL
    assert pack(fill=None) == B.ENGRAM_EINVAL
    assert pack(sr=-1) == B.ENGRAM_EINVAL
    assert lib.engram_unpack_fixed_capacity(f, 320, f, 8, 16, f, -1, None, None) == B.ENGRAM_EINVAL
    assert lib.engram_permute_rows(f, 6, f, 10, f, None) == B.ENGRAM_EINVAL
    assert lib.engram_unpermute_rows(None, 8, f, 10, f, None) == B.ENGRAM_EINVAL
    # (src, row_bytes, split_sizes, world, capacity, order, n, dst, status, stream)
    uu = lambda src=f, rb=320, cs=f, W=8, cap=16, order=f, n=100, dst=f: \
        lib.engram_unpack_unpermute_rows(src, rb, cs, W, cap, order, n, dst, None, None)
    assert uu(W=0) == B.ENGRAM_EINVAL and uu(W=256) == B.ENGRAM_EINVAL
    assert uu(cap=-1) == B.ENGRAM_EINVAL and uu(n=-1) == B.ENGRAM_EINVAL
    assert uu(rb=10) == B.ENGRAM_EINVAL                      # rows are whole 4-byte words
    assert uu(cs=None) == B.ENGRAM_EINVAL
    assert uu(order=None) == B.ENGRAM_EINVAL and uu(dst=None) == B.ENGRAM_EINVAL and uu(src=None) == B.ENGRAM_EINVAL
    assert uu(order=ctypes.c_void_p(0x1004)) == B.ENGRAM_EINVAL  # int64 order, 8-byte aligned
    # (src, row_bytes, order, n, split_sizes, world, capacity, fill, fill_bytes, dst, status, stream)
    pp = lambda src=f, rb=320, order=f, n=100, cs=f, W=8, cap=16, fill=ctypes.cast(one, ctypes.c_void_p), fb=2, dst=f: \
        lib.engram_permute_pack_rows(src, rb, order, n, cs, W, cap, fill, fb, dst, None, None)
    assert pp(W=0) == B.ENGRAM_EINVAL and pp(cap=-1) == B.ENGRAM_EINVAL and pp(n=-1) == B.ENGRAM_EINVAL
    assert pp(rb=10) == B.ENGRAM_EINVAL and pp(fb=3) == B.ENGRAM_EINVAL and pp(fb=8, rb=12) == B.ENGRAM_EINVAL
    assert pp(fill=None) == B.ENGRAM_EINVAL and pp(cs=None) == B.ENGRAM_EINVAL
    assert pp(order=None) == B.ENGRAM_EINVAL and pp(src=None) == B.ENGRAM_EINVAL and pp(dst=None) == B.ENGRAM_EINVAL
    # (table, dtype, row_begin, num_rows, dim, ids, split_sizes, world, capacity, out, status, stream)
    gp = lambda table=f, dt=B.ENGRAM_BF16, rb=0, nr=1000, dim=160, ids=f, cs=f, W=8, cap=16, out=f: \
        lib.engram_gather_padded(table, dt, rb, nr, dim, ids, cs, W, cap, out, None, None)
    assert gp(dt=7) == B.ENGRAM_EDTYPE
    assert gp(dim=0) == B.ENGRAM_EINVAL and gp(W=0) == B.ENGRAM_EINVAL and gp(W=256) == B.ENGRAM_EINVAL
    assert gp(cap=-1) == B.ENGRAM_EINVAL and gp(nr=-1) == B.ENGRAM_EINVAL and gp(rb=-1) == B.ENGRAM_EINVAL
    assert gp(cs=None) == B.ENGRAM_EINVAL and gp(ids=None) == B.ENGRAM_EINVAL and gp(out=None) == B.ENGRAM_EINVAL
    assert gp(table=None) == B.ENGRAM_EINVAL
    assert gp(out=ctypes.c_void_p(0x1008)) == B.ENGRAM_EINVAL   # rows of values are 16-byte aligned
    # (ids, split_sizes, world, capacity, row_begin, num_rows, dim, uniq_rows, num_uniq, workspace, bytes, status, stream)
    ws = ctypes.c_void_p(0x100000)
    spp = lambda ids=f, cs=f, W=8, cap=16, rb=0, nr=1000, dim=160, wsb=1 << 30: \
        lib.engram_scatter_add_plan_padded(ids, cs, W, cap, rb, nr, dim, None, None, ws, wsb, None, None)
    assert spp(W=0) == B.ENGRAM_EINVAL and spp(W=256) == B.ENGRAM_EINVAL and spp(cap=-1) == B.ENGRAM_EINVAL
    assert spp(cs=None) == B.ENGRAM_EINVAL and spp(ids=None) == B.ENGRAM_EINVAL and spp(dim=0) == B.ENGRAM_EINVAL
    assert spp(cap=1 << 30) == B.ENGRAM_EINVAL                  # world * capacity < 2^31
    assert spp(wsb=16) == B.ENGRAM_EWORKSPACE


def test_ple_rejects_bad_arguments(lib):
    B._bind_ple(lib)
    fake = ctypes.c_void_p(0x1000)
    bf, f32 = B.ENGRAM_BF16, B.ENGRAM_F32
    conv = lib.engram_short_conv
    # (x, dtype, batch, seq, channels, weight, bias, K, d, halo, y, stream)
    assert conv(fake, 7, 1, 4, 16, fake, None, 4, 3, None, fake, None) == B.ENGRAM_EDTYPE
    assert conv(fake, bf, 1, 4, 12, fake, None, 4, 3, None, fake, None) == B.ENGRAM_EINVAL   # 24 B rows
    assert conv(fake, f32, 1, 4, 6, fake, None, 4, 3, None, fake, None) == B.ENGRAM_EINVAL
    assert conv(fake, bf, 1, 4, 16, fake, None, 5, 3, None, fake, None) == B.ENGRAM_EINVAL   # K > 4
    assert conv(fake, bf, 1, 4, 16, fake, None, 0, 3, None, fake, None) == B.ENGRAM_EINVAL
    assert conv(fake, bf, 1, 4, 16, fake, None, 4, 0, None, fake, None) == B.ENGRAM_EINVAL   # dilation
    assert conv(fake, bf, 1, 4, 16, None, None, 4, 3, None, fake, None) == B.ENGRAM_EINVAL   # weight
    assert conv(None, bf, 1, 4, 16, fake, None, 4, 3, None, fake, None) == B.ENGRAM_EINVAL
    assert conv(fake, bf, -1, 4, 16, fake, None, 4, 3, None, fake, None) == B.ENGRAM_EINVAL
    assert conv(None, bf, 0, 4, 16, fake, None, 4, 3, None, None, None) == B.ENGRAM_OK      # empty: no-op
    assert lib.engram_short_conv_workspace(2, 100, 16, 4) >= 2 * 16 * 5 * 8     # one fp64 partial per batch row at least
    assert lib.engram_short_conv_workspace(2, 100, 16, 5) == 0
    bwd = lib.engram_short_conv_backward
    # (x, dy, dtype, B, S, C, w, K, d, halo, dx, dw, db, dhalo, ws, ws_bytes, stream)
    assert bwd(fake, fake, bf, 1, 4, 16, fake, 4, 3, None, fake, fake, None, None, None, 0, None) == \
        B.ENGRAM_EWORKSPACE
    assert bwd(fake, fake, bf, 1, 4, 16, fake, 4, 3, None, fake, fake, None, None, ctypes.c_void_p(0x1010), 4096,
               None) == B.ENGRAM_EWORKSPACE                                                   # misaligned
    assert bwd(fake, fake, bf, 1, 4, 16, fake, 4, 3, None, fake, None, None, None, fake, 4096, None) == \
        B.ENGRAM_EINVAL                                                                       # dweight
    assert bwd(fake, None, bf, 1, 4, 16, fake, 4, 3, None, fake, fake, None, None, fake, 4096, None) == \
        B.ENGRAM_EINVAL
    norm = lib.engram_grouped_rms_norm
    # (x, dtype, rows, hidden, group, weight, eps, y, stream)
    assert norm(fake, bf, 2, 64, 24, fake, 1e-6, fake, None) == B.ENGRAM_EINVAL        # hidden % group
    assert norm(fake, bf, 2, 60, 12, fake, 1e-6, fake, None) == B.ENGRAM_EINVAL        # 24-byte group
    assert norm(fake, bf, 1, 5128, 5128, fake, 1e-6, fake, None) == B.ENGRAM_EINVAL    # group > 5120 bf16
    assert norm(fake, f32, 1, 2564, 2564, fake, 1e-6, fake, None) == B.ENGRAM_EINVAL   # group > 2560 fp32
    assert norm(fake, bf, 2, 64, 32, fake, -1.0, fake, None) == B.ENGRAM_EINVAL        # eps < 0
    assert norm(fake, bf, 2, 64, 32, fake, float("nan"), fake, None) == B.ENGRAM_EINVAL
    assert norm(fake, bf, 2, 64, 32, None, 1e-6, fake, None) == B.ENGRAM_EINVAL
    assert norm(fake, 3, 2, 64, 32, fake, 1e-6, fake, None) == B.ENGRAM_EDTYPE
    assert norm(None, bf, 0, 64, 32, fake, 1e-6, None, None) == B.ENGRAM_OK            # empty: no-op
    assert lib.engram_grouped_rms_norm_workspace(65, 64) >= 64 * 8
    assert lib.engram_grouped_rms_norm_workspace(-1, 64) == 0
    nb = lib.engram_grouped_rms_norm_backward
    assert nb(fake, fake, bf, 2, 64, 32, fake, 1e-6, fake, fake, None, 0, None) == B.ENGRAM_EWORKSPACE
    assert nb(fake, fake, bf, 2, 64, 32, fake, 1e-6, fake, None, fake, 4096, None) == B.ENGRAM_EINVAL


def test_misaligned_pointers_rejected(lib):
    """Every call checks device pointers against their access width before
    anything is enqueued (the pointers here are never dereferenced)."""
    B._bind_route(lib)
    B._bind_ple(lib)
    ok, odd8, odd16 = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x10004), ctypes.c_void_p(0x10008)
    s = E.qwen3_8_flash_next_spec()
    assert lib.engram_hash(odd8, 1, 4, ctypes.byref(s), ok, None) == B.ENGRAM_EINVAL
    assert lib.engram_hash(ok, 1, 4, ctypes.byref(s), odd8, None) == B.ENGRAM_EINVAL
    assert lib.engram_hash(ok, 1, 4, ctypes.byref(s), odd16, None) == B.ENGRAM_EINVAL   # rows: 16-byte pairs
    assert lib.engram_hash_slice(ok, 1, 8, 2, 6, ctypes.byref(s), odd16, None) == B.ENGRAM_EINVAL
    g = lambda table=ok, rows=ok, out=ok: lib.engram_gather(table, B.ENGRAM_BF16, 0, 100, 160, rows, 10, out, None, None)
    assert g(table=odd16) == B.ENGRAM_EINVAL
    assert g(out=odd16) == B.ENGRAM_EINVAL
    assert g(rows=odd8) == B.ENGRAM_EINVAL
    ws = ctypes.c_void_p(0x100000)
    need = lib.engram_scatter_add_workspace(10, 100, 160)
    assert lib.engram_scatter_add_plan(odd8, 10, 0, 100, 160, None, None, ws, need, None, None) == B.ENGRAM_EINVAL
    assert lib.engram_scatter_add_apply(odd16, B.ENGRAM_BF16, 160, 10, 0, 100, None, ok, ws, need, None) == \
        B.ENGRAM_EINVAL
    assert lib.engram_pack_fixed_capacity(ctypes.c_void_p(0x10002), 10, 8, ok, 2, 4, ok, 4, ok, None, None) == \
        B.ENGRAM_EINVAL
    assert lib.engram_permute_rows(ok, 8, odd8, 10, ctypes.c_void_p(0x10001), None) == B.ENGRAM_EINVAL
    assert lib.engram_short_conv(odd16, B.ENGRAM_BF16, 1, 4, 16, ok, None, 4, 3, None, ok, None) == B.ENGRAM_EINVAL
    assert lib.engram_short_conv(ok, B.ENGRAM_BF16, 1, 4, 16, ctypes.c_void_p(0x10002), None, 4, 3, None, ok,
                                 None) == B.ENGRAM_EINVAL
    assert lib.engram_grouped_rms_norm(ok, B.ENGRAM_BF16, 2, 64, 32, ok, 1e-6, odd16, None) == B.ENGRAM_EINVAL


def test_oversized_ple_calls_rejected(lib):
    B._bind_ple(lib)
    ok = ctypes.c_void_p(0x10000)
    bf = B.ENGRAM_BF16
    assert lib.engram_short_conv(ok, bf, 1 << 20, 1 << 20, 8, ok, None, 4, 3, None, ok, None) == B.ENGRAM_EINVAL
    assert lib.engram_short_conv(ok, bf, 1, 1, 1 << 27, ok, None, 4, 3, None, ok, None) == B.ENGRAM_EINVAL
    assert lib.engram_grouped_rms_norm(ok, bf, 1 << 30, 16, 8, ok, 1e-6, ok, None) == B.ENGRAM_EINVAL


def test_calls_past_the_launch_limits_rejected(lib):
    """Sizes whose launches would hold 2^32 work-items or more are refused up front."""
    B._bind_ple(lib)
    ok = ctypes.c_void_p(0x10000)
    bf = B.ENGRAM_BF16
    s = E.qwen3_8_flash_next_spec()
    assert lib.engram_hash(ok, 1, 1 << 32, ctypes.byref(s), ok, None) == B.ENGRAM_EINVAL
    assert lib.engram_hash(ok, 1 << 26, 64, ctypes.byref(s), ok, None) == B.ENGRAM_EINVAL
    assert lib.engram_hash_slice(ok, 1 << 26, 128, 0, 64, ctypes.byref(s), ok, None) == B.ENGRAM_EINVAL
    # PLE: 2^36 elements per tensor at most
    assert lib.engram_short_conv(ok, bf, 1 << 18, 1 << 10, 512, ok, None, 4, 3, None, ok, None) == B.ENGRAM_EINVAL
    # PLE: within 2^36 elements, but one position per batch row: the dilation-3
    # launches (a 256-lane block per batch row) and the other dilations' launches
    # (a lane per 8 channels) would reach 2^32 work-items
    assert lib.engram_short_conv(ok, bf, 1 << 24, 1, 8, ok, None, 4, 3, None, ok, None) == B.ENGRAM_EINVAL
    assert lib.engram_short_conv_backward(ok, ok, bf, 1 << 24, 1, 8, ok, 4, 3, None, ok, ok, None, None, ok,
                                          1 << 60, None) == B.ENGRAM_EINVAL
    assert lib.engram_short_conv(ok, bf, 1 << 32, 1, 16, ok, None, 4, 2, None, ok, None) == B.ENGRAM_EINVAL
    # no positions, but a halo gradient to clear for 2^40 batch rows
    assert lib.engram_short_conv_backward(None, None, bf, 1 << 40, 0, 8, ok, 4, 3, None, None, ok, None, ok, None,
                                          0, None) == B.ENGRAM_EINVAL
    # norm: 2^25 (row, group) pairs at most
    assert lib.engram_grouped_rms_norm(ok, bf, (1 << 24) + 1, 16, 8, ok, 1e-6, ok, None) == B.ENGRAM_EINVAL
    assert lib.engram_grouped_rms_norm_backward(ok, ok, bf, (1 << 24) + 1, 16, 8, ok, 1e-6, ok, ok, ok, 1 << 40,
                                                None) == B.ENGRAM_EINVAL


def test_missing_library_fails_loudly(monkeypatch):
    """Without libengram.so every product call raises; there is no fallback path."""
    import torch

    import hashed_gram_embedding_engram_amd as E
    from hashed_gram_embedding_engram_amd import engram as EB
    monkeypatch.setattr(EB, "_lib", None)
    monkeypatch.setattr(EB.load_library, "__defaults__", ("/nonexistent/libengram.so",))
    with pytest.raises(RuntimeError, match="libengram.so not found"):
        EB.load_library()
    table = torch.zeros((4, 160), dtype=torch.bfloat16)
    rows = torch.zeros(3, dtype=torch.int64)
    with pytest.raises(RuntimeError, match="libengram.so not found"):
        E.engram_gather(table, rows)
    with pytest.raises(RuntimeError, match="libengram.so not found"):
        E.engram_hash(torch.zeros((1, 8), dtype=torch.int64), E.qwen3_8_flash_next_spec())
    with pytest.raises(RuntimeError, match="libengram.so not found"):
        E.engram_scatter_add(rows, torch.zeros((3, 160), dtype=torch.bfloat16), 4)


def test_noalloc_refuses_sizes_past_its_scratch(lib):
    """The no-allocation scatter-add refuses lookup counts whose workspace exceeds its
    fixed scratch before it looks up the scratch or touches a device."""
    fake = ctypes.c_void_p(0x10000)
    n = 1_300_000
    assert lib.engram_scatter_add_workspace(n, 1000, 160) > B.NOALLOC_SCRATCH_BYTES
    assert lib.engram_scatter_add_noalloc(fake, n, fake, B.ENGRAM_BF16, 160, 0, 1000, fake, None, None, None, None,
                                          None) == B.ENGRAM_EWORKSPACE
    text = open(os.path.join(ROOT, "include", "engram.h")).read()
    assert "#define ENGRAM_NOALLOC_SCRATCH_BYTES (64u << 20)" in text and B.NOALLOC_SCRATCH_BYTES == 64 << 20


def test_hash_gather_rejects_bad_arguments(lib):
    """engram_hash_gather checks everything engram_hash and engram_gather check, and
    refuses a NULL rows_out where the forward needs it (any but the fused layout)."""
    f = ctypes.c_void_p(0x10000)
    mis = ctypes.c_void_p(0x10008)  # 8-byte but not 16-byte aligned
    bf, f32 = B.ENGRAM_BF16, B.ENGRAM_F32
    s = ctypes.byref(E.qwen3_8_flash_next_spec())
    call = lib.engram_hash_gather
    assert call(f, 1, 8, s, f, 7, 0, 10, 160, f, f, None, None) == B.ENGRAM_EDTYPE
    for dim in (0, 100, 1024):
        assert call(f, 1, 8, s, f, bf, 0, 10, dim, f, f, None, None) == B.ENGRAM_EINVAL
    bad = E.qwen3_8_flash_next_spec()
    bad.head_mod[3] = 1
    assert call(f, 1, 8, ctypes.byref(bad), f, bf, 0, 10, 160, f, f, None, None) == B.ENGRAM_ESPEC
    assert call(f, 1, 8, None, f, bf, 0, 10, 160, f, f, None, None) == B.ENGRAM_EINVAL
    assert call(f, -1, 8, s, f, bf, 0, 10, 160, f, f, None, None) == B.ENGRAM_EINVAL
    assert call(f, 1, 8, s, f, bf, -1, 10, 160, f, f, None, None) == B.ENGRAM_EINVAL
    assert call(f, 1, 8, s, f, bf, 0, -10, 160, f, f, None, None) == B.ENGRAM_EINVAL
    assert call(None, 1, 8, s, f, bf, 0, 10, 160, f, f, None, None) == B.ENGRAM_EINVAL
    assert call(f, 1, 8, s, None, bf, 0, 10, 160, f, f, None, None) == B.ENGRAM_EINVAL
    assert call(f, 1, 8, s, f, bf, 0, 10, 160, None, f, None, None) == B.ENGRAM_EINVAL
    assert call(f, 1, 8, s, f, bf, 0, 10, 160, mis, f, None, None) == B.ENGRAM_EINVAL
    assert call(f, 1, 8, s, f, bf, 0, 10, 160, f, mis, None, None) == B.ENGRAM_EINVAL
    # rows_out may be NULL only for the fused layout (3-gram, 8 heads per order, bf16 x 160)
    assert call(f, 1, 8, s, f, f32, 0, 10, 160, f, None, None, None) == B.ENGRAM_EINVAL
    assert call(f, 1, 8, s, f, bf, 0, 10, 128, f, None, None, None) == B.ENGRAM_EINVAL
    two = E.make_hash_spec(2, 8, 7, (3, 5), [101] * 8, [101 * h for h in range(8)])
    assert call(f, 1, 8, ctypes.byref(two), f, bf, 0, 10, 160, f, None, None, None) == B.ENGRAM_EINVAL
    # launches of 2^32 work-items or more are refused; empty work succeeds
    assert call(f, 1 << 26, 64, s, f, bf, 0, 10, 160, f, f, None, None) == B.ENGRAM_EINVAL
    assert call(None, 0, 8, s, None, bf, 0, 10, 160, None, None, None, None) == B.ENGRAM_OK
    # the slice form: 0 <= seq_begin <= seq_end <= seq_len, the rest as above
    sl = lib.engram_hash_gather_slice
    assert sl(f, 1, 8, 3, 2, s, f, bf, 0, 10, 160, f, f, None, None) == B.ENGRAM_EINVAL
    assert sl(f, 1, 8, -1, 2, s, f, bf, 0, 10, 160, f, f, None, None) == B.ENGRAM_EINVAL
    assert sl(f, 1, 8, 0, 9, s, f, bf, 0, 10, 160, f, f, None, None) == B.ENGRAM_EINVAL
    assert sl(f, 1, 8, 2, 5, s, f, 7, 0, 10, 160, f, f, None, None) == B.ENGRAM_EDTYPE
    assert sl(f, 1, 8, 2, 5, s, f, bf, 0, 10, 160, mis, f, None, None) == B.ENGRAM_EINVAL
    assert sl(f, 1, 8, 2, 5, s, f, f32, 0, 10, 160, f, None, None, None) == B.ENGRAM_EINVAL
    assert sl(f, 1 << 27, 64, 0, 32, s, f, bf, 0, 10, 160, f, f, None, None) == B.ENGRAM_EINVAL
    assert sl(None, 1, 8, 4, 4, s, None, bf, 0, 10, 160, None, None, None, None) == B.ENGRAM_OK


def test_plan_from_token_slice_rejects_bad_arguments(lib):
    f = ctypes.c_void_p(0x10000)
    s = ctypes.byref(E.qwen3_8_flash_next_spec())
    call = lib.engram_scatter_add_plan_from_tokens_slice
    ws = lib.engram_scatter_add_workspace(8 * 16, 1000, 160)
    # (tokens, batch, seq_len, seq_begin, seq_end, spec, row_begin, num_rows, dim, uniq_rows, num_uniq,
    #  workspace, bytes, status, stream)
    for a, b in [(-1, 4), (5, 4), (0, 9), (9, 9)]:
        assert call(f, 1, 8, a, b, s, 0, 1000, 160, None, None, f, ws, None, None) == B.ENGRAM_EINVAL
    assert call(f, 1, 1 << 32, 0, 8, s, 0, 1000, 160, None, None, f, ws, None, None) == B.ENGRAM_EINVAL
    assert call(f, 1 << 20, 1 << 9, 0, 1 << 7, s, 0, 1000, 160, None, None, f, ws, None, None) == B.ENGRAM_EINVAL
    assert call(f, 1, 64, 8, 16, s, 0, 1000, 160, None, None, f, ws - 1, None, None) == B.ENGRAM_EWORKSPACE
    two = E.make_hash_spec(2, 8, 7, (3, 5), [101] * 8, [101 * h for h in range(8)])
    assert call(f, 1, 8, 0, 8, ctypes.byref(two), 0, 1000, 160, None, None, f, ws, None, None) == B.ENGRAM_EINVAL


def test_plan_from_tokens_rejects_bad_arguments(lib):
    f = ctypes.c_void_p(0x10000)
    mis = ctypes.c_void_p(0x10004)
    s = ctypes.byref(E.qwen3_8_flash_next_spec())
    call = lib.engram_scatter_add_plan_from_tokens
    ws = lib.engram_scatter_add_workspace(8 * 16, 1000, 160)
    # (tokens, batch, seq_len, spec, row_begin, num_rows, dim, uniq_rows, num_uniq, workspace, bytes, status, stream)
    two = E.make_hash_spec(2, 8, 7, (3, 5), [101] * 8, [101 * h for h in range(8)])
    assert call(f, 1, 8, ctypes.byref(two), 0, 1000, 160, None, None, f, ws, None, None) == B.ENGRAM_EINVAL
    bad = E.qwen3_8_flash_next_spec()
    bad.head_mod[0] = 0
    assert call(f, 1, 8, ctypes.byref(bad), 0, 1000, 160, None, None, f, ws, None, None) == B.ENGRAM_ESPEC
    assert call(None, 1, 8, s, 0, 1000, 160, None, None, f, ws, None, None) == B.ENGRAM_EINVAL
    assert call(mis, 1, 8, s, 0, 1000, 160, None, None, f, ws, None, None) == B.ENGRAM_EINVAL
    assert call(f, -1, 8, s, 0, 1000, 160, None, None, f, ws, None, None) == B.ENGRAM_EINVAL
    assert call(f, 1 << 20, 1 << 7, s, 0, 1000, 160, None, None, f, ws, None, None) == B.ENGRAM_EINVAL  # n = 2^31
    assert call(f, 1, 8, s, 0, 1000, 160, None, None, f, ws - 1, None, None) == B.ENGRAM_EWORKSPACE
    assert call(f, 1, 8, s, 0, 1000, 160, None, None, None, ws, None, None) == B.ENGRAM_EWORKSPACE
    assert call(f, 1, 8, s, 0, 1000, 0, None, None, f, ws, None, None) == B.ENGRAM_EINVAL
