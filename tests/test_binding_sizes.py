"""The Python binding refuses caller-supplied buffers whose dtype, shape or
size differs from what the C call will assume, before anything is enqueued:
an undersized buffer on the GPU would otherwise turn into an out-of-bounds
device access.  The helper that does the checking runs on the CPU here; the
bindings' use of it runs on GPU tensors (marked gpu), every case raising
before the C call."""
import pytest
import torch

import hashed_gram_embedding_engram_amd as E
from hashed_gram_embedding_engram_amd import engram as B


@pytest.fixture(scope="module", autouse=True)
def lib():
    import os
    if not os.path.exists(B.LIB_PATH):
        from hashed_gram_embedding_engram_amd import build
        build.build()
    return B.load_library()


DEV = "cuda"


def i64(*shape):
    return torch.zeros(shape, dtype=torch.int64, device=DEV)


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32, device=DEV)


def bf16(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16, device=DEV)


def u8(n):
    return torch.zeros(n, dtype=torch.uint8, device=DEV)


SIZE = "must (hold|have shape)"


def test_helper_checks_sizes_before_the_device():
    """On CPU tensors the size checks fire first, so each is seen."""
    t = torch.zeros((4, 8), dtype=torch.float32)
    with pytest.raises(ValueError, match="must be torch.int64"):
        B._dev_ptr(t, "t", torch.int64)
    with pytest.raises(ValueError, match="must have shape"):
        B._dev_ptr(t, "t", torch.float32, shape=(4, 9))
    with pytest.raises(ValueError, match="must hold 33 elements"):
        B._dev_ptr(t, "t", numel=33)
    with pytest.raises(ValueError, match="at least 33"):
        B._dev_ptr(t, "t", min_numel=33)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        B._dev_ptr(t, "t", torch.float32, shape=(4, 8), numel=32, min_numel=32)
    assert B._dev_ptr(None, "t", torch.int64, numel=5) is None
    with pytest.raises(ValueError, match="must hold 1 elements"):
        B._status_ptr(torch.zeros(2, dtype=torch.int64))


def test_apply_refuses_a_plan_made_for_other_sizes():
    """The plan's sizes, recorded on the workspace, are checked before any pointer."""
    ws = torch.zeros(1, dtype=torch.uint8)
    ws._engram_plan = (10, 100, 160, 0)        # what a plan call records
    g = torch.zeros((12, 160), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="workspace holds a plan"):
        E.engram_scatter_add_apply(g, 12, 100, ws, uniq_grad=torch.zeros((12, 160)))
    with pytest.raises(ValueError, match="workspace holds a plan"):
        E.engram_scatter_add_apply(g[:10], 10, 200, ws, uniq_grad=torch.zeros((10, 160)))
    with pytest.raises(ValueError, match="workspace holds a plan"):
        E.engram_scatter_add_apply(g[:10], 10, 100, ws, row_begin=5, uniq_grad=torch.zeros((10, 160)))


@pytest.mark.gpu
def test_hash_output():
    spec = E.qwen3_8_flash_next_spec()
    with pytest.raises(ValueError, match=SIZE):
        E.engram_hash(i64(2, 8), spec, rows_out=i64(2, 8, 15))
    with pytest.raises(ValueError, match=SIZE):
        E.engram_hash_slice(i64(2, 8), 2, 6, spec, rows_out=i64(2, 3, 16))
    with pytest.raises(ValueError, match="must be torch.int64"):
        E.engram_hash(i64(2, 8), spec, rows_out=torch.zeros((2, 8, 16), dtype=torch.int32))


@pytest.mark.gpu
def test_gather_output_and_status():
    table, rows = bf16(100, 160), i64(10)
    with pytest.raises(ValueError, match=SIZE):
        E.engram_gather(table, rows, out=bf16(9, 160), validate=False)
    with pytest.raises(ValueError, match="must be torch.bfloat16"):
        E.engram_gather(table, rows, out=f32(10, 160), validate=False)
    with pytest.raises(ValueError, match=SIZE):
        E.engram_gather(table, rows, out=bf16(10, 160), status=i64(2), validate=False)


@pytest.mark.gpu
def test_scatter_add_outputs():
    rows, dy = i64(10), bf16(10, 160)
    with pytest.raises(ValueError, match="one row per lookup"):
        E.engram_scatter_add(rows, bf16(9, 160), 100, workspace=u8(1))
    ws = u8(1)
    with pytest.raises(ValueError, match=SIZE):
        E.engram_scatter_add(rows, dy, 100, grad_dense=f32(99, 160), workspace=ws, validate=False)
    with pytest.raises(ValueError, match=SIZE):
        E.engram_scatter_add(rows, dy, 100, compact=(i64(9), f32(10, 160), i64()), workspace=ws, validate=False)
    with pytest.raises(ValueError, match=SIZE):
        E.engram_scatter_add(rows, dy, 100, compact=(i64(10), f32(10, 159), i64()), workspace=ws, validate=False)
    with pytest.raises(ValueError, match=SIZE):
        E.engram_scatter_add(rows, dy, 100, compact=(i64(10), f32(10, 160), i64(2)), workspace=ws, validate=False)


@pytest.mark.gpu
def test_plan_and_apply():
    rows, ws = i64(10), u8(1)
    with pytest.raises(ValueError, match=SIZE):
        E.engram_scatter_add_plan(rows, 100, 160, workspace=ws, uniq_rows=i64(9))
    with pytest.raises(ValueError, match=SIZE):
        E.engram_scatter_add_apply(bf16(9, 160), 10, 100, ws, uniq_grad=f32(10, 160))
    with pytest.raises(ValueError, match=SIZE):
        E.engram_scatter_add_apply(bf16(10, 160), 10, 100, ws, grad_dense=f32(100, 80))
    with pytest.raises(ValueError, match=SIZE):
        E.engram_scatter_add_apply(bf16(10, 160), 10, 100, ws, uniq_grad=f32(9, 160))


@pytest.mark.gpu
def test_routing_buffers():
    ids, counts = i64(20), i64(4)
    with pytest.raises(ValueError, match=SIZE):
        E.engram_route_plan(ids, 400, 4, out=(i64(19), i64(20), i64(4)), workspace=u8(1))
    with pytest.raises(ValueError, match=SIZE):
        E.engram_route_plan(ids, 400, 4, out=(i64(20), i64(20), i64(3)), workspace=u8(1))
    with pytest.raises(ValueError, match=SIZE):
        E.engram_route_validate(ids, i64(3), 400, 4)
    with pytest.raises(ValueError, match=SIZE):
        E.engram_pack_fixed_capacity(bf16(20, 160), i64(3), 4, 8)
    with pytest.raises(ValueError, match=SIZE):
        E.engram_pack_fixed_capacity(bf16(20, 160), counts, 4, 8, out=bf16(4, 7, 160))
    with pytest.raises(ValueError, match=SIZE):
        E.engram_unpack_fixed_capacity(bf16(4, 8, 160), counts, 20, out=bf16(19, 160))
    with pytest.raises(ValueError, match=SIZE):
        E.engram_permute_rows(bf16(9, 160), i64(10))
    with pytest.raises(ValueError, match=SIZE):
        E.engram_unpermute_rows(bf16(10, 160), i64(10), out=bf16(9, 160))
    with pytest.raises(ValueError, match=SIZE):
        E.engram_unpack_unpermute_rows(bf16(4, 8, 160), counts, i64(20), out=bf16(19, 160))
    with pytest.raises(ValueError, match=SIZE):
        E.engram_unpack_unpermute_rows(bf16(4, 8, 160), i64(3), i64(20))
    with pytest.raises(ValueError, match=SIZE):
        E.engram_permute_pack_rows(bf16(19, 160), i64(20), counts, 4, 8)
    with pytest.raises(ValueError, match=SIZE):
        E.engram_gather_padded(bf16(100, 160), i64(4, 8), counts, out=bf16(4, 7, 160))
    with pytest.raises(ValueError, match=SIZE):
        E.engram_gather_padded(bf16(100, 160), i64(4, 8), i64(3))
    with pytest.raises(ValueError, match=SIZE):
        E.engram_scatter_add_plan_padded(i64(4, 8), i64(3), 100, 160)
    with pytest.raises(ValueError, match=SIZE):
        E.engram_permute_pack_rows(bf16(20, 160), i64(20), counts, 4, 8, out=bf16(4, 7, 160))


@pytest.mark.gpu
def test_ple_buffers():
    x, w = bf16(2, 12, 16), f32(16, 4)
    with pytest.raises(ValueError, match="weight must be"):
        E.engram_short_conv(x, f32(8, 4))
    with pytest.raises(ValueError, match=SIZE):
        E.engram_short_conv(x, w, bias=f32(15))
    with pytest.raises(ValueError, match=SIZE):
        E.engram_short_conv(x, w, halo=bf16(2, 8, 16))
    with pytest.raises(ValueError, match=SIZE):
        E.engram_short_conv(x, w, out=bf16(2, 11, 16))
    ws = u8(1)
    with pytest.raises(ValueError, match=SIZE):
        E.engram_short_conv_backward(x, bf16(2, 11, 16), w, workspace=ws)
    with pytest.raises(ValueError, match=SIZE):
        E.engram_short_conv_backward(x, bf16(2, 12, 16), w, workspace=ws,
                                     out=(bf16(2, 12, 16), f32(16, 3), None, None))
    with pytest.raises(ValueError, match=SIZE):
        E.engram_short_conv_backward(x, bf16(2, 12, 16), w, workspace=ws,
                                     out=(bf16(2, 12, 16), f32(16, 4), None, bf16(2, 8, 16)))
    xn = bf16(6, 64)
    with pytest.raises(ValueError, match=SIZE):
        E.engram_grouped_rms_norm(xn, f32(63), 32)
    with pytest.raises(ValueError, match=SIZE):
        E.engram_grouped_rms_norm(xn, f32(64), 32, out=bf16(5, 64))
    with pytest.raises(ValueError, match=SIZE):
        E.engram_grouped_rms_norm_backward(xn, bf16(6, 64), f32(64), 32, workspace=ws, out=(bf16(6, 64), f32(32)))
