"""engram_scatter_add_noalloc, called through the C ABI: the scatter-add on the
library's fixed 64 MiB scratch array, for callers that cannot allocate.  Its
outputs must equal those of engram_scatter_add (same kernels, a workspace the
caller allocated) bit for bit, and the fp64 oracle within the backward's
tolerance, on two calls in a row on the same GPU, the second with a smaller
input (the scratch keeps the first call's contents), in both output forms.
Sizes the scratch cannot hold are refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

from hashed_gram_embedding_engram_amd import engram as B
from oracle import c_oracle
from tests.gpu_common import assert_close_to_fp64, requires_gpu, to_host

pytestmark = [pytest.mark.gpu, requires_gpu]

DIM = 160


def ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def call_noalloc(lib, rows, dy, num_rows, row_begin, dense=None, compact=None, status=None):
    ur, ug, nu = compact if compact is not None else (None, None, None)
    dt = B.ENGRAM_BF16 if dy.dtype == torch.bfloat16 else B.ENGRAM_F32
    return lib.engram_scatter_add_noalloc(ptr(rows), rows.numel(), ptr(dy), dt, DIM, row_begin, num_rows, ptr(dense),
                                          ptr(ur), ptr(ug), ptr(nu), ptr(status),
                                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def zipf_rows(seed, n, num_rows, row_begin):
    rng = np.random.default_rng(seed)
    rows = (rng.zipf(1.2, size=n) % num_rows).astype(np.int64) + row_begin
    return rows


def grads(seed, n, dtype):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn((n, DIM), generator=g, device="cuda").to(dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noalloc_compact_equals_workspace_call(dtype):
    lib = B.load_library()
    num_rows, row_begin = 3_000_000, 1000
    # the first call near the scratch's limit, the second much smaller
    for seed, n in ((1, 1_000_000), (2, 37_003)):
        rows_np = zipf_rows(seed, n, num_rows, row_begin)
        rows = torch.from_numpy(rows_np).cuda()
        dy = grads(seed, n, dtype)
        ur = torch.full((n,), -7, dtype=torch.int64, device="cuda")
        ug = torch.full((n, DIM), float("nan"), dtype=torch.float32, device="cuda")
        nu = torch.empty((), dtype=torch.int64, device="cuda")
        st = torch.empty((), dtype=torch.int64, device="cuda")
        assert call_noalloc(lib, rows, dy, num_rows, row_begin, compact=(ur, ug, nu), status=st) == B.ENGRAM_OK
        ref_r, ref_g = B.engram_scatter_add(rows, dy, num_rows, row_begin)
        torch.cuda.synchronize()
        u = int(nu.item())
        assert int(st.item()) == -1
        assert u == ref_r.numel()
        assert torch.equal(ur[:u], ref_r)
        assert torch.equal(ug[:u].view(torch.int32), ref_g.view(torch.int32))
        rur, rug, bad = c_oracle.scatter_add_compact(rows_np, to_host(dy), num_rows, row_begin)
        assert bad == -1 and np.array_equal(ur[:u].cpu().numpy(), rur)
        assert_close_to_fp64(ug[:u].cpu().numpy(), rug, "noalloc compact, n=%d" % n)


def test_noalloc_dense_equals_workspace_call():
    lib = B.load_library()
    num_rows, row_begin = 200_000, 0
    for seed, n in ((3, 900_000), (4, 5_001)):
        rows_np = zipf_rows(seed, n, num_rows, row_begin)
        rows_np[::1000] = num_rows + 3          # out of the shard: dropped and reported
        rows = torch.from_numpy(rows_np).cuda()
        dy = grads(seed, n, torch.bfloat16)
        prior = torch.randn((num_rows, DIM), device="cuda")
        g1, g2 = prior.clone(), prior.clone()
        st = torch.empty((), dtype=torch.int64, device="cuda")
        assert call_noalloc(lib, rows, dy, num_rows, row_begin, dense=g1, status=st) == B.ENGRAM_OK
        B.engram_scatter_add(rows, dy, num_rows, row_begin, grad_dense=g2, validate=False)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        assert torch.equal(g1.view(torch.int32), g2.view(torch.int32))
        ref, bad = c_oracle.scatter_add_dense(rows_np, to_host(dy), num_rows, row_begin, prior.cpu().numpy())
        assert bad == 0
        touched = np.unique(rows_np[rows_np < num_rows])
        assert_close_to_fp64(g1[torch.from_numpy(touched).cuda()].cpu().numpy(), ref[touched],
                             "noalloc dense, n=%d" % n)


def test_noalloc_refuses_sizes_past_the_scratch():
    lib = B.load_library()
    n = 1_300_000                      # needs about 70 MiB of workspace at dim 160
    assert lib.engram_scatter_add_workspace(n, 1000, DIM) > B.NOALLOC_SCRATCH_BYTES
    rows = torch.zeros(n, dtype=torch.int64, device="cuda")
    dy = torch.zeros((n, DIM), dtype=torch.bfloat16, device="cuda")
    dense = torch.zeros((1000, DIM), dtype=torch.float32, device="cuda")
    assert call_noalloc(lib, rows, dy, 1000, 0, dense=dense) == B.ENGRAM_EWORKSPACE
    with pytest.raises(B.EngramError):
        B.engram_scatter_add_noalloc(rows, dy, 1000, grad_dense=dense)
    torch.cuda.synchronize()
    assert int((dense != 0).sum().item()) == 0       # nothing ran
