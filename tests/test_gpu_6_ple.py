"""PLE causal short convolution and grouped RMSNorm on the GPU against the fp64
oracle (oracle/ple_ref.py).

Tolerance, from the arithmetic: the kernels compute in fp32 (the layers page
fixes fp32 for the norm; the convolution follows it), so an fp32 result may
differ from the fp64 oracle by rounding proportional to the magnitude of the
terms that form it.  With mag = the same formula evaluated on absolute values,
    |got - ref| <= ATOL + RTOL * (|ref| + mag)            (fp32 outputs)
and a bf16 output may in addition be off by its own rounding, at most one
bf16 ulp (2^-8 relative):
    |got - ref| <= 2^-8 * |ref| + ATOL + RTOL * mag       (bf16 outputs).
Exact checks: the halo form equals the full-sequence form bit for bit, zero
weights give exactly the bias, the weight gradients are bit-identical between
two calls (fixed reduction order)."""
import numpy as np
import pytest
import torch

import hashed_gram_embedding_engram_amd as E
from oracle import ple_ref as P
from tests.gpu_common import ATOL, RTOL, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]

BF16_REL = 2.0 ** -8


def device_input(rng, shape, dtype, scale=1.0):
    t = torch.from_numpy((rng.standard_normal(shape) * scale).astype(np.float32)).to(dtype)
    return t.cuda(), t.double().numpy()


def assert_within(got, ref, mag, bf16, what):
    got = got.detach().double().cpu().numpy()
    ref = np.asarray(ref, dtype=np.float64)
    mag = np.asarray(mag, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    bound = ATOL + RTOL * mag + (BF16_REL * np.abs(ref) if bf16 else RTOL * np.abs(ref))
    bad = np.abs(got - ref) > bound
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError("%s: %d of %d out of tolerance; first at %s: got %r ref %r bound %r" %
                             (what, int(bad.sum()), bad.size, i, got[i], ref[i], bound[i]))


def conv_mag(x, w, b, d, halo):
    return P.short_conv(np.abs(x), np.abs(w), None if b is None else np.abs(b), d,
                        None if halo is None else np.abs(halo))


CONV_CASES = [
    # (B, S, C, K, d, dtype, halo, bias)
    (2, 300, 10240, 4, 3, torch.bfloat16, False, True),    # the layer's shape: 4 branches x 2560
    (2, 300, 10240, 4, 3, torch.bfloat16, True, False),
    (3, 77, 24, 4, 3, torch.float32, True, True),
    (1, 1, 8, 4, 3, torch.bfloat16, True, True),           # one position, all but one tap in the halo
    (2, 5, 16, 4, 3, torch.bfloat16, True, True),          # sequence shorter than the halo
    (2, 129, 64, 1, 3, torch.float32, False, True),
    (2, 129, 64, 2, 7, torch.bfloat16, True, True),
    (4, 65, 40, 3, 1, torch.bfloat16, False, False),
]


@pytest.mark.parametrize("case", CONV_CASES, ids=lambda c: "B%d_S%d_C%d_K%d_d%d_%s%s%s" % (
    c[0], c[1], c[2], c[3], c[4], "bf16" if c[5] == torch.bfloat16 else "f32", "_halo" if c[6] else "",
    "_bias" if c[7] else ""))
def test_short_conv_forward_and_backward(case):
    B, S, C, K, d, dtype, use_halo, use_bias = case
    rng = np.random.default_rng(B * 1000 + S + C + K * 7 + d)
    H = (K - 1) * d
    x, xh = device_input(rng, (B, S, C), dtype)
    dy, dyh = device_input(rng, (B, S, C), dtype)
    halo, haloh = device_input(rng, (B, H, C), dtype) if use_halo else (None, None)
    w_np = (rng.standard_normal((C, K)) * 0.5).astype(np.float32)
    b_np = (rng.standard_normal(C) * 0.1).astype(np.float32) if use_bias else None
    w = torch.from_numpy(w_np).cuda()
    b = torch.from_numpy(b_np).cuda() if use_bias else None
    bf16 = dtype == torch.bfloat16

    y = E.engram_short_conv(x, w, b, dilation=d, halo=halo)
    ref = P.short_conv(xh, w_np, b_np, d, haloh)
    assert_within(y, ref, conv_mag(xh, w_np, b_np, d, haloh), bf16, "y")

    dx, dw, db, dhalo = E.engram_short_conv_backward(x, dy, w, dilation=d, halo=halo, want_bias=True,
                                                     want_halo=True)
    rdx, rdw, rdb, rdhalo = P.short_conv_backward(xh, dyh, w_np, d, haloh)
    adx, adw, adb, adhalo = P.short_conv_backward(np.abs(xh), np.abs(dyh), np.abs(w_np), d,
                                                  None if haloh is None else np.abs(haloh))
    assert_within(dx, rdx, adx, bf16, "dx")
    assert_within(dhalo, rdhalo, adhalo, bf16, "dhalo")
    assert_within(dw, rdw, adw, False, "dweight")
    assert_within(db, rdb, adb, False, "dbias")
    # fixed reduction order: a second call gives the same bits
    _, dw2, db2, _ = E.engram_short_conv_backward(x, dy, w, dilation=d, halo=halo)
    assert torch.equal(dw, dw2) and torch.equal(db, db2)


def test_short_conv_halo_equals_full_sequence():
    """A shard that receives the preceding nine tokens as its halo computes the
    same outputs, bit for bit, as the unsplit sequence at those positions."""
    rng = np.random.default_rng(5)
    B, S, C, K, d = 2, 257, 2560, 4, 3
    H = (K - 1) * d
    x, _ = device_input(rng, (B, S, C), torch.bfloat16)
    w = torch.from_numpy((rng.standard_normal((C, K)) * 0.5).astype(np.float32)).cuda()
    b = torch.from_numpy((rng.standard_normal(C) * 0.1).astype(np.float32)).cuda()
    full = E.engram_short_conv(x, w, b, dilation=d)
    for cut in (1, 9, 100, 200):
        lo = max(0, cut - H)
        halo = torch.zeros((B, H, C), dtype=x.dtype, device="cuda")
        halo[:, H - (cut - lo):] = x[:, lo:cut]
        part = E.engram_short_conv(x[:, cut:].contiguous(), w, b, dilation=d, halo=halo.contiguous())
        assert torch.equal(part, full[:, cut:]), cut


def test_short_conv_zero_weights_give_bias():
    """The convolution starts at zero (init_weights): the output is exactly the bias."""
    rng = np.random.default_rng(6)
    x, _ = device_input(rng, (2, 50, 64), torch.bfloat16)
    w = torch.zeros((64, 4), dtype=torch.float32, device="cuda")
    b = torch.from_numpy(rng.standard_normal(64).astype(np.float32)).cuda()
    y = E.engram_short_conv(x, w, b)
    assert torch.equal(y, b.to(torch.bfloat16).expand(2, 50, 64))
    assert torch.equal(E.engram_short_conv(x, w), torch.zeros_like(x))


def test_short_conv_empty_sequence():
    w = torch.ones((16, 4), dtype=torch.float32, device="cuda")
    x = torch.empty((3, 0, 16), dtype=torch.bfloat16, device="cuda")
    halo = torch.ones((3, 9, 16), dtype=torch.bfloat16, device="cuda")
    assert E.engram_short_conv(x, w, halo=halo).shape == (3, 0, 16)
    dx, dw, db, dhalo = E.engram_short_conv_backward(x, x, w, halo=halo, want_halo=True)
    assert dx.shape == (3, 0, 16)
    assert not dw.any() and not db.any() and not dhalo.any()


NORM_CASES = [
    # (rows, hidden, group, dtype)
    (300, 10240, 2560, torch.bfloat16),     # the layer's branch norm: 4 branches of 2560
    (77, 10240, 2560, torch.float32),
    (33, 10240, 5120, torch.bfloat16),      # largest bf16 group: 10 chunks per lane
    (33, 5120, 2560, torch.float32),        # largest fp32 group
    (65, 1040, 520, torch.bfloat16),        # 65 chunks: one lane holds a second chunk
    (40, 64, 8, torch.bfloat16),            # one chunk per group
    (1, 12, 4, torch.float32),
]


@pytest.mark.parametrize("case", NORM_CASES, ids=lambda c: "r%d_h%d_g%d_%s" % (
    c[0], c[1], c[2], "bf16" if c[3] == torch.bfloat16 else "f32"))
def test_grouped_rms_norm_forward_and_backward(case):
    rows, hidden, group, dtype = case
    rng = np.random.default_rng(rows + hidden + group)
    eps = 1e-6
    x, xh = device_input(rng, (rows, hidden), dtype, scale=2.0)
    dy, dyh = device_input(rng, (rows, hidden), dtype)
    w_np = (rng.standard_normal(hidden) * 0.3).astype(np.float32)
    w = torch.from_numpy(w_np).cuda()
    bf16 = dtype == torch.bfloat16

    y = E.engram_grouped_rms_norm(x, w, group, eps)
    ref = P.grouped_rms_norm(xh, w_np, group, eps)
    assert_within(y, ref, np.abs(ref), bf16, "y")

    dx, dw = E.engram_grouped_rms_norm_backward(x, dy, w, group, eps)
    rdx, rdw = P.grouped_rms_norm_backward(xh, dyh, w_np, group, eps)
    # magnitudes: |dx| terms inv*|dy*(1+w)| + inv^3 |x| sum|dy*(1+w)*x| / group; |dw| terms sum |dy * n|
    g = xh.reshape(rows, hidden // group, group)
    inv = 1.0 / np.sqrt((g * g).mean(axis=-1, keepdims=True) + eps)
    dn = np.abs(dyh * (1.0 + w_np)).reshape(g.shape)
    mag_dx = inv * dn + inv ** 3 * np.abs(g) * (dn * np.abs(g)).mean(axis=-1, keepdims=True)
    mag_dw = (np.abs(dyh) * np.abs(g * inv).reshape(rows, hidden)).sum(axis=0)
    assert_within(dx, rdx, mag_dx.reshape(rows, hidden), bf16, "dx")
    assert_within(dw, rdw, mag_dw, False, "dweight")
    _, dw2 = E.engram_grouped_rms_norm_backward(x, dy, w, group, eps)
    assert torch.equal(dw, dw2)


def test_grouped_rms_norm_zero_weight_unit_rms():
    """Weight zero (the initial state), eps 0 and groups whose mean square is 1:
    the output equals the input exactly."""
    eps = 1e-6
    x = torch.tensor([[1.0, -1.0, 1.0, -1.0, 2.0, 0.0, 0.0, 0.0]], dtype=torch.float32, device="cuda")
    w = torch.zeros(8, dtype=torch.float32, device="cuda")
    y = E.engram_grouped_rms_norm(x, w, 4, 0.0)
    assert torch.equal(y, x)
    z = E.engram_grouped_rms_norm(torch.zeros(3, 16, dtype=torch.bfloat16, device="cuda"), w.repeat(2), 8, eps)
    assert not z.float().any()   # zero input stays zero (eps keeps the scale finite)


def test_grouped_rms_norm_empty():
    w = torch.zeros(64, dtype=torch.float32, device="cuda")
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    assert E.engram_grouped_rms_norm(x, w, 32).shape == (0, 64)
    dx, dw = E.engram_grouped_rms_norm_backward(x, x, w, 32)
    assert dx.shape == (0, 64) and not dw.any()


def test_ple_bench_shape_sampled():
    """The benchmarked layer shape, [8, 4096, 10240] bf16 with a halo, through the
    same kernels the benchmark times.  Outputs are checked at sampled positions
    (the oracle gets just the inputs they depend on), the weight gradients over
    whole channels and one whole group of the norm."""
    import workloads as W
    B, S, C, G, d, K = 8, 4096, 10240, 2560, 3, 4
    H = (K - 1) * d
    t = W.ple_tensors(torch.device("cuda"), 2000, B, S, C)
    x, dy, halo, w, b, nw = t["x"], t["dy"], t["halo"], t["conv_w"], t["conv_b"], t["norm_w"]
    y = E.engram_short_conv(x, w, b, dilation=d, halo=halo)
    dx, dw, db, dhalo = E.engram_short_conv_backward(x, dy, w, dilation=d, halo=halo, want_bias=True,
                                                     want_halo=True)
    z = E.engram_grouped_rms_norm(x.reshape(B * S, C), nw, G)
    dxn, dnw = E.engram_grouped_rms_norm_backward(x.reshape(B * S, C), dy.reshape(B * S, C), nw, G)
    w_np, b_np, nw_np = w.cpu().numpy(), b.cpu().numpy(), nw.cpu().numpy()
    halo_h = halo.double().cpu().numpy()
    rng = np.random.default_rng(77)
    samples = [(0, 0), (0, 1), (7, 8), (3, 9), (5, S - 1), (1, S - 10)] + \
        [(int(rng.integers(B)), int(rng.integers(S))) for _ in range(10)]
    for bi, ti in samples:
        # conv output at (bi, ti): its window and, near the start, the halo
        lo = max(0, ti - H)
        xs = x[bi, lo:ti + 1].double().cpu().numpy()[None]
        hs = halo_h[bi:bi + 1] if lo == 0 else np.zeros((1, H, C))
        ref = P.short_conv(xs, w_np, b_np, d, hs)[0, -1]
        mag = conv_mag(xs, w_np, b_np, d, hs)[0, -1]
        assert_within(y[bi, ti], ref, mag, True, "y at %s" % ((bi, ti),))
        # conv input gradient at (bi, ti): the output gradients after it
        hi = min(S, ti + H + 1)
        xs2 = x[bi, ti:hi].double().cpu().numpy()[None]
        dys2 = dy[bi, ti:hi].double().cpu().numpy()[None]
        rdx = P.short_conv_backward(xs2, dys2, w_np, d, np.zeros((1, H, C)))[0][0, 0]
        adx = P.short_conv_backward(np.abs(xs2), np.abs(dys2), np.abs(w_np), d, np.zeros((1, H, C)))[0][0, 0]
        assert_within(dx[bi, ti], rdx, adx, True, "dx at %s" % ((bi, ti),))
        # the norm of row (bi, ti) and its input gradient
        r = bi * S + ti
        xr = x.reshape(B * S, C)[r].double().cpu().numpy()[None]
        dyr = dy.reshape(B * S, C)[r].double().cpu().numpy()[None]
        zr = P.grouped_rms_norm(xr, nw_np, G)
        assert_within(z[r], zr[0], np.abs(zr[0]), True, "norm at row %d" % r)
        rdxn, _ = P.grouped_rms_norm_backward(xr, dyr, nw_np, G)
        g3 = xr.reshape(1, C // G, G)
        inv = 1.0 / np.sqrt((g3 * g3).mean(axis=-1, keepdims=True) + 1e-6)
        dn = np.abs(dyr * (1.0 + nw_np)).reshape(g3.shape)
        mag_dx = (inv * dn + inv ** 3 * np.abs(g3) * (dn * np.abs(g3)).mean(axis=-1, keepdims=True)).reshape(1, C)
        assert_within(dxn[r], rdxn[0], mag_dx[0], True, "norm dx at row %d" % r)
    # halo gradient: the first 9 positions' output gradients of every batch row
    xs = x[:, :H].double().cpu().numpy()
    dys = dy[:, :H].double().cpu().numpy()
    rdh = P.short_conv_backward(xs, dys, w_np, d, halo_h)[3]
    adh = P.short_conv_backward(np.abs(xs), np.abs(dys), np.abs(w_np), d, np.abs(halo_h))[3]
    assert_within(dhalo, rdh, adh, True, "dhalo")
    # conv weight and bias gradients of a few whole channels (channels are independent)
    cs = np.array([0, 1, 2559, 2560, 5000, 7681, C - 1])
    xc = x[:, :, cs].double().cpu().numpy()
    dyc = dy[:, :, cs].double().cpu().numpy()
    hc = halo_h[:, :, cs]
    _, rdw, rdb, _ = P.short_conv_backward(xc, dyc, w_np[cs], d, hc)
    _, adw, adb, _ = P.short_conv_backward(np.abs(xc), np.abs(dyc), np.abs(w_np[cs]), d, np.abs(hc))
    assert_within(dw[torch.from_numpy(cs).cuda()], rdw, adw, False, "dweight")
    assert_within(db[torch.from_numpy(cs).cuda()], rdb, adb, False, "dbias")
    # norm weight gradient over every row for the features of one whole group
    g0 = 2 * G
    xg = x.reshape(B * S, C)[:, g0:g0 + G].double().cpu().numpy()
    dyg = dy.reshape(B * S, C)[:, g0:g0 + G].double().cpu().numpy()
    _, rdnw = P.grouped_rms_norm_backward(xg, dyg, nw_np[g0:g0 + G], G)
    invg = 1.0 / np.sqrt((xg * xg).mean(axis=-1, keepdims=True) + 1e-6)
    mag_dnw = (np.abs(dyg) * np.abs(xg * invg)).sum(axis=0)
    assert_within(dnw[g0:g0 + G], rdnw, mag_dnw, False, "norm dweight")
