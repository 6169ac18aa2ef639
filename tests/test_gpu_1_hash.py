"""Hash kernel parity: bit-exact against the oracle on every workload shape,
brute-force enumerations, int64 extremes and the slice (context-parallel) form."""
import itertools

import numpy as np
import pytest
import torch

import hashed_gram_embedding_engram_amd as E
import workloads as W
from oracle import constants as C, hash_ref
from tests.gpu_common import full_oracle_spec, oracle_hash, product_spec_from, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


def gpu_hash(ids, spec):
    t = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int64)).cuda()
    out = E.engram_hash(t, spec)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def tiny_ws():
    return W.tiny_spec()


def test_tiny_case():
    ws = tiny_ws()
    ids = W.tiny_tokens()
    got = gpu_hash(ids, product_spec_from(ws))
    assert np.array_equal(got, oracle_hash(ids, ws))
    # and the pure-Python statement
    py = hash_ref.hash_input_ids(ids.tolist(), 3, 8, ws["eos"], 0, C.LAYER_MULTIPLIERS, ws["vocab_sizes"], ws["offsets"])
    assert np.array_equal(got, np.asarray(py, dtype=np.int64))


@pytest.mark.parametrize("length", [1, 2, 3, 5, 7])
def test_brute_force_enumeration(length):
    """All sequences over {0, 1, 2, EOS} of the given length, one batch row each."""
    ws = tiny_ws()
    letters = [0, 1, 2, ws["eos"]]
    ids = np.array(list(itertools.product(letters, repeat=length)), dtype=np.int64)
    assert np.array_equal(gpu_hash(ids, product_spec_from(ws)), oracle_hash(ids, ws))


@pytest.mark.parametrize("fill", [0, -1, (1 << 63) - 1, -(1 << 63)])
def test_int64_extremes(fill):
    rng = np.random.default_rng(5)
    ids = rng.integers(-(1 << 63), (1 << 63) - 1, size=(5, 333), dtype=np.int64)
    ids[:, :6] = [-(1 << 63), (1 << 63) - 1, -1, 0, 1, C.EOS_TOKEN_ID]
    ids[rng.random(ids.shape) < 0.03] = C.EOS_TOKEN_ID
    got = gpu_hash(ids, E.qwen3_8_flash_next_spec(fill_id=fill))
    assert np.array_equal(got, oracle_hash(ids, full_oracle_spec(fill)))


def test_wrap_closed_form_on_gpu():
    """Token M0^-1 mod 2^64 wraps to 1, its negation to -1 (segment start, fill 0)."""
    inv = pow(C.LAYER_MULTIPLIERS[0], -1, 1 << 64)
    x = inv - (1 << 64) if inv >= 1 << 63 else inv
    got = gpu_hash(np.array([[x], [-x]], dtype=np.int64), E.qwen3_8_flash_next_spec())
    offs = np.array(C.head_offsets())
    assert np.array_equal(got[0, 0], offs + 1)
    assert np.array_equal(got[1, 0], offs + np.array(C.head_vocab_sizes()) - 1)


@pytest.mark.parametrize("shape", [(1, 1), (1, 2), (1, 63), (1, 64), (1, 65), (3, 100), (7, 129), (2, 4097)])
def test_ragged_shapes(shape):
    rng = np.random.default_rng(sum(shape))
    ids = W.zipf_token_ids(rng, shape[0] * shape[1], 1.1).reshape(shape)
    ids[rng.random(shape) < 0.05] = C.EOS_TOKEN_ID
    assert np.array_equal(gpu_hash(ids, E.qwen3_8_flash_next_spec()), oracle_hash(ids, full_oracle_spec()))


def test_sft_batch():
    ids, _ = W.sft_batch(0)
    assert np.array_equal(gpu_hash(ids, E.qwen3_8_flash_next_spec()), oracle_hash(ids, full_oracle_spec()))


def test_sft_spec_table():
    ws = W.sft_spec()
    ids, _ = W.sft_batch(0)
    got = gpu_hash(ids, product_spec_from(ws))
    assert np.array_equal(got, oracle_hash(ids, ws))
    assert got.max() < ws["num_rows"]


def test_long_context_stream():
    ids, _ = W.long_context_stream(0)
    assert np.array_equal(gpu_hash(ids, E.qwen3_8_flash_next_spec()), oracle_hash(ids, full_oracle_spec()))


def test_owner_batches_sample():
    ids = W.owner_token_batches(seeds=range(100, 108)).reshape(-1, 4096)
    assert np.array_equal(gpu_hash(ids, E.qwen3_8_flash_next_spec()), oracle_hash(ids, full_oracle_spec()))


@pytest.mark.parametrize("ngram,hpn", [(4, 3), (2, 5), (5, 8), (8, 9), (2, 64)])
def test_other_head_layouts(ngram, hpn):
    """Runtime-layout kernels: other n-gram orders and heads per order."""
    rng = np.random.default_rng(ngram * 100 + hpn)
    H = (ngram - 1) * hpn
    mods = sorted(rng.choice(np.arange(1000, 50000), H, replace=False).tolist())
    offs = np.concatenate([[0], np.cumsum(mods)[:-1]]).tolist()
    mult = [int(v) | 1 for v in rng.integers(1, 1 << 62, size=ngram)]
    ids = rng.integers(0, 30, size=(3, 77)).astype(np.int64)
    ids[ids == 7] = 29
    ws = {"ngram_size": ngram, "heads_per_ngram": hpn, "eos": 29, "fill": 3, "vocab_sizes": mods, "offsets": offs}
    spec = E.make_hash_spec(ngram, hpn, 29, mult, mods, offs, fill_id=3)
    got = gpu_hash(ids, spec)
    assert np.array_equal(got, oracle_hash(ids, ws, multipliers=mult))
    py = hash_ref.hash_input_ids(ids.tolist(), ngram, hpn, 29, 3, mult, mods, offs)
    assert np.array_equal(got, np.asarray(py, dtype=np.int64))


def test_large_moduli():
    """Moduli up to 2^62 exercise the full Barrett range."""
    rng = np.random.default_rng(9)
    mods = [(1 << 62), (1 << 62) - 57, (1 << 40) + 15, (1 << 33) - 9, 3, 2, 1000003, (1 << 31) - 1] * 2
    offs = [0] * 16
    ids = rng.integers(-(1 << 63), (1 << 63) - 1, size=(2, 500), dtype=np.int64)
    ws = {"ngram_size": 3, "heads_per_ngram": 8, "eos": C.EOS_TOKEN_ID, "fill": 0, "vocab_sizes": mods, "offsets": offs}
    got = gpu_hash(ids, E.make_hash_spec(3, 8, C.EOS_TOKEN_ID, C.LAYER_MULTIPLIERS, mods, offs))
    assert np.array_equal(got, oracle_hash(ids, ws))


def test_slice_equals_full_columns():
    """_forward_global_slice: a slice hashed with its global history equals the
    full hash's columns, across EOS and slice boundaries (context-parallel form)."""
    ids, lengths = W.long_context_stream(3, total=20000)
    t = torch.from_numpy(ids).cuda()
    spec = E.qwen3_8_flash_next_spec()
    ref = oracle_hash(ids, full_oracle_spec())          # the oracle's hash of the whole sequence
    full = E.engram_hash(t, spec).cpu().numpy()
    assert np.array_equal(full, ref)
    ends = np.cumsum(lengths)
    assert ids[0, int(ends[0]) - 1] == C.EOS_TOKEN_ID   # the cuts below straddle EOS positions
    cuts = [0, 1, 2, 3, 63, 64, 65, 2500, 19999, 20000] + [int(e) + d for e in ends[:3] for d in (-2, -1, 0, 1, 2)]
    for a in cuts:
        for b in (a, a + 1, a + 2, a + 64, a + 1000, 20000):
            if not (0 <= a <= b <= 20000):
                continue
            part = E.engram_hash_slice(t, a, b, spec).cpu().numpy()
            assert np.array_equal(part, ref[:, a:b]), (a, b)
            assert np.array_equal(part, full[:, a:b]), (a, b)
    # a batched slice: two independent rows
    ids2 = np.stack([ids[0, :5000], ids[0, 5000:10000]])
    t2 = torch.from_numpy(np.ascontiguousarray(ids2)).cuda()
    ref2 = oracle_hash(ids2, full_oracle_spec())
    part2 = E.engram_hash_slice(t2, 1234, 4321, spec).cpu().numpy()
    assert np.array_equal(part2, ref2[:, 1234:4321])
    assert np.array_equal(part2, E.engram_hash(t2, spec).cpu().numpy()[:, 1234:4321])


def test_rehash_in_backward():
    """Rows need not be kept from the forward: rows hashed again in the backward,
    slice by slice as context-parallel ranks would, give the same gradient bits."""
    ids, _ = W.long_context_stream(5, total=30000)
    t = torch.from_numpy(ids).cuda()
    spec = E.qwen3_8_flash_next_spec()
    kept = E.engram_hash(t, spec).reshape(-1)
    g = torch.Generator(device="cuda")
    g.manual_seed(9)
    dy = torch.randn((kept.numel(), 160), generator=g, device="cuda").to(torch.bfloat16)
    ur, ug = E.engram_scatter_add(kept, dy, W.FULL_ROWS)
    again = torch.cat([E.engram_hash_slice(t, a, b, spec).reshape(-1)
                       for a, b in ((0, 7000), (7000, 7001), (7001, 30000))])
    assert np.array_equal(again.cpu().numpy(), oracle_hash(ids, full_oracle_spec()).reshape(-1))
    ur2, ug2 = E.engram_scatter_add(again, dy, W.FULL_ROWS)
    assert torch.equal(ur, ur2)
    assert torch.equal(ug.view(torch.int32), ug2.view(torch.int32))


def test_empty():
    spec = E.qwen3_8_flash_next_spec()
    out = E.engram_hash(torch.empty((0, 5), dtype=torch.int64, device="cuda"), spec)
    assert out.shape == (0, 5, 16)
    out = E.engram_hash(torch.empty((3, 0), dtype=torch.int64, device="cuda"), spec)
    assert out.shape == (3, 0, 16)
