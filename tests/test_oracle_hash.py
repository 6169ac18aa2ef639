"""Pins of the hash oracle (Python and C) — no GPU."""
import numpy as np
import pytest

import workloads as W
from oracle import c_oracle, constants as C, hash_ref
from tests import oracle_pins as P


def full_spec():
    return {"ngram_size": C.NGRAM_SIZE, "heads_per_ngram": C.HEADS_PER_NGRAM, "eos": C.EOS_TOKEN_ID,
            "fill": 0, "multipliers": C.LAYER_MULTIPLIERS, "vocab_sizes": C.head_vocab_sizes(),
            "offsets": C.head_offsets()}


def tiny_spec():
    s = dict(W.tiny_spec())
    s["multipliers"] = C.LAYER_MULTIPLIERS
    return s


def py_hash(ids, spec):
    return np.asarray(hash_ref.hash_input_ids(np.asarray(ids).tolist(), spec["ngram_size"],
                                              spec["heads_per_ngram"], spec["eos"], spec["fill"],
                                              spec["multipliers"], spec["vocab_sizes"], spec["offsets"]),
                      dtype=np.int64).reshape(np.shape(ids) + ((spec["ngram_size"] - 1) * spec["heads_per_ngram"],))


def c_hash(ids, spec):
    return c_oracle.hash_input_ids(np.asarray(ids, dtype=np.int64), spec["ngram_size"], spec["heads_per_ngram"],
                                   spec["eos"], spec["fill"], spec["multipliers"], spec["vocab_sizes"],
                                   spec["offsets"])


ORACLES = {"python": py_hash, "c": c_hash}


@pytest.mark.parametrize("which", sorted(ORACLES))
@pytest.mark.parametrize("specname", ["tiny", "full"])
def test_all_pins(which, specname):
    spec = tiny_spec() if specname == "tiny" else full_spec()
    msgs = P.all_pins(ORACLES[which], spec, np.random.default_rng(7))
    assert not msgs, msgs


@pytest.mark.parametrize("which", sorted(ORACLES))
def test_brute_force_length6(which):
    assert P.pin_brute_force(ORACLES[which], tiny_spec(), max_len=6) is None


def test_wrap_matches_numpy_int64():
    """64-bit wrap-around of the products equals numpy's native int64 multiply."""
    rng = np.random.default_rng(3)
    a = np.concatenate([rng.integers(-2**63, 2**63 - 1, size=2000, dtype=np.int64),
                        np.array([-2**63, 2**63 - 1, -1, 0, 1, 248044, 389113, -389113], dtype=np.int64)])
    for m in C.LAYER_MULTIPLIERS:
        with np.errstate(over="ignore"):
            ref = a * np.int64(m)
        got = [hash_ref.wrap_int64(int(x) * m) for x in a]
        assert got == ref.tolist()


def test_c_equals_python_extreme_inputs():
    """Random int64 IDs including negatives and values next to +-2**63, both fill values."""
    rng = np.random.default_rng(11)
    ids = rng.integers(-2**63, 2**63 - 1, size=(3, 64), dtype=np.int64)
    ids[:, :4] = [[-2**63, 2**63 - 1, -1, C.EOS_TOKEN_ID]] * 3
    ids[rng.random(ids.shape) < 0.05] = C.EOS_TOKEN_ID
    for fill in (0, -1, 2**63 - 1):
        spec = dict(full_spec(), fill=fill)
        assert np.array_equal(c_hash(ids, spec), py_hash(ids, spec))
        assert P.pin_range(c_hash, spec, ids) is None


def test_c_equals_python_workload_sample():
    ids, _ = W.sft_batch(0)
    ids = ids[:, :300]
    spec = full_spec()
    assert np.array_equal(c_hash(ids, spec), py_hash(ids, spec))


def test_range_on_workloads():
    spec = full_spec()
    ids, _ = W.long_context_stream(0)
    assert P.pin_range(c_hash, spec, ids) is None
    ids, _ = W.sft_batch(0)
    assert P.pin_range(c_hash, spec, ids) is None


def test_thd_rows_independent_of_batch_split():
    """Batch rows are hashed independently: hashing a [2, T] batch equals hashing
    each row alone; a packed row hashes like its EOS-terminated documents."""
    spec = full_spec()
    ids, lengths = W.long_context_stream(1, total=4096)
    whole = c_hash(ids, spec)[0]
    start = 0
    for L in lengths:
        doc = ids[:, start:start + L]
        assert np.array_equal(c_hash(doc, spec)[0], whole[start:start + L])
        start += L
    two = np.stack([ids[0, :2048], ids[0, 2048:]])
    assert np.array_equal(c_hash(two, spec)[0], c_hash(ids[:, :2048], spec)[0])
