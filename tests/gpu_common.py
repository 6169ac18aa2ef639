"""Shared helpers of the GPU parity tests: both sides' hash specs, dtype views,
the tolerance check.  The product side takes its constants from the binding,
the oracle side from the oracle's own derivation."""
import numpy as np
import pytest
import torch

import hashed_gram_embedding_engram_amd as E
import workloads as W
from oracle import c_oracle, constants as C

# Backward tolerance: fp32 results against the fp64 oracle, |got - ref| <= ATOL + RTOL * |ref|.
RTOL, ATOL = 1e-5, 1e-6


def gpu_available():
    try:
        return torch.cuda.is_available()
    except Exception:
        return False


requires_gpu = pytest.mark.skipif(not gpu_available(), reason="no GPU visible")


def full_oracle_spec(fill=0):
    return {"ngram_size": C.NGRAM_SIZE, "heads_per_ngram": C.HEADS_PER_NGRAM, "eos": C.EOS_TOKEN_ID, "fill": fill,
            "vocab_sizes": C.head_vocab_sizes(), "offsets": C.head_offsets(), "num_rows": C.padded_rows()}


def product_spec_from(ws, fill=None):
    """Binding spec for a workloads-built head layout (small test tables)."""
    return E.make_hash_spec(ws["ngram_size"], ws["heads_per_ngram"], ws["eos"], E.QWEN3_8_FLASH_NEXT_LAYER_MULTIPLIERS,
                            ws["vocab_sizes"], ws["offsets"], ws.get("fill", 0) if fill is None else fill)


def oracle_hash(ids, ws, fill=None, multipliers=None):
    return c_oracle.hash_input_ids(np.asarray(ids, dtype=np.int64), ws["ngram_size"], ws["heads_per_ngram"], ws["eos"],
                                   ws.get("fill", 0) if fill is None else fill,
                                   C.LAYER_MULTIPLIERS if multipliers is None else multipliers,
                                   ws["vocab_sizes"], ws["offsets"])


def to_host(t):
    """GPU tensor -> numpy; bf16 as uint16 bit patterns (the oracle's bf16 form)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def assert_close_to_fp64(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    err = np.abs(got - ref)
    bound = ATOL + RTOL * np.abs(ref)
    bad = err > bound
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError("%s: %d elements out of tolerance; first at %s: got %r ref %r" %
                             (what, int(bad.sum()), tuple(i), got[tuple(i)], ref[tuple(i)]))


def head_layout(base, gap=0, start=0, descending=False):
    """A 3-gram, 8-heads-per-order layout of 16 consecutive primes above `base`,
    the heads' ranges one after another from `start` (with `gap` rows between
    them), in head order or, with descending, in reverse head order."""
    vocab = C.consecutive_primes_above(base, 16)
    offsets, at = [0] * 16, start
    for h in (range(15, -1, -1) if descending else range(16)):
        offsets[h] = at
        at += vocab[h] + gap
    return {"ngram_size": 3, "heads_per_ngram": 8, "eos": 999, "fill": 0, "vocab_sizes": tuple(vocab),
            "offsets": tuple(offsets), "num_rows": at}
