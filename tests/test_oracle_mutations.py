"""Planted mistakes in the Python hash oracle must each fail at least one pin.

Every mutant is a plausible slip (wrong EOS side, wrong shift, swapped
multipliers, truncating remainder, missing offset, head groups swapped, no
64-bit wrap, dropped trigram term).  A pin set that let one through would not
pin the oracle.  Mutants live only in this test, on the CPU."""
import numpy as np
import pytest

from oracle import constants as C, hash_ref
from tests import oracle_pins as P
from tests.test_oracle_hash import full_spec, py_hash, tiny_spec


def shift_reset_before_eos(ids, shift, eos, fill):
    out = []
    for t in range(len(ids)):
        if t < shift or eos in ids[t - shift + 1:t + 1]:
            out.append(fill)
        else:
            out.append(ids[t - shift])
    return out


def shift_off_by_one(ids, shift, eos, fill):
    return hash_ref.__dict__["_orig_shift"](ids, shift - 1, eos, fill) if shift > 1 else list(ids)


def shift_fill_eos(ids, shift, eos, fill):
    return hash_ref.__dict__["_orig_shift"](ids, shift, eos, eos)


def make_row_mutant(kind):
    orig = hash_ref.hash_row

    def hash_row(ids, ngram_size, heads_per_ngram, eos, fill, multipliers, vocab_sizes, offsets):
        mult = list(multipliers)
        if kind == "swap_mult":
            mult[1], mult[2] = mult[2], mult[1]
        shifted = [ids] + [hash_ref.shift_right_after_eos(ids, s, eos, fill) for s in range(1, ngram_size)]
        out = []
        for t in range(len(ids)):
            prods = [hash_ref.wrap_int64(shifted[k][t] * mult[k]) for k in range(ngram_size)]
            if kind == "no_wrap":
                prods = [shifted[k][t] * mult[k] for k in range(ngram_size)]
            rows = []
            mix = prods[0]
            for order in range(2, ngram_size + 1):
                if not (kind == "drop_trigram" and order == 3):
                    mix = mix ^ prods[order - 1]
                for j in range(heads_per_ngram):
                    h = (order - 2) * heads_per_ngram + j
                    if kind == "swap_groups":
                        h = ((order - 1) % (ngram_size - 1)) * heads_per_ngram + j
                    p = vocab_sizes[h]
                    r = mix % p
                    if kind == "trunc_mod" and mix < 0 and r:
                        r -= p
                    rows.append(r + (0 if kind == "no_offset" else offsets[h]))
            out.append(rows)
        return out
    return hash_row


SHIFT_MUTANTS = {"reset_before_eos": shift_reset_before_eos, "off_by_one": shift_off_by_one,
                 "fill_is_eos": shift_fill_eos}
ROW_MUTANTS = ["swap_mult", "no_wrap", "drop_trigram", "swap_groups", "trunc_mod", "no_offset"]


def run_pins():
    msgs = []
    for spec in (tiny_spec(), full_spec()):
        msgs += P.all_pins(py_hash, spec, np.random.default_rng(5))
        rng = np.random.default_rng(6)
        ids = rng.integers(-2**63, 2**63 - 1, size=(2, 16), dtype=np.int64)
        msgs += [m for m in [P.pin_range(py_hash, dict(spec, fill=-1), ids)] if m]
    return msgs


@pytest.mark.parametrize("name", sorted(SHIFT_MUTANTS))
def test_shift_mutant_caught(monkeypatch, name):
    monkeypatch.setitem(hash_ref.__dict__, "_orig_shift", hash_ref.shift_right_after_eos)
    monkeypatch.setattr(hash_ref, "shift_right_after_eos", SHIFT_MUTANTS[name])
    assert run_pins(), "mutant %s passed every pin" % name


@pytest.mark.parametrize("kind", ROW_MUTANTS)
def test_row_mutant_caught(monkeypatch, kind):
    monkeypatch.setattr(hash_ref, "hash_row", make_row_mutant(kind))
    assert run_pins(), "mutant %s passed every pin" % kind


def test_unmutated_passes():
    assert run_pins() == []
