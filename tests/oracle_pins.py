"""Pins of the hash oracle: facts fixed by the pages or by mathematics.

Each ``pin_*`` takes a hash function ``h(ids_2d, spec) -> int array [B, T, H]``
and returns None when the fact holds, else a message.  The oracle tests run
every pin on the Python and the C oracle; the mutation tests plant plausible
mistakes in the Python oracle and check that some pin fails.
"""
import itertools

import numpy as np


def heads_of(spec):
    return (spec["ngram_size"] - 1) * spec["heads_per_ngram"]


def pin_range(h, spec, ids):
    """Every row of head k lies in [offset_k, offset_k + vocab_k): the engram API
    page, Qwen3_8_FlashNextNGramEmbedding parameters ngram_heads_vocab_sizes /
    ngram_heads_offsets (prime modulus and global offset per head)."""
    rows = np.asarray(h(ids, spec))
    lo = np.asarray(spec["offsets"], dtype=np.int64)
    hi = lo + np.asarray(spec["vocab_sizes"], dtype=np.int64)
    if rows.shape != tuple(np.shape(ids)) + (heads_of(spec),):
        return "shape %s" % (rows.shape,)
    if not ((rows >= lo).all() and (rows < hi).all()):
        return "row outside its head range"
    return None


def pin_segment_start_closed_form(h, spec):
    """At a segment start every missing history token is the fill value 0, so
    every order's mix is the current token's product alone.  A token equal to
    head k's prime therefore has a mix divisible by that prime and lands on
    row offset_k exactly; token 0 lands on offset_k for every head.  Checked
    at position 0 and right after an EOS (context resets after EOS)."""
    assert spec["fill"] == 0
    eos = spec["eos"]
    H = heads_of(spec)
    rows = np.asarray(h(np.zeros((1, 1), dtype=np.int64), spec))
    if list(rows[0, 0]) != list(spec["offsets"]):
        return "token 0 at sequence start"
    for k in range(H):
        p = spec["vocab_sizes"][k]
        if p * max(abs(m) for m in spec["multipliers"]) >= 2 ** 63:
            continue  # product would wrap; the closed form needs no wrap
        seq = np.array([[p, 5, 7, eos, p]], dtype=np.int64)
        rows = np.asarray(h(seq, spec))
        if rows[0, 0, k] != spec["offsets"][k] or rows[0, 4, k] != spec["offsets"][k]:
            return "prime token at segment start, head %d" % k
    return None


def pin_wrap_closed_form(h, spec):
    """Signed 64-bit overflow (engram API page, class description): the token
    x = M0^-1 mod 2**64 (M0 is odd, so it has an inverse) has a product that
    wraps to exactly 1, and -x one that wraps to -1.  At a segment start
    (fill 0) they land on offset_k + 1 and, by the positive remainder, on
    offset_k + vocab_k - 1 for every head k."""
    assert spec["fill"] == 0
    m0 = spec["multipliers"][0]
    inv = pow(m0, -1, 1 << 64)
    x = inv - (1 << 64) if inv >= 1 << 63 else inv
    rows = np.asarray(h(np.array([[x], [-x]], dtype=np.int64), spec))
    offs = np.asarray(spec["offsets"], dtype=np.int64)
    sizes = np.asarray(spec["vocab_sizes"], dtype=np.int64)
    if not np.array_equal(rows[0, 0], offs + 1):
        return "product wrapping to +1"
    if not np.array_equal(rows[1, 0], offs + sizes - 1):
        return "product wrapping to -1"
    return None


def pin_eos_metamorphic(h, spec, rng, trials=20, alphabet=50):
    """Context resets after EOS: hash(prefix + [EOS] + s)[len(prefix)+1:] == hash(s)
    for any prefix; and the EOS token keeps its own history, so its rows differ
    from an EOS at a sequence start when its predecessor differs."""
    eos = spec["eos"]
    for _ in range(trials):
        p = rng.integers(0, alphabet, size=rng.integers(0, 6))
        s = rng.integers(0, alphabet, size=rng.integers(1, 8))
        a = np.concatenate([p, [eos], s]).astype(np.int64)[None]
        ra = np.asarray(h(a, spec))[0, len(p) + 1:]
        rb = np.asarray(h(s.astype(np.int64)[None], spec))[0]
        if not np.array_equal(ra, rb):
            return "prefix leaked across EOS"
    r1 = np.asarray(h(np.array([[3, eos]], dtype=np.int64), spec))[0, 1]
    r0 = np.asarray(h(np.array([[eos]], dtype=np.int64), spec))[0, 0]
    if np.array_equal(r1, r0):
        return "EOS token lost its own history"
    return None


def pin_locality(h, spec, rng, trials=20):
    """Row t depends on x[t], x[t-1] (bigram heads) and x[t-2] (trigram heads)
    only: the page's ngram_size counts the current token, and heads_per_ngram
    heads hash each order from two up (bigram heads first)."""
    hp = spec["heads_per_ngram"]
    for _ in range(trials):
        x = rng.integers(0, 1000, size=(1, 8)).astype(np.int64)
        x[x == spec["eos"]] = 1
        base = np.asarray(h(x, spec))[0, 6]
        for back, expect_bigram_change, expect_trigram_change in ((3, False, False), (2, False, True),
                                                                  (1, True, True), (0, True, True)):
            y = x.copy()
            y[0, 6 - back] += 1 + (y[0, 6 - back] + 1 == spec["eos"])
            r = np.asarray(h(y, spec))[0, 6]
            big_changed = not np.array_equal(r[:hp], base[:hp])
            tri_changed = not np.array_equal(r[hp:2 * hp], base[hp:2 * hp])
            if big_changed != expect_bigram_change:
                return "bigram heads vs token t-%d" % back
            # a trigram mix can still collide mod a small prime; require most heads to move
            if expect_trigram_change and (r[hp:2 * hp] == base[hp:2 * hp]).sum() > 2:
                return "trigram heads ignore token t-%d" % back
            if not expect_trigram_change and tri_changed:
                return "trigram heads see token t-%d" % back
    return None


def _wrap(v):
    v %= 1 << 64
    return v - (1 << 64) if v >= 1 << 63 else v


def brute_force_rows(seq, spec):
    """Segment-based statement of the hash, written independently of the oracle's
    shift-based one: the n-gram ending at t is the last n tokens of t's
    segment (the segment starts after the latest EOS strictly before t), padded
    on the left with the fill value; its mix is the XOR of the wrapped products
    of token k-back with multiplier k."""
    eos, fill, M = spec["eos"], spec["fill"], spec["multipliers"]
    out = []
    for t in range(len(seq)):
        start = 0
        for u in range(t):
            if seq[u] == eos:
                start = u + 1
        rows = []
        for order in range(2, spec["ngram_size"] + 1):
            gram = [seq[t - k] if t - k >= start else fill for k in range(order)]
            mix = 0
            for k, tok in enumerate(gram):
                mix ^= _wrap(tok * M[k])
            for j in range(spec["heads_per_ngram"]):
                hh = (order - 2) * spec["heads_per_ngram"] + j
                rows.append(mix % spec["vocab_sizes"][hh] + spec["offsets"][hh])
        out.append(rows)
    return out


def pin_brute_force(h, spec, max_len=6, alphabet=(0, 1, 2)):
    """Every sequence over a small alphabet plus EOS up to ``max_len`` tokens,
    against the segment-based statement, all sequences of one length batched."""
    letters = list(alphabet) + [spec["eos"]]
    for L in range(1, max_len + 1):
        seqs = np.array(list(itertools.product(letters, repeat=L)), dtype=np.int64)
        got = np.asarray(h(seqs, spec))
        for i, s in enumerate(seqs.tolist()):
            if got[i].tolist() != brute_force_rows(s, spec):
                return "sequence %s" % s
    return None


def all_pins(h, spec, rng):
    msgs = []
    ids = rng.integers(-5, 2000, size=(3, 40)).astype(np.int64)
    ids[rng.random(ids.shape) < 0.1] = spec["eos"]
    for name, fn in (("range", lambda: pin_range(h, spec, ids)),
                     ("closed_form", lambda: pin_segment_start_closed_form(h, spec)),
                     ("wrap", lambda: pin_wrap_closed_form(h, spec)),
                     ("eos", lambda: pin_eos_metamorphic(h, spec, rng)),
                     ("locality", lambda: pin_locality(h, spec, rng)),
                     ("brute_force", lambda: pin_brute_force(h, spec, max_len=5))):
        m = fn()
        if m:
            msgs.append("%s: %s" % (name, m))
    return msgs
