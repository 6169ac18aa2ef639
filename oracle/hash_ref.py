"""Pure-Python oracle of the Engram n-gram hash — test infrastructure.

Follows ``Qwen3_8_FlashNextNGramEmbedding`` on the engram API page
(class description, ``_shift_right_after_eos``, ``_hash_input_ids``):

1. For every shift s = 1 .. ngram_size-1, read the token s positions back
   without crossing an EOS boundary; positions with no such token take the
   fill value.  Context resets *after* an EOS token, so an EOS token still sees
   its own predecessors and the token after it starts a new segment.
2. Multiply the current token and each shifted token by its signed int64
   layer multiplier with 64-bit wrap-around ("signed int64 overflow").
3. The order-n mix combines the products of the current token and the n-1
   preceding ones; the combining operator is 64-bit XOR (reading: the
   multiplicative-XOR hash of the Engram design the model-coverage page's
   References cite; the pages do not print the operator).
4. Head h of order n takes the positive remainder of the order-n mix modulo
   the head's prime and adds the head's global offset.  The first
   heads_per_ngram heads are the bigram heads, the next group the trigram
   heads, and so on.

Arbitrary-precision integers make every step explicit: ``wrap_int64`` is the
only place a result is reduced to 64 bits, and Python's ``%`` with a positive
divisor is the floor remainder the pages ask for.
"""

MOD64 = 1 << 64


def wrap_int64(v):
    """Reduce an integer to signed 64-bit two's complement (multiplication overflow)."""
    v %= MOD64
    return v - MOD64 if v >= (1 << 63) else v


def shift_right_after_eos(ids, shift, eos, fill):
    """``_shift_right_after_eos`` for one batch row (a list of ints).

    out[t] = ids[t-shift] when t >= shift and none of ids[t-shift .. t-1] is
    EOS; otherwise ``fill`` (the history lies before the sequence start or in
    an earlier segment).
    """
    out = []
    for t in range(len(ids)):
        if t < shift:
            out.append(fill)
            continue
        window = ids[t - shift:t]
        out.append(fill if eos in window else ids[t - shift])
    return out


def hash_row(ids, ngram_size, heads_per_ngram, eos, fill, multipliers, vocab_sizes, offsets):
    """``_hash_input_ids`` for one batch row -> list of per-position head-row lists."""
    heads = (ngram_size - 1) * heads_per_ngram
    assert len(multipliers) >= ngram_size
    assert len(vocab_sizes) == heads and len(offsets) == heads
    shifted = [ids] + [shift_right_after_eos(ids, s, eos, fill) for s in range(1, ngram_size)]
    out = []
    for t in range(len(ids)):
        products = [wrap_int64(shifted[k][t] * multipliers[k]) for k in range(ngram_size)]
        rows = []
        mix = products[0]
        for order in range(2, ngram_size + 1):
            mix = mix ^ products[order - 1]
            for j in range(heads_per_ngram):
                h = (order - 2) * heads_per_ngram + j
                rows.append(mix % vocab_sizes[h] + offsets[h])
        out.append(rows)
    return out


def hash_input_ids(ids_2d, ngram_size, heads_per_ngram, eos, fill, multipliers, vocab_sizes, offsets):
    """``[batch][sequence]`` raw IDs -> ``[batch][sequence][heads]`` global rows.

    Each batch row is hashed on its own; a packed (THD) stream is one batch
    row whose documents are separated only by EOS.
    """
    return [hash_row(list(r), ngram_size, heads_per_ngram, eos, fill, multipliers, vocab_sizes, offsets)
            for r in ids_2d]
