"""Oracle constants of the Qwen3.8-Flash-Next Engram table — test infrastructure.

Derived from their definition, not copied from the product package:

* Head moduli: the engram API page (data ``QWEN3_8_FLASH_NEXT_NGRAM_HEAD_VOCAB_SIZES``
  and the ``ngram_heads_vocab_sizes`` parameter of
  ``Qwen3_8_FlashNextNGramEmbedding``) gives one prime per head; the printed
  tuple shows the first eight and they are exactly the eight consecutive
  primes above 20,000,000.  The tuple is cut off after them; the reading taken
  here is that the sixteen heads use the sixteen consecutive primes above
  20,000,000 (the tests pin the eight printed ones and the printed total).
* Head offsets: data ``QWEN3_8_FLASH_NEXT_NGRAM_HEAD_OFFSETS`` is the global
  packed-table start of each head; the printed values are the prefix sums of
  the moduli.
* Padded rows: data ``QWEN3_8_FLASH_NEXT_NGRAM_PADDED_ROWS``; the table config
  (``Qwen3_8_FlashNextEngramTableConfig.num_embeddings``) must divide by the
  owner group size, which is 64 or 128 on the model-coverage page (Validated
  Configuration, "Engram ownership").  Rounding the summed moduli up to a
  multiple of 128 is the reading taken here.
* Multipliers: data ``QWEN3_8_FLASH_NEXT_LAYER_MULTIPLIERS`` is printed whole;
  it is input data, kept here as printed.
"""

NGRAM_SIZE = 3          # engram API page, Qwen3_8_FlashNextNGramEmbedding(ngram_size=3)
HEADS_PER_NGRAM = 8     # same signature, heads_per_ngram=8
EOS_TOKEN_ID = 248044   # same signature, eos_token_id=248044
EMBEDDING_DIM = 160     # model-coverage page, Architecture: rows of width 160
LAYER_MULTIPLIERS = (23703573157769, 20109073645365, 8052911324071)
PRIME_BASE = 20_000_000
PAD_MULTIPLE = 128


def is_prime(n):
    """Trial division; exact for every n the oracle needs (n < 2**31)."""
    if n < 2:
        return False
    if n % 2 == 0:
        return n == 2
    d = 3
    while d * d <= n:
        if n % d == 0:
            return False
        d += 2
    return True


def consecutive_primes_above(base, count):
    out = []
    n = base + 1
    while len(out) < count:
        if is_prime(n):
            out.append(n)
        n += 1
    return tuple(out)


def head_vocab_sizes():
    heads = (NGRAM_SIZE - 1) * HEADS_PER_NGRAM
    return consecutive_primes_above(PRIME_BASE, heads)


def head_offsets(vocab_sizes=None):
    if vocab_sizes is None:
        vocab_sizes = head_vocab_sizes()
    offs, acc = [], 0
    for p in vocab_sizes:
        offs.append(acc)
        acc += p
    return tuple(offs)


def padded_rows(vocab_sizes=None, multiple=PAD_MULTIPLE):
    if vocab_sizes is None:
        vocab_sizes = head_vocab_sizes()
    total = sum(vocab_sizes)
    return -(-total // multiple) * multiple
