"""The oracle's derived table constants against the values the pages print."""
from oracle import constants as C


def test_printed_prime_prefix(golden_constants):
    derived = C.head_vocab_sizes()
    printed = golden_constants["head_vocab_sizes_prefix"]
    assert len(derived) == 16
    assert list(derived[:len(printed)]) == printed


def test_printed_offset_prefix(golden_constants):
    offs = C.head_offsets()
    printed = golden_constants["head_offsets_prefix"]
    assert list(offs[:len(printed)]) == printed
    lead = str(golden_constants["head_offset_9_leading_digits"][0])
    assert str(offs[len(printed)]).startswith(lead)


def test_padded_rows(golden_constants):
    r = C.padded_rows()
    assert r == golden_constants["padded_rows"][0]
    for g in golden_constants["owner_group_sizes"]:
        assert r % g == 0
    # the padding is less than one multiple: the table is the summed heads, rounded up
    assert 0 <= r - sum(C.head_vocab_sizes()) < C.PAD_MULTIPLE


def test_head_layout(golden_constants):
    assert C.NGRAM_SIZE == golden_constants["ngram_size"][0]
    assert C.HEADS_PER_NGRAM == golden_constants["heads_per_ngram"][0]
    assert C.EOS_TOKEN_ID == golden_constants["eos_token_id"][0]
    assert C.EMBEDDING_DIM == golden_constants["embedding_dim"][0]
    assert list(C.LAYER_MULTIPLIERS) == golden_constants["layer_multipliers"]
    sizes = C.head_vocab_sizes()
    assert all(C.is_prime(p) for p in sizes)
    assert sorted(set(sizes)) == list(sizes)            # distinct, increasing
    # consecutive: no prime is skipped between the base and the last head
    assert [p for p in range(C.PRIME_BASE, sizes[-1] + 1) if C.is_prime(p)] == list(sizes)


def test_is_prime_against_sieve():
    n = 5000
    sieve = [True] * n
    sieve[0] = sieve[1] = False
    for i in range(2, n):
        if sieve[i]:
            for j in range(i * i, n, i):
                sieve[j] = False
    assert [i for i in range(n) if sieve[i]] == [i for i in range(n) if C.is_prime(i)]
