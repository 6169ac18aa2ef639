"""Seeded synthetic inputs shaped like the pages' workloads.

Shared by the product tests, the benchmark and the oracle tests.  This module
draws token streams, table values and output gradients, and builds the
per-head modulus lists of the small test tables.  It holds none of the
method's arithmetic: no context shifting, no mixing, no remainders, no lookup
and no gradient sums.

The pages train on HellaSwag (non-packed, right-tail padded to 4,096 tokens)
and packed (THD) Tulu-3 SFT (model-coverage page, Validated Configuration).
Neither dataset is used; these generators reproduce only their shapes:
right-padded 4,096-token rows and EOS-separated packed documents, with Zipf
token frequencies over the 248,320-entry vocabulary.
"""
import numpy as np

VOCAB = 248_320          # tokenizer vocabulary of the token streams
EOS = 248_044            # engram API page, Qwen3_8_FlashNextNGramEmbedding(eos_token_id=248044)
DIM = 160                # model-coverage page, Architecture: table rows of width 160
FULL_ROWS = 320_001_536  # engram API page, QWEN3_8_FLASH_NEXT_NGRAM_PADDED_ROWS
OWNER_WORLD = 64         # model-coverage page, Validated Configuration: 64 contiguous shards
OWNER_ROWS = FULL_ROWS // OWNER_WORLD
HC_COUNT = 4             # model-coverage page, Architecture: four persistent HyperConnection streams
HC_WIDTH = 2_560         # ... each 2,560 wide (the width of one branch, the grouped norm's group)

_zipf_cdf_cache = {}


def _zipf_cdf(s, vocab):
    key = (s, vocab)
    if key not in _zipf_cdf_cache:
        w = np.arange(1, vocab + 1, dtype=np.float64) ** (-s)
        c = np.cumsum(w)
        _zipf_cdf_cache[key] = c / c[-1]
    return _zipf_cdf_cache[key]


def zipf_token_ids(rng, size, s, vocab=VOCAB, exclude=EOS):
    """Token IDs k-1 with P(k) proportional to k**-s on [1, vocab] (exact bounded
    inverse CDF).  Draws equal to ``exclude`` are redrawn, so EOS appears only
    where a generator places it."""
    cdf = _zipf_cdf(s, vocab)
    out = np.searchsorted(cdf, rng.random(size), side="right").astype(np.int64)
    np.minimum(out, vocab - 1, out=out)
    bad = out == exclude
    while bad.any():
        redraw = np.searchsorted(cdf, rng.random(int(bad.sum())), side="right").astype(np.int64)
        np.minimum(redraw, vocab - 1, out=redraw)
        out[bad] = redraw
        bad = out == exclude
    return out


def _is_prime(n):
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


def _spec_from_moduli(moduli, eos, num_rows):
    offsets, acc = [], 0
    for p in moduli:
        offsets.append(acc)
        acc += p
    assert acc <= num_rows
    return {"ngram_size": 3, "heads_per_ngram": 8, "eos": int(eos), "fill": 0,
            "vocab_sizes": tuple(int(p) for p in moduli), "offsets": tuple(offsets),
            "num_rows": int(num_rows)}


# ---------------------------------------------------------------- Tiny case

TINY_EOS = 999


def tiny_spec():
    """16 distinct primes from [3800, 4400) picked with default_rng(0), sorted;
    offsets are their running totals; 65,152 rows (multiple of 128).  The
    caller supplies the layer multipliers."""
    primes = [p for p in range(3800, 4400) if _is_prime(p)]
    pick = sorted(np.random.default_rng(0).choice(primes, 16, replace=False).tolist())
    total = sum(pick)
    return _spec_from_moduli(pick, TINY_EOS, -(-total // 128) * 128)


def tiny_tokens(seed=0, seq=256):
    """[1, 256] uniform IDs in [0, 1000); each position independently EOS (999) with p = 1/64."""
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, 1000, size=(1, seq), dtype=np.int64)
    ids[rng.random((1, seq)) < 1.0 / 64] = TINY_EOS
    return ids


def tiny_table(num_rows, seed=1, dim=DIM):
    return np.random.default_rng(seed).normal(0.0, 0.02, size=(num_rows, dim)).astype(np.float32)


def tiny_grad(n, seed=2, dim=DIM):
    return np.random.default_rng(seed).standard_normal((n, dim)).astype(np.float32)


# ---------------------------------------------------------------- SFT shape

def sft_spec():
    """16 consecutive primes above 624,000 inside a 10,000,000-row table."""
    primes, p = [], 624_001
    while len(primes) < 16:
        if _is_prime(p):
            primes.append(p)
        p += 1
    return _spec_from_moduli(primes, EOS, 10_000_000)


def sft_batch(seed=0, batch=8, seq=4096, s=1.1, full_length=False):
    """[8, 4096] right-tail padded rows.  Row b has a real length L_b ~ U{512..4096}
    (4096 when ``full_length``) whose last token is EOS; positions after it are
    EOS padding.  Returns (ids, lengths)."""
    rng = np.random.default_rng(seed)
    lengths = np.full(batch, seq, dtype=np.int64) if full_length else \
        rng.integers(512, seq + 1, size=batch).astype(np.int64)
    ids = np.full((batch, seq), EOS, dtype=np.int64)
    for b in range(batch):
        L = int(lengths[b])
        ids[b, :L - 1] = zipf_token_ids(rng, L - 1, s)
    return ids, lengths


# ---------------------------------------------------------------- Owner shard

def owner_token_batches(seeds=range(100, 164), batch=8, seq=4096, s=1.2):
    """The 64 request ranks of a world-64 step: each [8, 4096] Zipf(1.2) rows of
    full length ending in EOS.  Returns int64 [64, 8, 4096]."""
    out = np.empty((len(seeds), batch, seq), dtype=np.int64)
    for k, sd in enumerate(seeds):
        ids, _ = sft_batch(sd, batch, seq, s, full_length=True)
        out[k] = ids
    return out


# ---------------------------------------------------------------- Long context

def long_context_stream(seed=0, total=262_144, s=1.1, lo=64, hi=16_384):
    """One packed THD row of ``total`` tokens.  Document lengths are
    floor(exp(U[ln lo, ln hi])); every document ends in EOS and the last one is
    cut to fit (still ending in EOS).  Returns (ids [1, total], doc_lengths)."""
    rng = np.random.default_rng(seed)
    lengths, used = [], 0
    while used < total:
        L = int(np.floor(np.exp(rng.uniform(np.log(lo), np.log(hi)))))
        L = max(1, min(L, total - used))
        lengths.append(L)
        used += L
    ids = zipf_token_ids(rng, total, s)
    ends = np.cumsum(lengths) - 1
    ids[ends] = EOS
    return ids.reshape(1, total), np.asarray(lengths, dtype=np.int64)


# ---------------------------------------------------------------- device tensors

def fill_normal_(tensor, seed, std=0.02, chunk_rows=1 << 22):
    """Fill a (possibly 100 GB) torch tensor in place with N(0, std), chunk by
    chunk, from one seeded generator on the tensor's device."""
    import torch
    g = torch.Generator(device=tensor.device)
    g.manual_seed(int(seed))
    rows = tensor.shape[0]
    for a in range(0, rows, chunk_rows):
        tensor[a:a + chunk_rows].normal_(0.0, std, generator=g)
    return tensor


def ple_tensors(dev, seed, batch, seq, channels=HC_COUNT * HC_WIDTH, dtype=None):
    """PLE-layer inputs on ``dev``: activations x and output gradients dy
    [batch, seq, channels] ~ N(0, 1) in bf16, one batch row's halo of the
    preceding 9 tokens, conv weights [channels, 4] ~ N(0, 0.5^2) and bias
    [channels] ~ N(0, 0.1^2), grouped-norm weights [channels] ~ N(0, 0.3^2)
    (fp32).  The pages start the conv and the norm weights at zero; random
    values here make every tap and scale visible in the results."""
    import torch
    dtype = dtype or torch.bfloat16
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed))
    shape = (batch, seq, channels)
    return {
        "x": torch.randn(shape, generator=g, device=dev).to(dtype),
        "dy": torch.randn(shape, generator=g, device=dev).to(dtype),
        "halo": torch.randn((batch, 9, channels), generator=g, device=dev).to(dtype),
        "conv_w": torch.randn((channels, 4), generator=g, device=dev) * 0.5,
        "conv_b": torch.randn(channels, generator=g, device=dev) * 0.1,
        "norm_w": torch.randn(channels, generator=g, device=dev) * 0.3,
    }
