"""Oracle for the Engram n-gram embedding hot path — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct CPU implementation of what the path computes:

* ``constants``   — the Qwen3.8-Flash-Next head primes, offsets and padded row
  count, derived from their definition (consecutive primes, prefix sums).
* ``hash_ref``    — pure-Python hash of raw token IDs into 16 head rows
  (arbitrary-precision integers with explicit 64-bit wrapping).
* ``c_oracle``    — ctypes wrapper of ``engram_oracle.c``: the same hash in
  scalar C, the row gather, and the gradient scatter-add with fp64 sums.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import anything here.  The product package never does, and
this package imports nothing from it: the two share no code, headers, helpers
or constant generators.  The only module both sides use is ``workloads``,
which draws seeded inputs and holds none of the method's arithmetic.

Every function cites the passage of the pages it follows, by page title and
section ("engram API page" is the page titled
``nemo_automodel.components.models.qwen3_8_flash_next.engram``; the
"model-coverage page" is the page titled ``Qwen3.8-Flash-Next``).
"""
