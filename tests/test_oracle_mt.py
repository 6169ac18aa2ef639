"""The OpenMP twin of the oracle (the all-core CPU baseline) computes the same
bits as the single-threaded oracle: hash, gather (including the lowest
out-of-range lookup) and compact scatter-add (rows, fp64 sums in ascending
lookup order, lowest bad lookup), at several thread counts, on inputs with
EOS resets, hot rows, out-of-range rows and both gradient dtypes.  Each run
is a fresh process so that OMP_NUM_THREADS takes effect."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

from oracle import c_oracle, constants as C

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r'''
import sys, json
import numpy as np
sys.path.insert(0, %(root)r)
from oracle import c_oracle, constants as C
import workloads as W
rng = np.random.default_rng(%(seed)d)
mods, offs = C.head_vocab_sizes(), C.head_offsets()
ids, _ = W.long_context_stream(%(seed)d, total=6000)
ids2 = rng.integers(-(1 << 63), (1 << 63) - 1, size=(3, 700), dtype=np.int64)
ids2[:, ::7] = C.EOS_TOKEN_ID
out = {"threads": c_oracle.mt_threads()}
for name, x in (("long", ids), ("extreme", ids2)):
    for fill in (0, -1):
        a = c_oracle.hash_input_ids(x, 3, 8, C.EOS_TOKEN_ID, fill, C.LAYER_MULTIPLIERS, mods, offs)
        b = c_oracle.hash_input_ids_mt(x, 3, 8, C.EOS_TOKEN_ID, fill, C.LAYER_MULTIPLIERS, mods, offs)
        out["hash_%%s_%%d" %% (name, fill)] = bool(np.array_equal(a, b))
# hot rows: Zipf over a small shard, some rows out of range on both sides
R, row_begin = 5000, 1000
rows = (rng.zipf(1.2, size=40000) %% (R + 40)).astype(np.int64) + row_begin - 20
table = rng.integers(0, 1 << 16, size=(R, 160), dtype=np.uint64).astype(np.uint16)
g1, b1 = c_oracle.gather(table, rows, row_begin)
g2, b2 = c_oracle.gather_mt(table, rows, row_begin)
out["gather"] = bool(np.array_equal(g1, g2)) and b1 == b2 and b1 >= 0
good = rows[(rows >= row_begin) & (rows < row_begin + R)]
g3, b3 = c_oracle.gather_mt(table, good, row_begin)
out["gather_clean"] = b3 == -1 and bool(np.array_equal(g3, c_oracle.gather(table, good, row_begin)[0]))
for dt in ("bf16", "f32"):
    dy = (rng.integers(0, 1 << 16, size=(rows.size, 160), dtype=np.uint64).astype(np.uint16) if dt == "bf16"
          else rng.standard_normal((rows.size, 160)).astype(np.float32))
    if dt == "bf16":
        dy[(dy & 0x7F80) == 0x7F80] = 0          # no inf or nan patterns
    r1, s1, e1 = c_oracle.scatter_add_compact(rows, dy, R, row_begin)
    r2, s2, e2 = c_oracle.scatter_add_compact_mt(rows, dy, R, row_begin)
    out["scatter_" + dt] = (bool(np.array_equal(r1, r2)) and bool(np.array_equal(s1.view(np.uint64), s2.view(np.uint64)))
                            and e1 == e2 and e1 >= 0)
r1, s1, e1 = c_oracle.scatter_add_compact(np.zeros(0, np.int64), np.zeros((0, 160), np.float32), R)
r2, s2, e2 = c_oracle.scatter_add_compact_mt(np.zeros(0, np.int64), np.zeros((0, 160), np.float32), R)
out["scatter_empty"] = r2.size == 0 and e2 == -1 and e1 == -1
print(json.dumps(out))
'''


@pytest.mark.parametrize("threads", [1, 3, 8])
def test_mt_oracle_equals_single_threaded(threads):
    c_oracle.load_mt()      # built before the child processes start
    env = dict(os.environ, OMP_NUM_THREADS=str(threads))
    r = subprocess.run([sys.executable, "-c", CHILD % {"root": ROOT, "seed": threads}], env=env,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    res = json.loads(r.stdout.strip().splitlines()[-1])
    assert res.pop("threads") == threads
    assert all(res.values()), res
