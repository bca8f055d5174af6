"""Host-side parts of bench.py (CPU only): the request chunks its CPU baseline
times give the same outputs as the whole batch, and the pool leg runs."""

import numpy as np

import bench
import oracle
from synth import make_config


def _concat(outs):
    return (np.concatenate([o.tokens for o in outs]), np.concatenate([o.num_accepted for o in outs]))


def test_sub_batches_reproduce_the_whole_batch():
    for n, kw in ((4, dict(vocab=900, batch=13)), (5, dict(vocab=700, batch=17))):
        inp = make_config(n, replicate=2, **kw)
        whole = oracle.verify(inp)
        cuts = [0, 3, 4, 9, inp.batch]
        parts = [oracle.verify(bench.sub_batch(inp, a, b)) for a, b in zip(cuts[:-1], cuts[1:])]
        tok, num = _concat(parts)
        assert np.array_equal(tok, whole.tokens) and np.array_equal(num, whole.num_accepted)


def test_cpu_baseline_pool_leg_runs():
    inp = make_config(3, replicate=1, vocab=4096, batch=8)
    r = bench.cpu_baseline(inp, budget_s=0.2, max_workers=2)
    assert r["kind"] == "oracle" and r["cores"] == 2 and r["value"] > 0
    assert r["one_core"]["cores"] == 1 and r["one_core"]["value"] > 0
    assert r["host_cpu_count"] >= 1
