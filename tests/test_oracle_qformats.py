"""Pins of the oracle's sparse / point-mass draft distributions and of its
acceptance counters (CPU only).

* A sparse q is the dense q that holds the listed probabilities at the listed
  ids and zero elsewhere: checked against a hand-written example, and by
  running the oracle on the same q stored both ways.
* A point-mass q (a draft proposed without a draft model: prompt lookup, the
  spec-decoding page's section 7) accepts the drafted token with probability
  p(x) and otherwise draws from p without x, so the emitted token follows p
  exactly; checked on a dyadic p with an exact stratified grid.
* The acceptance counters are checked against hand-computed values and
  against invariants that tie them to num_accepted and gamma_b.
"""

import dataclasses
import json
import os

import numpy as np
import pytest

import oracle
from synth import make_point_config, make_sparse_config, to_point, to_sparse
from synth.workloads import CONFIGS, make_inputs
from tests.helpers import explicit_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_sparse_q_golden_example():
    g = _golden("sparse_q_example.json")
    ids = np.array(g["topk_ids"], dtype=np.int32)
    pr = np.array(g["topk_probs"], dtype=np.float32)
    D = len(ids)
    inp = explicit_inputs(np.zeros((1, D + 1, g["vocab"])), np.zeros((1, D, g["vocab"])),
                          np.zeros((1, D), int), [1.0], np.zeros((1, D + 2)))
    inp = dataclasses.replace(inp, draft_probs=None, q_format="sparse", topk_ids=ids, topk_probs=pr)
    q = oracle.draft_q_rows(inp, np.arange(D))
    assert np.array_equal(q, np.array(g["dense"]))
    # rows in any order
    assert np.array_equal(oracle.draft_q_rows(inp, [2, 0]), np.array(g["dense"])[[2, 0]])


@pytest.mark.parametrize("bad", [[[4, 4, 1]], [[6, -1, 1]], [[-2, -1, 1]]])
def test_sparse_q_rejects_repeated_or_out_of_range_ids(bad):
    ids = np.array(bad, dtype=np.int32)
    inp = explicit_inputs(np.zeros((1, 2, 6)), np.zeros((1, 1, 6)), [[0]], [1.0], np.zeros((1, 3)))
    inp = dataclasses.replace(inp, draft_probs=None, q_format="sparse", topk_ids=ids,
                              topk_probs=np.full((1, 3), 0.25, dtype=np.float32))
    with pytest.raises(ValueError):
        oracle.draft_q_rows(inp, [0])


def test_point_mass_q_is_the_drafted_token():
    inp = explicit_inputs(np.zeros((2, 3, 5)), np.zeros((2, 2, 5)), [[3, 0], [4, 4]], [1.0, 1.0],
                          np.zeros((2, 4)))
    inp = to_point(inp)
    q = oracle.draft_q_rows(inp, np.arange(4))
    want = np.zeros((4, 5))
    want[[0, 1, 2, 3], [3, 0, 4, 4]] = 1.0
    assert np.array_equal(q, want)


def test_point_mass_draft_emits_p_exactly():
    """x proposed with certainty: P(emit x) = p(x) (accept), P(emit y != x) =
    (1 - p(x)) * p(y) / (1 - p(x)) = p(y).  Dyadic p with 1 - p(x) a power of
    two makes both laws exact on a 16-point stratified grid of each uniform."""
    p = np.array([0.25, 0.5, 0.125, 0.125])
    V, N = 4, 16
    grid = (np.arange(N) + 0.5) / N
    u0, v = np.meshgrid(grid, grid, indexing="ij")
    n = u0.size
    logits = np.broadcast_to(np.log(p), (n, 2, V)).astype(np.float32)
    u = np.stack([u0.ravel(), v.ravel(), v.ravel()], axis=1)
    inp = to_point(explicit_inputs(logits, np.zeros((n, 1, V)), np.ones((n, 1), int), np.ones(n), u))
    o = oracle.verify(inp)
    assert np.mean(o.num_accepted == 1) == p[1]
    assert np.array_equal(np.bincount(o.tokens[:, 0], minlength=V) / n, p)
    # a rejection never redraws the drafted token
    assert not np.any(o.tokens[o.num_accepted == 0, 0] == 1)


def _same_outputs(a, b):
    assert np.array_equal(a.tokens, b.tokens)
    assert np.array_equal(a.num_accepted, b.num_accepted)
    assert np.array_equal(a.ratio, b.ratio, equal_nan=True)


def test_sparse_and_dense_storage_of_one_q_agree():
    """The top-50 workload's q stored dense and as 50 (id, prob) entries."""
    spec = CONFIGS[5].with_(q_mode="topk", vocab=3000, batch=24)
    dense = make_inputs(spec, seed=77)
    sparse = to_sparse(dense, 50, seed=3)
    assert sparse.draft_probs is None and sparse.topk_ids.shape == (dense.total_draft, 50)
    _same_outputs(oracle.verify(dense), oracle.verify(sparse))


def test_point_and_one_hot_dense_q_agree():
    spec = CONFIGS[3].with_(q_mode="argmax", vocab=4000, batch=16)
    dense = make_inputs(spec, seed=78)
    assert np.all(dense.draft_probs.sum(axis=1) == 1.0)
    _same_outputs(oracle.verify(dense), oracle.verify(to_point(dense)))


def test_sparse_and_point_workloads_build():
    s = make_sparse_config(vocab=2000, batch=12)
    assert s.q_format == "sparse" and np.all((s.topk_ids >= -1) & (s.topk_ids < 2000))
    p = make_point_config(vocab=2000, batch=4)
    assert p.q_format == "point" and p.draft_probs is None
    oracle.verify(s)
    oracle.verify(p)


def test_acceptance_stats_golden():
    g = _golden("acceptance_stats_example.json")
    got = oracle.acceptance_stats(np.array(g["num_accepted"]), np.array(g["gammas"]), g["gamma"])
    assert got.tolist() == g["stats"]


def test_acceptance_stats_invariants():
    inp = make_inputs(CONFIGS[5].with_(vocab=1500, batch=64), seed=79)
    o = oracle.verify(inp)
    G, gam, k = inp.gamma, inp.gammas, o.num_accepted.astype(np.int64)
    s = oracle.acceptance_stats(k, gam, G)
    hist = s[4:5 + G]
    tested, accepted = s[5 + G:5 + 2 * G], s[5 + 2 * G:]
    assert s[0] == inp.batch == hist.sum()
    assert s[1] == gam.sum() and s[2] == k.sum() == (np.arange(G + 1) * hist).sum() == accepted.sum()
    assert s[3] == np.sum(k == gam)
    # a tested draft is accepted or is the request's first rejection
    rejected_at = np.bincount(k[k < gam], minlength=G)[:G]
    assert np.array_equal(tested - accepted, rejected_at)


def test_draft_side_sampling_is_categorical():
    """With gamma = 0 the step is a batched categorical draw from softmax(l / T)
    (the draft-side sampler x ~ q of the spec-decoding page's section 3.1): on a
    dyadic p and an exact 64-point stratified grid the sampled law is p."""
    p = np.array([0.5, 0.25, 0.125, 0.0625, 0.0625])
    V, N = 5, 64
    grid = (np.arange(N) + 0.5) / N
    logits = np.broadcast_to(np.log(p), (N, 1, V)).astype(np.float32)
    u = np.stack([np.zeros(N), grid], axis=1)
    o = oracle.verify(explicit_inputs(logits, np.zeros((N, 0, V)), np.zeros((N, 0), int), np.ones(N), u))
    assert np.all(o.num_accepted == 0) and np.all(o.draw_kind == 2)
    assert np.array_equal(np.bincount(o.tokens[:, 0], minlength=V) / N, p)


def test_sample_workload_builds():
    from synth import make_sample_config
    s = make_sample_config(batch=3, vocab=777)
    assert s.gamma == 0 and s.total_draft == 0 and s.uniforms.shape == (3, 2)
    assert np.all(oracle.verify(s).tokens[:, 0] >= 0)
