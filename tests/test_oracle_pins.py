"""Pins of the CPU oracle against facts fixed by the page and by mathematics.

Each test states what it pins and where that fact comes from; none of them
re-derives the oracle's own formula.  The page is the spec-decoding page at
dpshk.com/news/5598276 (sections cited as [page §n]).
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
from oracle.rejection_sampler import DRAW_BONUS, DRAW_DEGENERATE, DRAW_NONE, DRAW_RESIDUAL
from tests.helpers import U_STEP, explicit_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- worked example
def test_worked_example_from_figure():
    """[page §4] figure: ratios 0.92, 0.75, 0.31 (die 0.31) -> 2 accepted, 3 tokens."""
    ex = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    g = ex["gamma"]
    V = 8
    logits = np.zeros((1, g + 1, V), dtype=np.float32)      # p = 1/8 exactly in every row
    ids = np.array([[1, 2, 3, 4, 5]], dtype=np.int32)
    q = np.full((1, g, V), 0.0, dtype=np.float32)
    u = np.zeros((1, g + 2), dtype=np.float32)
    for i, (ratio, die) in enumerate(zip(ex["ratios"], ex["uniforms_accept"])):
        qx = np.float32(0.125 / ratio)
        u32 = np.float32(die)
        # a die equal to the printed ratio must not fall below the computed ratio
        while 0.125 / float(qx) > float(u32) and die == ratio:
            qx = np.nextafter(qx, np.float32(1.0))
        q[0, i, :] = (1.0 - qx) / (V - 1)
        q[0, i, ids[0, i]] = qx
        u[0, i] = u32
    u[0, g] = 0.4
    u[0, g + 1] = 0.9
    o = oracle.verify(explicit_inputs(logits, q, ids, [1.0], u))
    assert o.num_accepted[0] == ex["expected_num_accepted"]
    emitted = o.tokens[0][o.tokens[0] >= 0]
    assert len(emitted) == ex["expected_emitted_tokens"]
    assert list(o.tokens[0, :2]) == [1, 2]
    assert o.draw_kind[0] == DRAW_RESIDUAL
    assert np.allclose(o.ratio[:3], ex["ratios"][:3], rtol=1e-6)
    # the residual at position 3 is (1/8 - q)_+ : zero at the drafted token
    assert o.tokens[0, 2] != 3
    assert list(o.tokens[0, 3:]) == [-1, -1, -1]


# ---------------------------------------------------------------- exact tie
@pytest.mark.parametrize("u0, accepted", [(0.25, False), (0.25 - U_STEP, True)])
def test_exact_tie_rejects(u0, accepted):
    """[page §5.2] the accept comparison is strict: a die equal to the ratio rejects.

    Equal logits at T = 1 give p = 1/8 exactly; q(x) = 1/2 gives ratio 1/4 exactly.
    """
    V, g = 8, 1
    logits = np.zeros((1, g + 1, V), dtype=np.float32)
    q = np.full((1, g, V), 0.5 / 7, dtype=np.float32)
    q[0, 0, 3] = 0.5
    ids = np.array([[3]])
    u = np.array([[u0, 0.5, 0.5]], dtype=np.float32)
    o = oracle.verify(explicit_inputs(logits, q, ids, [1.0], u))
    assert o.ratio[0] == 0.25
    assert o.num_accepted[0] == (1 if accepted else 0)


# ---------------------------------------------------------------- normaliser
@pytest.mark.parametrize("T", [0.3, 1.0, 2.5])
def test_equal_logits_normaliser_is_V(T):
    """Equal logits: every exp((l - max l)/T) is exp(0) = 1, so Z = V exactly."""
    V, g = 1000, 2
    logits = np.full((1, g + 1, V), 1.75, dtype=np.float32)
    q = np.full((1, g, V), 1.0 / V, dtype=np.float32)
    o = oracle.verify(explicit_inputs(logits, q, [[0, 1]], [T], np.zeros((1, g + 2))))
    assert np.all(o.row_norm == V)
    assert np.all(o.row_max == 1.75)


def test_normaliser_matches_logsumexp():
    """log Z + m/T = logsumexp(l/T) (scipy), and m is the max raw logit."""
    rng = np.random.default_rng(5)
    V, g, B = 3000, 3, 4
    logits = rng.normal(0, 3, size=(B, g + 1, V)).astype(np.float32)
    T = np.array([0.3, 0.8, 1.0, 1.7])
    q = np.full((B, g, V), 1.0 / V, dtype=np.float32)
    o = oracle.verify(explicit_inputs(logits, q, np.zeros((B, g), int), T, np.zeros((B, g + 2))))
    l64 = logits.astype(np.float64).reshape(B * (g + 1), V)
    Tr = np.repeat(T.astype(np.float32).astype(np.float64), g + 1)   # T is an fp32 input
    lse = scipy.special.logsumexp(l64 / Tr[:, None], axis=-1)
    assert np.allclose(np.log(o.row_norm) + o.row_max / Tr, lse, rtol=0, atol=1e-12)
    assert np.array_equal(o.row_max, l64.max(-1))


# ---------------------------------------------------------------- inverse CDF
def test_inverse_cdf_half_open_intervals():
    """Hand-computed intervals for w = [1, 0, 2, 1] / 4 (S = 4):
    [0, 1/4) -> 0, [1/4, 3/4) -> 2 (the zero-weight token 1 is skipped and the
    boundary 1/4 belongs to the next token), [3/4, 1) -> 3."""
    w = np.array([1.0, 0.0, 2.0, 1.0])
    for k in range(64):
        v = k / 64
        expect = 0 if v < 0.25 else (2 if v < 0.75 else 3)
        y, S, fb = oracle.inverse_cdf(w, v)
        assert int(y) == expect and S == 4.0 and not fb
    y, _, _ = oracle.inverse_cdf(np.array([0.0, 0.0, 3.0, 0.0]), 0.0)
    assert int(y) == 2                       # leading zero weights are never chosen
    y, _, _ = oracle.inverse_cdf(np.array([0.5, 0.5]), 1 - U_STEP)
    assert int(y) == 1


# ---------------------------------------------------------------- invariants
def _bonus_by_hand(w, v):
    acc = 0.0
    S = math.fsum(w)
    for x, wx in enumerate(w):
        acc += wx
        if acc > v * S:
            return x
    return int(np.nonzero(w > 0)[0][-1])


def test_p_equals_q_accepts_everything():
    """q equal to p (computed independently with scipy, stored fp32) gives ratios
    within 2^-24 of 1, which every uniform <= 1 - 2^-24 passes; the bonus then
    comes from the last row with the column gamma+1 uniform [page §5.3]."""
    rng = np.random.default_rng(11)
    B, g, V, T = 16, 5, 257, float(np.float32(0.8))    # T is an fp32 input
    logits = rng.normal(0, 3, size=(B, g + 1, V)).astype(np.float32)
    p = scipy.special.softmax(logits.astype(np.float64) / T, axis=-1)
    q = p[:, :g].astype(np.float32)
    ids = np.stack([[rng.choice(V, p=p[b, i]) for i in range(g)] for b in range(B)])
    u = rng.integers(0, 1 << 24, size=(B, g + 2)) * U_STEP
    u[:, :g] = 1 - U_STEP                     # the hardest uniform for acceptance
    u[:, g] = 0.0
    o = oracle.verify(explicit_inputs(logits, q, ids, np.full(B, T), u))
    assert np.all(o.num_accepted == g)
    assert np.all(np.abs(o.ratio - 1) <= 2.0 ** -23)
    assert np.all(o.draw_kind == DRAW_BONUS)
    for b in range(B):
        assert list(o.tokens[b, :g]) == list(ids[b])
        assert o.tokens[b, g] == _bonus_by_hand(p[b, g], float(np.float32(u[b, g + 1])))


def test_disjoint_supports_reject_first():
    """p(x) = 0 where the draft puts its mass: ratio 0, so position 0 is rejected
    for every uniform, and the residual (p - q)_+ equals p [page §3.2]."""
    rng = np.random.default_rng(12)
    B, g, V = 32, 4, 64
    logits = rng.normal(0, 2, size=(B, g + 1, V)).astype(np.float32)
    logits[:, :, V // 2:] = -np.inf
    q = np.zeros((B, g, V), dtype=np.float32)
    q[:, :, V // 2:] = rng.dirichlet(np.ones(V // 2), size=(B, g))
    ids = V // 2 + rng.integers(0, V // 2, size=(B, g))
    u = rng.integers(0, 1 << 24, size=(B, g + 2)) * U_STEP
    u[:, 0] = 0.0                             # even the smallest uniform rejects
    o = oracle.verify(explicit_inputs(logits, q, ids, np.ones(B), u))
    assert np.all(o.num_accepted == 0)
    p0 = scipy.special.softmax(logits[:, 0].astype(np.float64), axis=-1)
    for b in range(B):
        assert o.tokens[b, 0] == _bonus_by_hand(p0[b], float(np.float32(u[b, g])))
        assert o.tokens[b, 0] < V // 2
        assert np.all(o.tokens[b, 1:] == -1)


def test_draw_columns():
    """Column gamma feeds the residual draw and column gamma+1 the bonus draw."""
    V, g = 4, 1
    logits = np.log(np.array([[[0.25, 0.25, 0.25, 0.25], [0.25, 0.25, 0.25, 0.25]]],
                             dtype=np.float32))
    q_all = np.full((1, 1, V), 0.25, dtype=np.float32)        # q = p: always accepted
    u = np.array([[0.0, 0.0, 0.99]], dtype=np.float32)
    o = oracle.verify(explicit_inputs(logits, q_all, [[1]], [1.0], u))
    assert o.num_accepted[0] == 1 and o.tokens[0, 1] == 3 and o.draw_value[0] == np.float32(0.99)
    q_rej = np.array([[[0.0, 1.0, 0.0, 0.0]]], dtype=np.float32)  # ratio 1/4 at token 1
    u = np.array([[0.5, 0.0, 0.99]], dtype=np.float32)
    o = oracle.verify(explicit_inputs(logits, q_rej, [[1]], [1.0], u))
    # residual (p - q)_+ = [1/4, 0, 1/4, 1/4]: uniform 0 (column gamma) -> token 0
    assert o.num_accepted[0] == 0 and o.tokens[0, 0] == 0 and o.draw_value[0] == 0.0


def test_gamma_zero_request_draws_bonus_from_row0():
    """A request with no drafts emits one bonus token from its only row."""
    V = 16
    offsets = np.array([0, 2, 2, 3])          # gamma_b = 2, 0, 1
    rng = np.random.default_rng(3)
    logits = rng.normal(0, 1, size=(6, V)).astype(np.float32)
    q = np.full((3, V), 1.0 / V, dtype=np.float32)
    ids = np.array([1, 2, 3])
    u = np.zeros((3, 4), dtype=np.float32)
    u[1, 3] = 0.7
    o = oracle.verify(explicit_inputs(logits, q, ids, [1.0, 1.0, 1.0], u, offsets=offsets))
    p = scipy.special.softmax(logits[3].astype(np.float64))
    assert o.num_accepted[1] == 0
    assert o.draw_kind[1] == DRAW_BONUS and o.draw_row[1] == 3
    assert o.tokens[1, 0] == _bonus_by_hand(p, float(np.float32(0.7)))
    assert np.all(o.tokens[1, 1:] == -1)


def test_one_hot_q_is_categorical_sampling():
    """A deterministic draft (q one-hot at x) emits exactly p: accept with
    probability p(x), else draw from p without x.  Dyadic p makes every
    boundary a multiple of 1/16, so a 16-point stratified grid is exact."""
    p = np.array([0.25, 0.5, 0.125, 0.125])
    V = 4
    N = 16
    grid = (np.arange(N) + 0.5) / N
    u0, v = np.meshgrid(grid, grid, indexing="ij")
    n = u0.size
    logits = np.broadcast_to(np.log(p), (n, 2, V)).astype(np.float32)
    q = np.zeros((n, 1, V), dtype=np.float32)
    q[:, 0, 1] = 1.0
    u = np.stack([u0.ravel(), v.ravel(), v.ravel()], axis=1)
    o = oracle.verify(explicit_inputs(logits, q, np.ones((n, 1), int), np.ones(n), u))
    law = np.bincount(o.tokens[:, 0], minlength=V) / n
    assert np.array_equal(law, p)


def test_degenerate_residual_falls_back_to_p():
    """q = 2p (not a distribution; the library takes q as given) makes the
    residual (p - q)_+ vanish; a rejection then draws from p."""
    V, g = 8, 1
    p = np.array([0.5, 0.25, 0.125, 0.0625, 0.03125, 0.015625, 0.0078125, 0.0078125])
    logits = np.broadcast_to(np.log(p), (1, g + 1, V)).astype(np.float32)
    q = (2 * p)[None, None, :].astype(np.float32)
    u = np.array([[0.75, 0.3, 0.0]], dtype=np.float32)     # ratio 1/2 -> rejected
    o = oracle.verify(explicit_inputs(logits, q, [[0]], [1.0], u))
    assert o.num_accepted[0] == 0 and o.draw_kind[0] == DRAW_DEGENERATE
    assert o.tokens[0, 0] == 0                               # 0.3 < p_0 = 0.5


# ---------------------------------------------------------------- greedy variant
def test_greedy_lowest_index_on_ties():
    V, g = 10, 2
    logits = np.zeros((1, g + 1, V), dtype=np.float32)
    logits[0, 0, [3, 7]] = 5.0
    logits[0, 1, [2, 4]] = 1.0
    logits[0, 2, [9, 0]] = 2.0
    q = np.zeros((1, g, V), dtype=np.float32)
    o = oracle.verify(explicit_inputs(logits, q, [[3, 2]], [0.0], np.zeros((1, g + 2))))
    assert o.num_accepted[0] == 2 and list(o.tokens[0]) == [3, 2, 0]
    assert o.draw_kind[0] == DRAW_NONE
    o = oracle.verify(explicit_inputs(logits, q, [[7, 2]], [0.0], np.zeros((1, g + 2))))
    assert o.num_accepted[0] == 0 and list(o.tokens[0]) == [3, -1, -1]


@pytest.mark.parametrize("T", [0.0, -1.0, float("nan")])
def test_nonpositive_or_nan_temperature_is_greedy(T):
    """[page §8, pitfall 2] temperature 0 is greedy; negative and NaN are read the same way."""
    V, g = 6, 1
    logits = np.array([[[0, 1, 2, 3, 2, 1], [5, 0, 0, 0, 0, 0]]], dtype=np.float32)
    q = np.full((1, g, V), np.nan, dtype=np.float32)       # never read by greedy requests
    o = oracle.verify(explicit_inputs(logits, q, [[3]], [T], np.full((1, g + 2), 0.5)))
    assert list(o.tokens[0]) == [3, 0] and o.num_accepted[0] == 1


def test_greedy_is_the_zero_temperature_limit():
    """With a clear argmax gap and T = 1e-3, p is one-hot to fp64 precision, so the
    sampled rule reproduces the greedy rule for every uniform in [2^-24, 1)."""
    rng = np.random.default_rng(21)
    B, g, V = 64, 4, 50
    logits = rng.normal(0, 1, size=(B, g + 1, V)).astype(np.float32)
    top = rng.integers(0, V, size=(B, g + 1))
    np.put_along_axis(logits, top[..., None], logits.max(-1, keepdims=True) + 0.5, axis=-1)
    q = rng.dirichlet(np.ones(V), size=(B, g)).astype(np.float32)
    ids = np.where(rng.random((B, g)) < 0.6, top[:, :g], rng.integers(0, V, size=(B, g)))
    u = (rng.integers(1, 1 << 24, size=(B, g + 2)) * U_STEP).astype(np.float32)
    gre = oracle.verify(explicit_inputs(logits, q, ids, np.zeros(B), u))
    smp = oracle.verify(explicit_inputs(logits, q, ids, np.full(B, 1e-3), u))
    assert np.array_equal(gre.num_accepted, smp.num_accepted)
    assert np.array_equal(gre.tokens, smp.tokens)


def test_rejects_out_of_range_ids():
    logits = np.zeros((1, 2, 4), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.verify(explicit_inputs(logits, np.zeros((1, 1, 4)), [[4]], [1.0], np.zeros((1, 3))))


def test_workload_half_with_q_equal_p_accepts_all():
    """The ragged top-k workload draws q = p (generator's own fp64 softmax, fp32
    stored) for half its requests; the oracle must accept every draft there."""
    from synth import make_config
    inp = make_config(5, vocab=4096, batch=48)
    o = oracle.verify(inp)
    gam = inp.gammas
    q = inp.draft_probs
    off = inp.draft_offsets
    for b in range(inp.batch):
        if gam[b] == 0:
            assert o.num_accepted[b] == 0 and o.draw_kind[b] == 2
            continue
        row = q[off[b]]
        equal_p = np.count_nonzero(row) > inp.vocab // 2      # dense rows are the q = p half
        if equal_p:
            assert o.num_accepted[b] == gam[b]
            assert np.all(np.abs(o.ratio[off[b]:off[b + 1]] - 1) <= 2.0 ** -23)
        assert np.all(o.tokens[b, o.num_accepted[b] + 1:] == -1)
