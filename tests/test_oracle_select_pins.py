"""Pins of the oracle parts that decide the draws at large vocabularies and the
multi-set path, each with a planted mistake that the pin must catch.

* the inverse-CDF selection for V > 4096 (a different code branch than the
  small-V one), against hand-computed intervals;
* verify(..., uniform_sets=[...]) against one call per uniform set;
* draw_weights / token_interval (what the GPU parity rules use to excuse a
  draw), against hand-computed residual, bonus and degenerate intervals.

The method is the spec-decoding page at dpshk.com/news/5598276: section 5.2
(the categorical draw from the residual, read here as the inverse CDF in
ascending token id with half-open intervals) and section 3.2 (the residual
(p - q)_+).  A mistake is planted in a copy of the oracle with monkeypatch,
on the CPU only.
"""

import dataclasses

import numpy as np
import pytest

import oracle
import oracle.rejection_sampler as rs
from oracle.rejection_sampler import DRAW_BONUS, DRAW_DEGENERATE, DRAW_RESIDUAL
from synth import make_config
from synth.workloads import uniforms_from_seed
from tests.helpers import explicit_inputs

# ---------------------------------------------------------------- inverse CDF, V > 4096
# Weights summing to S = 8 on a 6000-token vocabulary (every value dyadic, so
# every running sum and every v * S below is exact in fp64):
#   w[7] = 1, w[4096] = 2, w[5000..5003] = 1/2 each, w[5999] = 3, 0 elsewhere.
# Running sums: C_7 = 1, C_4096 = 3, C_5000 = 3.5, C_5001 = 4, C_5002 = 4.5,
# C_5003 = 5, C_5999 = 8.  Token y owns the uniforms [C_{y-1}/S, C_y/S).
BIG_V = 6000
BIG_W = {7: 1.0, 4096: 2.0, 5000: 0.5, 5001: 0.5, 5002: 0.5, 5003: 0.5, 5999: 3.0}
# (t = v * S lower bound, token) in ascending order, written out by hand
BIG_STEPS = [(0.0, 7), (1.0, 4096), (3.0, 5000), (3.5, 5001), (4.0, 5002), (4.5, 5003), (5.0, 5999)]


def _big_weights():
    w = np.zeros(BIG_V)
    for x, wx in BIG_W.items():
        w[x] = wx
    return w


def _expected_big(v):
    t = v * 8.0
    tok = None
    for lo, y in BIG_STEPS:
        if t >= lo:
            tok = y
    return tok


def check_big_vocab_intervals():
    w = _big_weights()
    # every multiple of 1/64 (v * S = k / 8) hits each boundary exactly once
    for k in range(64):
        v = k / 64
        y, S, fb = oracle.inverse_cdf(w, v)
        assert S == 8.0 and not fb
        assert int(y) == _expected_big(v), (v, int(y), _expected_big(v))
    # a uniform exactly on a running sum goes to the next token with weight
    for lo, y in BIG_STEPS[1:]:
        assert int(oracle.inverse_cdf(w, lo / 8.0)[0]) == y
    # just below a boundary stays in the earlier token
    assert int(oracle.inverse_cdf(w, 1.0 / 8.0 - 2.0 ** -40)[0]) == 7
    assert int(oracle.inverse_cdf(w, 5.0 / 8.0 - 2.0 ** -40)[0]) == 5003
    # zero-weight runs (8..4095, 4097..4999, 5004..5998) are never returned
    for v in np.linspace(0.0, 1.0 - 2.0 ** -24, 997):
        assert int(oracle.inverse_cdf(w, v)[0]) in BIG_W


def test_select_big_vocab_hand_computed():
    assert BIG_V > 4096
    check_big_vocab_intervals()


def check_big_vocab_rounding_fallback():
    # S is the smallest subnormal: v * S rounds back to S for v close to 1, so no
    # running sum exceeds it and the last token of positive weight is returned
    w = np.zeros(BIG_V)
    w[4100] = 5e-324
    y, S, fb = oracle.inverse_cdf(w, 1.0 - 2.0 ** -24)
    assert S == 5e-324 and bool(fb) and int(y) == 4100
    y, S, fb = oracle.inverse_cdf(w, 0.25)
    assert not fb and int(y) == 4100


def test_select_big_vocab_rounding_fallback():
    check_big_vocab_rounding_fallback()


def check_branches_agree(seed=0):
    """The same integer weights on V = 3000 and padded with zeros to V = 9000: the
    two branches of the selection must return identical tokens, boundary hits
    included (S = 2^20, so v = C_x / S is exact)."""
    rng = np.random.default_rng(seed)
    V0 = 3000
    w0 = rng.integers(0, 700, size=V0).astype(np.float64)
    w0[rng.random(V0) < 0.3] = 0.0                 # runs of zero weight
    w0[-1] = 0.0
    w0[0] += (1 << 20) - w0.sum()                  # total exactly 2^20
    assert w0.sum() == 2.0 ** 20 and w0[0] > 0
    C = np.cumsum(w0)
    vs = list(C[rng.integers(0, V0 - 1, size=200)] / 2.0 ** 20)          # boundary hits
    vs += list(rng.integers(0, 1 << 24, size=200) * 2.0 ** -24)         # ordinary uniforms
    vs = [v for v in vs if v < 1.0]
    w1 = np.concatenate([w0, np.zeros(9000 - V0)])
    for v in vs:
        a = oracle.inverse_cdf(w0, v)
        b = oracle.inverse_cdf(w1, v)
        assert int(a[0]) == int(b[0]) and a[1] == b[1] and bool(a[2]) == bool(b[2]), v
        # and the token's weight is positive, with v inside its interval
        y = int(a[0])
        lo = (C[y - 1] if y else 0.0) / 2.0 ** 20
        assert w0[y] > 0 and lo <= v < C[y] / 2.0 ** 20


def test_small_and_big_vocab_branches_agree():
    check_branches_agree(0)
    check_branches_agree(1)


def _select_side_left(C, w, v):
    """The large-V branch with side='left' (a boundary hit stays in the earlier token)."""
    lead = C.shape[:-1]
    V = C.shape[-1]
    C2 = C.reshape(-1, V)
    w2 = w.reshape(-1, V)
    S = C2[:, -1].copy()
    t = np.broadcast_to(np.asarray(v, dtype=np.float64), lead).reshape(-1) * S
    y = np.array([np.searchsorted(C2[i], t[i], side="left") for i in range(len(t))], dtype=np.int64)
    fb = y >= V
    for i in np.nonzero(fb)[0]:
        pos = np.nonzero(w2[i] > 0)[0]
        y[i] = pos[-1] if len(pos) else V - 1
    return y.reshape(lead), S.reshape(lead), fb.reshape(lead)


def test_planted_side_left_is_caught(monkeypatch):
    monkeypatch.setattr(rs, "_select", _select_side_left)
    with pytest.raises(AssertionError):
        check_big_vocab_intervals()
    with pytest.raises(AssertionError):
        check_branches_agree(0)


def test_planted_missing_fallback_is_caught(monkeypatch):
    real = rs._select

    def no_fallback(C, w, v):
        y, S, fb = real(C, w, v)
        # the mistake: a rounding miss returns the last token of the vocabulary
        y = np.where(fb, C.shape[-1] - 1, y)
        return y, S, fb

    monkeypatch.setattr(rs, "_select", no_fallback)
    with pytest.raises(AssertionError):
        check_big_vocab_rounding_fallback()


# ---------------------------------------------------------------- several uniform sets
def _ragged_mixed():
    inp = make_config(4, replicate=11, vocab=700, batch=24, ragged=True)
    assert len(set(inp.gammas.tolist())) > 2
    T = inp.temperature.astype(np.float64)
    assert (T > 0).any() and (~(T > 0)).any()
    return inp


def check_uniform_sets_equal_single_calls(inp, sets):
    multi = oracle.verify(inp, uniform_sets=sets)
    assert len(multi) == len(sets)
    for u, o in zip(sets, multi):
        one = oracle.verify(dataclasses.replace(inp, uniforms=np.asarray(u, dtype=np.float32)))
        assert np.array_equal(o.tokens, one.tokens)
        assert np.array_equal(o.num_accepted, one.num_accepted)
        assert np.array_equal(o.draw_kind, one.draw_kind)
        assert np.array_equal(o.draw_row, one.draw_row)
        assert np.array_equal(o.row_norm, one.row_norm) and np.array_equal(o.row_max, one.row_max)
        assert np.array_equal(o.ratio, one.ratio, equal_nan=True)


def _three_sets(inp):
    return [uniforms_from_seed(inp.uniforms.shape, 40 + s) for s in range(3)]


def test_uniform_sets_equal_single_calls():
    inp = _ragged_mixed()
    sets = _three_sets(inp)
    # the sets differ enough to change some outputs
    outs = oracle.verify(inp, uniform_sets=sets)
    assert not np.array_equal(outs[0].tokens, outs[1].tokens)
    check_uniform_sets_equal_single_calls(inp, sets)


def test_planted_set_index_off_by_one_is_caught(monkeypatch):
    inp = _ragged_mixed()
    sets = _three_sets(inp)
    real = rs.verify

    def shifted(inp_, uniform_sets=None, **kw):
        if uniform_sets is None:
            return real(inp_, **kw)
        # the mistake: output j is computed with set j + 1 (the last wraps)
        rolled = list(uniform_sets[1:]) + list(uniform_sets[:1])
        return real(inp_, uniform_sets=rolled, **kw)

    monkeypatch.setattr(oracle, "verify", shifted)
    with pytest.raises(AssertionError):
        check_uniform_sets_equal_single_calls(inp, sets)


# ---------------------------------------------------------------- draw weights and intervals
# One request, gamma = 2, V = 4, T = 1.  Logits are 0 or -inf, so every e is 0 or 1
# exactly and every p below is exact:
#   row 0: logits [0, 0, 0, 0]       -> p0 = [1/4, 1/4, 1/4, 1/4]
#   row 1: logits [0, -inf, 0, -inf] -> p1 = [1/2, 0, 1/2, 0]
#   row 2: logits [-inf, 0, 0, 0]    -> e2 = [0, 1, 1, 1] (bonus weights)
#   q0 = [1/2, 1/8, 1/4, 1/8]  -> residual at 0 = [0, 1/8, 0, 1/8], S = 1/4
#   q1 = [1/4, 1/4, 1/4, 1/4]  -> residual at 1 = [1/4, 0, 1/4, 0], S = 1/2
# Hand-computed intervals [C_{y-1}/S, C_y/S):
HAND_INTERVALS = {
    (0, DRAW_RESIDUAL): {1: (0.0, 0.5), 3: (0.5, 1.0), 0: (0.0, 0.0), 2: (0.5, 0.5)},
    (1, DRAW_RESIDUAL): {0: (0.0, 0.5), 2: (0.5, 1.0), 1: (0.5, 0.5), 3: (1.0, 1.0)},
    (2, DRAW_BONUS): {0: (0.0, 0.0), 1: (0.0, 1 / 3), 2: (1 / 3, 2 / 3), 3: (2 / 3, 1.0)},
}


def _interval_request(q0=(0.5, 0.125, 0.25, 0.125)):
    ninf = -np.inf
    logits = np.array([[[0, 0, 0, 0], [0, ninf, 0, ninf], [ninf, 0, 0, 0]]], dtype=np.float32)
    q = np.array([[list(q0), [0.25, 0.25, 0.25, 0.25]]], dtype=np.float32)
    return explicit_inputs(logits, q, [[0, 1]], [1.0], np.zeros((1, 4)))


def check_draw_intervals():
    inp = _interval_request()
    for (k, kind), want in HAND_INTERVALS.items():
        w, got_kind = rs.draw_weights(inp, 0, k)
        assert got_kind == kind, (k, got_kind)
        for y, (lo, hi) in want.items():
            glo, ghi = rs.token_interval(w, y)
            assert glo == pytest.approx(lo, abs=1e-15) and ghi == pytest.approx(hi, abs=1e-15), (k, y, glo, ghi)


def test_draw_weights_and_intervals_hand_computed():
    check_draw_intervals()


def test_degenerate_draw_weights_are_p():
    # q0 = 2 p0 everywhere: the residual vanishes and the draw falls back to p0
    inp = _interval_request(q0=(0.5, 0.5, 0.5, 0.5))
    w, kind = rs.draw_weights(inp, 0, 0)
    assert kind == DRAW_DEGENERATE
    for y in range(4):
        assert rs.token_interval(w, y) == pytest.approx((y / 4, (y + 1) / 4), abs=1e-15)


def test_planted_bonus_row_is_caught(monkeypatch):
    real_decode = rs.decode_logits
    calls = {}

    def draw_weights_prev_row(inp, b, k):
        # the mistake: the bonus weights come from the row before the bonus row
        off = np.asarray(inp.draft_offsets, dtype=np.int64)
        g = int(off[b + 1] - off[b])
        if k >= g:
            t0 = int(off[b]) + b
            l = real_decode(inp.logits[t0 + k - 1], inp.dtype)
            m, e, Z, p = rs.target_distribution(l, float(inp.temperature[b]))
            return e, DRAW_BONUS
        return real_draw_weights(inp, b, k)

    real_draw_weights = rs.draw_weights
    monkeypatch.setattr(rs, "draw_weights", draw_weights_prev_row)
    with pytest.raises(AssertionError):
        check_draw_intervals()


def test_planted_residual_sign_is_caught(monkeypatch):
    # the mistake: the residual taken as (q - p)_+
    monkeypatch.setattr(rs, "residual_weights", lambda p, q: np.maximum(q - p, 0.0))
    with pytest.raises(AssertionError):
        check_draw_intervals()


def test_planted_interval_shift_is_caught(monkeypatch):
    # the mistake: intervals closed on the left at C_y instead of C_{y-1}
    def shifted(w, y):
        C = np.cumsum(w)
        return float(C[y] / C[-1]), float(C[min(y + 1, len(w) - 1)] / C[-1])

    monkeypatch.setattr(rs, "token_interval", shifted)
    with pytest.raises(AssertionError):
        check_draw_intervals()
