"""Distributional pins of the CPU oracle.

* [page §3.2] claims the accept / residual procedure emits tokens distributed
  exactly as the target p.  Checked exactly by brute force on dyadic inputs and
  by chi-square tests with 10^6 trials on random inputs, together with the
  exact joint law of (rejection position, emitted token) that the rejection
  sampling argument gives.  A planted mistake (drawing from p instead of the
  residual) must fail the same chi-square test.
* [page §3.3] E[tokens per round] = (1 - a^(gamma+1)) / (1 - a) when every
  draft is accepted with probability a.  Checked with inputs built so that
  sum_x min(p, q) = a exactly.
"""

from fractions import Fraction
from itertools import product

import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle
import oracle.rejection_sampler as ov
from tests.helpers import U_STEP, explicit_inputs


def _law_exact(p_rows, q_rows):
    """Exact law of (k, emitted tokens) from the rejection-sampling argument.

    P(k=j, x_0..x_{j-1}, y) = prod_{i<j} min(p_i, q_i)(x_i) * [(1-a_j) r_j(y)] for
    j < gamma, and prod_{i<gamma} min(p_i, q_i)(x_i) * p_gamma(y) for j = gamma,
    with a_i = sum_x min(p_i, q_i) and r_j = (p_j - q_j)_+ / sum (p_j - q_j)_+.
    """
    g = len(q_rows)
    V = len(p_rows[0])
    law = {}
    for j in range(g + 1):
        for xs in product(range(V), repeat=j):
            pref = Fraction(1)
            for i, x in enumerate(xs):
                pref *= min(p_rows[i][x], q_rows[i][x])
            if pref == 0:
                continue
            if j < g:
                a = sum(min(p_rows[j][x], q_rows[j][x]) for x in range(V))
                res = [max(p_rows[j][x] - q_rows[j][x], Fraction(0)) for x in range(V)]
                S = sum(res)
                for y in range(V):
                    if res[y]:
                        law[(j,) + xs + (y,)] = pref * (1 - a) * res[y] / S
            else:
                for y in range(V):
                    if p_rows[g][y]:
                        law[(j,) + xs + (y,)] = pref * p_rows[g][y]
    return law


def test_exhaustive_dyadic_joint_law():
    """Every draft sequence (weighted by q) x a 16-point stratified grid on each
    uniform.  All thresholds and residual boundaries are multiples of 1/16, so
    the grid law equals the exact law."""
    F = Fraction
    p_rows = [[F(3, 8), F(3, 8), F(1, 8), F(1, 8)],
              [F(1, 8), F(5, 16), F(1, 8), F(7, 16)],
              [F(1, 8), F(3, 8), F(1, 4), F(1, 4)]]
    q_rows = [[F(1, 8), F(1, 8), F(1, 2), F(1, 4)],
              [F(1, 4), F(1, 4), F(1, 4), F(1, 4)]]
    g, V, N = 2, 4, 16
    grid = (np.arange(N) + 0.5) / N
    combos = list(product(range(V), range(V), range(N), range(N), range(N)))
    n = len(combos)
    c = np.array(combos)
    logits = np.broadcast_to(np.log(np.array(p_rows, dtype=np.float64)), (n, g + 1, V))
    q = np.broadcast_to(np.array(q_rows, dtype=np.float64), (n, g, V))
    ids = c[:, :2]
    u = np.stack([grid[c[:, 2]], grid[c[:, 3]], grid[c[:, 4]], grid[c[:, 4]]], axis=1)
    w = np.array([float(q_rows[0][a] * q_rows[1][b]) for a, b in ids]) / N ** 3
    o = oracle.verify(explicit_inputs(logits.astype(np.float32), q.astype(np.float32),
                                      ids, np.ones(n), u))
    emp = {}
    for i in range(n):
        k = int(o.num_accepted[i])
        key = (k,) + tuple(int(t) for t in o.tokens[i, :k + 1])
        emp[key] = emp.get(key, 0.0) + w[i]
    exact = _law_exact(p_rows, q_rows)
    assert set(emp) == set(exact)
    for key, val in exact.items():
        assert abs(emp[key] - float(val)) < 1e-12, key
    # marginal at every emitted position is p (losslessness)
    for j in range(g + 1):
        reach = sum(v for kk, v in exact.items() if kk[0] >= j)
        for y in range(V):
            mass = sum(v for kk, v in exact.items() if kk[0] >= j and kk[1 + j] == y)
            assert mass == reach * p_rows[j][y]


def _random_case(seed, V=12, g=3, T=0.7):
    rng = np.random.default_rng(seed)
    logits = rng.normal(0, 1.5, size=(g + 1, V)).astype(np.float32)
    logits[0, 0] = -np.inf                   # a token the target never emits
    q = rng.dirichlet(np.full(V, 0.8), size=g).astype(np.float32)
    T32 = float(np.float32(T))
    p = scipy.special.softmax(logits.astype(np.float64) / T32, axis=-1)
    return logits, q, p, T32


def _run_trials(logits, q, T, n, seed):
    rng = np.random.default_rng(seed)
    g, V = q.shape
    qn = q.astype(np.float64) / q.astype(np.float64).sum(-1, keepdims=True)
    ids = np.stack([rng.choice(V, size=n, p=qn[i]) for i in range(g)], axis=1)
    u = (rng.integers(0, 1 << 24, size=(n, g + 2)) * U_STEP).astype(np.float32)
    L = np.broadcast_to(logits, (n,) + logits.shape)
    Q = np.broadcast_to(q, (n,) + q.shape)
    return oracle.verify(explicit_inputs(L, Q, ids, np.full(n, T), u))


def _chi2_pvalue(counts, probs):
    counts = np.asarray(counts, dtype=np.float64)
    exp = probs * counts.sum()
    keep = exp > 0
    assert counts[~keep].sum() == 0, "token emitted with zero probability"
    return scipy.stats.chisquare(counts[keep], exp[keep]).pvalue


N_TRIALS = 1_000_000
# Bonferroni over the 4 position tests + 1 joint test of each case, 2 cases
ALPHA = 1e-3 / 10


@pytest.mark.parametrize("seed", [1, 2])
def test_chi_square_emitted_tokens_follow_p(seed):
    logits, q, p, T = _random_case(seed)
    g, V = q.shape
    o = _run_trials(logits, q, T, N_TRIALS, seed + 100)
    k = o.num_accepted
    for j in range(g + 1):
        reached = k >= j
        counts = np.bincount(o.tokens[reached, j], minlength=V)
        assert _chi2_pvalue(counts, p[j]) > ALPHA, f"position {j}"
    # joint law of (k, tokens[k])
    q64 = q.astype(np.float64)
    qn = q64 / q64.sum(-1, keepdims=True)
    alpha = [float((qn[i] * np.minimum(1.0, p[i] / np.maximum(q64[i], 1e-10))).sum())
             for i in range(g)]
    probs = []
    for j in range(g + 1):
        pre = np.prod(alpha[:j])
        if j < g:
            res = np.maximum(p[j] - q64[j], 0)
            probs.append(pre * (1 - alpha[j]) * res / res.sum())
        else:
            probs.append(pre * p[g])
    probs = np.concatenate(probs)
    last = o.tokens[np.arange(len(k)), k]
    counts = np.bincount(k * V + last, minlength=(g + 1) * V)
    assert _chi2_pvalue(counts, probs) > ALPHA


def test_chi_square_power_planted_mistake(monkeypatch):
    """Drawing the rejected position from p instead of (p - q)_+ must be caught."""
    logits, q, p, T = _random_case(1)
    monkeypatch.setattr(ov, "residual_weights", lambda pk, qk: pk.copy())
    o = _run_trials(logits, q, T, N_TRIALS, 101)
    counts = np.bincount(o.tokens[:, 0], minlength=q.shape[1])
    assert _chi2_pvalue(counts, p[0]) < 1e-12


def _alpha_case(alpha, g, V=8, seed=0):
    """p on the first half (logits -inf on the second), q = a p + (1 - a) s with s on
    the second half: sum_x min(p, q) = a exactly, at every position."""
    rng = np.random.default_rng(seed)
    h = V // 2
    pa = rng.dirichlet(np.ones(h), size=g + 1)
    logits = np.full((g + 1, V), -np.inf)
    logits[:, :h] = np.log(pa)
    s = rng.dirichlet(np.ones(h), size=g)
    q = np.zeros((g, V))
    q[:, :h] = alpha * pa[:g]
    q[:, h:] = (1 - alpha) * s
    return logits.astype(np.float32), q.astype(np.float32)


@pytest.mark.parametrize("alpha", [0.2, 0.5, 0.8, 1.0])
@pytest.mark.parametrize("g", [1, 5, 8])
def test_mean_tokens_per_round_closed_form(alpha, g):
    """[page §3.3] E[emitted] = (1 - a^(g+1)) / (1 - a); z-test against the
    truncated-geometric variance (P(k >= j) = a^j)."""
    n = 200_000
    logits, q = _alpha_case(alpha, g, seed=g)
    o = _run_trials(logits, q, 1.0, n, seed=int(alpha * 100) + g)
    emitted = o.num_accepted.astype(np.float64) + 1
    if alpha == 1.0:
        assert np.all(emitted == g + 1)
        return
    expect = (1 - alpha ** (g + 1)) / (1 - alpha)
    ek = sum(alpha ** j for j in range(1, g + 1))
    ek2 = sum((2 * j - 1) * alpha ** j for j in range(1, g + 1))
    var = ek2 - ek ** 2
    z = (emitted.mean() - expect) / np.sqrt(var / n)
    assert abs(z) < 4.0, (emitted.mean(), expect, z)
