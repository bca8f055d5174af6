"""Plain fp64 CPU oracle of the lossless rejection-sampling verifier.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg, never by the library.  It shares no code with the
HIP path.

Source of the method: the spec-decoding page at dpshk.com/news/5598276
(scraped title "企业官网建设流程全解析"), cited below as [page §n]:

* [page §3.1] problem statement: the target model gives gamma+1 distributions
  p; draft token x_i is accepted with probability min(1, p(x_i)/q(x_i));
  verification stops at the first rejection; the rejected position is redrawn
  from (p - q)_+ normalised.
* [page §3.2] the residual r(x) = (p(x) - q(x))_+ / sum (p - q)_+ and the claim
  that the combined procedure emits tokens distributed exactly as p.
* [page §4] the worked example figure (ratios 0.92, 0.75, 0.31; three tokens).
* [page §5.2] the vectorised sampler: softmax of the target logits, q clamped
  below at 1e-10, a strict comparison of the uniform with the accept
  probability, a cumulative product as the prefix
  mask, and the residual clamp / normalise / categorical draw.
* [page §5.3] the bonus token: when all gamma drafts are accepted, one more
  token is drawn from the (gamma+1)-th target distribution.
* [page §8, pitfall 2] temperature 0 is greedy decoding.
* [page §7] prompt lookup decoding: drafts taken from the prompt, with no
  draft model.  Such a draft proposes its token with certainty, i.e. q is the
  point mass at the drafted token.
* [page §6.2] the serving log reports the draft acceptance rate and the
  accepted tokens per step (acceptance_stats counts what these are made of).

Readings where the page is silent:
temperature enters as softmax(l / T) with the max over the raw logits; T <= 0
or NaN selects the greedy variant (argmax of the raw logits, lowest index on
ties); uniforms arrive as an input of shape [B, gamma+2] whose columns
0..gamma_b-1 drive the accept tests, column gamma the residual draw and column
gamma+1 the bonus draw; a uniform v maps to the token min{x : C_x > v * S},
with C the running sum of the weights in ascending token id and S their total;
a residual with S <= 0 (impossible in exact arithmetic) falls back to p.
A sparse q, given as (id, prob) entries per draft row, is the q that holds
those probabilities at those ids and zero everywhere else.

All floating point is fp64 from the exact fp32 / bf16 input values.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence, Tuple

import numpy as np

# [page §5.2]: q is clamped below before dividing (the code clamps at 1e-10).
RESIDUAL_Q_FLOOR = 1e-10

DRAW_NONE = 0        # greedy request: no draw
DRAW_RESIDUAL = 1    # rejected at position k: draw from (p_k - q_k)_+
DRAW_BONUS = 2       # all drafts accepted: draw from p_gamma
DRAW_DEGENERATE = 3  # residual mass <= 0 after rounding: draw from p_k instead


def decode_logits(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Stored logits to fp64 (exact): fp32 as is, bf16 bit patterns widened."""
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(raw, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown logits dtype {dtype!r}")


def target_distribution(l: np.ndarray, T) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """p = softmax(l / T) along the last axis [page §3.1, §5.2].

    Returns (m, e, Z, p): m = max of the raw logits, e = exp((l - m) / T),
    Z = sum of e, p = e / Z.  T must be > 0 and broadcast against l.
    """
    m = l.max(axis=-1)
    e = np.exp((l - m[..., None]) / T)
    Z = e.sum(axis=-1)
    p = e / Z[..., None]
    return m, e, Z, p


def greedy_tokens(l: np.ndarray) -> np.ndarray:
    """argmax of the raw logits along the last axis, lowest index on ties."""
    return l.argmax(axis=-1)


def accept_ratio(p_x: np.ndarray, q_x: np.ndarray) -> np.ndarray:
    """p(x) / q(x) with q clamped below at 1e-10 [page §5.2]."""
    return p_x / np.maximum(q_x, RESIDUAL_Q_FLOOR)


def residual_weights(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Unnormalised residual (p - q)_+ [page §3.2, §5.2]."""
    return np.maximum(p - q, 0.0)


def inverse_cdf(w: np.ndarray, v) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Tokens drawn by uniforms ``v`` from unnormalised weights ``w`` [..., V].

    C_x = w_0 + ... + w_x in ascending token id, S = C_{V-1}; the token is
    min{x : C_x > v * S}.  Zero-weight tokens are never chosen and a uniform
    landing exactly on a boundary goes to the next token.  If rounding leaves
    no such x, the last token with positive weight is used.
    Returns (tokens, S, fallback_used), each with the leading shape of ``w``.
    """
    w = np.asarray(w, dtype=np.float64)
    C = np.cumsum(w, axis=-1)
    return _select(C, w, v)


def _select(C: np.ndarray, w: np.ndarray, v) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Inverse-CDF selection from running sums C (see inverse_cdf)."""
    lead = C.shape[:-1]
    V = C.shape[-1]
    C2 = C.reshape(-1, V)
    w2 = w.reshape(-1, V)
    S = C2[:, -1].copy()
    t = np.broadcast_to(np.asarray(v, dtype=np.float64), lead).reshape(-1) * S
    if V <= 4096:
        y = (C2 <= t[:, None]).sum(axis=-1)      # number of x with C_x <= t
    else:
        y = np.array([np.searchsorted(C2[i], t[i], side="right") for i in range(len(t))],
                     dtype=np.int64)
    fb = y >= V
    for i in np.nonzero(fb)[0]:
        pos = np.nonzero(w2[i] > 0)[0]
        y[i] = pos[-1] if len(pos) else V - 1
    return y.reshape(lead), S.reshape(lead), fb.reshape(lead)


def draft_q_rows(inp, drows: np.ndarray) -> np.ndarray:
    """q of draft rows ``drows`` as dense fp64 rows [len(drows), V].

    Dense q is read as stored.  A sparse q (``inp.q_format == "sparse"``) holds
    ``topk_probs[d, s]`` at token ``topk_ids[d, s]`` and zero at every token not
    listed (id -1 marks an unused entry; the ids of a row must be distinct).  A
    point-mass q (``"point"``, a draft proposed without a draft model,
    [page §7]) is 1 at the drafted token and 0 elsewhere.
    """
    drows = np.asarray(drows, dtype=np.int64).ravel()
    V = inp.vocab
    fmt = getattr(inp, "q_format", "dense")
    if fmt == "dense":
        return np.asarray(inp.draft_probs[drows], dtype=np.float64).reshape(len(drows), V)
    q = np.zeros((len(drows), V))
    if fmt == "point":
        q[np.arange(len(drows)), np.asarray(inp.draft_ids, dtype=np.int64)[drows]] = 1.0
        return q
    if fmt != "sparse":
        raise ValueError(f"unknown q format {fmt!r}")
    for j, d in enumerate(drows):
        ids = np.asarray(inp.topk_ids[d], dtype=np.int64)
        pr = np.asarray(inp.topk_probs[d], dtype=np.float32).astype(np.float64)
        used = ids != -1
        if np.any((ids[used] < 0) | (ids[used] >= V)):
            raise ValueError(f"sparse q row {d}: id outside [-1, V)")
        if len(np.unique(ids[used])) != int(used.sum()):
            raise ValueError(f"sparse q row {d}: repeated id")
        q[j, ids[used]] = pr[used]
    return q


def acceptance_stats(num_accepted: np.ndarray, gammas: np.ndarray, gamma: int) -> np.ndarray:
    """Counts behind the acceptance figures of [page §6.2] for one step.

    [0] requests, [1] drafts proposed (sum gamma_b), [2] drafts accepted (sum k_b),
    [3] requests with every draft accepted, [4 + k] requests with k_b == k
    (k = 0..gamma), [5 + gamma + i] requests whose draft i was tested
    (i < gamma_b and i <= k_b), [5 + 2 gamma + i] requests whose draft i was
    accepted (i < k_b).
    """
    k = np.asarray(num_accepted, dtype=np.int64)
    g = np.asarray(gammas, dtype=np.int64)
    out = np.zeros(5 + 3 * gamma, dtype=np.int64)
    out[0] = len(k)
    out[1] = g.sum()
    out[2] = k.sum()
    out[3] = int((k == g).sum())
    for kb, gb in zip(k, g):
        out[4 + kb] += 1
        for i in range(gb):
            if i <= kb:
                out[5 + gamma + i] += 1
            if i < kb:
                out[5 + 2 * gamma + i] += 1
    return out


def _first_rejection(accepted: np.ndarray, g: int) -> np.ndarray:
    """Index of the first False along the last axis, g if none (the prefix of
    accepted drafts, [page §5.2])."""
    if g == 0:
        return np.zeros(accepted.shape[0], dtype=np.int64)
    return np.where(accepted.all(axis=-1), g, accepted.argmin(axis=-1))


@dataclass
class OracleOutputs:
    tokens: np.ndarray          # [B, gamma+1] int32, -1 padded
    num_accepted: np.ndarray    # [B] int32
    row_max: np.ndarray         # [R] fp64: max raw logit of every target row
    row_norm: np.ndarray        # [R] fp64: Z of sampled rows, 0 for greedy rows
    ratio: np.ndarray           # [D] fp64: p(x)/max(q(x),1e-10) of sampled rows, NaN for greedy
    draw_kind: np.ndarray       # [B] DRAW_* code
    draw_row: np.ndarray        # [B] target row of the draw (-1 if none)
    draw_value: np.ndarray      # [B] uniform used by the draw (NaN if none)
    fallbacks: int = 0          # inverse-CDF rounding fallbacks taken


def _is_greedy(T: np.ndarray) -> np.ndarray:
    return ~(T > 0)      # 0, negative and NaN temperatures are greedy


def verify(inp, uniform_sets: Optional[Sequence[np.ndarray]] = None,
           max_chunk_elems: int = 1 << 24):
    """Run the verifier on ``inp`` (a synth.VerifyInputs-like object).

    With ``uniform_sets`` (a list of [B, gamma+2] arrays) the per-row target
    distributions are computed once and the accept / draw steps are repeated
    for each uniform set; a list of outputs is returned.  Otherwise the
    inputs' own uniforms are used and one OracleOutputs is returned.
    """
    single = uniform_sets is None
    if single:
        uniform_sets = [inp.uniforms]
    B, G, V = inp.batch, inp.gamma, inp.vocab
    off = np.asarray(inp.draft_offsets, dtype=np.int64)
    gam = np.diff(off)
    if len(off) != B + 1 or off[0] != 0 or np.any(gam < 0) or np.any(gam > G):
        raise ValueError("offsets must be nondecreasing prefix sums with 0 <= gamma_b <= gamma")
    D = int(off[-1])
    R = D + B
    ids_all = np.asarray(inp.draft_ids, dtype=np.int64)
    if D and (ids_all.min() < 0 or ids_all.max() >= V):
        raise ValueError("draft ids out of range")
    T_all = np.asarray(inp.temperature, dtype=np.float64)
    greedy = _is_greedy(T_all)
    us = [np.asarray(u, dtype=np.float64) for u in uniform_sets]
    for u in us:
        if u.shape != (B, G + 2):
            raise ValueError("uniforms must have shape [B, gamma+2]")

    outs = [OracleOutputs(tokens=np.full((B, G + 1), -1, dtype=np.int32),
                          num_accepted=np.zeros(B, dtype=np.int32),
                          row_max=np.zeros(R), row_norm=np.zeros(R),
                          ratio=np.full(D, np.nan),
                          draw_kind=np.zeros(B, dtype=np.int32),
                          draw_row=np.full(B, -1, dtype=np.int64),
                          draw_value=np.full(B, np.nan))
            for _ in us]

    for g in np.unique(gam):
        g = int(g)
        for want_greedy in (True, False):
            sel_all = np.nonzero((gam == g) & (greedy == want_greedy))[0]
            per_req = (g + 1) * V + g * V
            n_chunk = max(1, max_chunk_elems // max(per_req, 1))
            for c0 in range(0, len(sel_all), n_chunk):
                sel = sel_all[c0:c0 + n_chunk]
                trows = (off[sel] + sel)[:, None] + np.arange(g + 1)[None, :]
                drows = off[sel][:, None] + np.arange(g)[None, :]
                l = decode_logits(inp.logits[trows.ravel()], inp.dtype).reshape(len(sel), g + 1, V)
                x = ids_all[drows]                                   # [n, g]
                if want_greedy:
                    _greedy_chunk(outs, us, sel, trows, l, x, g)
                else:
                    q = draft_q_rows(inp, drows).reshape(len(sel), g, V)
                    _sampled_chunk(outs, us, sel, trows, drows, l, q, x, T_all[sel], g, G)
    return outs[0] if single else outs


def _greedy_chunk(outs, us, sel, trows, l, x, g):
    gidx = greedy_tokens(l)                                   # [n, g+1]
    m = l.max(axis=-1)
    match = x == gidx[:, :g]
    k = _first_rejection(match, g)
    n = len(sel)
    for o in outs:
        o.row_max[trows] = m
        o.num_accepted[sel] = k
        for j in range(g):
            keep = k > j
            o.tokens[sel[keep], j] = x[keep, j]
        o.tokens[sel, k] = gidx[np.arange(n), k]
        o.draw_kind[sel] = DRAW_NONE


def _sampled_chunk(outs, us, sel, trows, drows, l, q, x, T, g, G):
    n, _, V = l.shape
    m, e, Z, p = target_distribution(l, T[:, None, None])
    if g:
        p_x = np.take_along_axis(p[:, :g], x[..., None], axis=-1)[..., 0]
        q_x = np.take_along_axis(q, x[..., None], axis=-1)[..., 0]
        r = accept_ratio(p_x, q_x)                             # [n, g]
    else:
        r = np.zeros((n, 0))
    # Every possible draw of this chunk: residual at k < g, bonus at k = g.
    W = np.empty((n, g + 1, V))
    if g:
        W[:, :g] = residual_weights(p[:, :g], q)
    W[:, g] = e[:, g]
    kind = np.full((n, g + 1), DRAW_RESIDUAL, dtype=np.int32)
    kind[:, g] = DRAW_BONUS
    C = np.cumsum(W, axis=-1)
    if g:
        lost = ~(C[:, :g, -1] > 0)          # residual mass lost to rounding: fall back to p_k
        if lost.any():
            jj, kk = np.nonzero(lost)
            W[jj, kk] = p[jj, kk]
            C[jj, kk] = np.cumsum(W[jj, kk], axis=-1)
            kind[jj, kk] = DRAW_DEGENERATE
    rows = np.arange(n)
    for o, u in zip(outs, us):
        o.row_max[trows] = m
        o.row_norm[trows] = Z
        if g:
            o.ratio[drows] = r
        us_ = u[sel]
        accepted = us_[:, :g] < np.minimum(1.0, r)             # [page §5.2] strict "<"
        k = _first_rejection(accepted, g)
        o.num_accepted[sel] = k
        for j in range(g):
            keep = k > j
            o.tokens[sel[keep], j] = x[keep, j]
        v = np.where(k < g, us_[:, G], us_[:, G + 1])
        y, _, fb = _select(C[rows, k], W[rows, k], v)
        o.tokens[sel, k] = y
        o.draw_kind[sel] = kind[rows, k]
        o.draw_row[sel] = trows[rows, k]
        o.draw_value[sel] = v
        o.fallbacks += int(fb.sum())


def draw_weights(inp, b: int, k: int) -> Tuple[np.ndarray, int]:
    """The oracle's draw weights for request ``b`` drawing at position ``k``.

    Used to locate a token's CDF interval when a parity mismatch is examined.
    """
    off = np.asarray(inp.draft_offsets, dtype=np.int64)
    g = int(off[b + 1] - off[b])
    t0 = int(off[b]) + b
    T = float(inp.temperature[b])
    l = decode_logits(inp.logits[t0 + k], inp.dtype)
    m, e, Z, p = target_distribution(l, T)
    if k >= g:
        return e, DRAW_BONUS
    qk = draft_q_rows(inp, [int(off[b]) + k])[0]
    w = residual_weights(p, qk)
    if not (w.sum() > 0):
        return p, DRAW_DEGENERATE
    return w, DRAW_RESIDUAL


def token_interval(w: np.ndarray, y: int) -> Tuple[float, float]:
    """[C_{y-1}/S, C_y/S): the uniforms that map to token y under weights w."""
    C = np.cumsum(w)
    S = C[-1]
    lo = C[y - 1] / S if y > 0 else 0.0
    return float(lo), float(C[y] / S)
