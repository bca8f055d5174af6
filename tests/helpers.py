"""Shared test helpers: explicit input construction and the parity rules."""

from __future__ import annotations

import numpy as np

from synth.workloads import VerifyInputs

U_STEP = 2.0 ** -24


def explicit_inputs(logits, q, ids, T, u, offsets=None, dtype="f32") -> VerifyInputs:
    """Pack per-request arrays into the library layout.

    logits: [B, g+1, V] (or already packed [R, V] when ``offsets`` is given),
    q: [B, g, V], ids: [B, g], T: [B], u: [B, g+2].
    """
    logits = np.asarray(logits)
    if offsets is None:
        B, g1, V = logits.shape
        g = g1 - 1
        lg = logits.reshape(B * g1, V)
        qq = np.asarray(q, dtype=np.float32).reshape(B * g, V)
        ii = np.asarray(ids, dtype=np.int32).reshape(B * g)
    else:
        B = len(offsets) - 1
        V = logits.shape[-1]
        g = int(np.max(np.diff(offsets))) if B else 0
        lg, qq, ii = logits, np.asarray(q, dtype=np.float32), np.asarray(ids, dtype=np.int32)
    if dtype == "f32":
        lg = lg.astype(np.float32)
    return VerifyInputs(batch=B, gamma=g if offsets is None else np.asarray(u).shape[1] - 2,
                        vocab=V, dtype=dtype, logits=np.ascontiguousarray(lg),
                        draft_probs=np.ascontiguousarray(qq), draft_ids=np.ascontiguousarray(ii),
                        temperature=np.asarray(T, dtype=np.float32),
                        uniforms=np.asarray(u, dtype=np.float32),
                        offsets=None if offsets is None else np.asarray(offsets, dtype=np.int32))


def uniform_grid_u(rng, shape):
    """Uniforms k * 2^-24, exact in fp32, in [0, 1 - 2^-24]."""
    return (rng.integers(0, 1 << 24, size=shape) * U_STEP).astype(np.float32)


def tile_request(logits, q, ids, T, n):
    """Repeat one request n times (same rows, fresh ids/uniforms supplied later)."""
    L = np.broadcast_to(logits, (n,) + logits.shape).copy()
    Q = np.broadcast_to(q, (n,) + q.shape).copy()
    I = np.broadcast_to(ids, (n,) + ids.shape).copy()
    return L, Q, I, np.full(n, T, dtype=np.float32)
