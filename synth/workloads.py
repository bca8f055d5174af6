"""Seeded synthetic verifier inputs shaped like the pages' workloads.

The spec-decoding page (dpshk.com/news/5598276) deploys a Qwen2.5-72B target
with a 0.5B draft, gamma = 5 and temperature 0.8 (section 6.1), and reports
batch-1 and 128-concurrent runs (section 6.3).  No weights or prompts are
available here, so every input is synthetic with those shapes:

* target logits  ~ N(0, sigma_t^2) plus a few +8 "peaks" per row, drawn in
  fp64 and rounded to fp32, or to bf16 (round-to-nearest-even from fp32);
* draft logits   = the rounded target logits + N(0, sigma_d^2) noise;
* draft probs q  = softmax(draft / T_b) in fp64, rounded to fp32 and stored
  without renormalising (optionally top-k sparsified, or equal to the target
  distribution itself);
* draft ids      ~ the stored fp32 q (numpy's categorical sampler);
  greedy (T_b = 0) requests take argmax(draft) and a one-hot q;
* uniforms       = k * 2^-24 with k uniform in [0, 2^24): exact fp32 values in
  [0, 1 - 2^-24].

Draw order is fixed: a structure stream first (gamma_b, T_b, sigma_b, q
kind), then one child stream per request, which draws target noise, peak
positions, draft noise, draft ids and uniforms in that order.  The module
holds no part of the verification arithmetic.
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional, Sequence, Tuple, Union

import numpy as np

UNIFORM_BITS = 24


@dataclass(frozen=True)
class WorkloadSpec:
    """Recipe for one synthetic workload."""

    name: str
    batch: int
    gamma: int                      # padded draft width (max gamma_b)
    vocab: int
    dtype: str                      # "f32" or "bf16" target logits
    target_sigma: float
    n_peaks: int
    peak_height: float
    draft_sigma: Union[float, Tuple[float, float]]   # fixed, or (lo, hi) per request
    temperatures: Tuple[float, ...]                  # per-request T uniform over these
    ragged: bool = False            # gamma_b ~ U{0..gamma}, packed with offsets
    q_mode: str = "dense"           # "dense" | "half_equal_half_topk" | "topk" | "argmax"
    top_k: int = 50
    explicit_offsets: bool = False  # pass offsets even when every gamma_b == gamma

    def with_(self, **kw) -> "WorkloadSpec":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    1: WorkloadSpec("B1_g4_V1000_f32", 1, 4, 1000, "f32", 2.0, 0, 0.0, 1.0, (1.0,)),
    2: WorkloadSpec("B8_g5_V32000_f32", 8, 5, 32000, "f32", 3.0, 5, 8.0, 1.5, (1.0,)),
    3: WorkloadSpec("B64_g5_V151936_bf16", 64, 5, 151936, "bf16", 3.0, 8, 8.0, 1.0, (0.8,)),
    4: WorkloadSpec("B128_g8_V151936_bf16_Tmix", 128, 8, 151936, "bf16", 3.0, 8, 8.0,
                    (0.5, 3.0), (0.0, 0.3, 0.7, 1.0)),
    5: WorkloadSpec("B256_ragged8_V128256_bf16_topk", 256, 8, 128256, "bf16", 3.0, 8, 8.0,
                    1.0, (1.0,), ragged=True, q_mode="half_equal_half_topk", top_k=50),
}


@dataclass
class VerifyInputs:
    """One batch of verifier inputs in the packed layout the library takes.

    Request b owns target rows off[b] + b ... off[b] + b + gamma_b and draft
    rows off[b] ... off[b] + gamma_b - 1, where off are the prefix sums of
    gamma_b (``offsets``; None means every gamma_b equals ``gamma``).
    """

    batch: int
    gamma: int
    vocab: int
    dtype: str
    logits: np.ndarray        # [R, V] float32, or uint16 bf16 bit patterns
    draft_probs: Optional[np.ndarray]   # [D, V] float32; None for sparse / point-mass q
    draft_ids: np.ndarray     # [D] int32
    temperature: np.ndarray   # [B] float32
    uniforms: np.ndarray      # [B, gamma + 2] float32
    offsets: Optional[np.ndarray] = None   # [B + 1] int32
    name: str = ""
    # how q is stored: "dense" (draft_probs), "sparse" (topk_ids / topk_probs
    # [D, K], id -1 = unused entry, q = 0 off the list) or "point" (q = 1 at the
    # drafted token, a draft proposed without a draft model)
    q_format: str = "dense"
    topk_ids: Optional[np.ndarray] = None
    topk_probs: Optional[np.ndarray] = None

    @property
    def gammas(self) -> np.ndarray:
        if self.offsets is None:
            return np.full(self.batch, self.gamma, dtype=np.int64)
        return np.diff(self.offsets.astype(np.int64))

    @property
    def draft_offsets(self) -> np.ndarray:
        if self.offsets is None:
            return (np.arange(self.batch + 1, dtype=np.int64) * self.gamma)
        return self.offsets.astype(np.int64)

    @property
    def total_draft(self) -> int:
        return int(self.draft_offsets[-1])

    @property
    def total_rows(self) -> int:
        return self.total_draft + self.batch

    def target_row(self, b: int, i: int) -> int:
        return int(self.draft_offsets[b]) + b + i

    def draft_row(self, b: int, i: int) -> int:
        return int(self.draft_offsets[b]) + i

    def nbytes(self) -> int:
        return sum(a.nbytes for a in (self.logits, self.draft_probs, self.draft_ids, self.temperature,
                                      self.uniforms, self.topk_ids, self.topk_probs) if a is not None)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); returns uint16 bits."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))
    return ((bits + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def _draft_distribution(x: np.ndarray) -> np.ndarray:
    """Normalised exponentials of draft scores along the last axis (fp64)."""
    z = x - x.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def _gen_request(spec: WorkloadSpec, rng: np.random.Generator, g: int, T: float,
                 sigma_d: float, q_kind: str):
    V = spec.vocab
    l64 = rng.normal(0.0, spec.target_sigma, size=(g + 1, V))
    if spec.n_peaks:
        for row in range(g + 1):
            pos = rng.choice(V, size=spec.n_peaks, replace=False)
            l64[row, pos] += spec.peak_height
    l32 = l64.astype(np.float32)
    if spec.dtype == "f32":
        stored = l32
        lt = l32.astype(np.float64)
    elif spec.dtype == "bf16":
        stored = f32_to_bf16_bits(l32)
        lt = bf16_bits_to_f32(stored).astype(np.float64)
    else:
        raise ValueError(f"unknown dtype {spec.dtype}")

    q32 = np.zeros((g, V), dtype=np.float32)
    ids = np.zeros(g, dtype=np.int32)
    if g > 0:
        if T > 0 and q_kind == "argmax":
            # a deterministic proposal: the draft's most likely token, q one-hot
            draft = lt[:g] + rng.normal(0.0, sigma_d, size=(g, V))
            ids[:] = draft.argmax(axis=-1)
            q32[np.arange(g), ids] = 1.0
        elif T > 0:
            if q_kind == "equal_p":
                q32[:] = _draft_distribution(lt[:g] / T)
            else:
                draft = lt[:g] + rng.normal(0.0, sigma_d, size=(g, V))
                q64 = _draft_distribution(draft / T)
                if q_kind == "topk":
                    k = spec.top_k
                    keep = np.argpartition(q64, V - k, axis=-1)[:, V - k:]
                    rows = np.arange(g)[:, None]
                    sparse = np.zeros_like(q64)
                    sparse[rows, keep] = q64[rows, keep]
                    q64 = sparse / sparse.sum(axis=-1, keepdims=True)
                q32[:] = q64
            for i in range(g):
                w = q32[i].astype(np.float64)
                ids[i] = rng.choice(V, p=w / w.sum())
        else:
            draft = lt[:g] + rng.normal(0.0, sigma_d, size=(g, V))
            ids[:] = draft.argmax(axis=-1)
            q32[np.arange(g), ids] = 1.0
    k = rng.integers(0, 1 << UNIFORM_BITS, size=spec.gamma + 2)
    u = (k.astype(np.float64) * 2.0 ** -UNIFORM_BITS).astype(np.float32)
    return stored, q32, ids, u


def make_inputs(spec: WorkloadSpec, seed: int) -> VerifyInputs:
    """Build one batch for ``spec`` from ``seed`` (deterministic)."""
    B, G = spec.batch, spec.gamma
    root = np.random.SeedSequence(seed)
    children = root.spawn(B + 1)
    srng = np.random.Generator(np.random.PCG64(children[0]))

    if spec.ragged:
        gam = srng.integers(0, G + 1, size=B)
    else:
        gam = np.full(B, G, dtype=np.int64)
    temps = np.asarray(spec.temperatures, dtype=np.float64)
    T = temps[srng.integers(0, len(temps), size=B)] if len(temps) > 1 else np.full(B, temps[0])
    if isinstance(spec.draft_sigma, tuple):
        lo, hi = spec.draft_sigma
        sig = srng.uniform(lo, hi, size=B)
    else:
        sig = np.full(B, float(spec.draft_sigma))
    kinds = np.array(["dense"] * B, dtype=object)
    if spec.q_mode in ("topk", "argmax"):
        kinds[:] = spec.q_mode
    elif spec.q_mode == "half_equal_half_topk":
        perm = srng.permutation(B)
        kinds[perm[: B // 2]] = "equal_p"
        kinds[perm[B // 2:]] = "topk"
    elif spec.q_mode != "dense":
        raise ValueError(spec.q_mode)

    offsets = np.zeros(B + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(gam)
    D = int(offsets[-1])
    R = D + B
    V = spec.vocab
    ldt = np.float32 if spec.dtype == "f32" else np.uint16
    logits = np.empty((R, V), dtype=ldt)
    q = np.empty((D, V), dtype=np.float32)
    ids = np.empty(D, dtype=np.int32)
    u = np.empty((B, G + 2), dtype=np.float32)
    for b in range(B):
        rng = np.random.Generator(np.random.PCG64(children[b + 1]))
        g = int(gam[b])
        stored, q32, idb, ub = _gen_request(spec, rng, g, float(T[b]), float(sig[b]), kinds[b])
        t0 = int(offsets[b]) + b
        logits[t0:t0 + g + 1] = stored
        q[offsets[b]:offsets[b] + g] = q32
        ids[offsets[b]:offsets[b] + g] = idb
        u[b] = ub
    use_offsets = spec.ragged or spec.explicit_offsets
    return VerifyInputs(
        batch=B, gamma=G, vocab=V, dtype=spec.dtype, logits=logits, draft_probs=q,
        draft_ids=ids, temperature=T.astype(np.float32), uniforms=u,
        offsets=offsets.astype(np.int32) if use_offsets else None, name=spec.name,
    )


def to_sparse(inp: VerifyInputs, k: int, seed: int = 0) -> VerifyInputs:
    """The same q stored as k (id, prob) entries per draft row: the row's nonzero
    entries in a seeded random slot order, unused slots id -1 / prob 0.  Every
    row must have at most k nonzeros."""
    D = inp.total_draft
    ids = np.full((D, k), -1, dtype=np.int32)
    probs = np.zeros((D, k), dtype=np.float32)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 13])))
    for d in range(D):
        nz = np.nonzero(inp.draft_probs[d])[0]
        if len(nz) > k:
            raise ValueError(f"draft row {d} has {len(nz)} nonzeros, more than {k}")
        slots = rng.permutation(k)[:len(nz)]
        ids[d, slots] = nz
        probs[d, slots] = inp.draft_probs[d, nz]
    return dataclasses.replace(inp, draft_probs=None, q_format="sparse", topk_ids=ids, topk_probs=probs,
                               name=inp.name + f"_sparse{k}")


def to_point(inp: VerifyInputs) -> VerifyInputs:
    """The same drafted tokens proposed without a draft model: q is the point mass
    at each drafted token (no q array is stored)."""
    return dataclasses.replace(inp, draft_probs=None, q_format="point", topk_ids=None, topk_probs=None,
                               name=inp.name + "_point")


# Workloads of the sparse-q formats (the page's section 7 prompt lookup, and the
# top-k draft of the ragged B=256 workload stored as (id, prob) lists).
SPARSE_TOPK = 50


def make_sparse_config(replicate: int = 0, **overrides) -> VerifyInputs:
    """B=256, ragged gamma_b, V=128256, bf16, T=1, every request's q top-50
    sparse-renormalised and stored as 50 (id, prob) entries per draft row."""
    spec = CONFIGS[5].with_(q_mode="topk", name="B256_ragged8_V128256_bf16_top50", **overrides)
    return to_sparse(make_inputs(spec, seed=5100 + replicate), SPARSE_TOPK, seed=5100 + replicate)


def make_point_config(replicate: int = 0, **overrides) -> VerifyInputs:
    """B=64, gamma=5, V=151936, bf16, T=0.8 with point-mass drafts: each drafted
    token is the argmax of the noisy draft logits, proposed with certainty."""
    spec = CONFIGS[3].with_(q_mode="argmax", name="B64_g5_V151936_bf16_argmax", **overrides)
    return to_point(make_inputs(spec, seed=3100 + replicate))


def make_sample_config(replicate: int = 0, batch: int = 64, vocab: int = 151936, dtype: str = "bf16",
                       temperature: float = 0.8) -> VerifyInputs:
    """Draft-side sampling x ~ softmax(l / T): one row of draft logits per request
    and no drafts to verify (gamma = 0), so the verify step's bonus draw is the
    categorical sample.  Logits ~ N(0, 3^2) with 8 peaks of +8 (the recipe of
    the B=64 workload); the sample's uniform is column 1 of [B, 2]."""
    spec = CONFIGS[3].with_(batch=batch, gamma=0, vocab=vocab, dtype=dtype, temperatures=(temperature,),
                            name=f"B{batch}_V{vocab}_{dtype}_sample")
    return make_inputs(spec, seed=3200 + replicate)


def make_config(n: int, replicate: int = 0, **overrides) -> VerifyInputs:
    """Inputs for workload configuration ``n`` (1..5); seed = 1000 * n + replicate."""
    spec = CONFIGS[n]
    if overrides:
        spec = spec.with_(**overrides)
    return make_inputs(spec, seed=1000 * n + replicate)


def with_uniforms(inp: VerifyInputs, seed: int) -> VerifyInputs:
    """Same inputs with a fresh set of uniforms (k * 2^-24) drawn from ``seed``."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7])))
    k = rng.integers(0, 1 << UNIFORM_BITS, size=inp.uniforms.shape)
    u = (k.astype(np.float64) * 2.0 ** -UNIFORM_BITS).astype(np.float32)
    return dataclasses.replace(inp, uniforms=u)


def uniforms_from_seed(shape: Sequence[int], seed: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 11])))
    k = rng.integers(0, 1 << UNIFORM_BITS, size=tuple(shape))
    return (k.astype(np.float64) * 2.0 ** -UNIFORM_BITS).astype(np.float32)
