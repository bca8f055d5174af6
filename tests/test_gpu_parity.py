"""Parity of the HIP verifier with the CPU oracle (runs on an MI355X).

Every case prints its name, shape and seed before touching the GPU.
"""

import numpy as np
import pytest

from synth import CONFIGS, make_config, make_inputs
from synth.workloads import uniforms_from_seed
from tests.gpu_helpers import log, parity_check

pytestmark = pytest.mark.gpu

EXCUSED_BUDGET = 1e-4


def _assert_ok(rep, errs, min_requests=0):
    assert not rep.unexcused, "\n".join(rep.unexcused[:10])
    assert not errs, errs
    assert rep.requests >= min_requests
    assert rep.excused <= EXCUSED_BUDGET * rep.requests + 1e-9 or rep.excused == 0, \
        f"excused {rep.excused} of {rep.requests}"


# ---------------------------------------------------------------- small cases
SMALL = [
    ("c1", dict(n=1)),
    ("c2", dict(n=2)),
    ("c3_small", dict(n=3, vocab=9001, batch=12)),                  # bf16, ragged tail block
    ("c4_small", dict(n=4, vocab=5000, batch=40)),                  # T mix incl. greedy
    ("c5_small", dict(n=5, vocab=4099, batch=64)),                  # ragged, gamma_b = 0, q = p
    ("c3_oddV_bf16", dict(n=3, vocab=1001, batch=16)),              # rows not 16-byte aligned
    ("c2_oddV_f32", dict(n=2, vocab=777, batch=8)),
    ("c2_offsets", dict(n=2, vocab=3000, batch=8, explicit_offsets=True)),
    ("c1_tinyV", dict(n=1, vocab=3, batch=33)),
    ("c1_tinyV_aligned", dict(n=1, vocab=8, batch=33)),             # one 32-byte row: one piece
    ("c3_aligned", dict(n=3, vocab=16384, batch=32)),
    ("c5_aligned", dict(n=5, vocab=4096, batch=64)),                # ragged, gamma_b = 0, q = p
    # more requests than a workgroup has threads: a thread counts several request
    # starts in the row-to-request lookup
    ("c5_wide", dict(n=5, vocab=520, batch=600)),
    ("c5_wide_oddV", dict(n=5, vocab=517, batch=300)),
]


def _aligned(inp) -> bool:
    esize = 2 if inp.dtype == "bf16" else 4
    return inp.vocab * esize % 16 == 0


SCHEDULES = ["twokernel"]


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("name,kw", SMALL, ids=[s[0] for s in SMALL])
def test_small_parity(name, kw, schedule):
    kw = dict(kw)
    n = kw.pop("n")
    inp = make_config(n, replicate=7, **kw)
    sets = [inp.uniforms] + [uniforms_from_seed(inp.uniforms.shape, s) for s in range(15)]
    rep, errs, sv = parity_check(inp, sets, label=name, schedule=schedule)
    _assert_ok(rep, errs)
    from lossless_rejection_sampling_sampler_amd._lib import SV_SCHEDULE_FLAT, SV_SCHEDULE_SPLIT
    want = SV_SCHEDULE_FLAT if _aligned(inp) else SV_SCHEDULE_SPLIT
    assert sv.last_schedule() == want


def test_temperature_edge_values():
    """NaN / negative / zero temperatures take the greedy path; tiny T still samples."""
    inp = make_config(2, replicate=3, vocab=2000, batch=8)
    inp.temperature[:] = np.array([0.0, -1.0, np.nan, 1e-3, 0.05, 1.0, 4.0, 0.0], dtype=np.float32)
    rep, errs, _ = parity_check(inp, label="T-edge")
    _assert_ok(rep, errs)


def test_greedy_requests_never_read_q():
    """q rows of greedy requests are NaN-poisoned: results must not change."""
    inp = make_config(4, replicate=5, vocab=3000, batch=32)
    greedy = ~(inp.temperature > 0)
    assert greedy.any() and (~greedy).any()
    off = inp.draft_offsets
    for b in np.nonzero(greedy)[0]:
        inp.draft_probs[off[b]:off[b + 1]] = np.nan
    rep, errs, _ = parity_check(inp, label="greedy-nan-q")
    _assert_ok(rep, errs)


def test_repeated_calls_are_identical():
    """The arrival counters reset themselves: back-to-back calls agree."""
    from tests.gpu_helpers import run_gpu
    inp = make_config(3, replicate=2, vocab=20000, batch=24)
    res, _, sv = run_gpu(inp, [inp.uniforms] * 4)
    for tok, num in res[1:]:
        assert np.array_equal(tok, res[0][0]) and np.array_equal(num, res[0][1])
    # a smaller batch through the same context, then the full one again
    small = make_config(3, replicate=3, vocab=20000, batch=5)
    rs, _, _ = run_gpu(small, sv=sv)
    res2, _, _ = run_gpu(inp, sv=sv)
    assert np.array_equal(res2[0][0], res[0][0])


# ---------------------------------------------------------------- full workloads
# >= 2e4 requests per configuration: fresh uniforms over the same logits.
FULL = [(1, 20000), (2, 2500), (3, 313), (4, 157), (5, 79)]


@pytest.mark.parametrize("n,nsets", FULL, ids=[f"config{n}" for n, _ in FULL])
def test_full_workload_parity(n, nsets):
    log(f"[full] config {n} ({CONFIGS[n].name}) seed={1000 * n} sets={nsets}")
    inp = make_config(n)
    sets = [inp.uniforms] + [uniforms_from_seed(inp.uniforms.shape, 100 + s) for s in range(nsets - 1)]
    rep, errs, _ = parity_check(inp, sets, label=f"config{n}")
    _assert_ok(rep, errs, min_requests=20000)


# distinct logits and q draws at full size (row statistics at V = 151936 over
# 8 x 384 rows of the headline shapes, not one draw under many uniform sets)
DISTINCT = [(3, 8, 8), (4, 2, 4)]


@pytest.mark.parametrize("n,ndraws,nsets", DISTINCT, ids=[f"config{n}" for n, _, _ in DISTINCT])
def test_full_workload_distinct_draws(n, ndraws, nsets):
    # (replicates 1 and 2 of configs 3 and 5 are the invariants file's)
    for r in range(3, 3 + ndraws):
        log(f"[distinct] config {n} seed={1000 * n + r} sets={nsets}")
        inp = make_config(n, replicate=r)
        sets = [inp.uniforms] + [uniforms_from_seed(inp.uniforms.shape, 700 + 10 * r + s) for s in range(nsets - 1)]
        rep, errs, _ = parity_check(inp, sets, label=f"config{n}-draw{r}")
        _assert_ok(rep, errs)


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("n", [3, 5], ids=["config3", "config5"])
def test_full_workload_each_schedule(n, schedule):
    """Every schedule on the full workloads (fewer uniform sets)."""
    log(f"[full-{schedule}] config {n} seed={1000 * n}")
    inp = make_config(n)
    sets = [inp.uniforms] + [uniforms_from_seed(inp.uniforms.shape, 500 + s) for s in range(19)]
    rep, errs, _ = parity_check(inp, sets, label=f"config{n}-{schedule}", schedule=schedule)
    _assert_ok(rep, errs)


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("dtype,V", [("f32", 50000), ("bf16", 60000), ("bf16", 1001)])
def test_greedy_ties_and_all_neg_inf_rows(dtype, V, schedule):
    """Greedy rows: a row of -inf logits gives index 0, and a maximum repeated far
    apart (other threads and pieces) gives its lowest index."""
    from synth.workloads import f32_to_bf16_bits
    from tests.helpers import explicit_inputs
    rng = np.random.default_rng(11)
    B, g = 4, 2
    l = rng.normal(0.0, 1.0, size=(B, g + 1, V)).astype(np.float32)
    l[0, 0, :] = -np.inf                          # request 0: draft 0 = argmax 0 is accepted
    l[1, :, [3, V // 2, V - 2]] = 9.0             # three-way tie on every row of request 1
    l[2, 1, :] = -np.inf
    l[3, 0, [V - 1, 0]] = 9.0
    ids = np.array([[0, 5], [3, V // 2], [int(l[2, 0].argmax()), 0], [0, 1]])
    u = np.zeros((B, g + 2), dtype=np.float32)
    inp = explicit_inputs(l, np.zeros((B, g, V)), ids, np.zeros(B), u)
    if dtype == "bf16":
        inp.logits = f32_to_bf16_bits(inp.logits)
        inp.dtype = "bf16"
    log(f"[greedy-ties] dtype={dtype} V={V} schedule={schedule}")
    rep, errs, _ = parity_check(inp, label="greedy-ties", schedule=schedule)
    _assert_ok(rep, errs)
    assert rep.mismatched == 0


# Few rows over a large vocabulary: rows are cut into more pieces than the draw
# kernel's resolve loads in one round (8), on the flat path (aligned rows) and
# on the split path (odd V, 19 pieces per row).
MANY_PIECES = [
    ("B1_g4_V151936_bf16", dict(n=3, batch=1, gamma=4)),          # ~20 pieces per row
    ("B2_g8_V65536_f32", dict(n=2, batch=2, gamma=8, vocab=65536)),  # ~16 pieces per row
    ("B3_g2_V300001_bf16_split", dict(n=3, batch=3, gamma=2, vocab=300001)),
    ("B2_T_mix_V151936", dict(n=4, batch=2, gamma=3)),            # greedy rows with many pieces
]


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("name,kw", MANY_PIECES, ids=[m[0] for m in MANY_PIECES])
def test_rows_with_many_pieces(name, kw, schedule):
    kw = dict(kw)
    n = kw.pop("n")
    inp = make_config(n, replicate=9, **kw)
    sets = [inp.uniforms] + [uniforms_from_seed(inp.uniforms.shape, 300 + s) for s in range(31)]
    rep, errs, _ = parity_check(inp, sets, label=name, schedule=schedule)
    _assert_ok(rep, errs)
