"""Sparse and point-mass draft distributions, and the acceptance counters, on
the HIP path (runs on an MI355X).

A sparse q arrives as (id, prob) entries per draft row; a point-mass q (drafts
proposed without a draft model, the spec-decoding page's section 7) needs no
q memory at all.  Parity is against the CPU oracle under the same rules as the
dense format.  Every case prints its name, shape and seed before touching the GPU.
"""

import numpy as np
import pytest

import oracle
from synth import make_config, make_point_config, make_sparse_config
from synth.workloads import uniforms_from_seed
from tests.gpu_helpers import log, parity_check, run_gpu, upload_inputs

pytestmark = pytest.mark.gpu

EXCUSED_BUDGET = 1e-4
SCHEDULES = ["twokernel"]


def _assert_ok(rep, errs, min_requests=0):
    assert not rep.unexcused, "\n".join(rep.unexcused[:10])
    assert not errs, errs
    assert rep.requests >= min_requests
    assert rep.excused <= EXCUSED_BUDGET * rep.requests + 1e-9 or rep.excused == 0, \
        f"excused {rep.excused} of {rep.requests}"


SMALL = [
    ("sparse", make_sparse_config, dict(vocab=9001, batch=40)),          # ragged tail block
    ("sparse_oddV", make_sparse_config, dict(vocab=4099, batch=24)),     # rows not 16-byte aligned
    ("sparse_aligned", make_sparse_config, dict(vocab=16384, batch=32)),
    ("sparse_wide", make_sparse_config, dict(vocab=1024, batch=520)),   # > 256 ragged requests
    ("point", make_point_config, dict(vocab=9001, batch=24)),
    ("point_oddV", make_point_config, dict(vocab=1001, batch=16)),
    ("point_aligned", make_point_config, dict(vocab=16384, batch=16)),
]


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("name,mk,kw", SMALL, ids=[s[0] for s in SMALL])
def test_small_qformat_parity(name, mk, kw, schedule):
    inp = mk(replicate=7, **kw)
    sets = [inp.uniforms] + [uniforms_from_seed(inp.uniforms.shape, 40 + s) for s in range(15)]
    rep, errs, _ = parity_check(inp, sets, label=f"{name} seed-rep=7", schedule=schedule)
    _assert_ok(rep, errs)


@pytest.mark.parametrize("name,mk,nsets", [("sparse", make_sparse_config, 79), ("point", make_point_config, 313)])
def test_full_qformat_parity(name, mk, nsets):
    inp = mk()
    log(f"[full-{name}] {inp.name} B={inp.batch} V={inp.vocab} sets={nsets}")
    sets = [inp.uniforms] + [uniforms_from_seed(inp.uniforms.shape, 700 + s) for s in range(nsets - 1)]
    rep, errs, _ = parity_check(inp, sets, label=f"{name}-full")
    _assert_ok(rep, errs, min_requests=20000)


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("name,mk,kw", [
    ("c4_Tmix", make_config, dict(n=4, vocab=5000, batch=40)),
    ("c5_ragged", make_config, dict(n=5, vocab=4099, batch=64)),
    ("sparse", make_sparse_config, dict(vocab=3000, batch=32)),
], ids=["c4_Tmix", "c5_ragged", "sparse"])
def test_acceptance_counters(name, mk, kw, schedule):
    """Counters accumulate over calls and equal the oracle's counts exactly."""
    import torch
    from tests.gpu_helpers import make_verifier
    kw = dict(kw)
    inp = mk(replicate=3, **kw)
    log(f"[stats] {name} schedule={schedule} B={inp.batch} V={inp.vocab}")
    sv = make_verifier(inp, schedule=schedule)
    db = upload_inputs(inp, diag=False, stats=True)
    sets = [inp.uniforms] + [uniforms_from_seed(inp.uniforms.shape, 60 + s) for s in range(3)]
    want = np.zeros(5 + 3 * inp.gamma, dtype=np.int64)
    for u in sets:
        db.uniforms.copy_(torch.from_numpy(u))
        db.run(sv)
        torch.cuda.synchronize()
        _, num = db.results()
        orc = oracle.verify(inp, uniform_sets=[u])[0]
        # the expected counts are the oracle's alone; these seeds have no decision
        # near a threshold, so the GPU's num_accepted must equal the oracle's
        assert np.array_equal(num, orc.num_accepted)
        want += oracle.acceptance_stats(orc.num_accepted, inp.gammas, inp.gamma)
    got = db.stats.cpu().numpy().astype(np.int64)
    assert np.array_equal(got, want), (got.tolist(), want.tolist())
    assert sv.device_errors() == 0


@pytest.mark.parametrize("schedule", SCHEDULES)
def test_bad_sparse_entries_set_error_word(schedule):
    from lossless_rejection_sampling_sampler_amd._lib import SV_DEVERR_TOPK
    inp = make_sparse_config(replicate=2, vocab=3000, batch=16)
    ids = inp.topk_ids
    off = inp.draft_offsets
    with_drafts = [b for b in range(inp.batch) if off[b + 1] > off[b]]
    assert len(with_drafts) >= 2
    b0, b1 = with_drafts[:2]
    # request b0: entry 0 of every draft row names a token outside the vocabulary;
    # request b1: its first drafted token is listed twice
    ids[off[b0]:off[b0 + 1], 0] = 3007
    ids[off[b1], :2] = inp.draft_ids[off[b1]]
    log(f"[api] bad sparse entries, schedule={schedule}")
    u = inp.uniforms.copy()
    u[:, :inp.gamma] = 0.999999              # reject early: residual draws read the entry lists
    inp.uniforms = u
    res, _, sv = run_gpu(inp, diag=False, schedule=schedule)
    assert sv.device_errors(clear=True) & SV_DEVERR_TOPK
    tok, num = res[0]
    # both requests break the contract: all -1; every other request is exact
    for b in (b0, b1):
        assert num[b] == -1 and np.all(tok[b] == -1)
    import bench
    keep = [b for b in range(inp.batch) if b not in (b0, b1)]
    for b in keep:
        o = oracle.verify(bench.sub_batch(inp, b, b + 1), uniform_sets=[inp.uniforms[b:b + 1]])[0]
        assert np.array_equal(tok[b], o.tokens[0]) and num[b] == o.num_accepted[0]


# ---------------------------------------------------------------- draft-side sampling
@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("kw", [dict(batch=16, vocab=9001, dtype="f32"), dict(batch=40, vocab=16384),
                                dict(batch=8, vocab=1001)], ids=["f32_ragged", "bf16_aligned", "bf16_oddV"])
def test_small_sample_parity(kw, schedule):
    from synth import make_sample_config
    inp = make_sample_config(replicate=5, **kw)
    sets = [inp.uniforms] + [uniforms_from_seed(inp.uniforms.shape, 80 + s) for s in range(15)]
    rep, errs, _ = parity_check(inp, sets, label=f"sample {kw}", schedule=schedule)
    _assert_ok(rep, errs)


def test_full_sample_parity():
    from synth import make_sample_config
    inp = make_sample_config()
    log(f"[full-sample] {inp.name} B={inp.batch} V={inp.vocab} sets=313")
    sets = [inp.uniforms] + [uniforms_from_seed(inp.uniforms.shape, 900 + s) for s in range(312)]
    rep, errs, _ = parity_check(inp, sets, label="sample-full")
    _assert_ok(rep, errs, min_requests=20000)
