"""Seeded randomized parity sweep of the HIP verifier against the CPU oracle
(runs on an MI355X): mixed batch sizes, draft widths, vocabularies (16-byte
aligned and not), logits dtypes, temperature mixes with greedy requests,
ragged offsets, and dense / sparse / point-mass draft distributions, on both
schedules.  Every case prints its parameters before touching the GPU."""

import numpy as np
import pytest

from synth.workloads import CONFIGS, make_inputs, to_point, to_sparse, uniforms_from_seed
from tests.gpu_helpers import log, parity_check

pytestmark = pytest.mark.gpu

N_CASES = 64


N_WIDE = 16       # batches of 200-600 requests: more than a workgroup's threads


def _case(k, wide=False):
    rng = np.random.default_rng((19000 if wide else 9000) + k)
    V = int(rng.choice([515, 777, 1000, 4096, 6001]) if wide else rng.choice([777, 1000, 4096, 6001, 16384, 20000]))
    spec = CONFIGS[4].with_(
        batch=int(rng.integers(200, 601) if wide else rng.integers(1, 41)),
        gamma=int(rng.integers(0, 9)),
        vocab=V,
        dtype=str(rng.choice(["f32", "bf16"])),
        target_sigma=float(rng.uniform(1.0, 4.0)),
        n_peaks=int(rng.integers(0, 6)),
        temperatures=tuple(float(t) for t in rng.choice([0.0, 0.3, 0.7, 1.0, 1.5], size=int(rng.integers(1, 4)))),
        ragged=bool(rng.integers(0, 2)),
        q_mode=str(rng.choice(["dense", "topk", "argmax"])),
        top_k=int(rng.integers(1, 65)),
        name=f"random{'_wide' if wide else ''}{k}",
    )
    inp = make_inputs(spec, seed=(19100 if wide else 9100) + k)
    fmt = "dense"
    if spec.q_mode == "topk" and inp.total_draft and rng.integers(0, 2):
        K = int(max(1, (inp.draft_probs != 0).sum(axis=1).max()))
        inp = to_sparse(inp, K, seed=k)
        fmt = f"sparse{K}"
    elif spec.q_mode == "argmax" and rng.integers(0, 2):
        inp = to_point(inp)
        fmt = "point"
    return spec, inp, fmt


@pytest.mark.parametrize("schedule", ["twokernel"])
@pytest.mark.parametrize("k", range(N_CASES))
def test_random_case(k, schedule):
    spec, inp, fmt = _case(k)
    log(f"[random {k}] B={inp.batch} gamma={inp.gamma} V={inp.vocab} {inp.dtype} T={spec.temperatures} "
        f"ragged={spec.ragged} q={spec.q_mode}/{fmt} schedule={schedule}")
    sets = [inp.uniforms] + [uniforms_from_seed(inp.uniforms.shape, 9500 + k * 10 + s) for s in range(5)]
    rep, errs, sv = parity_check(inp, sets, label=f"random{k}", schedule=schedule)
    assert not rep.unexcused, "\n".join(rep.unexcused[:10])
    assert not errs, errs
    assert rep.excused <= 1e-4 * rep.requests + 1e-9 or rep.excused == 0
    assert sv.device_errors() == 0


@pytest.mark.parametrize("schedule", ["twokernel"])
@pytest.mark.parametrize("k", range(N_WIDE))
def test_random_wide_case(k, schedule):
    spec, inp, fmt = _case(k, wide=True)
    log(f"[random wide {k}] B={inp.batch} gamma={inp.gamma} V={inp.vocab} {inp.dtype} T={spec.temperatures} "
        f"ragged={spec.ragged} q={spec.q_mode}/{fmt} schedule={schedule}")
    sets = [inp.uniforms] + [uniforms_from_seed(inp.uniforms.shape, 29500 + k * 10 + s) for s in range(3)]
    rep, errs, sv = parity_check(inp, sets, label=f"random_wide{k}", schedule=schedule)
    assert not rep.unexcused, "\n".join(rep.unexcused[:10])
    assert not errs, errs
    assert rep.excused <= 1e-4 * rep.requests + 1e-9 or rep.excused == 0
    assert sv.device_errors() == 0
