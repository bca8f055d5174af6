"""The library's largest and smallest shapes through the HIP path, element by
element against the CPU oracle (runs on an MI355X).

The boundary takes vocabularies up to 524,288 (256 draw blocks of 2048 tokens
per row: every slot of the select's block scan) and drafts up to 128 tokens
per request (129 target rows: one more than the resolve's threads of a wave,
so its row owners span three waves).  At the other end, a vocabulary of one
token (every draw is token 0 and every draft is accepted) or two, and the
vocabularies around one draw block.  Each case prints its name and shape before
touching the GPU.
"""

import numpy as np
import pytest

import oracle
from synth import make_config
from synth.workloads import uniforms_from_seed
from tests.gpu_helpers import log, parity_check

pytestmark = pytest.mark.gpu

MAX_V = 524288
MAX_GAMMA = 128

LIMITS = [
    # (name, config, overrides, least max(num_accepted) the oracle must reach)
    ("maxV_bf16", 3, dict(vocab=MAX_V, batch=3, gamma=2), 0),                 # flat rows, 256 blocks
    ("maxV_f32", 2, dict(vocab=MAX_V, batch=2, gamma=3), 0),
    ("maxV_odd_bf16", 3, dict(vocab=MAX_V - 1, batch=2, gamma=2), 0),         # unaligned rows, ragged block
    ("maxgamma_f32", 2, dict(vocab=3000, batch=4, gamma=MAX_GAMMA, draft_sigma=0.05), 64),
    ("maxgamma_ragged_bf16", 5, dict(vocab=4099, batch=6, gamma=MAX_GAMMA), 100),   # q = p: bonus at depth
    ("maxgamma_tmix_bf16", 4, dict(vocab=2048, batch=8, gamma=MAX_GAMMA, draft_sigma=0.05), 64),
]


@pytest.mark.parametrize("name,n,kw,depth", LIMITS, ids=[c[0] for c in LIMITS])
def test_largest_shapes(name, n, kw, depth):
    inp = make_config(n, replicate=11, **kw)
    log(f"[limits] {name} B={inp.batch} gamma={inp.gamma} V={inp.vocab} {inp.dtype} rows={inp.total_rows}")
    if depth:
        # the case reaches the depth it is meant to exercise
        assert int(oracle.verify(inp).num_accepted.max()) >= depth
    sets = [inp.uniforms] + [uniforms_from_seed(inp.uniforms.shape, 300 + s) for s in range(11)]
    rep, errs, _ = parity_check(inp, sets, label=name)
    assert not rep.unexcused, "\n".join(rep.unexcused[:10])
    assert not errs, errs
    assert rep.excused <= 1e-4 * rep.requests + 1e-9 or rep.excused == 0


SMALLEST = [
    ("V1_f32", 1, dict(vocab=1, batch=5)),                                    # 4-byte rows: unaligned path
    ("V2_f32", 1, dict(vocab=2, batch=7)),
    ("V1_bf16", 3, dict(vocab=1, batch=4, n_peaks=0)),
    ("V1_bf16_tmix", 4, dict(vocab=1, batch=9, n_peaks=0)),                  # greedy rows of one token
    ("V2_bf16_tmix", 4, dict(vocab=2, batch=9, n_peaks=0)),
    ("V2_bf16_ragged", 5, dict(vocab=2, batch=9, n_peaks=0, top_k=2)),
    ("V8_bf16", 3, dict(vocab=8, batch=4)),                                   # one 16-byte vector per row
    ("V2049_f32", 2, dict(vocab=2049, batch=6)),                              # a second block of one token
    ("V2047_bf16", 3, dict(vocab=2047, batch=6)),                             # one block, unaligned rows
]


@pytest.mark.parametrize("name,n,kw", SMALLEST, ids=[c[0] for c in SMALLEST])
def test_smallest_shapes(name, n, kw):
    inp = make_config(n, replicate=5, **kw)
    log(f"[limits] {name} B={inp.batch} gamma={inp.gamma} V={inp.vocab} {inp.dtype} rows={inp.total_rows}")
    sets = [inp.uniforms] + [uniforms_from_seed(inp.uniforms.shape, 400 + s) for s in range(15)]
    rep, errs, _ = parity_check(inp, sets, label=name)
    assert not rep.unexcused, "\n".join(rep.unexcused[:10])
    assert not errs, errs
    assert rep.excused <= 1e-4 * rep.requests + 1e-9 or rep.excused == 0
