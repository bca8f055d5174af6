"""The library's largest shapes through the HIP path, element by element against
the CPU oracle (runs on an MI355X).

The boundary takes vocabularies up to 524,288 (256 draw blocks of 2048 tokens
per row: every slot of the select's block scan) and drafts up to 128 tokens
per request (129 target rows: one more than the resolve's threads of a wave,
so its row owners span three waves).  Each case prints its name and shape
before touching the GPU.
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
