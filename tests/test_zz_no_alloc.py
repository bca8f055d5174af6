"""spec_verify_run_static (the entry point that allocates nothing, its scratch a
file-scope device array) against spec_verify_run on the same inputs, through
the C ABI (runs on an MI355X): two calls in a row, the second smaller, each
bit-exact with the context-based call and with the oracle."""

import numpy as np
import pytest

import oracle
from synth import make_config
from tests.gpu_helpers import log, make_verifier, upload_inputs

pytestmark = pytest.mark.gpu


def _static_run(inp):
    import torch
    from lossless_rejection_sampling_sampler_amd._lib import run_static
    db = upload_inputs(inp, diag=False)
    st = run_static(inp.dtype, db.args(), torch.cuda.current_stream().cuda_stream)
    assert st == 0, st
    torch.cuda.synchronize()
    return db.results()


def _context_run(inp):
    import torch
    sv = make_verifier(inp)
    db = upload_inputs(inp, diag=False)
    db.run(sv)
    torch.cuda.synchronize()
    out = db.results()
    sv.close()
    return out


@pytest.mark.parametrize("first,second", [
    ((3, dict(vocab=20000, batch=24)), (3, dict(vocab=20000, batch=5))),
    ((5, dict(vocab=4099, batch=200)), (2, dict(vocab=1000, batch=3))),
], ids=["bf16_then_fewer_requests", "ragged_then_fp32_small"])
def test_static_matches_context_twice(first, second):
    for n, kw in (first, second):
        inp = make_config(n, replicate=6, **kw)
        log(f"[static] config {n} B={inp.batch} gamma={inp.gamma} V={inp.vocab} {inp.dtype}")
        tok_s, num_s = _static_run(inp)
        tok_c, num_c = _context_run(inp)
        assert np.array_equal(tok_s, tok_c) and np.array_equal(num_s, num_c)
        o = oracle.verify(inp)
        assert np.array_equal(tok_s, o.tokens) and np.array_equal(num_s, o.num_accepted)


def test_static_rejects_sizes_beyond_its_limits():
    import torch
    from lossless_rejection_sampling_sampler_amd._lib import SV_ERR_CAPACITY, run_static
    inp = make_config(2, replicate=1, vocab=1000, batch=4)
    db = upload_inputs(inp, diag=False)
    s = torch.cuda.current_stream().cuda_stream
    a = db.args()
    a.batch = 257
    a.total_draft = 257 * a.gamma
    assert run_static(inp.dtype, a, s) == SV_ERR_CAPACITY
    a = db.args()
    a.gamma = 16
    a.batch = 250
    a.total_draft = 250 * 16            # 4250 target rows > 4096
    assert run_static(inp.dtype, a, s) == SV_ERR_CAPACITY
    torch.cuda.synchronize()
    assert torch.all(db.out_tokens == -7)
