"""Host-side contract of the C ABI, exercised on a GPU: argument checks,
status codes, no-op batches, the sticky device-error word, profiling."""

import ctypes

import numpy as np
import pytest

from synth import make_config
from tests.gpu_helpers import log, run_gpu, upload_inputs

pytestmark = pytest.mark.gpu


def _lib():
    from lossless_rejection_sampling_sampler_amd import load_library
    return load_library()


def _args(db, **over):
    from lossless_rejection_sampling_sampler_amd import SVArgs
    p = lambda t: 0 if t is None else t.data_ptr()
    a = SVArgs(db.batch, db.gamma, db.total_draft, db.vocab, p(db.draft_offsets), p(db.target_logits),
               p(db.draft_probs), p(db.draft_ids), p(db.temperature), p(db.uniforms), p(db.out_tokens),
               p(db.out_num_accepted), 0, 0, 0, 0, 0, 0, 0)
    for k, v in over.items():
        setattr(a, k, v)
    return a


def test_create_argument_checks():
    from lossless_rejection_sampling_sampler_amd import SVConfig
    lib = _lib()
    h = ctypes.c_void_p()
    bad = [SVConfig(0, 4, 100, 1, 0), SVConfig(4, -1, 100, 1, 0), SVConfig(4, 129, 100, 1, 0),
           SVConfig(4, 4, 0, 1, 0)]
    for cfg in bad:
        assert lib.spec_verify_create(ctypes.byref(cfg), 0, ctypes.byref(h)) == 1
        assert not h.value
    assert lib.spec_verify_create(ctypes.byref(SVConfig(4, 4, 100, 7, 0)), 0, ctypes.byref(h)) == 4
    # row counts beyond 32-bit indices are refused; scratch beyond the device's memory fails cleanly
    assert lib.spec_verify_create(ctypes.byref(SVConfig(1 << 24, 128, 100, 1, 0)), 0, ctypes.byref(h)) == 4
    assert not h.value
    assert lib.spec_verify_create(ctypes.byref(SVConfig(1 << 22, 128, 100, 1, 0)), 0, ctypes.byref(h)) == 2
    assert not h.value
    assert lib.spec_verify_create(ctypes.byref(SVConfig(4, 4, 100, 1, 0)), 99, ctypes.byref(h)) == 3
    assert lib.spec_verify_destroy(None) == 0


def test_run_argument_checks():
    import torch
    inp = make_config(2, replicate=1, vocab=1000, batch=4)
    from tests.gpu_helpers import make_verifier
    sv = make_verifier(inp)
    db = upload_inputs(inp, diag=False)
    s = torch.cuda.current_stream().cuda_stream
    assert sv.run_args(_args(db), s) == 0
    assert sv.run_args(_args(db, batch=0), s) == 0                         # no-op
    assert sv.run_args(_args(db, batch=5, total_draft=25), s) == 5        # over max_batch
    assert sv.run_args(_args(db, gamma=6, total_draft=24), s) == 5        # over max_gamma
    assert sv.run_args(_args(db, vocab=999), s) == 1                      # vocab mismatch
    assert sv.run_args(_args(db, total_draft=19), s) == 1                 # inconsistent without offsets
    assert sv.run_args(_args(db, target_logits=None), s) == 1
    assert sv.run_args(_args(db, out_tokens=None), s) == 1
    assert sv.run_args(_args(db, target_logits=db.target_logits.data_ptr() + 2), s) == 1  # misaligned fp32
    assert sv.run_args(_args(db, batch=-1), s) == 1
    # sparse q: at most 64 entries per row, and the entry arrays when entries are used
    assert sv.run_args(_args(db, draft_probs=None, draft_topk=65), s) == 1
    assert sv.run_args(_args(db, draft_probs=None, draft_topk=-1), s) == 1
    assert sv.run_args(_args(db, draft_probs=None, draft_topk=4), s) == 1
    assert sv.run_args(_args(db, draft_probs=None, draft_topk=0), s) == 0      # point-mass drafts
    assert sv.run_args(_args(db, stats=db.out_tokens.data_ptr() + 2), s) == 1  # misaligned counters
    torch.cuda.synchronize()
    assert sv.device_errors() == 0


def test_zero_batch_leaves_outputs_untouched():
    import torch
    inp = make_config(2, replicate=1, vocab=1000, batch=4)
    from tests.gpu_helpers import make_verifier
    sv = make_verifier(inp)
    db = upload_inputs(inp, diag=False)
    assert sv.run_args(_args(db, batch=0), torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    assert torch.all(db.out_tokens == -7) and torch.all(db.out_num_accepted == -7)


SCHEDULES = ["onelaunch", "twokernel"]


@pytest.mark.parametrize("schedule", SCHEDULES)
def test_out_of_range_draft_id_sets_error_word(schedule):
    import torch
    from lossless_rejection_sampling_sampler_amd._lib import SV_DEVERR_DRAFT_ID
    inp = make_config(2, replicate=1, vocab=1000, batch=4)
    inp.draft_ids[0] = 1000
    inp.draft_ids[6] = -3
    log(f"[api] out-of-range draft ids, schedule={schedule}")
    res, _, sv = run_gpu(inp, diag=False, schedule=schedule)
    assert sv.device_errors(clear=True) & SV_DEVERR_DRAFT_ID
    assert sv.device_errors() == 0
    tok, num = res[0]
    assert num[0] == 0 and num[1] <= 0        # an invalid draft counts as rejected
    assert np.all((tok >= -1) & (tok < 1000))


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("batch,bad", [(8, 3), (300, 270)])   # 300: a thread counts two starts
def test_bad_offsets_set_error_word_without_faulting(schedule, batch, bad):
    from lossless_rejection_sampling_sampler_amd._lib import SV_DEVERR_OFFSETS
    inp = make_config(5, replicate=1, vocab=600, batch=batch)
    inp.offsets[bad] = inp.offsets[bad + 1] + 3    # gamma_bad negative
    log(f"[api] inconsistent offsets B={batch} at {bad}, schedule={schedule}")
    res, _, sv = run_gpu(inp, diag=False, schedule=schedule)
    assert sv.device_errors(clear=True) & SV_DEVERR_OFFSETS
    assert sv.device_errors() == 0
    # a following valid call on the same context is exact again
    good = make_config(5, replicate=1, vocab=600, batch=batch)
    res2, _, _ = run_gpu(good, sv=sv)
    res3, _, _ = run_gpu(good, schedule=schedule)
    assert np.array_equal(res2[0][0], res3[0][0]) and np.array_equal(res2[0][1], res3[0][1])


def test_profile_counters():
    import torch
    inp = make_config(2, replicate=1, vocab=4000, batch=4)
    from tests.gpu_helpers import make_verifier
    sv = make_verifier(inp, profile=True)
    db = upload_inputs(inp, diag=False)
    for _ in range(5):
        db.run(sv)
    torch.cuda.synchronize()
    rows_ms, draw_ms, n = sv.profile_read()
    assert n == 5 and rows_ms > 0 and draw_ms >= 0
    assert sv.profile_read()[2] == 0


@pytest.mark.parametrize("n,kw", [(3, dict(vocab=20000, batch=16)), (5, dict(vocab=4099, batch=24))],
                         ids=["flat", "split_ragged"])
def test_graph_capture_replays_match_eager(n, kw):
    """A two-kernel call captured in a HIP graph: every replay, with fresh
    uniforms and eager calls and synchronisations between replays, equals the
    eager call on the same inputs and the oracle (the arrival counters reset
    themselves, so replays need no host work)."""
    import torch
    import oracle
    from synth.workloads import uniforms_from_seed
    from tests.gpu_helpers import make_verifier
    inp = make_config(n, replicate=4, **kw)
    log(f"[graph] config {n} {kw}")
    sv = make_verifier(inp, schedule="twokernel")
    db = upload_inputs(inp, diag=False)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        db.run(sv)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        db.run(sv)
    torch.cuda.synchronize()
    for rep in range(4):
        u = uniforms_from_seed(inp.uniforms.shape, 1234 + rep)
        db.uniforms.copy_(torch.from_numpy(u))
        db.out_tokens.fill_(-7)
        db.out_num_accepted.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        tok_g, num_g = db.results()
        db.out_tokens.fill_(-7)
        db.out_num_accepted.fill_(-7)
        db.run(sv)
        torch.cuda.synchronize()
        tok_e, num_e = db.results()
        assert np.array_equal(tok_g, tok_e) and np.array_equal(num_g, num_e)
        orc = oracle.verify(inp, uniform_sets=[u])[0]
        assert np.array_equal(num_g, orc.num_accepted) and np.array_equal(tok_g, orc.tokens)
    assert sv.device_errors() == 0
