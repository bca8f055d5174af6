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


def _run_once(sv, inp):
    """One call; returns (tokens, num_accepted) after synchronising."""
    import torch
    db = upload_inputs(inp, diag=False)
    db.run(sv)
    torch.cuda.synchronize()
    return db.results()


def _expect_blocked_then_cleared(sv, inp, want_bits):
    """After a violating call has run, the next call is refused with
    SV_ERR_DEVICE_CONTRACT and enqueues nothing; clearing the word unblocks it."""
    import torch
    from lossless_rejection_sampling_sampler_amd import SpecVerifyError
    from lossless_rejection_sampling_sampler_amd._lib import SV_ERR_DEVICE_CONTRACT
    db = upload_inputs(inp, diag=False)
    with pytest.raises(SpecVerifyError) as ei:
        db.run(sv)
    assert ei.value.status == SV_ERR_DEVICE_CONTRACT
    torch.cuda.synchronize()
    assert torch.all(db.out_tokens == -7) and torch.all(db.out_num_accepted == -7)   # nothing ran
    bits = sv.device_errors(clear=True)
    assert bits & want_bits, bits
    assert sv.device_errors() == 0


def _valid_rest_matches_oracle(inp, tok, num, first_valid):
    import bench
    import oracle
    o = oracle.verify(bench.sub_batch(inp, first_valid, inp.batch))
    assert np.array_equal(tok[first_valid:], o.tokens) and np.array_equal(num[first_valid:], o.num_accepted)


@pytest.mark.parametrize("greedy", [False, True], ids=["sampled", "greedy"])
def test_out_of_range_draft_id_poisons_its_request(greedy):
    from lossless_rejection_sampling_sampler_amd._lib import SV_DEVERR_DRAFT_ID
    inp = make_config(2, replicate=1, vocab=1000, batch=6)
    if greedy:
        inp.temperature[:] = 0.0
    good_ids = inp.draft_ids.copy()
    inp.draft_ids[0] = 1000          # request 0, draft 0
    inp.draft_ids[6] = -3            # request 1, draft 1
    log(f"[api] out-of-range draft ids, greedy={greedy}")
    from tests.gpu_helpers import make_verifier
    sv = make_verifier(inp)
    tok, num = _run_once(sv, inp)
    assert np.all(tok[:2] == -1) and np.all(num[:2] == -1)
    _valid_rest_matches_oracle(inp, tok, num, 2)
    inp.draft_ids[:] = good_ids
    _expect_blocked_then_cleared(sv, inp, SV_DEVERR_DRAFT_ID)
    tok2, num2 = _run_once(sv, inp)          # unblocked and exact again
    import oracle
    o = oracle.verify(inp)
    assert np.array_equal(tok2, o.tokens) and np.array_equal(num2, o.num_accepted)


@pytest.mark.parametrize("batch,bad", [(8, 3), (300, 270)])   # 300: a thread counts two starts
def test_bad_offsets_poison_the_request_without_faulting(batch, bad):
    from lossless_rejection_sampling_sampler_amd._lib import SV_DEVERR_OFFSETS
    inp = make_config(5, replicate=1, vocab=600, batch=batch)
    inp.offsets[bad] = inp.offsets[bad + 1] + 3    # gamma_bad negative
    log(f"[api] inconsistent offsets B={batch} at {bad}")
    res, _, sv = run_gpu(inp, diag=False)
    tok, num = res[0]
    assert num[bad] == -1 and np.all(tok[bad] == -1)
    good = make_config(5, replicate=1, vocab=600, batch=batch)
    _expect_blocked_then_cleared(sv, good, SV_DEVERR_OFFSETS)
    # a following valid call on the same context is exact again
    res2, _, _ = run_gpu(good, sv=sv)
    res3, _, _ = run_gpu(good)
    assert np.array_equal(res2[0][0], res3[0][0]) and np.array_equal(res2[0][1], res3[0][1])


def test_nonfinite_sampled_row_poisons_its_request():
    from lossless_rejection_sampling_sampler_amd._lib import SV_DEVERR_NONFINITE
    inp = make_config(3, replicate=2, vocab=5000, batch=6)
    V = inp.vocab
    g1 = inp.gamma + 1
    neg_inf_bf16 = np.uint16(0xff80)
    inp.logits[1 * g1 + 2, :] = neg_inf_bf16        # request 1: a row with no finite logit
    inp.logits[3 * g1 + 0, 17] = np.uint16(0x7fc0)   # request 3: a NaN logit
    log("[api] non-finite sampled rows")
    from tests.gpu_helpers import make_verifier
    sv = make_verifier(inp)
    tok, num = _run_once(sv, inp)
    for b in (1, 3):
        assert num[b] == -1 and np.all(tok[b] == -1)
    import bench
    import oracle
    for b0, b1 in ((0, 1), (2, 3), (4, 6)):
        o = oracle.verify(bench.sub_batch(inp, b0, b1))
        assert np.array_equal(tok[b0:b1], o.tokens) and np.array_equal(num[b0:b1], o.num_accepted)
    bits = sv.device_errors(clear=True)
    assert bits & SV_DEVERR_NONFINITE


def test_sparse_entry_violations_poison_the_request():
    from lossless_rejection_sampling_sampler_amd._lib import SV_DEVERR_TOPK
    from synth import make_sparse_config
    inp = make_sparse_config(replicate=3, vocab=3000, batch=8)
    off = inp.draft_offsets
    gam = inp.gammas
    bs = [b for b in range(inp.batch) if gam[b] > 0][:2]
    assert len(bs) == 2
    d0 = off[bs[0]]
    inp.topk_ids[d0, 1] = inp.vocab + 5              # an entry id outside [-1, V)
    d1 = off[bs[1]]
    x = inp.draft_ids[d1]
    inp.topk_ids[d1, :2] = x                          # the drafted token listed twice
    log(f"[api] sparse entry violations in requests {bs}")
    from tests.gpu_helpers import make_verifier
    sv = make_verifier(inp)
    tok, num = _run_once(sv, inp)
    for b in bs:
        assert num[b] == -1 and np.all(tok[b] == -1)
    assert sv.device_errors(clear=True) & SV_DEVERR_TOPK


def test_device_errors_waits_for_this_context_only():
    """spec_verify_device_errors returns while another stream is still busy: it
    waits for the context's last call and its own stream, not the device."""
    import time
    import torch
    inp = make_config(2, replicate=1, vocab=1000, batch=4)
    from tests.gpu_helpers import make_verifier
    sv = make_verifier(inp)
    _run_once(sv, inp)
    other = torch.cuda.Stream()
    a = torch.randn(8192, 8192, device="cuda:0")
    torch.cuda.synchronize()
    with torch.cuda.stream(other):
        for _ in range(30):
            a = a @ a
            a = a / a.norm()
        busy_end = torch.cuda.Event()
        busy_end.record(other)
    t0 = time.perf_counter()
    assert sv.device_errors() == 0
    dt = time.perf_counter() - t0
    still_busy = not busy_end.query()
    torch.cuda.synchronize()
    log(f"[api] device_errors took {dt * 1e3:.2f} ms; other stream still busy: {still_busy}")
    assert still_busy, "the other stream finished before device_errors returned"


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
