"""Invariants the method fixes, run through the HIP path and compared element by
element with the CPU oracle (runs on an MI355X).

The method is the spec-decoding page at dpshk.com/news/5598276: section 3.2
(with disjoint supports p(x) = 0 at the drafted token, so position 0 is
rejected and the residual is p itself), section 4 (the worked example),
section 5.2 (q floored at 1e-10, strict comparison, the categorical draw) and
the normaliser's closed form for equal logits (Z = V).  Every case prints its
name and shape before touching the GPU.
"""

import json
import os

import numpy as np
import pytest
import scipy.special

import oracle
from synth import make_config
from synth.workloads import f32_to_bf16_bits, uniforms_from_seed
from tests.gpu_helpers import log, parity_check, run_gpu
from tests.helpers import U_STEP, explicit_inputs, uniform_grid_u

pytestmark = pytest.mark.gpu

FULL_V = 151936
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _as(inp, dtype):
    if dtype == "bf16":
        inp.logits = f32_to_bf16_bits(inp.logits)
        inp.dtype = "bf16"
    return inp


def _assert_exact(rep, errs):
    assert not rep.unexcused, "\n".join(rep.unexcused[:10])
    assert not errs, errs
    assert rep.mismatched == 0


# ---------------------------------------------------------------- disjoint supports
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_disjoint_supports_reject_first_full_vocab(dtype):
    """Sampled rows with the upper half of the vocabulary at -inf and q living on
    that half: every request is rejected at position 0 and draws from p_0."""
    rng = np.random.default_rng(31)
    B, g, V = 24, 5, FULL_V
    log(f"[disjoint] dtype={dtype} B={B} gamma={g} V={V}")
    l = rng.normal(0.0, 3.0, size=(B, g + 1, V)).astype(np.float32)
    l[:, :, V // 2:] = -np.inf
    q = np.zeros((B, g, V), dtype=np.float32)
    w = rng.gamma(1.0, size=(B, g, V // 2))
    q[:, :, V // 2:] = w / w.sum(-1, keepdims=True)
    ids = V // 2 + rng.integers(0, V // 2, size=(B, g))
    u = (rng.integers(0, 1 << 24, size=(B, g + 2)) * U_STEP).astype(np.float32)
    u[:B // 2, 0] = 0.0                       # even the smallest uniform rejects
    inp = _as(explicit_inputs(l, q, ids, np.full(B, 0.8), u), dtype)
    sets = [inp.uniforms] + [np.where(np.arange(g + 2) == 0, 0.0, uniforms_from_seed(u.shape, 70 + s)).astype(np.float32)
                             for s in range(3)]
    rep, errs, _ = parity_check(inp, sets, label=f"disjoint-{dtype}")
    _assert_exact(rep, errs)
    res, _, _ = run_gpu(inp, sets, diag=False)
    for (tok, num), uu in zip(res, sets):
        assert np.all(num == 0)
        assert np.all(tok[:, 0] < V // 2) and np.all(tok[:, 1:] == -1)


# ---------------------------------------------------------------- exact tie
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V", [8, 131072])
def test_exact_tie_rejects_on_gpu(V, dtype):
    """Equal logits (0) at T = 1 give p = 1/V exactly; q(x) = 4/V gives the ratio
    1/4 exactly.  A uniform of exactly 1/4 rejects (strict comparison), and
    1/4 - 2^-24 accepts."""
    g, B = 2, 8
    log(f"[tie] V={V} dtype={dtype}")
    l = np.zeros((B, g + 1, V), dtype=np.float32)
    q = np.full((B, g, V), (1.0 - 4.0 / V) / (V - 1), dtype=np.float32)
    ids = np.tile(np.array([[3, 5]]), (B, 1))
    q[:, 0, 3] = 4.0 / V
    q[:, 1, 5] = 4.0 / V
    u = np.zeros((B, g + 2), dtype=np.float32)
    u[0::2, 0] = 0.25                          # reject at 0
    u[1::2, 0] = 0.25 - U_STEP                 # accept at 0 ...
    u[1::2, 1] = 0.25                          # ... then reject at 1
    u[:, g] = np.linspace(0.0, 0.9, B, dtype=np.float32)
    inp = _as(explicit_inputs(l, q, ids, np.ones(B), u), dtype)
    rep, errs, _ = parity_check(inp, label=f"tie-V{V}-{dtype}")
    _assert_exact(rep, errs)
    (tok, num), = run_gpu(inp, diag=False)[0]
    assert np.array_equal(num, np.tile([0, 1], B // 2))
    o = oracle.verify(inp)
    assert np.all(o.ratio == 0.25)


# ---------------------------------------------------------------- worked example
def test_worked_example_on_gpu():
    """The page's section 4 figure: ratios 0.92, 0.75, 0.31 with dice 0.5, 0.5, 0.31
    (the third equal to its ratio) -> two drafts accepted, three tokens emitted."""
    ex = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    g, V = ex["gamma"], 8
    log(f"[worked example] gamma={g} V={V}")
    logits = np.zeros((1, g + 1, V), dtype=np.float32)
    ids = np.array([[1, 2, 3, 4, 5]], dtype=np.int32)
    q = np.zeros((1, g, V), dtype=np.float32)
    u = np.zeros((1, g + 2), dtype=np.float32)
    for i, (ratio, die) in enumerate(zip(ex["ratios"], ex["uniforms_accept"])):
        qx = np.float32(0.125 / ratio)
        u32 = np.float32(die)
        while 0.125 / float(qx) > float(u32) and die == ratio:
            qx = np.nextafter(qx, np.float32(1.0))
        q[0, i, :] = (1.0 - qx) / (V - 1)
        q[0, i, ids[0, i]] = qx
        u[0, i] = u32
    u[0, g], u[0, g + 1] = 0.4, 0.9
    inp = explicit_inputs(logits, q, ids, [1.0], u)
    rep, errs, _ = parity_check(inp, label="worked-example")
    _assert_exact(rep, errs)
    (tok, num), = run_gpu(inp, diag=False)[0]
    assert num[0] == ex["expected_num_accepted"]
    assert int((tok[0] >= 0).sum()) == ex["expected_emitted_tokens"]
    assert list(tok[0, :2]) == [1, 2] and tok[0, 2] != 3


# ---------------------------------------------------------------- normaliser
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_equal_logits_normaliser_is_V(dtype):
    """Logits all 0: every term is 2^0 = 1 in the rows pass too, so Z = V exactly;
    logits all 1.75 (T = 0.7): Z = V within the 1e-5 rule, and the oracle's Z is
    exactly V."""
    B, g, V = 4, 3, FULL_V
    for level, T in ((0.0, 1.0), (1.75, 0.7)):
        log(f"[Z=V] dtype={dtype} level={level} T={T} V={V}")
        l = np.full((B, g + 1, V), level, dtype=np.float32)
        rng = np.random.default_rng(5)
        w = rng.gamma(1.0, size=(B, g, V))
        q = (w / w.sum(-1, keepdims=True)).astype(np.float32)
        ids = rng.integers(0, V, size=(B, g))
        u = uniforms_from_seed((B, g + 2), 77)
        inp = _as(explicit_inputs(l, q, ids, np.full(B, T), u), dtype)
        o = oracle.verify(inp)
        assert np.all(o.row_norm == V)
        rep, errs, _ = parity_check(inp, label=f"Z=V-{dtype}-{level}")
        _assert_exact(rep, errs)
        _, dg, _ = run_gpu(inp)
        if level == 0.0:
            assert np.all(dg["row_norm"] == V)
        assert np.all(np.abs(dg["row_norm"] / V - 1) <= 1e-5)


# ---------------------------------------------------------------- q rows never read
@pytest.mark.parametrize("n", [3, 5], ids=["config3", "config5"])
def test_q_after_first_rejection_is_never_read(n):
    """NaN in every q element the outputs do not depend on: the q rows after the
    oracle's first rejection (their drafted-token values are gathered before the
    first rejection is known, and then ignored), and every element of the
    earlier draft rows except the drafted token's.  Tokens and num_accepted must
    not change."""
    inp = make_config(n, replicate=21, batch=32 if n == 3 else 64)
    log(f"[nan-q] config {n} B={inp.batch} V={inp.vocab}")
    clean = oracle.verify(inp)
    off = inp.draft_offsets
    gam = inp.gammas
    q = inp.draft_probs
    for b in range(inp.batch):
        k = int(clean.num_accepted[b])
        for i in range(gam[b]):
            d = off[b] + i
            if i < k:
                keep = q[d, inp.draft_ids[d]]
                q[d, :] = np.nan
                q[d, inp.draft_ids[d]] = keep
            elif i > k:
                q[d, :] = np.nan
    (tok, num), = run_gpu(inp, diag=False)[0]
    assert np.array_equal(num, clean.num_accepted)
    assert np.array_equal(tok, clean.tokens)


# ---------------------------------------------------------------- output canaries
def test_outputs_stay_inside_their_buffers():
    """Canary words before and after every output and diagnostic buffer (and the
    counters) survive a call; the buffers themselves match the oracle."""
    import torch
    from lossless_rejection_sampling_sampler_amd import SpecVerify, upload
    inp = make_config(5, replicate=4, vocab=4099, batch=48)
    log(f"[canary] B={inp.batch} V={inp.vocab}")
    db = upload(logits=inp.logits, logits_dtype=inp.dtype, draft_probs=inp.draft_probs, draft_ids=inp.draft_ids,
                temperature=inp.temperature, uniforms=inp.uniforms, gamma=inp.gamma, draft_offsets=inp.offsets,
                device="cuda:0", diag=True, stats=True)
    PAD = 64
    guarded = {}

    def guard(name, t, canary):
        flat = t.reshape(-1)
        big = torch.full((flat.numel() + 2 * PAD,), canary, dtype=flat.dtype, device=flat.device)
        big[PAD:PAD + flat.numel()] = flat
        guarded[name] = (big, canary, flat.numel())
        return big[PAD:PAD + flat.numel()].view(t.shape)

    db.out_tokens = guard("tokens", db.out_tokens, 0x5A5A5A5A)
    db.out_num_accepted = guard("num", db.out_num_accepted, 0x5A5A5A5A)
    db.diag_row_max = guard("row_max", db.diag_row_max, 12345.0)
    db.diag_row_norm = guard("row_norm", db.diag_row_norm, 12345.0)
    db.diag_ratio = guard("ratio", db.diag_ratio, 12345.0)
    db.stats = guard("stats", db.stats, 0x5A5A5A5A)
    sv = SpecVerify(inp.batch, inp.gamma, inp.vocab, inp.dtype, device=0)
    db.run(sv)
    torch.cuda.synchronize()
    for name, (big, canary, n) in guarded.items():
        h = big.cpu()
        assert torch.all(h[:PAD] == canary) and torch.all(h[PAD + n:] == canary), name
    o = oracle.verify(inp)
    tok, num = db.results()
    assert np.array_equal(tok, o.tokens) and np.array_equal(num, o.num_accepted)
    assert sv.device_errors() == 0


# ---------------------------------------------------------------- more logits draws at full size
@pytest.mark.parametrize("n,rep_id,nsets", [(3, 1, 60), (3, 2, 60), (5, 1, 16), (5, 2, 16)],
                         ids=["config3-r1", "config3-r2", "config5-r1", "config5-r2"])
def test_full_size_more_logits_replicates(n, rep_id, nsets):
    inp = make_config(n, replicate=rep_id)
    log(f"[full replicate] config {n} replicate={rep_id} seed={1000 * n + rep_id} sets={nsets}")
    sets = [inp.uniforms] + [uniforms_from_seed(inp.uniforms.shape, 900 + s) for s in range(nsets - 1)]
    rep, errs, _ = parity_check(inp, sets, label=f"config{n}-rep{rep_id}")
    assert not rep.unexcused, "\n".join(rep.unexcused[:10])
    assert not errs, errs
    assert rep.excused <= 1e-4 * rep.requests + 1e-9 or rep.excused == 0


# ---------------------------------------------------------------- marginal tokens
def _marginal_case(dtype, seed, only):
    """Residual rows whose blocks hold 0, 1, 2, 3 and 2048 tokens with q within
    4e-6 of p (the draw's fp32-normaliser sign test cannot place them: they are
    captured inline, or their block is summed again from its tokens) and a
    drafted token with a large q, so that position 0 is rejected.  The other
    tokens have q = p / 2 (the drafted token's q takes the rest of the mass), or,
    with `only`, q = 1.001 p and the marginal ones q < p, so that every token of
    positive residual weight is a marginal one (q is then not normalised: the
    arithmetic is the same)."""
    rng = np.random.default_rng(seed)
    B, g, V, blk = 24, 2, 5 * 2048, 2048
    logits = rng.normal(0.0, 1.5, size=(B, g + 1, V))
    # a +10 peak in each of the first four blocks: in the marginal picks of blocks
    # 1-3 (below), so that those blocks hold most of the positive residual weight
    peaks = np.array([rng.integers(j * blk, (j + 1) * blk) for j in range(4)])
    logits[:, :, peaks] += 10.0
    logits = logits.astype(np.float32)
    if dtype == "bf16":
        logits = (f32_to_bf16_bits(logits).astype(np.uint32) << 16).view(np.float32)
    q = np.zeros((B, g, V), dtype=np.float32)
    ids = np.zeros((B, g), dtype=np.int32)
    for b in range(B):
        for i in range(g):
            p = scipy.special.softmax(logits[b, i].astype(np.float64))
            qq = (1.001 if only else 0.5) * p
            for j, count in enumerate([0, 1, 2, 3, blk]):
                toks = np.arange(j * blk, (j + 1) * blk)
                pick = toks if count == blk else rng.choice(toks, count, replace=False)
                if 0 < count < blk and peaks[j] not in pick:
                    pick[0] = peaks[j]
                eps = rng.uniform(-4e-6, -1e-6, size=len(pick)) if only else rng.uniform(-4e-6, 4e-6, size=len(pick))
                qq[pick] = p[pick] * (1.0 + eps)
            x = int(np.argmin(p[:blk]))              # a drafted token far less likely under p
            qq[x] = 0.0
            qq[x] = 0.5 if only else 1.0 - qq.sum()
            q[b, i] = qq.astype(np.float32)
            ids[b, i] = x
    u = uniform_grid_u(rng, (B, g + 2))
    inp = explicit_inputs(logits, q, ids, np.ones(B, dtype=np.float32), u)
    if dtype == "bf16":
        inp = _as(inp, "bf16")
    return inp


@pytest.mark.parametrize("only", [False, True], ids=["mixed", "only_marginal"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_marginal_tokens_in_residual_blocks(dtype, only):
    inp = _marginal_case(dtype, (77 if dtype == "f32" else 78) + (10 if only else 0), only)
    log(f"[marginal] B={inp.batch} gamma={inp.gamma} V={inp.vocab} {inp.dtype} only={only}")
    o = oracle.verify(inp)
    assert (o.num_accepted == 0).all()                # every request draws from a residual row
    sets = [inp.uniforms] + [uniforms_from_seed(inp.uniforms.shape, 600 + s) for s in range(15)]
    if only:
        # the drawn tokens are marginal ones, in blocks of 1 and 2 inline tokens
        # and in blocks summed again from their tokens
        drawn = {int(t) // 2048 for t in o.tokens[:, 0]}
        assert {1, 2, 3} <= drawn and 0 not in drawn
    rep, errs, _ = parity_check(inp, sets, label=f"marginal-{dtype}-{'only' if only else 'mixed'}")
    assert not rep.unexcused, "\n".join(rep.unexcused[:10])
    assert not errs, errs
