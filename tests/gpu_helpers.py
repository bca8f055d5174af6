"""GPU-side test helpers: run the HIP path on synthetic inputs, apply the parity rules.

Parity rules (GPU vs the CPU oracle on identical inputs and uniforms):
  * tokens and num_accepted are bit-exact per request, except in an excused
    request, whose first differing decision is either an accept test with
    |u - min(1, r_oracle)| < 1e-6, or a draw whose GPU token has an oracle
    interval [C_{y-1}/S, C_y/S) within 1e-6 of the uniform.  Greedy requests
    are never excused.  Excused requests must stay below 1e-4 of all requests.
  * every target row's max is bit-exact; Z of sampled rows and p(x)/q(x) of
    sampled drafts agree to 1e-5 relative (below p = 2^-126, absolutely).
"""

from __future__ import annotations

import dataclasses
import sys
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

import oracle
from oracle.rejection_sampler import draw_weights, token_interval

THRESH = 1e-6
REL_TOL = 1e-5


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


@dataclass
class ParityReport:
    requests: int = 0
    mismatched: int = 0
    excused: int = 0
    unexcused: List[str] = field(default_factory=list)

    def merge(self, other: "ParityReport") -> None:
        self.requests += other.requests
        self.mismatched += other.mismatched
        self.excused += other.excused
        self.unexcused.extend(other.unexcused)


def upload_inputs(inp, device="cuda:0", diag=True, stats=False):
    from lossless_rejection_sampling_sampler_amd import upload
    return upload(logits=inp.logits, logits_dtype=inp.dtype, draft_probs=inp.draft_probs,
                  draft_ids=inp.draft_ids, temperature=inp.temperature, uniforms=inp.uniforms,
                  gamma=inp.gamma, draft_offsets=inp.offsets, device=device, diag=diag,
                  topk_ids=getattr(inp, "topk_ids", None), topk_probs=getattr(inp, "topk_probs", None),
                  stats=stats)


def make_verifier(inp, max_batch=None, max_gamma=None, profile=False, schedule=None):
    """A context for ``inp``; schedule None is the library's choice, else "twokernel"."""
    from lossless_rejection_sampling_sampler_amd import SpecVerify
    return SpecVerify(max_batch or inp.batch, inp.gamma if max_gamma is None else max_gamma,
                      inp.vocab, inp.dtype, device=0, profile=profile, schedule=schedule)


def run_gpu(inp, uniform_sets: Optional[list] = None, sv=None, diag=True, schedule=None):
    """Run the HIP path; returns (list of (tokens, num_accepted), diag dict)."""
    import torch
    if sv is None:
        sv = make_verifier(inp, schedule=schedule)
    db = upload_inputs(inp, diag=diag)
    sets = uniform_sets if uniform_sets is not None else [inp.uniforms]
    results = []
    for u in sets:
        db.uniforms.copy_(torch.from_numpy(np.ascontiguousarray(u, dtype=np.float32)))
        db.out_tokens.fill_(-7)
        db.out_num_accepted.fill_(-7)
        db.run(sv)
        torch.cuda.synchronize()
        results.append(db.results())
    dg = {}
    if diag:
        dg = dict(row_max=db.diag_row_max.cpu().numpy(), row_norm=db.diag_row_norm.cpu().numpy(),
                  ratio=db.diag_ratio.cpu().numpy())
    return results, dg, sv


def compare(inp, u: np.ndarray, gpu_tokens, gpu_num, orc) -> ParityReport:
    rep = ParityReport(requests=inp.batch)
    gam = inp.gammas
    off = inp.draft_offsets
    greedy = ~(inp.temperature.astype(np.float64) > 0)
    G = inp.gamma
    for b in range(inp.batch):
        if gpu_num[b] == orc.num_accepted[b] and np.array_equal(gpu_tokens[b], orc.tokens[b]):
            continue
        rep.mismatched += 1
        ko, kg = int(orc.num_accepted[b]), int(gpu_num[b])
        why = f"request {b}: oracle k={ko} tokens={orc.tokens[b].tolist()} gpu k={kg} tokens={gpu_tokens[b].tolist()}"
        if greedy[b]:
            rep.unexcused.append("greedy " + why)
            continue
        if not (0 <= kg <= gam[b]):
            rep.unexcused.append("bad k " + why)
            continue
        if ko != kg:
            i = min(ko, kg)
            r = float(orc.ratio[off[b] + i])
            if abs(float(u[b, i]) - min(1.0, r)) < THRESH:
                rep.excused += 1
            else:
                rep.unexcused.append(f"accept@{i} u={u[b, i]!r} r={r!r} " + why)
            continue
        k = ko
        if not np.array_equal(gpu_tokens[b, :k], orc.tokens[b, :k]) or np.any(gpu_tokens[b, k + 1:] != -1):
            rep.unexcused.append("layout " + why)
            continue
        y = int(gpu_tokens[b, k])
        if not (0 <= y < inp.vocab):
            rep.unexcused.append("token range " + why)
            continue
        w, _ = draw_weights(inp, b, k)
        lo, hi = token_interval(w, y)
        v = float(u[b, G] if k < gam[b] else u[b, G + 1])
        dist = 0.0 if lo <= v < hi else min(abs(v - lo), abs(v - hi))
        if dist < THRESH:
            rep.excused += 1
        else:
            rep.unexcused.append(f"draw v={v!r} gpu interval=[{lo!r},{hi!r}) " + why)
    return rep


def check_diag(inp, orc, dg) -> List[str]:
    errs = []
    if not dg:
        return errs
    R = inp.total_rows
    if not np.array_equal(dg["row_max"].astype(np.float64), orc.row_max[:R]):
        bad = np.nonzero(dg["row_max"].astype(np.float64) != orc.row_max)[0]
        errs.append(f"row max differs at rows {bad[:10].tolist()}")
    T = inp.temperature.astype(np.float64)
    gam = inp.gammas
    off = inp.draft_offsets
    sampled_rows = np.zeros(R, dtype=bool)
    sampled_drafts = np.zeros(inp.total_draft, dtype=bool)
    for b in range(inp.batch):
        if T[b] > 0:
            sampled_rows[off[b] + b: off[b] + b + gam[b] + 1] = True
            sampled_drafts[off[b]: off[b] + gam[b]] = True
    zo, zg = orc.row_norm[sampled_rows], dg["row_norm"][sampled_rows]
    rel = np.abs(zg - zo) / zo
    if rel.size and not np.all(rel <= REL_TOL):
        errs.append(f"row norm rel err max {rel.max():.3e}")
    if np.any(dg["row_norm"][~sampled_rows] != 0):
        errs.append("greedy row norm not 0")
    ro = orc.ratio[sampled_drafts]
    rg = dg["ratio"][sampled_drafts].astype(np.float64)
    big = np.abs(ro) >= 2.0 ** -126          # the fp32 output is relative-accurate there
    relr = np.abs(rg[big] - ro[big]) / np.abs(ro[big])
    if relr.size and not np.all(relr <= REL_TOL):
        errs.append(f"ratio rel err max {relr.max():.3e}")
    small = ~big
    if np.any(np.abs(rg[small] - ro[small]) > 2.0 ** -126):
        errs.append("tiny ratio abs err")
    if not np.all(np.isnan(dg["ratio"][~sampled_drafts])):
        errs.append("greedy ratio not NaN")
    return errs


def parity_check(inp, uniform_sets: Optional[list] = None, sv=None, label="", schedule=None):
    """Run GPU and oracle on ``inp`` (optionally many uniform sets); returns the report."""
    sets = uniform_sets if uniform_sets is not None else [inp.uniforms]
    log(f"[parity] {label} B={inp.batch} gamma={inp.gamma} V={inp.vocab} {inp.dtype} sets={len(sets)} "
        f"schedule={schedule or 'auto'}: gpu")
    res, dg, sv = run_gpu(inp, sets, sv=sv, schedule=schedule)
    rep = ParityReport()
    errs = []
    chunk = 16                      # sets per oracle call: a progress line every few seconds
    for c0 in range(0, len(sets), chunk):
        log(f"[parity] {label}: oracle sets {c0}..{min(c0 + chunk, len(sets)) - 1}")
        orcs = oracle.verify(inp, uniform_sets=sets[c0:c0 + chunk])
        for (tok, num), orc, u in zip(res[c0:c0 + chunk], orcs, sets[c0:c0 + chunk]):
            rep.merge(compare(inp, u, tok, num, orc))
        if c0 == 0:
            errs = check_diag(inp, orcs[0], dg)
    log(f"[parity] {label}: requests={rep.requests} mismatched={rep.mismatched} "
        f"excused={rep.excused} unexcused={len(rep.unexcused)} diag_errors={errs}")
    return rep, errs, sv
