"""Moves host (numpy) verifier inputs into torch device tensors and back.

Marshalling only; no part of the verify arithmetic lives here.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np


@dataclass
class DeviceBatch:
    batch: int
    gamma: int
    vocab: int
    total_draft: int
    logits_dtype: str
    target_logits: "object"         # torch tensor [R, V] bfloat16 / float32
    draft_probs: "object"           # [D, V] float32
    draft_ids: "object"             # [D] int32
    temperature: "object"           # [B] float32
    uniforms: "object"              # [B, gamma+2] float32
    draft_offsets: Optional["object"]   # [B+1] int32 or None
    out_tokens: "object"            # [B, gamma+1] int32
    out_num_accepted: "object"      # [B] int32
    diag_row_max: Optional["object"] = None
    diag_row_norm: Optional["object"] = None
    diag_ratio: Optional["object"] = None
    draft_topk: int = 0                     # sparse q entries per row (draft_probs None)
    draft_topk_ids: Optional["object"] = None
    draft_topk_probs: Optional["object"] = None
    stats: Optional["object"] = None        # [SV_STATS_LEN(gamma)] uint32 counters (int32 storage)

    def run(self, sv, stream=None) -> None:
        sv.run(target_logits=self.target_logits, draft_probs=self.draft_probs,
               draft_ids=self.draft_ids, temperature=self.temperature, uniforms=self.uniforms,
               out_tokens=self.out_tokens, out_num_accepted=self.out_num_accepted,
               gamma=self.gamma, draft_offsets=self.draft_offsets, total_draft=self.total_draft,
               diag_row_max=self.diag_row_max, diag_row_norm=self.diag_row_norm,
               diag_ratio=self.diag_ratio, draft_topk=self.draft_topk, draft_topk_ids=self.draft_topk_ids,
               draft_topk_probs=self.draft_topk_probs, stats=self.stats, stream=stream)

    def args(self):
        """The packed C argument block for this batch (for repeated raw calls)."""
        from ._lib import SVArgs
        p = lambda t: 0 if t is None else int(t.data_ptr())
        return SVArgs(self.batch, self.gamma, self.total_draft, self.vocab, p(self.draft_offsets),
                      p(self.target_logits), p(self.draft_probs), p(self.draft_ids), p(self.temperature),
                      p(self.uniforms), p(self.out_tokens), p(self.out_num_accepted),
                      p(self.diag_row_max), p(self.diag_row_norm), p(self.diag_ratio),
                      int(self.draft_topk), p(self.draft_topk_ids), p(self.draft_topk_probs), p(self.stats))

    def results(self):
        """(tokens, num_accepted) as numpy arrays (synchronises)."""
        return self.out_tokens.cpu().numpy(), self.out_num_accepted.cpu().numpy()


def upload(*, logits: np.ndarray, logits_dtype: str, draft_probs: Optional[np.ndarray], draft_ids: np.ndarray,
           temperature: np.ndarray, uniforms: np.ndarray, gamma: int,
           draft_offsets: Optional[np.ndarray] = None, device="cuda:0", diag: bool = False,
           fill_outputs: int = -7, topk_ids: Optional[np.ndarray] = None,
           topk_probs: Optional[np.ndarray] = None, stats: bool = False) -> DeviceBatch:
    """Copy one batch to the device.  bf16 logits arrive as uint16 bit patterns.

    draft_probs None: q is sparse when topk_ids / topk_probs ([D, K]) are given,
    else a point mass at each drafted token.  stats: allocate zeroed acceptance
    counters."""
    import torch
    dev = torch.device(device)
    B = int(temperature.shape[0])
    V = int(logits.shape[-1])
    if logits_dtype == "bf16":
        lt = torch.from_numpy(np.ascontiguousarray(logits).view(np.int16)).to(dev).view(torch.bfloat16)
    elif logits_dtype == "f32":
        lt = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).to(dev)
    else:
        raise ValueError(logits_dtype)
    D = int(draft_ids.shape[0])
    R = int(logits.shape[0])
    q = None
    if draft_probs is not None:
        q = torch.from_numpy(np.ascontiguousarray(draft_probs, dtype=np.float32)).to(dev)
    ids = torch.from_numpy(np.ascontiguousarray(draft_ids, dtype=np.int32)).to(dev)
    T = torch.from_numpy(np.ascontiguousarray(temperature, dtype=np.float32)).to(dev)
    u = torch.from_numpy(np.ascontiguousarray(uniforms, dtype=np.float32)).to(dev)
    off = None
    if draft_offsets is not None:
        off = torch.from_numpy(np.ascontiguousarray(draft_offsets, dtype=np.int32)).to(dev)
    out_t = torch.full((B, gamma + 1), fill_outputs, dtype=torch.int32, device=dev)
    out_n = torch.full((B,), fill_outputs, dtype=torch.int32, device=dev)
    db = DeviceBatch(B, int(gamma), V, D, logits_dtype, lt, q, ids, T, u, off, out_t, out_n)
    if draft_probs is None and topk_ids is not None:
        db.draft_topk = int(topk_ids.shape[1])
        db.draft_topk_ids = torch.from_numpy(np.ascontiguousarray(topk_ids, dtype=np.int32)).to(dev)
        db.draft_topk_probs = torch.from_numpy(np.ascontiguousarray(topk_probs, dtype=np.float32)).to(dev)
    if stats:
        from ._lib import stats_len
        db.stats = torch.zeros(stats_len(gamma), dtype=torch.int32, device=dev)
    if diag:
        db.diag_row_max = torch.full((R,), float("nan"), dtype=torch.float32, device=dev)
        db.diag_row_norm = torch.full((R,), float("nan"), dtype=torch.float64, device=dev)
        db.diag_ratio = torch.full((D,), float("nan"), dtype=torch.float32, device=dev)
    return db
