"""Helpers shared by the GPU parity tests: host copies, routing comparison
with near-tie accounting, and the row-wise relative error."""
from __future__ import annotations

import numpy as np
import torch

from oracle import moe as M


def host(t):
    """fp64 (or int64) numpy copy of a tensor."""
    if t.dtype in (torch.int32, torch.int64, torch.uint8):
        return t.detach().cpu().numpy().astype(np.int64)
    return t.detach().float().cpu().numpy().astype(np.float64)


def logit_tolerance(x, wr):
    """Per-token bound on |fp32 logit - exact logit| used to call a top-k
    margin a near tie: 64 ulps of fp32 at the scale ||x_t|| * max_e ||w_e||
    (the size of the largest partial sum of the dot product)."""
    xn = np.linalg.norm(x, axis=1)
    wn = np.max(np.linalg.norm(wr, axis=1))
    return 64 * 2.0 ** -24 * xn * wn


def compare_routing(gpu_idx, ora_logits, ora_idx, tol):
    """Tokens whose k-th / (k+1)-th logit margin exceeds ``tol`` must select
    exactly the oracle's experts in the oracle's order; near-tie tokens must
    select a valid set (every chosen logit within tol of the k-th largest).
    Returns the boolean mask of tokens that matched exactly."""
    T, k = ora_idx.shape
    E = ora_logits.shape[1]
    srt = -np.sort(-ora_logits, axis=1)
    kth = srt[:, k - 1]
    nxt = srt[:, k] if k < E else np.full(T, -np.inf)
    clear = (kth - nxt) > tol
    same = np.all(gpu_idx == ora_idx, axis=1)
    bad = clear & ~same
    assert not bad.any(), f"{bad.sum()} tokens with a clear margin routed differently: {np.nonzero(bad)[0][:10]}"
    for t in np.nonzero(~clear)[0]:
        chosen = ora_logits[t, gpu_idx[t]]
        assert len(set(gpu_idx[t].tolist())) == k
        assert np.all(chosen >= kth[t] - tol[t]), f"token {t}: invalid near-tie choice"
    return same


def row_rel_err(got, want, rows=None):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    if rows is not None:
        got, want = got[rows], want[rows]
    return M.max_row_rel_err(got, want)
