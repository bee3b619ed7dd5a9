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


def dgate_err(got, want, floor=0.1):
    """Error of dgate [T, k].  Each entry is a dot product over I terms, and a
    token row holds only k of them: with small k a row whose entries all sit
    near zero by cancellation is common, and its row-relative error then
    measures the rounding of the bf16 operands, not the path.  Returns the
    larger of (a) the max error relative to the whole tensor's max norm and
    (b) the row-relative error over rows whose max norm is at least
    ``floor`` times the tensor's."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    scale = np.max(np.abs(want)) if want.size else 0.0
    if scale == 0.0:
        return float(np.max(np.abs(got))) if got.size else 0.0
    glob = float(np.max(np.abs(got - want)) / scale)
    rows = np.max(np.abs(want), axis=1) >= floor * scale
    return max(glob, M.max_row_rel_err(got[rows], want[rows]) if rows.any() else 0.0)
