"""fp64 CPU oracle of the MoE layer: route, count, lay out, gather, expert
SwiGLU FFN, weighted combine, the backward of the expert path, and the
router backward through the gates.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Plain numpy, fp64 for
every floating-point step; the one place where floating point decides an
integer (top-k selection) compares the logits in the precision they are
handed in, which is the kernel's fp32.

Citations: "MoK flash" = the page "Cursor's MoK achieves 2.37x performance
boost on NVIDIA GB300 NVL72" (KuCoin news flash), by article section.

Storage conventions (the same ones the C ABI declares):
  x    [T, d]      token activations
  wr   [E, d]      router weight, row e scores expert e
  bias [E] | None  added to the logits
  w1   [E, I, d]   gate projection, row i is output feature i
  w3   [E, I, d]   up projection
  w2   [E, d, I]   down projection
  A routed assignment is numbered a = t*k + j (token t, slot j).

Readings the pages leave open (each is listed in the design notes):
  * selection = the k largest logits, ties to the lower expert index
    (softmax and sigmoid are strictly increasing, so this is the top-k of
    the scores without their rounding);
  * rows inside an expert's segment are in increasing assignment order
    (stable counting sort), which makes the permutation unique;
  * SwiGLU is silu(x W1^T) * (x W3^T), followed by W2;
  * no capacity limit: every assignment is processed.
"""
from __future__ import annotations

import numpy as np

SOFTMAX = "softmax"
SIGMOID = "sigmoid"


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# Router.  MoK flash §01: the router re-decides every step which experts a
# token goes to.  The score function and normalisation are not on the page;
# the workloads fix them (softmax or sigmoid, gates renormalised over the
# chosen experts).
# --------------------------------------------------------------------------
def router_logits(x, wr, bias=None):
    """logits[t, e] = <x[t], wr[e]> (+ bias[e]), in fp64."""
    logits = _f64(x) @ _f64(wr).T
    if bias is not None:
        logits = logits + _f64(bias)[None, :]
    return logits


def select_topk(logits, k):
    """The k experts with the largest logit per token, largest first; exact
    ties go to the lower expert index.  Returns int64 [T, k].

    A stable sort of the negated logits keeps equal logits in increasing
    expert order, so its first k entries are exactly this selection.
    """
    logits = np.asarray(logits)
    T, E = logits.shape
    if not (1 <= k <= E):
        raise ValueError("need 1 <= k <= E")
    order = np.argsort(-logits, axis=1, kind="stable")
    return order[:, :k].astype(np.int64)


def gates_from_logits(logits, idx, score, renorm):
    """fp64 gates for the selected experts.

    softmax, renorm    : exp(l_j - m) / sum over the selected set
    softmax, no renorm : the full softmax over all E experts, read at j
    sigmoid, renorm    : s_j / sum of the selected s
    sigmoid, no renorm : s_j
    """
    l = _f64(logits)
    T, k = idx.shape
    sel = np.take_along_axis(l, idx, axis=1)
    if score == SOFTMAX:
        if renorm:
            m = sel.max(axis=1, keepdims=True)
            ex = np.exp(sel - m)
            return ex / ex.sum(axis=1, keepdims=True)
        m = l.max(axis=1, keepdims=True)
        ex_all = np.exp(l - m)
        return np.exp(sel - m) / ex_all.sum(axis=1, keepdims=True)
    if score == SIGMOID:
        s = 1.0 / (1.0 + np.exp(-sel))
        if renorm:
            return s / s.sum(axis=1, keepdims=True)
        return s
    raise ValueError(f"unknown score function {score!r}")


def select_grouped(keys, k, n_group, topk_group):
    """Group-limited selection.  The E experts form n_group groups of E /
    n_group consecutive ids; a group's score is the sum of its two largest
    keys (its only key when a group holds one expert); the topk_group groups
    with the largest scores are kept (ties to the lower group), and the k
    largest keys among the kept experts are chosen (ties to the lower
    expert), largest first."""
    keys = np.asarray(keys)
    T, E = keys.shape
    if E % n_group or not (1 <= topk_group <= n_group) or k > topk_group * (E // n_group):
        raise ValueError("bad grouping")
    gs = E // n_group
    grouped = keys.reshape(T, n_group, gs)
    top = -np.sort(-grouped, axis=2)
    gscore = top[:, :, 0] + (top[:, :, 1] if gs > 1 else 0.0)
    kept = np.argsort(-gscore, axis=1, kind="stable")[:, :topk_group]
    allowed = np.zeros((T, n_group), dtype=bool)
    np.put_along_axis(allowed, kept, True, axis=1)
    masked = np.where(np.repeat(allowed, gs, axis=1), keys, -np.inf)
    return select_topk(masked, k)


def route(logits, k, score, renorm, bias=None, select_only=False, n_group=0, topk_group=0,
          routed_scale=1.0):
    """Top-k selection and gates from router logits.

    ``bias`` (if given) is added to the logits in the logits' own dtype
    before anything else, so an fp32 caller gets the same fp32 sums the
    kernel forms; selection then compares those values directly.

    DeepSeek-V3-style options (sigmoid scores only):
      select_only  the bias steers the selection only: the experts are
                   ranked by sigmoid(logit) + bias and the gates come from
                   the unbiased logits
      n_group > 1  group-limited selection (select_grouped) over the keys
                   sigmoid(z) + (bias if select_only), z the gate logits
    With either option the keys live in score space; the plain path ranks
    the (biased) logits themselves.  routed_scale multiplies every gate.
    """
    logits = np.asarray(logits)
    keyed = select_only or n_group > 1
    if keyed and score != SIGMOID:
        raise ValueError("selection-only bias and grouped routing need sigmoid scores")
    z = logits
    if bias is not None and not select_only:
        z = logits + np.asarray(bias, dtype=logits.dtype)[None, :]
    if keyed:
        keys = sigmoid(_f64(z))
        if select_only and bias is not None:
            keys = keys + _f64(bias)[None, :]
        idx = select_grouped(keys, k, n_group, topk_group) if n_group > 1 else select_topk(keys, k)
    else:
        idx = select_topk(z, k)
    gate = gates_from_logits(z, idx, score, renorm) * routed_scale
    return idx, gate


# --------------------------------------------------------------------------
# Counting and layout.  MoK flash §01: count how many tokens each expert has
# first, then decide where each lands, keeping one expert's rows together so
# the grouped GEMM gets organised input.  §02: the same contiguity is why
# push senders must know their target section in advance.
# --------------------------------------------------------------------------
def layout(topk_idx, E):
    """Stable counting sort of the T*k assignments by expert.

    counts[e]   rows routed to expert e
    offsets     exclusive prefix sum of counts, length E+1
    perm[r]     the assignment a = t*k+j that lands on row r
    inv[a]      the row of assignment a (inv o perm = id)
    src[r]      the source token of row r (= perm[r] // k)
    """
    idx = np.asarray(topk_idx)
    T, k = idx.shape
    flat = idx.reshape(-1)
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert index out of range")
    counts = np.zeros(E, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    fill = offsets[:-1].copy()
    R = T * k
    perm = np.empty(R, dtype=np.int64)
    inv = np.empty(R, dtype=np.int64)
    for a in range(R):
        e = flat[a]
        r = fill[e]
        fill[e] += 1
        perm[r] = a
        inv[a] = r
    src = perm // k
    return counts, offsets, perm, inv, src


# --------------------------------------------------------------------------
# Pull dispatch = gather.  MoK flash §02: the receiver pulls each token it
# needs given only where the token lives, and lays rows out itself.  On one
# GPU the source is always local, so this is a row gather.
# --------------------------------------------------------------------------
def gather(x, src):
    return np.asarray(x)[np.asarray(src)]


# --------------------------------------------------------------------------
# Expert FFN.  MoK flash §02 names the SwiGLU expert FFN behind the grouped
# GEMM; the formula is the usual gated form.
# --------------------------------------------------------------------------
def silu(a):
    return a / (1.0 + np.exp(-a))


def sigmoid(a):
    return 1.0 / (1.0 + np.exp(-a))


def expert_ffn(xp_e, w1_e, w3_e, w2_e):
    """One expert over its rows: returns (A, B, H, Yp) in fp64."""
    xp_e = _f64(xp_e)
    A = xp_e @ _f64(w1_e).T
    B = xp_e @ _f64(w3_e).T
    H = silu(A) * B
    Yp = H @ _f64(w2_e).T
    return A, B, H, Yp


def grouped_ffn(xp, offsets, w1, w3, w2):
    """Apply each expert to its contiguous segment of rows."""
    R = xp.shape[0]
    E, I, d = np.shape(w1)
    A = np.zeros((R, I))
    B = np.zeros((R, I))
    H = np.zeros((R, I))
    Yp = np.zeros((R, d))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        A[lo:hi], B[lo:hi], H[lo:hi], Yp[lo:hi] = expert_ffn(
            xp[lo:hi], w1[e], w3[e], w2[e])
    return A, B, H, Yp


# --------------------------------------------------------------------------
# Combine and final weighted merge.  MoK flash §01: results go back to each
# token's original position; §03: the benchmark includes the final weighted
# merge.
# --------------------------------------------------------------------------
def combine(yp, gate, inv, T, k):
    yp = _f64(yp)
    gate = _f64(gate)
    d = yp.shape[1]
    y = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            y[t] += gate[t, j] * yp[inv[t * k + j]]
    return y


def forward(x, wr, bias, w1, w3, w2, k, score, renorm, logits=None, **routing):
    """The whole forward.  Returns a dict of every intermediate.

    ``logits`` may be given to route on fixed logits (fp32 as the kernel
    would form them); otherwise the fp64 router GEMM is used.  ``routing``
    takes route()'s DeepSeek-V3-style options.
    """
    T = np.shape(x)[0]
    E = np.shape(w1)[0]
    if logits is None:
        logits = router_logits(x, wr, None)
    idx, gate = route(logits, k, score, renorm, bias, **routing)
    counts, offsets, perm, inv, src = layout(idx, E)
    xp = gather(_f64(x), src)
    A, B, H, Yp = grouped_ffn(xp, offsets, w1, w3, w2)
    y = combine(Yp, gate, inv, T, k)
    return dict(logits=logits, topk_idx=idx, gate=gate, counts=counts,
                offsets=offsets, perm=perm, inv=inv, src=src, xp=xp,
                A=A, B=B, H=H, Yp=Yp, y=y)


# --------------------------------------------------------------------------
# Backward of the expert path with the routing frozen.  MoK flash §01:
# training adds two exchanges in the opposite direction; §02: the backward
# pulls the reverse-combine and pushes the reverse-dispatch.
# --------------------------------------------------------------------------
def backward(dy, fwd, w1, w3, w2, k):
    """Gradients of L = <dy, y> w.r.t. x (expert path), w1, w3, w2, gates.

    Steps, in order:
      (i)   reverse combine: G[r] = dy[src[r]]   (a pull gather)
      (ii)  dHu = G W2;  dgate_row[r] = <dHu[r], H[r]>;  dH = g_r dHu
      (iii) dW2_e = (g G)_e^T H_e
      (iv)  SwiGLU backward: dA = dH * B * s(A)(1 + A(1 - s(A))),
            dB = dH * silu(A)
      (v)   dXp = dA W1 + dB W3
      (vi)  dW1_e = dA_e^T Xp_e,  dW3_e = dB_e^T Xp_e
      (vii) reverse dispatch: dx[t] = sum_j dXp[inv[t*k+j]]  (scatter-add)
    """
    dy = _f64(dy)
    T, d = dy.shape
    E, I, _ = np.shape(w1)
    offsets, perm, inv, src = fwd["offsets"], fwd["perm"], fwd["inv"], fwd["src"]
    gate = _f64(fwd["gate"])
    A, B, H, xp = fwd["A"], fwd["B"], fwd["H"], fwd["xp"]
    R = perm.shape[0]
    g_row = gate.reshape(-1)[perm]                 # gate of each row
    G = dy[src]                                    # (i)
    dHu = np.zeros((R, I))
    dW1 = np.zeros((E, I, d))
    dW3 = np.zeros((E, I, d))
    dW2 = np.zeros((E, d, I))
    dXp = np.zeros((R, d))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        dHu[lo:hi] = G[lo:hi] @ _f64(w2[e])                            # (ii)
        dW2[e] = (g_row[lo:hi, None] * G[lo:hi]).T @ H[lo:hi]          # (iii)
    dgate_row = np.sum(dHu * H, axis=1)
    dH = g_row[:, None] * dHu
    sA = sigmoid(A)
    dA = dH * B * sA * (1.0 + A * (1.0 - sA))                          # (iv)
    dB = dH * silu(A)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        dXp[lo:hi] = dA[lo:hi] @ _f64(w1[e]) + dB[lo:hi] @ _f64(w3[e])  # (v)
        dW1[e] = dA[lo:hi].T @ xp[lo:hi]                                # (vi)
        dW3[e] = dB[lo:hi].T @ xp[lo:hi]
    dx = np.zeros((T, d))
    for t in range(T):                                                  # (vii)
        for j in range(k):
            dx[t] += dXp[inv[t * k + j]]
    dgate = dgate_row[inv].reshape(T, k)
    return dict(dx=dx, dw1=dW1, dw3=dW3, dw2=dW2, dgate=dgate,
                G=G, dHu=dHu, dA=dA, dB=dB, dXp=dXp)


# --------------------------------------------------------------------------
# Router backward with the selection frozen.  MoK flash §01: the router
# decides every step which experts a token goes to; training runs the layer
# backwards, and the router's part of that is the gradient through the gates
# (the choice itself is piecewise constant and passes no gradient).
# --------------------------------------------------------------------------
def gate_grad_to_logits(z, idx, dgate, score, renorm, routed_scale=1.0):
    """dL/dz [T, E] from dL/dgate [T, k] for the gate logits z [T, E] (the
    logits the gates are computed from).  Gates scaled by routed_scale c pass
    c dL/dgate to the unscaled gates g below.

    Two chain-rule steps, gates -> scores -> logits:
      softmax, renorm    : g = exp(z_sel) / sum exp(z_sel);
                           dz_j = g_j (dg_j - sum_i g_i dg_i), chosen j only
      softmax, no renorm : g_j = p(z)[e_j] with p the softmax over all E;
                           dz_e = p_e ([e chosen] dg_e - sum_j g_j dg_j)
      sigmoid, renorm    : g = s_sel / S, S = sum s_sel, s = sigmoid(z);
                           dL/ds_j = (dg_j - sum_i g_i dg_i) / S,
                           dz_j = dL/ds_j * s_j (1 - s_j)
      sigmoid, no renorm : dz_j = dg_j s_j (1 - s_j)
    """
    z = _f64(z)
    dg = _f64(dgate) * routed_scale
    T, E = z.shape
    k = idx.shape[1]
    zsel = np.take_along_axis(z, idx, axis=1)
    dz = np.zeros((T, E))
    if score == SOFTMAX:
        if renorm:
            g = np.exp(zsel - zsel.max(axis=1, keepdims=True))
            g = g / g.sum(axis=1, keepdims=True)
            dsel = g * (dg - np.sum(g * dg, axis=1, keepdims=True))
        else:
            p = np.exp(z - z.max(axis=1, keepdims=True))
            p = p / p.sum(axis=1, keepdims=True)
            g = np.take_along_axis(p, idx, axis=1)
            dp = np.zeros((T, E))
            np.put_along_axis(dp, idx, dg, axis=1)
            return p * (dp - np.sum(g * dg, axis=1, keepdims=True))
    elif score == SIGMOID:
        sv = sigmoid(zsel)
        if renorm:
            S = sv.sum(axis=1, keepdims=True)
            g = sv / S
            ds = (dg - np.sum(g * dg, axis=1, keepdims=True)) / S
        else:
            ds = dg
        dsel = ds * sv * (1.0 - sv)
    else:
        raise ValueError(f"unknown score function {score!r}")
    np.put_along_axis(dz, idx, dsel, axis=1)
    return dz


def router_backward(x, wr, z, idx, dgate, score, renorm, routed_scale=1.0, select_only=False):
    """Gradients of the router for the gate logits z = x wr^T (+ bias unless
    the bias only steers the selection): dz = gate_grad_to_logits(...),
    dwr = dz^T x, dbias = sum_t dz (zero for a selection-only bias, which the
    gates never see), dx_router = dz wr (to be added to the expert path's
    dx)."""
    dz = gate_grad_to_logits(z, idx, dgate, score, renorm, routed_scale)
    dbias = np.zeros(dz.shape[1]) if select_only else dz.sum(axis=0)
    return dict(dlogits=dz, dwr=dz.T @ _f64(x), dbias=dbias, dx=dz @ _f64(wr))


# --------------------------------------------------------------------------
# Per-token and per-expert slices, used to check full-size runs at sampled
# outputs without the whole layer on the CPU.
# --------------------------------------------------------------------------
def token_output(x_t, experts, gates, w1, w3, w2):
    """y[t] for one token given its chosen experts and gates (fp64)."""
    y = np.zeros(np.shape(w2)[1])
    for e, g in zip(experts, gates):
        _, _, _, yp = expert_ffn(_f64(x_t)[None, :], w1[e], w3[e], w2[e])
        y += g * yp[0]
    return y


def expert_backward(x_rows, dy_rows, g_rows, w1_e, w3_e, w2_e, saved=None):
    """Backward of one expert over its rows (in segment order).

    ``saved`` = (A, B, H) of this expert's forward, recomputed when None.
    Returns dW1_e, dW3_e, dW2_e, the per-row dXp and the per-row dgate.
    """
    if saved is None:
        A, B, H, _ = expert_ffn(x_rows, w1_e, w3_e, w2_e)
    else:
        A, B, H = saved
    G = _f64(dy_rows)
    g = _f64(g_rows)
    dHu = G @ _f64(w2_e)
    dgate_row = np.sum(dHu * H, axis=1)
    dH = g[:, None] * dHu
    dW2 = (g[:, None] * G).T @ H
    sA = sigmoid(A)
    dA = dH * B * sA * (1.0 + A * (1.0 - sA))
    dB = dH * silu(A)
    dXp = dA @ _f64(w1_e) + dB @ _f64(w3_e)
    xr = _f64(x_rows)
    return dict(dw1=dA.T @ xr, dw3=dB.T @ xr, dw2=dW2, dxp=dXp,
                dgate=dgate_row)


# --------------------------------------------------------------------------
# Dense brute force: every expert on every token, masked by the top-k gates.
# Used only to pin the routed oracle above.
# --------------------------------------------------------------------------
def dense_brute_force(x, w1, w3, w2, topk_idx, gate):
    x = _f64(x)
    T = x.shape[0]
    E = np.shape(w1)[0]
    mask = np.zeros((T, E))
    for t in range(T):
        for j in range(topk_idx.shape[1]):
            mask[t, topk_idx[t, j]] = gate[t, j]
    y = np.zeros((T, np.shape(w2)[1]))
    for e in range(E):
        _, _, _, yp = expert_ffn(x, w1[e], w3[e], w2[e])
        y += mask[:, e:e + 1] * yp
    return y


# --------------------------------------------------------------------------
# Comparison metric for floating outputs: per output row, the max-norm error
# relative to the max norm of the expected row; rows whose expected max norm
# is zero are skipped.
# --------------------------------------------------------------------------
def max_row_rel_err(got, want):
    got = _f64(got).reshape(np.shape(want)[0], -1)
    want = _f64(want).reshape(np.shape(want)[0], -1)
    num = np.max(np.abs(got - want), axis=1)
    den = np.max(np.abs(want), axis=1)
    ok = den > 0
    if not np.any(ok):
        return float(np.max(num)) if num.size else 0.0
    return float(np.max(num[ok] / den[ok]))
