"""fp64 oracle of the MXFP8 format: E4M3 elements, one E8M0 scale per block
of 32 consecutive elements along the contraction axis.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

MoK flash §02 folds MXFP8 quantisation into the dispatch, grouped GEMM and
SwiGLU datapath; the page names the format only.  The element and scale
encodings and the scale rule follow the OCP Microscaling Formats (MX) v1.0
specification (a public standard):
  * E4M3: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent field
    0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; the largest finite
    magnitude is 1.75 * 2^8 = 448; there is no infinity.
  * E8M0 scale: an unsigned biased exponent, value 2^(code-127); 255 is NaN.
  * Block scale: shared_exp = floor(log2(max |v|)) - 8 (8 = the largest
    E4M3 exponent), clamped to [-127, 127]; each element is v / 2^shared_exp
    rounded to nearest-even E4M3, with magnitudes beyond 448 clamped to 448.
    A block of zeros takes scale code 0 and zero elements.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
E4M3_MAX = 448.0
E4M3_EMAX = 8


def e4m3_value(code):
    """Decode one E4M3 code (0..255) to fp64 by the field definitions."""
    code = int(code)
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** (-6)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


def e4m3_table():
    """fp64 values of all 256 codes (NaN at 0x7F and 0xFF)."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


_POS = None


def _positive_codes():
    """(values, codes) of the 127 finite non-negative codes, increasing."""
    global _POS
    if _POS is None:
        codes = np.arange(0, 127, dtype=np.int64)          # 0x00 .. 0x7E
        vals = np.array([e4m3_value(c) for c in codes])
        assert np.all(np.diff(vals) > 0)
        _POS = (vals, codes)
    return _POS


def e4m3_encode_nearest(v):
    """Round fp64 values to E4M3 codes: nearest, ties to the even code
    (the even mantissa), magnitudes above 448 clamped to 448.  The
    definition, by search in the table of representable values."""
    v = np.asarray(v, dtype=np.float64)
    vals, codes = _positive_codes()
    mag = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(vals, mag, side="left")           # vals[hi] >= mag
    hi = np.clip(hi, 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    d_lo = mag - vals[lo]
    d_hi = vals[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0))
    pick_hi |= (hi == lo)
    out = np.where(pick_hi, codes[hi], codes[lo])
    neg = np.signbit(v) & (out != 0)
    return (out | np.where(neg, 0x80, 0)).astype(np.uint8)


def e4m3_encode(v):
    """The rounding of e4m3_encode_nearest in arithmetic form (fast on large
    arrays; the two are pinned equal in the tests).  With m = min(|v|, 448):
    the representable magnitudes are the multiples of 2^-9 below 2^-6
    (subnormals) and, in the binade [2^e, 2^(e+1)) for e >= -6, the
    multiples of 2^(e-3) (3 mantissa bits).  m divided by that step is
    exact in fp64 and is rounded half-to-even; counting grid points from
    zero (8 subnormal codes, then 8 codes per binade) gives the code, and a
    quotient that rounds up to 16 lands on the first code of the next
    binade."""
    v = np.asarray(v, dtype=np.float64)
    mag = np.minimum(np.abs(v), E4M3_MAX)
    _, ex = np.frexp(mag)                       # mag = f 2^ex, f in [0.5, 1)
    e = np.where(mag > 0, np.maximum(ex - 1, -6), -6)   # floor(log2 mag), at least -6
    q = np.rint(np.ldexp(mag, 3 - e))           # half to even
    out = ((e + 6) * 8 + q).astype(np.int64)
    neg = np.signbit(v) & (out != 0)
    return (out | np.where(neg, 0x80, 0)).astype(np.uint8)


def e8m0_value(code):
    code = np.asarray(code, dtype=np.int64)
    return np.where(code == 255, np.nan, np.ldexp(1.0, code - 127))


def block_scale_code(amax):
    """E8M0 code of the shared scale for blocks with the given max |v|."""
    amax = np.asarray(amax, dtype=np.float64)
    out = np.zeros(amax.shape, dtype=np.int64)
    nz = amax > 0
    # floor(log2(amax)) exactly, from frexp: amax = m * 2^e with m in [0.5, 1)
    _, e = np.frexp(amax[nz])
    shared = (e - 1) - E4M3_EMAX
    out[nz] = np.clip(shared, -127, 127) + 127
    return out.astype(np.uint8)


def _quantize_rows(v):
    K = v.shape[-1]
    blocks = v.reshape(v.shape[:-1] + (K // BLOCK, BLOCK))
    amax = np.max(np.abs(blocks), axis=-1)
    sc = block_scale_code(amax)
    scale = e8m0_value(sc)[..., None]
    codes = e4m3_encode(blocks / scale)
    return codes.reshape(v.shape), sc


def quantize(v):
    """Quantise along the last axis in blocks of 32.

    Returns (codes uint8 [..., K], scales uint8 [..., K/32]).  Rows are
    independent; large inputs go through in chunks of rows only to keep the
    temporaries small.
    """
    v = np.asarray(v, dtype=np.float64)
    K = v.shape[-1]
    if K % BLOCK:
        raise ValueError("last axis must be a multiple of 32")
    flat = v.reshape(-1, K)
    codes = np.empty(flat.shape, dtype=np.uint8)
    sc = np.empty((flat.shape[0], K // BLOCK), dtype=np.uint8)
    step = max(1, (1 << 19) // K)
    for r in range(0, flat.shape[0], step):
        codes[r:r + step], sc[r:r + step] = _quantize_rows(flat[r:r + step])
    return codes.reshape(v.shape), sc.reshape(v.shape[:-1] + (K // BLOCK,))


def dequantize(codes, scales):
    """fp64 values of codes [..., K] with scales [..., K/32] (exact)."""
    codes = np.asarray(codes, dtype=np.uint8)
    K = codes.shape[-1]
    table = e4m3_table()
    vals = table[codes.astype(np.int64)]
    sc = e8m0_value(np.asarray(scales)).repeat(BLOCK, axis=-1)
    return (vals.reshape(codes.shape) * sc.reshape(codes.shape[:-1] + (K,)))


def fake_quant(v):
    """quantize then dequantize, in fp64 (row chunks as in quantize)."""
    v = np.asarray(v, dtype=np.float64)
    K = v.shape[-1]
    flat = v.reshape(-1, K)
    out = np.empty(flat.shape)
    step = max(1, (1 << 16) // K)
    for r in range(0, flat.shape[0], step):
        out[r:r + step] = dequantize(*quantize(flat[r:r + step]))
    return out.reshape(v.shape)


def quantize_tokens(x):
    """The dispatch's quantisation: every token row of x [T, d] in blocks of
    32 along d (the up projection's contraction axis), fp64 values."""
    return fake_quant(np.asarray(x, dtype=np.float64))


def round_bf16(v):
    """fp64 -> the nearest bfloat16 value (8 significant bits: 1 implicit
    and 7 stored), ties to the even significand, returned as fp64.  From
    the format: v = m 2^e with m in [0.5, 1) (frexp), so the significand
    kept is rint(m 2^8) / 2^8; zero stays zero.  (Magnitudes below the
    bfloat16 normal range do not occur here.)"""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def quantize_along_rows(v):
    """v [n, C] quantised in blocks of 32 consecutive rows of each column:
    the token axis, which is the contraction axis of a weight gradient.
    Blocks start at row 0; a last partial block is filled with zero rows,
    which change no block maximum.  Returns the fp64 values [n, C]."""
    v = np.asarray(v, dtype=np.float64)
    n = v.shape[0]
    pad = (-n) % BLOCK
    if pad:
        v = np.concatenate([v, np.zeros((pad,) + v.shape[1:])])
    return fake_quant(v.T).T[:n]


def wgrad_mxfp8(lhs_rows, rhs_rows):
    """lhs^T rhs over the rows of one expert (lhs [n, P], rhs [n, Q] -> [P,
    Q]) with both operands quantised along the rows (quantize_along_rows)."""
    return quantize_along_rows(lhs_rows).T @ quantize_along_rows(rhs_rows)


def expert_ffn_mxfp8(xq_rows, w1, w3, w2):
    """One expert's SwiGLU FFN on rows that are already quantised (xq_rows,
    fp64 values of MXFP8 codes): W1/W3 quantised along d and W2 along I
    (blocks along each GEMM's contraction axis), H quantised along I after
    SwiGLU.  Returns (A, B, H, Yp) with H before its quantisation."""
    from . import moe as M
    w1q = fake_quant(w1)          # [I, d], blocks along d
    w3q = fake_quant(w3)
    w2q = fake_quant(w2)          # [d, I], blocks along I
    A = xq_rows @ w1q.T
    B = xq_rows @ w3q.T
    h = M.silu(A) * B
    return A, B, h, fake_quant(h) @ w2q.T


def _starmap(fn, jobs):
    for job in jobs:
        yield fn(*job)


def forward_mxfp8(x, wr, bias, w1, w3, w2, k, score, renorm, logits=None, expert_map=None):
    """The forward with the expert GEMMs in MXFP8.

    MoK flash §02 folds quantisation into dispatch, the grouped GEMM and
    SwiGLU.  Quantised here: each gathered token row along d (the dispatch),
    W1/W3 along d and W2 along I (blocks along the contraction axis of each
    GEMM), and H along I after SwiGLU (expert_ffn_mxfp8).  Routing and the
    weighted combine stay in high precision.  Every product of dequantised
    operands is exact in fp64 before summation.  ``expert_map(fn, jobs)``
    runs fn(*job) for each expert's job in order and yields the results (a
    process pool may stand in for the default loop).
    """
    from . import moe as M
    T = np.shape(x)[0]
    E = np.shape(w1)[0]
    if logits is None:
        logits = M.router_logits(x, wr, None)
    idx, gate = M.route(logits, k, score, renorm, bias)
    counts, offsets, perm, inv, src = M.layout(idx, E)
    xq = quantize_tokens(x)                          # per token along d
    xp = xq[src]
    I = np.shape(w1)[1]
    d = np.shape(w1)[2]
    R = perm.shape[0]
    A = np.zeros((R, I))
    B = np.zeros((R, I))
    H = np.zeros((R, I))
    Yp = np.zeros((R, d))
    live = [e for e in range(E) if offsets[e + 1] > offsets[e]]
    jobs = ((xp[offsets[e]:offsets[e + 1]], w1[e], w3[e], w2[e]) for e in live)
    for e, res in zip(live, (expert_map or _starmap)(expert_ffn_mxfp8, jobs)):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        A[lo:hi], B[lo:hi], H[lo:hi], Yp[lo:hi] = res
    y = M.combine(Yp, gate, inv, T, k)
    return dict(logits=logits, topk_idx=idx, gate=gate, counts=counts,
                offsets=offsets, perm=perm, inv=inv, src=src, A=A, B=B, H=H, Yp=Yp,
                y=y)


def expert_backward_mxfp8(x_rows, dy_rows, g_rows, A, B, H, w1_e, w3_e, w2_e, mx_wgrad=True,
                          saved_bf16=False):
    """One expert's part of backward_mxfp8 over its rows (the gathered x and
    dY rows, the rows' gates and the forward's A, B, H of those rows), in
    the steps of oracle.moe.backward: dHu = G W2 with G quantised along d
    per row and W2 as [I, d] (W2^T) along d; dgate = <dHu, H>; dW2 = (g G)^T
    H; dH = g dHu; the SwiGLU backward; dXp = dA W1 + dB W3 with dA, dB
    quantised along I per row and W1, W3 as [d, I] along I; dW1 = dA^T x,
    dW3 = dB^T x.  The three weight gradients contract over the expert's
    rows: with mx_wgrad their operands (g G, H, dA, dB, x) are quantised
    along the rows (wgrad_mxfp8), else taken unquantised.  With saved_bf16
    dA and dB are rounded to bfloat16 (round_bf16) before they are
    quantised, as the layer stores them between its GEMMs (A, B, H arrive
    rounded from backward_mxfp8).  Returns dict dw1, dw3, dw2, dxp, dgate
    (per row), dHu, dA, dB."""
    from . import moe as M
    xr = np.asarray(x_rows, dtype=np.float64)
    G = np.asarray(dy_rows, dtype=np.float64)
    g = np.asarray(g_rows, dtype=np.float64)
    w2t = fake_quant(np.asarray(w2_e, dtype=np.float64).T)          # [I, d] along d
    dHu = quantize_tokens(G) @ w2t.T
    dgate = np.sum(dHu * H, axis=1)
    wg = wgrad_mxfp8 if mx_wgrad else (lambda l, r: l.T @ r)
    dW2 = wg(g[:, None] * G, H)
    dH = g[:, None] * dHu
    sA = M.sigmoid(A)
    dA = dH * B * sA * (1.0 + A * (1.0 - sA))
    dB = dH * M.silu(A)
    if saved_bf16:
        dA, dB = round_bf16(dA), round_bf16(dB)
    w1t = fake_quant(np.asarray(w1_e, dtype=np.float64).T)          # [d, I] along I
    w3t = fake_quant(np.asarray(w3_e, dtype=np.float64).T)
    dXp = fake_quant(dA) @ w1t.T + fake_quant(dB) @ w3t.T
    return dict(dw1=wg(dA, xr), dw3=wg(dB, xr), dw2=dW2, dxp=dXp, dgate=dgate, dHu=dHu, dA=dA, dB=dB)


def backward_mxfp8(dy, x, fwd, w1, w3, w2, k, expert_map=None, mx_wgrad=True, saved_bf16=True):
    """The backward of the expert path (routing frozen) with its GEMMs in
    MXFP8.

    MoK flash §03 quotes the backward in MXFP8 but does not say which
    products are quantised.  Reading taken: every product of the expert
    backward runs in MXFP8, each operand quantised along that product's
    contraction axis.  The data gradients: dHu = G W2 with the upstream rows
    G along d and W2 as [I, d] (W2^T) along d; dXp = dA W1 + dB W3 with
    [dA | dB] along I and W1, W3 as [d, I] (W^T) along I.  The weight
    gradients contract over the expert's rows: dW2 = (g G)^T H, dW1 = dA^T
    x and dW3 = dB^T x with all five operands quantised along the rows, in
    blocks of 32 rows from the expert's first row (the last block filled
    with zeros); ``mx_wgrad=False`` keeps those three unquantised.  The
    steps are those of moe.backward, expert by expert (expert_backward_mxfp8,
    through ``expert_map`` as in forward_mxfp8); fwd holds the forward's
    gate, layout and A, B, H.

    Reading taken for the stored values: the layer keeps the activations its
    forward saves (A, B, H) and the SwiGLU gradients [dA | dB] it hands from
    one GEMM to the next in bfloat16, so those are the values the MXFP8
    quantisations see.  With ``saved_bf16`` (the default) A, B, H are
    rounded to bfloat16 on entry and dA, dB where they are formed
    (round_bf16); the upstream gradient and x arrive as bfloat16 already,
    and g G is a product formed without rounding.
    """
    dy = np.asarray(dy, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    T, d = dy.shape
    E, I, _ = np.shape(w1)
    offsets, perm, inv, src = fwd["offsets"], fwd["perm"], fwd["inv"], fwd["src"]
    gate = np.asarray(fwd["gate"], dtype=np.float64)
    A, B, H = fwd["A"], fwd["B"], fwd["H"]
    if saved_bf16:
        A, B, H = round_bf16(A), round_bf16(B), round_bf16(H)
    R = perm.shape[0]
    g_row = gate.reshape(-1)[perm]
    out = dict(dHu=np.zeros((R, I)), dA=np.zeros((R, I)), dB=np.zeros((R, I)), dXp=np.zeros((R, d)))
    dgate_row = np.zeros(R)
    dW1 = np.zeros((E, I, d))
    dW3 = np.zeros((E, I, d))
    dW2 = np.zeros((E, d, I))
    live = [e for e in range(E) if offsets[e + 1] > offsets[e]]

    def job(e):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        rows = src[lo:hi]
        return (x[rows], dy[rows], g_row[lo:hi], A[lo:hi], B[lo:hi], H[lo:hi], w1[e], w3[e], w2[e], mx_wgrad,
                saved_bf16)

    for e, b in zip(live, (expert_map or _starmap)(expert_backward_mxfp8, (job(e) for e in live))):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        dW1[e], dW3[e], dW2[e] = b["dw1"], b["dw3"], b["dw2"]
        dgate_row[lo:hi] = b["dgate"]
        out["dHu"][lo:hi], out["dA"][lo:hi], out["dB"][lo:hi], out["dXp"][lo:hi] = b["dHu"], b["dA"], b["dB"], b["dxp"]
    dx = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            dx[t] += out["dXp"][inv[t * k + j]]
    dgate = dgate_row[inv].reshape(T, k)
    return dict(dx=dx, dw1=dW1, dw3=dW3, dw2=dW2, dgate=dgate, **out)
