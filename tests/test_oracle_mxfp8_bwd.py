"""Pins of the MXFP8 backward oracle (oracle/mxfp8.py backward_mxfp8).

The data gradients quantise each operand along the contraction axis of its
product: dY rows and W2^T along d, [dA | dB] and W1^T, W3^T along I.  The
pins build inputs that MXFP8 represents exactly along those axes but not
along the other one (each test checks that the construction does tell the
axes apart), so backward_mxfp8 must equal the unquantised fp64 backward
(oracle/moe.py backward, the bf16 path's oracle) exactly; a transposed
quantisation, a dropped term or a wrong operand breaks the equality.  A
random case bounds the MXFP8 error against the same unquantised backward.
"""
import numpy as np

from oracle import moe as M
from oracle import mxfp8 as Q


def _problem(T, d, E, I, seed):
    """k = 1 routing (expert t % E), gates 1, and the layout."""
    idx = (np.arange(T) % E).reshape(T, 1)
    counts, offsets, perm, inv, src = M.layout(idx, E)
    return dict(gate=np.ones((T, 1)), offsets=offsets, perm=perm, inv=inv, src=src, counts=counts)


def _mixed(rng, shape, axis):
    """(1 + m/8) 2^-(j % 16) with j the index along `axis`, random signs:
    exact in MXFP8 along any other axis, inexact along `axis`."""
    m = rng.integers(0, 7, size=shape)
    j = np.arange(shape[axis]) % 16
    sh = [1] * len(shape)
    sh[axis] = shape[axis]
    v = (1.0 + m / 8.0) * np.exp2(-j.reshape(sh))
    return v * rng.choice([-1.0, 1.0], size=shape)


def _pow2(rng, shape):
    return rng.choice([-1.0, 1.0], size=shape) * np.exp2(rng.integers(0, 3, size=shape))


def _full(fwd, x, A, B, H):
    f = dict(fwd)
    f.update(A=A, B=B, H=H, xp=x[fwd["src"]])
    return f


def test_dxp_through_w1_exact_along_I():
    # A = 0, B = 2, g = 1: dA = dH = dHu, dB = 0; dY one-hot and W2 powers
    # of two make dHu rows of powers of two (exact along I)
    T, d, E, I = 24, 64, 3, 64
    rng = np.random.default_rng(1)
    fwd = _problem(T, d, E, I, 1)
    R = T
    dy = np.zeros((T, d))
    dy[np.arange(T), rng.integers(0, d, size=T)] = 1.0
    w2 = _pow2(rng, (E, d, I))
    w1 = _mixed(rng, (E, I, d), axis=2)      # W1[i, c]: exponent set by c -> W1^T exact along I
    w3 = rng.standard_normal((E, I, d))
    x = rng.standard_normal((T, d))
    H = rng.integers(-3, 4, size=(R, I)).astype(np.float64)
    f = _full(fwd, x, np.zeros((R, I)), np.full((R, I), 2.0), H)
    got = Q.backward_mxfp8(dy, x, f, w1, w3, w2, 1)
    want = M.backward(dy, f, w1, w3, w2, 1)
    assert not np.array_equal(Q.fake_quant(w1[0]), w1[0])   # along d it would not be exact
    assert np.array_equal(Q.fake_quant(w1[0].T), w1[0].T)
    for n in ("dx", "dw1", "dw3", "dw2", "dgate"):
        assert np.array_equal(got[n], want[n]), n
    assert np.count_nonzero(got["dx"]) > T


def test_dxp_through_w3_exact_along_I():
    # A = 40 (sigmoid 1.0 and silu 40.0 in fp64), B = 0: dA = 0, dB = 40 dHu,
    # 40 * 2^j = 1.25 * 2^(j+5) is exact in E4M3
    T, d, E, I = 24, 64, 3, 64
    rng = np.random.default_rng(2)
    fwd = _problem(T, d, E, I, 2)
    R = T
    dy = np.zeros((T, d))
    dy[np.arange(T), rng.integers(0, d, size=T)] = 1.0
    w2 = _pow2(rng, (E, d, I))
    w1 = rng.standard_normal((E, I, d))
    w3 = _mixed(rng, (E, I, d), axis=2)
    x = rng.standard_normal((T, d))
    H = rng.integers(-3, 4, size=(R, I)).astype(np.float64)
    f = _full(fwd, x, np.full((R, I), 40.0), np.zeros((R, I)), H)
    assert M.silu(np.array([40.0]))[0] == 40.0
    got = Q.backward_mxfp8(dy, x, f, w1, w3, w2, 1)
    want = M.backward(dy, f, w1, w3, w2, 1)
    assert not np.array_equal(Q.fake_quant(w3[0]), w3[0])
    for n in ("dx", "dw1", "dw3", "dw2", "dgate"):
        assert np.array_equal(got[n], want[n]), n
    assert np.count_nonzero(got["dx"]) > T


def test_dh_exact_along_d():
    # dY rows exact along d; W2 exact along d for every i but not along I
    # (the axis the forward quantises W2 along): dHu, dgate and dW2 exact
    T, d, E, I = 40, 64, 4, 64
    rng = np.random.default_rng(3)
    fwd = _problem(T, d, E, I, 3)
    R = T
    dy = _mixed(rng, (T, d), axis=0)
    w2 = _mixed(rng, (E, d, I), axis=2)
    w1 = rng.standard_normal((E, I, d))
    w3 = rng.standard_normal((E, I, d))
    x = rng.standard_normal((T, d))
    H = rng.integers(-3, 4, size=(R, I)).astype(np.float64)
    A = rng.standard_normal((R, I))
    B = rng.standard_normal((R, I))
    f = _full(fwd, x, A, B, H)
    got = Q.backward_mxfp8(dy, x, f, w1, w3, w2, 1)
    want = M.backward(dy, f, w1, w3, w2, 1)
    assert not np.array_equal(Q.fake_quant(w2[0]), w2[0])   # along I it would not be exact
    assert np.array_equal(got["dHu"], want["dHu"])
    for n in ("dgate", "dw2", "dw1", "dw3"):
        assert np.array_equal(got[n], want[n]), n


def test_random_case_within_mxfp8_error():
    # random Gaussian operands: each quantised operand carries at most 2^-4
    # relative error per element (3 mantissa bits) away from the subnormal
    # range, so the data gradients stay within a few percent of the
    # unquantised ones; the weight gradients only inherit dA, dB's error
    T, d, E, I, k = 64, 128, 4, 64, 2
    rng = np.random.default_rng(4)
    x = rng.standard_normal((T, d))
    logits = rng.standard_normal((T, E))
    w1 = rng.standard_normal((E, I, d)) / np.sqrt(d)
    w3 = rng.standard_normal((E, I, d)) / np.sqrt(d)
    w2 = rng.standard_normal((E, d, I)) / np.sqrt(I)
    dy = rng.standard_normal((T, d))
    fq = Q.forward_mxfp8(x, None, None, w1, w3, w2, k, M.SOFTMAX, True, logits=logits)
    f = dict(fq)
    f["xp"] = x[fq["src"]]
    got = Q.backward_mxfp8(dy, x, f, w1, w3, w2, k)
    want = M.backward(dy, f, w1, w3, w2, k)
    # two chained MXFP8 products: about 6% per dX row (median), 13% worst
    rel = np.linalg.norm(got["dx"] - want["dx"], axis=1) / np.linalg.norm(want["dx"], axis=1)
    assert 1e-3 < np.median(rel) < 0.1 and rel.max() < 0.2, (np.median(rel), rel.max())
    # dgate sums products of both signs: compare in norm over all tokens
    eg = np.linalg.norm(got["dgate"] - want["dgate"]) / np.linalg.norm(want["dgate"])
    assert 1e-3 < eg < 0.1, eg
    for n in ("dw1", "dw3", "dw2"):
        err = M.max_row_rel_err(got[n].reshape(E, -1), want[n].reshape(E, -1))
        assert err < 0.1, (n, err)
    assert np.array_equal(got["dw2"], want["dw2"])   # dW2 takes no quantised operand
