"""Pins of the MXFP8 backward oracle (oracle/mxfp8.py backward_mxfp8).

Each product quantises its operands along its own contraction axis: the
data gradients dY rows and W2^T along d, [dA | dB] and W1^T, W3^T along I;
the weight gradients g G, H, dA, dB and the x rows along the expert's rows
(the token axis), in blocks of 32 rows from the expert's first row.  The
pins build inputs that MXFP8 represents exactly along those axes but not
along the other one (each test checks that the construction does tell the
axes apart), so backward_mxfp8 must equal the unquantised fp64 backward
(oracle/moe.py backward, the bf16 path's oracle) exactly; a transposed
quantisation, a dropped term or a wrong operand breaks the equality.  The
data-gradient pins switch the weight-gradient quantisation off
(mx_wgrad=False), whose own pins follow them.  Hand-computed roundings pin
quantize_along_rows, including the zero fill of a last partial block; a
random case bounds the MXFP8 error against the unquantised backward, and
planted mistakes in the weight-gradient quantisation must be caught.  By
default backward_mxfp8 takes A, B, H and forms dA, dB in bfloat16, as the
layer stores them: round_bf16 is pinned by hand-computed ties and against
torch's float32 -> bfloat16 conversion, and a stored value that bfloat16
cannot hold must act as its rounded neighbour.
"""
import numpy as np
import pytest

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
    got = Q.backward_mxfp8(dy, x, f, w1, w3, w2, 1, mx_wgrad=False)
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
    got = Q.backward_mxfp8(dy, x, f, w1, w3, w2, 1, mx_wgrad=False)
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
    got = Q.backward_mxfp8(dy, x, f, w1, w3, w2, 1, mx_wgrad=False, saved_bf16=False)
    want = M.backward(dy, f, w1, w3, w2, 1)
    assert not np.array_equal(Q.fake_quant(w2[0]), w2[0])   # along I it would not be exact
    assert np.array_equal(got["dHu"], want["dHu"])
    for n in ("dgate", "dw2", "dw1", "dw3"):
        assert np.array_equal(got[n], want[n]), n


def test_random_case_within_mxfp8_error():
    # random Gaussian operands: each quantised operand carries at most 2^-4
    # relative error per element (3 mantissa bits) away from the subnormal
    # range, so every gradient stays within a few percent of the
    # unquantised one
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
    # the weight gradients chain up to three quantised operands (dA, dB
    # come out of the quantised data path): 5-11% of the matrix maximum here
    for n in ("dw1", "dw3", "dw2"):
        err = M.max_row_rel_err(got[n].reshape(E, -1), want[n].reshape(E, -1))
        assert 1e-3 < err < 0.2, (n, err)
    # with the weight gradients unquantised, dW2 takes no quantised operand
    # and dW1, dW3 only inherit dA, dB's error
    plain = Q.backward_mxfp8(dy, x, f, w1, w3, w2, k, mx_wgrad=False, saved_bf16=False)
    assert np.array_equal(plain["dw2"], want["dw2"])
    assert np.array_equal(plain["dx"], Q.backward_mxfp8(dy, x, f, w1, w3, w2, k, saved_bf16=False)["dx"])
    for n in ("dw1", "dw3"):
        assert 0 < M.max_row_rel_err(plain[n].reshape(E, -1), want[n].reshape(E, -1)) < 0.1


# ------------------------------------------------------------- weight gradients
def test_quantize_along_rows_hand_computed():
    # column 0: 1 and 1.0625 share a block with max 1.0625, scale 2^-8;
    # 1.0625 * 2^8 = 272 lies in E4M3's top binade (quantum 32): 272/32 =
    # 8.5 rounds to even, 8 -> 256 -> 1.0.  Row 32 is alone in the second
    # block (zero fill): 3.3 * 2^7 = 422.4 -> 13 quanta of 32 = 416 -> 3.25.
    v = np.zeros((33, 2))
    v[0, 0], v[1, 0], v[32, 0] = 1.0, 1.0625, 3.3
    v[:, 1] = 0.5   # a column of one value: exact
    q = Q.quantize_along_rows(v)
    assert q.shape == (33, 2)
    assert q[0, 0] == 1.0 and q[1, 0] == 1.0 and q[32, 0] == 3.25
    assert np.count_nonzero(q[2:32, 0]) == 0 and np.all(q[:, 1] == 0.5)
    # the same values along a row are one block with max 3.3 (scale 2^-7):
    # 1.0625 * 2^7 = 136 -> quantum 16, 8.5 -> 8 -> 128 -> 1.0, but 1.0
    # stays; quantising the transpose's rows is the column quantisation
    assert np.array_equal(Q.quantize_along_rows(v[:, :1]).ravel(), q[:, 0])


def test_quantize_along_rows_axis():
    rng = np.random.default_rng(5)
    v = _mixed(rng, (45, 64), axis=1)       # exponent set by the column
    assert np.array_equal(Q.quantize_along_rows(v), v)
    assert not np.array_equal(Q.fake_quant(v), v)
    w = _mixed(rng, (45, 64), axis=0)       # exponent set by the row
    assert not np.array_equal(Q.quantize_along_rows(w), w)


def _wgrad_case(A_val, B_val, seed):
    """k = 1 routing over 3 experts with 34, 33, 33 rows (partial last
    blocks); dY one-hot and W2 powers of two make dHu powers of two, so with
    A = 0, B = 2 dA = dHu (and dB = 0), with A = 40, B = 0 dB = 40 dHu (and
    dA = 0): exact along any axis.  H and x are exact along the rows but not
    along their feature axis."""
    T, d, E, I = 100, 64, 3, 64
    rng = np.random.default_rng(seed)
    fwd = _problem(T, d, E, I, seed)
    dy = np.zeros((T, d))
    dy[np.arange(T), rng.integers(0, d, size=T)] = 1.0
    w2 = _pow2(rng, (E, d, I))
    w1 = rng.standard_normal((E, I, d))
    w3 = rng.standard_normal((E, I, d))
    x = _mixed(rng, (T, d), axis=1)
    H = _mixed(rng, (T, I), axis=1)
    f = _full(fwd, x, np.full((T, I), A_val), np.full((T, I), B_val), H)
    assert not np.array_equal(Q.fake_quant(x), x) and not np.array_equal(Q.fake_quant(H), H)
    return dy, x, f, w1, w3, w2


def _hand_case():
    """One column of 33 rows: 0.001 in rows 0..31, 300 in row 32.  Blocks
    from the first row: 0.001 alone in its block has floor(log2) = -10,
    scale 2^-18, 0.001 * 2^18 = 262.1 -> 8 quanta of 32 -> 256 -> 2^-10;
    300 alone: scale 2^0, 300 -> 9 quanta of 32 = 288.  So q^T q = 32 *
    2^-20 + 288^2 exactly.  (Blocks aligned to the last row would put
    rows 1..32 with 300: 0.001 then rounds to the subnormal 2^-9.)"""
    v = np.full((33, 1), 0.001)
    v[32, 0] = 300.0
    return v, 32.0 * 2.0 ** -20 + 288.0 ** 2


def wgrad_pins_hold():
    """The weight-gradient pins as one predicate (for the mutants below)."""
    try:
        v, want_vv = _hand_case()
        if Q.wgrad_mxfp8(v, v)[0, 0] != want_vv:
            return False
        for A_val, B_val, seed, names in ((0.0, 2.0, 6, ("dw1", "dw2")), (40.0, 0.0, 7, ("dw3", "dw2"))):
            dy, x, f, w1, w3, w2 = _wgrad_case(A_val, B_val, seed)
            got = Q.backward_mxfp8(dy, x, f, w1, w3, w2, 1)
            want = M.backward(dy, f, w1, w3, w2, 1)
            for n in names:
                if not np.array_equal(got[n], want[n]) or np.count_nonzero(got[n]) == 0:
                    return False
    except ValueError:   # e.g. a quantisation along an axis that is not a multiple of 32
        return False
    # the operands are quantised at all: a random case moves every dW, by
    # less than 20% of the matrix maximum (32 rows per expert)
    T, d, E, I, k = 64, 64, 2, 64, 1
    rng = np.random.default_rng(8)
    fwd = _problem(T, d, E, I, 8)
    x, dy = rng.standard_normal((T, d)), rng.standard_normal((T, d))
    w1, w3, w2 = (rng.standard_normal((E, I, d)), rng.standard_normal((E, I, d)),
                  rng.standard_normal((E, d, I)))
    f = _full(fwd, x, rng.standard_normal((T, I)), rng.standard_normal((T, I)), rng.standard_normal((T, I)))
    got = Q.backward_mxfp8(dy, x, f, w1, w3, w2, k)
    plain = Q.backward_mxfp8(dy, x, f, w1, w3, w2, k, mx_wgrad=False)
    return all(not np.array_equal(got[n], plain[n])
               and M.max_row_rel_err(got[n].reshape(E, -1), plain[n].reshape(E, -1)) < 0.2
               for n in ("dw1", "dw3", "dw2"))


def test_weight_gradients_exact_along_tokens():
    assert wgrad_pins_hold()


def _wgrad_mutants():
    orig = Q.wgrad_mxfp8

    def along_features(l, r):      # each row quantised along its features
        return Q.fake_quant(np.asarray(l, np.float64)).T @ Q.fake_quant(np.asarray(r, np.float64))

    def lhs_only(l, r):
        return Q.quantize_along_rows(l).T @ np.asarray(r, np.float64)

    def rhs_only(l, r):
        return np.asarray(l, np.float64).T @ Q.quantize_along_rows(r)

    def blocks_from_the_end(l, r):  # blocks aligned to the last row instead
        q = lambda v: Q.quantize_along_rows(np.asarray(v, np.float64)[::-1])[::-1]
        return q(l).T @ q(r)

    def unquantised(l, r):
        return np.asarray(l, np.float64).T @ np.asarray(r, np.float64)

    return {"along_features": along_features, "lhs_only": lhs_only, "rhs_only": rhs_only,
            "blocks_from_the_end": blocks_from_the_end, "unquantised": unquantised,
            "unmutated_is_equivalent": orig}


@pytest.mark.parametrize("name", sorted(_wgrad_mutants()))
def test_weight_gradient_mutant_is_caught(name, monkeypatch):
    monkeypatch.setattr(Q, "wgrad_mxfp8", _wgrad_mutants()[name])
    if name.startswith("unmutated"):
        assert wgrad_pins_hold()
    else:
        assert not wgrad_pins_hold(), f"no pin catches {name}"


# ------------------------------------------------------------- bfloat16 storage
def test_round_bf16_hand_computed_and_against_torch():
    # bfloat16 keeps 8 significant bits: the spacing at 1 is 2^-7
    assert Q.round_bf16(1 + 2.0 ** -8) == 1.0                     # a tie: to the even significand
    assert Q.round_bf16(1 + 3 * 2.0 ** -8) == 1 + 2.0 ** -6        # a tie: to the even one above
    assert Q.round_bf16(1 + 2.0 ** -8 + 2.0 ** -20) == 1 + 2.0 ** -7
    assert Q.round_bf16(-3.0) == -3.0 and Q.round_bf16(0.0) == 0.0
    assert Q.round_bf16(255.5) == 256.0 and Q.round_bf16(254.5) == 254.0
    import torch
    rng = np.random.default_rng(9)
    v = (rng.standard_normal(4096) * np.exp2(rng.integers(-20, 20, 4096))).astype(np.float32).astype(np.float64)
    want = torch.tensor(v, dtype=torch.float32).to(torch.bfloat16).double().numpy()
    assert np.array_equal(Q.round_bf16(v), want)


def test_saved_activations_enter_as_bf16():
    # B = 1 + 2^-10 is stored as 1.0 (bfloat16): with the stored values the
    # backward equals the one given B = 1 exactly, without them it differs
    T, d, E, I = 64, 64, 2, 64
    rng = np.random.default_rng(10)
    fwd = _problem(T, d, E, I, 10)
    x, dy = rng.standard_normal((T, d)), rng.standard_normal((T, d))
    w1, w3, w2 = (rng.standard_normal((E, I, d)), rng.standard_normal((E, I, d)),
                  rng.standard_normal((E, d, I)))
    A, H = rng.standard_normal((T, I)), rng.standard_normal((T, I))
    A, H = Q.round_bf16(A), Q.round_bf16(H)
    f1 = _full(fwd, x, A, np.full((T, I), 1 + 2.0 ** -10), H)
    f0 = _full(fwd, x, A, np.ones((T, I)), H)
    a = Q.backward_mxfp8(dy, x, f1, w1, w3, w2, 1)
    b = Q.backward_mxfp8(dy, x, f0, w1, w3, w2, 1)
    c = Q.backward_mxfp8(dy, x, f1, w1, w3, w2, 1, saved_bf16=False)
    for n in ("dx", "dw1", "dw3", "dw2", "dgate"):
        assert np.array_equal(a[n], b[n]), n
    assert not np.array_equal(a["dw1"], c["dw1"])
    # and dA, dB are rounded where they are formed
    assert np.array_equal(a["dA"], Q.round_bf16(a["dA"])) and np.array_equal(a["dB"], Q.round_bf16(a["dB"]))

