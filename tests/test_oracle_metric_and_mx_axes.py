"""Pins of two oracle parts every GPU parity test leans on.

1. The comparison metric ``oracle.moe.max_row_rel_err``: per output row the
   max-norm error over the max norm of the expected row, rows whose expected
   max norm is zero skipped, the largest such ratio returned.  The expected
   values below are worked by hand from that definition (each case states
   its arithmetic); five plausible mistakes (min over rows, one global
   norm, the norm of the wrong operand, mean instead of max along a row,
   zero rows kept) are planted and each must fail at least one case.

2. The block axes of the MXFP8 forward (``oracle.mxfp8.forward_mxfp8`` and
   ``expert_ffn_mxfp8``; MoK flash §02: MXFP8 folded into the dispatch,
   grouped GEMM and SwiGLU).  The blocks run along each GEMM's contraction
   axis: x along d, W1/W3 along d, H along I, W2 along I.  The inputs are
   built so that MXFP8 holds them exactly along those axes but not along the
   other one (every test checks that its construction does tell the axes
   apart), so the quantised forward must equal the unquantised fp64 forward
   (``oracle.moe.forward``) bit for bit; quantising any operand along the
   other axis, or dropping H's quantisation, breaks the equality.
"""
import numpy as np
import pytest

from oracle import moe as M
from oracle import mxfp8 as Q


# ---------------------------------------------------------------- metric
# (got, want, expected value, the arithmetic)
_METRIC_CASES = [
    # row 0: max|diff| = max(0, 1) = 1, max|want| = 1 -> 1; row 1: 1 / 4
    # -> the max over rows is 1.0 (a min would give 0.25)
    ([[1.0, 2.0], [3.0, 4.0]], [[1.0, 1.0], [4.0, 4.0]], 1.0),
    # row 0 has an all-zero expected row: skipped; row 1: |1 - 0| / 2
    ([[7.0, 7.0], [2.0, 1.0]], [[0.0, 0.0], [2.0, 0.0]], 0.5),
    # a dominant row does not hide a small one: row 1 is 0.5 / 2 = 0.25
    # (one global norm would give 0.5 / 1000)
    ([[1000.0, 0.0], [1.5, -2.0]], [[1000.0, 0.0], [1.0, -2.0]], 0.25),
    # normalised by the expected row: |2 - 4| / 4 = 0.5 (by got: 1.0)
    ([[2.0]], [[4.0]], 0.5),
    # the max along the row, not the mean: 0.1 / 1 = 0.1 (mean: 0.025)
    ([[1.1, 1.0, 1.0, 1.0]], [[1.0, 1.0, 1.0, 1.0]], 0.1),
    # higher-rank inputs: rows are the first axis, the rest flattened;
    # row 0 = [1, 2, 3, 4] vs [1, 2, 3, 5] -> 1 / 5, row 1 = [8, 0, 0, 0]
    # vs [10, 0, 0, 0] -> 2 / 10
    ([[[1.0, 2.0], [3.0, 4.0]], [[8.0, 0.0], [0.0, 0.0]]],
     [[[1.0, 2.0], [3.0, 5.0]], [[10.0, 0.0], [0.0, 0.0]]], 0.2),
    # every expected row zero: the largest absolute difference
    ([[0.0, 3.0]], [[0.0, 0.0]], 3.0),
    # an exact match is 0
    ([[1.0, -2.0], [0.5, 0.25]], [[1.0, -2.0], [0.5, 0.25]], 0.0),
]


def metric_pins_hold(fn):
    for got, want, val in _METRIC_CASES:
        with np.errstate(divide="ignore", invalid="ignore"):
            r = fn(np.array(got), np.array(want))
        if not (np.isfinite(r) and abs(r - val) <= 1e-15 * max(1.0, abs(val))):
            return False
    return True


def test_max_row_rel_err_hand_computed():
    for got, want, val in _METRIC_CASES:
        assert M.max_row_rel_err(np.array(got), np.array(want)) == pytest.approx(val, rel=1e-15, abs=0)


def _metric_mutants():
    def _rows(got, want):
        got = np.asarray(got, np.float64).reshape(np.shape(want)[0], -1)
        want = np.asarray(want, np.float64).reshape(np.shape(want)[0], -1)
        return got, want

    def min_over_rows(got, want):
        got, want = _rows(got, want)
        num, den = np.max(np.abs(got - want), 1), np.max(np.abs(want), 1)
        ok = den > 0
        return float(np.min(num[ok] / den[ok])) if ok.any() else float(np.max(num))

    def global_norm(got, want):
        got, want = _rows(got, want)
        den = np.max(np.abs(want))
        return float(np.max(np.abs(got - want)) / den) if den > 0 else float(np.max(np.abs(got - want)))

    def norm_of_got(got, want):
        got, want = _rows(got, want)
        num, den = np.max(np.abs(got - want), 1), np.max(np.abs(got), 1)
        ok = np.max(np.abs(want), 1) > 0
        return float(np.max(num[ok] / den[ok])) if ok.any() else float(np.max(num))

    def mean_along_row(got, want):
        got, want = _rows(got, want)
        num, den = np.mean(np.abs(got - want), 1), np.max(np.abs(want), 1)
        ok = den > 0
        return float(np.max(num[ok] / den[ok])) if ok.any() else float(np.max(num))

    def zero_rows_kept(got, want):
        got, want = _rows(got, want)
        return float(np.max(np.max(np.abs(got - want), 1) / np.max(np.abs(want), 1)))

    return dict(min_over_rows=min_over_rows, global_norm=global_norm, norm_of_got=norm_of_got,
                mean_along_row=mean_along_row, zero_rows_kept=zero_rows_kept)


def test_metric_pins_pass_unmutated():
    assert metric_pins_hold(M.max_row_rel_err)


@pytest.mark.parametrize("name", sorted(_metric_mutants()))
def test_metric_mutant_is_caught(name):
    assert not metric_pins_hold(_metric_mutants()[name]), f"no case catches {name}"


# ---------------------------------------------------------------- MXFP8 axes
def _mixed(rng, shape, axis):
    """(1 + m/8) 2^-(j % 16), j the index along `axis`, random signs, with
    m = 1 wherever j % 16 == 15: a block of 32 along `axis` spans 15
    binades, so its smallest members fall below E4M3's normal range relative
    to the block scale and lose a bit -- inexact along `axis`; along any
    other axis a block shares one exponent and 3 mantissa bits -- exact."""
    m = rng.integers(0, 7, size=shape)
    j = np.arange(shape[axis]) % 16
    sh = [1] * len(shape)
    sh[axis] = shape[axis]
    jj = np.broadcast_to(j.reshape(sh), shape)
    m = np.where(jj == 15, 1, m)
    v = (1.0 + m / 8.0) * np.exp2(-jj)
    return v * rng.choice([-1.0, 1.0], size=shape)


def _exact_along_last(v):
    return np.array_equal(Q.fake_quant(v), v)


def _exact_along_rows(v):
    """v [n, K]: quantised in blocks of 32 down each column (n padded with
    zero rows to a multiple of 32; zeros change no block maximum)."""
    n = v.shape[0]
    pad = np.zeros(((-n) % 32, v.shape[1]))
    vt = np.concatenate([v, pad]).T
    return np.array_equal(Q.fake_quant(vt).T[:n], v)


def _logits(rng, T, E):
    return rng.standard_normal((T, E)).astype(np.float32).astype(np.float64)


def _case_gemm1(seed=11):
    """x exact along d (not T); W1, W3 exact along d (not I)."""
    rng = np.random.default_rng(seed)
    T, d, E, I, k = 64, 64, 4, 64, 2
    x = _mixed(rng, (T, d), axis=0)
    w1 = _mixed(rng, (E, I, d), axis=1)
    w3 = _mixed(rng, (E, I, d), axis=1)
    w2 = rng.standard_normal((E, d, I)) / 8.0
    return dict(x=x, w1=w1, w3=w3, w2=w2, k=k, logits=_logits(rng, T, E))


def _case_gemm2(seed=12):
    """x one-hot (value 1 in column t % d); W1 in {2^6, 2^21} by column parity
    (silu is then the identity in fp64: exp(-64) vanishes against 1), W3 of
    3 mantissa bits with exponents 0 or -1, so H = W1 * W3 is exact along I
    but spans 15 binades down a column (rows of even and odd token columns);
    W2 exact along I (not d)."""
    rng = np.random.default_rng(seed)
    T, d, E, I, k = 64, 64, 4, 64, 2
    x = np.zeros((T, d))
    x[np.arange(T), np.arange(T) % d] = 1.0
    w1 = np.broadcast_to(np.exp2(6.0 + 15.0 * (np.arange(d) % 2)), (E, I, d)).copy()
    m = rng.integers(0, 7, size=(E, I, d))
    m[..., 1::2] = rng.choice([1, 3, 5], size=(E, I, d // 2))   # odd mantissas where scaled by 2^21
    w3 = (1.0 + m / 8.0) * np.exp2(-(np.arange(I) % 2))[None, :, None] * rng.choice([-1.0, 1.0], size=(E, I, d))
    w2 = _mixed(rng, (E, d, I), axis=1)
    return dict(x=x, w1=w1, w3=w3, w2=w2, k=k, logits=_logits(rng, T, E))


def _case_h(seed=13):
    """Every operand exact along both axes (3 mantissa bits, one exponent);
    H = silu(A) B is then the only inexact value, and it is quantised along
    I: the MXFP8 down projection must equal that H, quantised in blocks of
    32 along each row, times W2."""
    rng = np.random.default_rng(seed)
    T, d, E, I, k = 64, 64, 4, 64, 2

    def small(shape, e):
        return (1.0 + rng.integers(0, 7, size=shape) / 8.0) * 2.0 ** e * rng.choice([-1.0, 1.0], size=shape)

    return dict(x=small((T, d), 0), w1=small((E, I, d), -3), w3=small((E, I, d), -3), w2=small((E, d, I), -3),
                k=k, logits=_logits(rng, T, E))


def _run(c):
    fm = Q.forward_mxfp8(c["x"], None, None, c["w1"], c["w3"], c["w2"], c["k"], M.SOFTMAX, True,
                         logits=c["logits"])
    fo = M.forward(c["x"], None, None, c["w1"], c["w3"], c["w2"], c["k"], M.SOFTMAX, True, logits=c["logits"])
    return fm, fo


def _constructions_discriminate():
    c1, c2, c3 = _case_gemm1(), _case_gemm2(), _case_h()
    ok = _exact_along_last(c1["x"]) and not _exact_along_rows(c1["x"])
    ok &= _exact_along_last(c1["w1"][0]) and not _exact_along_rows(c1["w1"][0])
    ok &= _exact_along_last(c1["w3"][1]) and not _exact_along_rows(c1["w3"][1])
    ok &= _exact_along_last(c2["w2"][0]) and not _exact_along_rows(c2["w2"][0])
    _, fo2 = _run(c2)
    lo, hi = int(fo2["offsets"][0]), int(fo2["offsets"][1])
    ok &= _exact_along_last(fo2["H"]) and not _exact_along_rows(fo2["H"][lo:hi])
    _, fo3 = _run(c3)
    ok &= not _exact_along_last(fo3["H"])
    lo, hi = int(fo3["offsets"][0]), int(fo3["offsets"][1])
    ok &= not np.array_equal(Q.fake_quant(fo3["H"][lo:hi]), _quant_rows(fo3["H"][lo:hi]))
    for c in (c3,):
        for n in ("x", "w1", "w3", "w2"):
            v = c[n].reshape(-1, c[n].shape[-1])
            ok &= _exact_along_last(v) and _exact_along_rows(v)
    return bool(ok)


def _quant_rows(v):
    n = v.shape[0]
    pad = np.zeros(((-n) % 32, v.shape[1]))
    return Q.fake_quant(np.concatenate([v, pad]).T).T[:n]


def mx_axis_pins_hold():
    """The three constructions; True when the oracle passes all of them."""
    fm, fo = _run(_case_gemm1())
    if not (np.array_equal(fm["A"], fo["A"]) and np.array_equal(fm["B"], fo["B"])):
        return False
    fm, fo = _run(_case_gemm2())
    if not (np.array_equal(fm["Yp"], fo["Yp"]) and np.array_equal(fm["y"], fo["y"])):
        return False
    c = _case_h()
    fm, fo = _run(c)
    Hq = Q.fake_quant(fo["H"])   # blocks of 32 along I within each row
    want = np.zeros_like(fo["Yp"])
    for e in range(c["w1"].shape[0]):
        lo, hi = int(fo["offsets"][e]), int(fo["offsets"][e + 1])
        want[lo:hi] = Hq[lo:hi] @ c["w2"][e].T
    return np.array_equal(fm["Yp"], want) and np.array_equal(fm["A"], fo["A"])


def test_mxfp8_constructions_tell_the_axes_apart():
    assert _constructions_discriminate()


def test_mxfp8_forward_block_axes():
    assert mx_axis_pins_hold()


def _mx_mutants():
    orig_ffn, orig_qt = Q.expert_ffn_mxfp8, Q.quantize_tokens

    def along_other(v):   # [n, K] quantised down the columns
        return _quant_rows(np.asarray(v, np.float64))

    def ffn(qw1, qw3, qw2, qh):
        def f(xq_rows, w1, w3, w2):
            w1q, w3q, w2q = qw1(w1), qw3(w3), qw2(w2)
            A = xq_rows @ w1q.T
            B = xq_rows @ w3q.T
            h = M.silu(A) * B
            return A, B, h, qh(h) @ w2q.T
        return f

    fq = Q.fake_quant
    ident = lambda v: np.asarray(v, np.float64)
    return {
        "w1_along_I": ("expert_ffn_mxfp8", ffn(along_other, fq, fq, fq)),
        "w3_along_I": ("expert_ffn_mxfp8", ffn(fq, along_other, fq, fq)),
        "w2_along_d": ("expert_ffn_mxfp8", ffn(fq, fq, along_other, fq)),
        "h_along_rows": ("expert_ffn_mxfp8", ffn(fq, fq, fq, along_other)),
        "h_not_quantised": ("expert_ffn_mxfp8", ffn(fq, fq, fq, ident)),
        "x_along_tokens": ("quantize_tokens", along_other),
        "unmutated_ffn_is_equivalent": ("expert_ffn_mxfp8", orig_ffn),
        "unmutated_qt_is_equivalent": ("quantize_tokens", orig_qt),
    }


@pytest.mark.parametrize("name", sorted(_mx_mutants()))
def test_mxfp8_axis_mutant_is_caught(name, monkeypatch):
    attr, fn = _mx_mutants()[name]
    monkeypatch.setattr(Q, attr, fn)
    if name.startswith("unmutated"):
        assert mx_axis_pins_hold()
    else:
        assert not mx_axis_pins_hold(), f"no construction catches {name}"
