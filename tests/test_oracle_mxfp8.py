"""Pins of the oracle's MXFP8 codec (no GPU): the published format tables,
torch's float8 types, exhaustive round trips and the rounding error bound."""
import math
import os

import numpy as np
import pytest
import torch

from oracle import mxfp8 as Q

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_e8m0_ocp_mx_v1.txt")


def _golden():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        fmt, code, val = line.split()
        rows.append((fmt, int(code, 16), float(val)))
    return rows


def test_published_table_points():
    for fmt, code, val in _golden():
        got = Q.e4m3_value(code) if fmt == "e4m3" else float(Q.e8m0_value(code))
        if math.isnan(val):
            assert math.isnan(got), (fmt, code)
        else:
            assert got == val, (fmt, code, got, val)


def test_decode_all_256_codes_vs_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.uint8)
    want = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = Q.e4m3_table()
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])


def test_e8m0_decode_vs_torch():
    codes = torch.arange(255, dtype=torch.uint8)
    want = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(Q.e8m0_value(np.arange(255)), want)


def test_encode_vs_torch_cast_with_ties():
    vals = Q.e4m3_table()[:127]
    mids = (vals[:-1] + vals[1:]) / 2                      # exact ties
    rng = np.random.default_rng(0)
    rand = rng.uniform(-447.9, 447.9, 20000)
    tiny = rng.uniform(-0.02, 0.02, 5000)
    v = np.concatenate([vals, -vals, mids, -mids, rand, tiny, [17.0, 19.0, 0.0]])
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = Q.e4m3_encode(v)
    # torch keeps the sign of values that round to zero; the codec writes +0
    zero = (want & 0x7F) == 0
    assert np.array_equal(got[~zero], want[~zero])
    assert np.all(got[zero] == 0)
    assert Q.e4m3_encode(17.0) == 0x58 and Q.e4m3_value(0x58) == 16.0   # tie to even
    assert Q.e4m3_value(Q.e4m3_encode(19.0)) == 20.0


def test_arithmetic_encode_equals_table_search():
    vals = Q.e4m3_table()[:127]
    mids = (vals[:-1] + vals[1:]) / 2
    rng = np.random.default_rng(1)
    wide = rng.standard_normal(200000) * np.exp2(rng.integers(-14, 10, 200000))
    v = np.concatenate([vals, -vals, mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                        wide, [0.0, -0.0, 448.0, 449.0, 480.0, 1e30, 2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11]])
    assert np.array_equal(Q.e4m3_encode(v), Q.e4m3_encode_nearest(v))


def test_saturation():
    assert Q.e4m3_encode(1e6) == 0x7E and Q.e4m3_encode(-500.0) == 0xFE
    assert Q.e4m3_encode(464.0) == 0x7E


def test_round_trip_exhaustive():
    vals = Q.e4m3_table()
    ok = ~np.isnan(vals)
    codes = np.arange(256)[ok]
    back = Q.e4m3_encode(vals[ok])
    zero = vals[ok] == 0
    assert np.array_equal(back[~zero], codes[~zero])


def test_block_scale_rule_and_error_bound():
    rng = np.random.default_rng(1)
    v = rng.standard_normal((64, 256)) * np.exp2(rng.integers(-20, 20, (64, 1)))
    codes, sc = Q.quantize(v)
    blocks = v.reshape(64, 8, 32)
    amax = np.abs(blocks).max(axis=-1)
    assert np.array_equal(sc.astype(int) - 127, np.floor(np.log2(amax)).astype(int) - 8)
    scale = np.exp2(sc.astype(np.float64) - 127)[..., None]
    q = Q.e4m3_table()[codes.astype(int)].reshape(64, 8, 32)
    # every element is within half a spacing of its binade, or saturated
    y = blocks / scale
    err = np.abs(q - y)
    e = np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -6)))
    half_ulp = 0.5 * np.exp2(e - 3)
    sat = np.abs(y) > 448
    assert np.all(err[~sat] <= half_ulp[~sat])
    assert np.all(np.abs(q[sat]) == 448)
    assert np.all(np.abs(q) <= 448)


def test_zero_block_and_dequantize_shapes():
    v = np.zeros((3, 64))
    v[1, 40] = 3.0
    c, s = Q.quantize(v)
    assert s.shape == (3, 2) and s[0, 0] == 0 and s[1, 0] == 0 and s[1, 1] == 127 + 1 - 8
    assert np.all(c[0] == 0)
    assert np.array_equal(Q.dequantize(c, s), v)


def test_powers_of_two_quantize_exactly():
    v = np.exp2(np.arange(-30, 30, dtype=np.float64))[:32][None, :].repeat(2, 0)
    v[1] *= -1
    # a block spanning 2^-30..2^1: small members flush per the spec
    q = Q.fake_quant(v)
    big = np.abs(v) >= np.exp2(1 - 8 - 9)
    assert np.array_equal(q[big], v[big])


def _dense_quantised(x, w1, w3, w2, idx, gate):
    """Every expert on every token with MXFP8 operands, masked by the gates."""
    from oracle import moe as M
    xq = Q.fake_quant(x)
    T, E = x.shape[0], w1.shape[0]
    y = np.zeros((T, w2.shape[1]))
    for e in range(E):
        a = xq @ Q.fake_quant(w1[e]).T
        b = xq @ Q.fake_quant(w3[e]).T
        h = Q.fake_quant(M.silu(a) * b)
        ye = h @ Q.fake_quant(w2[e]).T
        m = np.zeros(T)
        for t in range(T):
            for j in range(idx.shape[1]):
                if idx[t, j] == e:
                    m[t] = gate[t, j]
        y += m[:, None] * ye
    return y


@pytest.mark.parametrize("seed", range(3))
def test_mxfp8_forward_matches_dense_quantised(seed):
    from mixture_experts_layer_layout_amd import synth
    w = synth.WORKLOADS["dsv3-mxfp8"].shrink(T=40, d=128, E=16, k=4, I=96)
    inp = synth.make_inputs(w, seed)
    t = {k: v.to(torch.float64).numpy() for k, v in inp.items() if v is not None}
    f = Q.forward_mxfp8(t["x"], t["wr"], None, t["w1"], t["w3"], t["w2"], w.k, w.score, True)
    want = _dense_quantised(t["x"], t["w1"], t["w3"], t["w2"], f["topk_idx"], f["gate"])
    assert np.max(np.abs(f["y"] - want)) <= 1e-12 * np.max(np.abs(want))
    # and MXFP8 stays close to the unquantised layer (a quality check)
    from oracle import moe as M
    ref = M.forward(t["x"], t["wr"], None, t["w1"], t["w3"], t["w2"], w.k, w.score, True)
    rel = np.max(np.abs(f["y"] - ref["y"])) / np.max(np.abs(ref["y"]))
    assert rel < 0.15
