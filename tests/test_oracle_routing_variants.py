"""Pins of the oracle's DeepSeek-V3-style routing options (no GPU):
selection-only bias, group-limited selection and a routed scaling factor.

Pins: group-limited selection against a brute force written from the
definition (explicit loops, repeated first maximum with ties to the lower
index) on keys with many ties; the special cases that reduce to plain top-k
(one group, or every group kept); a zero selection-only bias reproduces the
plain sigmoid route; with a selection-only bias the gates are the unbiased
scores' gates, and a large bias forces its expert in; the scaling factor
scales every gate; the scaled gate gradient against central differences.
Planted mistakes in each option are caught."""
import numpy as np
import pytest

from oracle import moe as M
from test_oracle_pins import brute_select


def brute_grouped(keys, k, n_group, topk_group):
    T, E = keys.shape
    gs = E // n_group
    out = []
    for t in range(T):
        gscore = []
        for g in range(n_group):
            vals = sorted((float(v) for v in keys[t, g * gs:(g + 1) * gs]), reverse=True)
            gscore.append(vals[0] + (vals[1] if gs > 1 else 0.0))
        kept = brute_select(gscore, topk_group)
        row = [float(keys[t, e]) if (e // gs) in kept else -np.inf for e in range(E)]
        out.append(brute_select(row, k))
    return np.array(out)


def pin_grouped(mod):
    rng = np.random.default_rng(7)
    bad = 0
    for E, n_group, topk_group, k in ((8, 2, 1, 2), (8, 4, 2, 3), (12, 3, 2, 5), (32, 8, 4, 8),
                                      (16, 16, 4, 4), (32, 4, 4, 6)):
        keys = np.round(rng.random((40, E)) * 6) / 6   # a coarse grid: many ties
        got = mod.select_grouped(keys, k, n_group, topk_group)
        bad += int(np.sum(np.any(got != brute_grouped(keys, k, n_group, topk_group), axis=1)))
    return bad


def test_grouped_selection_matches_brute_force_with_ties():
    assert pin_grouped(M) == 0


def test_grouping_special_cases_reduce_to_plain_topk():
    rng = np.random.default_rng(8)
    keys = rng.standard_normal((50, 16))
    assert np.array_equal(M.select_grouped(keys, 4, 1, 1), M.select_topk(keys, 4))
    assert np.array_equal(M.select_grouped(keys, 4, 4, 4), M.select_topk(keys, 4))


def pin_select_only(mod):
    """Largest deviation over: zero selection-only bias vs the plain sigmoid
    route; biased gates vs the unbiased gates of the chosen experts; a large
    bias forcing expert 5 in; the scaling factor."""
    rng = np.random.default_rng(9)
    lg = rng.standard_normal((60, 16)).astype(np.float32)
    worst = 0.0
    i0, g0 = mod.route(lg, 4, M.SIGMOID, True)
    i1, g1 = mod.route(lg, 4, M.SIGMOID, True, np.zeros(16, np.float32), select_only=True)
    worst = max(worst, float(np.any(i0 != i1)), float(np.max(np.abs(g0 - g1))))
    b = (rng.standard_normal(16) * 0.3).astype(np.float32)
    b[5] = 10.0
    i2, g2 = mod.route(lg, 4, M.SIGMOID, True, b, select_only=True, routed_scale=2.5)
    worst = max(worst, float(np.any(~np.any(i2 == 5, axis=1))))
    s = 1.0 / (1.0 + np.exp(-np.take_along_axis(lg.astype(np.float64), i2, axis=1)))
    worst = max(worst, float(np.max(np.abs(g2 - 2.5 * s / s.sum(axis=1, keepdims=True)))))
    keys = 1.0 / (1.0 + np.exp(-lg.astype(np.float64))) + b.astype(np.float64)[None, :]
    worst = max(worst, float(np.any(i2 != M.select_topk(keys, 4))))
    i3, g3 = mod.route(lg, 4, M.SOFTMAX, True, routed_scale=0.5)
    _, g4 = mod.route(lg, 4, M.SOFTMAX, True)
    worst = max(worst, float(np.max(np.abs(g3 - 0.5 * g4))))
    return worst


def test_selection_only_bias_and_scaling():
    assert pin_select_only(M) < 1e-12


def test_grouped_route_uses_score_space_keys():
    rng = np.random.default_rng(10)
    lg = rng.standard_normal((30, 32)).astype(np.float32)
    b = (rng.standard_normal(32) * 0.2).astype(np.float32)
    idx, _ = M.route(lg, 8, M.SIGMOID, True, b, select_only=True, n_group=8, topk_group=4)
    keys = 1.0 / (1.0 + np.exp(-lg.astype(np.float64))) + b.astype(np.float64)[None, :]
    assert np.array_equal(idx, brute_grouped(keys, 8, 8, 4))
    with pytest.raises(ValueError):
        M.route(lg, 8, M.SOFTMAX, True, b, select_only=True)


def pin_scaled_gradient(mod):
    rng = np.random.default_rng(11)
    worst = 0.0
    for score in (M.SOFTMAX, M.SIGMOID):
        z = rng.standard_normal((5, 9))
        idx = mod.select_topk(z, 3)
        dg = rng.standard_normal((5, 3))
        c = 2.5
        got = mod.gate_grad_to_logits(z, idx, dg, score, True, c)
        num = np.zeros_like(z)
        h = 1e-6
        for i in np.ndindex(z.shape):
            p = z.copy(); p[i] += h
            m = z.copy(); m[i] -= h
            num[i] = (np.sum(dg * c * mod.gates_from_logits(p, idx, score, True))
                      - np.sum(dg * c * mod.gates_from_logits(m, idx, score, True))) / (2 * h)
        worst = max(worst, float(np.max(np.abs(got - num)) / np.max(np.abs(num))))
    return worst


def test_scaled_gate_gradient_matches_finite_differences():
    assert pin_scaled_gradient(M) < 1e-8


def test_selection_only_bias_gets_no_gradient():
    rng = np.random.default_rng(12)
    x, wr = rng.standard_normal((6, 8)), rng.standard_normal((5, 8))
    z = x @ wr.T
    idx = M.select_topk(z, 2)
    r = M.router_backward(x, wr, z, idx, rng.standard_normal((6, 2)), M.SIGMOID, True, 2.5, True)
    assert np.all(r["dbias"] == 0.0)


# ---------------------------------------------------------------- mutations
def _mutants():
    orig_grouped, orig_route = M.select_grouped, M.route

    def grouped_top1(keys, k, n_group, topk_group):
        keys = np.asarray(keys)
        T, E = keys.shape
        gs = E // n_group
        gscore = keys.reshape(T, n_group, gs).max(axis=2)
        kept = np.argsort(-gscore, axis=1, kind="stable")[:, :topk_group]
        allowed = np.zeros((T, n_group), dtype=bool)
        np.put_along_axis(allowed, kept, True, axis=1)
        return M.select_topk(np.where(np.repeat(allowed, gs, axis=1), keys, -np.inf), k)

    def route_bias_ignored(logits, k, score, renorm, bias=None, select_only=False, **kw):
        return orig_route(logits, k, score, renorm, None if select_only else bias, select_only, **kw)

    def route_gates_biased(logits, k, score, renorm, bias=None, select_only=False, routed_scale=1.0, **kw):
        idx, _ = orig_route(logits, k, score, renorm, bias, select_only, routed_scale=routed_scale, **kw)
        z = np.asarray(logits) + (np.asarray(bias)[None, :] if bias is not None else 0)
        return idx, M.gates_from_logits(z, idx, score, renorm) * routed_scale

    def route_unscaled(logits, k, score, renorm, bias=None, select_only=False, routed_scale=1.0, **kw):
        return orig_route(logits, k, score, renorm, bias, select_only, **kw)

    return {"grouped_top1": ("select_grouped", grouped_top1),
            "select_only_bias_ignored": ("route", route_bias_ignored),
            "select_only_gates_biased": ("route", route_gates_biased),
            "scale_dropped": ("route", route_unscaled)}


def _any_pin_fails():
    return pin_grouped(M) != 0 or pin_select_only(M) > 1e-12 or pin_scaled_gradient(M) > 1e-8


def test_unmutated_routing_options_pass_every_pin():
    assert not _any_pin_fails()


@pytest.mark.parametrize("name", sorted(_mutants()))
def test_planted_routing_mistake_is_caught(name, monkeypatch):
    attr, fn = _mutants()[name]
    monkeypatch.setattr(M, attr, fn)
    assert _any_pin_fails(), f"no pin catches mutant {name}"
