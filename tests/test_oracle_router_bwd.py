"""Pins of the oracle's router backward (no GPU).

The router backward is the chain rule through the gate function with the
selection frozen.  Its pins are outside it: central finite differences of the
oracle's own forward gate function, the invariances of the normalised gates,
and a finite difference of the whole layer's loss <dy, y> with respect to the
router weight, the router bias and the input (which feeds both the experts and
the router).  Mutation tests plant plausible mistakes and check a pin fails.
"""
import numpy as np
import pytest

from oracle import moe as M

COMBOS = [(M.SOFTMAX, True), (M.SOFTMAX, False), (M.SIGMOID, True), (M.SIGMOID, False)]


def _fd(f, arr, h=1e-6):
    num = np.zeros_like(arr)
    it = np.nditer(arr, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        p = arr.copy(); p[i] += h
        m = arr.copy(); m[i] -= h
        num[i] = (f(p) - f(m)) / (2 * h)
    return num


def pin_gate_fd(mod):
    """max relative error of dL/dz against central differences of the
    forward gates, over the four score/normalisation combinations."""
    rng = np.random.default_rng(3)
    worst = 0.0
    for score, renorm in COMBOS:
        z = rng.standard_normal((5, 7))
        idx = mod.select_topk(z, 3)
        dg = rng.standard_normal((5, 3))
        got = mod.gate_grad_to_logits(z, idx, dg, score, renorm)
        num = _fd(lambda zz: float(np.sum(dg * mod.gates_from_logits(zz, idx, score, renorm))), z)
        worst = max(worst, np.max(np.abs(got - num)) / np.max(np.abs(num)))
    return worst


def test_gate_gradient_matches_finite_differences():
    assert pin_gate_fd(M) < 1e-8


def pin_invariances(mod):
    """Renormalised gates are unchanged by adding a constant to the chosen
    logits (softmax) or by scaling the chosen scores (sigmoid), so the
    gradient is orthogonal to those directions; unchosen logits get zero
    gradient whenever the gates read only the chosen logits."""
    rng = np.random.default_rng(4)
    worst = 0.0
    z = rng.standard_normal((50, 16)) * 2
    idx = M.select_topk(z, 4)
    dg = rng.standard_normal((50, 4))
    for score, renorm in ((M.SOFTMAX, True), (M.SIGMOID, True), (M.SIGMOID, False)):
        dz = mod.gate_grad_to_logits(z, idx, dg, score, renorm)
        sel = np.take_along_axis(dz, idx, axis=1)
        mask = np.ones_like(dz, dtype=bool)
        np.put_along_axis(mask, idx, False, axis=1)
        worst = max(worst, float(np.max(np.abs(dz[mask]))))
        if renorm and score == M.SOFTMAX:
            worst = max(worst, float(np.max(np.abs(sel.sum(axis=1)))))
        if renorm and score == M.SIGMOID:
            s = 1 / (1 + np.exp(-np.take_along_axis(z, idx, axis=1)))
            worst = max(worst, float(np.max(np.abs((sel / (1 - s)).sum(axis=1)))))
    return worst


def test_normalised_gate_gradient_invariances():
    assert pin_invariances(M) < 1e-13


def _layer(seed):
    rng = np.random.default_rng(seed)
    T, d, E, k, I = 6, 8, 5, 2, 6
    return dict(T=T, d=d, E=E, k=k, I=I,
                x=rng.standard_normal((T, d)), wr=rng.standard_normal((E, d)) * 0.5,
                bias=rng.standard_normal(E) * 0.3,
                w1=rng.standard_normal((E, I, d)) * 0.3, w3=rng.standard_normal((E, I, d)) * 0.3,
                w2=rng.standard_normal((E, d, I)) * 0.3, dy=rng.standard_normal((T, d)))


def pin_layer_fd(mod, score, renorm=True):
    """Whole-layer check: with the selection of the unperturbed forward
    frozen, d<dy, y>/d(wr, bias, x) by central differences against the
    router backward plus the expert path's backward."""
    L = _layer(11)
    k = L["k"]
    f = mod.forward(L["x"], L["wr"], L["bias"], L["w1"], L["w3"], L["w2"], k, score, renorm)
    b = mod.backward(L["dy"], f, L["w1"], L["w3"], L["w2"], k)
    z = f["logits"] + L["bias"][None, :]
    r = mod.router_backward(L["x"], L["wr"], z, f["topk_idx"], b["dgate"], score, renorm)
    idx = f["topk_idx"]

    def loss(x, wr, bias):
        # the reference forward, from the oracle's own pieces, routing frozen
        gate = mod.gates_from_logits(x @ wr.T + bias[None, :], idx, score, renorm)
        xp = mod.gather(x, f["src"])
        _, _, _, yp = mod.grouped_ffn(xp, f["offsets"], L["w1"], L["w3"], L["w2"])
        return float(np.sum(L["dy"] * mod.combine(yp, gate, f["inv"], L["T"], k)))

    worst = 0.0
    for name, grad in (("wr", r["dwr"]), ("bias", r["dbias"]), ("x", b["dx"] + r["dx"])):
        def f1(v, name=name):
            a = dict(x=L["x"], wr=L["wr"], bias=L["bias"])
            a[name] = v
            return loss(a["x"], a["wr"], a["bias"])
        num = _fd(f1, L[name])
        worst = max(worst, np.max(np.abs(num - grad)) / np.max(np.abs(num)))
    return worst


@pytest.mark.parametrize("score,renorm", COMBOS)
def test_layer_router_gradients_match_finite_differences(score, renorm):
    assert pin_layer_fd(M, score, renorm) < 1e-7


def test_router_backward_shapes_and_bias_sum():
    L = _layer(12)
    z = L["x"] @ L["wr"].T + L["bias"][None, :]
    idx = M.select_topk(z, L["k"])
    dg = np.random.default_rng(5).standard_normal((L["T"], L["k"]))
    r = M.router_backward(L["x"], L["wr"], z, idx, dg, M.SIGMOID, True)
    assert r["dlogits"].shape == (L["T"], L["E"])
    assert r["dwr"].shape == L["wr"].shape and r["dx"].shape == L["x"].shape
    assert np.allclose(r["dbias"], r["dlogits"].sum(axis=0), rtol=0, atol=1e-15)


# ---------------------------------------------------------------- mutations
def _mutants():
    orig = M.gate_grad_to_logits

    def no_centering(z, idx, dgate, score, renorm):
        # drops the - sum g dg term of the normalisation
        return orig(z, idx, dgate, score, False if score == M.SIGMOID else renorm) if score == M.SIGMOID \
            else _softmax_uncentred(z, idx, dgate, renorm)

    def _softmax_uncentred(z, idx, dgate, renorm):
        zs = np.take_along_axis(z, idx, axis=1)
        g = np.exp(zs - zs.max(axis=1, keepdims=True))
        g = g / g.sum(axis=1, keepdims=True)
        out = np.zeros_like(z)
        np.put_along_axis(out, idx, g * dgate, axis=1)
        return out

    def no_sigmoid_slope(z, idx, dgate, score, renorm):
        if score != M.SIGMOID:
            return orig(z, idx, dgate, score, renorm)
        s = 1 / (1 + np.exp(-np.take_along_axis(z, idx, axis=1)))
        S = s.sum(axis=1, keepdims=True) if renorm else 1.0
        g = s / S
        ds = (dgate - np.sum(g * dgate, axis=1, keepdims=True)) / S if renorm else dgate
        out = np.zeros_like(z)
        np.put_along_axis(out, idx, ds, axis=1)
        return out

    def slots_swapped(z, idx, dgate, score, renorm):
        return orig(z, idx, np.asarray(dgate)[:, ::-1], score, renorm)

    return {"no_centering": no_centering, "no_sigmoid_slope": no_sigmoid_slope,
            "slots_swapped": slots_swapped}


def _any_pin_fails():
    return (pin_gate_fd(M) > 1e-8 or pin_invariances(M) > 1e-13
            or any(pin_layer_fd(M, s, r) > 1e-7 for s, r in COMBOS))


def test_unmutated_router_backward_passes_every_pin():
    assert not _any_pin_fails()


@pytest.mark.parametrize("name", sorted(_mutants()))
def test_planted_router_mistake_is_caught(name, monkeypatch):
    monkeypatch.setattr(M, "gate_grad_to_logits", _mutants()[name])
    assert _any_pin_fails(), f"no pin catches mutant {name}"
