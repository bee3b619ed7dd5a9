"""GPU runs at the full workload sizes, in the launch configuration bench.py
times (persistent kernels, default tiles and grid), checked against the fp64
oracle where the oracle can follow:

  * routing and layout over ALL tokens, bit-exact: the oracle selects on the
    fp32 logits the GPU exported (the same fp32 decision on both sides), and
    those logits agree with the oracle's own fp64 router GEMM to within fp32
    rounding on sampled tokens;
  * y (and dX, dgate) on sampled tokens: each token's output depends only on
    its own row, so the oracle forward/backward run on a subset of tokens
    gives those tokens' exact values;
  * dW1/dW3/dW2 of sampled experts from the oracle's per-expert backward
    over exactly that expert's rows;
  * the router backward over every token and expert, given the GPU's saved
    routing and dgate.
Expert weights are drawn on the device (as bench.py does); the oracle reads
the experts it needs back one at a time."""
import numpy as np
import pytest
import torch

from oracle import moe as M
from mixture_experts_layer_layout_amd import synth

pytestmark = pytest.mark.gpu

api = pytest.importorskip("mixture_experts_layer_layout_amd.api")
from mixture_experts_layer_layout_amd import layer  # noqa: E402
from parity import dgate_err, host, logit_tolerance, row_rel_err  # noqa: E402

BF16_TOL = 2e-2


class DeviceExperts:
    """[E, rows, cols] weights on the GPU seen by the oracle as fp64 host
    arrays, one expert at a time."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)
        self.cache = {}

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            self.cache[e] = self.t[e].float().cpu().numpy().astype(np.float64)
        return self.cache[e]


def full_inputs(w, seed):
    inp = synth.make_inputs(w, seed, device="cpu", experts=False, with_dy=w.backward)
    dev = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    wdt = torch.bfloat16
    dev["w1"] = torch.empty((w.E, w.I, w.d), dtype=wdt, device="cuda")
    dev["w3"] = torch.empty((w.E, w.I, w.d), dtype=wdt, device="cuda")
    dev["w2"] = torch.empty((w.E, w.d, w.I), dtype=wdt, device="cuda")
    for e in range(w.E):
        dev["w1"][e], dev["w3"][e], dev["w2"][e] = synth.expert_weights(w, seed, e, "cuda")
    return inp, dev


def sample_tokens(T, n, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, T - 1], rng.choice(T, n - 2, replace=False)]))


@pytest.mark.parametrize("name", ["mixtral-bf16", "dsv3-bf16", "dsv3-fwdbwd-zipf"])
def test_fullsize_bf16(name):
    w = synth.WORKLOADS[name]
    print(f"\nfull-size {name}: T={w.T} d={w.d} E={w.E} k={w.k} I={w.I}", flush=True)
    inp, dev = full_inputs(w, 0)
    y, sv = layer.forward(w, dev, fused=True)
    g = layer.backward(w, dev, sv, fused=True) if w.backward else None
    torch.cuda.synchronize()
    assert sv["status"].item() == 0

    x = host(inp["x"])
    wr = host(inp["wr"])
    bias = None if inp["bias"] is None else inp["bias"].numpy()
    logits = sv["logits"].cpu().numpy()
    # routing + layout over every token, bit-exact
    idx, gate = M.route(logits, w.k, w.score, w.renorm, bias)
    assert np.array_equal(host(sv["topk_idx"]), idx)
    assert np.max(np.abs(host(sv["gate"]) - gate)) < 2e-6
    counts, offsets, perm, inv, src = M.layout(idx, w.E)
    for n, want in (("counts", counts), ("offsets", offsets), ("perm", perm), ("inv", inv)):
        assert np.array_equal(host(sv[n]), want), n
    assert counts.sum() == w.R

    ts = sample_tokens(w.T, 8, 1)
    own = M.router_logits(x[ts], wr)
    lt = logit_tolerance(x[ts], wr)
    assert np.max(np.abs(own - logits[ts]) / lt[:, None]) < 1.0

    W1, W3, W2 = (DeviceExperts(dev[n]) for n in ("w1", "w3", "w2"))
    f = M.forward(x[ts], wr, bias, W1, W3, W2, w.k, w.score, w.renorm, logits=logits[ts])
    err = row_rel_err(host(y)[ts], f["y"])
    print(f"  y sampled max row-rel err {err:.2e}", flush=True)
    assert err <= BF16_TOL
    if not w.backward:
        return
    dy = host(inp["dy"])
    # dX and dgate of the sampled tokens: the oracle's per-expert backward
    # on each (token, slot) row, summed over the token's slots
    want = {"dx": np.zeros((len(ts), w.d)), "dgate": np.zeros((len(ts), w.k))}
    for i, t in enumerate(ts):
        for j in range(w.k):
            e = int(idx[t, j])
            eb = M.expert_backward(x[[t]], dy[[t]], gate[t, [j]], W1[e], W3[e], W2[e])
            want["dx"][i] += eb["dxp"][0]
            want["dgate"][i, j] = eb["dgate"][0]
    for n in ("dx", "dgate"):
        e2 = (dgate_err if n == "dgate" else row_rel_err)(host(g[n])[ts], want[n])
        print(f"  {n} sampled max row-rel err {e2:.2e}", flush=True)
        assert e2 <= BF16_TOL, n
    # weight gradients of the least-loaded expert and of a median one
    order = np.argsort(counts, kind="stable")
    g_row = gate.reshape(-1)[perm]
    for e in (int(order[0]), int(order[len(order) // 2])):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        rows = src[lo:hi]
        eb = M.expert_backward(x[rows], dy[rows], g_row[lo:hi], W1[e], W3[e], W2[e])
        for n in ("dw1", "dw3", "dw2"):
            e3 = row_rel_err(host(g[n][e]).reshape(1, -1), eb[n].reshape(1, -1))
            print(f"  {n}[{e}] ({hi - lo} rows) rel err {e3:.2e}", flush=True)
            assert e3 <= BF16_TOL, (n, e)


def test_fullsize_mxfp8():
    """dsv3-mxfp8 at full size: routing and layout over every token exact;
    y of a sampled token against the oracle's MXFP8 forward, which quantises
    that token's experts' bf16 weights itself."""
    from oracle import mxfp8 as Q
    w = synth.WORKLOADS["dsv3-mxfp8"]
    print(f"\nfull-size {w.name}: T={w.T} d={w.d} E={w.E} k={w.k} I={w.I}", flush=True)
    inp, dev = full_inputs(w, 0)
    y, sv = layer.forward(w, dev, fused=True)
    torch.cuda.synchronize()
    assert sv["status"].item() == 0
    x = host(inp["x"])
    wr = host(inp["wr"])
    bias = None if inp["bias"] is None else inp["bias"].numpy()
    logits = sv["logits"].cpu().numpy()
    idx, gate = M.route(logits, w.k, w.score, w.renorm, bias)
    assert np.array_equal(host(sv["topk_idx"]), idx)
    counts, offsets, perm, inv, src = M.layout(idx, w.E)
    for n, want in (("counts", counts), ("offsets", offsets), ("perm", perm), ("inv", inv)):
        assert np.array_equal(host(sv[n]), want), n
    ts = np.array([w.T - 1])
    W1, W3, W2 = (DeviceExperts(dev[n]) for n in ("w1", "w3", "w2"))
    f = Q.forward_mxfp8(x[ts], wr, bias, W1, W3, W2, w.k, w.score, w.renorm, logits=logits[ts])
    err = row_rel_err(host(y)[ts], f["y"])
    print(f"  y sampled max row-rel err {err:.2e}", flush=True)
    assert err <= 6e-2


def test_fullsize_router_backward():
    """moe_router_backward at the DeepSeek-V3 Zipf shape, fed the routing the
    GPU forward saved and the dgate its backward produced; the oracle takes
    the same routing and dgate.  dlogits and dbias over every token (fp32,
    1e-5 of the tensor max), dWr per expert row and dx per token row (bf16,
    1e-2), computed in full on the host."""
    w = synth.WORKLOADS["dsv3-fwdbwd-zipf"]
    print(f"\nfull-size router backward {w.name}: T={w.T} d={w.d} E={w.E} k={w.k}", flush=True)
    inp, dev = full_inputs(w, 0)
    _, sv = layer.forward(w, dev, fused=True)
    g = layer.backward(w, dev, sv, fused=True)
    dx_in = g["dx"].clone()
    r = layer.router_backward(w, dev, sv, g["dgate"], g["dx"])
    torch.cuda.synchronize()
    assert sv["status"].item() == 0
    x = host(inp["x"])
    wr = host(inp["wr"])
    z = host(sv["logits"]) + inp["bias"].numpy().astype(np.float64)[None, :]
    o = M.router_backward(x, wr, z, host(sv["topk_idx"]), host(g["dgate"]), w.score, w.renorm)
    rel = lambda a, b: float(np.max(np.abs(a - b)) / np.max(np.abs(b)))
    e1, e2 = rel(host(r["dlogits"]), o["dlogits"]), rel(host(r["dbias"]), o["dbias"])
    e3 = max(row_rel_err(host(r["dwr"])[e:e + 1], o["dwr"][e:e + 1]) for e in range(w.E))
    e4 = row_rel_err(host(g["dx"]), host(dx_in) + o["dx"])
    print(f"  dlogits {e1:.2e} dbias {e2:.2e} dwr {e3:.2e} dx {e4:.2e}", flush=True)
    assert e1 <= 1e-5 and e2 <= 1e-5
    assert e3 <= 1e-2 and e4 <= 1e-2


def test_fullsize_mxfp8_backward():
    """dsv3-fwdbwd-zipf-mxfp8 at full size (MXFP8 forward, MXFP8 data
    gradients, bf16 weight gradients), as bench.py runs it: routing exact;
    dX and dgate of one sampled token against the oracle's MXFP8 forward and
    backward over that token alone (its rows depend on nothing else); dW2 of
    the least-loaded expert, which takes no quantised operand, against the
    oracle's per-expert backward given the oracle's MXFP8 H."""
    from oracle import mxfp8 as Q
    w = synth.WORKLOADS["dsv3-fwdbwd-zipf-mxfp8"]
    print(f"\nfull-size {w.name}: T={w.T} d={w.d} E={w.E} k={w.k} I={w.I}", flush=True)
    inp, dev = full_inputs(w, 0)
    y, sv = layer.forward(w, dev, fused=True)
    g = layer.backward(w, dev, sv, fused=True)
    torch.cuda.synchronize()
    assert sv["status"].item() == 0
    x = host(inp["x"])
    wr = host(inp["wr"])
    dy = host(inp["dy"])
    bias = None if inp["bias"] is None else inp["bias"].numpy()
    logits = sv["logits"].cpu().numpy()
    idx, gate = M.route(logits, w.k, w.score, w.renorm, bias)
    assert np.array_equal(host(sv["topk_idx"]), idx)
    counts, offsets, perm, inv, src = M.layout(idx, w.E)
    assert np.array_equal(host(sv["perm"]), perm)
    W1, W3, W2 = (DeviceExperts(dev[n]) for n in ("w1", "w3", "w2"))
    ts = np.array([w.T // 3])
    f = Q.forward_mxfp8(x[ts], wr, bias, W1, W3, W2, w.k, w.score, w.renorm, logits=logits[ts])
    b = Q.backward_mxfp8(dy[ts], x[ts], f, W1, W3, W2, w.k)
    for n in ("dx", "dgate"):
        e2 = (dgate_err if n == "dgate" else row_rel_err)(host(g[n])[ts], b[n])
        print(f"  {n} sampled max row-rel err {e2:.2e}", flush=True)
        assert e2 <= 6e-2, n
    e = int(np.argsort(counts, kind="stable")[np.count_nonzero(counts == 0)])   # least-loaded with rows
    lo, hi = int(offsets[e]), int(offsets[e + 1])
    rows = src[lo:hi]
    # the oracle's MXFP8 H of expert e's rows (x quantised along d, W1/W3 along d)
    _, _, H_e, _ = Q.expert_ffn_mxfp8(Q.fake_quant(x[rows]), W1[e], W3[e], W2[e])
    g_row = gate.reshape(-1)[perm][lo:hi]
    dw2 = (g_row[:, None] * dy[rows]).T @ H_e
    e3 = row_rel_err(host(g["dw2"][e]).reshape(1, -1), dw2.reshape(1, -1))
    print(f"  dw2[{e}] ({hi - lo} rows) rel err {e3:.2e}", flush=True)
    assert e3 <= 6e-2
