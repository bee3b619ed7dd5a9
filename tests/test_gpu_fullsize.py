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
import os

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
    """[E, rows, cols] weights on the GPU seen by the oracle as host arrays,
    one expert at a time (fp32 copies, exactly the bf16 values; the oracle
    computes in fp64), the last `keep` experts cached."""

    def __init__(self, t, keep=16):
        self.t = t
        self.shape = tuple(t.shape)
        self.keep = keep
        self.cache = {}

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            if len(self.cache) >= self.keep:
                self.cache.pop(next(iter(self.cache)))
            self.cache[e] = self.t[e].float().cpu().numpy()
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


def edge_tokens(offsets, perm, k, experts, BM=128):
    """Tokens of the rows at the edges of the given experts' row tiles: the
    first row, the last row of the first tile and the first of the second
    (a tile boundary), and the expert's last row (the ragged tail)."""
    out = []
    for e in experts:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        for r in (lo, lo + BM - 1, lo + BM, hi - 1):
            if lo <= r < hi:
                out.append(int(perm[r]) // k)
    return out


def pick_tokens(idx, E, required, n, seed):
    """`required` tokens plus others up to n, each next one chosen among
    random candidates to add the fewest experts not yet covered (so the
    oracle fetches fewer experts), at least n distinct tokens."""
    rng = np.random.default_rng(seed)
    chosen = list(dict.fromkeys(int(t) for t in required))
    have = np.zeros(E, bool)
    for t in chosen:
        have[idx[t]] = True
    T = idx.shape[0]
    while len(chosen) < n:
        cand = rng.choice(T, 64, replace=False)
        cand = [int(t) for t in cand if int(t) not in chosen]
        new = [int(np.count_nonzero(~have[idx[t]])) for t in cand]
        t = cand[int(np.argmin(new))]
        chosen.append(t)
        have[idx[t]] = True
    return np.array(sorted(chosen))


def expert_rows_backward(x, dy, idx, gate, ts, W1, W3, W2):
    """dX and dgate of tokens ts by the oracle's per-expert backward: each
    (token, slot) row of expert e goes through expert_backward with e's
    weights (fetched once per expert), and a token's dX sums its slots."""
    k = idx.shape[1]
    dx = np.zeros((len(ts), x.shape[1]))
    dg = np.zeros((len(ts), k))
    by_e = {}
    for i, t in enumerate(ts):
        for j in range(k):
            by_e.setdefault(int(idx[t, j]), []).append((i, j, int(t)))
    for e, rows in sorted(by_e.items()):
        tt = [t for _, _, t in rows]
        eb = M.expert_backward(x[tt], dy[tt], np.array([gate[t, j] for _, j, t in rows]), W1[e], W3[e], W2[e])
        for q, (i, j, _) in enumerate(rows):
            dx[i] += eb["dxp"][q]
            dg[i, j] = eb["dgate"][q]
    return dx, dg


def oracle_pool(n=8):
    """A process pool for the MXFP8 oracle's per-expert work (the codec costs
    about a second per expert matrix), started by spawn (the parent holds
    the GPU) with two BLAS threads per worker; and a map that feeds it n
    experts at a time, so at most n experts' weights are in flight."""
    import multiprocessing as mp
    import itertools
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS")}
    os.environ["OMP_NUM_THREADS"] = os.environ["OPENBLAS_NUM_THREADS"] = "2"
    try:
        pool = mp.get_context("spawn").Pool(n)
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v

    def expert_map(fn, jobs):
        jobs = iter(jobs)
        done = 0
        while True:
            batch = list(itertools.islice(jobs, n))
            if not batch:
                return
            yield from pool.starmap(fn, batch)
            done += len(batch)
            print(f"  oracle {fn.__name__}: {done} experts", flush=True)

    return pool, expert_map


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

    ts8 = sample_tokens(w.T, 8, 1)
    own = M.router_logits(x[ts8], wr)
    lt = logit_tolerance(x[ts8], wr)
    assert np.max(np.abs(own - logits[ts8]) / lt[:, None]) < 1.0

    # 32+ tokens: the edges of the heaviest, a median and the lightest
    # non-empty expert's row tiles, then tokens adding few new experts
    order = np.argsort(counts, kind="stable")
    nz = order[counts[order] > 0]
    edges = [int(nz[-1]), int(nz[len(nz) // 2]), int(nz[0])]
    ts = pick_tokens(idx, w.E, [0, w.T - 1] + edge_tokens(offsets, perm, w.k, edges), 32, 2)
    W1, W3, W2 = (DeviceExperts(dev[n]) for n in ("w1", "w3", "w2"))
    f = M.forward(x[ts], wr, bias, W1, W3, W2, w.k, w.score, w.renorm, logits=logits[ts])
    err = row_rel_err(host(y)[ts], f["y"])
    print(f"  y on {len(ts)} tokens max row-rel err {err:.2e}", flush=True)
    assert err <= BF16_TOL
    if not w.backward:
        return
    dy = host(inp["dy"])
    want_dx, want_dg = expert_rows_backward(x, dy, idx, gate, ts, W1, W3, W2)
    e1 = row_rel_err(host(g["dx"])[ts], want_dx)
    e2 = dgate_err(host(g["dgate"])[ts], want_dg)
    print(f"  dx on {len(ts)} tokens {e1:.2e}, dgate {e2:.2e}", flush=True)
    assert e1 <= BF16_TOL and e2 <= BF16_TOL
    # weight gradients of the lightest non-empty, a median and the heaviest
    # expert (the heaviest runs the longest streamed weight-gradient band)
    g_row = gate.reshape(-1)[perm]
    for e in edges[::-1]:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        rows = src[lo:hi]
        eb = M.expert_backward(x[rows], dy[rows], g_row[lo:hi], W1[e], W3[e], W2[e])
        for n in ("dw1", "dw3", "dw2"):
            e3 = row_rel_err(host(g[n][e]).reshape(1, -1), eb[n].reshape(1, -1))
            print(f"  {n}[{e}] ({hi - lo} rows) rel err {e3:.2e}", flush=True)
            assert e3 <= BF16_TOL, (n, e)


def test_fullsize_mxfp8():
    """dsv3-mxfp8 at full size: routing and layout over every token exact;
    y of 64 tokens against the oracle's MXFP8 forward, which quantises those
    tokens' experts' bf16 weights itself: the tokens of the row-tile edges
    (first row, a tile boundary, the ragged tail) of eight experts, the
    rest chosen to add few new experts."""
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
    order = np.argsort(counts, kind="stable")
    edges = [int(e) for e in order[np.linspace(0, w.E - 1, 8).astype(int)] if counts[e] > 0]
    ts = pick_tokens(idx, w.E, [w.T - 1] + edge_tokens(offsets, perm, w.k, edges), 64, 3)
    assert len(np.unique(idx[ts])) >= 32
    W1, W3, W2 = (DeviceExperts(dev[n]) for n in ("w1", "w3", "w2"))
    pool, emap = oracle_pool()
    try:
        f = Q.forward_mxfp8(x[ts], wr, bias, W1, W3, W2, w.k, w.score, w.renorm, logits=logits[ts],
                            expert_map=emap)
    finally:
        pool.terminate()
    err = row_rel_err(host(y)[ts], f["y"])
    print(f"  y on {len(ts)} tokens ({len(np.unique(idx[ts]))} experts) max row-rel err {err:.2e}", flush=True)
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


@pytest.mark.parametrize("mx_wgrad", [False, True])
def test_fullsize_mxfp8_backward(mx_wgrad):
    """dsv3-fwdbwd-zipf-mxfp8 at full size (MXFP8 forward, MXFP8 data
    gradients, bf16 weight gradients -- or MXFP8 ones with
    MOE_FLAG_MXFP8_WGRAD), as bench.py runs it: routing exact;
    dX and dgate of 16 tokens (tile-edge tokens of the heaviest expert
    included) against the oracle's MXFP8 forward and backward over those
    tokens alone (their rows depend on nothing else); dW1, dW3 and dW2 of a
    heavy expert (the third heaviest: a full streamed band) against the
    oracle's per-expert MXFP8 backward over exactly that expert's rows, given
    the oracle's MXFP8 A, B, H of those rows, rounded to bfloat16 as the
    layer saves them."""
    from oracle import mxfp8 as Q
    w = synth.WORKLOADS["dsv3-fwdbwd-zipf-mxfp8"]
    print(f"\nfull-size {w.name}: T={w.T} d={w.d} E={w.E} k={w.k} I={w.I}", flush=True)
    inp, dev = full_inputs(w, 0)
    y, sv = layer.forward(w, dev, fused=True)
    g = layer.backward(w, dev, sv, fused=True, flags=api.MOE_FLAG_MXFP8_WGRAD if mx_wgrad else 0)
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
    order = np.argsort(counts, kind="stable")
    heavy = int(order[-1])
    ts = pick_tokens(idx, w.E, [w.T // 3] + edge_tokens(offsets, perm, w.k, [heavy]), 16, 4)
    W1, W3, W2 = (DeviceExperts(dev[n]) for n in ("w1", "w3", "w2"))
    pool, emap = oracle_pool()
    try:
        f = Q.forward_mxfp8(x[ts], wr, bias, W1, W3, W2, w.k, w.score, w.renorm, logits=logits[ts],
                            expert_map=emap)
        b = Q.backward_mxfp8(dy[ts], x[ts], f, W1, W3, W2, w.k, expert_map=emap, mx_wgrad=mx_wgrad)
        for n in ("dx", "dgate"):
            e2 = (dgate_err if n == "dgate" else row_rel_err)(host(g[n])[ts], b[n])
            print(f"  {n} on {len(ts)} tokens max row-rel err {e2:.2e}", flush=True)
            assert e2 <= 6e-2, n
        e = int(order[-3])
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        rows = src[lo:hi]
        g_row = gate.reshape(-1)[perm][lo:hi]
        A, B, H, _ = Q.expert_ffn_mxfp8(Q.quantize_tokens(x[rows]), W1[e], W3[e], W2[e])
        A, B, H = Q.round_bf16(A), Q.round_bf16(B), Q.round_bf16(H)
        eb = Q.expert_backward_mxfp8(x[rows], dy[rows], g_row, A, B, H, W1[e], W3[e], W2[e], mx_wgrad=mx_wgrad,
                                     saved_bf16=True)
    finally:
        pool.terminate()
    for n in ("dw1", "dw3", "dw2"):
        e3 = row_rel_err(host(g[n][e]).reshape(1, -1), eb[n].reshape(1, -1))
        print(f"  {n}[{e}] ({hi - lo} rows) rel err {e3:.2e}", flush=True)
        assert e3 <= 6e-2, n
