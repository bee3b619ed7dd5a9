"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module draws random numbers and nothing else of the method: no routing,
no layout, no GEMM.  Both the HIP path and the CPU oracle receive the tensors
it returns.  Every tensor has its own generator, seeded from (seed, tensor
name, expert), so any one expert's weights can be redrawn on their own.

Workloads (sizes from the MoE shapes the method is measured on):
  tiny-fp32          T=64   d=128  E=8   k=2 I=256   fp32, softmax top-2 renorm
  mixtral-bf16       T=4096 d=4096 E=8   k=2 I=14336 bf16, softmax top-2 renorm
  dsv3-bf16          T=4096 d=7168 E=256 k=8 I=2048  bf16, sigmoid top-8 renorm
  dsv3-mxfp8         T=8192, otherwise as dsv3-bf16, expert GEMMs in MXFP8
  dsv3-fwdbwd-zipf   as dsv3-bf16 plus a router bias giving Zipf(1.2) expert
                     loads, and an upstream gradient dY for the backward
  dsv3-fwdbwd-zipf-mxfp8  the same with the expert GEMMs in MXFP8 (forward,
                     and the backward's data gradients)
  dsv3-ep8-share     one GPU's share of the DeepSeek-V3 layer split 8 ways by
                     expert: E=32 local experts, ~1024 rows each (a
                     matrix-core-bound shape; not one of the five parity
                     configurations)

Distributions: tiny-fp32 draws everything from N(0, 0.02^2).  The others draw
X ~ N(0,1), W1 and W3 ~ N(0, 1/d), W2 ~ N(0, 1/I) (fan-in scaling keeps every
intermediate O(1)), the router ~ N(0, 1/d) (Mixtral shape) or
U(-sqrt(3/d), sqrt(3/d)) (DeepSeek-V3 shapes, variance 1/d), dY ~ N(0,1);
all are drawn in fp32 and rounded to bf16 to nearest-even.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    E: int
    k: int
    I: int
    act: str = "bf16"          # X, Y, dY, dX element type: "f32" | "bf16"
    experts: str = "bf16"      # expert GEMM operands: "f32" | "bf16" | "mxfp8"
    score: str = "sigmoid"     # "softmax" | "sigmoid"
    renorm: bool = True
    x_std: float = 1.0
    wr_dist: str = "uniform"   # "normal" (std) | "uniform" (+-bound)
    wr_scale: float | None = None
    w1_std: float | None = None
    w2_std: float | None = None
    zipf_s: float | None = None
    backward: bool = False
    # DeepSeek-V3-style routing options (see moe_desc): selection-only
    # bias, group-limited selection, routed scaling factor
    select_only: bool = False
    n_group: int = 0
    topk_group: int = 0
    routed_scale: float = 1.0
    # forward in macrobatches of this many tokens (0: one call over all T)
    macro_tokens: int = 0

    @property
    def R(self):
        return self.T * self.k

    def shrink(self, **kw):
        """A smaller workload of the same kind (distribution scales follow
        the new d and I unless given)."""
        kw.setdefault("name", self.name + "-small")
        return dataclasses.replace(self, **kw)

    def scales(self):
        """(x_std, router scale, w1/w3 std, w2 std) with defaults applied."""
        d, I = self.d, self.I
        if self.wr_scale is not None:
            wr = self.wr_scale
        elif self.wr_dist == "uniform":
            wr = math.sqrt(3.0 / d)
        else:
            wr = 1.0 / math.sqrt(d)
        w1 = self.w1_std if self.w1_std is not None else 1.0 / math.sqrt(d)
        w2 = self.w2_std if self.w2_std is not None else 1.0 / math.sqrt(I)
        return self.x_std, wr, w1, w2


WORKLOADS = {
    "tiny-fp32": Workload("tiny-fp32", T=64, d=128, E=8, k=2, I=256,
                          act="f32", experts="f32", score="softmax",
                          renorm=True, x_std=0.02, wr_dist="normal",
                          wr_scale=0.02, w1_std=0.02, w2_std=0.02),
    "mixtral-bf16": Workload("mixtral-bf16", T=4096, d=4096, E=8, k=2,
                             I=14336, score="softmax", renorm=True,
                             wr_dist="normal"),
    "dsv3-bf16": Workload("dsv3-bf16", T=4096, d=7168, E=256, k=8, I=2048),
    "dsv3-mxfp8": Workload("dsv3-mxfp8", T=8192, d=7168, E=256, k=8, I=2048,
                           experts="mxfp8"),
    "dsv3-fwdbwd-zipf": Workload("dsv3-fwdbwd-zipf", T=4096, d=7168, E=256,
                                 k=8, I=2048, zipf_s=1.2, backward=True),
    "dsv3-fwdbwd-zipf-mxfp8": Workload("dsv3-fwdbwd-zipf-mxfp8", T=4096, d=7168, E=256,
                                       k=8, I=2048, zipf_s=1.2, backward=True,
                                       experts="mxfp8"),
    "dsv3-ep8-share": Workload("dsv3-ep8-share", T=4096, d=7168, E=32, k=8,
                               I=2048),
}

_TAGS = {"x": 1, "wr": 2, "w1": 3, "w3": 4, "w2": 5, "dy": 6, "zipf": 7,
         "extra": 8}


def _seed_for(seed, tag, index=0):
    ss = np.random.SeedSequence([int(seed), _TAGS[tag], int(index)])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def _gen(device, seed, tag, index=0):
    g = torch.Generator(device=device)
    g.manual_seed(_seed_for(seed, tag, index))
    return g


def _torch_dtype(kind):
    return torch.float32 if kind == "f32" else torch.bfloat16


def _normal(shape, std, g, device, dtype):
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return (v * std).to(dtype)


def _uniform(shape, bound, g, device, dtype):
    v = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    return ((v * 2.0 - 1.0) * bound).to(dtype)


def capped_zipf_targets(E, T, k, s):
    """Expected rows per expert rank for Zipf(s) loads with each expert
    capped at T rows (one row per token).  Water-filling: saturated ranks
    hold T, the rest share the remainder in Zipf proportion."""
    p = 1.0 / np.arange(1, E + 1, dtype=np.float64) ** s
    total = float(T * k)
    sat = np.zeros(E, dtype=bool)
    while True:
        free = ~sat
        rem = total - T * sat.sum()
        t = np.where(sat, float(T), rem * p / p[free].sum())
        over = free & (t > T)
        if not over.any():
            return t
        sat |= over


def zipf_router_bias(w: Workload, seed, iters=200):
    """Router bias that makes expert loads follow a capped Zipf(s).

    Calibrated on a stand-in for the router logits: i.i.d. normal values
    with the logits' expected spread (here 1: unit X times a router of
    variance 1/d).  Each round adds 0.3*(log target - log load) to every
    expert's bias.  Expert ranks are a seeded permutation of expert ids.
    Returns fp32 [E].
    """
    rng = np.random.Generator(np.random.PCG64(_seed_for(seed, "zipf")))
    E, T, k = w.E, w.T, w.k
    order = rng.permutation(E)
    target = np.empty(E)
    target[order] = capped_zipf_targets(E, T, k, w.zipf_s)
    x_std, wr, _, _ = w.scales()
    spread = x_std * math.sqrt(w.d) * (wr / math.sqrt(3.0) if
                                       w.wr_dist == "uniform" else wr)
    z = rng.standard_normal((T, E)) * spread
    b = np.zeros(E)
    for _ in range(iters):
        top = np.argpartition(-(z + b[None, :]), k - 1, axis=1)[:, :k]
        load = np.bincount(top.reshape(-1), minlength=E)
        b += 0.3 * spread * (np.log(target + 0.5) - np.log(load + 0.5))
    return b.astype(np.float32)


def make_inputs(w: Workload, seed: int = 0, device="cpu", experts=True,
                with_dy=None):
    """All inputs of one layer call as torch tensors on ``device``.

    x [T,d], wr [E,d], bias [E] fp32 or None, w1/w3 [E,I,d], w2 [E,d,I],
    dy [T,d] (when the workload has a backward, or ``with_dy``).
    ``experts=False`` skips the expert weights (routing-only tests).
    """
    dev = torch.device(device)
    act = _torch_dtype(w.act)
    wdt = torch.float32 if w.experts == "f32" else torch.bfloat16
    x_std, wr_s, w1_s, w2_s = w.scales()
    out = {}
    out["x"] = _normal((w.T, w.d), x_std, _gen(dev, seed, "x"), dev, act)
    g = _gen(dev, seed, "wr")
    if w.wr_dist == "uniform":
        out["wr"] = _uniform((w.E, w.d), wr_s, g, dev, act)
    else:
        out["wr"] = _normal((w.E, w.d), wr_s, g, dev, act)
    out["bias"] = (torch.from_numpy(zipf_router_bias(w, seed)).to(dev)
                   if w.zipf_s else None)
    if experts:
        w1 = torch.empty((w.E, w.I, w.d), dtype=wdt, device=dev)
        w3 = torch.empty((w.E, w.I, w.d), dtype=wdt, device=dev)
        w2 = torch.empty((w.E, w.d, w.I), dtype=wdt, device=dev)
        for e in range(w.E):
            w1[e], w3[e], w2[e] = expert_weights(w, seed, e, dev)
        out["w1"], out["w3"], out["w2"] = w1, w3, w2
    if with_dy or (with_dy is None and w.backward):
        out["dy"] = _normal((w.T, w.d), 1.0, _gen(dev, seed, "dy"), dev, act)
    return out


def expert_weights(w: Workload, seed: int, e: int, device="cpu"):
    """(w1[e], w3[e], w2[e]) exactly as ``make_inputs`` draws them, for one
    expert on its own."""
    dev = torch.device(device)
    wdt = torch.float32 if w.experts == "f32" else torch.bfloat16
    _, _, w1_s, w2_s = w.scales()
    return (_normal((w.I, w.d), w1_s, _gen(dev, seed, "w1", e), dev, wdt),
            _normal((w.I, w.d), w1_s, _gen(dev, seed, "w3", e), dev, wdt),
            _normal((w.d, w.I), w2_s, _gen(dev, seed, "w2", e), dev, wdt))


def random_logits(T, E, seed, device="cpu", ties=False):
    """fp32 router logits N(0,1) for routing-only tests.  With ``ties`` the
    values are drawn from a small integer grid so exact ties are common."""
    g = _gen(torch.device(device), seed, "extra", 1)
    if ties:
        v = torch.randint(-3, 4, (T, E), generator=g, device=device)
        return v.to(torch.float32) * 0.5
    return torch.randn((T, E), generator=g, device=device, dtype=torch.float32)


def random_topk(T, E, k, seed, device="cpu", skew=None):
    """Distinct expert ids per token, int32 [T, k], for layout-only tests.
    ``skew`` = "one" routes every token to experts 0..k-1; "zipf" draws
    from Zipf-like weights."""
    rng = np.random.Generator(np.random.PCG64(_seed_for(seed, "extra", 2)))
    if skew == "one":
        idx = np.tile(np.arange(k), (T, 1))
    else:
        if skew == "zipf":
            p = 1.0 / np.arange(1, E + 1) ** 1.2
            p = p[rng.permutation(E)]
            p /= p.sum()
        else:
            p = None
        idx = np.stack([rng.choice(E, size=k, replace=False, p=p)
                        for _ in range(T)]) if T else np.zeros((0, k))
    return torch.from_numpy(idx.astype(np.int32)).to(device)
