"""Allocation helpers around the C ABI: device buffers for one layer call.

Only allocation and argument marshalling happen here; every step of the
layer runs in libmoe.so.
"""
from __future__ import annotations

import torch

from . import api

_ACT = {"f32": torch.float32, "bf16": torch.bfloat16}


def desc_for(w, fused=True, stage_rows=0, n_workgroups=0, flags=0, T=None, n_producer_cus=0):
    """moe_desc of a synth.Workload."""
    if w.select_only:
        flags |= api.MOE_FLAG_BIAS_SELECT_ONLY
    return api.make_desc(w.T if T is None else T, w.d, w.E, w.k, w.I, act=w.act,
                         experts=w.experts, score=w.score, renorm=w.renorm, fused=fused,
                         stage_rows=stage_rows, n_workgroups=n_workgroups, flags=flags,
                         n_group=w.n_group, topk_group=w.topk_group,
                         routed_scale=0.0 if w.routed_scale == 1.0 else w.routed_scale,
                         macro_tokens=w.macro_tokens, n_producer_cus=n_producer_cus)


def workspace(desc, device="cuda"):
    return torch.empty(api.moe_workspace_size(desc), dtype=torch.uint8, device=device)


def quantize_mxfp8(t: torch.Tensor):
    """E4M3 codes and E8M0 scales of a bf16 tensor along its last axis, by
    the library's quantise kernel."""
    K = t.shape[-1]
    codes = torch.empty(t.shape, dtype=torch.uint8, device=t.device)
    scales = torch.empty(t.shape[:-1] + (K // 32,), dtype=torch.uint8, device=t.device)
    api.moe_quantize_mxfp8(t.contiguous(), codes, scales)
    return codes, scales


def quantize_mxfp8_t(t: torch.Tensor):
    """E4M3 codes and E8M0 scales of the transpose of each matrix of t
    ([batch, rows, cols] -> [batch, cols, rows], blocks along rows), by the
    library's kernel."""
    t = t.contiguous()
    rows, cols = t.shape[-2], t.shape[-1]
    codes = torch.empty(t.shape[:-2] + (cols, rows), dtype=torch.uint8, device=t.device)
    scales = torch.empty(t.shape[:-2] + (cols, rows // 32), dtype=torch.uint8, device=t.device)
    api.moe_quantize_mxfp8_t(t, codes, scales)
    return codes, scales


def backward_weights_of(w, inp):
    """moe_weights for moe_backward: the bf16 weights, or for MXFP8 experts
    the transposed weights quantised along the data gradients' contraction
    axes (kept alive in the returned dict)."""
    if w.experts == "mxfp8":
        keep = {}
        for n in ("w1", "w3", "w2"):
            keep[n], keep[n + "_scale"] = quantize_mxfp8_t(inp[n])
        return api.make_weights(keep["w1"], keep["w3"], keep["w2"], keep["w1_scale"],
                                keep["w3_scale"], keep["w2_scale"]), keep
    return api.make_weights(inp["w1"], inp["w3"], inp["w2"]), {}


def weights_of(w, inp):
    """moe_weights for the workload (MXFP8 weights are quantised first and
    kept alive in the returned dict)."""
    if w.experts == "mxfp8":
        keep = {}
        for n in ("w1", "w3", "w2"):
            keep[n], keep[n + "_scale"] = quantize_mxfp8(inp[n])
        return api.make_weights(keep["w1"], keep["w3"], keep["w2"], keep["w1_scale"],
                                keep["w3_scale"], keep["w2_scale"]), keep
    return api.make_weights(inp["w1"], inp["w3"], inp["w2"]), {}


def alloc_saved(w, device="cuda", full=True, T=None):
    T = w.T if T is None else T
    R = T * w.k
    i32 = dict(dtype=torch.int32, device=device)
    f32 = dict(dtype=torch.float32, device=device)
    out = dict(
        logits=torch.empty((T, w.E), **f32),
        topk_idx=torch.empty((T, w.k), **i32),
        gate=torch.empty((T, w.k), **f32),
        counts=torch.empty((w.E,), **i32),
        offsets=torch.empty((w.E + 1,), **i32),
        perm=torch.empty((R,), **i32),
        inv=torch.empty((R,), **i32),
        status=torch.zeros((1,), **i32),
    )
    if w.macro_tokens and w.macro_tokens < T:
        # macrobatches: per-token outputs only (no layout over all T)
        for n in ("counts", "offsets", "perm", "inv"):
            del out[n]
        return out
    if full:
        act = _ACT[w.act]
        for n in ("a", "b", "h"):
            out[n] = torch.empty((R, w.I), dtype=act, device=device)
    return out


def forward(w, inp, fused=True, saved=None, ws=None, stage_rows=0, n_workgroups=0, flags=0,
            weights=None, n_producer_cus=0):
    """Runs moe_forward; returns (y, saved dict)."""
    dev = inp["x"].device
    d = desc_for(w, fused, stage_rows, n_workgroups, flags, T=inp["x"].shape[0], n_producer_cus=n_producer_cus)
    if weights is None:
        weights, keep = weights_of(w, inp)
    if saved is None:
        saved = alloc_saved(w, dev, T=inp["x"].shape[0])
    if ws is None:
        ws = workspace(d, dev)
    y = torch.empty(inp["x"].shape, dtype=_ACT[w.act], device=dev)
    api.moe_forward(d, inp["x"], inp["wr"], inp.get("bias"), weights, y,
                    api.make_saved(**saved), ws)
    return y, saved


def backward(w, inp, saved, fused=True, ws=None, flags=0, n_workgroups=0, weights=None):
    """Runs moe_backward; returns dict dx, dw1, dw3, dw2, dgate."""
    dev = inp["x"].device
    T = inp["x"].shape[0]
    d = desc_for(w, fused, 0, n_workgroups, flags, T=T)
    if weights is None:
        weights, keep = backward_weights_of(w, inp)
    if ws is None:
        ws = workspace(d, dev)
    act = _ACT[w.act]
    out = dict(dx=torch.empty((T, w.d), dtype=act, device=dev),
               dw1=torch.empty((w.E, w.I, w.d), dtype=act, device=dev),
               dw3=torch.empty((w.E, w.I, w.d), dtype=act, device=dev),
               dw2=torch.empty((w.E, w.d, w.I), dtype=act, device=dev),
               dgate=torch.empty((T, w.k), dtype=torch.float32, device=dev))
    api.moe_backward(d, inp["dy"], inp["x"], weights, api.make_saved(**saved), out["dx"],
                     out["dw1"], out["dw3"], out["dw2"], out["dgate"], ws)
    return out


def router_backward(w, inp, saved, dgate, dx, ws=None, dlogits=True):
    """Runs moe_router_backward: adds the router's part into dx (in place)
    and returns dict dwr, dbias (None without a bias) and dlogits (None when
    not asked for)."""
    dev = inp["x"].device
    T = inp["x"].shape[0]
    d = desc_for(w, True, T=T)
    if ws is None:
        ws = workspace(d, dev)
    out = dict(dwr=torch.empty((w.E, w.d), dtype=_ACT[w.act], device=dev),
               dbias=(torch.empty((w.E,), dtype=torch.float32, device=dev)
                      if inp.get("bias") is not None else None),
               dlogits=torch.empty((T, w.E), dtype=torch.float32, device=dev) if dlogits else None)
    api.moe_router_backward(d, inp["x"], inp["wr"], inp.get("bias"), api.make_saved(**saved), dgate,
                            out["dlogits"], out["dwr"], out["dbias"], dx, ws)
    return out
