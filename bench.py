#!/usr/bin/env python3
"""Throughput of one GPU's share of the fused MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--unfused] [--no-cpu-baseline] [--no-ablation]
    python bench.py --copy-calibration      # a plain copy of known size, for
                                            # scaling HBM byte counters

One step is one pass of the whole layer over one batch of seeded synthetic
input already resident in HBM: router, top-k and gates, per-expert counting
and layout, pull gather, SwiGLU grouped GEMMs, weighted combine, and (for a
workload with a backward) the backward of the expert path.  W untimed steps
run first; then exactly K steps are timed between two device
synchronisations.  Rank 0 prints one JSON line.

The line carries
  roofline      the dominant unit (the backward call when the step has
                one, else the forward call), timed with HIP events on the
                stream it runs on, against the roofline that bounds it: for
                a unit whose algorithmic intensity (expert FLOPs per
                algorithmic byte) is below the matrix cores' balance point
                the HBM peak (algorithmic bytes / duration), above it the
                dense matrix-core peak of the GEMMs' operand type (expert
                FLOPs / duration); ``traffic`` is the HBM byte count read
                from the committed counter summary when that summary was
                taken on the current kernel sources, else null
  cpu_baseline  the CPU oracle timed on the host cores over a bounded
                sample of the same workload (the rows of the first experts,
                routing and layout over all tokens), scaled to tokens/s
  phases        forward / backward times, the step timed again with a
                512 MB buffer written between steps (so no input of a step
                sits in the caches; ``step_ms_flushed``), the same step
                through the separate kernels (``unfused_step_ms``,
                ``fused_speedup``: the ablation of the persistent path), the
                standalone layout, gathers and merge, and for MXFP8 experts
                the weight quantisation a weight update costs (outside the
                step)
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
# dense matrix-core peaks, TFLOP/s, by the expert GEMMs' operand type
MFMA_PEAK_TFS = {"bf16": 2500.0, "mxfp8": 5000.0, "f32": 157.3}

DEFAULT_WORKLOAD = "dsv3-fwdbwd-zipf"
METRIC = "MoE layer tokens/s fwd+bwd on 1 MI355X; grouped-GEMM MFMA util %; gather GB/s"


def source_digest():
    """sha256 over the HIP sources and the C header: identifies the kernels a
    counter summary was taken on."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "mixture_experts_layer_layout_amd", "csrc", "*")))
    files.append(os.path.join(ROOT, "include", "moe.h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(kernel, workload):
    """HBM bytes per launch from profiles/<kernel>_<workload>_traffic.txt
    (lines 'key: value'), or None when missing or taken on other sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line:
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_digest():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------- workload
def algorithmic_bytes(w, counts, part):
    """Bytes a launch must move at minimum (each tensor touched once).

    forward : expert weights of the experts that received rows, X, router
              weight, Y, the saved activations a/b/h when kept for the
              backward, and the small routing/layout arrays
    backward: expert weights read + weight gradients written, dY, X, the
              saved a/b/h, dX, dgate, and the routing/layout arrays
    """
    es = 2 if w.act == "bf16" else 4
    # MXFP8 weights: one code byte per element plus one scale byte per 32
    wes = {"f32": 4.0, "bf16": 2.0, "mxfp8": 1.0 + 1.0 / 32}[w.experts]
    active = int((counts > 0).sum())
    wbytes = int(active * 3 * w.I * w.d * wes)
    tok = w.T * w.d * es
    small = w.R * 4 * 4 + (w.E + 1) * 8
    saved = 3 * w.R * w.I * es if w.backward else 0
    if part == "forward":
        return wbytes + 2 * tok + w.E * w.d * es + saved + w.T * w.E * 4 + small
    # the weight gradients are written in the activation type
    gbytes = int(active * 3 * w.I * w.d * es)
    return wbytes + gbytes + 3 * tok + saved + w.R * 4 + small


def expert_flops(w, part):
    f = 6.0 * w.d * w.I * w.R
    return f if part == "forward" else 2.0 * f


def cpu_baseline(w, inp_cpu, w_gpu, budget_s=15.0):
    """The oracle on the host cores over a bounded sample: routing and layout
    over all T tokens, then the expert path (forward, and backward when the
    workload has one) of experts 0, 1, ... until the budget is spent.
    Returns the result dict for the JSON line."""
    import numpy as np
    import threadpoolctl
    from oracle import moe as M

    f64 = lambda t: t.detach().cpu().double().numpy()
    t0 = time.perf_counter()
    x = f64(inp_cpu["x"])
    bias = None if inp_cpu["bias"] is None else inp_cpu["bias"].numpy()
    logits = M.router_logits(x, f64(inp_cpu["wr"]))
    idx, gate = M.route(logits, w.k, w.score, w.renorm, bias)
    counts, offsets, perm, inv, src = M.layout(idx, w.E)
    mx = w.experts == "mxfp8"
    if mx:
        from oracle import mxfp8 as Q
        x = Q.fake_quant(x)      # the dispatch's quantisation of every token
    t_route = time.perf_counter() - t0
    g_row = gate.reshape(-1)[perm]
    dy = f64(inp_cpu["dy"]) if w.backward else None
    rows_done, t_exp, n_exp = 0, 0.0, 0
    for e in range(w.E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        w1, w3, w2 = (f64(w_gpu[n][e]) for n in ("w1", "w3", "w2"))
        t1 = time.perf_counter()
        xr = M.gather(x, src[lo:hi])
        a, b, h, yp = (Q.expert_ffn_mxfp8 if mx else M.expert_ffn)(xr, w1, w3, w2)
        contrib = g_row[lo:hi, None] * yp          # this expert's share of the combine
        if w.backward:
            M.expert_backward(xr, M.gather(dy, src[lo:hi]), g_row[lo:hi], w1, w3, w2, saved=(a, b, h))
        t_exp += time.perf_counter() - t1
        del contrib, a, b, h, yp
        rows_done += hi - lo
        n_exp += 1
        if t_exp + t_route > budget_s:
            break
    frac = rows_done / w.R
    secs = t_exp + t_route * frac
    threads = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] or [1])
    return {"value": w.T * frac / secs, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": (f"fp64 numpy oracle: routing+layout{'+quantisation' if mx else ''} of all "
                       f"{'(backward data gradients unquantised) ' if mx and w.backward else ''}"
                       f"{w.T} tokens, expert "
                       f"{'forward+backward' if w.backward else 'forward'} of experts 0..{n_exp - 1} "
                       f"({rows_done} of {w.R} routed rows), scaled by rows")}


def copy_calibration():
    """A plain device copy of a known size, for scaling counter readings."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--unfused", action="store_true", help="one launch per step instead of the persistent kernel")
    ap.add_argument("--no-ablation", action="store_true",
                    help="skip timing the same step through the separate kernels")
    ap.add_argument("--stage-rows", type=int, default=0)
    ap.add_argument("--flags", type=lambda v: int(v, 0), default=0, help="moe_desc.flags (MOE_FLAG_*)")
    ap.add_argument("--workgroups", type=int, default=0, help="persistent grid size (0: automatic)")
    ap.add_argument("--producer-cus", type=int, default=0,
                    help="CU partition of the fused forward: CUs whose workgroups run only routing, "
                         "layout, gather and combine (0: none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--tokens", type=int, default=0, help="override the workload's T")
    ap.add_argument("--macro-tokens", type=int, default=0,
                    help="forward in macrobatches of this many tokens (forward-only workloads)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the layer on a single GPU; "
              "runs on more than one GPU are not supported", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import numpy as np
    import torch
    from mixture_experts_layer_layout_amd import api, layer, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    import dataclasses
    w = synth.WORKLOADS[args.workload]
    if args.tokens:
        w = dataclasses.replace(w, T=args.tokens)
    if args.macro_tokens:
        if w.backward:
            sys.exit("--macro-tokens: macrobatches are a forward-only mode")
        w = dataclasses.replace(w, macro_tokens=args.macro_tokens)
    t_gen = time.perf_counter()
    # x, router and bias on the host (shared with the CPU baseline), expert
    # weights and dY drawn on the device
    inp_cpu = synth.make_inputs(w, args.seed, device="cpu", experts=False, with_dy=w.backward)
    dev = {k: (v.cuda() if v is not None else None) for k, v in inp_cpu.items()}
    wdt = torch.float32 if w.experts == "f32" else torch.bfloat16
    dev["w1"] = torch.empty((w.E, w.I, w.d), dtype=wdt, device="cuda")
    dev["w3"] = torch.empty((w.E, w.I, w.d), dtype=wdt, device="cuda")
    dev["w2"] = torch.empty((w.E, w.d, w.I), dtype=wdt, device="cuda")
    for e in range(w.E):
        dev["w1"][e], dev["w3"][e], dev["w2"][e] = synth.expert_weights(w, args.seed, e, "cuda")
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen

    fused = not args.unfused
    weights, keep = layer.weights_of(w, dev)
    # the backward's weights (MXFP8: transposed, quantised along its
    # contraction axes, once per weight update and outside the step)
    bweights, bkeep = layer.backward_weights_of(w, dev) if w.backward else (None, {})
    saved = layer.alloc_saved(w, "cuda", full=w.backward)
    desc = layer.desc_for(w, fused=fused, stage_rows=args.stage_rows, flags=args.flags,
                          n_workgroups=args.workgroups, n_producer_cus=args.producer_cus)
    ws = layer.workspace(desc)
    y = torch.empty((w.T, w.d), dtype=torch.bfloat16 if w.act == "bf16" else torch.float32, device="cuda")
    if w.backward:
        bdesc = layer.desc_for(w, fused=fused, flags=args.flags, n_workgroups=args.workgroups)
        bws = layer.workspace(bdesc)
        act = y.dtype
        grads = dict(dx=torch.empty((w.T, w.d), dtype=act, device="cuda"),
                     dw1=torch.empty((w.E, w.I, w.d), dtype=act, device="cuda"),
                     dw3=torch.empty((w.E, w.I, w.d), dtype=act, device="cuda"),
                     dw2=torch.empty((w.E, w.d, w.I), dtype=act, device="cuda"),
                     dgate=torch.empty((w.T, w.k), dtype=torch.float32, device="cuda"))
    sv = api.make_saved(**saved)
    stream = torch.cuda.current_stream()

    def fwd():
        api.moe_forward(desc, dev["x"], dev["wr"], dev["bias"], weights, y, sv, ws, stream)

    def bwd():
        api.moe_backward(bdesc, dev["dy"], dev["x"], bweights, sv, grads["dx"], grads["dw1"],
                         grads["dw3"], grads["dw2"], grads["dgate"], bws, stream)

    ev = lambda: torch.cuda.Event(enable_timing=True)
    for _ in range(args.warmup):
        fwd()
        if w.backward:
            bwd()
    torch.cuda.synchronize()
    if saved["status"].item() != 0:
        raise RuntimeError("device status " + api.moe_status_string(saved["status"].item()))

    marks = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        e0, e1, e2 = ev(), ev(), ev()
        e0.record(stream)
        fwd()
        e1.record(stream)
        if w.backward:
            bwd()
        e2.record(stream)
        marks.append((e0, e1, e2))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    if saved["status"].item() != 0:
        raise RuntimeError("device status " + api.moe_status_string(saved["status"].item()))

    # the step again with a 512 MB buffer written before each step (outside
    # the events), so no input of the step is left in the L2s or the MALL
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    fl_ms = []
    for _ in range(min(args.steps, 5)):
        flush.zero_()
        a, b = ev(), ev()
        a.record(stream)
        fwd()
        if w.backward:
            bwd()
        b.record(stream)
        torch.cuda.synchronize()
        fl_ms.append(a.elapsed_time(b))
    del flush
    # ablation: the same step through the separate kernels (fused = 0: one
    # ordinary grid per phase, the stream ordering them), on the same
    # buffers, timed with events around a few steps
    unfused_ms = None
    if fused and not args.no_ablation:
        udesc = layer.desc_for(w, fused=False, stage_rows=args.stage_rows, flags=args.flags)
        ubdesc = layer.desc_for(w, fused=False, flags=args.flags) if w.backward else None

        def ustep():
            api.moe_forward(udesc, dev["x"], dev["wr"], dev["bias"], weights, y, sv, ws, stream)
            if w.backward:
                api.moe_backward(ubdesc, dev["dy"], dev["x"], bweights, sv, grads["dx"], grads["dw1"],
                                 grads["dw3"], grads["dw2"], grads["dgate"], bws, stream)
        ustep()
        a, b = ev(), ev()
        n_u = min(args.steps, 5)
        a.record(stream)
        for _ in range(n_u):
            ustep()
        b.record(stream)
        torch.cuda.synchronize()
        unfused_ms = a.elapsed_time(b) / n_u
        if saved["status"].item() != 0:
            raise RuntimeError("device status " + api.moe_status_string(saved["status"].item()))
    # MXFP8 experts: the weight quantisation one weight update costs (the
    # forward's three weights along their contraction axes, and for a
    # backward the three transposed ones), timed on the same stream
    quant_ms = None
    if w.experts == "mxfp8":
        a, b = ev(), ev()
        a.record(stream)
        layer.weights_of(w, dev)
        if w.backward:
            layer.backward_weights_of(w, dev)
        b.record(stream)
        torch.cuda.synchronize()
        quant_ms = a.elapsed_time(b)

    # the standalone layout and gather (moe_layout, moe_gather: token-major
    # by inv, and the pull by perm) on this step's routing, timed with events
    # on the same stream
    side = {}
    if w.experts != "f32" and "perm" in saved:
        gdesc = layer.desc_for(w, fused=False)
        xq_ = torch.empty((w.R, w.d), dtype=torch.uint8 if w.experts == "mxfp8" else torch.bfloat16,
                          device="cuda")
        xs_ = torch.empty((w.R, w.d // 32), dtype=torch.uint8, device="cuda") if w.experts == "mxfp8" else None
        lay = {n: torch.empty_like(saved[n]) for n in ("counts", "offsets", "perm", "inv")}
        lws = layer.workspace(gdesc)
        # the combine alone (moe_combine, the forward's own merge kernel) on
        # this step's gates and layout, over an expert-output buffer
        yp_ = torch.zeros((w.R, w.d), dtype=torch.bfloat16, device="cuda")
        yc_ = torch.empty((w.T, w.d), dtype=torch.bfloat16, device="cuda")
        reps = 20
        for name, fn in (("layout", lambda: api.moe_layout(gdesc, saved["topk_idx"], lay["counts"], lay["offsets"],
                                                           lay["perm"], lay["inv"], None, lws, stream)),
                         ("gather", lambda: api.moe_gather(gdesc, dev["x"], None, xq_, xs_, stream,
                                                           inv=saved["inv"])),
                         ("gather_pull", lambda: api.moe_gather(gdesc, dev["x"], saved["perm"], xq_, xs_,
                                                                stream)),
                         ("combine", lambda: api.moe_combine(gdesc, yp_, saved["gate"], saved["inv"], yc_,
                                                             stream))):
            fn()
            a, b = ev(), ev()
            a.record(stream)
            for _ in range(reps):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            side[name] = a.elapsed_time(b) / reps
        del xq_, xs_, lay, lws, yp_, yc_
    if w.backward and not (w.score == "softmax" and not w.renorm):
        # the router backward (moe_router_backward) after the step's
        # backward, timed apart: it is not part of the measured step
        rdesc = layer.desc_for(w, fused=fused)
        rws = layer.workspace(rdesc)
        rout = dict(dwr=torch.empty((w.E, w.d), dtype=y.dtype, device="cuda"),
                    dbias=torch.empty((w.E,), dtype=torch.float32, device="cuda"),
                    dlogits=torch.empty((w.T, w.E), dtype=torch.float32, device="cuda"))
        dx_r = grads["dx"].clone()
        rfn = lambda: api.moe_router_backward(rdesc, dev["x"], dev["wr"], dev["bias"], sv, grads["dgate"],
                                              rout["dlogits"], rout["dwr"],
                                              rout["dbias"] if dev["bias"] is not None else None, dx_r, rws,
                                              stream)
        rfn()
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(10):
            rfn()
        b.record(stream)
        torch.cuda.synchronize()
        side["router_backward"] = a.elapsed_time(b) / 10
        del rws, rout, dx_r
    fwd_ms = sum(a.elapsed_time(b) for a, b, _ in marks) / args.steps
    bwd_ms = sum(b.elapsed_time(c) for _, b, c in marks) / args.steps if w.backward else 0.0
    ms_step = elapsed * 1e3 / args.steps
    counts = saved["counts"].cpu().numpy() if "counts" in saved else None
    if counts is None:
        # macrobatches: the per-expert loads from the saved routing
        counts = np.bincount(saved["topk_idx"].cpu().numpy().reshape(-1), minlength=w.E)

    part = "backward" if w.backward else "forward"
    kern_ms = bwd_ms if w.backward else fwd_ms
    kname = ("k_fused_bwd" if w.backward else "k_fused_fwd") if fused else ("moe_backward" if w.backward else "moe_forward")
    abytes = algorithmic_bytes(w, counts, part)
    aflops = expert_flops(w, part)
    mfma_peak = MFMA_PEAK_TFS[w.experts]
    # the roofline that bounds the unit: matrix cores when its intensity
    # exceeds their balance point (peak FLOP/s over peak bytes/s)
    if aflops / abytes > mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9):
        achieved = aflops / (kern_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": mfma_peak, "unit": "TFLOP/s",
                "frac": round(achieved / mfma_peak, 4)}
    else:
        achieved = abytes / (kern_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roof.update({"traffic": read_traffic(kname, w.name), "kernel": kname, "algorithmic_bytes": abytes,
                 "algorithmic_flops": aflops, "avg_ms": round(kern_ms, 4)})
    phases = {"forward_ms": round(fwd_ms, 4), "backward_ms": round(bwd_ms, 4),
              "forward_expert_tflops": round(expert_flops(w, "forward") / (fwd_ms * 1e-3) / 1e12, 1),
              "forward_mfma_util": round(expert_flops(w, "forward") / (fwd_ms * 1e-3) / 1e12
                                         / MFMA_PEAK_TFS[w.experts], 4),
              "forward_hbm_frac": round(algorithmic_bytes(w, counts, "forward") / (fwd_ms * 1e-3) / 1e9
                                        / HBM_PEAK_GBS, 4),
              "workspace_mb": round(ws.numel() / 1e6, 1)}
    phases["step_ms_flushed"] = round(sum(fl_ms) / len(fl_ms), 4)
    if unfused_ms is not None:
        phases["unfused_step_ms"] = round(unfused_ms, 4)
        phases["fused_speedup"] = round(unfused_ms / ms_step, 3)
    if quant_ms is not None:
        phases["weight_quant_ms_per_update"] = round(quant_ms, 4)
        phases["tokens_s_with_quant_every_step"] = round(w.T / ((ms_step + quant_ms) * 1e-3), 1)
    phases["max_rows_per_expert"] = int(counts.max())
    phases["min_rows_per_expert"] = int(counts.min())
    if side:
        # gather: X read once, the routed rows written (MXFP8: codes + scales)
        gbytes = w.T * w.d * 2 + (w.R * w.d * (1 + 1 / 32) if w.experts == "mxfp8" else w.R * w.d * 2)
        phases["layout_us"] = round(side["layout"] * 1e3, 1)
        phases["gather_ms"] = round(side["gather"], 4)
        phases["gather_gbs"] = round(gbytes / (side["gather"] * 1e-3) / 1e9, 1)
        phases["gather_hbm_frac"] = round(gbytes / (side["gather"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        phases["gather_pull_gbs"] = round(gbytes / (side["gather_pull"] * 1e-3) / 1e9, 1)
        phases["gather_pull_hbm_frac"] = round(gbytes / (side["gather_pull"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        # combine: the expert outputs read, y written, gates and inv read
        cbytes = w.R * w.d * 2 + w.T * w.d * 2 + w.R * 8
        phases["combine_ms"] = round(side["combine"], 4)
        phases["combine_gbs"] = round(cbytes / (side["combine"] * 1e-3) / 1e9, 1)
        phases["combine_hbm_frac"] = round(cbytes / (side["combine"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    if "router_backward" in side:
        phases["router_backward_ms"] = round(side["router_backward"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, inp_cpu, dev)

    line = {"metric": METRIC, "value": round(w.T / (ms_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.experts,
            "data": "synthetic (seeded; random-init expert weights)",
            "config": {"workload": w.name + (" fwd+bwd" if w.backward else " fwd"), "T": w.T, "d": w.d,
                       "E": w.E, "k": w.k, "I": w.I, "score": w.score, "fused": fused,
                       "stage_rows": args.stage_rows, "flags": args.flags, "workgroups": args.workgroups,
                       "producer_cus": args.producer_cus,
                       "macro_tokens": args.macro_tokens},
            "roofline": roof, "cpu_baseline": cpu, "phases": phases,
            "input_gen_s": round(t_gen, 1), "source_sha256": source_digest()}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
