"""GPU parity of the whole forward layer (moe_forward, fused and unfused)
against the fp64 oracle on seeded inputs spanning several tiles with ragged
tails.  Routing indices and the layout must match exactly on every token
whose top-k margin is clear of fp32 rounding; floating outputs are compared
per row (max-norm relative error)."""
import numpy as np
import pytest
import torch

from oracle import moe as M
from mixture_experts_layer_layout_amd import synth

pytestmark = pytest.mark.gpu

api = pytest.importorskip("mixture_experts_layer_layout_amd.api")
from mixture_experts_layer_layout_amd import layer  # noqa: E402
from parity import compare_routing, host, logit_tolerance, row_rel_err  # noqa: E402

BF16_TOL = 2e-2     # max row-relative error for bf16 operands, fp32 accumulation
F32_TOL = 1e-4      # fp32 layer: fp32 accumulation over d, I <= 256


def run_and_check(w, seed, fused, stage_rows=0, flags=0, n_workgroups=0, tol=None, n_producer_cus=0):
    inp = synth.make_inputs(w, seed)
    h = {k: (host(v) if v is not None else None) for k, v in inp.items()}
    dev = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    y, sv = layer.forward(w, dev, fused=fused, stage_rows=stage_rows, flags=flags,
                          n_workgroups=n_workgroups, n_producer_cus=n_producer_cus)
    torch.cuda.synchronize()
    assert sv["status"].item() == 0
    f = M.forward(h["x"], h["wr"], h["bias"], h["w1"], h["w3"], h["w2"], w.k, w.score, w.renorm)
    # logits (bias excluded) agree with the fp64 router GEMM
    lt = logit_tolerance(h["x"], h["wr"])
    assert np.max(np.abs(host(sv["logits"]) - f["logits"]) / lt[:, None]) < 1.0
    ora_biased = f["logits"] + (h["bias"][None, :] if h["bias"] is not None else 0)
    same = compare_routing(host(sv["topk_idx"]), ora_biased, f["topk_idx"], lt)
    gi = host(sv["topk_idx"])
    if same.all():
        assert np.array_equal(host(sv["counts"]), f["counts"])
        assert np.array_equal(host(sv["offsets"]), f["offsets"])
        assert np.array_equal(host(sv["perm"]), f["perm"])
        assert np.array_equal(host(sv["inv"]), f["inv"])
    else:  # near ties changed the routing: the layout must still be valid for it
        c, o, p, i, _ = M.layout(gi, w.E)
        assert np.array_equal(host(sv["perm"]), p) and np.array_equal(host(sv["inv"]), i)
    g = host(sv["gate"])
    assert np.max(np.abs(g[same] - f["gate"][same])) < 1e-4
    tol = tol if tol is not None else (F32_TOL if w.act == "f32" else BF16_TOL)
    err = row_rel_err(host(y), f["y"], rows=same)
    assert err <= tol, f"y row-rel err {err:.3e} > {tol}"
    # saved pre-activations and SwiGLU output, row by row (matched routing)
    if same.all():
        for name in ("A", "B", "H"):
            e2 = row_rel_err(host(sv[name.lower()]), f[name])
            assert e2 <= tol, f"{name} err {e2:.3e}"
    return err, int((~same).sum())


TINY = synth.WORKLOADS["tiny-fp32"]


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny_fp32(fused, seed):
    run_and_check(TINY, seed, fused)


SMALL = {
    "mixtral-small": synth.WORKLOADS["mixtral-bf16"].shrink(T=300, d=512, I=384),
    "dsv3-small": synth.WORKLOADS["dsv3-bf16"].shrink(T=333, d=768, E=32, I=256),
    "dsv3-zipf-small": synth.WORKLOADS["dsv3-fwdbwd-zipf"].shrink(T=500, d=512, E=64, I=256),
    "one-expert": synth.WORKLOADS["mixtral-bf16"].shrink(T=70, d=256, E=1, k=1, I=128),
    "k-equals-E": synth.WORKLOADS["dsv3-bf16"].shrink(T=129, d=256, E=8, k=8, I=128),
    # about 350 rows per expert: 256-row stages run full 256-row tiles and
    # ragged tails of either narrower tile
    "mixtral-long": synth.WORKLOADS["mixtral-bf16"].shrink(T=1400, d=512, I=384),
}


@pytest.mark.parametrize("name", sorted(SMALL))
@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("stage_rows", [64, 128, 256])
def test_bf16_small(name, fused, stage_rows):
    run_and_check(SMALL[name], 5, fused, stage_rows=stage_rows)


@pytest.mark.parametrize("name", ["dsv3-small", "mixtral-small"])
def test_bf16_direct_pull(name):
    run_and_check(SMALL[name], 6, True, flags=api.MOE_FLAG_DIRECT_PULL)


@pytest.mark.parametrize("n_wg", [1, 3, 8, 1000])
def test_fused_any_grid_size(n_wg):
    run_and_check(SMALL["dsv3-small"], 7, True, n_workgroups=n_wg)


@pytest.mark.parametrize("name", ["tiny-fp32", "dsv3-small"])
def test_auto_grid_matches_large_grid_bitwise(name):
    # the automatic grid is capped at the most tasks a phase can have (a
    # handful for the 64-token fp32 layer); any grid size gives the same bits
    w = synth.WORKLOADS[name] if name in synth.WORKLOADS else SMALL[name]
    inp = {k: (v.cuda() if v is not None else None) for k, v in synth.make_inputs(w, 10).items()}
    y1, _ = layer.forward(w, inp, fused=True, n_workgroups=0)
    y2, _ = layer.forward(w, inp, fused=True, n_workgroups=1000)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("fused", [True, False])
def test_stage_rows_same_bits(fused):
    # 64-, 128- and 256-row stages (and the automatic choice, 256 here: about
    # 350 rows an expert) run different tiles with the same k order into
    # each accumulator, so every output bit agrees
    w = SMALL["mixtral-long"]
    inp = {k: (v.cuda() if v is not None else None) for k, v in synth.make_inputs(w, 11).items()}
    ys = [layer.forward(w, inp, fused=fused, stage_rows=sr)[0] for sr in (0, 64, 128, 256)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(ys[0], y)


def test_fused_equals_unfused_bitwise():
    w = SMALL["dsv3-zipf-small"]
    inp = {k: (v.cuda() if v is not None else None) for k, v in synth.make_inputs(w, 8).items()}
    y1, s1 = layer.forward(w, inp, fused=True)
    y2, s2 = layer.forward(w, inp, fused=False)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    for n in ("topk_idx", "counts", "offsets", "perm", "inv", "h"):
        assert torch.equal(s1[n], s2[n]), n


def test_empty_batch():
    w = SMALL["dsv3-small"].shrink(T=0)
    inp = {k: (v.cuda() if v is not None else None) for k, v in synth.make_inputs(w, 0).items()}
    y, sv = layer.forward(w, inp, fused=True)
    torch.cuda.synchronize()
    assert y.numel() == 0
    assert host(sv["counts"]).sum() == 0 and np.all(host(sv["offsets"]) == 0)


@pytest.mark.parametrize("flags", ["PERSISTENT_SPLIT", "PERSISTENT_SINGLE", "PERSISTENT_GEMM_APART", "DIRECT_PULL"])
def test_forward_persistent_variants_equal_unfused(flags):
    w = SMALL["dsv3-zipf-small"]
    f = getattr(api, "MOE_FLAG_" + flags)
    inp = {k: (v.cuda() if v is not None else None) for k, v in synth.make_inputs(w, 10).items()}
    y1, s1 = layer.forward(w, inp, fused=True, flags=f)
    y2, s2 = layer.forward(w, inp, fused=False)
    torch.cuda.synchronize()
    assert s1["status"].item() == 0
    assert torch.equal(y1, y2)
    for n in ("topk_idx", "counts", "offsets", "perm", "inv", "h", "a", "b"):
        assert torch.equal(s1[n], s2[n]), n


MACRO = {
    "dsv3-zipf-bf16": (synth.WORKLOADS["dsv3-fwdbwd-zipf"].shrink(T=300, d=512, E=64, I=256, backward=False), 96),
    "mixtral-bf16": (synth.WORKLOADS["mixtral-bf16"].shrink(T=300, d=512, I=512), 128),
    "dsv3-mxfp8": (synth.WORKLOADS["dsv3-mxfp8"].shrink(T=200, d=512, E=16, k=4, I=256), 64),
    "tiny-fp32": (synth.WORKLOADS["tiny-fp32"], 24),
}


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("name", sorted(MACRO))
def test_macrobatched_forward_equals_one_call(name, fused):
    """moe_forward in macrobatches (the last one ragged) through the ring of
    two workspace slots writes the same bits as one call over all tokens,
    from a workspace sized for two macrobatches; fused: each macrobatch's
    merge runs in the next one's launch, else the plain kernels in stream
    order."""
    import dataclasses
    w, tm = MACRO[name]
    wm = dataclasses.replace(w, macro_tokens=tm)
    inp = synth.make_inputs(w, 5)
    dev = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    y0, s0 = layer.forward(w, dev)
    y1, s1 = layer.forward(wm, dev, fused=fused)
    torch.cuda.synchronize()
    assert s0["status"].item() == 0 and s1["status"].item() == 0
    assert "perm" not in s1
    for n in ("logits", "topk_idx", "gate"):
        assert torch.equal(s0[n], s1[n]), n
    assert torch.equal(y0, y1)
    assert api.moe_workspace_size(layer.desc_for(wm)) < api.moe_workspace_size(layer.desc_for(w))


@pytest.mark.parametrize("n_prod", [1, 4, 32])
@pytest.mark.parametrize("name", ["dsv3-zipf-small", "mixtral-small"])
def test_cu_partition_equals_unfused(name, n_prod):
    """moe_desc.n_producer_cus: producer workgroups run routing, layout,
    gather and combine, the rest the GEMM tiles; the same bits as the
    separate kernels, and the oracle's routing and outputs."""
    w = SMALL[name]
    run_and_check(w, 12, True, n_producer_cus=n_prod)
    inp = {k: (v.cuda() if v is not None else None) for k, v in synth.make_inputs(w, 13).items()}
    y1, s1 = layer.forward(w, inp, fused=True, n_producer_cus=n_prod)
    y2, s2 = layer.forward(w, inp, fused=False)
    torch.cuda.synchronize()
    assert s1["status"].item() == 0
    assert torch.equal(y1, y2)
    for n in ("topk_idx", "perm", "inv", "h"):
        assert torch.equal(s1[n], s2[n]), n


def test_cu_partition_rejects_unresident_grid():
    w = SMALL["dsv3-small"]
    inp = {k: (v.cuda() if v is not None else None) for k, v in synth.make_inputs(w, 14).items()}
    with pytest.raises(api.MoeError) as err:
        layer.forward(w, inp, fused=True, n_producer_cus=4, n_workgroups=100000)
    assert err.value.code == api.MOE_ERR_INVALID_ARG
