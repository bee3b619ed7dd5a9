"""GPU parity of the MXFP8 path against the fp64 oracle (oracle/mxfp8.py):

  * moe_quantize_mxfp8 and the quantising moe_gather: codes and scales
    bit-exact (the inputs are bf16, so scale and rounding decisions are exact
    on both sides), on values built to hit every branch of the encoding:
    ties, saturation, subnormal codes, zero blocks, both signs, powers of two;
  * moe_forward with expert_dtype MXFP8 (fused, split and unfused): routing
    and layout exact, y within the MXFP8 tolerance per row;
  * the persistent variants produce bit-identical outputs to the separate
    kernels.
The oracle quantises the bf16 weights itself; no input of it comes from the
GPU."""
import numpy as np
import pytest
import torch

from oracle import moe as M
from oracle import mxfp8 as Q
from mixture_experts_layer_layout_amd import synth

pytestmark = pytest.mark.gpu

api = pytest.importorskip("mixture_experts_layer_layout_amd.api")
from mixture_experts_layer_layout_amd import layer  # noqa: E402
from parity import compare_routing, host, logit_tolerance, row_rel_err  # noqa: E402

MX_TOL = 6e-2   # max row-relative error of y for MXFP8 operands, fp32 accumulation


def edge_matrix(rows, K, seed):
    """bf16 [rows, K] whose 32-blocks cover the encoding's cases."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((rows, K), generator=g, dtype=torch.float64)
    mag = torch.exp2(torch.randint(-30, 30, (rows, K // 32, 1), generator=g).double())
    x = (x.view(rows, K // 32, 32) * mag).view(rows, K)
    xb = x.to(torch.bfloat16)
    nb = K // 32
    blk = xb.view(rows, nb, 32)
    blk[0, 0] = 0                                                # zero block
    if nb > 1:
        # amax 1.9 * 2^k: elements near amax scale past 448 and saturate
        blk[0, 1] = torch.linspace(-1.9, 1.9, 32).to(torch.bfloat16)
    if nb > 2:
        # scale 2^0 block (amax in [256, 512)) holding exact E4M3 ties
        ties = torch.tensor([256.0, 1.0625, 1.1875, -1.0625, 17.0, 19.0, 0.5 + 1 / 32, 2.0 ** -10,
                             3 * 2.0 ** -11, -2.0 ** -10, 2.0 ** -9, 1.5 * 2.0 ** -9] + [0.0] * 20)
        blk[0, 2] = ties.to(torch.bfloat16)
    if nb > 3 and rows > 1:
        blk[1, 3] = torch.exp2(torch.arange(-16, 16).double()).to(torch.bfloat16)   # powers of two
        blk[1, 0] = (torch.randn(32, generator=g) * 2.0 ** -120).to(torch.bfloat16)  # tiny: scale clamps
    return xb


@pytest.mark.parametrize("rows,K", [(7, 256), (129, 7168), (1000, 2048)])
def test_quantize_bit_exact(rows, K):
    x = edge_matrix(rows, K, rows)
    codes, scales = layer.quantize_mxfp8(x.cuda())
    torch.cuda.synchronize()
    want_c, want_s = Q.quantize(x.double().numpy())
    assert np.array_equal(host(scales), want_s.astype(np.int64))
    assert np.array_equal(host(codes), want_c.astype(np.int64))


@pytest.mark.parametrize("mode", ["pull", "push"])
def test_gather_quantises_bit_exact(mode):
    w = synth.WORKLOADS["dsv3-mxfp8"].shrink(T=100, d=512, E=16, k=4, I=256)
    x = edge_matrix(w.T, w.d, 3)
    logits = synth.random_logits(w.T, w.E, 4)
    d = layer.desc_for(w)
    idx = torch.empty((w.T, w.k), dtype=torch.int32, device="cuda")
    gate = torch.empty((w.T, w.k), dtype=torch.float32, device="cuda")
    api.moe_route(d, logits.cuda(), None, idx, gate)
    counts = torch.empty(w.E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(w.E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(w.R, dtype=torch.int32, device="cuda")
    inv = torch.empty(w.R, dtype=torch.int32, device="cuda")
    ws = layer.workspace(d)
    api.moe_layout(d, idx, counts, offsets, perm, inv, None, ws)
    xq = torch.empty((w.R, w.d), dtype=torch.uint8, device="cuda")
    xs = torch.empty((w.R, w.d // 32), dtype=torch.uint8, device="cuda")
    if mode == "pull":
        api.moe_gather(d, x.cuda(), perm, xq, xs)
    else:
        api.moe_gather(d, x.cuda(), None, xq, xs, inv=inv)
    torch.cuda.synchronize()
    src = host(perm) // w.k
    want_c, want_s = Q.quantize(x.double().numpy()[src])
    assert np.array_equal(host(xq), want_c.astype(np.int64))
    assert np.array_equal(host(xs), want_s.astype(np.int64))


def run_mx(w, seed, fused, flags=0, n_workgroups=0):
    inp = synth.make_inputs(w, seed)
    h = {k: (host(v) if v is not None else None) for k, v in inp.items()}
    dev = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    y, sv = layer.forward(w, dev, fused=fused, flags=flags, n_workgroups=n_workgroups)
    torch.cuda.synchronize()
    assert sv["status"].item() == 0
    f = Q.forward_mxfp8(h["x"], h["wr"], h["bias"], h["w1"], h["w3"], h["w2"], w.k, w.score, w.renorm)
    lt = logit_tolerance(h["x"], h["wr"])
    assert np.max(np.abs(host(sv["logits"]) - f["logits"]) / lt[:, None]) < 1.0
    ora_biased = f["logits"] + (h["bias"][None, :] if h["bias"] is not None else 0)
    same = compare_routing(host(sv["topk_idx"]), ora_biased, f["topk_idx"], lt)
    if same.all():
        for n in ("counts", "offsets", "perm", "inv"):
            assert np.array_equal(host(sv[n]), f[n]), n
        # H before its quantisation (bf16 copy) from quantised x and weights
        e_h = row_rel_err(host(sv["h"]), f["H"])
        assert e_h <= 2e-2, f"H err {e_h:.3e}"
    err = row_rel_err(host(y), f["y"], rows=same)
    assert err <= MX_TOL, f"y row-rel err {err:.3e} > {MX_TOL}"
    return y, sv


SMALL = {
    "dsv3-mx-small": synth.WORKLOADS["dsv3-mxfp8"].shrink(T=300, d=768, E=32, I=256),
    "mixtral-mx-small": synth.WORKLOADS["mixtral-bf16"].shrink(T=200, d=512, I=384, experts="mxfp8"),
    "one-expert-mx": synth.WORKLOADS["dsv3-mxfp8"].shrink(T=70, d=256, E=1, k=1, I=128),
    "k-equals-E-mx": synth.WORKLOADS["dsv3-mxfp8"].shrink(T=129, d=256, E=8, k=8, I=128),
}


@pytest.mark.parametrize("name", sorted(SMALL))
@pytest.mark.parametrize("fused", [True, False])
def test_forward_mxfp8_small(name, fused):
    run_mx(SMALL[name], 11, fused)


@pytest.mark.parametrize("n_wg", [1, 5, 1000])
def test_forward_mxfp8_any_grid(n_wg):
    run_mx(SMALL["dsv3-mx-small"], 12, True, n_workgroups=n_wg)


@pytest.mark.parametrize("flags", [0, "PERSISTENT_SPLIT"])
def test_forward_mxfp8_fused_equals_unfused(flags):
    w = SMALL["dsv3-mx-small"]
    f = getattr(api, "MOE_FLAG_" + flags) if flags else 0
    inp = {k: (v.cuda() if v is not None else None) for k, v in synth.make_inputs(w, 13).items()}
    y1, s1 = layer.forward(w, inp, fused=True, flags=f)
    y2, s2 = layer.forward(w, inp, fused=False)
    torch.cuda.synchronize()
    assert s1["status"].item() == 0 and s2["status"].item() == 0
    assert torch.equal(y1, y2)
    for n in ("topk_idx", "counts", "offsets", "perm", "inv", "h", "a", "b"):
        assert torch.equal(s1[n], s2[n]), n


def test_forward_mxfp8_empty_batch():
    w = SMALL["dsv3-mx-small"].shrink(T=0)
    inp = {k: (v.cuda() if v is not None else None) for k, v in synth.make_inputs(w, 0).items()}
    y, sv = layer.forward(w, inp, fused=True)
    torch.cuda.synchronize()
    assert y.numel() == 0 and host(sv["counts"]).sum() == 0
