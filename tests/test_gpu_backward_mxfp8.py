"""GPU parity of the MXFP8 backward (moe_backward with MXFP8 experts: the
data gradients dHu = G W2 and dXp = dA W1 + dB W3 on the scaled matrix
cores with their operands quantised along d and along I; the weight
gradients dW2 = (g G)^T H, dW1 = dA^T x, dW3 = dB^T x in bf16 by default,
and with MOE_FLAG_MXFP8_WGRAD on the scaled matrix cores too, their
operands quantised along the expert's rows) and of moe_quantize_mxfp8_t
against the fp64 oracle (oracle/mxfp8.py backward_mxfp8 with mx_wgrad
matching the flag, and quantize):

  * the transposed quantisation: codes and scales bit-exact (bf16 inputs,
    so every scale and rounding decision is exact on both sides), with
    ragged column counts and the encoding's edge cases;
  * the backward on seeded inputs with several row tiles, ragged tails,
    experts without rows, k = E and one expert, on both the 4-stage (wide)
    and the per-stage scale reads.  The oracle routes on the logits the GPU
    forward exported; the GPU backward consumes the bf16 A, B, H its MXFP8
    forward saved, the oracle its own, rounded to bfloat16 as the layer
    saves them (and [dA | dB] likewise).  Both quantise dY, W2^T, W1^T, W3^T
    and the x rows identically, g dY from the same product (fp32 against
    fp64), and H, dA, dB from bfloat16 values that differ only where the
    fp32 and fp64 arithmetic before them round to different bfloat16
    neighbours.  Tolerance: max row-relative error 6e-2 (as for the MXFP8
    forward's output)."""
import numpy as np
import pytest
import torch

from oracle import mxfp8 as Q
from mixture_experts_layer_layout_amd import synth

pytestmark = pytest.mark.gpu

api = pytest.importorskip("mixture_experts_layer_layout_amd.api")
from mixture_experts_layer_layout_amd import layer  # noqa: E402
from parity import dgate_err, host, row_rel_err  # noqa: E402
from test_gpu_mxfp8 import edge_matrix  # noqa: E402

MX_TOL = 6e-2


@pytest.mark.parametrize("batch,rows,cols", [(1, 64, 300), (3, 256, 512), (2, 1024, 96)])
def test_quantize_transposed_bit_exact(batch, rows, cols):
    src = torch.stack([edge_matrix(cols, rows, 7 + b).t().contiguous() for b in range(batch)])  # [b, rows, cols]
    codes, scales = layer.quantize_mxfp8_t(src.cuda())
    torch.cuda.synchronize()
    for b in range(batch):
        want_c, want_s = Q.quantize(src[b].double().numpy().T)
        assert np.array_equal(host(codes[b]), want_c.astype(np.int64))
        assert np.array_equal(host(scales[b]), want_s.astype(np.int64))


SMALL = {
    "dsv3-mx-small": synth.WORKLOADS["dsv3-mxfp8"].shrink(T=300, d=768, E=32, I=256),
    "wide-mx": synth.WORKLOADS["dsv3-mxfp8"].shrink(T=260, d=1024, E=16, I=512),
    "one-expert-mx": synth.WORKLOADS["dsv3-mxfp8"].shrink(T=70, d=256, E=1, k=1, I=128),
    "k-equals-E-mx": synth.WORKLOADS["dsv3-mxfp8"].shrink(T=129, d=256, E=8, k=8, I=128),
    "sparse-mx": synth.WORKLOADS["dsv3-mxfp8"].shrink(T=40, d=256, E=64, k=2, I=256),
}


WG = api.MOE_FLAG_MXFP8_WGRAD


def run(w, seed, flags=0):
    inp = synth.make_inputs(w, seed, with_dy=True)
    dev = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    y, sv = layer.forward(w, dev, fused=True)
    g = layer.backward(w, dev, sv, flags=flags)
    torch.cuda.synchronize()
    assert sv["status"].item() == 0
    return inp, sv, g


@pytest.mark.parametrize("flags", [0, WG])
@pytest.mark.parametrize("name", sorted(SMALL))
def test_backward_mxfp8_matches_oracle(name, flags):
    w = SMALL[name]
    inp, sv, g = run(w, 21, flags)
    h = {k: (host(v) if v is not None else None) for k, v in inp.items()}
    logits = sv["logits"].cpu().numpy()
    f = Q.forward_mxfp8(h["x"], h["wr"], h["bias"], h["w1"], h["w3"], h["w2"], w.k, w.score, w.renorm,
                        logits=logits)
    assert np.array_equal(host(sv["topk_idx"]), f["topk_idx"])
    assert np.array_equal(host(sv["perm"]), f["perm"])
    b = Q.backward_mxfp8(h["dy"], h["x"], f, h["w1"], h["w3"], h["w2"], w.k, mx_wgrad=bool(flags & WG))
    errs = {"dx": row_rel_err(host(g["dx"]), b["dx"]), "dgate": dgate_err(host(g["dgate"]), b["dgate"])}
    for n in ("dw1", "dw3", "dw2"):
        got = host(g[n])
        worst = 0.0
        for e in range(w.E):
            if f["counts"][e] == 0:
                assert np.all(got[e] == 0), f"{n}[{e}] of an expert without rows is not zero"
                continue
            worst = max(worst, row_rel_err(got[e].reshape(1, -1), b[n][e].reshape(1, -1)))
        errs[n] = worst
    print(name, hex(flags), {k: f"{v:.2e}" for k, v in errs.items()})
    for n, e in errs.items():
        assert e <= MX_TOL, f"{n} max row-relative error {e:.3e} > {MX_TOL}"


@pytest.mark.parametrize("flags", [0, WG])
def test_backward_mxfp8_persistent_equals_plain_bitwise(flags):
    # the persistent launches and the ordinary grids run the same tiles
    w = SMALL["wide-mx"]
    inp = synth.make_inputs(w, 6, with_dy=True)
    dev = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    y, sv = layer.forward(w, dev, fused=True)
    g1 = layer.backward(w, dev, sv, fused=True, flags=flags)
    g2 = layer.backward(w, dev, sv, fused=False, flags=flags)
    torch.cuda.synchronize()
    assert sv["status"].item() == 0
    for n in g1:
        assert torch.equal(g1[n], g2[n]), n


@pytest.mark.parametrize("flags", [0, WG])
@pytest.mark.parametrize("n_wg", [1, 7, 1000])
def test_backward_mxfp8_any_grid_bitwise(n_wg, flags):
    # the persistent launches with any number of workgroups (one workgroup
    # runs every task in ticket order, so every wait is on work already
    # claimed) give the default grid's bits
    w = SMALL["dsv3-mx-small"]
    inp = synth.make_inputs(w, 8, with_dy=True)
    dev = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    y, sv = layer.forward(w, dev, fused=True)
    g1 = layer.backward(w, dev, sv, fused=True, flags=flags)
    g2 = layer.backward(w, dev, sv, fused=True, n_workgroups=n_wg, flags=flags)
    torch.cuda.synchronize()
    assert sv["status"].item() == 0
    for n in g1:
        assert torch.equal(g1[n], g2[n]), n


@pytest.mark.parametrize("flags", [0, WG])
def test_backward_mxfp8_repeatable_and_empty(flags):
    w = SMALL["dsv3-mx-small"]
    inp = synth.make_inputs(w, 5, with_dy=True)
    dev = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    y, sv = layer.forward(w, dev, fused=True)
    g1 = layer.backward(w, dev, sv, flags=flags)
    g2 = layer.backward(w, dev, sv, flags=flags)
    torch.cuda.synchronize()
    for n in g1:
        assert torch.equal(g1[n], g2[n]), n
    w0 = w.shrink(T=0)
    inp0 = {k: (v.cuda() if v is not None else None) for k, v in synth.make_inputs(w0, 0, with_dy=True).items()}
    y0, sv0 = layer.forward(w0, inp0, fused=True)
    g0 = layer.backward(w0, inp0, sv0, flags=flags)
    torch.cuda.synchronize()
    assert g0["dx"].numel() == 0
    for n in ("dw1", "dw3", "dw2"):
        assert torch.count_nonzero(g0[n]).item() == 0, n
