"""GPU parity of moe_backward (expert path, routing frozen) against the fp64
oracle: dX, dW1, dW3, dW2 and dgate on seeded inputs that span several row
tiles with ragged tails, experts with no rows, and skewed loads.

The oracle routes on the logits the GPU forward exported, so both sides
take the same (fp32) routing decision; the GPU backward then consumes the
bf16 pre-activations its own forward saved.  Tolerance: bf16 operands with
fp32 accumulation, max row-relative error <= 2e-2 (per token row for dX, per
expert matrix for the weight gradients; dgate as in parity.dgate_err)."""
import numpy as np
import pytest
import torch

from oracle import moe as M
from mixture_experts_layer_layout_amd import synth

pytestmark = pytest.mark.gpu

api = pytest.importorskip("mixture_experts_layer_layout_amd.api")
from mixture_experts_layer_layout_amd import layer  # noqa: E402
from parity import dgate_err, host, row_rel_err  # noqa: E402

BF16_TOL = 2e-2

SMALL = {
    "dsv3-zipf-small": synth.WORKLOADS["dsv3-fwdbwd-zipf"].shrink(T=500, d=512, E=64, I=256),
    "mixtral-small": synth.WORKLOADS["mixtral-bf16"].shrink(T=300, d=512, I=512, backward=True),
    "one-expert": synth.WORKLOADS["mixtral-bf16"].shrink(T=70, d=256, E=1, k=1, I=256, backward=True),
    "k-equals-E": synth.WORKLOADS["dsv3-bf16"].shrink(T=129, d=256, E=8, k=8, I=256, backward=True),
    "sparse-experts": synth.WORKLOADS["dsv3-bf16"].shrink(T=40, d=256, E=64, k=2, I=256, backward=True),
    # about 350 rows an expert: the forward takes 256-row stages (the
    # automatic choice), the backward its own 128-row tiles
    "mixtral-long": synth.WORKLOADS["mixtral-bf16"].shrink(T=1400, d=512, I=384, backward=True),
}


def run_fwd_bwd(w, seed, fused, n_workgroups=0):
    inp = synth.make_inputs(w, seed, with_dy=True)
    dev = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    y, sv = layer.forward(w, dev, fused=fused, n_workgroups=n_workgroups)
    g = layer.backward(w, dev, sv, fused=fused, n_workgroups=n_workgroups)
    torch.cuda.synchronize()
    assert sv["status"].item() == 0
    return inp, y, sv, g


def check_against_oracle(w, inp, sv, g):
    h = {k: (host(v) if v is not None else None) for k, v in inp.items()}
    logits = sv["logits"].cpu().numpy()          # fp32: the GPU's routing decision
    f = M.forward(h["x"], h["wr"], h["bias"], h["w1"], h["w3"], h["w2"], w.k, w.score, w.renorm,
                  logits=logits)
    assert np.array_equal(host(sv["topk_idx"]), f["topk_idx"])
    assert np.array_equal(host(sv["perm"]), f["perm"])
    b = M.backward(h["dy"], f, h["w1"], h["w3"], h["w2"], w.k)
    errs = {}
    errs["dx"] = row_rel_err(host(g["dx"]), b["dx"])
    errs["dgate"] = dgate_err(host(g["dgate"]), b["dgate"])
    for n in ("dw1", "dw3", "dw2"):
        got = host(g[n])
        worst = 0.0
        for e in range(w.E):
            if f["counts"][e] == 0:
                assert np.all(got[e] == 0), f"{n}[{e}] of an expert without rows is not zero"
                continue
            worst = max(worst, row_rel_err(got[e].reshape(1, -1), b[n][e].reshape(1, -1)))
        errs[n] = worst
    for n, e in errs.items():
        assert e <= BF16_TOL, f"{n} max row-relative error {e:.3e} > {BF16_TOL}"
    return errs


@pytest.mark.parametrize("name", sorted(SMALL))
@pytest.mark.parametrize("fused", [True, False])
def test_backward_matches_oracle(name, fused):
    w = SMALL[name]
    inp, y, sv, g = run_fwd_bwd(w, 3, fused)
    check_against_oracle(w, inp, sv, g)


def test_backward_fused_equals_unfused_bitwise():
    w = SMALL["dsv3-zipf-small"]
    _, _, _, g1 = run_fwd_bwd(w, 4, True)
    _, _, _, g2 = run_fwd_bwd(w, 4, False)
    for n in ("dx", "dw1", "dw3", "dw2", "dgate"):
        assert torch.equal(g1[n], g2[n]), n


@pytest.mark.parametrize("n_wg", [1, 5, 1000])
def test_backward_any_grid_size(n_wg):
    w = SMALL["dsv3-zipf-small"]
    inp, y, sv, g = run_fwd_bwd(w, 5, True, n_workgroups=n_wg)
    check_against_oracle(w, inp, sv, g)


def test_auto_grid_matches_large_grid_bitwise():
    # the automatic grid is capped at the most tasks a phase can have; any
    # grid size computes the same bits
    w = SMALL["dsv3-zipf-small"]
    a = run_fwd_bwd(w, 9, True, n_workgroups=0)
    b = run_fwd_bwd(w, 9, True, n_workgroups=1000)
    assert torch.equal(a[1], b[1])
    for n in a[3]:
        assert torch.equal(a[3][n], b[3][n]), n


def test_backward_repeatable():
    w = SMALL["dsv3-zipf-small"]
    inp = synth.make_inputs(w, 6, with_dy=True)
    dev = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    y, sv = layer.forward(w, dev, fused=True)
    outs = [layer.backward(w, dev, sv, fused=True) for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        for n in o:
            assert torch.equal(o[n], outs[0][n]), n


def test_backward_empty_batch_zeroes_weight_grads():
    w = SMALL["sparse-experts"].shrink(T=0)
    inp = synth.make_inputs(w, 0, with_dy=True)
    dev = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    y, sv = layer.forward(w, dev, fused=True)
    g = layer.backward(w, dev, sv, fused=True)
    torch.cuda.synchronize()
    for n in ("dw1", "dw3", "dw2"):
        assert g[n].abs().max().item() == 0.0


def test_backward_rejects_unsupported_shapes():
    w = synth.WORKLOADS["tiny-fp32"].shrink(T=8, backward=True)   # the backward is bf16 only
    d = layer.desc_for(w)
    with pytest.raises(api.MoeError) as e:
        api.moe_backward(d, None, None, api.make_weights(None, None, None), api.make_saved(), None,
                         None, None, None, None, None)
    assert e.value.code == api.MOE_ERR_UNSUPPORTED


@pytest.mark.parametrize("flags", [0, "PERSISTENT_SINGLE", "PERSISTENT_WGRAD_APART"])
def test_backward_persistent_variants_equal_unfused(flags):
    """Every way of running the persistent scheduler gives the bits of the
    one-kernel-per-step backward."""
    flags = getattr(api, "MOE_FLAG_" + flags) if flags else 0
    w = SMALL["dsv3-zipf-small"]
    inp = synth.make_inputs(w, 9, with_dy=True)
    dev = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    y, sv = layer.forward(w, dev, fused=False)
    g1 = layer.backward(w, dev, sv, fused=True, flags=flags)
    g2 = layer.backward(w, dev, sv, fused=False)
    torch.cuda.synchronize()
    assert sv["status"].item() == 0
    for n in ("dx", "dw1", "dw3", "dw2", "dgate"):
        assert torch.equal(g1[n], g2[n]), n
