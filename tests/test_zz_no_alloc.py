"""moe_forward_noalloc (the forward with its workspace in the library's
static device array) against moe_forward with a caller workspace, through
the C ABI, two calls in a row on one GPU, the second with a smaller input:

* shapes whose workspace fits the array: one call, every saved output, the
  same bits as moe_forward (y, routing, layout, activations);
* a DeepSeek-V3-width shape whose workspace for all tokens exceeds the
  256 MiB array: macrobatches, y and the per-token outputs the same bits
  as one moe_forward call over all tokens; asking for the layout then
  returns MOE_ERR_WORKSPACE.
"""
import dataclasses

import pytest
import torch

from mixture_experts_layer_layout_amd import synth

pytestmark = pytest.mark.gpu

api = pytest.importorskip("mixture_experts_layer_layout_amd.api")
from mixture_experts_layer_layout_amd import layer  # noqa: E402

PER_TOKEN = ("logits", "topk_idx", "gate")
LAYOUT = ("counts", "offsets", "perm", "inv", "a", "b", "h")


def _dev(w, seed):
    return {k: (v.cuda() if v is not None else None) for k, v in synth.make_inputs(w, seed).items()}


def _noalloc(w, inp, full=True):
    d = layer.desc_for(w, T=inp["x"].shape[0])
    weights, keep = layer.weights_of(w, inp)
    saved = layer.alloc_saved(w, "cuda", full=full, T=inp["x"].shape[0])
    if not full:
        for n in ("counts", "offsets", "perm", "inv"):
            saved.pop(n)
    y = torch.empty(inp["x"].shape, dtype=inp["x"].dtype, device="cuda")
    api.moe_forward_noalloc(d, inp["x"], inp["wr"], inp.get("bias"), weights, y, api.make_saved(**saved))
    return y, saved


def _check_pair(w, seeds_T, full):
    for seed, T in seeds_T:
        wt = dataclasses.replace(w, T=T)
        inp = _dev(wt, seed)
        print(f"\nnoalloc {w.name} T={T} seed={seed} "
              f"workspace {api.moe_workspace_size(layer.desc_for(wt)) / 2**20:.0f} MiB", flush=True)
        y1, s1 = _noalloc(wt, inp, full=full)
        y0, s0 = layer.forward(wt, inp)
        torch.cuda.synchronize()
        assert s0["status"].item() == 0 and s1["status"].item() == 0
        assert torch.equal(y0, y1)
        for n in PER_TOKEN + (LAYOUT if full else ()):
            assert torch.equal(s0[n], s1[n]), n


@pytest.mark.parametrize("name,w", [
    ("dsv3-bf16", synth.WORKLOADS["dsv3-bf16"].shrink(T=333, d=768, E=32, I=256)),
    ("mixtral-bf16", synth.WORKLOADS["mixtral-bf16"].shrink(T=300, d=512, I=384)),
    ("dsv3-mxfp8", synth.WORKLOADS["dsv3-mxfp8"].shrink(T=300, d=512, E=16, k=4, I=256)),
    ("tiny-fp32", synth.WORKLOADS["tiny-fp32"]),
])
def test_noalloc_fits_equals_forward(name, w):
    _check_pair(w, [(1, w.T), (2, max(1, w.T // 3))], full=True)


def test_noalloc_macrobatches_equal_one_forward():
    # d = 7168, I = 2048, E = 16, k = 4: about 130 KB of workspace a token,
    # so 3000 tokens (about 390 MiB) and 2200 tokens need macrobatches
    w = synth.WORKLOADS["dsv3-bf16"].shrink(T=3000, E=16, k=4)
    assert api.moe_workspace_size(layer.desc_for(w)) > api.MOE_NOALLOC_SCRATCH_BYTES
    _check_pair(w, [(3, 3000), (4, 2200)], full=False)
    # the layout of all tokens cannot come from macrobatches
    inp = _dev(w, 5)
    with pytest.raises(api.MoeError) as err:
        _noalloc(w, inp, full=True)
    assert err.value.code == api.MOE_ERR_WORKSPACE
