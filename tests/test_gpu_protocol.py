"""The persistent kernels' hand-off protocol on the GPU.

* A counter held back from the host (the test-only MOE_FLAG_TEST_DROP_READY:
  the gather of row tile 0 does not raise its ready counter) with the
  test-only tiny spin limit: the call must record MOE_ERR_TIMEOUT in the
  device status word and every kernel must exit (the stream synchronises);
  the next ordinary call on the same workspace must give the same bits as a
  call on a fresh one.
* Workgroups claiming from hashed home sub-queues (the test-only
  MOE_FLAG_TEST_SHUFFLE_CLAIMS) must give the same bits as the default.
* The MXFP8 forward (whose up projection reads the layout's source index
  written in the same launch) and the single-launch variants, run on one
  workspace for a sequence of different routings, must give for each the
  bits of a call on a fresh workspace (no index or scale survives from an
  earlier call or another tile).
MoK flash §01/§02: compute waits until its rows are complete; GPU-local
counters signal it.
"""
import pytest
import torch

from mixture_experts_layer_layout_amd import synth

pytestmark = pytest.mark.gpu

api = pytest.importorskip("mixture_experts_layer_layout_amd.api")
from mixture_experts_layer_layout_amd import layer  # noqa: E402

W = {
    "dsv3-bf16": synth.WORKLOADS["dsv3-bf16"].shrink(T=333, d=768, E=32, I=256),
    "dsv3-mxfp8": synth.WORKLOADS["dsv3-mxfp8"].shrink(T=300, d=512, E=16, k=4, I=256),
    "zipf-bf16": synth.WORKLOADS["dsv3-fwdbwd-zipf"].shrink(T=500, d=512, E=64, I=256),
}


def _dev(w, seed):
    return {k: (v.cuda() if v is not None else None) for k, v in synth.make_inputs(w, seed).items()}


def _same(a, b, names):
    for n in names:
        assert torch.equal(a[n], b[n]), n


@pytest.mark.parametrize("name", ["dsv3-bf16", "dsv3-mxfp8"])
def test_held_back_counter_times_out_and_drains(name):
    w = W[name]
    inp = _dev(w, 3)
    print(f"\nheld-back counter {name}", flush=True)
    d = layer.desc_for(w)
    ws = layer.workspace(d)
    y0, s0 = layer.forward(w, inp, ws=ws, flags=api.MOE_FLAG_SPIN_LIMIT_TINY | api.MOE_FLAG_TEST_DROP_READY)
    torch.cuda.synchronize()   # every kernel of the call has exited
    assert s0["status"].item() == api.MOE_ERR_TIMEOUT
    y1, s1 = layer.forward(w, inp, ws=ws)
    y2, s2 = layer.forward(w, inp)
    torch.cuda.synchronize()
    assert s1["status"].item() == 0 and s2["status"].item() == 0
    assert torch.equal(y1, y2)
    _same(s1, s2, ("topk_idx", "counts", "offsets", "perm", "inv", "h"))


@pytest.mark.parametrize("name", sorted(W))
def test_shuffled_claims_give_the_same_bits(name):
    w = W[name]
    inp = _dev(w, 4)
    y0, s0 = layer.forward(w, inp)
    y1, s1 = layer.forward(w, inp, flags=api.MOE_FLAG_TEST_SHUFFLE_CLAIMS)
    torch.cuda.synchronize()
    assert s0["status"].item() == 0 and s1["status"].item() == 0
    assert torch.equal(y0, y1)
    _same(s0, s1, ("topk_idx", "counts", "offsets", "perm", "inv", "h", "a", "b"))
    if w.backward:
        g0 = layer.backward(w, inp, s0)
        g1 = layer.backward(w, inp, s1, flags=api.MOE_FLAG_TEST_SHUFFLE_CLAIMS)
        torch.cuda.synchronize()
        _same(g0, g1, ("dx", "dw1", "dw3", "dw2", "dgate"))


@pytest.mark.parametrize("name,flags", [("dsv3-mxfp8", 0), ("dsv3-mxfp8", api.MOE_FLAG_PERSISTENT_SINGLE),
                                        ("dsv3-bf16", api.MOE_FLAG_DIRECT_PULL),
                                        ("zipf-bf16", api.MOE_FLAG_PERSISTENT_SINGLE)])
def test_reused_workspace_over_changing_routings(name, flags):
    w = W[name]
    d = layer.desc_for(w, flags=flags)
    ws = layer.workspace(d)
    for seed in (11, 12, 13):
        inp = _dev(w, seed)
        y1, s1 = layer.forward(w, inp, ws=ws, flags=flags)
        y2, s2 = layer.forward(w, inp, flags=flags)
        torch.cuda.synchronize()
        assert s1["status"].item() == 0 and s2["status"].item() == 0
        assert torch.equal(y1, y2), seed
        _same(s1, s2, ("topk_idx", "perm", "inv"))


@pytest.mark.parametrize("name", sorted(W))
@pytest.mark.parametrize("flags", [0, api.MOE_FLAG_PERSISTENT_SINGLE])
def test_prefilled_workspace_gives_the_separate_kernels_bits(name, flags):
    # Every byte the call reads it has written first: a workspace and saved
    # buffers pre-filled with byte patterns must give the bits of the
    # separate kernels, at the automatic grid, at 75 workgroups and at 512.
    # (With the router's slices published by the L2 write-back, a top-k on
    # another XCD now and then read them before the router's values: the
    # pattern's logits for 2 or 4 tokens.)
    w = W[name]
    T = w.T
    for seed in (11, 12):
        inp = _dev(w, seed)
        ref, _ = layer.forward(w, inp, fused=False)
        d = layer.desc_for(w, flags=flags, T=T)
        weights, keep = layer.weights_of(w, inp)
        for nwg in (0, 75, 512):
            d.n_workgroups = nwg
            for fill in (0x7F, 0x41, 0x00):
                ws = layer.workspace(d)
                ws.fill_(fill)
                sv = layer.alloc_saved(w, "cuda", T=T)
                for k, v in sv.items():
                    if v is not None and k != "status":
                        v.view(torch.uint8).fill_(fill)
                y = torch.empty_like(ref)
                api.moe_forward(d, inp["x"], inp["wr"], inp.get("bias"), weights, y, api.make_saved(**sv), ws)
                torch.cuda.synchronize()
                assert sv["status"].item() == 0
                assert torch.equal(y, ref), (seed, nwg, hex(fill))
