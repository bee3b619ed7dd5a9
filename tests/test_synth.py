"""The seeded input generator (no GPU): determinism, shapes, distributions."""
import numpy as np
import torch

from mixture_experts_layer_layout_amd import synth


def test_same_seed_same_tensors_and_expert_independence():
    w = synth.WORKLOADS["dsv3-bf16"].shrink(T=32, d=64, E=6, k=2, I=32)
    a = synth.make_inputs(w, 3)
    b = synth.make_inputs(w, 3)
    c = synth.make_inputs(w, 4)
    for k in ("x", "wr", "w1", "w3", "w2"):
        assert torch.equal(a[k], b[k])
        assert not torch.equal(a[k], c[k])
    w2 = w.shrink(E=3)
    d = synth.make_inputs(w2, 3)
    assert torch.equal(d["w1"], a["w1"][:3])      # per-expert streams


def test_dtypes_and_scales():
    w = synth.WORKLOADS["mixtral-bf16"].shrink(T=256, d=512, I=1024)
    t = synth.make_inputs(w, 0)
    assert t["x"].dtype == torch.bfloat16 and t["w1"].shape == (8, 1024, 512)
    assert abs(t["x"].float().std().item() - 1.0) < 0.05
    assert abs(t["w1"].float().std().item() * np.sqrt(512) - 1.0) < 0.05
    assert abs(t["w2"].float().std().item() * np.sqrt(1024) - 1.0) < 0.05
    tiny = synth.make_inputs(synth.WORKLOADS["tiny-fp32"], 0)
    assert tiny["x"].dtype == torch.float32
    assert abs(tiny["w1"].std().item() - 0.02) < 0.002


def test_capped_zipf_targets():
    t = synth.capped_zipf_targets(256, 4096, 8, 1.2)
    assert abs(t.sum() - 4096 * 8) < 1e-6
    assert t.max() <= 4096 + 1e-9
    assert np.all(np.diff(t) <= 1e-9)
    assert t[0] == 4096 and t[1] == 4096 and 10 < t[-1] < 15


def test_zipf_bias_skews_loads():
    w = synth.WORKLOADS["dsv3-fwdbwd-zipf"].shrink(T=1024, d=256)
    b = synth.zipf_router_bias(w, 0, iters=100)
    assert b.dtype == np.float32 and b.shape == (256,)
    # on stand-in logits the loads follow the targets
    rng = np.random.default_rng(9)
    z = rng.standard_normal((1024, 256))
    top = np.argpartition(-(z + b), 7, axis=1)[:, :8]
    load = np.sort(np.bincount(top.reshape(-1), minlength=256))[::-1]
    want = synth.capped_zipf_targets(256, 1024, 8, 1.2)
    assert load[0] > 0.9 * 1024 and load[:8].sum() > 0.8 * want[:8].sum()
    assert load.max() / load.mean() > 10
