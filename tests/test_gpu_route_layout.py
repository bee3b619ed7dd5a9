"""GPU parity of the integer steps: top-k routing, counting/layout and the
pull gather, bit-exact against the oracle on the same inputs."""
import numpy as np
import pytest
import torch

from oracle import moe as M
from mixture_experts_layer_layout_amd import synth

pytestmark = pytest.mark.gpu

api = pytest.importorskip("mixture_experts_layer_layout_amd.api")
from parity import host  # noqa: E402


def _route_case(T, E, k, score, renorm, bias, ties, seed):
    lg = synth.random_logits(T, E, seed, ties=ties)
    b = None
    if bias:
        b = torch.from_numpy(np.linspace(-1, 1, E).astype(np.float32))
        if ties:
            b = torch.round(b * 2) / 2
    d = api.make_desc(T, 256, E, k, 128, score=score, renorm=renorm)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, k), dtype=torch.float32, device="cuda")
    api.moe_route(d, lg.cuda(), None if b is None else b.cuda(), idx, gate)
    torch.cuda.synchronize()
    want_idx, want_g = M.route(lg.numpy(), k, score, renorm,
                               None if b is None else b.numpy())
    return host(idx), host(gate), want_idx, want_g


@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (64, 8, 2), (300, 256, 8), (1000, 64, 6),
                                   (77, 1024, 16), (130, 16, 16)])
@pytest.mark.parametrize("score,renorm", [("softmax", True), ("sigmoid", True),
                                          ("softmax", False), ("sigmoid", False)])
def test_route_bitexact(T, E, k, score, renorm):
    for ties in (False, True):
        for bias in (False, True):
            gi, gg, wi, wg = _route_case(T, E, k, score, renorm, bias, ties, seed=T + E)
            assert np.array_equal(gi, wi), f"ties={ties} bias={bias}"
            assert np.max(np.abs(gg - wg)) <= 2e-6 * max(1.0, np.max(np.abs(wg)))


@pytest.mark.parametrize("T,E,k,skew", [(1, 4, 4, None), (64, 8, 2, None), (100, 8, 2, "one"),
                                        (4096, 256, 8, None), (4096, 256, 8, "zipf"),
                                        (513, 1024, 16, "zipf"), (2000, 32, 8, "one"),
                                        (8192, 256, 8, None)])
def test_layout_bitexact(T, E, k, skew):
    idx = synth.random_topk(T, E, k, seed=T * 7 + E, skew=skew)
    d = api.make_desc(T, 256, E, k, 128)
    ws = torch.empty(api.moe_workspace_size(d), dtype=torch.uint8, device="cuda")
    R = T * k
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(R, dtype=torch.int32, device="cuda")
    inv = torch.empty(R, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    api.moe_layout(d, idx.cuda(), counts, offsets, perm, inv, status, ws)
    torch.cuda.synchronize()
    c, o, p, i, _ = M.layout(idx.numpy(), E)
    assert status.item() == 0
    assert np.array_equal(host(counts), c)
    assert np.array_equal(host(offsets), o)
    assert np.array_equal(host(perm), p)
    assert np.array_equal(host(inv), i)


def test_layout_repeatable_and_invalid_route():
    T, E, k = 1000, 64, 4
    idx = synth.random_topk(T, E, k, seed=3).cuda()
    d = api.make_desc(T, 256, E, k, 128)
    ws = torch.empty(api.moe_workspace_size(d), dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(20):
        bufs = [torch.empty(n, dtype=torch.int32, device="cuda") for n in (E, E + 1, T * k, T * k)]
        st = torch.zeros(1, dtype=torch.int32, device="cuda")
        api.moe_layout(d, idx, *bufs, st, ws)
        outs.append([host(b) for b in bufs])
    for o in outs[1:]:
        for a, b in zip(o, outs[0]):
            assert np.array_equal(a, b)
    bad = idx.clone()
    bad[5, 1] = E + 3
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    bufs = [torch.empty(n, dtype=torch.int32, device="cuda") for n in (E, E + 1, T * k, T * k)]
    api.moe_layout(d, bad, *bufs, st, ws)
    torch.cuda.synchronize()
    assert st.item() == api.MOE_ERR_INVALID_ROUTE
    dup = idx.clone()
    dup[7, 1] = dup[7, 0]
    st.zero_()
    api.moe_layout(d, dup, *bufs, st, ws)
    torch.cuda.synchronize()
    assert st.item() == api.MOE_ERR_INVALID_ROUTE


@pytest.mark.parametrize("mode", ["pull", "push"])
@pytest.mark.parametrize("act,d", [("bf16", 7168), ("bf16", 256), ("f32", 128)])
def test_gather_bitexact(act, d, mode):
    T, E, k = 777, 32, 4
    idx = synth.random_topk(T, E, k, seed=11)
    _, _, perm, inv, src = M.layout(idx.numpy(), E)
    dt = torch.bfloat16 if act == "bf16" else torch.float32
    x = torch.randn((T, d), dtype=torch.float32).to(dt)
    desc = api.make_desc(T, d, E, k, 128, act=act, experts=act)
    xp = torch.empty((T * k, d), dtype=dt, device="cuda")
    dev = lambda a: torch.from_numpy(a.astype(np.int32)).cuda()
    if mode == "pull":
        api.moe_gather(desc, x.cuda(), dev(perm), xp)
    else:
        api.moe_gather(desc, x.cuda(), None, xp, inv=dev(inv))
    torch.cuda.synchronize()
    assert torch.equal(xp.cpu(), x[torch.from_numpy(src)])


def test_gather_push_skips_rows_out_of_range():
    T, d, E, k = 130, 256, 16, 2
    idx = synth.random_topk(T, E, k, seed=5)
    _, _, _, inv, src = M.layout(idx.numpy(), E)
    bad = inv.copy()
    lost = [int(bad[3]), int(bad[100])]
    bad[3], bad[100] = -1, T * k
    x = torch.randn((T, d), dtype=torch.float32).to(torch.bfloat16)
    desc = api.make_desc(T, d, E, k, 128)
    xp = torch.full((T * k, d), 7.0, dtype=torch.bfloat16, device="cuda")
    api.moe_gather(desc, x.cuda(), None, xp, inv=torch.from_numpy(bad.astype(np.int32)).cuda())
    torch.cuda.synchronize()
    want = x[torch.from_numpy(src)]
    want[lost] = 7.0
    assert torch.equal(xp.cpu(), want)


def test_host_validation_errors():
    d = api.make_desc(64, 256, 8, 9, 128)
    with pytest.raises(api.MoeError) as e:
        api.moe_route(d, None, None, None, None)
    assert e.value.code == api.MOE_ERR_INVALID_ARG


def test_route_layout_at_the_maximum_expert_count_and_k():
    """E = 1024 experts and k = 16 (the library's limits): routing and layout
    bit-exact against the oracle."""
    T, E, k = 300, 1024, 16
    lg = synth.random_logits(T, E, 21, ties=True)
    d = api.make_desc(T, 256, E, k, 128)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, k), dtype=torch.float32, device="cuda")
    api.moe_route(d, lg.cuda(), None, idx, gate)
    ws = torch.empty(api.moe_workspace_size(d), dtype=torch.uint8, device="cuda")
    bufs = [torch.empty(n, dtype=torch.int32, device="cuda") for n in (E, E + 1, T * k, T * k)]
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    api.moe_layout(d, idx, *bufs, st, ws)
    torch.cuda.synchronize()
    assert st.item() == 0
    want_idx, want_g = M.route(lg.numpy(), k, "sigmoid", True)
    assert np.array_equal(idx.cpu().numpy(), want_idx)
    assert np.max(np.abs(gate.cpu().numpy() - want_g)) < 2e-6
    counts, offsets, perm, inv, _ = M.layout(want_idx, E)
    for got, want in zip(bufs, (counts, offsets, perm, inv)):
        assert np.array_equal(got.cpu().numpy(), want)


def test_gather_push_of_an_empty_batch_is_a_no_op():
    desc = api.make_desc(0, 256, 8, 2, 128)
    xp = torch.full((4, 256), 3.0, dtype=torch.bfloat16, device="cuda")
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    inv = torch.empty((0,), dtype=torch.int32, device="cuda")
    api.moe_gather(desc, x, None, xp, inv=inv)
    torch.cuda.synchronize()
    assert torch.all(xp == 3.0)
