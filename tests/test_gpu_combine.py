"""GPU parity of moe_combine, the weighted merge on its own (MoK flash §01:
each expert's result returns to its token's position, weighted by the
token's gates), against the fp64 oracle (oracle/moe.py combine) on seeded
routings: every k path (the unrolled k = 1, 2, 4, 6, 8 and the generic one),
ragged token counts, bf16 and f32 activations.  Tolerance: fp32 accumulation
of k products then one rounding to the output type, so the max row-relative
error stays below 2^-8 for bf16 (half a bf16 step is 2^-9 of a value) and
1e-6 for f32.  An entry of inv outside [0, R) must read row 0, and T = 0 is a
no-op."""
import numpy as np
import pytest
import torch

from oracle import moe as M
from mixture_experts_layer_layout_amd import synth

pytestmark = pytest.mark.gpu

api = pytest.importorskip("mixture_experts_layer_layout_amd.api")
from parity import host, row_rel_err  # noqa: E402

CASES = [(333, 512, 16, 1, "bf16"), (300, 768, 32, 2, "bf16"), (129, 256, 8, 4, "bf16"),
         (200, 1024, 64, 6, "bf16"), (4100, 512, 256, 8, "bf16"), (77, 256, 16, 3, "bf16"),
         (150, 256, 8, 2, "f32"), (64, 128, 32, 5, "f32")]


def _case(T, d, E, k, act, seed):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx, gate = M.route(logits, k, M.SIGMOID, True)
    counts, offsets, perm, inv, src = M.layout(idx, E)
    R = T * k
    dt = torch.bfloat16 if act == "bf16" else torch.float32
    yp = torch.randn(R, d, generator=torch.Generator().manual_seed(seed)).to(dt)
    return yp, gate.astype(np.float32), inv.astype(np.int32)


def _run(T, d, E, k, act, yp, gate, inv):
    desc = api.make_desc(T, d, E, k, 2 * 128, act=act, experts=act)
    y = torch.empty((T, d), dtype=yp.dtype, device="cuda")
    api.moe_combine(desc, yp.cuda(), torch.from_numpy(gate).cuda(), torch.from_numpy(inv).cuda(), y)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("T,d,E,k,act", CASES)
def test_combine_matches_oracle(T, d, E, k, act):
    yp, gate, inv = _case(T, d, E, k, act, 31 + k)
    y = _run(T, d, E, k, act, yp, gate, inv)
    want = M.combine(host(yp), gate, inv, T, k)
    err = row_rel_err(host(y), want)
    assert err <= (2.0 ** -8 if act == "bf16" else 1e-6), err
    # the same call again: the same bits (fixed slot order)
    assert torch.equal(y, _run(T, d, E, k, act, yp, gate, inv))


def test_combine_out_of_range_row_reads_row_zero_and_empty_batch():
    T, d, E, k = 40, 256, 8, 2
    yp, gate, inv = _case(T, d, E, k, "bf16", 5)
    inv = inv.copy()
    inv[3 * k + 1] = -7
    inv[5 * k] = T * k + 11
    y = _run(T, d, E, k, "bf16", yp, gate, inv)
    fixed = inv.copy()
    fixed[3 * k + 1] = 0
    fixed[5 * k] = 0
    want = M.combine(host(yp), gate, fixed, T, k)
    assert row_rel_err(host(y), want) <= 2.0 ** -8
    desc = api.make_desc(0, d, E, k, 256)
    api.moe_combine(desc, None, None, None, None)   # T = 0: nothing to do, no pointer read


def test_combine_rejects_missing_buffers():
    desc = api.make_desc(8, 256, 8, 2, 256)
    t = torch.zeros(16, 256, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(api.MoeError):
        api.moe_combine(desc, t, None, None, t)
