"""Decode step on the GPU vs the fp64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_state_amd import synth
from helpers import rel_l2, say, tol_for

pytestmark = pytest.mark.gpu


def setup_module(module):
    oracle.build(force=False)


@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("out_f32", [False, True])
def test_decode_small(D, dtype, out_f32):
    import gated_deltanet_state_amd as g
    N, H, steps = 5, 3, 6
    say(f"decode small D={D} dtype={dtype} out_f32={out_f32}")
    inp = synth.make_decode(N, H, D, D, steps, dtype, s_std=0.02, seed=D)
    st_gpu = inp["state"].clone().cuda()
    st_ref = inp["state"].double().numpy().copy()
    out_dt = torch.float32 if out_f32 else dtype
    for t in range(steps):
        args = [inp[n][t].contiguous() for n in ("q", "k", "v", "beta", "log_alpha")]
        o = g.gdn_decode_step(st_gpu, *[a.cuda() for a in args], out_dtype=out_dt)
        o_ref = oracle.decode_step(st_ref, *args)
        torch.cuda.synchronize()
        tol = 1e-5 if (out_f32 or dtype == torch.float32) else 2e-3
        assert rel_l2(o, o_ref) <= tol, (t, rel_l2(o, o_ref))
    assert rel_l2(st_gpu, st_ref) <= 1e-5


def test_decode_workload_full_size_sampled():
    """256 sequences x 32 heads x 128x128 fp32 states, 100 in-place steps; the oracle follows
    64 sampled (sequence, head) states through all steps (each state is independent)."""
    import gated_deltanet_state_amd as g
    c = synth.WORKLOADS[3]
    say("decode workload: 256x32 states, 100 steps")
    inp = synth.make_workload(3)
    rng = np.random.default_rng(0)
    pick = rng.choice(c.N * c.H, 64, replace=False)
    n_idx, h_idx = pick // c.H, pick % c.H
    st_ref = inp["state"][n_idx, h_idx].double().numpy()[:, None].copy()   # [64,1,D,D]
    st = inp["state"].cuda()
    dev_in = {k: inp[k].cuda() for k in ("q", "k", "v", "beta", "log_alpha")}
    errs = []
    for t in range(c.steps):
        o = g.gdn_decode_step(st, *(dev_in[k][t] for k in ("q", "k", "v", "beta", "log_alpha")))
        sel = [inp[k][t][n_idx, h_idx].unsqueeze(1).contiguous() for k in ("q", "k", "v", "beta", "log_alpha")]
        o_ref = oracle.decode_step(st_ref, *sel)
        errs.append(rel_l2(o[n_idx, h_idx].unsqueeze(1), o_ref))
    torch.cuda.synchronize()
    assert max(errs) <= 2e-3, max(errs)
    assert rel_l2(st[n_idx, h_idx].unsqueeze(1), st_ref) <= 2e-3


def test_decode_exact_overwrite_on_gpu():
    """beta = 1 with a unit key: after the step the state maps k to v (to fp32 rounding)."""
    import gated_deltanet_state_amd as g
    N, H, D = 8, 4, 128
    st = torch.randn(N, H, D, D, device="cuda") * 0.05
    k = torch.zeros(N, H, D, device="cuda")
    k[..., 3] = 1.0
    v = torch.randn(N, H, D, device="cuda")
    g.gdn_decode_step(st, torch.randn(N, H, D, device="cuda"), k, v, torch.ones(N, H, device="cuda"),
                      torch.full((N, H), -0.3, device="cuda"))
    torch.cuda.synchronize()
    assert torch.allclose(torch.einsum("nhvk,nhk->nhv", st, k), v, atol=1e-6)
