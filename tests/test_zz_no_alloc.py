"""The allocation-free KDA prefill (kda_chunk_fwd_noalloc, through the C ABI) against the
allocating entry point kda_chunk_fwd with its workspace: two calls in a row, the second smaller
than the first, each equal to kda_chunk_fwd bit for bit (the same kernels on the same operands;
slabs only change where the records live), and within tolerance of the oracle.  The first call
is larger than the 64 MiB scratch holds at once (2,048 records), so it runs slab by slab."""
import ctypes

import pytest
import torch

import oracle
from gated_deltanet_state_amd import synth
from helpers import TOL_BF16, rel_l2, say

pytestmark = pytest.mark.gpu


def _noalloc_cabi(g, d, o, sf, sc, every):
    B, H, T, D = d["q"].shape
    desc = g.GdnChunkDesc(B, H, T, D, D, 64, g.GDN_BF16, g.GDN_F32 if o.dtype == torch.float32 else g.GDN_BF16,
                          every)
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    st = g.lib.kda_chunk_fwd_noalloc(ctypes.byref(desc), p(d["q"]), p(d["k"]), p(d["v"]), p(d["beta"]),
                                     p(d["log_alpha"]), p(d["s0"]), p(o), p(sf), p(sc),
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == g.GDN_SUCCESS, g.gdn_status_string(st)


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_workspace_entry_point(order):
    import gated_deltanet_state_amd as g
    oracle.build(force=False)
    cases = [(2, 8, 8192, 0, torch.bfloat16), (1, 3, 700, 128, torch.float32)]
    for B, H, T, every, out_dt in cases:
        say(f"kda no-alloc B={B} H={H} T={T} every={every} out={out_dt}")
        inp = synth.make_prefill(B, H, T, 128, 128, torch.bfloat16, kda=True, s0_std=0.01, seed=300 + T)
        d = {k: v.cuda() for k, v in inp.items()}
        n_ck = T // every if every else 0
        o = torch.full((B, H, T, 128), float("nan"), dtype=out_dt, device="cuda")
        sf = torch.full((B, H, 128, 128), float("nan"), device="cuda")
        sc = torch.full((B, H, n_ck, 128, 128), float("nan"), device="cuda") if n_ck else None
        _noalloc_cabi(g, d, o, sf, sc, every)
        ref = g.kda_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["s0"], ckpt_every=every,
                              out_dtype=out_dt)
        torch.cuda.synchronize()
        assert torch.equal(o, ref[0]) and torch.equal(sf, ref[1])
        if n_ck:
            assert torch.equal(sc, ref[2])
        sel = [(0, 0), (B - 1, H - 1)]
        sub = {k: (torch.stack([v[b, h] for b, h in sel])[None].contiguous() if v is not None else None)
               for k, v in inp.items()}
        o_ref, s_ref, _ = oracle.forward(sub["q"], sub["k"], sub["v"], sub["beta"], sub["log_alpha"], sub["s0"],
                                         kda=True)
        eo = rel_l2(torch.stack([o[b, h] for b, h in sel])[None], o_ref)
        es = rel_l2(torch.stack([sf[b, h] for b, h in sel])[None], s_ref)
        print(f"no-alloc vs oracle: o {eo:.3e} s_final {es:.3e}", flush=True)
        assert eo <= TOL_BF16 and es <= 1e-3
