"""Prefill with grouped query/key heads and the raw gate projections (gdn_chunk_fwd_ex through
the C ABI, matrix-core kernel) vs the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from oracle import serving
from gated_deltanet_state_amd import synth
from helpers import rel_l2, say

pytestmark = pytest.mark.gpu


def setup_module(module):
    oracle.build(force=False)


def _cuda(d):
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


@pytest.mark.parametrize("T", [192, 200])
@pytest.mark.parametrize("raw", [False, True])
@pytest.mark.parametrize("out_f32", [False, True])
def test_chunk_ex_small(T, raw, out_f32):
    import gated_deltanet_state_amd as g
    B, H, Hqk, D = 2, 4, 2, 128
    say(f"chunk_ex T={T} raw={raw} out_f32={out_f32}")
    inp = synth.make_prefill_ex(B, H, Hqk, T, D, raw=raw, seed=T + raw)
    d = _cuda(inp)
    ck = 64 if T % 64 == 0 else 0
    o, sf, sc = g.gdn_chunk_fwd_ex(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["s0"], A_log=d["A_log"],
                                   dt_bias=d["dt_bias"], ckpt_every=ck,
                                   out_dtype=torch.float32 if out_f32 else None)
    torch.cuda.synchronize()
    o_ref, sf_ref, sc_ref = serving.forward_ex(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], inp["s0"],
                                               raw_gates=raw, A_log=inp["A_log"], dt_bias=inp["dt_bias"],
                                               ckpt_every=ck)
    assert rel_l2(o, o_ref) <= (1e-3 if out_f32 else 2e-3)
    assert rel_l2(sf, sf_ref) <= 2e-3
    if ck:
        assert rel_l2(sc, sc_ref) <= 2e-3


def test_chunk_ex_plain_is_chunk_fwd():
    """H_qk = H and no raw gates: bit-identical to gdn_chunk_fwd."""
    import gated_deltanet_state_amd as g
    inp = _cuda(synth.make_prefill(1, 4, 256, 128, 128, seed=3))
    a = g.gdn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], inp["s0"])
    b = g.gdn_chunk_fwd_ex(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], inp["s0"])
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_chunk_ex_grouped_32_16_heads():
    """The published 32 value / 16 query-key head layout, raw gates, T = 1024, all heads."""
    import gated_deltanet_state_amd as g
    B, H, Hqk, T, D = 1, 32, 16, 1024, 128
    say("chunk_ex 32/16 heads T=1024 raw gates")
    inp = synth.make_prefill_ex(B, H, Hqk, T, D, raw=True, seed=77)
    d = _cuda(inp)
    o, sf, _ = g.gdn_chunk_fwd_ex(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["s0"], A_log=d["A_log"],
                                  dt_bias=d["dt_bias"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, sf_ref, _ = serving.forward_ex(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], inp["s0"],
                                          raw_gates=True, A_log=inp["A_log"], dt_bias=inp["dt_bias"])
    assert rel_l2(o, o_ref) <= 1e-3
    assert rel_l2(sf, sf_ref) <= 2e-3
