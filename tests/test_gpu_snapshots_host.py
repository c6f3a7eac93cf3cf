"""Snapshots written straight into pinned host memory by the prefill kernels (s_ckpt on the
host): the same bits as snapshots in device memory, on the matrix-core, KDA, vector and
grouped-head paths, checked against the fp64 oracle once; pageable host memory is refused
before anything is launched."""
import ctypes

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


def _both(fn, d, every, **kw):
    """Run fn with device snapshots and with host snapshots; return both snapshot tensors
    (the host ones read after a stream synchronisation) and the two final states."""
    a = fn(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["s0"], ckpt_every=every, **kw)
    b = fn(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["s0"], ckpt_every=every, snapshots_to_host=True, **kw)
    torch.cuda.synchronize()
    assert b[2].device.type == "cpu" and b[2].is_pinned()
    return a, b


@pytest.mark.parametrize("path", ["mfma", "kda", "valu"])
def test_host_snapshots_equal_device(path):
    import gated_deltanet_state_amd as g
    say(f"host snapshots {path}")
    if path == "valu":
        inp = synth.make_prefill(2, 3, 96, 16, 16, torch.float32, seed=41)
        every, fn, kw = 32, g.gdn_chunk_fwd, dict(chunk=16)
    else:
        inp = synth.make_prefill(1, 4, 1024, 128, 128, kda=path == "kda", seed=42)
        every, fn, kw = 256, (g.kda_chunk_fwd if path == "kda" else g.gdn_chunk_fwd), {}
    d = {k: v.cuda() for k, v in inp.items()}
    a, b = _both(fn, d, every, **kw)
    assert torch.equal(a[2].cpu(), b[2]) and torch.equal(a[1], b[1]) and torch.equal(a[0], b[0])
    if path == "mfma":
        _, _, c_ref = oracle.forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], inp["s0"],
                                     ckpt_every=every)
        assert rel_l2(b[2], c_ref) <= 2e-3


def test_host_snapshots_grouped_heads():
    """gdn_chunk_fwd_ex (32 value / 16 query-key heads, raw gates, in-kernel q/k normalisation)
    with host snapshots every 128 tokens, against the oracle."""
    import gated_deltanet_state_amd as g
    B, H, Hqk, T, D = 1, 8, 4, 512, 128
    say("host snapshots grouped heads")
    inp = synth.make_prefill_ex(B, H, Hqk, T, D, raw=True, unit=False, seed=43)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    a, b = _both(g.gdn_chunk_fwd_ex, d, 128, A_log=d["A_log"], dt_bias=d["dt_bias"], qk_l2norm=True)
    assert torch.equal(a[2].cpu(), b[2])
    _, _, c_ref = serving.forward_ex(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], inp["s0"],
                                     raw_gates=True, A_log=inp["A_log"], dt_bias=inp["dt_bias"], qk_l2norm=True,
                                     ckpt_every=128)
    assert rel_l2(b[2], c_ref) <= 2e-3


def test_pageable_host_snapshots_refused():
    """A pageable host buffer as s_ckpt: the binding refuses it, and so does the C ABI (its
    runtime pointer query reports unregistered memory) before launching anything."""
    import gated_deltanet_state_amd as g
    inp = {k: v.cuda() for k, v in synth.make_prefill(1, 2, 256, 128, 128, seed=44).items()}
    pageable = torch.empty(1, 2, 2, 128, 128)
    with pytest.raises(ValueError):
        g.gdn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], inp["s0"], ckpt_every=128,
                        s_ckpt=pageable)
    buf = np.zeros(2 * 2 * 128 * 128 + 16, np.float32)
    addr = (buf.ctypes.data + 15) // 16 * 16
    o = torch.empty_like(inp["v"])
    d = g._desc(1, 2, 256, 128, 64, torch.bfloat16, torch.bfloat16, 128)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = g.lib.gdn_chunk_fwd(ctypes.byref(d), p(inp["q"]), p(inp["k"]), p(inp["v"]), p(inp["beta"]),
                             p(inp["log_alpha"]), p(inp["s0"]), p(o), None, ctypes.c_void_p(addr), None, 0, None)
    torch.cuda.synchronize()
    assert st == g.GDN_ERROR_INVALID_VALUE
    assert not buf.any()
