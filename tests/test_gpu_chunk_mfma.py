"""Matrix-core chunkwise prefill (bf16 inputs, d = 128, chunk 64) vs the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_state_amd import synth
from helpers import TOL_BF16, rel_l2, say

pytestmark = pytest.mark.gpu


def setup_module(module):
    oracle.build(force=False)


def _gpu(kda, inp, ckpt_every=0, out_dtype=None, **kw):
    import gated_deltanet_state_amd as g
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    fn = g.kda_chunk_fwd if kda else g.gdn_chunk_fwd
    r = fn(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["s0"], chunk=64, ckpt_every=ckpt_every,
           out_dtype=out_dtype, **kw)
    torch.cuda.synchronize()
    return r


def _ref(kda, inp, ckpt_every=0):
    return oracle.forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], inp["s0"], kda=kda,
                          ckpt_every=ckpt_every)


@pytest.mark.parametrize("T", [1, 64, 200, 1000])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_gdn_mfma_small(T, out_dtype):
    say(f"mfma gdn T={T} out={out_dtype}")
    inp = synth.make_prefill(1, 3, T, 128, 128, torch.bfloat16, s0_std=0.01, seed=T)
    o, sf, _ = _gpu(False, inp, out_dtype=out_dtype)
    o_ref, s_ref, _ = _ref(False, inp)
    eo, es = rel_l2(o, o_ref), rel_l2(sf, s_ref)
    print(f"rel-L2 o={eo:.3e} s_final={es:.3e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16
    if out_dtype == torch.float32:
        assert eo <= 1e-3  # compute error alone (fp16 operands, fp32 accumulation)


def test_gdn_mfma_zero_initial_state_and_empty():
    import gated_deltanet_state_amd as g
    say("mfma gdn s0=None, T=0")
    inp = synth.make_prefill(2, 2, 130, 128, 128, torch.bfloat16, s0_std=0.0, seed=3)
    o, sf, _ = _gpu(False, inp)
    o_ref, s_ref, _ = _ref(False, inp)
    assert rel_l2(o, o_ref) <= TOL_BF16 and rel_l2(sf, s_ref) <= TOL_BF16
    e = synth.make_prefill(1, 2, 0, 128, 128, torch.bfloat16, s0_std=0.01, seed=4)
    o, sf, _ = _gpu(False, e)
    assert o.shape == (1, 2, 0, 128) and torch.equal(sf.cpu(), e["s0"])


def test_gdn_mfma_in_place_and_deterministic():
    import gated_deltanet_state_amd as g
    say("mfma gdn in-place/determinism")
    inp = synth.make_prefill(2, 4, 300, 128, 128, torch.bfloat16, s0_std=0.01, seed=5)
    d = {k: v.cuda() for k, v in inp.items()}
    args = [d[k] for k in ("q", "k", "v", "beta", "log_alpha")]
    o1, s1, _ = g.gdn_chunk_fwd(*args, d["s0"], chunk=64)
    o2, s2, _ = g.gdn_chunk_fwd(*args, d["s0"], chunk=64)
    s = d["s0"].clone()
    o3, _, _ = g.gdn_chunk_fwd(*args, s, chunk=64, s_final=s)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)       # bitwise run to run
    assert torch.equal(o1, o3) and torch.equal(s1, s)        # in place == out of place


def test_gdn_mfma_snapshots_and_resume():
    import gated_deltanet_state_amd as g
    say("mfma gdn snapshots/resume")
    T, every = 640, 128
    inp = synth.make_prefill(1, 2, T, 128, 128, torch.bfloat16, s0_std=0.01, seed=6)
    o, sf, sc = _gpu(False, inp, ckpt_every=every, out_dtype=torch.float32)
    o_ref, s_ref, c_ref = _ref(False, inp, ckpt_every=every)
    assert sc.shape == (1, 2, 5, 128, 128)
    assert rel_l2(sc, c_ref) <= TOL_BF16
    assert torch.equal(sc[:, :, -1], sf)
    # resume from snapshot 2 (after token 384): identical chunk alignment -> bitwise equal
    tail = {k: (v[:, :, 384:].contiguous() if k != "s0" else None) for k, v in inp.items()}
    tail["s0"] = sc[:, :, 2].cpu()
    o2, sf2, _ = _gpu(False, tail, out_dtype=torch.float32)
    assert torch.equal(o2, o[:, :, 384:]) and torch.equal(sf2, sf)


def test_gdn_mfma_matches_decode_steps():
    """T decode steps and one prefill agree (within the bf16 tolerance)."""
    import gated_deltanet_state_amd as g
    say("mfma gdn vs decode steps")
    T = 96
    inp = synth.make_prefill(1, 2, T, 128, 128, torch.bfloat16, s0_std=0.01, seed=7)
    o, sf, _ = _gpu(False, inp, out_dtype=torch.float32)
    st = inp["s0"].cuda().clone()
    outs = []
    for t in range(T):
        outs.append(g.gdn_decode_step(st, *(inp[k][:, :, t].contiguous().cuda()
                                            for k in ("q", "k", "v", "beta", "log_alpha")),
                                      out_dtype=torch.float32))
    torch.cuda.synchronize()
    od = torch.stack(outs, 2)
    assert rel_l2(o, od) <= TOL_BF16 and rel_l2(sf, st) <= TOL_BF16


def test_workload_prefill_full_size():
    """B=4, H=16, T=4096, d=128, chunk 64, bf16; S0 = 0.01 N(0,1): all outputs and final states."""
    c = synth.WORKLOADS[1]
    say("prefill workload B=4 H=16 T=4096")
    inp = synth.make_workload(1)
    o, sf, _ = _gpu(False, inp)
    o_ref, s_ref, _ = _ref(False, inp)
    eo, es = rel_l2(o, o_ref), rel_l2(sf, s_ref)
    print(f"prefill workload rel-L2 o={eo:.3e} s_final={es:.3e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16


def test_workload_long_prefill_snapshots_sampled_heads():
    """B=1, H=32, T=65536 with a snapshot every 8192 tokens: the oracle follows 3 sampled
    heads through the whole sequence (heads are independent); snapshot 8 equals the final
    state bitwise."""
    c = synth.WORKLOADS[2]
    say("long prefill workload H=32 T=65536, 8 snapshots")
    inp = synth.make_workload(2)
    o, sf, sc = _gpu(False, inp, ckpt_every=c.ckpt_every)
    assert sc.shape == (1, 32, 8, 128, 128)
    assert torch.equal(sc[:, :, -1], sf)
    heads = [0, 13, 31]
    sub = {k: (v[:, heads].contiguous() if v is not None else None) for k, v in inp.items()}
    o_ref, s_ref, c_ref = _ref(False, sub, ckpt_every=c.ckpt_every)
    eo = rel_l2(o[:, heads], o_ref)
    es = rel_l2(sf[:, heads], s_ref)
    ec = rel_l2(sc[:, heads], c_ref)
    print(f"long prefill rel-L2 o={eo:.3e} s_final={es:.3e} snapshots={ec:.3e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16 and ec <= TOL_BF16


# ------------------------------------------------------------------ KDA (per-channel decay)
@pytest.mark.parametrize("T", [1, 64, 200, 1000])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_kda_mfma_small(T, out_dtype):
    say(f"mfma kda T={T} out={out_dtype}")
    inp = synth.make_prefill(1, 3, T, 128, 128, torch.bfloat16, kda=True, s0_std=0.01, seed=50 + T)
    o, sf, _ = _gpu(True, inp, out_dtype=out_dtype)
    o_ref, s_ref, _ = _ref(True, inp)
    eo, es = rel_l2(o, o_ref), rel_l2(sf, s_ref)
    print(f"kda rel-L2 o={eo:.3e} s_final={es:.3e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16
    if out_dtype == torch.float32:
        assert eo <= 1e-3


def test_kda_mfma_equal_channel_gates_match_gdn():
    """KDA with the same rate on every key channel is the gated delta rule ("Attention,
    Part 4", section 7): the two matrix-core kernels agree to within the bf16 tolerance."""
    say("mfma kda == gdn for equal gates")
    inp = synth.make_prefill(2, 2, 300, 128, 128, torch.bfloat16, s0_std=0.01, seed=61)
    kinp = dict(inp)
    kinp["log_alpha"] = inp["log_alpha"][..., None].expand(2, 2, 300, 128).contiguous()
    o1, s1, _ = _gpu(False, inp, out_dtype=torch.float32)
    o2, s2, _ = _gpu(True, kinp, out_dtype=torch.float32)
    assert rel_l2(o2, o1) <= 1e-3 and rel_l2(s2, s1) <= 1e-3


def test_kda_mfma_strong_gates():
    """log alpha in [-1.2, -0.5] per channel: e^{-G} reaches e^{77} inside a 64-token chunk,
    far beyond half precision; the per-block reference points keep every operand bounded."""
    say("mfma kda strong gates")
    inp = synth.make_prefill(1, 2, 256, 128, 128, torch.bfloat16, kda=True, s0_std=0.01, seed=62,
                             log_alpha_range=(-1.2, -0.5))
    o, sf, _ = _gpu(True, inp, out_dtype=torch.float32)
    o_ref, s_ref, _ = _ref(True, inp)
    assert torch.isfinite(o).all() and torch.isfinite(sf).all()
    assert rel_l2(o, o_ref) <= TOL_BF16 and rel_l2(sf, s_ref) <= TOL_BF16


def test_kda_mfma_snapshots_resume_empty():
    import gated_deltanet_state_amd as g
    say("mfma kda snapshots/resume/empty")
    T, every = 448, 128
    inp = synth.make_prefill(1, 2, T, 128, 128, torch.bfloat16, kda=True, s0_std=0.01, seed=63)
    o, sf, sc = _gpu(True, inp, ckpt_every=every, out_dtype=torch.float32)
    o_ref, s_ref, c_ref = _ref(True, inp, ckpt_every=every)
    assert sc.shape == (1, 2, 3, 128, 128) and rel_l2(sc, c_ref) <= TOL_BF16
    tail = {k: (v[:, :, 256:].contiguous() if k != "s0" else None) for k, v in inp.items()}
    tail["s0"] = sc[:, :, 1].cpu()
    o2, sf2, _ = _gpu(True, tail, out_dtype=torch.float32)
    assert torch.equal(o2, o[:, :, 256:]) and torch.equal(sf2, sf)
    e = synth.make_prefill(1, 2, 0, 128, 128, torch.bfloat16, kda=True, s0_std=0.01, seed=64)
    o, sf, _ = _gpu(True, e)
    assert o.shape == (1, 2, 0, 128) and torch.equal(sf.cpu(), e["s0"])


@pytest.mark.parametrize("T,every", [(200, 0), (256, 64), (1, 0), (1000, 0), (1984, 320)])
def test_kda_two_kernel_form_is_the_single_kernel(T, every):
    """With its workspace the KDA prefill computes every chunk's state-independent tiles in a
    separate parallel kernel; the sequential kernel then runs the same arithmetic on the same
    operands, so outputs, final state and snapshots equal the single kernel's bit for bit."""
    import gated_deltanet_state_amd as g
    say(f"kda two-kernel form T={T} every={every}")
    inp = synth.make_prefill(2, 3, T, 128, 128, torch.bfloat16, kda=True, s0_std=0.01, seed=70 + T)
    d = {k: v.cuda() for k, v in inp.items()}
    need = g.gdn_chunk_workspace_size(2, 3, T, 128, kda=True, ckpt_every=every)
    assert need == 2 * 3 * ((T + 63) // 64) * 65536
    ws = torch.full((need,), 0xAB, dtype=torch.uint8, device="cuda")   # stale bytes must not matter
    run = lambda w: g.kda_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["s0"], ckpt_every=every,
                                    out_dtype=torch.float32, workspace=w)
    a, b = run(False), run(ws)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    if every:
        assert torch.equal(a[2], b[2])
    with pytest.raises(g.GdnError):   # a workspace that is too small is refused
        run(ws[:need - 16])


def test_workload_kda_full_size_sampled_heads():
    """B=2, H=32, T=8192, d=128, chunk 64, bf16, per-channel gates: the oracle follows 3
    sampled (batch, head) streams through the whole sequence."""
    say("kda workload B=2 H=32 T=8192")
    inp = synth.make_workload(4)
    o, sf, _ = _gpu(True, inp)
    sel = [(0, 0), (0, 17), (1, 31)]
    sub = {k: (torch.stack([v[b, h] for b, h in sel])[None].contiguous() if v is not None else None)
           for k, v in inp.items()}
    o_ref, s_ref, _ = _ref(True, sub)
    og = torch.stack([o[b, h] for b, h in sel])[None]
    sg = torch.stack([sf[b, h] for b, h in sel])[None]
    eo, es = rel_l2(og, o_ref), rel_l2(sg, s_ref)
    print(f"kda workload rel-L2 o={eo:.3e} s_final={es:.3e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16
