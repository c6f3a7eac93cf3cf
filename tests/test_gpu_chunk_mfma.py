"""Matrix-core chunkwise prefill (bf16 inputs, d = 128, chunk 64) vs the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_state_amd import synth
from helpers import TOL_BF16, check_streams, rel_l2, say

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
    """B=4, H=16, T=4096, d=128, chunk 64, bf16; S0 = 0.01 N(0,1): every output and final state
    of all 64 streams against the oracle, with bf16 outputs (the workload's) and with fp32
    outputs (the kernel's own error, without the output rounding).  Whole-tensor and
    worst-stream relative L2 errors are both bounded."""
    say("prefill workload B=4 H=16 T=4096")
    inp = synth.make_workload(1)
    o_ref, s_ref, _ = _ref(False, inp)
    for out_dtype, tol in ((torch.bfloat16, TOL_BF16), (torch.float32, 1e-3)):
        say(f"prefill workload out={out_dtype}")
        o, sf, _ = _gpu(False, inp, out_dtype=out_dtype)
        check_streams(f"prefill o ({out_dtype})", o, o_ref, 2, tol, tol)
        check_streams(f"prefill s_final ({out_dtype})", sf, s_ref, 2, 1e-3, 1e-3)
        del o, sf


def test_workload_long_prefill_snapshots_all_heads():
    """B=1, H=32, T=65536 with a snapshot every 8192 tokens: all 32 heads through the whole
    sequence against the oracle (outputs, the 8 snapshots of every head, final states), bf16
    and fp32 outputs; snapshot 8 equals the final state bitwise."""
    c = synth.WORKLOADS[2]
    say("long prefill workload H=32 T=65536, 8 snapshots")
    inp = synth.make_workload(2)
    o_ref, s_ref, c_ref = _ref(False, inp, ckpt_every=c.ckpt_every)
    for out_dtype, tol in ((torch.bfloat16, TOL_BF16), (torch.float32, 1e-3)):
        say(f"long prefill out={out_dtype}")
        o, sf, sc = _gpu(False, inp, ckpt_every=c.ckpt_every, out_dtype=out_dtype)
        assert sc.shape == (1, 32, 8, 128, 128)
        assert torch.equal(sc[:, :, -1], sf)
        check_streams(f"long prefill o ({out_dtype})", o, o_ref, 2, tol, tol)
        check_streams(f"long prefill s_final ({out_dtype})", sf, s_ref, 2, 1e-3, 1e-3)
        check_streams(f"long prefill snapshots ({out_dtype})", sc, c_ref, 3, 1e-3, 1e-3)
        del o, sf, sc
        torch.cuda.empty_cache()


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
    operands, so outputs, final state and snapshots equal the single kernel's bit for bit.  The
    same holds slab by slab, for workspaces that hold only some of the records (streams split
    into groups, chunks into consecutive slabs with the state carried between them)."""
    import gated_deltanet_state_amd as g
    say(f"kda two-kernel form T={T} every={every}")
    inp = synth.make_prefill(2, 3, T, 128, 128, torch.bfloat16, kda=True, s0_std=0.01, seed=70 + T)
    d = {k: v.cuda() for k, v in inp.items()}
    need = g.gdn_chunk_workspace_size(2, 3, T, 128, kda=True, ckpt_every=every)
    assert need == 2 * 3 * ((T + 63) // 64) * 65536
    ws = torch.full((need,), 0xAB, dtype=torch.uint8, device="cuda")   # stale bytes must not matter
    run = lambda w: g.kda_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["s0"], ckpt_every=every,
                                    out_dtype=torch.float32, workspace=w)
    a = run(False)
    rec = 65536
    sizes = [need] + [n * rec for n in (2, 3, 7, 13) if n * rec < need]
    for nb in sizes:
        b = run(torch.full((nb,), 0xCD, dtype=torch.uint8, device="cuda"))
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]), nb
        if every:
            assert torch.equal(a[2], b[2]), nb
    with pytest.raises(g.GdnError):   # a workspace under two records is refused
        run(ws[:2 * rec - 16])


@pytest.mark.parametrize("form", ["two_kernel", "single_kernel"])
def test_workload_kda_full_size(form):
    """B=2, H=32, T=8192, d=128, chunk 64, bf16, per-channel gates: all 64 streams against the
    oracle, in the two-kernel form (with its workspace, as benchmarked) and the single kernel,
    bf16 and fp32 outputs; whole-tensor and worst-stream relative L2 errors bounded."""
    say(f"kda workload B=2 H=32 T=8192 ({form})")
    inp = synth.make_workload(4)
    o_ref, s_ref, _ = _kda_workload_ref(inp)
    ws = None if form == "two_kernel" else False
    for out_dtype, tol in ((torch.bfloat16, TOL_BF16), (torch.float32, 1e-3)):
        say(f"kda workload {form} out={out_dtype}")
        o, sf, _ = _gpu(True, inp, out_dtype=out_dtype, workspace=ws)
        check_streams(f"kda o ({form}, {out_dtype})", o, o_ref, 2, tol, tol)
        check_streams(f"kda s_final ({form}, {out_dtype})", sf, s_ref, 2, 1e-3, 1e-3)
        del o, sf


_KDA_REF = {}


def _kda_workload_ref(inp):
    if "r" not in _KDA_REF:
        _KDA_REF["r"] = _ref(True, inp)
    return _KDA_REF["r"]


@pytest.mark.parametrize("handle", [False, True])
def test_side_stream_binding_allocations(handle):
    """Work enqueued on a stream other than torch's current one: the KDA prefill (its workspace
    and outputs allocated by the binding) and a decode step give the current-stream results bit
    for bit, while the current stream allocates and overwrites memory of the same size (the
    binding marks what it allocated as used by the side stream, so none of it is handed out
    again before the side stream's kernels are done).  The stream is passed as a torch stream
    or as a raw hipStream_t handle."""
    import gated_deltanet_state_amd as g
    say(f"side stream (raw handle={handle})")
    inp = synth.make_prefill(2, 3, 1000, 128, 128, torch.bfloat16, kda=True, s0_std=0.01, seed=81)
    d = {k: v.cuda() for k, v in inp.items()}
    args = [d[k] for k in ("q", "k", "v", "beta", "log_alpha", "s0")]
    o_ref, s_ref, _ = g.kda_chunk_fwd(*args, out_dtype=torch.float32)
    dec = synth.make_decode(64, 8, 128, 128, 1, torch.bfloat16, seed=82)
    st_ref = dec["state"].cuda()
    dargs = [dec[k][0].cuda() for k in ("q", "k", "v", "beta", "log_alpha")]
    od_ref = g.gdn_decode_step(st_ref, *dargs)
    need = g.gdn_chunk_workspace_size(2, 3, 1000, 128, kda=True)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    st = dec["state"].cuda()
    side.wait_stream(torch.cuda.current_stream())
    s_arg = side.cuda_stream if handle else side
    o, sf, _ = g.kda_chunk_fwd(*args, out_dtype=torch.float32, stream=s_arg)
    od = g.gdn_decode_step(st, *dargs, stream=s_arg)
    for _ in range(4):   # the current stream churns through blocks of the workspace's size
        x = torch.empty(need, dtype=torch.uint8, device="cuda")
        x.fill_(0x5A)
        y = torch.empty(o.numel() * 4, dtype=torch.uint8, device="cuda")
        y.fill_(0xA5)
        del x, y
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(sf, s_ref)
    assert torch.equal(od, od_ref) and torch.equal(st, st_ref)


def _kda_gates(B, H, T, seed, spec):
    """Per-channel log-gates [B, H, T, 128] for the strong-gate tests (bf16 values)."""
    g = torch.Generator("cpu").manual_seed(seed)
    la = torch.rand(B, H, T, 128, generator=g) * 0.195 - 0.2          # the usual U[-0.2, -0.005]
    if spec == "all_strong":                                           # every channel in [-4, -1]
        la = torch.rand(B, H, T, 128, generator=g) * 3.0 - 4.0
    elif spec == "few_channels_minus8":                                # 5 channels at -8
        la[..., [3, 40, 77, 100, 127]] = -8.0
    elif spec == "strong_chunks":                                      # every other chunk in [-4, -1]
        for c0 in range(0, T, 128):
            la[:, :, c0:c0 + 64] = torch.rand(B, H, min(64, T - c0), 128, generator=g) * 3.0 - 4.0
    elif spec == "extreme":                                            # down to -80 per token
        la[..., 0::16] = -80.0
        la[..., 5::16] = -30.0
        la[:, :, 100:140, 64:] = -12.0
    return la.to(torch.bfloat16)


@pytest.mark.parametrize("spec", ["all_strong", "few_channels_minus8", "strong_chunks", "extreme"])
@pytest.mark.parametrize("form", ["two_kernel", "single_kernel"])
def test_kda_mfma_any_gate_strength(spec, form):
    """Per-channel gates far beyond what the middle-token split of a 16-token block can hold in
    half precision ("Hybrid Linear Attention Architecture Design Explained", section 4: the
    division form needs overflow protection).  Those blocks are flagged, their rows take the
    block start as reference and their diagonal tiles are formed exactly, so the results stay
    finite and match the oracle for any finite log alpha <= 0."""
    say(f"kda any gate strength: {spec} ({form})")
    B, H, T = 1, 3, 300
    inp = synth.make_prefill(B, H, T, 128, 128, torch.bfloat16, kda=True, s0_std=0.01, seed=90)
    inp["log_alpha"] = _kda_gates(B, H, T, 91, spec)
    ws = None if form == "two_kernel" else False
    o_ref, s_ref, _ = _ref(True, inp)
    for out_dtype, tol in ((torch.float32, 1e-3), (torch.bfloat16, TOL_BF16)):
        o, sf, _ = _gpu(True, inp, out_dtype=out_dtype, workspace=ws)
        assert torch.isfinite(o).all() and torch.isfinite(sf).all()
        eo, es = rel_l2(o, o_ref), rel_l2(sf, s_ref)
        print(f"kda {spec} {form} out={out_dtype}: rel-L2 o={eo:.3e} s_final={es:.3e}")
        assert eo <= tol and es <= 1e-3


def test_kda_mfma_large_rows_flagged():
    """Queries of length 1000 (elements up to ~300) with gates that keep the middle-token
    factors below e^8 (log alpha in [-0.95, -0.85]) but would push rows times factors past
    half range: the magnitude check flags those blocks too, and the outputs (about 1000 times
    the usual size) stay finite and match the oracle."""
    say("kda large rows")
    B, H, T = 1, 2, 192
    inp = synth.make_prefill(B, H, T, 128, 128, torch.bfloat16, kda=True, s0_std=0.01, seed=92,
                             log_alpha_range=(-0.95, -0.85))
    inp["q"] = (inp["q"].float() * 1000.0).to(torch.bfloat16)
    o_ref, s_ref, _ = _ref(True, inp)
    for ws in (None, False):
        o, sf, _ = _gpu(True, inp, out_dtype=torch.float32, workspace=ws)
        assert torch.isfinite(o).all() and torch.isfinite(sf).all()
        eo, es = rel_l2(o, o_ref), rel_l2(sf, s_ref)
        print(f"kda large rows ws={ws}: rel-L2 o={eo:.3e} s_final={es:.3e}")
        assert eo <= 1e-3 and es <= 1e-3
