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


@pytest.mark.parametrize("T", [64, 200])
@pytest.mark.parametrize("raw", [False, True])
@pytest.mark.parametrize("out_f32", [False, True])
def test_chunk_ex_l2norm(T, raw, out_f32):
    """Unnormalised q, k (the layer's projections, rows of length about 11) normalised in the
    kernel, against the oracle's normalisation in fp64."""
    import gated_deltanet_state_amd as g
    B, H, Hqk, D = 2, 4, 2, 128
    say(f"chunk_ex l2norm T={T} raw={raw} out_f32={out_f32}")
    inp = synth.make_prefill_ex(B, H, Hqk, T, D, raw=raw, unit=False, seed=300 + T + raw)
    d = _cuda(inp)
    o, sf, _ = g.gdn_chunk_fwd_ex(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["s0"], A_log=d["A_log"],
                                  dt_bias=d["dt_bias"], qk_l2norm=True,
                                  out_dtype=torch.float32 if out_f32 else None)
    torch.cuda.synchronize()
    o_ref, sf_ref, _ = serving.forward_ex(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], inp["s0"],
                                          raw_gates=raw, A_log=inp["A_log"], dt_bias=inp["dt_bias"],
                                          qk_l2norm=True)
    assert rel_l2(o, o_ref) <= (1e-3 if out_f32 else 2e-3)
    assert rel_l2(sf, sf_ref) <= 2e-3


def test_chunk_ex_l2norm_scale_invariant():
    """Scaling q and k rows by powers of two (exact in bf16) leaves the normalised prefill
    unchanged up to the epsilon, and the unnormalised one not."""
    import gated_deltanet_state_amd as g
    B, H, T, D = 1, 4, 256, 128
    inp = _cuda(synth.make_prefill_ex(B, H, H, T, D, unit=False, seed=31))
    gen = torch.Generator("cpu").manual_seed(5)
    sq = (2.0 ** torch.randint(-3, 4, (B, H, T, 1), generator=gen)).to(torch.bfloat16).cuda()
    sk = (2.0 ** torch.randint(-3, 4, (B, H, T, 1), generator=gen)).to(torch.bfloat16).cuda()
    run = lambda q, k, l2: g.gdn_chunk_fwd_ex(q, k, inp["v"], inp["beta"], inp["log_alpha"], inp["s0"],
                                              qk_l2norm=l2, out_dtype=torch.float32)
    a, b = run(inp["q"], inp["k"], True), run(inp["q"] * sq, inp["k"] * sk, True)
    torch.cuda.synchronize()
    # the epsilon and fp16 rounding of the normalised rows leave differences far below 1e-4
    assert rel_l2(a[0], b[0]) <= 1e-4 and rel_l2(a[1], b[1]) <= 1e-4
    # without the normalisation the outputs follow the scale of q (keys of unit length here:
    # unnormalised keys of length ~11 make the recurrence diverge)
    kf = inp["k"].float()
    kn = (kf / kf.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
    c, e = run(inp["q"] * sq, kn, False)[0], run(inp["q"], kn, False)[0]
    torch.cuda.synchronize()
    assert rel_l2(c, e) > 0.1


def test_chunk_ex_plain_is_chunk_fwd():
    """H_qk = H and no raw gates: bit-identical to gdn_chunk_fwd."""
    import gated_deltanet_state_amd as g
    inp = _cuda(synth.make_prefill(1, 4, 256, 128, 128, seed=3))
    a = g.gdn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], inp["s0"])
    b = g.gdn_chunk_fwd_ex(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], inp["s0"])
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("l2", [False, True])
def test_chunk_ex_grouped_32_16_heads(l2):
    """The published 32 value / 16 query-key head layout, raw gates (and, with l2, the q/k
    normalisation: the whole layer prologue), T = 1024, all heads."""
    import gated_deltanet_state_amd as g
    B, H, Hqk, T, D = 1, 32, 16, 1024, 128
    say(f"chunk_ex 32/16 heads T=1024 raw gates l2={l2}")
    inp = synth.make_prefill_ex(B, H, Hqk, T, D, raw=True, unit=not l2, seed=77)
    d = _cuda(inp)
    o, sf, _ = g.gdn_chunk_fwd_ex(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["s0"], A_log=d["A_log"],
                                  dt_bias=d["dt_bias"], qk_l2norm=l2, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, sf_ref, _ = serving.forward_ex(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], inp["s0"],
                                          raw_gates=True, A_log=inp["A_log"], dt_bias=inp["dt_bias"], qk_l2norm=l2)
    assert rel_l2(o, o_ref) <= 1e-3
    assert rel_l2(sf, sf_ref) <= 2e-3


@pytest.mark.parametrize("raw,l2", [(False, False), (True, False), (True, True)])
def test_ragged_batch(raw, l2):
    """Six sequences of lengths 130, 64, 1, 0, 200, 65 (ragged tails, a single token, an empty
    one) prefilled in one call; per-sequence outputs and final states against the oracle."""
    import gated_deltanet_state_amd as g
    lens = [130, 64, 1, 0, 200, 65]
    B, H, Hqk, D = len(lens), 4, 2, 128
    say(f"ragged batch raw={raw} l2={l2}")
    seqs = [synth.make_prefill_ex(1, H, Hqk, n, D, raw=raw, unit=not l2, seed=100 + i) for i, n in enumerate(lens)]
    cat = lambda key, heads: torch.cat([s_[key][0].reshape(heads * s_[key].shape[2], *s_[key].shape[3:])
                                        for s_ in seqs], 0)
    q, k, v = cat("q", Hqk), cat("k", Hqk), cat("v", H)
    beta, la = cat("beta", H), cat("log_alpha", H)
    s0 = torch.cat([s_["s0"] for s_ in seqs], 0)
    A_log, dt = seqs[0]["A_log"], seqs[0]["dt_bias"]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    o, sf = g.gdn_chunk_fwd_ragged(q.cuda(), k.cuda(), v.cuda(), beta.cuda(), la.cuda(), cu.cuda(), H=H, H_qk=Hqk,
                                   s0=s0.cuda(), A_log=None if A_log is None else A_log.cuda(),
                                   dt_bias=None if dt is None else dt.cuda(), qk_l2norm=l2,
                                   out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, sf_ref = serving.forward_ragged(q, k, v, beta, la, cu, H=H, Hqk=Hqk, s0=s0, raw_gates=raw,
                                           A_log=A_log, dt_bias=dt, qk_l2norm=l2)
    assert rel_l2(o, o_ref) <= 1e-3
    assert rel_l2(sf, sf_ref) <= 2e-3
    assert torch.equal(sf[3].cpu(), s0[3])   # the empty sequence keeps its state exactly


def test_ragged_equal_lengths_bitwise():
    """Equal lengths: the ragged call is the batched call, bit for bit."""
    import gated_deltanet_state_amd as g
    B, H, T, D = 3, 4, 192, 128
    inp = synth.make_prefill(B, H, T, D, D, seed=12)
    d = {k: v.cuda() for k, v in inp.items()}
    a = g.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["s0"])
    cu = torch.tensor([0, T, 2 * T, 3 * T], dtype=torch.int32, device="cuda")
    o, sf = g.gdn_chunk_fwd_ragged(d["q"].reshape(-1, D), d["k"].reshape(-1, D), d["v"].reshape(-1, D),
                                   d["beta"].reshape(-1), d["log_alpha"].reshape(-1), cu, H=H, s0=d["s0"])
    torch.cuda.synchronize()
    assert torch.equal(o.reshape(B, H, T, D), a[0]) and torch.equal(sf, a[1])


def test_ragged_bad_offsets_stay_in_bounds():
    """Offsets out of order are clamped: the call completes and the clamped sequences come out
    empty (state unchanged)."""
    import gated_deltanet_state_amd as g
    H, D, T = 2, 128, 128
    inp = synth.make_prefill(1, H, T, D, D, seed=13)
    d = {k: v.cuda() for k, v in inp.items()}
    s0 = torch.randn(3, H, D, D, device="cuda") * 0.01
    cu = torch.tensor([0, 100, 40, 10**6], dtype=torch.int32, device="cuda")   # 100 > 40, end past T
    o, sf = g.gdn_chunk_fwd_ragged(d["q"].reshape(-1, D), d["k"].reshape(-1, D), d["v"].reshape(-1, D),
                                   d["beta"].reshape(-1), d["log_alpha"].reshape(-1), cu, H=H, s0=s0)
    torch.cuda.synchronize()
    assert torch.equal(sf[1], s0[1])           # [100, 40) clamps to empty
    assert torch.isfinite(o).all() and torch.isfinite(sf).all()


def test_ragged_many_sequences_any_order():
    """40 sequences of seeded lengths 0..300 with ties (the kernel processes them longest
    first, each (sequence, head) stream exactly once): outputs and final states against the
    oracle, empty sequences keep their state."""
    import gated_deltanet_state_amd as g
    gen = torch.Generator("cpu").manual_seed(21)
    lens = [int(x) for x in torch.randint(0, 301, (40,), generator=gen)]
    lens[3] = lens[7] = lens[11] = 130   # ties
    lens[5] = 0
    B, H, Hqk, D = len(lens), 4, 2, 128
    say("ragged 40 sequences, longest first")
    seqs = [synth.make_prefill_ex(1, H, Hqk, n, D, seed=500 + i) for i, n in enumerate(lens)]
    cat = lambda key, heads: torch.cat([s_[key][0].reshape(heads * s_[key].shape[2], *s_[key].shape[3:])
                                        for s_ in seqs], 0)
    q, k, v = cat("q", Hqk), cat("k", Hqk), cat("v", H)
    beta, la = cat("beta", H), cat("log_alpha", H)
    s0 = torch.cat([s_["s0"] for s_ in seqs], 0)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    o, sf = g.gdn_chunk_fwd_ragged(q.cuda(), k.cuda(), v.cuda(), beta.cuda(), la.cuda(), cu.cuda(), H=H, H_qk=Hqk,
                                   s0=s0.cuda(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, sf_ref = serving.forward_ragged(q, k, v, beta, la, cu, H=H, Hqk=Hqk, s0=s0)
    assert rel_l2(o, o_ref) <= 1e-3
    assert rel_l2(sf, sf_ref) <= 2e-3
    assert torch.equal(sf[5].cpu(), s0[5])
    for b in (0, 17, 39):   # per sequence too: a stream swapped with another would show here
        assert rel_l2(sf[b], sf_ref[b]) <= 2e-3


@pytest.mark.parametrize("B,H,lo,hi", [(5, 3, 0, 200), (800, 2, 0, 5)])
def test_ragged_dispatch_orders(B, H, lo, hi):
    """B * H not a multiple of 8 (no XCD grouping of the slots) and B above the 768 sequences
    the kernel ranks by length (dispatch in argument order): every stream still lands once."""
    import gated_deltanet_state_amd as g
    gen = torch.Generator("cpu").manual_seed(B + H)
    lens = [int(x) for x in torch.randint(lo, hi + 1, (B,), generator=gen)]
    Hqk, D = 1, 128
    say(f"ragged B={B} H={H}")
    seqs = [synth.make_prefill_ex(1, H, Hqk, n, D, s0_std=0.05, seed=900 + i) for i, n in enumerate(lens)]
    cat = lambda key, heads: torch.cat([s_[key][0].reshape(heads * s_[key].shape[2], *s_[key].shape[3:])
                                        for s_ in seqs], 0)
    q, k, v = cat("q", Hqk), cat("k", Hqk), cat("v", H)
    beta, la = cat("beta", H), cat("log_alpha", H)
    s0 = torch.cat([s_["s0"] for s_ in seqs], 0)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    o, sf = g.gdn_chunk_fwd_ragged(q.cuda(), k.cuda(), v.cuda(), beta.cuda(), la.cuda(), cu.cuda(), H=H, H_qk=Hqk,
                                   s0=s0.cuda(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, sf_ref = serving.forward_ragged(q, k, v, beta, la, cu, H=H, Hqk=Hqk, s0=s0)
    assert rel_l2(o, o_ref) <= 1e-3
    assert rel_l2(sf, sf_ref) <= 2e-3
    worst = max(rel_l2(sf[b], sf_ref[b]) for b in range(B))   # a swapped stream would stand out
    assert worst <= 5e-3
