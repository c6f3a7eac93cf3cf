"""Serving-side decode windows on the GPU (gdn_decode_ex through the C ABI) vs the fp64 oracle:
slot-addressed states, grouped heads, KDA, fused gate activations and q/k normalisation,
verification of draft tokens and commit of the accepted ones."""
import numpy as np
import pytest
import torch

import oracle
from oracle import serving
from gated_deltanet_state_amd import synth
from helpers import check_streams, rel_l2, say, tol_for

pytestmark = pytest.mark.gpu


def setup_module(module):
    oracle.build(force=False)


def _cuda(d):
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def _ref(inp, *, kda, raw, write_state, n_commit=True, l2=None):
    pool = inp["pool"].double().numpy().copy()
    o = serving.decode_window(pool, inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"],
                              slots=inp["slots"], kda=kda, n_commit=inp["n_commit"] if n_commit else None,
                              write_state=write_state, qk_l2norm=raw if l2 is None else l2, raw_gates=raw,
                              A_log=inp["A_log"], dt_bias=inp["dt_bias"])
    return o, pool


def _live(inp):
    s = inp["slots"].numpy()
    return np.nonzero((s >= 0) & (s < inp["pool"].shape[0]))[0]


@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("kda,raw", [(False, False), (True, False), (False, True)])
def test_window_verify_then_commit(D, dtype, kda, raw):
    import gated_deltanet_state_amd as g
    N, T, H, Hqk, P = 7, 3, 4, 2, 12
    say(f"decode_ex D={D} dtype={dtype} kda={kda} raw={raw}")
    inp = synth.make_serving(N, T, H, Hqk, D, P, dtype, kda=kda, raw=raw, seed=D + 7 * kda + 13 * raw,
                             skip_every=3)
    d = _cuda(inp)
    kw = dict(slots=d["slots"], kda=kda, qk_l2norm=raw, A_log=d["A_log"], dt_bias=d["dt_bias"],
              out_dtype=torch.float32)
    live = _live(inp)
    # verification: outputs of every draft token, the pool untouched bit for bit
    pool0 = d["pool"].clone()
    o = torch.full((N, T, H, D), 7.0, device="cuda")
    g.gdn_decode_verify(d["pool"], d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], o=o, **kw)
    torch.cuda.synchronize()
    o_ref, _ = _ref(inp, kda=kda, raw=raw, write_state=False)
    assert torch.equal(d["pool"], pool0)
    skipped = np.setdiff1d(np.arange(N), live)
    assert bool((o[torch.as_tensor(skipped)] == 7.0).all())
    tol = 1e-5 if dtype == torch.float32 else 2e-3
    assert rel_l2(o[torch.as_tensor(live)], o_ref[live]) <= tol
    # commit of the accepted tokens: pool rows of live sequences advance, the others stay
    g.gdn_decode_commit(d["pool"], d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["n_commit"], **kw)
    torch.cuda.synchronize()
    _, pool_ref = _ref(inp, kda=kda, raw=raw, write_state=True)
    used = inp["slots"].numpy()[live]
    untouched = np.setdiff1d(np.arange(P), used)
    assert torch.equal(d["pool"][torch.as_tensor(untouched)], pool0[torch.as_tensor(untouched)])
    zero = used[inp["n_commit"].numpy()[live] == 0]
    if len(zero):
        assert torch.equal(d["pool"][torch.as_tensor(zero)], pool0[torch.as_tensor(zero)])
    assert rel_l2(d["pool"][torch.as_tensor(used)], pool_ref[used]) <= tol


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_window_equals_single_steps(dtype):
    """T = 1 windows through the slot table, repeated, equal one commit of the whole window
    on the GPU bit for bit, and match the plain decode step."""
    import gated_deltanet_state_amd as g
    N, T, H, D = 5, 4, 3, 128
    say(f"decode_ex single steps dtype={dtype}")
    inp = synth.make_serving(N, T, H, H, D, N, dtype, seed=5)
    d = _cuda(inp)
    a, b = d["pool"].clone(), d["pool"].clone()
    o_win = g.gdn_decode_ex(a, d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], out_dtype=torch.float32)
    steps = []
    for t in range(T):
        sl = lambda x: x[:, t:t + 1].contiguous()
        steps.append(g.gdn_decode_ex(b, sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["beta"]), sl(d["log_alpha"]),
                                     out_dtype=torch.float32))
    c = d["pool"].clone()
    o_step = [g.gdn_decode_step(c, d["q"][:, t].contiguous(), d["k"][:, t].contiguous(), d["v"][:, t].contiguous(),
                                d["beta"][:, t].contiguous(), d["log_alpha"][:, t].contiguous(),
                                out_dtype=torch.float32) for t in range(T)]
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(o_win, torch.cat(steps, 1))
    assert rel_l2(a, c) <= 1e-6 and rel_l2(o_win, torch.stack(o_step, 1)) <= 1e-6
    o_ref, pool_ref = _ref(dict(inp, slots=torch.arange(N, dtype=torch.int32)), kda=False, raw=False,
                           write_state=True, n_commit=False)
    assert rel_l2(o_win, o_ref) <= 1e-5 and rel_l2(a, pool_ref) <= 1e-5


def test_commit_zero_and_no_outputs():
    import gated_deltanet_state_amd as g
    N, T, H, D = 4, 2, 2, 32
    inp = synth.make_serving(N, T, H, H, D, 8, torch.bfloat16, seed=9)
    d = _cuda(inp)
    pool0 = d["pool"].clone()
    zeros = torch.zeros(N, dtype=torch.int32, device="cuda")
    g.gdn_decode_commit(d["pool"], d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], zeros, slots=d["slots"])
    torch.cuda.synchronize()
    assert torch.equal(d["pool"], pool0)


def _check_outputs(name, o_bf16, o_f32, o_ref):
    """Outputs [N, T, H, D] of a window against the oracle, per (sequence, value head).

    With bf16 outputs the whole tensor is held to the bf16 bound; a stream here has only
    T x 128 values, so its own error is dominated by the output rounding, whose worst case over
    8,192 streams reaches about 2.2e-3.  The per-stream bound is therefore taken on the fp32
    outputs of the same kernel, where the arithmetic (fp32 throughout) is the only error."""
    x, x32 = o_bf16.permute(0, 2, 1, 3), o_f32.permute(0, 2, 1, 3)
    r = np.transpose(o_ref, (0, 2, 1, 3))
    check_streams(name + " (bf16)", x, r, 2, 2e-3, 3e-3)
    check_streams(name + " (fp32)", x32, r, 2, 1e-4, 1e-4)


def test_verify_workload_full_size():
    """256 sequences x 32 value heads (16 query/key heads) x 128x128 states in a pool of 512,
    4 draft tokens with the raw gate projections and unnormalised q, k: verification then
    commit of the accepted tokens.  Every output of every sequence and every committed pool row
    against the oracle (whole tensor and worst (sequence, head)); every pool row no sequence
    addresses is unchanged bit for bit."""
    import gated_deltanet_state_amd as g
    c = synth.SERVING["verify"]
    say("decode_ex verify workload: 256 x 32 heads, T=4, pool 512")
    inp = synth.make_serving(c.N, c.T, c.H, c.Hqk, c.D, c.P, c.dtype, raw=True, s_std=c.s_std, seed=2001)
    d = _cuda(inp)
    kw = dict(slots=d["slots"], qk_l2norm=True, A_log=d["A_log"], dt_bias=d["dt_bias"])
    pool0 = d["pool"].clone()
    o = g.gdn_decode_verify(d["pool"], d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], **kw)
    o32 = g.gdn_decode_verify(d["pool"], d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], out_dtype=torch.float32,
                              **kw)
    torch.cuda.synchronize()
    o_ref, _ = _ref(inp, kda=False, raw=True, write_state=False)
    assert torch.equal(d["pool"], pool0)       # verification writes no state
    _check_outputs("verify o", o, o32, o_ref)
    g.gdn_decode_commit(d["pool"], d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["n_commit"], **kw)
    torch.cuda.synchronize()
    _, pool_ref = _ref(inp, kda=False, raw=True, write_state=True)
    rows = inp["slots"].numpy()
    check_streams("commit pool rows", d["pool"][torch.as_tensor(rows)], pool_ref[rows], 2, 1e-4, 1e-4)
    unused = np.setdiff1d(np.arange(c.P), rows)
    assert torch.equal(d["pool"][torch.as_tensor(unused)], pool0[torch.as_tensor(unused)])


def test_kda_step_workload_full_size():
    """KDA decode step on 256 sequences x 32 heads of 128x128 states (per-channel gates, one
    token): every output and every state against the oracle."""
    import gated_deltanet_state_amd as g
    c = synth.SERVING["kda"]
    say("decode_ex kda step workload: 256 x 32 heads, T=1")
    inp = synth.make_serving(c.N, c.T, c.H, c.Hqk, c.D, c.P, c.dtype, kda=True, s_std=c.s_std, seed=2002)
    d = _cuda(inp)
    o32 = g.gdn_decode_ex(d["pool"].clone(), d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], slots=d["slots"],
                          kda=True, out_dtype=torch.float32)
    o = g.gdn_decode_ex(d["pool"], d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], slots=d["slots"], kda=True)
    torch.cuda.synchronize()
    o_ref, pool_ref = _ref(dict(inp, n_commit=None), kda=True, raw=False, write_state=True, n_commit=False)
    _check_outputs("kda step o", o, o32, o_ref)
    rows = inp["slots"].numpy()
    check_streams("kda step pool rows", d["pool"][torch.as_tensor(rows)], pool_ref[rows], 2, 1e-4, 1e-4)


@pytest.mark.parametrize("T", [1, 2, 4, 5, 8, 9])
@pytest.mark.parametrize("kda,raw", [(False, False), (True, False), (False, True)])
def test_window_lengths_d128(T, kda, raw):
    """Windows of 1 to 9 tokens at d = 128, plain, KDA and with the fused prologue (verification
    of up to 8 tokens runs on the matrix cores, longer windows and commits token by token)."""
    import gated_deltanet_state_amd as g
    N, H, Hqk, D, P = 6, 4, 2, 128, 9
    say(f"decode_ex d128 T={T} kda={kda} raw={raw}")
    inp = synth.make_serving(N, T, H, Hqk, D, P, torch.float32, kda=kda, raw=raw, seed=40 + T + 3 * kda + 7 * raw,
                             skip_every=4)
    d = _cuda(inp)
    kw = dict(slots=d["slots"], kda=kda, qk_l2norm=raw, A_log=d["A_log"], dt_bias=d["dt_bias"])
    o = g.gdn_decode_verify(d["pool"], d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], **kw)
    g.gdn_decode_commit(d["pool"], d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["n_commit"], **kw)
    torch.cuda.synchronize()
    o_ref, _ = _ref(inp, kda=kda, raw=raw, write_state=False)
    _, pool_ref = _ref(inp, kda=kda, raw=raw, write_state=True)
    live = _live(inp)
    assert rel_l2(o[torch.as_tensor(live)], o_ref[live]) <= 1e-5
    assert rel_l2(d["pool"], pool_ref) <= 1e-5


@pytest.mark.parametrize("T", [3, 8])
def test_verify_l2norm_plain_gates_one_qk_head(T):
    """Verification with the q/k normalisation but plain gates, q and k rows far from unit
    length, all four value heads reading one query/key head, bf16 outputs."""
    import gated_deltanet_state_amd as g
    N, H, Hqk, D, P = 6, 4, 1, 128, 8
    say(f"decode_ex verify l2norm plain gates T={T}")
    inp = synth.make_serving(N, T, H, Hqk, D, P, torch.bfloat16, seed=70 + T, skip_every=5)
    inp["q"] = (inp["q"].float() * 2.5).to(torch.bfloat16)
    inp["k"] = (inp["k"].float() * 0.4).to(torch.bfloat16)
    d = _cuda(inp)
    o = g.gdn_decode_verify(d["pool"], d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], slots=d["slots"],
                            qk_l2norm=True, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16
    o_ref, _ = _ref(inp, kda=False, raw=False, write_state=False, l2=True)
    live = _live(inp)
    assert rel_l2(o[torch.as_tensor(live)], o_ref[live]) <= 2e-3
    # without the normalisation the same rows give other outputs
    o_raw = g.gdn_decode_verify(d["pool"], d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], slots=d["slots"],
                                out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert rel_l2(o_raw[torch.as_tensor(live)], o_ref[live]) > 1e-2


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_verify_misaligned_qk_views(dtype):
    """q and k, then v, passed as views one element past an aligned address (allowed by the
    ABI, which asks only for element alignment) give the same outputs as aligned copies, to
    rounding: such windows take the token loop instead of the matrix-core form."""
    import gated_deltanet_state_amd as g
    N, T, H, D, P = 5, 4, 2, 128, 6
    say(f"decode_ex verify misaligned q/k dtype={dtype}")
    inp = synth.make_serving(N, T, H, H, D, P, dtype, seed=91)
    d = _cuda(inp)

    def shifted(x):
        buf = torch.empty(x.numel() + 1, dtype=x.dtype, device=x.device)
        view = buf[1:].view(x.shape)
        view.copy_(x)
        return view

    qs, ks = shifted(d["q"]), shifted(d["k"])
    assert qs.data_ptr() % 16 != 0 and ks.data_ptr() % 16 != 0
    o_a = g.gdn_decode_verify(d["pool"], d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], out_dtype=torch.float32)
    o_m = g.gdn_decode_verify(d["pool"], qs, ks, d["v"], d["beta"], d["log_alpha"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, _ = _ref(dict(inp, slots=torch.arange(N, dtype=torch.int32)), kda=False, raw=False, write_state=False,
                    l2=False)
    tol = 1e-5 if dtype == torch.float32 else 2e-3
    assert rel_l2(o_m, o_ref) <= tol and rel_l2(o_a, o_ref) <= tol
    assert rel_l2(o_m, o_a) <= 1e-5
    vs = shifted(d["v"])
    assert vs.data_ptr() % 16 != 0
    o_v = g.gdn_decode_verify(d["pool"], d["q"], d["k"], vs, d["beta"], d["log_alpha"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert rel_l2(o_v, o_ref) <= tol and rel_l2(o_v, o_a) <= 1e-5


@pytest.mark.parametrize("D,T", [(16, 6), (128, 6), (128, 33)])
def test_commit_strong_decay_against_oracle(D, T):
    """Commit keeps the state as a running scale times rows and folds the scale in once the
    decays' product would fall below 2^-60.  Gates that cross that point at different tokens
    (log alpha -15 per token folds at the third; -50 folds at once; -30/-2 alternate; -0.01
    never folds; one token at -200, whose decay is 0 in fp32), every token committed, fp32
    inputs: pool rows against the oracle.  A window of 33 tokens folds many times along the
    way."""
    import gated_deltanet_state_amd as g
    N, H, Hqk, P = 5, 4, 2, 9
    say(f"commit strong decay D={D} T={T}")
    inp = synth.make_serving(N, T, H, Hqk, D, P, torch.float32, seed=71 + D)
    la = torch.empty(N, T, H)
    la[0] = -15.0
    la[1] = -0.05
    la[1, 0] = -50.0
    la[2, 0::2], la[2, 1::2] = -30.0, -2.0
    la[3] = -0.01
    la[4] = torch.linspace(-40.0, -1.0, T).view(T, 1)
    la[3, T // 2] = -200.0
    inp["log_alpha"] = la
    inp["n_commit"] = torch.full((N,), T, dtype=torch.int32)
    d = _cuda(inp)
    g.gdn_decode_commit(d["pool"], d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["n_commit"],
                        slots=d["slots"])
    torch.cuda.synchronize()
    _, pool_ref = _ref(inp, kda=False, raw=False, write_state=True)
    used = inp["slots"].numpy()[_live(inp)]
    for r in used:
        assert rel_l2(d["pool"][int(r)], pool_ref[int(r)]) <= 1e-5, r
