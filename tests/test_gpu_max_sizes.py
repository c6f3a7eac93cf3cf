"""The largest stream the matrix-core prefill accepts: T = 4,194,240 tokens at d = 128, just
under the 2 GiB that one stream's q/k/v (and fp32 o) may span for the 32-bit buffer offsets.

With beta = 0 the delta correction vanishes and the recurrence only decays the state, so
every output has a closed form at any length:
    GDN:  o_t = e^{G_t} S0 q_t,              G_t = sum_{s<=t} log alpha_s
    KDA:  o_t = S0 Diag(e^{G_t}) q_t,        G_t per key channel
and the snapshots and the final state are the decayed S0.  The log-gates are constant per
token (per channel for KDA), so G_t = (t + 1) c exactly.  Outputs are checked on sampled
tokens spread over the whole stream (chunk starts, chunk ends, the last token).

The decode kernels are checked the same way over a 16 GiB state pool, whose rows lie past
2^32 bytes: with beta = 0 a step is S <- alpha S and o = alpha S q."""
import numpy as np
import pytest
import torch

from helpers import rel_l2, say

pytestmark = pytest.mark.gpu

D = 128
T_MAX = ((2**31 - 1) // (D * 4)) // 64 * 64   # 4,194,240: largest multiple of 64 with T*D*4 < 2^31


def _sample_tokens(T):
    picks = {0, 1, 63, 64, 65, 4095, 4096, 2**20 - 1, 2**20, 2**21 + 7, 3 * 2**20 + 64, T - 65, T - 64, T - 1}
    rng = np.random.default_rng(5)
    picks |= set(int(x) for x in rng.integers(0, T, 40))
    return np.array(sorted(picks))


def _inputs(kda, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    q = torch.randn(1, 1, T_MAX, D, generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn(1, 1, T_MAX, D, generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn(1, 1, T_MAX, D, generator=g, device="cuda").to(torch.bfloat16)
    beta = torch.zeros(1, 1, T_MAX, dtype=torch.bfloat16, device="cuda")
    if kda:   # one small rate per channel: the decay over the whole stream spans e^-0.4 .. e^-4.6
        c = (-1e-7 * (1.0 + 10.0 * torch.arange(D, device="cuda") / D)).to(torch.bfloat16)
        log_alpha = c.view(1, 1, 1, D).expand(1, 1, T_MAX, D).contiguous()
    else:
        c = torch.tensor([-5e-7], device="cuda").to(torch.bfloat16)
        log_alpha = c.expand(1, 1, T_MAX).contiguous()
    s0 = torch.randn(1, 1, D, D, generator=g, device="cuda")
    return q, k, v, beta, log_alpha, s0, c.double().cpu().numpy()


def _decay(c, t):
    """e^{G_t} for token index t (G_t = (t + 1) c), fp64: a scalar (GDN) or one per channel."""
    return np.exp((t + 1) * c)


@pytest.mark.parametrize("kda", [False, True])
def test_prefill_longest_stream_closed_form(kda):
    import gated_deltanet_state_amd as g
    say(f"longest stream T={T_MAX} kda={kda}")
    q, k, v, beta, log_alpha, s0, c = _inputs(kda, seed=17 + kda)
    every = 2**20
    fn = g.kda_chunk_fwd if kda else g.gdn_chunk_fwd
    o, sf, sc = fn(q, k, v, beta, log_alpha, s0, chunk=64, ckpt_every=every, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert o.shape == (1, 1, T_MAX, D) and sc.shape == (1, 1, T_MAX // every, D, D)

    S0 = s0[0, 0].double().cpu().numpy()
    ts = _sample_tokens(T_MAX)
    qs = q[0, 0, torch.as_tensor(ts, device="cuda")].double().cpu().numpy()   # [n, D]
    dec = np.stack([_decay(c, t) for t in ts]) if kda else np.array([_decay(c, t) for t in ts])
    if kda:   # o_t = S0 (e^{G_t} * q_t)
        o_ref = (dec.reshape(len(ts), D) * qs) @ S0.T
    else:     # o_t = e^{G_t} S0 q_t
        o_ref = dec.reshape(-1, 1) * (qs @ S0.T)
    o_got = o[0, 0, torch.as_tensor(ts, device="cuda")]
    e_o = rel_l2(o_got, o_ref)

    def state_at(t):   # state after token t: S0 decayed by e^{G_t}
        d = _decay(c, t)
        return S0 * d.reshape(1, D) if kda else S0 * float(np.asarray(d).reshape(-1)[0])

    e_f = rel_l2(sf[0, 0], state_at(T_MAX - 1))
    e_c = max(rel_l2(sc[0, 0, n], state_at((n + 1) * every - 1)) for n in range(T_MAX // every))
    print(f"rel-L2 o={e_o:.3e} s_final={e_f:.3e} snapshots={e_c:.3e}")
    assert e_o <= 2e-3 and e_f <= 2e-3 and e_c <= 2e-3


# ------------------------------------------------------------------ decode over a 16 GiB state pool
def _big_pool(P, H, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randn(P, H, D, D, generator=g, device="cuda"), g


def test_decode_step_16gib_pool_closed_form():
    """262,144 states of 128x128 fp32 (16 GiB, offsets past 2^32 bytes), beta = 0: the step
    decays every state, S <- alpha S, and o = alpha S q; checked on sampled states."""
    import gated_deltanet_state_amd as g
    N, H = 4096, 64
    say(f"decode step over {N * H} states")
    state, gen = _big_pool(N, H, seed=23)
    q = torch.randn(N, H, D, generator=gen, device="cuda").to(torch.bfloat16)
    k = torch.randn(N, H, D, generator=gen, device="cuda").to(torch.bfloat16)
    v = torch.randn(N, H, D, generator=gen, device="cuda").to(torch.bfloat16)
    beta = torch.zeros(N, H, dtype=torch.bfloat16, device="cuda")
    la = (-0.3 * torch.rand(N, H, generator=gen, device="cuda")).to(torch.bfloat16)
    pick = [(0, 0), (1, 63), (2047, 31), (4095, 63), (4095, 0), (3000, 17)]
    before = {p: state[p].double().cpu().numpy() for p in pick}
    o = g.gdn_decode_step(state, q, k, v, beta, la, out_dtype=torch.float32)
    torch.cuda.synchronize()
    for p in pick:
        a = float(np.exp(float(la[p])))
        S1 = a * before[p]
        assert rel_l2(state[p], S1) <= 1e-6, p
        assert rel_l2(o[p], S1 @ q[p].double().cpu().numpy()) <= 1e-5, p


def test_verify_and_commit_16gib_pool_closed_form():
    """Windows of 4 tokens through a slot table into a 16 GiB pool (rows past 2^32 bytes),
    beta = 0: verification gives o_t = e^{G_t} S q_t, commit of m tokens leaves e^{G_{m-1}} S."""
    import gated_deltanet_state_amd as g
    P, H, N, T = 4096, 64, 64, 4
    say(f"verify/commit over a pool of {P * H} states")
    pool, gen = _big_pool(P, H, seed=29)
    slots = torch.randperm(P, generator=gen, device="cuda")[:N].to(torch.int32)
    slots[0], slots[1] = P - 1, P - 2   # the last rows of the pool
    q = torch.randn(N, T, H, D, generator=gen, device="cuda").to(torch.bfloat16)
    k = torch.randn(N, T, H, D, generator=gen, device="cuda").to(torch.bfloat16)
    v = torch.randn(N, T, H, D, generator=gen, device="cuda").to(torch.bfloat16)
    beta = torch.zeros(N, T, H, dtype=torch.bfloat16, device="cuda")
    la = (-0.2 * torch.rand(N, T, H, generator=gen, device="cuda")).to(torch.bfloat16)
    n_commit = torch.randint(0, T + 1, (N,), generator=gen, device="cuda").to(torch.int32)
    seqs = [0, 1, 17, 63]
    rows = slots.cpu().numpy()
    before = {n: pool[int(rows[n])].double().cpu().numpy() for n in seqs}      # [H, D, D]
    o = g.gdn_decode_verify(pool, q, k, v, beta, la, slots=slots, out_dtype=torch.float32)
    g.gdn_decode_commit(pool, q, k, v, beta, la, n_commit, slots=slots)
    torch.cuda.synchronize()
    G = torch.cumsum(la.double(), 1).cpu().numpy()                           # [N, T, H]
    qn = q.double().cpu().numpy()
    for n in seqs:
        for h in (0, 33, 63):
            S = before[n][h]
            o_ref = np.stack([np.exp(G[n, t, h]) * (S @ qn[n, t, h]) for t in range(T)])
            assert rel_l2(o[n, :, h], o_ref) <= 1e-5, (n, h)
            m = int(n_commit[n])
            S_ref = S * (np.exp(G[n, m - 1, h]) if m > 0 else 1.0)
            assert rel_l2(pool[int(rows[n]), h], S_ref) <= 1e-6, (n, h, m)
