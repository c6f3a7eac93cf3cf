"""Pins of the fp64 oracle against what the pages and the mathematics fix (CPU only).

Each test names the passage it pins and the mistakes it would catch.  None of them
re-types the oracle's loop: they use the printed closed forms (evaluated in exact
rational arithmetic), printed worked examples and tables, special cases with a
textbook answer (the masked quadratic form of linear attention), and invariants.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def setup_module(module):
    oracle.build(force=False)


# --------------------------------------------------------------------------- helpers
def _fr_matmul(A, B):
    n, m, p = len(A), len(B), len(B[0])
    return [[sum((A[i][t] * B[t][j] for t in range(m)), Fraction(0)) for j in range(p)] for i in range(n)]


def _fr_add(A, B):
    return [[a + b for a, b in zip(ra, rb)] for ra, rb in zip(A, B)]


def _fr_scale(c, A):
    return [[c * a for a in r] for r in A]


def _fr_eye(n):
    return [[Fraction(int(i == j)) for j in range(n)] for i in range(n)]


def _fr_outer(u, w):
    return [[a * b for b in w] for a in u]


def _dyadic(rng, shape, denom=8, lo=-8, hi=8):
    """Random dyadic rationals (exact in fp64 and in bf16 when |num| < 256)."""
    return rng.integers(lo, hi + 1, size=shape).astype(np.float64) / denom


def _rel(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(np.asarray(b)), 1e-300))


# --------------------------------------------------------------------------- p1: rational brute force
@pytest.mark.parametrize("kda", [False, True])
def test_rational_bruteforce_closed_form(kda):
    """Closed forms evaluated exactly in rationals.

    GDN: S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T, o_t = S_t q_t
    ("Hybrid models: what Gated DeltaNet replaces in the KV cache", section "Gated
    DeltaNet: add decay"; read from the updated state per "From Traditional Attention to
    hybrid ones", section 5).  KDA: S_t = S_{t-1} Diag(alpha_t)(I - beta_t k_t k_t^T) +
    beta_t v_t k_t^T (same page, section 7).
    Catches: decay applied after the correction, reading the pre-update state, beta on
    the wrong term, a transposed state (d_v != d_k and a non-symmetric S0), KDA decaying
    rows instead of columns.
    """
    rng = np.random.default_rng(7 + int(kda))
    Dk, Dv, T = 3, 2, 6
    q = _dyadic(rng, (1, 1, T, Dk))
    k = _dyadic(rng, (1, 1, T, Dk))
    v = _dyadic(rng, (1, 1, T, Dv))
    beta = rng.integers(1, 8, size=(1, 1, T)).astype(np.float64) / 8
    la = -rng.uniform(0.01, 0.4, size=(1, 1, T, Dk) if kda else (1, 1, T))
    s0 = _dyadic(rng, (1, 1, Dv, Dk))
    o, sf, _ = oracle.forward(q, k, v, beta, la, s0, kda=kda)

    # exact rational evaluation; alpha is the exact binary value of the fp64 exp(log alpha)
    S = [[Fraction(float(x)) for x in row] for row in s0[0, 0]]
    o_exact = []
    for t in range(T):
        kt = [Fraction(float(x)) for x in k[0, 0, t]]
        qt = [Fraction(float(x)) for x in q[0, 0, t]]
        vt = [Fraction(float(x)) for x in v[0, 0, t]]
        bt = Fraction(float(beta[0, 0, t]))
        erase = _fr_add(_fr_eye(Dk), _fr_scale(-bt, _fr_outer(kt, kt)))
        if kda:
            a = [Fraction(math.exp(float(x))) for x in la[0, 0, t]]
            decay = [[a[i] if i == j else Fraction(0) for j in range(Dk)] for i in range(Dk)]
            S = _fr_add(_fr_matmul(_fr_matmul(S, decay), erase), _fr_scale(bt, _fr_outer(vt, kt)))
        else:
            a = Fraction(math.exp(float(la[0, 0, t])))
            S = _fr_add(_fr_scale(a, _fr_matmul(S, erase)), _fr_scale(bt, _fr_outer(vt, kt)))
        o_exact.append([sum((S[i][j] * qt[j] for j in range(Dk)), Fraction(0)) for i in range(Dv)])
    o_ref = np.array([[float(x) for x in r] for r in o_exact])
    s_ref = np.array([[float(x) for x in r] for r in S])
    assert _rel(o[0, 0], o_ref) < 1e-13
    assert _rel(sf[0, 0], s_ref) < 1e-13


# --------------------------------------------------------------------------- p2: exact overwrite
@pytest.mark.parametrize("kda", [False, True])
def test_exact_overwrite_unit_key(kda):
    """beta_t = 1 and a unit-length key give S_t k_t = v_t, whatever the gate.

    "Attention, Part 4", section 4 (the delta rule: with beta_t = 1 and a unit-length key,
    reading right after writing returns exactly v_t); "Hybrid attention", section "Writing
    with the delta rule".  Catches: reading with the undecayed state (then S_t k_t != v_t
    whenever alpha_t < 1), a missing or doubled beta, a wrong sign of the correction.
    """
    rng = np.random.default_rng(11)
    B, H, T, Dk, Dv = 1, 3, 12, 8, 5
    # unit keys exactly representable: signed, permuted (0.6, 0.8, 0, ...)
    k = np.zeros((B, H, T, Dk))
    for h in range(H):
        for t in range(T):
            i, j = rng.choice(Dk, 2, replace=False)
            k[0, h, t, i] = 0.6 * rng.choice([-1, 1])
            k[0, h, t, j] = 0.8 * rng.choice([-1, 1])
    q = rng.standard_normal((B, H, T, Dk))
    v = rng.standard_normal((B, H, T, Dv))
    beta = np.ones((B, H, T))
    la = -rng.uniform(0.005, 0.5, size=(B, H, T, Dk) if kda else (B, H, T))
    s0 = rng.standard_normal((B, H, Dv, Dk))
    _, _, ck = oracle.forward(q, k, v, beta, la, s0, kda=kda, ckpt_every=1)
    for h in range(H):
        for t in range(T):
            read = ck[0, h, t] @ k[0, h, t]
            np.testing.assert_allclose(read, v[0, h, t], rtol=0, atol=1e-13)


def test_exact_overwrite_decode_step():
    """Same pin on the single-token decode step."""
    rng = np.random.default_rng(12)
    N, H, Dk, Dv = 4, 2, 8, 6
    k = np.zeros((N, H, Dk))
    for n in range(N):
        for h in range(H):
            k[n, h, (n + h) % Dk] = -1.0
    state = rng.standard_normal((N, H, Dv, Dk))
    v = rng.standard_normal((N, H, Dv))
    oracle.decode_step(state, rng.standard_normal((N, H, Dk)), k, v, np.ones((N, H)),
                       -rng.uniform(0.01, 0.3, (N, H)))
    np.testing.assert_allclose(np.einsum("nhvk,nhk->nhv", state, k), v, rtol=0, atol=1e-13)


# --------------------------------------------------------------------------- p5: no change
def test_no_change_when_state_already_maps_k_to_v():
    """alpha_t = 1 and v_t = S_{t-1} k_t leave the state unchanged.

    "Hybrid models...", section "The delta rule: write the correction, not the sum" (if the
    state already maps k_t to v_t, nothing changes); "From Traditional Attention...",
    section 4 (DeltaNet writes only the prediction error).  Catches: an additive write
    (linear attention) and a wrong sign of the retrieved value.
    """
    rng = np.random.default_rng(5)
    B, H, T, Dk, Dv = 2, 2, 9, 6, 4
    s0 = rng.standard_normal((B, H, Dv, Dk))
    k = rng.standard_normal((B, H, T, Dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = np.einsum("bhvk,bhtk->bhtv", s0, k)
    q = rng.standard_normal((B, H, T, Dk))
    beta = rng.uniform(0.05, 1.0, (B, H, T))
    o, sf, _ = oracle.forward(q, k, v, beta, np.zeros((B, H, T)), s0)
    np.testing.assert_allclose(sf, s0, rtol=0, atol=1e-14)
    np.testing.assert_allclose(o, np.einsum("bhvk,bhtk->bhtv", s0, q), rtol=0, atol=1e-13)


# --------------------------------------------------------------------------- p3: forget only
@pytest.mark.parametrize("kda", [False, True])
def test_beta_zero_only_forgets(kda):
    """beta_t = 0: the state only decays -- S_T = (prod alpha) S_0 (GDN), S_0 Diag(prod alpha) (KDA);
    with alpha = 1 as well it does not change at all and o_t = S_0 q_t.

    "Attention, Part 4", section 6 (if alpha_t = 1 it is the plain delta rule; if
    beta_t = 0 it only forgets); section 7 for the per-channel rates.
    Catches: decay on the wrong axis for KDA (rows instead of key channels), a write
    that ignores beta, a missing decay.
    """
    rng = np.random.default_rng(3)
    B, H, T, Dk, Dv = 1, 2, 17, 5, 3
    q = rng.standard_normal((B, H, T, Dk))
    k = rng.standard_normal((B, H, T, Dk))
    v = rng.standard_normal((B, H, T, Dv))
    s0 = rng.standard_normal((B, H, Dv, Dk))
    la = -rng.uniform(0.005, 0.2, (B, H, T, Dk) if kda else (B, H, T))
    _, sf, _ = oracle.forward(q, k, v, np.zeros((B, H, T)), la, s0, kda=kda)
    tot = np.exp(la.sum(axis=2))
    expect = s0 * tot[:, :, None, :] if kda else s0 * tot[:, :, None, None]
    np.testing.assert_allclose(sf, expect, rtol=1e-13, atol=0)

    o, sf, _ = oracle.forward(q, k, v, np.zeros((B, H, T)), np.zeros(la.shape), s0, kda=kda)
    np.testing.assert_array_equal(sf, s0)
    np.testing.assert_allclose(o, np.einsum("bhvk,bhtk->bhtv", s0, q), rtol=0, atol=1e-13)


# --------------------------------------------------------------------------- p7: decay table
def test_decay_table_golden():
    """Printed alpha^t table: with beta = 0 and a constant gate, ||S_t|| / ||S_0|| = alpha^t.

    Fixture: tests/golden/decay_table.txt ("Attention, Part 4", section 5).  Catches: an
    off-by-one snapshot index (alpha^9 vs alpha^10 differ in the third decimal), a gate
    applied as exp(-log alpha) or twice per token.
    """
    rows = [l.split() for l in open(os.path.join(GOLDEN, "decay_table.txt")) if l.strip() and l[0] != "#"]
    table = {}
    for a, t, s in rows:
        table.setdefault(float(a), {})[int(t)] = float(s)
    alphas = sorted(table)
    T = 500
    rng = np.random.default_rng(1)
    Dk = Dv = 4
    H = len(alphas)
    s0 = rng.standard_normal((1, H, Dv, Dk))
    la = np.stack([np.full(T, math.log(a)) for a in alphas])[None]
    z = np.zeros((1, H, T, Dk))
    _, _, ck = oracle.forward(z, z, np.zeros((1, H, T, Dv)), np.zeros((1, H, T)), la, s0, ckpt_every=10)
    for h, a in enumerate(alphas):
        for t, printed in table[a].items():
            st = s0[0, h] if t == 0 else ck[0, h, t // 10 - 1]
            ratio = np.linalg.norm(st) / np.linalg.norm(s0[0, h])
            assert f"{ratio:.3f}" == f"{printed:.3f}", (a, t, ratio, printed)


# --------------------------------------------------------------------------- p6: worked example
def test_overwrite_worked_example_golden():
    """x = 1, y = 7, x = 5 with perpendicular keys: the delta rule reads back x = 5, y = 7.

    Fixture: tests/golden/overwrite_xy.txt ("Attention, Part 4", section 3, Test 1).  The
    linear-attention row of the fixture is checked against the plain sum of outer products
    (section 2 of the same page), which shows the fixture is read correctly.
    """
    rows = {l.split()[0]: tuple(map(float, l.split()[1:])) for l in
            open(os.path.join(GOLDEN, "overwrite_xy.txt")) if l.strip() and l[0] != "#"}
    ex, ey = np.array([1.0, 0.0]), np.array([0.0, 1.0])
    keys = np.stack([ex, ey, ex])[None, None]
    vals = np.array([1.0, 7.0, 5.0]).reshape(1, 1, 3, 1)
    _, sf, _ = oracle.forward(keys, keys, vals, np.ones((1, 1, 3)), np.zeros((1, 1, 3)))
    x, y = sf[0, 0] @ ex, sf[0, 0] @ ey
    assert (round(float(x[0]), 2), round(float(y[0]), 2)) == rows["delta"]
    lin = sum(np.outer(vals[0, 0, t], keys[0, 0, t]) for t in range(3))
    assert (round(float((lin @ ex)[0]), 2), round(float((lin @ ey)[0]), 2)) == rows["linear"]


# --------------------------------------------------------------------------- p4: masked quadratic form
@pytest.mark.parametrize("gated", [False, True])
def test_reduction_to_masked_quadratic_form(gated):
    """With S0 = 0 and mutually orthonormal keys the erase term never fires, so the gated
    delta rule is unnormalised linear attention with values beta_t v_t: in parallel form
    O = (tril(Q K^T) * D) diag(beta) V, D[t, j] = prod_{s=j+1..t} alpha_s (D = 1 when ungated),
    and with beta = 1 it is exactly plain linear attention O = tril(Q K^T) V.

    Plain linear attention S_t = S_{t-1} + v_t k_t^T, o_t = S_t q_t ("From Traditional
    Attention...", section 1, the linear case) and its masked quadratic (parallel) form
    ("Attention, Part 4", section 2, "Proof: the two forms give the same answer";
    "Hybrid attention", section "Attention without the softmax").
    Catches: exclusive vs inclusive causal mask (reading before the write), a missing
    beta, a gate applied to the current token's own write, a transposed score matrix.
    """
    rng = np.random.default_rng(21 + int(gated))
    H, T, D = 2, 24, 32
    Qm, _ = np.linalg.qr(rng.standard_normal((H, D, D)))
    k = np.transpose(Qm, (0, 2, 1))[:, :T][None]             # T orthonormal rows per head
    q = rng.standard_normal((1, H, T, D))
    v = rng.standard_normal((1, H, T, D))
    for beta in (np.ones((1, H, T)), rng.uniform(0.1, 1.0, (1, H, T))):
        la = -rng.uniform(0.005, 0.3, (1, H, T)) if gated else np.zeros((1, H, T))
        o, _, _ = oracle.forward(q, k, v, beta, la)
        for h in range(H):
            scores = np.tril(q[0, h] @ k[0, h].T)
            c = np.concatenate([[0.0], np.cumsum(la[0, h])])
            Dm = np.exp(c[1:, None] - c[None, 1:])           # prod_{s=j+1..t} alpha_s
            par = (scores * Dm) @ (beta[0, h][:, None] * v[0, h])
            np.testing.assert_allclose(o[0, h], par, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------- p8: KDA with equal gates
def test_kda_with_equal_channel_gates_is_gdn():
    """KDA with the same rate on every key channel is Gated DeltaNet ("Attention, Part 4",
    section 7: everything as in Gated DeltaNet except alpha_t is a vector)."""
    rng = np.random.default_rng(9)
    B, H, T, Dk, Dv = 2, 2, 20, 6, 5
    q, k = rng.standard_normal((B, H, T, Dk)), rng.standard_normal((B, H, T, Dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, H, T, Dv))
    beta = rng.uniform(0, 1, (B, H, T))
    g = -rng.uniform(0.005, 0.2, (B, H, T))
    s0 = rng.standard_normal((B, H, Dv, Dk))
    a = oracle.forward(q, k, v, beta, g, s0, ckpt_every=5)
    b = oracle.forward(q, k, v, beta, np.repeat(g[..., None], Dk, -1), s0, kda=True, ckpt_every=5)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


# --------------------------------------------------------------------------- snapshots, decode, widening
def test_snapshot_n_is_state_after_n_times_every():
    """Snapshot n holds the state after token n * ckpt_every ("Hybrid models...", section
    "What a recurrent state changes for serving", item 1: a snapshot taken at N); the last
    snapshot of a whole multiple equals the final state."""
    rng = np.random.default_rng(4)
    B, H, T, D = 1, 2, 48, 8
    q, k, v = (rng.standard_normal((B, H, T, D)) for _ in range(3))
    beta, la = rng.uniform(0, 1, (B, H, T)), -rng.uniform(0, 0.2, (B, H, T))
    s0 = rng.standard_normal((B, H, D, D))
    _, sf, ck = oracle.forward(q, k, v, beta, la, s0, ckpt_every=16)
    assert ck.shape == (B, H, 3, D, D)
    np.testing.assert_array_equal(ck[:, :, -1], sf)
    for n in (1, 2):
        _, sfn, _ = oracle.forward(q[:, :, :16 * n], k[:, :, :16 * n], v[:, :, :16 * n],
                                   beta[:, :, :16 * n], la[:, :, :16 * n], s0)
        np.testing.assert_array_equal(ck[:, :, n - 1], sfn)


@pytest.mark.parametrize("kda", [False, True])
def test_decode_steps_equal_forward(kda):
    """T single-token steps from S0 give the forward pass's outputs and final state (the
    recurrent form is how the layer writes text one token at a time: "Hybrid attention",
    section "Attention without the softmax")."""
    rng = np.random.default_rng(8)
    B, H, T, Dk, Dv = 2, 3, 7, 6, 4
    q, k = rng.standard_normal((B, H, T, Dk)), rng.standard_normal((B, H, T, Dk))
    v = rng.standard_normal((B, H, T, Dv))
    beta = rng.uniform(0, 1, (B, H, T))
    la = -rng.uniform(0, 0.2, (B, H, T, Dk) if kda else (B, H, T))
    s0 = rng.standard_normal((B, H, Dv, Dk))
    o, sf, _ = oracle.forward(q, k, v, beta, la, s0, kda=kda)
    st = s0.copy()
    for t in range(T):
        ot = oracle.decode_step(st, q[:, :, t].copy(), k[:, :, t].copy(), v[:, :, t].copy(),
                                beta[:, :, t].copy(), la[:, :, t].copy(), kda=kda)
        np.testing.assert_array_equal(ot, o[:, :, t])
    np.testing.assert_array_equal(st, sf)


def test_bf16_and_fp32_inputs_widen_exactly():
    """The oracle reads bf16 / fp32 storage as the exact same values as their fp64 widening
    (torch's conversion), so it sees bit-for-bit what the GPU is given."""
    g = torch.Generator().manual_seed(0)
    shp = (1, 2, 10, 8)
    for dt in (torch.bfloat16, torch.float32):
        q, k, v = (torch.randn(*shp, generator=g).to(dt) for _ in range(3))
        beta = torch.rand(1, 2, 10, generator=g).to(dt)
        la = (-0.2 * torch.rand(1, 2, 10, generator=g)).to(dt)
        a = oracle.forward(q, k, v, beta, la)
        b = oracle.forward(*(x.double().numpy() for x in (q, k, v, beta, la)))
        np.testing.assert_array_equal(a[0], b[0])
        np.testing.assert_array_equal(a[1], b[1])
