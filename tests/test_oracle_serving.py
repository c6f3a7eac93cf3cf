"""Pins of the serving-path oracle (oracle/serving.py) against closed forms and against the
independent token loop of oracle.forward.  CPU only."""
import math

import numpy as np
import pytest

import oracle
from oracle import serving


def test_gates_closed_forms():
    # sigmoid(0) = 1/2; softplus(0) = ln 2; softplus(ln(e - 1)) = 1; exp(A_log = 0) = 1
    b = np.array([[0.0, 40.0, -40.0]])
    a = np.array([[0.0, math.log(math.e - 1.0), 0.0]])
    A_log = np.array([0.0, 0.0, math.log(3.0)])
    dt = np.array([0.0, 0.0, 0.0])
    beta, g = serving.gates_from_raw(b, a, A_log, dt)
    assert beta[0, 0] == 0.5
    assert abs(beta[0, 1] - 1.0) < 1e-15 and beta[0, 2] < 1e-17
    assert abs(g[0, 0] + math.log(2.0)) < 1e-15          # -1 * ln 2
    assert abs(g[0, 1] + 1.0) < 1e-15                    # -1 * 1
    assert abs(g[0, 2] + 3.0 * math.log(2.0)) < 1e-14    # -3 * ln 2
    # dt_bias shifts the softplus argument; large arguments are linear, never overflow
    _, g2 = serving.gates_from_raw(np.zeros(2), np.array([1000.0, -1.0]), np.zeros(2), np.array([0.0, 1.0]))
    assert abs(g2[0] + 1000.0) < 1e-9 and abs(g2[1] + math.log(2.0)) < 1e-15


def test_gates_always_forget():
    rng = np.random.default_rng(0)
    beta, g = serving.gates_from_raw(rng.normal(0, 5, (50, 8)), rng.normal(0, 5, (50, 8)),
                                     rng.normal(0, 2, 8), rng.normal(0, 2, 8))
    assert np.all((beta > 0) & (beta < 1)) and np.all(g < 0)
    assert np.all(np.exp(g) < 1)


def test_l2_normalize_closed_forms():
    x = np.array([[3.0, 4.0], [0.0, 0.0], [0.0, -2.0]])
    y = serving.l2_normalize(x)
    assert np.allclose(y[0], [0.6, 0.8], atol=2e-7)
    assert np.all(y[1] == 0.0)
    assert np.allclose(y[2], [0.0, -1.0], atol=1e-6)
    r = np.random.default_rng(1).normal(0, 1, (20, 128))
    assert np.allclose(np.linalg.norm(serving.l2_normalize(r), axis=-1), 1.0, atol=1e-8)


def _window_inputs(rng, N, T, H, Hqk, D, kda=False):
    q = rng.normal(0, 1, (N, T, Hqk, D))
    k = rng.normal(0, 1, (N, T, Hqk, D))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.normal(0, 1, (N, T, H, D))
    beta = 1.0 / (1.0 + np.exp(-rng.normal(0, 1, (N, T, H))))
    la = rng.uniform(-0.2, -0.005, (N, T, H, D) if kda else (N, T, H))
    return q, k, v, beta, la


@pytest.mark.parametrize("kda", [False, True])
def test_window_matches_forward(kda):
    """A window of T decode steps equals the forward token loop started from the same state
    (different code path: ora_forward), for outputs and the final state."""
    rng = np.random.default_rng(2)
    N, T, H, D = 3, 5, 2, 8
    q, k, v, beta, la = _window_inputs(rng, N, T, H, H, D, kda)
    pool = rng.normal(0, 0.1, (N, H, D, D))
    ref_o, ref_s, _ = oracle.forward(q.transpose(0, 2, 1, 3).copy(), k.transpose(0, 2, 1, 3).copy(),
                                     v.transpose(0, 2, 1, 3).copy(), beta.transpose(0, 2, 1).copy(),
                                     (la.transpose(0, 2, 1, 3) if kda else la.transpose(0, 2, 1)).copy(),
                                     pool.copy(), kda=kda)
    p = pool.copy()
    o = serving.decode_window(p, q, k, v, beta, la, kda=kda)
    assert np.allclose(o, ref_o.transpose(0, 2, 1, 3), rtol=0, atol=1e-13)
    assert np.allclose(p, ref_s, rtol=0, atol=1e-13)


def test_grouped_heads_read_their_key_head():
    """Value head h uses query/key head h // (H / Hqk): equal to the ungrouped window on
    inputs with each query/key head repeated for its value heads."""
    rng = np.random.default_rng(3)
    N, T, H, Hqk, D = 2, 3, 4, 2, 8
    q, k, v, beta, la = _window_inputs(rng, N, T, H, Hqk, D)
    pool = rng.normal(0, 0.1, (N, H, D, D))
    p1, p2 = pool.copy(), pool.copy()
    o1 = serving.decode_window(p1, q, k, v, beta, la)
    o2 = serving.decode_window(p2, np.repeat(q, 2, axis=2), np.repeat(k, 2, axis=2), v, beta, la)
    assert np.array_equal(o1, o2) and np.array_equal(p1, p2)
    # the other possible mapping (h % Hqk, heads tiled) reads different keys for heads 1, 2
    o3 = serving.decode_window(pool.copy(), np.tile(q, (1, 1, 2, 1)), np.tile(k, (1, 1, 2, 1)), v, beta, la)
    assert np.array_equal(o3[:, :, [0, 3]], o1[:, :, [0, 3]])
    assert not np.allclose(o3[:, :, [1, 2]], o1[:, :, [1, 2]])


def test_verify_commit_rollback():
    rng = np.random.default_rng(4)
    N, T, H, D = 4, 4, 2, 8
    q, k, v, beta, la = _window_inputs(rng, N, T, H, H, D)
    pool = rng.normal(0, 0.1, (N, H, D, D))
    # verification leaves the pool bit-identical and gives every draft token's output
    p = pool.copy()
    o_ver = serving.decode_window(p, q, k, v, beta, la, write_state=False)
    assert np.array_equal(p, pool)
    o_all = serving.decode_window(pool.copy(), q, k, v, beta, la)
    assert np.array_equal(o_ver, o_all)
    # commit of n accepted tokens == a window of only those n tokens; n = 0 keeps the state
    n_acc = np.array([0, 1, 3, 4])
    p = pool.copy()
    serving.decode_window(p, q, k, v, beta, la, n_commit=n_acc)
    assert np.array_equal(p[0], pool[0])
    for n in range(1, N):
        ref = pool[n:n + 1].copy()
        m = int(n_acc[n])
        serving.decode_window(ref, q[n:n + 1, :m], k[n:n + 1, :m], v[n:n + 1, :m], beta[n:n + 1, :m],
                              la[n:n + 1, :m])
        assert np.array_equal(p[n], ref[0])
    # committing the rest afterwards equals committing the whole window at once
    p_rest = p.copy()
    for n in range(N):
        m = int(n_acc[n])
        if m < T:
            one = p_rest[n:n + 1]
            serving.decode_window(one, q[n:n + 1, m:], k[n:n + 1, m:], v[n:n + 1, m:], beta[n:n + 1, m:],
                                  la[n:n + 1, m:])
            p_rest[n] = one[0]
    p_once = pool.copy()
    serving.decode_window(p_once, q, k, v, beta, la)
    assert np.allclose(p_rest, p_once, rtol=0, atol=1e-14)


def test_slots_address_the_pool():
    rng = np.random.default_rng(5)
    N, T, H, D, P = 3, 2, 2, 8, 6
    q, k, v, beta, la = _window_inputs(rng, N, T, H, H, D)
    pool = rng.normal(0, 0.1, (P, H, D, D))
    slots = np.array([4, -1, 1])
    p = pool.copy()
    o = serving.decode_window(p, q, k, v, beta, la, slots=slots)
    assert np.isnan(o[1]).all() and np.array_equal(p[[0, 2, 3, 5]], pool[[0, 2, 3, 5]])
    dense = pool[[4, 1]].copy()
    od = serving.decode_window(dense, q[[0, 2]], k[[0, 2]], v[[0, 2]], beta[[0, 2]], la[[0, 2]])
    assert np.array_equal(o[[0, 2]], od) and np.array_equal(p[[4, 1]], dense)
    # a slot past the pool is skipped like a negative one
    p2 = pool.copy()
    o2 = serving.decode_window(p2, q, k, v, beta, la, slots=np.array([P, 0, 2]))
    assert np.isnan(o2[0]).all() and np.array_equal(p2[[1, 3, 4, 5]], pool[[1, 3, 4, 5]])


def test_fused_prologue_composes():
    """raw gates + in-kernel normalisation == the window on pre-normalised q, k and the
    gates computed by gates_from_raw."""
    rng = np.random.default_rng(6)
    N, T, H, Hqk, D = 2, 3, 4, 2, 8
    q = rng.normal(0, 3, (N, T, Hqk, D))
    k = rng.normal(0, 3, (N, T, Hqk, D))
    v = rng.normal(0, 1, (N, T, H, D))
    b, a = rng.normal(0, 1, (N, T, H)), rng.normal(0, 1, (N, T, H))
    A_log, dt = rng.normal(-1, 0.5, H), rng.normal(0, 0.5, H)
    pool = rng.normal(0, 0.1, (N, H, D, D))
    p1, p2 = pool.copy(), pool.copy()
    o1 = serving.decode_window(p1, q, k, v, b, a, qk_l2norm=True, raw_gates=True, A_log=A_log, dt_bias=dt)
    beta, la = serving.gates_from_raw(b, a, A_log, dt)
    o2 = serving.decode_window(p2, serving.l2_normalize(q), serving.l2_normalize(k), v, beta, la)
    assert np.array_equal(o1, o2) and np.array_equal(p1, p2)


def test_forward_ex_matches_decode_windows():
    """The prefill with grouped heads and raw gates (ora_forward underneath) equals the same
    tokens run as decode windows (ora_decode_step underneath)."""
    rng = np.random.default_rng(7)
    B, Hqk, H, T, D = 2, 2, 4, 9, 8
    q = rng.normal(0, 1, (B, Hqk, T, D))
    k = rng.normal(0, 1, (B, Hqk, T, D))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.normal(0, 1, (B, H, T, D))
    b, a = rng.normal(0, 1, (B, H, T)), rng.normal(0, 1, (B, H, T))
    A_log, dt = rng.normal(-1, 0.5, H), rng.normal(0, 0.5, H)
    s0 = rng.normal(0, 0.1, (B, H, D, D))
    o, sf, _ = serving.forward_ex(q, k, v, b, a, s0, raw_gates=True, A_log=A_log, dt_bias=dt)
    pool = s0.copy()
    ow = serving.decode_window(pool, q.transpose(0, 2, 1, 3), k.transpose(0, 2, 1, 3), v.transpose(0, 2, 1, 3),
                               b.transpose(0, 2, 1), a.transpose(0, 2, 1), raw_gates=True, A_log=A_log, dt_bias=dt)
    assert np.allclose(o, ow.transpose(0, 2, 1, 3), rtol=0, atol=1e-13)
    assert np.allclose(sf, pool, rtol=0, atol=1e-13)


def test_ragged_equal_lengths_is_the_batch():
    """With equal lengths the concatenated layout is the batched [B, H, T, D] one: the ragged
    oracle and forward_ex agree exactly; an empty sequence keeps its state."""
    rng = np.random.default_rng(8)
    B, H, Hqk, T, D = 3, 4, 2, 6, 8
    q = rng.normal(0, 1, (B, Hqk, T, D))
    k = rng.normal(0, 1, (B, Hqk, T, D))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.normal(0, 1, (B, H, T, D))
    beta, la = rng.uniform(0.1, 0.9, (B, H, T)), rng.uniform(-0.2, -0.01, (B, H, T))
    s0 = rng.normal(0, 0.1, (B, H, D, D))
    o, sf, _ = serving.forward_ex(q, k, v, beta, la, s0)
    cu = [0, T, 2 * T, 3 * T]
    orag, sfrag = serving.forward_ragged(q.reshape(-1, D), k.reshape(-1, D), v.reshape(-1, D), beta.reshape(-1),
                                         la.reshape(-1), cu, H=H, Hqk=Hqk, s0=s0)
    assert np.array_equal(orag, o.reshape(-1, D)) and np.array_equal(sfrag, sf)
    # lengths 6, 0, 12: the empty sequence leaves s0 untouched
    cu2 = [0, T, T, 3 * T]
    _, sf2 = serving.forward_ragged(q.reshape(-1, D), k.reshape(-1, D), v.reshape(-1, D), beta.reshape(-1),
                                    la.reshape(-1), cu2, H=H, Hqk=Hqk, s0=s0)
    assert np.array_equal(sf2[1], s0[1]) and np.array_equal(sf2[0], sf[0])


def test_forward_ex_l2norm_scale_invariant():
    """With the q/k normalisation the prefill depends on each q and k row only through its
    direction: a positive scale per (head, token) row leaves it unchanged (up to the 1e-6
    epsilon under the square root, negligible at these norms), while without it the result
    moves.  A missing normalisation, one over the wrong axis, or one applied to q only or k
    only fails this."""
    rng = np.random.default_rng(11)
    B, Hqk, H, T, D = 2, 2, 4, 7, 8
    q = rng.normal(0, 10, (B, Hqk, T, D))
    k = rng.normal(0, 10, (B, Hqk, T, D))
    v = rng.normal(0, 1, (B, H, T, D))
    beta, la = rng.uniform(0.1, 0.9, (B, H, T)), rng.uniform(-0.2, -0.01, (B, H, T))
    s0 = rng.normal(0, 0.1, (B, H, D, D))
    cq = rng.uniform(1, 10, (B, Hqk, T, 1))
    ck = rng.uniform(1, 10, (B, Hqk, T, 1))
    o1, sf1, _ = serving.forward_ex(q, k, v, beta, la, s0, qk_l2norm=True)
    o2, sf2, _ = serving.forward_ex(q * cq, k * ck, v, beta, la, s0, qk_l2norm=True)
    assert np.allclose(o1, o2, rtol=0, atol=1e-8) and np.allclose(sf1, sf2, rtol=0, atol=1e-8)
    o3, _, _ = serving.forward_ex(q * cq, k, v, beta, la, s0, qk_l2norm=False)
    o4, _, _ = serving.forward_ex(q, k, v, beta, la, s0, qk_l2norm=False)
    assert not np.allclose(o3, o4, rtol=0, atol=1e-3)


def test_forward_ex_l2norm_keeps_unit_rows():
    """Rows that already have unit length are scaled by 1 / sqrt(1 + 1e-6) only: the
    normalised prefill matches the plain one to that factor."""
    rng = np.random.default_rng(12)
    B, H, T, D = 1, 2, 9, 8
    q = rng.normal(0, 1, (B, H, T, D))
    k = rng.normal(0, 1, (B, H, T, D))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.normal(0, 1, (B, H, T, D))
    beta, la = rng.uniform(0.1, 0.9, (B, H, T)), rng.uniform(-0.2, -0.01, (B, H, T))
    o1, sf1, _ = serving.forward_ex(q, k, v, beta, la, qk_l2norm=True)
    o2, sf2, _ = serving.forward_ex(q, k, v, beta, la)
    assert np.allclose(o1, o2, rtol=1e-5, atol=1e-6) and np.allclose(sf1, sf2, rtol=1e-5, atol=1e-6)
    assert not np.array_equal(o1, o2)
