"""fp64 model of the chunkwise algebra that the HIP prefill kernels implement (CPU only).

This is a design check, not the oracle: it restates, in plain numpy, the chunkwise
form of "Hybrid Linear Attention Architecture Design Explained" (intl.cloud.baidu.com),
section 4 "Hardware-Friendly Chunkwise Parallel Algorithm" (cross-chunk state update and
intra-chunk output, with the UT/WY triangular system that "Hybrid attention"
(xmarva.github.io), section "Training a recurrence in parallel", describes), read in
the d_v x d_k state convention.  It is compared with the token-by-token oracle; the
pages report the chunked form agreeing with the token loop to about 1e-15 in fp64.

Readings (the page's symbols are partly garbled):
  * the output term uses the decay from the chunk start to token r, inclusive
    (exp(G_r)); the state term uses the decay from token r to the chunk end
    (exp(G_C - G_r)).
  * W and U ("weight and value matrices", never defined on the page) come from the
    unit lower-triangular system (I + A) U = diag(beta) (V - diag(gamma) K S^T) with
    A = strict_tril(diag(beta) (K K^T * D)); the kernels solve it as U = T X with
    T = (I + A)^-1 computed from 16x16 diagonal blocks.
  * KDA: the factors exp(G_r - G_j) of the intra-chunk products are split at a
    reference point per 16-token sub-block so that no factor overflows half
    precision; this model checks that the split form equals the direct form.
"""
import numpy as np
import pytest

import oracle


def setup_module(module):
    oracle.build(force=False)


def _blocked_unit_lower_inverse(A, blk=16):
    """(I + A)^-1 for strictly lower A: forward substitution on blk x blk diagonal blocks,
    then block rows T_ij = -T_ii sum_{k=j..i-1} A_ik T_kj (the kernels' order)."""
    n = A.shape[0]
    nb = (n + blk - 1) // blk
    T = np.zeros_like(A)
    sl = [slice(i * blk, min(n, (i + 1) * blk)) for i in range(nb)]
    for i in range(nb):
        Ai = A[sl[i], sl[i]]
        m = Ai.shape[0]
        Ti = np.eye(m)
        for r in range(m):
            Ti[r, :r] = -Ai[r, :r] @ Ti[:r, :r]
        T[sl[i], sl[i]] = Ti
    for i in range(1, nb):
        for j in range(i - 1, -1, -1):
            acc = sum(A[sl[i], sl[k]] @ T[sl[k], sl[j]] for k in range(j, i))
            T[sl[i], sl[j]] = -T[sl[i], sl[i]] @ acc
    return T


def chunk_gdn(q, k, v, beta, g, S0, C):
    """One (batch, head) stream: q, k [T,Dk], v [T,Dv], beta, g [T], S0 [Dv,Dk]."""
    T = q.shape[0]
    S = S0.copy()
    O = np.zeros((T, v.shape[1]))
    for c0 in range(0, T, C):
        sl = slice(c0, min(T, c0 + C))
        Q, K, V, b = q[sl], k[sl], v[sl], beta[sl]
        G = np.cumsum(g[sl])                                  # inclusive prefix of log alpha
        gam = np.exp(G)
        Dm = np.exp(G[:, None] - G[None, :])
        n = len(G)
        A = np.tril(b[:, None] * (K @ K.T) * Dm, -1)
        Tm = _blocked_unit_lower_inverse(A)
        X = b[:, None] * (V - gam[:, None] * (K @ S.T))
        U = Tm @ X
        P = np.tril((Q @ K.T) * Dm)
        O[sl] = gam[:, None] * (Q @ S.T) + P @ U
        S = gam[-1] * S + U.T @ (np.exp(G[-1] - G)[:, None] * K)
        assert n <= C
    return O, S


def chunk_kda(q, k, v, beta, g, S0, C, blk=16):
    """KDA stream, g [T,Dk]; intra-chunk products use per-sub-block reference points."""
    T, Dk = q.shape
    S = S0.copy()
    O = np.zeros((T, v.shape[1]))
    for c0 in range(0, T, C):
        sl = slice(c0, min(T, c0 + C))
        Q, K, V, b = q[sl], k[sl], v[sl], beta[sl]
        G = np.cumsum(g[sl], axis=0)                          # [n, Dk]
        n = G.shape[0]
        Gpad = np.vstack([np.zeros((1, Dk)), G])              # Gpad[r + 1] = G_r, Gpad[0] = 0
        ref = lambda R: Gpad[R * blk]                          # G at the end of the previous block
        # left factor exp(G_r - G_ref(R(r))) <= 1 ; right factor exp(G_ref(R) - G_j) <= 1 off the
        # diagonal block, <= exp(blk * max|g|) on it
        QK = np.zeros((n, n))
        KK = np.zeros((n, n))
        for r in range(n):
            R = r // blk
            left = np.exp(G[r] - ref(R))
            assert np.all(left <= 1.0 + 1e-15)
            for j in range(r + 1):
                right = np.exp(ref(R) - G[j])
                if j // blk < R:
                    assert np.all(right <= 1.0 + 1e-15)
                QK[r, j] = (Q[r] * left) @ (K[j] * right)
                KK[r, j] = (K[r] * left) @ (K[j] * right)
        A = np.tril(b[:, None] * KK, -1)
        Tm = _blocked_unit_lower_inverse(A)
        Gam = np.exp(G)
        X = b[:, None] * (V - (K * Gam) @ S.T)
        U = Tm @ X
        O[sl] = (Q * Gam) @ S.T + np.tril(QK) @ U
        S = S * Gam[-1][None, :] + U.T @ (K * np.exp(G[-1] - G))
    return O, S


def _inputs(rng, H, T, Dk, Dv, kda):
    q = rng.standard_normal((1, H, T, Dk))
    k = rng.standard_normal((1, H, T, Dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((1, H, T, Dv))
    beta = 1 / (1 + np.exp(-rng.standard_normal((1, H, T))))
    g = rng.uniform(-0.2, -0.005, (1, H, T, Dk) if kda else (1, H, T))
    s0 = 0.1 * rng.standard_normal((1, H, Dv, Dk))
    return q, k, v, beta, g, s0


@pytest.mark.parametrize("C,T", [(16, 64), (16, 75), (64, 200), (64, 64)])
def test_gdn_chunk_form_matches_token_loop(C, T):
    rng = np.random.default_rng(C * 1000 + T)
    q, k, v, beta, g, s0 = _inputs(rng, 2, T, 24, 20, False)
    o_ref, s_ref, _ = oracle.forward(q, k, v, beta, g, s0)
    for h in range(2):
        O, S = chunk_gdn(q[0, h], k[0, h], v[0, h], beta[0, h], g[0, h], s0[0, h], C)
        assert np.linalg.norm(O - o_ref[0, h]) / np.linalg.norm(o_ref[0, h]) < 1e-13
        assert np.linalg.norm(S - s_ref[0, h]) / np.linalg.norm(s_ref[0, h]) < 1e-13


@pytest.mark.parametrize("C,T", [(16, 40), (64, 130)])
def test_kda_chunk_form_with_reference_points_matches_token_loop(C, T):
    rng = np.random.default_rng(C * 7 + T)
    q, k, v, beta, g, s0 = _inputs(rng, 1, T, 16, 12, True)
    o_ref, s_ref, _ = oracle.forward(q, k, v, beta, g, s0, kda=True)
    O, S = chunk_kda(q[0, 0], k[0, 0], v[0, 0], beta[0, 0], g[0, 0], s0[0, 0], C)
    assert np.linalg.norm(O - o_ref[0, 0]) / np.linalg.norm(o_ref[0, 0]) < 1e-13
    assert np.linalg.norm(S - s_ref[0, 0]) / np.linalg.norm(s_ref[0, 0]) < 1e-13


def test_tail_padding_is_an_identity_step():
    """Padding a ragged tail with q = k = v = 0, beta = 0, log alpha = 0 changes nothing
    ("Attention, Part 4", section 6: with beta = 0 the step only forgets, and alpha = 1
    forgets nothing)."""
    rng = np.random.default_rng(2)
    q, k, v, beta, g, s0 = _inputs(rng, 1, 50, 16, 16, False)
    O, S = chunk_gdn(q[0, 0], k[0, 0], v[0, 0], beta[0, 0], g[0, 0], s0[0, 0], 16)
    pad = lambda x, n: np.concatenate([x, np.zeros((n,) + x.shape[1:])])
    Op, Sp = chunk_gdn(pad(q[0, 0], 14), pad(k[0, 0], 14), pad(v[0, 0], 14), pad(beta[0, 0], 14),
                       pad(g[0, 0], 14), s0[0, 0], 16)
    np.testing.assert_allclose(Op[:50], O, rtol=0, atol=1e-14)
    np.testing.assert_allclose(Sp, S, rtol=0, atol=1e-14)
