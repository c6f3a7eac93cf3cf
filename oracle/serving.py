"""fp64 oracle of the serving-side decode paths -- TEST INFRASTRUCTURE ONLY.

Same rules as the rest of ``oracle/``: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it; it imports nothing from the product.

Everything here is a plain composition of pinned pieces:
  * ``l2_normalize``     -- q, k scaled to unit length.  Pinned by closed forms
                            (3-4-5 vector, basis vectors, zero vector, unit norms).
  * ``gates_from_raw``   -- beta and log alpha from the raw per-head projections.
                            Pinned by closed forms (sigmoid(0) = 1/2, softplus(0) = ln 2,
                            softplus(ln(e - 1)) = 1, limits, sign of log alpha).
  * ``forward_ex``       -- the prefill with grouped query/key heads, raw gates and the q/k
                            normalisation: the pinned ``oracle.forward`` on repeated heads,
                            gates_from_raw and l2_normalize.  Pinned also by invariance of
                            the normalised form to a positive scale of each q, k row.
  * ``decode_window``    -- T tokens per sequence on slot-addressed states, each token one
                            call of the pinned single-token step (``oracle.decode_step``).
                            Pinned against the independent token loop of ``oracle.forward``
                            and by the verify / commit / rollback invariants.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import _as_np, decode_step, BF16

# The pages fix no epsilon for the normalisation; this one only keeps a zero vector at zero.
L2_EPS = 1e-6


def widen(x) -> np.ndarray:
    """Exact fp64 copy of an fp64 / fp32 / bf16 (numpy or CPU torch) array."""
    a, dt = _as_np(x)
    if dt == BF16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def l2_normalize(x, eps: float = L2_EPS) -> np.ndarray:
    """x / sqrt(sum(x^2) + eps) over the last axis, in fp64.

    A Gated DeltaNet layer normalises queries and keys to length 1 before the memory step
    ("Attention, Part 4", section 6, the paragraph after "Where alpha and beta come from").
    """
    x = widen(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def gates_from_raw(b, a, A_log, dt_bias):
    """(beta, log_alpha) in fp64 from the raw per-value-head projections b, a [..., H] and the
    per-head parameters A_log, dt_bias [H]:

        beta      = sigmoid(b)
        log_alpha = -exp(A_log) * softplus(a + dt_bias),   softplus(x) = log(1 + e^x)

    ("Attention, Part 4", section "Where alpha and beta come from": b and a come from the
    token through learned matrices; the gate is kept as g = log alpha, always negative).
    """
    b, a, A_log, dt_bias = widen(b), widen(a), widen(A_log), widen(dt_bias)
    beta = 1.0 / (1.0 + np.exp(-b))
    x = a + dt_bias
    softplus = np.logaddexp(0.0, x)  # log(e^0 + e^x), exact form of log(1 + e^x)
    return beta, -np.exp(A_log) * softplus


def decode_window(pool: np.ndarray, q, k, v, beta, log_alpha, *, slots=None, kda: bool = False,
                  n_commit=None, write_state: bool = True, qk_l2norm: bool = False,
                  raw_gates: bool = False, A_log=None, dt_bias=None) -> np.ndarray:
    """T decode steps per sequence on states addressed through a slot table, in fp64.

    pool       [P, H, Dv, Dk] fp64 state pool (updated in place when ``write_state``)
    q, k       [N, T, Hqk, Dk]; value head h reads query/key head h // (H // Hqk)
    v          [N, T, H, Dv]
    beta       [N, T, H]            (raw b when ``raw_gates``)
    log_alpha  [N, T, H] or [N, T, H, Dk] for KDA (raw a when ``raw_gates``)
    slots      [N] pool row of each sequence (< 0 or >= P: the sequence is skipped), or None
               for slots[n] = n
    n_commit   [N] tokens whose state is kept (clamped to 0..T), or None for all T

    Sequence n runs its tokens one at a time through ``decode_step`` (forget, correct with
    the decayed state, read the updated state: "From Traditional Attention to hybrid
    ones", section 5) starting from pool[slots[n]]; o[n, t] is the output of token t.
    When ``write_state`` the pool row becomes the state after the first n_commit[n]
    tokens; otherwise (verification of draft tokens) the pool is left untouched, so
    rejected tokens never need to be undone ("Hybrid models: what Gated DeltaNet replaces
    in the KV cache", section "What a recurrent state changes for serving": speculative
    decoding needs the state from before the draft).
    Returns o [N, T, H, Dv] fp64, NaN for skipped sequences.
    """
    if not (isinstance(pool, np.ndarray) and pool.dtype == np.float64 and pool.flags.c_contiguous):
        raise TypeError("oracle: pool must be a C-contiguous fp64 numpy array")
    P, H, Dv, Dk = pool.shape
    q, k, v = widen(q), widen(k), widen(v)
    N, T, Hqk, _ = q.shape
    if H % Hqk != 0 or k.shape != q.shape or v.shape != (N, T, H, Dv):
        raise ValueError("oracle: decode_window shape mismatch")
    G = H // Hqk
    if raw_gates:
        if kda:
            raise ValueError("oracle: raw gates are defined for the scalar gate only")
        beta, log_alpha = gates_from_raw(beta, log_alpha, A_log, dt_bias)
    else:
        beta, log_alpha = widen(beta), widen(log_alpha)
    if beta.shape != (N, T, H) or log_alpha.shape != ((N, T, H, Dk) if kda else (N, T, H)):
        raise ValueError("oracle: decode_window gate shape mismatch")
    if qk_l2norm:
        q, k = l2_normalize(q), l2_normalize(k)
    heads = np.arange(H) // G  # query/key head of each value head
    sl = np.arange(N) if slots is None else widen_int(slots)
    nc = np.full(N, T, np.int64) if n_commit is None else np.clip(widen_int(n_commit), 0, T)
    o = np.full((N, T, H, Dv), np.nan)
    for n in range(N):
        s = int(sl[n])
        if s < 0 or s >= P:
            continue
        S = pool[s][None].copy()  # [1, H, Dv, Dk]
        kept = S.copy() if nc[n] == 0 else None
        for t in range(T):
            o[n, t] = decode_step(S, q[n, t, heads][None], k[n, t, heads][None], v[n, t][None],
                                  beta[n, t][None], log_alpha[n, t][None], kda=kda)[0]
            if t + 1 == nc[n]:
                kept = S.copy()
        if write_state:
            pool[s] = kept[0]
    return o


def widen_int(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x).astype(np.int64)


def forward_ex(q, k, v, beta, log_alpha, s0=None, *, raw_gates: bool = False, A_log=None, dt_bias=None,
               ckpt_every: int = 0, qk_l2norm: bool = False):
    """The token-loop forward pass (``oracle.forward``) with H value heads reading
    Hqk = q.shape[1] query/key heads (value head h reads head h // (H / Hqk)), with the
    raw gate projections b, a turned into beta and log alpha by ``gates_from_raw`` when
    ``raw_gates``, and with every q and k row scaled to unit length by ``l2_normalize`` when
    ``qk_l2norm``.  q, k [B, Hqk, T, Dk]; v [B, H, T, Dv]; beta, log_alpha [B, H, T] (b, a for
    raw gates; A_log, dt_bias [H]).  Returns (o, s_final, s_ckpt) in fp64."""
    from . import forward
    q, k, v = widen(q), widen(k), widen(v)
    if qk_l2norm:
        q, k = l2_normalize(q), l2_normalize(k)
    B, Hqk, T, Dk = q.shape
    H = v.shape[1]
    if H % Hqk != 0:
        raise ValueError("oracle: H must be a multiple of Hqk")
    G = H // Hqk
    q, k = np.repeat(q, G, axis=1), np.repeat(k, G, axis=1)
    if raw_gates:
        beta, log_alpha = gates_from_raw(np.moveaxis(widen(beta), 1, -1), np.moveaxis(widen(log_alpha), 1, -1),
                                         A_log, dt_bias)
        beta, log_alpha = np.moveaxis(beta, -1, 1).copy(), np.moveaxis(log_alpha, -1, 1).copy()
    else:
        beta, log_alpha = widen(beta), widen(log_alpha)
    s0 = None if s0 is None else widen(s0)
    return forward(q, k, v, beta, log_alpha, s0, ckpt_every=ckpt_every)


def forward_ragged(q, k, v, beta, log_alpha, cu_seqlens, *, H: int, Hqk: int, s0=None, raw_gates: bool = False,
                   A_log=None, dt_bias=None, qk_l2norm: bool = False):
    """A ragged batch: sequence b is tokens cu[b] .. cu[b+1]-1, each per-token tensor being the
    concatenation of the sequences in their own [heads, T_b, ...] layout (q, k [Hqk * T, D];
    v [H * T, D]; beta, log_alpha [H * T]; s0 [B, H, D, D] or None).  Each sequence runs
    through ``forward_ex`` on its own.  Returns (o [H * T, D], s_final [B, H, D, D])."""
    cu = widen_int(cu_seqlens)
    q, k, v, beta, log_alpha = widen(q), widen(k), widen(v), widen(beta), widen(log_alpha)
    B, D = len(cu) - 1, q.shape[1]
    s0 = None if s0 is None else widen(s0)
    o = np.empty((v.shape[0], D))
    sf = np.empty((B, H, D, D))
    for b in range(B):
        t0, t1 = int(cu[b]), int(cu[b + 1])
        n = t1 - t0
        sl = lambda x, h: x[h * t0:h * t1].reshape(h, n, *x.shape[1:])[None]
        ob, sfb, _ = forward_ex(sl(q, Hqk), sl(k, Hqk), sl(v, H), sl(beta, H), sl(log_alpha, H),
                                None if s0 is None else s0[b:b + 1], raw_gates=raw_gates, A_log=A_log,
                                dt_bias=dt_bias, qk_l2norm=qk_l2norm)
        o[H * t0:H * t1] = ob[0].reshape(H * n, D)
        sf[b] = sfb[0]
    return o, sf
