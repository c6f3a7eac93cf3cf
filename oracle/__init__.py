"""fp64 CPU oracle of the gated delta rule and of KDA -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never imports it, and it imports nothing from the product.

The arithmetic lives in ``gdn_oracle.c`` (plain C, fp64, a token-by-token loop;
its header comment cites the pages it follows).  This module only builds it with
gcc and marshals numpy / CPU-torch arrays into it.

Function status (see ``tests/test_oracle_pins.py`` for the pins):
  forward (GDN)  -- pinned: rational brute force of the printed closed form, exact
                    overwrite, no-change, forget-only, decay table, x/y worked
                    example, reduction to the masked quadratic form.
  forward (KDA)  -- pinned: rational brute force of the printed KDA form, equal
                    channel gates == GDN, column-wise forget-only, exact overwrite.
  decode_step    -- pinned: exact overwrite; T single steps == one forward pass.
  serving.*      -- the serving-side decode (slot-addressed states, grouped heads, fused
                    gate activations and q/k normalisation, verify / commit windows): a
                    composition of decode_step; pinned in tests/test_oracle_serving.py.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F64, F32, BF16 = 0, 1, 2

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc -O2 (no fast-math) into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    i64, vp, dp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double), ctypes.c_int
    lib.ora_forward.argtypes = [i64, i64, i64, i64, i64, ci, ci, vp, vp, vp, vp, vp, vp, ci,
                                vp, vp, vp, i64, ci]
    lib.ora_forward.restype = ci
    lib.ora_decode_step.argtypes = [i64, i64, i64, i64, ci, ci, vp, vp, vp, vp, vp, vp, vp, ci]
    lib.ora_decode_step.restype = ci
    lib.ora_hardware_threads.argtypes = []
    lib.ora_hardware_threads.restype = ci
    del dp
    _lib = lib
    return lib


def _as_np(x):
    """Return (contiguous numpy array, dtype code).  bf16 torch tensors travel as uint16 bits."""
    try:
        import torch  # local import: the oracle itself does not need torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).numpy().view(np.uint16), BF16
            x = x.numpy()
    except ImportError:  # pragma: no cover
        pass
    x = np.ascontiguousarray(x)
    if x.dtype == np.float64:
        return x, F64
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.uint16:
        return x, BF16
    raise TypeError(f"oracle: unsupported input dtype {x.dtype}")


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def hardware_threads() -> int:
    return int(_load().ora_hardware_threads())


def forward(q, k, v, beta, log_alpha, s0=None, *, kda: bool = False, ckpt_every: int = 0,
            nthreads: int = 0, return_threads: bool = False):
    """Token-by-token fp64 forward pass.

    Shapes: q, k [B,H,T,Dk]; v [B,H,T,Dv]; beta [B,H,T]; log_alpha [B,H,T] (GDN) or
    [B,H,T,Dk] (KDA); s0 [B,H,Dv,Dk] or None.  Inputs may be fp64, fp32 or bf16; q, k, v,
    beta and log_alpha must share one dtype.  Returns (o, s_final, s_ckpt) as fp64 numpy
    arrays (s_ckpt is None when ckpt_every == 0).
    """
    qa, dt = _as_np(q)
    ka, dk_ = _as_np(k)
    va, dv_ = _as_np(v)
    ba, db = _as_np(beta)
    la, dl = _as_np(log_alpha)
    if len({dt, dk_, dv_, db, dl}) != 1:
        raise TypeError("oracle: q, k, v, beta, log_alpha must share one dtype")
    B, H, T, Dk = qa.shape
    Dv = va.shape[-1]
    if ka.shape != (B, H, T, Dk) or va.shape != (B, H, T, Dv) or ba.shape != (B, H, T):
        raise ValueError("oracle: shape mismatch")
    if la.shape != ((B, H, T, Dk) if kda else (B, H, T)):
        raise ValueError("oracle: log_alpha shape mismatch")
    s0a, ds0 = (None, F64) if s0 is None else _as_np(s0)
    if s0a is not None and s0a.shape != (B, H, Dv, Dk):
        raise ValueError("oracle: s0 shape mismatch")
    o = np.empty((B, H, T, Dv), np.float64)
    sf = np.empty((B, H, Dv, Dk), np.float64)
    nck = T // ckpt_every if ckpt_every > 0 else 0
    sc = np.empty((B, H, nck, Dv, Dk), np.float64) if ckpt_every > 0 else None
    n = _load().ora_forward(B, H, T, Dk, Dv, int(kda), dt, _ptr(qa), _ptr(ka), _ptr(va), _ptr(ba),
                            _ptr(la), _ptr(s0a), ds0, _ptr(o), _ptr(sf), _ptr(sc), int(ckpt_every),
                            int(nthreads))
    if n < 0:
        raise RuntimeError("oracle: ora_forward failed")
    if return_threads:
        return o, sf, sc, n
    return o, sf, sc


def decode_step(state: np.ndarray, q, k, v, beta, log_alpha, *, kda: bool = False,
                nthreads: int = 0) -> np.ndarray:
    """One recurrent step on every (sequence, head) state, in place on the fp64 ``state``.

    Shapes: state [N,H,Dv,Dk] fp64 (modified); q, k [N,H,Dk]; v [N,H,Dv]; beta [N,H];
    log_alpha [N,H] (GDN) or [N,H,Dk] (KDA).  Returns o [N,H,Dv] fp64.
    """
    if not (isinstance(state, np.ndarray) and state.dtype == np.float64 and state.flags.c_contiguous):
        raise TypeError("oracle: state must be a C-contiguous fp64 numpy array (updated in place)")
    qa, dt = _as_np(q)
    ka, _ = _as_np(k)
    va, _ = _as_np(v)
    ba, _ = _as_np(beta)
    la, _ = _as_np(log_alpha)
    N, H, Dv, Dk = state.shape
    if qa.shape != (N, H, Dk) or ka.shape != (N, H, Dk) or va.shape != (N, H, Dv) or ba.shape != (N, H):
        raise ValueError("oracle: decode shape mismatch")
    if la.shape != ((N, H, Dk) if kda else (N, H)):
        raise ValueError("oracle: decode log_alpha shape mismatch")
    o = np.empty((N, H, Dv), np.float64)
    n = _load().ora_decode_step(N, H, Dk, Dv, int(kda), dt, _ptr(state), _ptr(qa), _ptr(ka), _ptr(va),
                                _ptr(ba), _ptr(la), _ptr(o), int(nthreads))
    if n < 0:
        raise RuntimeError("oracle: ora_decode_step failed")
    return o
