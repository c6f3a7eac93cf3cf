"""MI355X (gfx950) gated delta rule core: Python binding of libgdn.so.

The functions here carry the names of the C ABI in ``include/gdn.h`` and only
marshal arguments: they check shapes, dtypes and devices, allocate outputs through
PyTorch when the caller does not pass them, and hand raw device pointers and the
HIP stream (the caller's, or torch's current one) to the library.  Every step of the computation runs in the HIP
kernels; there is no fallback.  If ``libgdn.so`` is missing, importing this package
fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "GdnError", "gdn_chunk_fwd", "kda_chunk_fwd", "gdn_decode_step", "gdn_chunk_workspace_size",
    "gdn_status_string", "gdn_version", "library_path", "lib",
    "GDN_F32", "GDN_BF16", "GDN_SUCCESS", "GDN_ERROR_INVALID_VALUE", "GDN_ERROR_NOT_SUPPORTED",
    "GDN_ERROR_HIP", "GdnChunkDesc", "GdnDecodeExDesc", "gdn_decode_ex", "gdn_decode_verify",
    "gdn_decode_commit", "GdnChunkExDesc", "gdn_chunk_fwd_ex", "gdn_chunk_fwd_ragged", "pack_ragged",
    "unpack_ragged", "kda_chunk_fwd_noalloc",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libgdn.so")

GDN_F32, GDN_BF16 = 0, 1
GDN_SUCCESS, GDN_ERROR_INVALID_VALUE, GDN_ERROR_NOT_SUPPORTED, GDN_ERROR_HIP = 0, 1, 2, 3


class GdnChunkDesc(ctypes.Structure):
    """Mirror of gdn_chunk_desc_t."""
    _fields_ = [
        ("B", ctypes.c_int64), ("H", ctypes.c_int64), ("T", ctypes.c_int64),
        ("Dk", ctypes.c_int64), ("Dv", ctypes.c_int64),
        ("chunk", ctypes.c_int32), ("in_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int),
        ("ckpt_every", ctypes.c_int64),
    ]


class GdnChunkExDesc(ctypes.Structure):
    """Mirror of gdn_chunk_ex_desc_t."""
    _fields_ = [("base", GdnChunkDesc), ("H_qk", ctypes.c_int64), ("raw_gates", ctypes.c_int32),
                ("qk_l2norm", ctypes.c_int32)]


class GdnDecodeExDesc(ctypes.Structure):
    """Mirror of gdn_decode_ex_desc_t."""
    _fields_ = [
        ("N", ctypes.c_int64), ("H", ctypes.c_int64), ("H_qk", ctypes.c_int64), ("Dk", ctypes.c_int64),
        ("Dv", ctypes.c_int64), ("T", ctypes.c_int64), ("P", ctypes.c_int64),
        ("in_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int),
        ("kda", ctypes.c_int32), ("qk_l2norm", ctypes.c_int32), ("raw_gates", ctypes.c_int32),
        ("write_state", ctypes.c_int32),
    ]


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {gdn_status_string(status)} (status {status})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(library_path):
        raise ImportError(
            f"{library_path} is not built; build it with `python gated_deltanet_state_amd/build.py` "
            "(hipcc --offload-arch=gfx950; `__graft_entry__.build()` does the same and also builds the "
            "test oracle). There is no CPU fallback.")
    L = ctypes.CDLL(library_path)
    vp, i64, ci, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    dp = ctypes.POINTER(GdnChunkDesc)
    L.gdn_chunk_workspace_size.argtypes = [dp, ci, ctypes.POINTER(sz)]
    L.gdn_chunk_workspace_size.restype = ci
    for name in ("gdn_chunk_fwd", "kda_chunk_fwd"):
        f = getattr(L, name)
        f.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        f.restype = ci
    L.kda_chunk_fwd_noalloc.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.kda_chunk_fwd_noalloc.restype = ci
    L.gdn_decode_step.argtypes = [i64, i64, i64, i64, ci, ci, vp, vp, vp, vp, vp, vp, vp, vp]
    L.gdn_decode_step.restype = ci
    L.gdn_chunk_fwd_ex.argtypes = [ctypes.POINTER(GdnChunkExDesc)] + [vp] * 13
    L.gdn_chunk_fwd_ex.restype = ci
    L.gdn_decode_ex.argtypes = [ctypes.POINTER(GdnDecodeExDesc)] + [vp] * 12
    L.gdn_decode_ex.restype = ci
    L.gdn_status_string.argtypes = [ci]
    L.gdn_status_string.restype = ctypes.c_char_p
    L.gdn_version.argtypes = []
    L.gdn_version.restype = ci
    return L


lib = _load()


def gdn_status_string(status: int) -> str:
    return lib.gdn_status_string(int(status)).decode()


def gdn_version() -> int:
    return int(lib.gdn_version())


_DT = {torch.float32: GDN_F32, torch.bfloat16: GDN_BF16}


def _code(dt: torch.dtype) -> int:
    if dt not in _DT:
        raise TypeError(f"unsupported dtype {dt}; use torch.float32 or torch.bfloat16")
    return _DT[dt]


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


class _Launch:
    """The stream a call runs on, and the tensors the binding allocated for it.

    Work is enqueued on ``stream`` (default: torch's current stream).  Tensors that the
    binding allocates come from torch's caching allocator on the current stream; when the
    kernels run on another stream, each such tensor is marked as used by that stream
    (``record_stream``), so that its memory is not handed to new work on the current stream
    while the kernels may still read or write it."""

    def __init__(self, stream):
        cur = torch.cuda.current_stream()
        if stream is None:
            stream = cur
        elif not isinstance(stream, torch.cuda.Stream):
            stream = torch.cuda.ExternalStream(int(stream))
        self.stream = stream
        self.handle = ctypes.c_void_p(stream.cuda_stream)
        self.other = stream.cuda_stream != cur.cuda_stream
        self.owned = []

    def new(self, *shape, **kw) -> torch.Tensor:
        t = torch.empty(*shape, **kw)
        self.owned.append(t)
        return t

    def done(self) -> None:
        if self.other:
            for t in self.owned:
                if t.is_cuda:
                    t.record_stream(self.stream)


def _ckpt_buffer(L: "_Launch", s_ckpt, shape, device, to_host: bool):
    """The snapshot buffer: on the device, or in pinned host memory (written by the kernel
    directly, see s_ckpt in include/gdn.h) when ``to_host`` or when a pinned CPU tensor is
    passed."""
    if s_ckpt is None:
        if to_host:
            return torch.empty(shape, dtype=torch.float32, pin_memory=True)
        return L.new(shape, dtype=torch.float32, device=device)
    if s_ckpt.device.type == "cpu":
        if not s_ckpt.is_pinned():
            raise ValueError("s_ckpt on the host must be pinned memory (pin_memory=True)")
        _check(s_ckpt, "s_ckpt", shape, torch.float32, s_ckpt.device)
    else:
        _check(s_ckpt, "s_ckpt", shape, torch.float32, device)
    return s_ckpt


def _check(t: torch.Tensor, name: str, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _desc(B, H, T, D, chunk, in_dt, out_dt, ckpt_every) -> GdnChunkDesc:
    return GdnChunkDesc(B, H, T, D, D, chunk, _code(in_dt), _code(out_dt), ckpt_every)


def gdn_chunk_workspace_size(B: int, H: int, T: int, D: int, *, chunk: int = 64,
                             in_dtype=torch.bfloat16, out_dtype=None, ckpt_every: int = 0,
                             kda: bool = False) -> int:
    d = _desc(B, H, T, D, chunk, in_dtype, out_dtype or in_dtype, ckpt_every)
    n = ctypes.c_size_t(0)
    st = lib.gdn_chunk_workspace_size(ctypes.byref(d), int(kda), ctypes.byref(n))
    if st != GDN_SUCCESS:
        raise GdnError(st, "gdn_chunk_workspace_size")
    return int(n.value)


def _chunk_fwd(kda: bool, q, k, v, beta, log_alpha, s0, chunk, ckpt_every, out_dtype, o, s_final,
               s_ckpt, return_final, stream,
               snapshots_to_host: bool = False, workspace=None) -> Tuple[torch.Tensor, Optional[torch.Tensor], Optional[torch.Tensor]]:
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, Dk]")
    B, H, T, D = q.shape
    dev, in_dt = q.device, q.dtype
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device (there is no CPU path)")
    L = _Launch(stream)
    out_dt = out_dtype or in_dt
    _check(k, "k", (B, H, T, D), in_dt, dev)
    _check(v, "v", (B, H, T, D), in_dt, dev)
    _check(beta, "beta", (B, H, T), in_dt, dev)
    _check(log_alpha, "log_alpha", (B, H, T, D) if kda else (B, H, T), in_dt, dev)
    _check(q, "q", (B, H, T, D), in_dt, dev)
    if s0 is not None:
        _check(s0, "s0", (B, H, D, D), torch.float32, dev)
    if o is None:
        o = L.new(B, H, T, D, dtype=out_dt, device=dev)
    _check(o, "o", (B, H, T, D), out_dt, dev)
    if s_final is None and return_final:
        s_final = L.new(B, H, D, D, dtype=torch.float32, device=dev)
    if s_final is not None:
        _check(s_final, "s_final", (B, H, D, D), torch.float32, dev)
    n_ck = T // ckpt_every if ckpt_every > 0 else 0
    s_ckpt = _ckpt_buffer(L, s_ckpt, (B, H, n_ck, D, D), dev, snapshots_to_host) if n_ck > 0 else None
    d = _desc(B, H, T, D, chunk, in_dt, out_dt, ckpt_every)
    fn = lib.kda_chunk_fwd if kda else lib.gdn_chunk_fwd
    # the matrix-core KDA prefill runs in its two-kernel form when given its workspace
    ws, ws_bytes = None, 0
    if workspace is not False:
        need = ctypes.c_size_t(0)
        st = lib.gdn_chunk_workspace_size(ctypes.byref(d), int(kda), ctypes.byref(need))
        if st != GDN_SUCCESS:
            raise GdnError(st, "gdn_chunk_workspace_size")
        if need.value > 0:
            if workspace is None:
                workspace = L.new(need.value, dtype=torch.uint8, device=dev)
            ws, ws_bytes = workspace, workspace.numel() * workspace.element_size()
    st = fn(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_alpha), _ptr(s0),
            _ptr(o), _ptr(s_final), _ptr(s_ckpt), _ptr(ws), ws_bytes, L.handle)
    if st != GDN_SUCCESS:
        raise GdnError(st, "kda_chunk_fwd" if kda else "gdn_chunk_fwd")
    L.done()
    return o, s_final, s_ckpt


def gdn_chunk_fwd(q, k, v, beta, log_alpha, s0=None, *, chunk: int = 64, ckpt_every: int = 0,
                  out_dtype=None, o=None, s_final=None, s_ckpt=None, return_final: bool = True,
                  stream=None, snapshots_to_host: bool = False):
    """Chunkwise prefill of the gated delta rule (see gdn_chunk_fwd in include/gdn.h).

    q, k [B,H,T,D]; v [B,H,T,D]; beta, log_alpha [B,H,T] (fp32 or bf16, one dtype);
    s0 [B,H,D,D] fp32 or None.  Returns (o [B,H,T,D], s_final [B,H,D,D] fp32 or None,
    s_ckpt [B,H,T//ckpt_every,D,D] fp32 or None).  Pass s_final=s0 to update in place.
    Asynchronous on `stream` (default: torch's current stream).  With snapshots_to_host (or a
    pinned CPU tensor as s_ckpt) the kernel writes the snapshots straight into pinned host
    memory; read them after synchronising the stream.
    """
    return _chunk_fwd(False, q, k, v, beta, log_alpha, s0, chunk, ckpt_every, out_dtype, o,
                      s_final, s_ckpt, return_final, stream, snapshots_to_host)


def kda_chunk_fwd(q, k, v, beta, log_alpha, s0=None, *, chunk: int = 64, ckpt_every: int = 0,
                  out_dtype=None, o=None, s_final=None, s_ckpt=None, return_final: bool = True,
                  stream=None, snapshots_to_host: bool = False, workspace=None):
    """Chunkwise prefill of KDA: as gdn_chunk_fwd with log_alpha [B,H,T,D] (one rate per key channel).

    workspace: None (default) allocates the device workspace of the two-kernel form through
    torch when the matrix-core path applies (gdn_chunk_workspace_size bytes); a uint8 device
    tensor of at least that size is used as given; False runs the single-kernel form."""
    return _chunk_fwd(True, q, k, v, beta, log_alpha, s0, chunk, ckpt_every, out_dtype, o,
                      s_final, s_ckpt, return_final, stream, snapshots_to_host, workspace)


def kda_chunk_fwd_noalloc(q, k, v, beta, log_alpha, s0=None, *, o, s_final=None, s_ckpt=None,
                          ckpt_every: int = 0, chunk: int = 64, stream=None):
    """kda_chunk_fwd with every output passed in and no allocation anywhere (the library runs on
    its fixed device scratch, see kda_chunk_fwd_noalloc in include/gdn.h): o [B,H,T,D] is
    required, s_final [B,H,D,D] fp32 and s_ckpt [B,H,T//ckpt_every,D,D] fp32 when wanted.
    Calls that overlap on one GPU race on the scratch."""
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, Dk]")
    B, H, T, D = q.shape
    dev, in_dt = q.device, q.dtype
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device (there is no CPU path)")
    L = _Launch(stream)
    for name, t, shp in (("k", k, (B, H, T, D)), ("v", v, (B, H, T, D)), ("beta", beta, (B, H, T)),
                         ("log_alpha", log_alpha, (B, H, T, D))):
        _check(t, name, shp, in_dt, dev)
    if s0 is not None:
        _check(s0, "s0", (B, H, D, D), torch.float32, dev)
    _check(o, "o", (B, H, T, D), o.dtype, dev)
    if s_final is not None:
        _check(s_final, "s_final", (B, H, D, D), torch.float32, dev)
    n_ck = T // ckpt_every if ckpt_every > 0 else 0
    if n_ck > 0:
        if s_ckpt is None:
            raise ValueError("s_ckpt must be passed when ckpt_every > 0 (nothing is allocated here)")
        _check(s_ckpt, "s_ckpt", (B, H, n_ck, D, D), torch.float32, s_ckpt.device)
    d = _desc(B, H, T, D, chunk, in_dt, o.dtype, ckpt_every)
    st = lib.kda_chunk_fwd_noalloc(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_alpha),
                                   _ptr(s0), _ptr(o), _ptr(s_final), _ptr(s_ckpt if n_ck > 0 else None), L.handle)
    if st != GDN_SUCCESS:
        raise GdnError(st, "kda_chunk_fwd_noalloc")
    return o, s_final, s_ckpt


def gdn_decode_step(state, q, k, v, beta, log_alpha, *, o=None, out_dtype=None, stream=None):
    """One decode step on every (sequence, head) fp32 state, in place (gdn_decode_step).

    state [N,H,D,D] fp32 (updated); q, k, v [N,H,D]; beta, log_alpha [N,H].  Returns o [N,H,D].
    """
    N, H, D, D2 = state.shape
    dev, in_dt = q.device, q.dtype
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device (there is no CPU path)")
    L = _Launch(stream)
    _check(state, "state", (N, H, D, D2), torch.float32, dev)
    for name, t, shp in (("q", q, (N, H, D2)), ("k", k, (N, H, D2)), ("v", v, (N, H, D)),
                         ("beta", beta, (N, H)), ("log_alpha", log_alpha, (N, H))):
        _check(t, name, shp, in_dt, dev)
    out_dt = out_dtype or in_dt
    if o is None:
        o = L.new(N, H, D, dtype=out_dt, device=dev)
    _check(o, "o", (N, H, D), out_dt, dev)
    st = lib.gdn_decode_step(N, H, D2, D, _code(in_dt), _code(out_dt), _ptr(state), _ptr(q), _ptr(k),
                             _ptr(v), _ptr(beta), _ptr(log_alpha), _ptr(o), L.handle)
    if st != GDN_SUCCESS:
        raise GdnError(st, "gdn_decode_step")
    L.done()
    return o


def gdn_decode_ex(pool, q, k, v, beta, log_alpha, *, slots=None, n_commit=None, write_state: bool = True,
                  kda: bool = False, qk_l2norm: bool = False, A_log=None, dt_bias=None, o=None,
                  out_dtype=None, return_o: bool = True, stream=None):
    """Serving-side decode window (gdn_decode_ex in include/gdn.h).

    pool [P,H,D,D] fp32 (rows slots[n] read, and written when write_state); q, k [N,T,Hqk,D];
    v [N,T,H,D]; beta [N,T,H]; log_alpha [N,T,H] or [N,T,H,D] (kda); with A_log and dt_bias
    ([H] fp32) given, beta and log_alpha are the raw b and a of the layer.  slots, n_commit:
    int32 [N] or None.  Returns o [N,T,H,D] (or None when return_o is False and o is None).
    """
    if q.dim() != 4 or pool.dim() != 4:
        raise ValueError("q must be [N, T, Hqk, D] and pool [P, H, D, D]")
    N, T, Hqk, D = q.shape
    P, H = pool.shape[0], pool.shape[1]
    dev, in_dt = q.device, q.dtype
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device (there is no CPU path)")
    L = _Launch(stream)
    _check(pool, "pool", (P, H, D, D), torch.float32, dev)
    for name, t, shp in (("k", k, (N, T, Hqk, D)), ("v", v, (N, T, H, D)), ("beta", beta, (N, T, H)),
                         ("log_alpha", log_alpha, (N, T, H, D) if kda else (N, T, H))):
        _check(t, name, shp, in_dt, dev)
    raw = A_log is not None
    if raw:
        _check(A_log, "A_log", (H,), torch.float32, dev)
        _check(dt_bias, "dt_bias", (H,), torch.float32, dev)
    for name, t in (("slots", slots), ("n_commit", n_commit)):
        if t is not None:
            _check(t, name, (N,), torch.int32, dev)
    out_dt = out_dtype or in_dt
    if o is None and return_o:
        o = L.new(N, T, H, D, dtype=out_dt, device=dev)
    if o is not None:
        _check(o, "o", (N, T, H, D), out_dt, dev)
    d = GdnDecodeExDesc(N, H, Hqk, D, D, T, P, _code(in_dt), _code(out_dt), int(kda), int(qk_l2norm),
                        int(raw), int(write_state))
    st = lib.gdn_decode_ex(ctypes.byref(d), _ptr(pool), _ptr(slots), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                           _ptr(log_alpha), _ptr(A_log), _ptr(dt_bias), _ptr(n_commit), _ptr(o), L.handle)
    if st != GDN_SUCCESS:
        raise GdnError(st, "gdn_decode_ex")
    L.done()
    return o


def gdn_decode_verify(pool, q, k, v, beta, log_alpha, **kw):
    """Outputs of all T draft tokens of each sequence; the pool is only read."""
    return gdn_decode_ex(pool, q, k, v, beta, log_alpha, write_state=False, **kw)


def gdn_decode_commit(pool, q, k, v, beta, log_alpha, n_commit, **kw):
    """Apply the first n_commit[n] tokens of each window to the pool rows in place."""
    kw.setdefault("return_o", False)
    return gdn_decode_ex(pool, q, k, v, beta, log_alpha, n_commit=n_commit, write_state=True, **kw)


def gdn_chunk_fwd_ex(q, k, v, beta, log_alpha, s0=None, *, A_log=None, dt_bias=None, qk_l2norm: bool = False,
                     chunk: int = 64, ckpt_every: int = 0, out_dtype=None, o=None, s_final=None, s_ckpt=None,
                     return_final: bool = True, stream=None, snapshots_to_host: bool = False):
    """Chunkwise prefill with grouped query/key heads and optionally the raw gate projections
    and the q/k normalisation (gdn_chunk_fwd_ex in include/gdn.h).

    q, k [B,Hqk,T,D]; v [B,H,T,D]; beta, log_alpha [B,H,T] (b and a when A_log, dt_bias [H]
    fp32 are given); s0 [B,H,D,D] fp32 or None; qk_l2norm scales q and k rows to unit length
    in the kernel.  Returns (o, s_final, s_ckpt) like gdn_chunk_fwd.
    """
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q must be [B, Hqk, T, D] and v [B, H, T, D]")
    B, Hqk, T, D = q.shape
    H = v.shape[1]
    dev, in_dt = q.device, q.dtype
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device (there is no CPU path)")
    L = _Launch(stream)
    out_dt = out_dtype or in_dt
    _check(k, "k", (B, Hqk, T, D), in_dt, dev)
    _check(v, "v", (B, H, T, D), in_dt, dev)
    _check(beta, "beta", (B, H, T), in_dt, dev)
    _check(log_alpha, "log_alpha", (B, H, T), in_dt, dev)
    raw = A_log is not None
    if raw:
        _check(A_log, "A_log", (H,), torch.float32, dev)
        _check(dt_bias, "dt_bias", (H,), torch.float32, dev)
    if s0 is not None:
        _check(s0, "s0", (B, H, D, D), torch.float32, dev)
    if o is None:
        o = L.new(B, H, T, D, dtype=out_dt, device=dev)
    _check(o, "o", (B, H, T, D), out_dt, dev)
    if s_final is None and return_final:
        s_final = L.new(B, H, D, D, dtype=torch.float32, device=dev)
    if s_final is not None:
        _check(s_final, "s_final", (B, H, D, D), torch.float32, dev)
    n_ck = T // ckpt_every if ckpt_every > 0 else 0
    s_ckpt = _ckpt_buffer(L, s_ckpt, (B, H, n_ck, D, D), dev, snapshots_to_host) if n_ck > 0 else None
    d = GdnChunkExDesc(_desc(B, H, T, D, chunk, in_dt, out_dt, ckpt_every), Hqk, int(raw), int(bool(qk_l2norm)))
    st = lib.gdn_chunk_fwd_ex(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_alpha),
                              _ptr(A_log), _ptr(dt_bias), None, _ptr(s0), _ptr(o), _ptr(s_final), _ptr(s_ckpt),
                              L.handle)
    if st != GDN_SUCCESS:
        raise GdnError(st, "gdn_chunk_fwd_ex")
    L.done()
    return o, s_final, s_ckpt


def pack_ragged(seqs):
    """Concatenate per-sequence tensors [heads, T_b, ...] into the packed [heads * sum T_b, ...]
    layout of a ragged batch; returns (packed, cu_seqlens as an int32 list)."""
    cu = [0]
    for x in seqs:
        cu.append(cu[-1] + int(x.shape[1]))
    flat = [x.reshape(x.shape[0] * x.shape[1], *x.shape[2:]) for x in seqs]
    return torch.cat(flat, 0), cu


def unpack_ragged(packed, cu, heads: int):
    """Inverse of pack_ragged: a list of [heads, T_b, ...] views."""
    out = []
    for b in range(len(cu) - 1):
        t0, t1 = cu[b], cu[b + 1]
        out.append(packed[heads * t0:heads * t1].reshape(heads, t1 - t0, *packed.shape[1:]))
    return out


def gdn_chunk_fwd_ragged(q, k, v, beta, log_alpha, cu_seqlens, *, H: int, H_qk: int = None, s0=None,
                         A_log=None, dt_bias=None, qk_l2norm: bool = False, out_dtype=None, o=None,
                         s_final=None, return_final: bool = True, stream=None):
    """Prefill of a ragged batch (gdn_chunk_fwd_ex with cu_seqlens): B sequences of different
    lengths in one call.

    cu_seqlens: int32 [B + 1] on the device (0 = cu[0] <= ... <= cu[B] = T).  Packed tensors
    (see pack_ragged): q, k [H_qk * T, D]; v [H * T, D]; beta, log_alpha [H * T]; s0, s_final
    [B, H, D, D] fp32.  Returns (o [H * T, D], s_final)."""
    H_qk = H if H_qk is None else H_qk
    if q.dim() != 2 or cu_seqlens.dim() != 1:
        raise ValueError("q must be [H_qk * T, D] and cu_seqlens [B + 1]")
    if H <= 0 or H_qk <= 0 or q.shape[0] % H_qk:
        raise ValueError("q rows must be a multiple of H_qk")
    T, D = q.shape[0] // H_qk, q.shape[1]
    B = cu_seqlens.shape[0] - 1
    dev, in_dt = q.device, q.dtype
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device (there is no CPU path)")
    L = _Launch(stream)
    out_dt = out_dtype or in_dt
    _check(k, "k", (H_qk * T, D), in_dt, dev)
    _check(v, "v", (H * T, D), in_dt, dev)
    _check(beta, "beta", (H * T,), in_dt, dev)
    _check(log_alpha, "log_alpha", (H * T,), in_dt, dev)
    _check(cu_seqlens, "cu_seqlens", (B + 1,), torch.int32, dev)
    raw = A_log is not None
    if raw:
        _check(A_log, "A_log", (H,), torch.float32, dev)
        _check(dt_bias, "dt_bias", (H,), torch.float32, dev)
    if s0 is not None:
        _check(s0, "s0", (B, H, D, D), torch.float32, dev)
    if o is None:
        o = L.new(H * T, D, dtype=out_dt, device=dev)
    _check(o, "o", (H * T, D), out_dt, dev)
    if s_final is None and return_final:
        s_final = L.new(B, H, D, D, dtype=torch.float32, device=dev)
    if s_final is not None:
        _check(s_final, "s_final", (B, H, D, D), torch.float32, dev)
    d = GdnChunkExDesc(_desc(B, H, T, D, 64, in_dt, out_dt, 0), H_qk, int(raw), int(bool(qk_l2norm)))
    st = lib.gdn_chunk_fwd_ex(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_alpha),
                              _ptr(A_log), _ptr(dt_bias), _ptr(cu_seqlens), _ptr(s0), _ptr(o), _ptr(s_final),
                              None, L.handle)
    if st != GDN_SUCCESS:
        raise GdnError(st, "gdn_chunk_fwd_ex")
    L.done()
    return o, s_final
