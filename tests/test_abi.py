"""The C-ABI library loads, exports what include/gdn.h declares, and rejects bad calls on
the host before launching anything (CPU only: no call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


@pytest.fixture(scope="module")
def g():
    import gated_deltanet_state_amd as g
    return g


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b((?:gdn|kda)_[a-z_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    assert _declared_functions() == sorted([
        "gdn_chunk_fwd", "gdn_chunk_fwd_ex", "gdn_chunk_workspace_size", "gdn_decode_ex", "gdn_decode_step",
        "gdn_status_string", "gdn_version", "kda_chunk_fwd", "kda_chunk_fwd_noalloc"])


def test_library_exports_every_declared_symbol(g):
    raw = ctypes.CDLL(g.library_path)
    for name in _declared_functions():
        assert hasattr(raw, name), name


def test_desc_struct_layout(g):
    assert ctypes.sizeof(g.GdnChunkDesc) == 64
    assert g.GdnChunkDesc.ckpt_every.offset == 56
    assert ctypes.sizeof(g.GdnDecodeExDesc) == 80
    assert ctypes.sizeof(g.GdnChunkExDesc) == 80 and g.GdnChunkExDesc.raw_gates.offset == 72
    assert g.GdnDecodeExDesc.in_dtype.offset == 56 and g.GdnDecodeExDesc.write_state.offset == 76


def test_version_and_status_strings(g):
    assert g.gdn_version() == 112
    for s in range(4):
        assert isinstance(g.gdn_status_string(s), str) and g.gdn_status_string(s)
    assert g.gdn_status_string(99) == "unknown status"


FAKE = 0x10000  # 16-byte aligned non-null value; never dereferenced because validation fails first


def _desc(g, **kw):
    base = dict(B=1, H=2, T=64, Dk=128, Dv=128, chunk=64, in_dtype=g.GDN_BF16, out_dtype=g.GDN_BF16,
                ckpt_every=0)
    base.update(kw)
    return g.GdnChunkDesc(**base)


def _call(g, d, kda=False, **ptrs):
    p = dict(q=FAKE, k=FAKE + 0x1000000, v=FAKE + 0x2000000, beta=FAKE + 0x3000000,
             log_alpha=FAKE + 0x4000000, s0=FAKE + 0x5000000, o=FAKE + 0x6000000,
             s_final=FAKE + 0x7000000, s_ckpt=FAKE + 0x8000000)
    p.update(ptrs)
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    fn = g.lib.kda_chunk_fwd if kda else g.lib.gdn_chunk_fwd
    return fn(None if d is None else ctypes.byref(d), v(p["q"]), v(p["k"]), v(p["v"]), v(p["beta"]),
              v(p["log_alpha"]), v(p["s0"]), v(p["o"]), v(p["s_final"]), v(p["s_ckpt"]), None, 0, None)


@pytest.mark.parametrize("kda", [False, True])
def test_chunk_validation_errors(g, kda):
    INV, NS = g.GDN_ERROR_INVALID_VALUE, g.GDN_ERROR_NOT_SUPPORTED
    assert _call(g, None, kda) == INV
    assert _call(g, _desc(g, chunk=48), kda) == INV
    assert _call(g, _desc(g, chunk=128), kda) == INV
    assert _call(g, _desc(g, T=-1), kda) == INV
    assert _call(g, _desc(g, Dk=0), kda) == INV
    assert _call(g, _desc(g, in_dtype=7), kda) == INV
    assert _call(g, _desc(g, ckpt_every=96), kda) == INV          # not a multiple of chunk
    assert _call(g, _desc(g, ckpt_every=-64), kda) == INV
    assert _call(g, _desc(g, Dk=128, Dv=64), kda) == NS
    assert _call(g, _desc(g, Dk=96, Dv=96), kda) == NS
    assert _call(g, _desc(g), kda, q=None) == INV
    assert _call(g, _desc(g), kda, o=None) == INV
    assert _call(g, _desc(g), kda, q=FAKE + 8) == INV              # misaligned
    assert _call(g, _desc(g), kda, s0=FAKE + 0x5000004) == INV
    # s_final partially overlapping s0
    assert _call(g, _desc(g), kda, s_final=FAKE + 0x5000000 + 4096) == INV
    # snapshots requested but no buffer
    assert _call(g, _desc(g, ckpt_every=64), kda, s_ckpt=None) == INV
    # o overlapping the state
    assert _call(g, _desc(g), kda, o=FAKE + 0x5000000 + 16) == INV
    # empty batch: nothing to launch
    assert _call(g, _desc(g, B=0), kda) == g.GDN_SUCCESS


def test_kda_workspace_validation(g):
    """The matrix-core KDA prefill's workspace: too small, misaligned, or overlapping an input or
    an output is INVALID_VALUE before anything is launched (B=1, H=2, T=64: two records of
    64 KiB)."""
    INV = g.GDN_ERROR_INVALID_VALUE
    d = _desc(g)
    need = g.gdn_chunk_workspace_size(1, 2, 64, 128, kda=True)
    assert need == 2 * 65536
    ws = FAKE + 0x40000000
    call = lambda addr, nbytes, **kw: _call_ws(g, d, addr, nbytes, **kw)
    assert call(ws, need - 16) == INV                 # too small
    assert call(ws + 8, need) == INV                  # misaligned
    assert call(FAKE + 0x6000000 - 64, need) == INV   # runs into o
    assert call(FAKE - 0x100, need) == INV            # covers q
    assert call(FAKE + 0x3000000, need) == INV        # covers beta and beyond


def _call_ws(g, d, ws, nbytes, **ptrs):
    p = dict(q=FAKE, k=FAKE + 0x1000000, v=FAKE + 0x2000000, beta=FAKE + 0x3000000,
             log_alpha=FAKE + 0x4000000, s0=FAKE + 0x5000000, o=FAKE + 0x6000000,
             s_final=FAKE + 0x7000000, s_ckpt=FAKE + 0x8000000)
    p.update(ptrs)
    args = [ctypes.c_void_p(p[n]) if p[n] is not None else None
            for n in ("q", "k", "v", "beta", "log_alpha", "s0", "o", "s_final", "s_ckpt")]
    return g.lib.kda_chunk_fwd(ctypes.byref(d), *args, ctypes.c_void_p(ws), nbytes, None)


def test_workspace_size(g):
    assert g.gdn_chunk_workspace_size(4, 16, 4096, 128) == 0
    # the matrix-core KDA prefill's two-kernel form: one 64 KiB record per (stream, chunk)
    assert g.gdn_chunk_workspace_size(2, 32, 8192, 128, kda=True) == 2 * 32 * 128 * 65536
    assert g.gdn_chunk_workspace_size(1, 3, 65, 128, kda=True) == 3 * 2 * 65536
    assert g.gdn_chunk_workspace_size(1, 2, 64, 16, chunk=16, in_dtype=__import__("torch").float32, kda=True) == 0
    assert g.gdn_chunk_workspace_size(1, 2, 64, 16, chunk=16, in_dtype=__import__("torch").float32) == 0
    with pytest.raises(g.GdnError):
        g.gdn_chunk_workspace_size(1, 1, 64, 96)
    n = ctypes.c_size_t(7)
    assert g.lib.gdn_chunk_workspace_size(None, 0, ctypes.byref(n)) == g.GDN_ERROR_INVALID_VALUE


def test_decode_validation_errors(g):
    INV, NS = g.GDN_ERROR_INVALID_VALUE, g.GDN_ERROR_NOT_SUPPORTED
    f = g.lib.gdn_decode_step
    p = [ctypes.c_void_p(FAKE + i * 0x1000000) for i in range(7)]
    assert f(-1, 2, 128, 128, 1, 1, *p, None) == INV
    assert f(2, 2, 128, 64, 1, 1, *p, None) == NS
    assert f(2, 2, 96, 96, 1, 1, *p, None) == NS
    assert f(2, 2, 128, 128, 5, 1, *p, None) == INV
    q = list(p)
    q[0] = None
    assert f(2, 2, 128, 128, 1, 1, *q, None) == INV
    q = list(p)
    q[0] = ctypes.c_void_p(FAKE + 4)          # misaligned state
    assert f(2, 2, 128, 128, 1, 1, *q, None) == INV
    q = list(p)
    q[6] = ctypes.c_void_p(FAKE + 64)         # o inside the state
    assert f(2, 2, 128, 128, 1, 1, *q, None) == INV
    assert f(0, 2, 128, 128, 1, 1, *p, None) == g.GDN_SUCCESS  # no-op


def _ex_desc(g, **kw):
    base = dict(N=4, H=4, H_qk=2, Dk=128, Dv=128, T=2, P=8, in_dtype=g.GDN_BF16, out_dtype=g.GDN_BF16,
                kda=0, qk_l2norm=0, raw_gates=0, write_state=1)
    base.update(kw)
    return g.GdnDecodeExDesc(**base)


def _ex_call(g, d, **ptrs):
    names = ["pool", "slots", "q", "k", "v", "beta", "log_alpha", "A_log", "dt_bias", "n_commit", "o"]
    p = {n: FAKE + i * 0x1000000 for i, n in enumerate(names)}
    p.update(ptrs)
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    return g.lib.gdn_decode_ex(None if d is None else ctypes.byref(d), *[v(p[n]) for n in names], None)


def test_decode_ex_validation_errors(g):
    INV, NS, OK = g.GDN_ERROR_INVALID_VALUE, g.GDN_ERROR_NOT_SUPPORTED, g.GDN_SUCCESS
    assert _ex_call(g, None) == INV
    assert _ex_call(g, _ex_desc(g, H=3, H_qk=2)) == INV            # H not a multiple of H_qk
    assert _ex_call(g, _ex_desc(g, H_qk=0)) == INV
    assert _ex_call(g, _ex_desc(g, T=0)) == INV
    assert _ex_call(g, _ex_desc(g, P=-1)) == INV
    assert _ex_call(g, _ex_desc(g, kda=2)) == INV
    assert _ex_call(g, _ex_desc(g, in_dtype=9)) == INV
    assert _ex_call(g, _ex_desc(g, Dk=128, Dv=64)) == NS
    assert _ex_call(g, _ex_desc(g, Dk=96, Dv=96)) == NS
    assert _ex_call(g, _ex_desc(g, kda=1, raw_gates=1)) == NS
    assert _ex_call(g, _ex_desc(g, P=2), slots=None) == INV          # identity slots need P >= N
    assert _ex_call(g, _ex_desc(g), q=None) == INV
    assert _ex_call(g, _ex_desc(g), pool=FAKE + 8) == INV             # misaligned pool
    assert _ex_call(g, _ex_desc(g), slots=FAKE + 0x1000002) == INV   # misaligned int32 table
    assert _ex_call(g, _ex_desc(g, raw_gates=1), A_log=None) == INV
    assert _ex_call(g, _ex_desc(g), o=FAKE + 64) == INV               # o inside the pool
    # no-ops: empty batch, empty pool, verification without outputs
    assert _ex_call(g, _ex_desc(g, N=0)) == OK
    assert _ex_call(g, _ex_desc(g, P=0)) == OK
    assert _ex_call(g, _ex_desc(g, write_state=0), o=None) == OK


def test_chunk_ex_validation_errors(g):
    INV, NS, OK = g.GDN_ERROR_INVALID_VALUE, g.GDN_ERROR_NOT_SUPPORTED, g.GDN_SUCCESS
    f = g.lib.gdn_chunk_fwd_ex
    p = [ctypes.c_void_p(FAKE + i * 0x1000000) for i in range(12)]
    p[7] = None  # cu_seqlens: not ragged unless a test sets it

    def call(d, **kw):
        q = list(p)
        for i, val in kw.items():
            q[int(i[1:])] = val
        return f(None if d is None else ctypes.byref(d), *q, None)

    def ex(h_qk=2, raw=0, l2=0, **kw):
        return g.GdnChunkExDesc(_desc(g, H=4, **kw), h_qk, raw, l2)

    assert call(None) == INV
    assert call(ex(l2=2)) == INV
    assert call(ex(h_qk=4, l2=1, in_dtype=g.GDN_F32, Dk=16, Dv=16, chunk=16)) == NS   # normalisation: matrix cores
    assert call(ex(h_qk=3)) == INV                        # H = 4 not a multiple of 3
    assert call(ex(h_qk=0)) == INV
    assert call(ex(raw=2)) == INV
    assert call(ex(raw=1), a5=None) == INV                # A_log missing
    assert call(ex(ckpt_every=64), a7=ctypes.c_void_p(FAKE + 0x7000000)) == NS   # ragged + snapshots
    assert call(ex(), a7=ctypes.c_void_p(FAKE + 0x7000002)) == INV              # misaligned cu_seqlens
    assert call(ex(in_dtype=g.GDN_F32)) == NS             # grouped heads: matrix-core path only
    assert call(ex(h_qk=4, in_dtype=g.GDN_F32, Dk=16, Dv=16, chunk=16)) != NS   # plain: vector path
    assert call(ex(B=0)) == OK
