"""C-ABI checks that need no GPU: the library loads, exports every function
include/sala.h declares, and rejects bad arguments on the host (before any
HIP call) with the documented status codes."""

import ctypes
import os
import re

import pytest

from hybrid_sparse_linear_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libsala.so not built")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3
F32, BF16 = 0, 1
P = ctypes.c_void_p
A = ctypes.c_void_p(0x10000)  # aligned, never dereferenced: every call below fails validation first
MIS = ctypes.c_void_p(0x10004)
NUL = ctypes.c_void_p(0)


def declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(sala_\w+)\s*\(", text, re.M))
    return names


def test_header_symbols_exported():
    names = declared_functions()
    assert {"sala_linear_prefill", "sala_linear_decode", "sala_sparse_select", "sala_sparse_prefill",
            "sala_sparse_decode"} <= names
    handle = ctypes.CDLL(_lib.LIB_PATH)
    for n in sorted(names):
        assert hasattr(handle, n), n


def test_status_strings_and_version():
    L = _lib.lib()
    for code, name in _lib.STATUS.items():
        assert L.sala_status_string(code).decode() == name
    assert L.sala_status_string(-99).decode() == "SALA_ERR_UNKNOWN"
    assert b"gfx950" in L.sala_version()


def lp(**kw):
    a = dict(dtype=BF16, B=1, H=2, N=256, d=128, chunk=128, q=A, k=A, v=A, o=A, decay=NUL, sin=NUL, sout=NUL,
             ws=NUL, wsb=0)
    a.update(kw)
    return _lib.lib().sala_linear_prefill(a["dtype"], a["B"], a["H"], a["N"], a["d"], a["chunk"], a["q"], a["k"],
                                          a["v"], a["o"], a["decay"], a["sin"], a["sout"], a["ws"], a["wsb"], NUL)


def test_linear_prefill_validation():
    assert lp(dtype=7) == INVALID
    assert lp(N=0) == INVALID
    assert lp(B=0) == INVALID
    assert lp(d=96) == UNSUPPORTED
    assert lp(chunk=32) == UNSUPPORTED
    assert lp(N=1 << 23) == UNSUPPORTED  # bf16: one head's rows reach 2 GiB
    assert lp(N=(1 << 23) - 1, ws=NUL, wsb=0) == WORKSPACE  # just under: accepted up to the workspace check
    assert lp(q=NUL) == INVALID
    assert lp(o=MIS) == INVALID
    assert lp(sin=MIS) == INVALID
    assert lp(q=NUL) == INVALID and b"q must not be NULL" in _lib.lib().sala_last_error()


def test_linear_prefill_workspace_rules():
    L = _lib.lib()
    need = L.sala_linear_prefill_workspace(BF16, 1, 32, 32768, 128, 128)
    assert need > 0 and need % (128 * 128 * 4) == 0
    # fp32 tiles by 32 tokens whatever the chunk: segment states of d * d floats
    f32 = L.sala_linear_prefill_workspace(F32, 1, 32, 32768, 128, 128)
    assert f32 > 0 and f32 % (128 * 128 * 4) == 0
    assert f32 == L.sala_linear_prefill_workspace(F32, 1, 32, 32768, 128, 64)
    assert L.sala_linear_prefill_workspace(F32, 1, 1, 32, 64, 64) == 0  # one tile: one segment, no workspace
    assert lp(B=1, H=32, N=32768, ws=NUL, wsb=0) == WORKSPACE
    assert lp(B=1, H=32, N=32768, ws=A, wsb=need - 1) == WORKSPACE
    assert L.sala_linear_prefill_workspace(BF16, 1, 32, 100, 128, 128) == 0  # one segment: no workspace


def test_linear_decode_validation():
    L = _lib.lib()
    assert L.sala_linear_decode(BF16, 1, 2, 128, A, A, A, A, NUL, NUL, NUL) == INVALID  # state NULL
    assert L.sala_linear_decode(BF16, 1, 2, 80, A, A, A, A, NUL, A, NUL) == UNSUPPORTED
    assert L.sala_linear_decode(3, 1, 2, 128, A, A, A, A, NUL, A, NUL) == INVALID


def ss(**kw):
    a = dict(dtype=BF16, B=1, Hq=4, Hkv=2, d=128, Nq=256, L=256, block=64, topk=4, n_init=1, n_local=2, q=A, k=A,
             kp=A, idx=A, scores=NUL, ws=NUL, wsb=0)
    a.update(kw)
    return _lib.lib().sala_sparse_select(a["dtype"], a["B"], a["Hq"], a["Hkv"], a["d"], a["Nq"], a["L"], a["block"],
                                         a["topk"], a["n_init"], a["n_local"], a["q"], a["k"], a["kp"], a["idx"],
                                         a["scores"], a["ws"], a["wsb"], NUL)


def test_sparse_select_validation():
    assert ss(Hq=3) == INVALID            # Hq not a multiple of Hkv
    assert ss(block=32) == UNSUPPORTED
    assert ss(Nq=7) == UNSUPPORTED
    assert ss(topk=-1) == INVALID
    assert ss(topk=0, n_init=0, n_local=0) == INVALID
    assert ss(kp=NUL) == INVALID
    assert ss(idx=MIS) == INVALID
    assert ss() == WORKSPACE              # prefill needs qbar + scores workspace
    L = _lib.lib()
    need = L.sala_sparse_select_workspace(BF16, 1, 4, 2, 128, 256, 256, 64, 4, 1, 2)
    assert need == 2 * 4 * 128 * 4 + 2 * 4 * 4 * 4
    assert ss(ws=A, wsb=need - 4) == WORKSPACE


def test_sparse_prefill_and_decode_validation():
    L = _lib.lib()
    f = L.sala_sparse_prefill
    # the sparse prefill needs no workspace (NULL is accepted); the remaining
    # cases fail validation before any device work
    assert L.sala_sparse_prefill_workspace(BF16, 1, 32, 2, 262144, 128, 64, 67) == 0
    assert L.sala_sparse_prefill_workspace(F32, 1, 4, 2, 2048, 64, 64, 7) == 0
    assert f(BF16, 1, 4, 3, 256, 128, 64, 7, ctypes.c_float(0.1), A, A, A, A, A, NUL, 0, NUL) == INVALID
    assert f(BF16, 1, 4, 2, 256, 128, 64, 0, ctypes.c_float(0.1), A, A, A, A, A, NUL, 0, NUL) == UNSUPPORTED
    assert f(BF16, 1, 4, 2, 256, 128, 64, 7, ctypes.c_float(float("nan")), A, A, A, A, A, A, 1 << 30, NUL) == INVALID
    assert f(F32, 1, 4, 2, 256, 128, 64, 7, ctypes.c_float(0.1), A, NUL, A, A, A, NUL, 0, NUL) == INVALID
    g = L.sala_sparse_decode
    assert g(BF16, 1, 128, 2, 4096, 128, 64, 67, ctypes.c_float(0.1), A, A, A, A, A, A, 1 << 30, NUL) == UNSUPPORTED
    assert g(BF16, 1, 32, 2, 4096, 128, 64, 67, ctypes.c_float(0.1), A, A, A, A, A, NUL, 0, NUL) == WORKSPACE
    assert L.sala_sparse_decode_workspace(BF16, 4, 32, 2, 1 << 20, 128, 64, 67) > 0


def test_empty_inputs_are_rejected():
    # a zero batch, head count or length is an argument error at every entry
    # point, reported before any device work
    L = _lib.lib()
    assert lp(N=0) == INVALID and lp(H=0) == INVALID
    assert L.sala_linear_decode(BF16, 0, 2, 128, A, A, A, A, NUL, A, NUL) == INVALID
    assert L.sala_linear_decode(BF16, 1, 0, 128, A, A, A, A, NUL, A, NUL) == INVALID
    assert ss(L=0, Nq=0) == INVALID and ss(B=0) == INVALID and ss(Hkv=0) == INVALID
    f = L.sala_sparse_prefill
    assert f(BF16, 0, 4, 2, 256, 128, 64, 7, ctypes.c_float(0.1), A, A, A, A, A, NUL, 0, NUL) == INVALID
    assert f(BF16, 1, 4, 2, 0, 128, 64, 7, ctypes.c_float(0.1), A, A, A, A, A, NUL, 0, NUL) == INVALID
    g = L.sala_sparse_decode
    assert g(BF16, 1, 32, 2, 0, 128, 64, 67, ctypes.c_float(0.1), A, A, A, A, A, A, 1 << 30, NUL) == INVALID
    assert g(BF16, 0, 32, 2, 4096, 128, 64, 67, ctypes.c_float(0.1), A, A, A, A, A, A, 1 << 30, NUL) == INVALID


def test_dense_prefill_and_ceiling_validation():
    L = _lib.lib()
    f = L.sala_dense_prefill
    assert f(F32, 1, 4, 2, 256, 128, ctypes.c_float(0.1), A, A, A, A, NUL) == UNSUPPORTED
    assert f(BF16, 1, 4, 3, 256, 128, ctypes.c_float(0.1), A, A, A, A, NUL) == INVALID
    assert f(BF16, 1, 4, 2, 256, 96, ctypes.c_float(0.1), A, A, A, A, NUL) == UNSUPPORTED
    assert f(BF16, 1, 4, 2, 0, 128, ctypes.c_float(0.1), A, A, A, A, NUL) == INVALID
    assert f(BF16, 1, 4, 2, 256, 128, ctypes.c_float(float("nan")), A, A, A, A, NUL) == INVALID
    assert f(BF16, 1, 4, 2, 256, 128, ctypes.c_float(0.1), A, NUL, A, A, NUL) == INVALID
    assert L.sala_ceiling_mfma(0, 10, A, NUL) == INVALID
    assert L.sala_ceiling_mfma(4, 10, NUL, NUL) == INVALID
    assert L.sala_ceiling_copy(A, A, 17, NUL) == INVALID
    assert L.sala_ceiling_copy(NUL, A, 16, NUL) == INVALID
    assert L.sala_ceiling_read(A, 17, A, NUL) == INVALID
    assert L.sala_ceiling_read(NUL, 16, A, NUL) == INVALID
    assert L.sala_ceiling_read(A, 16, NUL, NUL) == INVALID


def lpf(**kw):
    a = dict(dtype=BF16, B=1, H=2, N=256, d=128, chunk=128, q=A, k=A, v=A, o=A, decay=NUL, sin=NUL, sout=NUL,
             gq=NUL, gk=NUL, eps=1e-6, base=10000.0, pos0=0, gate=NUL, ws=NUL, wsb=0)
    a.update(kw)
    return _lib.lib().sala_linear_prefill_fused(
        a["dtype"], a["B"], a["H"], a["N"], a["d"], a["chunk"], a["q"], a["k"], a["v"], a["o"], a["decay"], a["sin"],
        a["sout"], a["gq"], a["gk"], a["eps"], a["base"], a["pos0"], a["gate"], a["ws"], a["wsb"], NUL)


def ldf(**kw):
    a = dict(dtype=BF16, B=2, H=2, d=128, q=A, k=A, v=A, o=A, decay=NUL, state=A, gq=NUL, gk=NUL, eps=1e-6,
             base=10000.0, pos=A, gate=NUL)
    a.update(kw)
    return _lib.lib().sala_linear_decode_fused(a["dtype"], a["B"], a["H"], a["d"], a["q"], a["k"], a["v"], a["o"],
                                               a["decay"], a["state"], a["gq"], a["gk"], a["eps"], a["base"],
                                               a["pos"], a["gate"], NUL)


def test_fused_linear_validation():
    assert lpf(dtype=F32) == UNSUPPORTED
    assert lpf(dtype=5) == INVALID
    assert lpf(N=0) == INVALID
    assert lpf(d=80) == UNSUPPORTED
    assert lpf(eps=-1.0) == INVALID
    assert lpf(eps=float("nan")) == INVALID
    assert lpf(base=0.5) == INVALID and b"rope_base" in _lib.lib().sala_last_error()
    assert lpf(base=float("nan")) == INVALID
    assert lpf(pos0=-1) == INVALID
    assert lpf(gate=MIS) == INVALID
    assert lpf(gq=MIS) == INVALID
    assert lpf(N=16 * 1024 * 1024, H=1) == UNSUPPORTED  # one head's rows past 2 GiB
    assert lpf(B=1, H=32, N=32768, ws=NUL, wsb=0) == WORKSPACE
    assert ldf(dtype=3) == INVALID
    assert ldf(pos=NUL) == INVALID and b"pos" in _lib.lib().sala_last_error()
    assert ldf(state=NUL) == INVALID
    assert ldf(base=1.0) == INVALID
    assert ldf(gk=MIS) == INVALID
    assert ldf(d=32) == UNSUPPORTED


def test_standalone_neighbour_validation():
    L = _lib.lib()
    nr = lambda **kw: L.sala_qk_norm_rope(kw.get("dtype", BF16), kw.get("B", 1), kw.get("H", 2), kw.get("N", 10),
                                          kw.get("d", 128), kw.get("x", A), kw.get("out", A), kw.get("gamma", NUL),
                                          kw.get("eps", 1e-6), kw.get("base", 10000.0), kw.get("pos0", 0), NUL)
    assert nr(dtype=9) == INVALID
    assert nr(N=0) == INVALID
    assert nr(d=100) == UNSUPPORTED
    assert nr(x=NUL) == INVALID
    assert nr(out=MIS) == INVALID
    assert nr(gamma=MIS) == INVALID
    assert nr(base=-3.0) == INVALID
    assert nr(pos0=-5) == INVALID
    og = lambda **kw: L.sala_output_gate(kw.get("dtype", BF16), kw.get("n", 64), kw.get("o", A), kw.get("g", A),
                                         kw.get("out", A), NUL)
    assert og(n=0) == INVALID
    assert og(n=12) == INVALID and b"multiple of 8" in L.sala_last_error()
    assert og(g=NUL) == INVALID
    assert og(out=MIS) == INVALID
    assert og(dtype=2) == INVALID


def test_generation_loop_validation():
    L = _lib.lib()

    def chunk(**kw):
        a = dict(dtype=BF16, B=1, Hq=4, Hkv=2, cap=1000, d=128, pos0=64, n=100, block=64, topk=4, ni=1, nl=2,
                 scale=0.1, ws=NUL, wsb=0)
        a.update(kw)
        return L.sala_sparse_prefill_chunk(a["dtype"], a["B"], a["Hq"], a["Hkv"], a["cap"], a["d"], a["pos0"], a["n"],
                                           a["block"], a["topk"], a["ni"], a["nl"], a["scale"], A, A, A, A, A, A, A, A,
                                           a["ws"], a["wsb"], NUL)

    def step(**kw):
        a = dict(dtype=BF16, B=1, Hq=4, Hkv=2, cap=1000, d=128, pos=500, block=64, topk=4, ni=1, nl=2, scale=0.1,
                 ws=NUL, wsb=0, k_cache=A)
        a.update(kw)
        return L.sala_sparse_decode_step(a["dtype"], a["B"], a["Hq"], a["Hkv"], a["cap"], a["d"], a["pos"], a["block"],
                                         a["topk"], a["ni"], a["nl"], a["scale"], A, A, A, a["k_cache"], A, A, A, A,
                                         a["ws"], a["wsb"], NUL)

    assert chunk(n=0) == INVALID
    assert chunk(pos0=70) == UNSUPPORTED and b"block boundary" in L.sala_last_error()
    assert chunk(pos0=960, n=100) == INVALID  # past the capacity
    assert chunk(Hq=3) == INVALID
    assert chunk(scale=float("nan")) == INVALID
    assert chunk() == WORKSPACE
    assert L.sala_sparse_prefill_chunk_workspace(BF16, 1, 4, 2, 1000, 128, 100, 64, 4, 1, 2) > 0
    assert chunk(ws=A, wsb=1) == WORKSPACE
    assert step(pos=1000) == INVALID and b"capacity" in L.sala_last_error()
    assert step(pos=-1) == INVALID
    assert step(k_cache=MIS) == INVALID
    assert step(d=48) == UNSUPPORTED
    assert step() == WORKSPACE
    assert L.sala_sparse_decode_step_workspace(BF16, 1, 4, 2, 1000, 128, 64, 4, 1, 2) > 0


def test_generic_workspace_query_matches_per_op_queries():
    """sala_workspace_bytes(op, dims, ndims) returns what each per-op query returns,
    and (size_t)-1 with a message for an unknown op, a wrong dimension count,
    NULL dims or a dimension beyond int."""
    L = _lib.lib()
    cases = [
        (0, L.sala_linear_prefill_workspace, (BF16, 1, 32, 32768, 128, 128)),
        (0, L.sala_linear_prefill_workspace, (BF16, 2, 3, 1000, 128, 64)),
        (1, L.sala_sparse_select_workspace, (BF16, 1, 32, 2, 128, 131072, 131072, 64, 64, 1, 2)),
        (1, L.sala_sparse_select_workspace, (BF16, 4, 32, 2, 128, 1, 1048576, 64, 64, 1, 2)),
        (2, L.sala_sparse_prefill_workspace, (BF16, 1, 32, 2, 262144, 128, 64, 67)),
        (3, L.sala_sparse_decode_workspace, (BF16, 4, 32, 2, 1048576, 128, 64, 67)),
        (4, L.sala_sparse_prefill_chunk_workspace, (BF16, 2, 8, 2, 587, 128, 256, 64, 3, 1, 2)),
        (5, L.sala_sparse_decode_step_workspace, (BF16, 2, 8, 2, 587, 128, 64, 3, 1, 2)),
        (6, L.sala_sparse_prefill_backward_workspace, (BF16, 1, 32, 2, 262144, 128, 64, 67)),
    ]
    for op, fn, dims in cases:
        arr = (ctypes.c_int64 * len(dims))(*dims)
        want = fn(*dims)
        assert L.sala_workspace_bytes(op, arr, len(dims)) == want, (op, dims)
    bad = ctypes.c_size_t(-1).value
    arr = (ctypes.c_int64 * 6)(BF16, 1, 2, 256, 128, 128)
    assert L.sala_workspace_bytes(7 + 3, arr, 6) == bad and b"unknown operation" in L.sala_last_error()
    assert L.sala_workspace_bytes(-1, arr, 6) == bad
    assert L.sala_workspace_bytes(0, arr, 5) == bad and b"takes 6" in L.sala_last_error()
    assert L.sala_workspace_bytes(0, None, 6) == bad and b"NULL" in L.sala_last_error()
    big = (ctypes.c_int64 * 6)(BF16, 1, 2, 1 << 40, 128, 128)
    assert L.sala_workspace_bytes(0, big, 6) == bad and b"does not fit" in L.sala_last_error()
    # the binding's query goes through the generic call
    import hybrid_sparse_linear_amd as sala
    assert sala.workspace_bytes("linear_prefill", dtype=BF16, B=1, H=32, N=32768, d=128, chunk=128) == \
        L.sala_linear_prefill_workspace(BF16, 1, 32, 32768, 128, 128)
    with pytest.raises(ValueError):
        sala.workspace_bytes("no_such_op")


def test_decode_selection_accepts_large_groups():
    """Decode selection sums every query head of a group (no upper limit on G);
    here the call gets as far as the workspace check for G = 64."""
    assert ss(Hq=128, Hkv=2, Nq=1, L=64 * 300, topk=8) == WORKSPACE


def test_noalloc_decode_step_validation():
    """The allocation-free decode step validates like the decode step, and rejects
    a step whose workspace exceeds its fixed scratch array, before any HIP call."""
    L = _lib.lib()

    def step(**kw):
        a = dict(dtype=BF16, B=4, Hq=32, Hkv=2, cap=1 << 20, d=128, pos=(1 << 20) - 1, block=64, topk=64, n_init=1,
                 n_local=2)
        a.update(kw)
        return L.sala_sparse_decode_step_noalloc(a["dtype"], a["B"], a["Hq"], a["Hkv"], a["cap"], a["d"], a["pos"],
                                                 a["block"], a["topk"], a["n_init"], a["n_local"],
                                                 ctypes.c_float(0.088), A, A, A, A, A, A, A, A, NUL)
    assert step(pos=1 << 20) == INVALID
    assert step(d=96) == UNSUPPORTED
    assert step(Hq=3) == INVALID
    # B = 64 rows of 32 heads: 64 * 32 * 67 split partials of 130 floats = 71 MB > 16 MiB
    assert step(B=64) == WORKSPACE and b"scratch" in L.sala_last_error()
    need = L.sala_sparse_decode_step_workspace(BF16, 4, 32, 2, 1 << 20, 128, 64, 64, 1, 2)
    assert 0 < need <= 16 << 20
