"""The C-ABI library loads, exports every entry point the header declares, and
rejects invalid arguments before touching the GPU (CPU only: no call here
reaches a kernel launch or a device query)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "int4gemv.h")
LIB = os.path.join(ROOT, "int4_group_quantized_quant_amd", "libint4gemv.so")

OK, NULL, SHAPE, ALIGN, ALIAS, ARG = 0, 1, 2, 3, 4, 5


def _ensure_built():
    if not os.path.exists(LIB):
        import __graft_entry__
        __graft_entry__.build()


@pytest.fixture(scope="module")
def lib():
    _ensure_built()
    import int4_group_quantized_quant_amd as pkg
    return pkg.lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(int4_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_every_entry_point():
    names = declared_functions()
    for n in ("int4_quantize_pack", "int4_matvec", "int4_matvec_split4", "int4_matvec_gated",
              "int4_matvec_norm", "int4_matvec_dual", "int4_matvec_sigmoid_gated",
              "int4_matvec_swiglu_gated", "int4_matvec_norm_swiglu", "int4_embedding_gather",
              "int4_status_str", "int4_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol():
    _ensure_built()
    raw = ctypes.CDLL(LIB)
    for name in declared_functions():
        assert hasattr(raw, name), f"{name} declared in int4gemv.h but not exported"


def test_status_strings(lib):
    assert lib.int4_status_str(0) == b"INT4_OK"
    assert lib.int4_status_str(4) == b"INT4_ERR_ALIAS"
    assert lib.int4_status_str(99) == b"INT4_ERR_UNKNOWN"


# Fake, never-dereferenced addresses: every call below fails validation.
A = 0x10000000
B = 0x20000000
C = 0x30000000
D = 0x40000000
E = 0x50000000
F = 0x60000000


def _err(lib):
    return lib.int4_last_error().decode()


def test_matvec_shape_errors(lib):
    assert lib.int4_matvec(A, 1, B, C, D, 16, 256, 48, E, None) == SHAPE      # gs % 32
    assert lib.int4_matvec(A, 1, B, C, D, 16, 256, 0, E, None) == SHAPE       # gs 0
    assert lib.int4_matvec(A, 1, B, C, D, 16, 96, 64, E, None) == SHAPE       # K % gs
    assert lib.int4_matvec(A, 1, B, C, D, 16, 32, 64, E, None) == SHAPE       # K < gs
    assert lib.int4_matvec(A, 9, B, C, D, 16, 256, 64, E, None) == SHAPE      # M > 8
    assert lib.int4_matvec(A, -1, B, C, D, 16, 256, 64, E, None) == SHAPE     # M < 0
    assert lib.int4_matvec(A, 1, B, C, D, -1, 256, 64, E, None) == SHAPE      # N < 0
    assert "group_size" in _err(lib) or "N must" in _err(lib)


def test_empty_calls_are_no_ops(lib):
    # N == 0 or M == 0: nothing to do; pointers are not needed.
    assert lib.int4_matvec(None, 1, None, None, None, 0, 256, 64, None, None) == OK
    assert lib.int4_matvec(None, 0, None, None, None, 16, 256, 64, None, None) == OK
    assert lib.int4_quantize_pack(None, 0, 256, 64, None, None, None, None) == OK
    assert lib.int4_matvec_split4(None, None, None, None, 0, 256, 64, 0, 0, 0,
                                  None, None, None, None, None) == OK
    assert lib.int4_matvec_gated(None, None, None, None, None, None, None, 0, 256, 64,
                                 None, None) == OK
    assert lib.int4_matvec_norm(None, None, None, ctypes.c_float(1e-6), None, None, None, 0,
                                256, 64, None, None, None, None) == OK


def test_null_errors(lib):
    assert lib.int4_matvec(None, 1, B, C, D, 16, 256, 64, E, None) == NULL
    assert lib.int4_matvec(A, 1, B, C, D, 16, 256, 64, None, None) == NULL
    assert lib.int4_quantize_pack(A, 4, 256, 64, None, C, D, None) == NULL
    assert lib.int4_matvec_gated(A, B, C, D, None, E, F, 16, 256, 64, A + 0x1000000, None) == NULL
    assert lib.int4_matvec_norm(A, None, C, ctypes.c_float(1e-6), D, E, F, 4, 256, 64, B,
                                None, None, None) == NULL


def test_alignment_errors(lib):
    assert lib.int4_matvec(A + 4, 1, B, C, D, 16, 256, 64, E, None) == ALIGN   # X 16B
    assert lib.int4_matvec(A, 1, B + 8, C, D, 16, 256, 64, E, None) == ALIGN   # q 16B
    assert lib.int4_matvec(A, 1, B, C + 2, D, 16, 256, 64, E, None) == ALIGN   # scales 4B
    assert lib.int4_matvec(A, 1, B, C, D, 16, 256, 64, E + 1, None) == ALIGN   # Y 4B
    assert lib.int4_quantize_pack(A + 4, 4, 256, 64, B, C, D, None) == ALIGN   # W 16B


def test_alias_errors(lib):
    N, K, gs = 16, 256, 64
    # Y overlapping X / q / scales.
    assert lib.int4_matvec(A, 1, B, C, D, N, K, gs, A + 16, None) == ALIAS
    assert lib.int4_matvec(A, 1, B, C, D, N, K, gs, B + N * K // 2 - 4, None) == ALIAS
    assert lib.int4_matvec(A, 1, B, C, D, N, K, gs, C, None) == ALIAS
    # Adjacent but not overlapping is fine only if nothing else is wrong: here Y
    # ends exactly where q starts, so this passes validation -- not called.
    # split4 outputs overlapping each other.
    assert lib.int4_matvec_split4(A, B, C, D, N, K, gs, 4, 8, 12, E, E + 8, F, F + 64,
                                  None) == ALIAS
    # norm outputs overlapping each other / an input.
    assert lib.int4_matvec_norm(A, A + 0x10000, A + 0x20000, ctypes.c_float(1e-6), B, C, D, N,
                                K, gs, E, E, None, None) == ALIAS
    assert lib.int4_matvec_norm(A, A + 0x10000, A + 0x20000, ctypes.c_float(1e-6), B, C, D, N,
                                K, gs, E, A + 0x10000, None, None) == ALIAS
    # quantize outputs overlapping the input.
    assert lib.int4_quantize_pack(A, N, K, gs, A + 256, C, D, None) == ALIAS
    assert "overlaps" in _err(lib)


def test_split4_argument_errors(lib):
    N, K, gs = 16, 256, 64
    assert lib.int4_matvec_split4(A, B, C, D, N, K, gs, 8, 4, 12, E, F, E + 0x1000, F + 0x1000,
                                  None) == ARG
    assert lib.int4_matvec_split4(A, B, C, D, N, K, gs, 4, 8, 17, E, F, E + 0x1000, F + 0x1000,
                                  None) == ARG
    assert lib.int4_matvec_split4(A, B, C, D, N, K, gs, -1, 8, 12, E, F, E + 0x1000, F + 0x1000,
                                  None) == ARG
    # A NULL output is allowed only for an empty range.
    assert lib.int4_matvec_split4(A, B, C, D, N, K, gs, 4, 8, 12, E, None, E + 0x1000,
                                  F + 0x1000, None) == NULL


def test_norm_eps_errors(lib):
    for eps in (-1e-6, float("nan"), float("inf")):
        assert lib.int4_matvec_norm(A, A + 0x10000, A + 0x20000, ctypes.c_float(eps), B, C, D, 16,
                                    256, 64, E, None, None, None) == ARG


# ------------------------------------------------ dual, input-gated, norm + SwiGLU

G_ = 0x70000000
H_ = 0x80000000


def test_next_variants_empty_calls_are_no_ops(lib):
    assert lib.int4_matvec_dual(None, 1, None, None, None, None, None, None, 0, 256, 64,
                                None, None, None) == OK
    assert lib.int4_matvec_dual(None, 0, None, None, None, None, None, None, 16, 256, 64,
                                None, None, None) == OK
    assert lib.int4_matvec_sigmoid_gated(None, None, 1, None, None, None, 0, 256, 64, None, None) == OK
    assert lib.int4_matvec_swiglu_gated(None, None, 0, None, None, None, 16, 256, 64, None, None) == OK
    assert lib.int4_matvec_norm_swiglu(None, None, None, ctypes.c_float(1e-6), None, None, None,
                                       None, None, None, 0, 256, 64, None, None, None) == OK


def test_next_variants_shape_null_align_alias(lib):
    N, K, gs = 16, 256, 64
    # shapes
    assert lib.int4_matvec_dual(A, 1, B, C, D, E, F, G_, N, K, 48, H_, H_ + 0x1000, None) == SHAPE
    assert lib.int4_matvec_dual(A, 9, B, C, D, E, F, G_, N, K, gs, H_, H_ + 0x1000, None) == SHAPE
    assert lib.int4_matvec_sigmoid_gated(A, A + 0x1000, 1, B, C, D, N, 96, 64, E, None) == SHAPE
    assert lib.int4_matvec_swiglu_gated(A, A + 0x1000, 1, B, C, D, -1, K, gs, E, None) == SHAPE
    assert lib.int4_matvec_swiglu_gated(A, A + 0x1000, -1, B, C, D, N, K, gs, E, None) == SHAPE
    # nulls
    assert lib.int4_matvec_dual(A, 1, B, C, D, E, F, G_, N, K, gs, H_, None, None) == NULL
    assert lib.int4_matvec_sigmoid_gated(A, None, 1, B, C, D, N, K, gs, E, None) == NULL
    assert lib.int4_matvec_swiglu_gated(A, A + 0x1000, 1, B, C, D, N, K, gs, None, None) == NULL
    assert lib.int4_matvec_norm_swiglu(A, A + 0x1000, A + 0x2000, ctypes.c_float(1e-6),
                                       B, C, D, None, F, G_, N, K, gs, H_, None, None) == NULL
    # alignment: the second input vector must be 16-byte aligned too
    assert lib.int4_matvec_sigmoid_gated(A, A + 0x1004, 1, B, C, D, N, K, gs, E, None) == ALIGN
    assert lib.int4_matvec_swiglu_gated(A, A + 0x1000, 1, B + 4, C, D, N, K, gs, E, None) == ALIGN
    assert lib.int4_matvec_dual(A, 1, B, C, D, E + 8, F, G_, N, K, gs, H_, H_ + 0x1000, None) == ALIGN
    # aliasing: outputs against each other and against either input vector
    assert lib.int4_matvec_dual(A, 1, B, C, D, E, F, G_, N, K, gs, H_, H_ + 8, None) == ALIAS
    # with M = 4 lanes y0 spans 4*N floats, so y1 right after N floats overlaps it
    assert lib.int4_matvec_dual(A, 4, B, C, D, E, F, G_, N, K, gs, H_, H_ + 4 * N, None) == ALIAS
    assert lib.int4_matvec_sigmoid_gated(A, A + 0x1000, 1, B, C, D, N, K, gs, A + 0x1010, None) == ALIAS
    assert lib.int4_matvec_swiglu_gated(A, A + 0x1000, 1, B, C, D, N, K, gs, A + 16, None) == ALIAS
    # with M = 2 lanes, y inside the second row of up [2][K] overlaps it
    assert lib.int4_matvec_swiglu_gated(A, A + 0x10000, 2, B, C, D, N, K, gs, A + 0x10000 + 4 * K + 64,
                                        None) == ALIAS
    assert lib.int4_matvec_norm_swiglu(A, A + 0x1000, A + 0x2000, ctypes.c_float(1e-6),
                                       B, C, D, E, F, G_, N, K, gs, H_, H_ + 16, None) == ALIAS
    # eps
    for eps in (-1.0, float("nan")):
        assert lib.int4_matvec_norm_swiglu(A, A + 0x1000, A + 0x2000, ctypes.c_float(eps),
                                           B, C, D, E, F, G_, N, K, gs, H_, None, None) == ARG


def test_embedding_gather_validation(lib):
    K, gs = 256, 64
    assert lib.int4_embedding_gather(None, 0, None, None, None, 16, K, gs, None, None) == OK   # T == 0
    assert lib.int4_embedding_gather(A, -1, B, C, D, 16, K, gs, E, None) == SHAPE
    assert lib.int4_embedding_gather(A, 4, B, C, D, 16, K, 48, E, None) == SHAPE
    assert lib.int4_embedding_gather(None, 4, B, C, D, 16, K, gs, E, None) == NULL
    assert lib.int4_embedding_gather(A, 4, None, C, D, 16, K, gs, E, None) == NULL
    assert lib.int4_embedding_gather(A + 2, 4, B, C, D, 16, K, gs, E, None) == ALIGN
    assert lib.int4_embedding_gather(A, 4, B, C, D, 16, K, gs, E + 4, None) == ALIGN
    assert lib.int4_embedding_gather(A, 4, B, C, D, 16, K, gs, B + 64, None) == ALIAS
    assert lib.int4_embedding_gather(A, 4, B, C, D, 16, K, gs, A - 16, None) == ALIAS


def test_gemm_workspace_and_validation(lib):
    lib.int4_gemm_workspace_bytes.restype = ctypes.c_size_t
    lib.int4_gemm_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32]
    T, N, K, gs = 5, 77, 96, 96
    need = lib.int4_gemm_workspace_bytes(T, N, K, gs)
    # Tp=128, Kp=128, Np=256, Gp=2: split activations 128*128*4, factors 128*4,
    # two transposed tables 2*128*4 each, every region rounded up to 256 bytes.
    assert need == 128 * 128 * 4 + 512 + 2048 + 2048
    assert lib.int4_gemm_workspace_bytes(0, N, K, gs) == 0
    W = 0x90000000
    sz = ctypes.c_size_t
    assert lib.int4_gemm(None, 0, None, None, None, N, K, gs, None, None, sz(0), None) == OK
    assert lib.int4_gemm(A, T, B, C, D, N, K, 48, E, W, sz(need), None) == SHAPE
    assert lib.int4_gemm(A, T, B, C, D, N, K, gs, E, W, sz(need - 1), None) == SHAPE
    assert lib.int4_gemm(A, T, B, C, D, N, K, gs, E, None, sz(need), None) == NULL
    assert lib.int4_gemm(A, T, B, C, D, N, K, gs, None, W, sz(need), None) == NULL
    assert lib.int4_gemm(A, T, B, C, D, N, K, gs, E, W + 128, sz(need), None) == ALIGN
    assert lib.int4_gemm(A + 4, T, B, C, D, N, K, gs, E, W, sz(need), None) == ALIGN
    assert lib.int4_gemm(A, T, B, C, D, N, K, gs, E, A, sz(need), None) == ALIAS      # workspace over X
    assert lib.int4_gemm(A, T, B, C, D, N, K, gs, W + 64, W, sz(need), None) == ALIAS  # Y inside workspace
    assert lib.int4_gemm(A, T, B, C, D, 1 << 20, 1 << 12, 128, E, W, sz(1 << 40), None) == SHAPE  # N*K/2 >= 2^31
    assert "2^31" in _err(lib)


def test_gemm_noalloc_validation(lib):
    # Every case fails (or returns) before the library looks up its scratch
    # array, so none of them touches a device.
    lib.int4_gemm_workspace_bytes.restype = ctypes.c_size_t
    lib.int4_gemm_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32]
    T, N, K, gs = 5, 77, 96, 96
    assert lib.int4_gemm_noalloc(None, 0, None, None, None, N, K, gs, None, None) == OK   # T == 0
    assert lib.int4_gemm_noalloc(A, T, B, C, D, 0, K, gs, None, None) == OK               # N == 0
    assert lib.int4_gemm_noalloc(A, -1, B, C, D, N, K, gs, E, None) == SHAPE
    assert lib.int4_gemm_noalloc(A, T, B, C, D, N, K, 48, E, None) == SHAPE
    assert lib.int4_gemm_noalloc(A, T, B, C, D, N, K, gs, None, None) == NULL
    assert lib.int4_gemm_noalloc(None, T, B, C, D, N, K, gs, E, None) == NULL
    assert lib.int4_gemm_noalloc(A + 4, T, B, C, D, N, K, gs, E, None) == ALIGN
    assert lib.int4_gemm_noalloc(A, T, B, C, D, N, K, gs, A + 16, None) == ALIAS         # Y over X
    # The scratch holds 64 MiB: T = 4096 at K = 4096 needs more and is refused.
    big = lib.int4_gemm_workspace_bytes(4096, 4096, 4096, 128)
    assert big > 64 << 20
    assert lib.int4_gemm_noalloc(A, 4096, B, C, D, 4096, 4096, 128, E, None) == SHAPE
    assert "scratch" in _err(lib)
    assert lib.int4_gemm_workspace_bytes(3968, 4096, 4096, 128) <= 64 << 20


def test_probe_validation(lib):
    sz = ctypes.c_size_t
    assert lib.int4_probe_stream_read(None, sz(1024), 4, 8, 4, B, None) == NULL
    assert lib.int4_probe_stream_read(A, sz(1024), 4, 8, 4, None, None) == NULL
    assert lib.int4_probe_stream_read(A + 8, sz(1024), 4, 8, 4, B, None) == ALIGN
    assert lib.int4_probe_stream_read(A, sz(1000), 4, 8, 4, B, None) == ALIGN
    assert lib.int4_probe_stream_read(A, sz(1024), 0, 8, 4, B, None) == SHAPE
    assert lib.int4_probe_stream_read(A, sz(1024), 4, 17, 4, B, None) == SHAPE
    assert lib.int4_probe_stream_read(A, sz(1 << 32), 1, 8, 4, B, None) == SHAPE  # a 4 GiB slice
    assert lib.int4_probe_stream_read(A, sz(1024), 4, 8, 3, B, None) == ARG


def test_mlp_workspace_and_validation(lib):
    lib.int4_mlp_workspace_bytes.restype = ctypes.c_size_t
    need = lib.int4_mlp_workspace_bytes()
    assert need >= 12
    sz = ctypes.c_size_t
    Dm, Fm, gs = 256, 512, 128
    base = 0x100000000
    x, qg, sg, zg, qu, su, zu, qd, sd, zd, h, y, ws = (base + i * 0x10000000 for i in range(13))

    def call(**kw):
        a = dict(x=x, qg=qg, sg=sg, zg=zg, qu=qu, su=su, zu=zu, qd=qd, sd=sd, zd=zd, D=Dm, F=Fm, gs=gs,
                 h=h, y=y, ws=ws, wsb=need)
        a.update(kw)
        return lib.int4_mlp(a["x"], a["qg"], a["sg"], a["zg"], a["qu"], a["su"], a["zu"], a["qd"], a["sd"],
                            a["zd"], a["D"], a["F"], a["gs"], a["h"], a["y"], a["ws"], sz(a["wsb"]), None)

    assert call(gs=48) == SHAPE
    assert call(F=Fm + 32) == SHAPE          # F not a multiple of the group size
    assert call(D=64) == SHAPE               # D below the group size
    assert call(x=None) == NULL
    assert call(zd=None) == NULL
    assert call(h=None) == NULL
    assert call(ws=None) == NULL
    assert "workspace" in _err(lib)
    assert call(wsb=need - 1) == SHAPE
    assert call(h=h + 4) == ALIGN            # h is the down projection's input: 16-byte aligned
    assert call(x=x + 8) == ALIGN
    assert call(qd=qd + 4) == ALIGN
    assert call(ws=ws + 2) == ALIGN
    assert call(y=x) == ALIAS                # y over x
    assert call(h=qd) == ALIAS               # h over the down codes
    assert call(ws=h + 16) == ALIAS          # workspace inside h
    assert call(y=h + 64) == ALIAS           # y inside h


def test_mlp_timed_out_validation(lib):
    out = ctypes.c_int32(7)
    assert lib.int4_mlp_timed_out(None, ctypes.byref(out), None) == NULL
    assert lib.int4_mlp_timed_out(0x100000000, None, None) == NULL
    assert lib.int4_mlp_timed_out(0x100000004, ctypes.byref(out), None) == ALIGN
    assert out.value == 7                    # untouched on an error


def test_embedding_gather_host_validation(lib):
    # Every error below is found before the table pointers are examined (no
    # runtime call is made).
    q, s, z, ids, out = (0x100000000 + i * 0x10000000 for i in range(5))
    N, K, gs, T = 64, 512, 64, 3
    assert lib.int4_embedding_gather_host(ids, 0, q, s, z, N, K, gs, out, None) == OK        # T == 0
    assert lib.int4_embedding_gather_host(ids, T, q, s, z, N, K, 48, out, None) == SHAPE
    assert lib.int4_embedding_gather_host(ids, -1, q, s, z, N, K, gs, out, None) == SHAPE
    assert lib.int4_embedding_gather_host(None, T, q, s, z, N, K, gs, out, None) == NULL
    assert lib.int4_embedding_gather_host(ids, T, None, s, z, N, K, gs, out, None) == NULL
    assert lib.int4_embedding_gather_host(ids, T, q, s, z, N, K, gs, out + 4, None) == ALIGN
    assert lib.int4_embedding_gather_host(ids, T, q, s, z, N, K, gs, q + 64, None) == ALIAS   # out over q
