"""Python binding of libint4gemv.so, the int4 group-quantized matvec library
for MI355X (gfx950).  The C ABI is declared in include/int4gemv.h.

This module only marshals arguments: it checks dtypes, devices,
contiguity and element counts of torch tensors (the C ABI takes bare
pointers, so a short buffer would otherwise be read or written past its
end), allocates outputs with torch when the caller passes none, and calls the C entry point of the same name on torch's current
HIP stream.  Every step of the computation runs in the library's HIP kernels;
there is no CPU or PyTorch fallback.  If the library has not been built, the
import fails.

Weight layout (as in the header): q uint32 (or int32 with the same bits)
[N, K/8], scales / zeros float32 [N, K/gs]; activations and outputs float32.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "Int4Error", "int4_quantize_pack", "int4_matvec", "int4_matvec_split4",
    "int4_matvec_gated", "int4_matvec_norm", "int4_matvec_dual", "int4_matvec_sigmoid_gated",
    "int4_matvec_swiglu_gated", "int4_matvec_norm_swiglu", "int4_embedding_gather", "int4_gemm",
    "int4_gemm_workspace_bytes", "int4_matvec_gated_lanes", "int4_mlp", "int4_mlp_workspace_bytes",
    "int4_mlp_timed_out", "int4_embedding_gather_host",
    "int4_gemm_noalloc", "INT4_GEMM_NOALLOC_SCRATCH_BYTES", "int4_probe_stream_read", "lib", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libint4gemv.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python -c 'import __graft_entry__ as g; g.build()')")

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32

lib = ctypes.CDLL(LIB_PATH)
lib.int4_status_str.argtypes = [ctypes.c_int]
lib.int4_status_str.restype = ctypes.c_char_p
lib.int4_last_error.argtypes = []
lib.int4_last_error.restype = ctypes.c_char_p
lib.int4_quantize_pack.argtypes = [_vp, _i64, _i64, _i32, _vp, _vp, _vp, _vp]
lib.int4_matvec.argtypes = [_vp, _i32, _vp, _vp, _vp, _i64, _i64, _i32, _vp, _vp]
lib.int4_matvec_split4.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i32, _i64, _i64, _i64,
                                   _vp, _vp, _vp, _vp, _vp]
lib.int4_matvec_gated.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i32, _vp, _vp]
lib.int4_matvec_norm.argtypes = [_vp, _vp, _vp, ctypes.c_float, _vp, _vp, _vp, _i64, _i64, _i32,
                                 _vp, _vp, _vp, _vp]
lib.int4_matvec_dual.argtypes = [_vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i32, _vp, _vp, _vp]
lib.int4_matvec_sigmoid_gated.argtypes = [_vp, _vp, _i32, _vp, _vp, _vp, _i64, _i64, _i32, _vp, _vp]
lib.int4_matvec_swiglu_gated.argtypes = [_vp, _vp, _i32, _vp, _vp, _vp, _i64, _i64, _i32, _vp, _vp]
lib.int4_matvec_norm_swiglu.argtypes = [_vp, _vp, _vp, ctypes.c_float, _vp, _vp, _vp, _vp, _vp, _vp,
                                        _i64, _i64, _i32, _vp, _vp, _vp]
lib.int4_embedding_gather.argtypes = [_vp, _i64, _vp, _vp, _vp, _i64, _i64, _i32, _vp, _vp]
lib.int4_embedding_gather_host.argtypes = [_vp, _i64, _vp, _vp, _vp, _i64, _i64, _i32, _vp, _vp]
lib.int4_embedding_gather_host.restype = ctypes.c_int
lib.int4_matvec_gated_lanes.argtypes = [_vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i32, _vp, _vp]
lib.int4_matvec_gated_lanes.restype = ctypes.c_int
lib.int4_gemm_workspace_bytes.argtypes = [_i64, _i64, _i64, _i32]
lib.int4_gemm_workspace_bytes.restype = ctypes.c_size_t
lib.int4_gemm.argtypes = [_vp, _i64, _vp, _vp, _vp, _i64, _i64, _i32, _vp, _vp, ctypes.c_size_t, _vp]
lib.int4_gemm_noalloc.argtypes = [_vp, _i64, _vp, _vp, _vp, _i64, _i64, _i32, _vp, _vp]
lib.int4_gemm_noalloc.restype = ctypes.c_int
lib.int4_probe_stream_read.argtypes = [_vp, ctypes.c_size_t, _i32, _i32, _i32, _vp, _vp]
lib.int4_probe_stream_read.restype = ctypes.c_int
lib.int4_mlp_workspace_bytes.argtypes = []
lib.int4_mlp_workspace_bytes.restype = ctypes.c_size_t
lib.int4_mlp.argtypes = [_vp] * 10 + [_i64, _i64, _i32, _vp, _vp, _vp, ctypes.c_size_t, _vp]
lib.int4_mlp.restype = ctypes.c_int
lib.int4_mlp_timed_out.argtypes = [_vp, ctypes.POINTER(ctypes.c_int32), _vp]
lib.int4_mlp_timed_out.restype = ctypes.c_int
for _fn in (lib.int4_gemm, lib.int4_embedding_gather, lib.int4_quantize_pack, lib.int4_matvec, lib.int4_matvec_split4,
            lib.int4_matvec_gated, lib.int4_matvec_norm, lib.int4_matvec_dual,
            lib.int4_matvec_sigmoid_gated, lib.int4_matvec_swiglu_gated,
            lib.int4_matvec_norm_swiglu):
    _fn.restype = ctypes.c_int


class Int4Error(RuntimeError):
    """A library call returned a status other than INT4_OK."""

    def __init__(self, status: int):
        self.status = status
        msg = lib.int4_last_error().decode() or lib.int4_status_str(status).decode()
        super().__init__(msg)


def _check(status: int) -> None:
    if status != 0:
        raise Int4Error(status)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: torch.Tensor, name: str, dtypes) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _size(t: torch.Tensor, n: int, name: str) -> torch.Tensor:
    if t.numel() != n:
        raise ValueError(f"{name} holds {t.numel()} elements; the call needs {n}")
    return t


_F32 = (torch.float32,)
_CODES = (torch.int32, torch.uint32)


def _weights(q, scales, zeros, tag=""):
    _dev(q, "q" + tag, _CODES)
    _dev(scales, "scales" + tag, _F32)
    _dev(zeros, "zeros" + tag, _F32)
    if q.dim() != 2 or scales.dim() != 2 or scales.shape != zeros.shape:
        raise ValueError("q must be [N, K/8] and scales/zeros [N, K/gs]")
    if scales.shape[0] != q.shape[0]:
        raise ValueError("q and scales disagree on N")
    N, K = q.shape[0], q.shape[1] * 8
    G = scales.shape[1]
    if G == 0 or K % G:
        raise ValueError(f"K={K} is not a multiple of the group count {G}")
    return N, K, K // G


def int4_quantize_pack(W: torch.Tensor, group_size: int, q=None, scales=None, zeros=None,
                       stream=None):
    """W float32 [N, K] -> (q int32 [N, K/8], scales [N, K/gs], zeros [N, K/gs])."""
    _dev(W, "W", _F32)
    if W.dim() != 2:
        raise ValueError("W must be [N, K]")
    N, K = W.shape
    G = K // group_size if group_size > 0 else 0
    q = torch.empty((N, K // 8), dtype=torch.int32, device=W.device) if q is None else q
    scales = torch.empty((N, G), dtype=torch.float32, device=W.device) if scales is None else scales
    zeros = torch.empty((N, G), dtype=torch.float32, device=W.device) if zeros is None else zeros
    _size(_dev(q, "q", _CODES), N * (K // 8), "q")
    _size(_dev(scales, "scales", _F32), N * G, "scales")
    _size(_dev(zeros, "zeros", _F32), N * G, "zeros")
    _check(lib.int4_quantize_pack(_ptr(W), N, K, group_size, _ptr(q), _ptr(scales), _ptr(zeros),
                                  _stream(stream)))
    return q, scales, zeros


def int4_matvec(X: torch.Tensor, q, scales, zeros, Y=None, stream=None) -> torch.Tensor:
    """X float32 [M, K] (or [K]) -> Y float32 [M, N] (or [N]); 0 <= M <= 8."""
    N, K, gs = _weights(q, scales, zeros)
    _dev(X, "X", _F32)
    squeeze = X.dim() == 1
    M = 1 if squeeze else X.shape[0]
    if X.dim() not in (1, 2) or X.shape[-1] != K:
        raise ValueError(f"X must be [{K}] or [M, {K}]")
    if Y is None:
        Y = torch.empty((N,) if squeeze else (M, N), dtype=torch.float32, device=X.device)
    _size(_dev(Y, "Y", _F32), M * N, "Y")
    _check(lib.int4_matvec(_ptr(X), M, _ptr(q), _ptr(scales), _ptr(zeros), N, K, gs, _ptr(Y),
                           _stream(stream)))
    return Y


def int4_matvec_split4(x: torch.Tensor, q, scales, zeros, n0: int, n1: int, n2: int,
                       outs=None, stream=None):
    """One matvec over N columns routed to (out0[n0], out1[n1-n0], out2[n2-n1], out3[N-n2])."""
    N, K, gs = _weights(q, scales, zeros)
    _size(_dev(x, "x", _F32), K, "x")
    sizes = [n0, n1 - n0, n2 - n1, N - n2]
    if outs is None:
        outs = [torch.empty(max(sz, 0), dtype=torch.float32, device=x.device) for sz in sizes]
    ptrs = []
    for i, o in enumerate(outs):
        if o is None:
            ptrs.append(None)
        else:
            _dev(o, f"out{i}", _F32)
            if sizes[i] >= 0:  # an unordered split is the library's INT4_ERR_ARG
                _size(o, sizes[i], f"out{i}")
            ptrs.append(_ptr(o) if o.numel() else None)
    _check(lib.int4_matvec_split4(_ptr(x), _ptr(q), _ptr(scales), _ptr(zeros), N, K, gs,
                                  n0, n1, n2, *ptrs, _stream(stream)))
    return tuple(outs)


def int4_matvec_gated(x: torch.Tensor, q_gate, s_gate, z_gate, q_up, s_up, z_up, h=None,
                      stream=None) -> torch.Tensor:
    """h[n] = silu(x . w_gate[n]) * (x . w_up[n])."""
    N, K, gs = _weights(q_gate, s_gate, z_gate, "_gate")
    N2, K2, gs2 = _weights(q_up, s_up, z_up, "_up")
    if (N, K, gs) != (N2, K2, gs2):
        raise ValueError("gate and up weights must share N, K and group size")
    _size(_dev(x, "x", _F32), K, "x")
    h = torch.empty(N, dtype=torch.float32, device=x.device) if h is None else h
    _size(_dev(h, "h", _F32), N, "h")
    _check(lib.int4_matvec_gated(_ptr(x), _ptr(q_gate), _ptr(s_gate), _ptr(z_gate), _ptr(q_up),
                                 _ptr(s_up), _ptr(z_up), N, K, gs, _ptr(h), _stream(stream)))
    return h


def int4_matvec_norm(a_a: torch.Tensor, a_b: torch.Tensor, w_norm: torch.Tensor, eps: float,
                     q, scales, zeros, y=None, residual_out=None, norm_out=None,
                     want_residual: bool = True, want_norm: bool = True, stream=None):
    """y = (RMSNorm(a_a + a_b) * w_norm) . w  -> (y, residual_out or None, norm_out or None)."""
    N, K, gs = _weights(q, scales, zeros)
    for t, name in ((a_a, "a_a"), (a_b, "a_b"), (w_norm, "w_norm")):
        _size(_dev(t, name, _F32), K, name)
    dev = a_a.device
    y = torch.empty(N, dtype=torch.float32, device=dev) if y is None else y
    if residual_out is None and want_residual:
        residual_out = torch.empty(K, dtype=torch.float32, device=dev)
    if norm_out is None and want_norm:
        norm_out = torch.empty(K, dtype=torch.float32, device=dev)
    for t, name, n in ((y, "y", N), (residual_out, "residual_out", K), (norm_out, "norm_out", K)):
        if t is not None:
            _size(_dev(t, name, _F32), n, name)
    _check(lib.int4_matvec_norm(_ptr(a_a), _ptr(a_b), _ptr(w_norm), float(eps), _ptr(q),
                                _ptr(scales), _ptr(zeros), N, K, gs,
                                _ptr(y) if N else None, _ptr(residual_out), _ptr(norm_out),
                                _stream(stream)))
    return y, residual_out, norm_out


def _pair(q0, s0, z0, q1, s1, z1, t0, t1):
    N, K, gs = _weights(q0, s0, z0, t0)
    if _weights(q1, s1, z1, t1) != (N, K, gs):
        raise ValueError(f"the{t0.replace('_', ' ')} and{t1.replace('_', ' ')} weights must share N, K and group size")
    return N, K, gs


def _lanes(X: torch.Tensor, K: int, name: str):
    """Rows of an activation tensor [K] (one lane) or [M, K]; returns (M, output shape fn)."""
    _dev(X, name, _F32)
    if X.shape[-1] != K or X.dim() not in (1, 2):
        raise ValueError(f"{name} must be [{K}] or [M, {K}]")
    M = 1 if X.dim() == 1 else X.shape[0]
    return M, (lambda N: (N,) if X.dim() == 1 else (M, N))


def int4_matvec_dual(X: torch.Tensor, q0, s0, z0, q1, s1, z1, y0=None, y1=None, stream=None):
    """(y0, y1) = (X . w0^T, X . w1^T): two projections of one input ([K] or [M, K], M <= 8)."""
    N, K, gs = _pair(q0, s0, z0, q1, s1, z1, "0", "1")
    M, shape = _lanes(X, K, "X")
    y0 = torch.empty(shape(N), dtype=torch.float32, device=X.device) if y0 is None else y0
    y1 = torch.empty(shape(N), dtype=torch.float32, device=X.device) if y1 is None else y1
    _size(_dev(y0, "y0", _F32), M * N, "y0")
    _size(_dev(y1, "y1", _F32), M * N, "y1")
    _check(lib.int4_matvec_dual(_ptr(X), M, _ptr(q0), _ptr(s0), _ptr(z0), _ptr(q1), _ptr(s1),
                                _ptr(z1), N, K, gs, _ptr(y0), _ptr(y1), _stream(stream)))
    return y0, y1


def int4_matvec_sigmoid_gated(a: torch.Tensor, gate: torch.Tensor, q, scales, zeros, y=None,
                              stream=None) -> torch.Tensor:
    """y = (a * sigmoid(gate)) . w^T for a, gate [K] or [M, K] (M <= 8)."""
    N, K, gs = _weights(q, scales, zeros)
    M, shape = _lanes(a, K, "a")
    if _lanes(gate, K, "gate")[0] != M or gate.dim() != a.dim():
        raise ValueError("a and gate must have the same shape")
    y = torch.empty(shape(N), dtype=torch.float32, device=a.device) if y is None else y
    _size(_dev(y, "y", _F32), M * N, "y")
    _check(lib.int4_matvec_sigmoid_gated(_ptr(a), _ptr(gate), M, _ptr(q), _ptr(scales),
                                         _ptr(zeros), N, K, gs, _ptr(y), _stream(stream)))
    return y


def int4_matvec_swiglu_gated(gate: torch.Tensor, up: torch.Tensor, q, scales, zeros, y=None,
                             stream=None) -> torch.Tensor:
    """y = (silu(gate) * up) . w^T for gate, up [K] or [M, K] (M <= 8)."""
    N, K, gs = _weights(q, scales, zeros)
    M, shape = _lanes(gate, K, "gate")
    if _lanes(up, K, "up")[0] != M or up.dim() != gate.dim():
        raise ValueError("gate and up must have the same shape")
    y = torch.empty(shape(N), dtype=torch.float32, device=gate.device) if y is None else y
    _size(_dev(y, "y", _F32), M * N, "y")
    _check(lib.int4_matvec_swiglu_gated(_ptr(gate), _ptr(up), M, _ptr(q), _ptr(scales),
                                        _ptr(zeros), N, K, gs, _ptr(y), _stream(stream)))
    return y


def int4_matvec_norm_swiglu(a_a: torch.Tensor, a_b: torch.Tensor, w_norm: torch.Tensor,
                            eps: float, q_gate, s_gate, z_gate, q_up, s_up, z_up, h=None,
                            residual_out=None, want_residual: bool = True, stream=None):
    """h = silu(x . w_gate) * (x . w_up), x = RMSNorm(a_a + a_b) * w_norm -> (h, residual_out or None)."""
    N, K, gs = _pair(q_gate, s_gate, z_gate, q_up, s_up, z_up, "_gate", "_up")
    for t, name in ((a_a, "a_a"), (a_b, "a_b"), (w_norm, "w_norm")):
        _size(_dev(t, name, _F32), K, name)
    dev = a_a.device
    h = torch.empty(N, dtype=torch.float32, device=dev) if h is None else h
    if residual_out is None and want_residual:
        residual_out = torch.empty(K, dtype=torch.float32, device=dev)
    for t, name, n in ((h, "h", N), (residual_out, "residual_out", K)):
        if t is not None:
            _size(_dev(t, name, _F32), n, name)
    _check(lib.int4_matvec_norm_swiglu(_ptr(a_a), _ptr(a_b), _ptr(w_norm), float(eps),
                                       _ptr(q_gate), _ptr(s_gate), _ptr(z_gate), _ptr(q_up),
                                       _ptr(s_up), _ptr(z_up), N, K, gs, _ptr(h) if N else None,
                                       _ptr(residual_out), _stream(stream)))
    return h, residual_out


def int4_embedding_gather(ids: torch.Tensor, q, scales, zeros, out=None, stream=None) -> torch.Tensor:
    """ids int32 [T] -> out float32 [T, K]: rows ids[t] of the int4 table, dequantized."""
    N, K, gs = _weights(q, scales, zeros)
    _dev(ids, "ids", (torch.int32,))
    T = ids.numel()
    out = torch.empty((T, K), dtype=torch.float32, device=ids.device) if out is None else out
    _dev(out, "out", _F32)
    if out.numel() != T * K:
        raise ValueError(f"out must hold T*K = {T * K} floats")
    _check(lib.int4_embedding_gather(_ptr(ids), T, _ptr(q), _ptr(scales), _ptr(zeros), N, K, gs,
                                     _ptr(out), _stream(stream)))
    return out


def _pinned(t: torch.Tensor, name: str, dtypes) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cpu" or not t.is_pinned():
        raise ValueError(f"{name} must be a page-locked host tensor (pin_memory=True)")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def int4_embedding_gather_host(ids: torch.Tensor, q, scales, zeros, out=None, stream=None) -> torch.Tensor:
    """As int4_embedding_gather, with the table (q, scales, zeros) in page-locked
    host memory: only the T gathered rows cross the host link, and the GPU
    dequantizes them.  ids int32 [T] and out float32 [T, K] are device tensors."""
    _pinned(q, "q", _CODES)
    _pinned(scales, "scales", _F32)
    _pinned(zeros, "zeros", _F32)
    if q.dim() != 2 or scales.dim() != 2 or scales.shape != zeros.shape or scales.shape[0] != q.shape[0]:
        raise ValueError("q must be [N, K/8] and scales/zeros [N, K/gs]")
    N, K = q.shape[0], q.shape[1] * 8
    G = scales.shape[1]
    if G == 0 or K % G:
        raise ValueError(f"K={K} is not a multiple of the group count {G}")
    gs = K // G
    _dev(ids, "ids", (torch.int32,))
    T = ids.numel()
    out = torch.empty((T, K), dtype=torch.float32, device=ids.device) if out is None else out
    _dev(out, "out", _F32)
    if out.numel() != T * K:
        raise ValueError(f"out must hold T*K = {T * K} floats")
    _check(lib.int4_embedding_gather_host(_ptr(ids), T, _ptr(q), _ptr(scales), _ptr(zeros), N, K, gs,
                                          _ptr(out), _stream(stream)))
    return out


def int4_gemm_workspace_bytes(T: int, N: int, K: int, group_size: int) -> int:
    """Bytes of device workspace int4_gemm needs for these sizes."""
    return int(lib.int4_gemm_workspace_bytes(T, N, K, group_size))


def int4_gemm(X: torch.Tensor, q, scales, zeros, Y=None, workspace=None, stream=None) -> torch.Tensor:
    """X float32 [T, K] -> Y float32 [T, N] (prefill GEMM on the matrix cores).

    workspace: a uint8 device tensor of at least int4_gemm_workspace_bytes bytes
    (256-byte aligned); allocated here when not given.
    """
    N, K, gs = _weights(q, scales, zeros)
    _dev(X, "X", _F32)
    if X.dim() != 2 or X.shape[1] != K:
        raise ValueError(f"X must be [T, {K}]")
    T = X.shape[0]
    Y = torch.empty((T, N), dtype=torch.float32, device=X.device) if Y is None else Y
    _size(_dev(Y, "Y", _F32), T * N, "Y")
    need = int4_gemm_workspace_bytes(T, N, K, gs)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=X.device)
    _dev(workspace, "workspace", (torch.uint8,))
    _check(lib.int4_gemm(_ptr(X), T, _ptr(q), _ptr(scales), _ptr(zeros), N, K, gs, _ptr(Y),
                         _ptr(workspace), workspace.numel(), _stream(stream)))
    return Y


# Size of the scratch array int4_gemm_noalloc uses on each GPU (the header's
# INT4_GEMM_NOALLOC_SCRATCH_BYTES).
INT4_GEMM_NOALLOC_SCRATCH_BYTES = 64 << 20


def int4_gemm_noalloc(X: torch.Tensor, q, scales, zeros, Y=None, stream=None) -> torch.Tensor:
    """int4_gemm with the library's own scratch: the C call allocates nothing.

    Pass Y to allocate nothing at all (otherwise torch allocates it here).
    Problems whose workspace exceeds INT4_GEMM_NOALLOC_SCRATCH_BYTES raise
    Int4Error (INT4_ERR_SHAPE); calls that overlap in time on one GPU race.
    """
    N, K, gs = _weights(q, scales, zeros)
    _dev(X, "X", _F32)
    if X.dim() != 2 or X.shape[1] != K:
        raise ValueError(f"X must be [T, {K}]")
    T = X.shape[0]
    Y = torch.empty((T, N), dtype=torch.float32, device=X.device) if Y is None else Y
    _size(_dev(Y, "Y", _F32), T * N, "Y")
    _check(lib.int4_gemm_noalloc(_ptr(X), T, _ptr(q), _ptr(scales), _ptr(zeros), N, K, gs, _ptr(Y),
                                 _stream(stream)))
    return Y


def int4_probe_stream_read(buf: torch.Tensor, sink: torch.Tensor, blocks: int, waves: int = 8,
                           unroll: int = 4, stream=None) -> None:
    """Measurement only: one streaming read of all of `buf` (any dtype, 16-byte
    multiple), XOR checksum of each block's slice into the int32 `sink`."""
    if not buf.is_cuda or not buf.is_contiguous() or not sink.is_cuda or sink.dtype not in _CODES:
        raise ValueError("buf must be a contiguous device tensor and sink a device int32 tensor")
    _size(sink, blocks, "sink")
    _check(lib.int4_probe_stream_read(_ptr(buf), buf.numel() * buf.element_size(), blocks, waves, unroll,
                                      _ptr(sink), _stream(stream)))


def int4_matvec_gated_lanes(X: torch.Tensor, q_gate, s_gate, z_gate, q_up, s_up, z_up, H=None,
                            stream=None) -> torch.Tensor:
    """H = silu(X . w_gate^T) * (X . w_up^T) for X [M, K] (M <= 8), one launch."""
    N, K, gs = _pair(q_gate, s_gate, z_gate, q_up, s_up, z_up, "_gate", "_up")
    M, shape = _lanes(X, K, "X")
    H = torch.empty(shape(N), dtype=torch.float32, device=X.device) if H is None else H
    _size(_dev(H, "H", _F32), M * N, "H")
    _check(lib.int4_matvec_gated_lanes(_ptr(X), M, _ptr(q_gate), _ptr(s_gate), _ptr(z_gate),
                                       _ptr(q_up), _ptr(s_up), _ptr(z_up), N, K, gs, _ptr(H),
                                       _stream(stream)))
    return H


def int4_mlp_workspace_bytes() -> int:
    """Bytes of zeroed device workspace int4_mlp needs."""
    return int(lib.int4_mlp_workspace_bytes())


def int4_mlp_timed_out(workspace: torch.Tensor, stream=None) -> bool:
    """Whether a fused int4_mlp wait on `workspace` has timed out (its word 1
    is set).  Waits for the stream's earlier work."""
    _dev(workspace, "workspace", (torch.int32, torch.uint32, torch.uint8))
    if workspace.numel() * workspace.element_size() < 8:
        raise ValueError("workspace must hold at least two 32-bit words")
    out = ctypes.c_int32(0)
    _check(lib.int4_mlp_timed_out(_ptr(workspace), ctypes.byref(out), _stream(stream)))
    return bool(out.value)


def int4_mlp(x: torch.Tensor, q_gate, s_gate, z_gate, q_up, s_up, z_up, q_down, s_down, z_down,
             h=None, y=None, workspace=None, stream=None):
    """(h, y): h = silu(x . w_gate^T) * (x . w_up^T) [F], y = h . w_down^T [D], one launch.

    workspace: an int32 device tensor of at least int4_mlp_workspace_bytes()
    bytes, zeroed before its first use and then kept as the calls leave it
    (calls sharing it must not overlap).  A fresh zeroed one is made when
    not given.  If a fused call's wait on its blocks times out
    (int4_mlp_timed_out), its h and y are undefined and every later call
    with that workspace writes NaN, until the workspace is zeroed again.
    """
    F, D, gs = _pair(q_gate, s_gate, z_gate, q_up, s_up, z_up, "_gate", "_up")
    D2, F2, gs2 = _weights(q_down, s_down, z_down, "_down")
    if (D2, F2, gs2) != (D, F, gs):
        raise ValueError(f"down weights must be [{D}, {F}/8] with group size {gs}")
    _dev(x, "x", _F32)
    if x.numel() != D:
        raise ValueError(f"x must hold D = {D} floats")
    h = torch.empty(F, dtype=torch.float32, device=x.device) if h is None else h
    y = torch.empty(D, dtype=torch.float32, device=x.device) if y is None else y
    _size(_dev(h, "h", _F32), F, "h")
    _size(_dev(y, "y", _F32), D, "y")
    if workspace is None:
        workspace = torch.zeros(int4_mlp_workspace_bytes() // 4, dtype=torch.int32, device=x.device)
    _dev(workspace, "workspace", (torch.int32, torch.uint32, torch.uint8))
    _check(lib.int4_mlp(_ptr(x), _ptr(q_gate), _ptr(s_gate), _ptr(z_gate), _ptr(q_up), _ptr(s_up),
                        _ptr(z_up), _ptr(q_down), _ptr(s_down), _ptr(z_down), D, F, gs, _ptr(h),
                        _ptr(y), _ptr(workspace), workspace.numel() * workspace.element_size(),
                        _stream(stream)))
    return h, y
