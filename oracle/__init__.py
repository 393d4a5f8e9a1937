"""CPU oracle for the int4 group-quantized matvec family (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path never does: the HIP
library and its binding share no code with it, and neither imports the other.

The arithmetic lives in ``oracle.c`` (plain C, fp64 dot products, the binary32
quantizer written out step by step).  This module only builds that file with
gcc and marshals numpy arrays to it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

GCC_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
             "-fno-fast-math", "-fopenmp", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (no GPU code involved)."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None

_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_u32p = np.ctypeslib.ndpointer(dtype=np.uint32, flags="C_CONTIGUOUS")
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_set_threads.argtypes = [_i32]
    lib.oracle_set_threads.restype = None
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = _i32
    lib.oracle_quantize_pack.argtypes = [_f32p, _i64, _i64, _i32, _u32p, _f32p, _f32p]
    lib.oracle_dequant.argtypes = [_u32p, _f32p, _f32p, _i64, _i64, _i32, _f32p]
    lib.oracle_matvec.argtypes = [_f32p, _i32, _u32p, _f32p, _f32p, _i64, _i64, _i32, _f64p, _f64p]
    lib.oracle_matvec_f32.argtypes = [_f32p, _i32, _u32p, _f32p, _f32p, _i64, _i64, _i32, _f32p]
    lib.oracle_split4.argtypes = [_f32p, _u32p, _f32p, _f32p, _i64, _i64, _i32, _i64, _i64, _i64,
                                  _f64p, _f64p, _f64p, _f64p, _f64p, _f64p, _f64p, _f64p]
    lib.oracle_gated.argtypes = [_f32p, _u32p, _f32p, _f32p, _u32p, _f32p, _f32p, _i64, _i64, _i32,
                                 _f64p, _f64p, _f64p, _f64p, _f64p]
    lib.oracle_norm.argtypes = [_f32p, _f32p, _f32p, ctypes.c_float, _u32p, _f32p, _f32p,
                                _i64, _i64, _i32, _f64p, _f64p, _f32p, _f64p]
    lib.oracle_dual.argtypes = [_f32p, _u32p, _f32p, _f32p, _u32p, _f32p, _f32p, _i64, _i64, _i32,
                                _f64p, _f64p, _f64p, _f64p]
    lib.oracle_input_gated.argtypes = [_i32, _f32p, _f32p, _u32p, _f32p, _f32p, _i64, _i64, _i32,
                                       _f64p, _f64p, _f64p]
    lib.oracle_norm_swiglu.argtypes = [_f32p, _f32p, _f32p, ctypes.c_float,
                                       _u32p, _f32p, _f32p, _u32p, _f32p, _f32p, _i64, _i64, _i32,
                                       _f64p, _f64p, _f64p, _f64p, _f64p, _f32p]
    lib.oracle_embedding.argtypes = [np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS"),
                                     _i64, _u32p, _f32p, _f32p, _i64, _i64, _i32, _f32p]
    lib.oracle_embedding.restype = None
    for fn in (lib.oracle_quantize_pack, lib.oracle_dequant, lib.oracle_matvec,
               lib.oracle_matvec_f32, lib.oracle_split4, lib.oracle_gated, lib.oracle_norm,
               lib.oracle_dual, lib.oracle_input_gated, lib.oracle_norm_swiglu):
        fn.restype = None
    _lib = lib
    return lib


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check_shape(K: int, gs: int):
    if gs <= 0 or gs % 8 or K % gs:
        raise ValueError(f"oracle needs group_size % 8 == 0 and K % group_size == 0 (K={K}, gs={gs})")


def quantize_pack(W: np.ndarray, group_size: int):
    """W f32 [N, K] -> (q u32 [N, K/8], scales f32 [N, K/gs], zeros f32 [N, K/gs])."""
    W = _c(W, np.float32)
    N, K = W.shape
    _check_shape(K, group_size)
    q = np.empty((N, K // 8), np.uint32)
    s = np.empty((N, K // group_size), np.float32)
    z = np.empty((N, K // group_size), np.float32)
    _load().oracle_quantize_pack(W, N, K, group_size, q, s, z)
    return q, s, z


def dequant(q, scales, zeros, K: int, group_size: int) -> np.ndarray:
    q = _c(q, np.uint32)
    N = q.shape[0]
    _check_shape(K, group_size)
    dq = np.empty((N, K), np.float32)
    _load().oracle_dequant(q, _c(scales, np.float32), _c(zeros, np.float32), N, K, group_size, dq)
    return dq


def matvec(X, q, scales, zeros, K: int, group_size: int):
    """X f32 [M, K] (or [K]) -> (Y f64 [M, N], B f64 [M, N]); shapes follow X's rank."""
    X = _c(X, np.float32)
    squeeze = X.ndim == 1
    X2 = X.reshape(1, -1) if squeeze else X
    M = X2.shape[0]
    q = _c(q, np.uint32)
    N = q.shape[0]
    _check_shape(K, group_size)
    Y = np.empty((M, N), np.float64)
    B = np.empty((M, N), np.float64)
    _load().oracle_matvec(X2, M, q, _c(scales, np.float32), _c(zeros, np.float32),
                          N, K, group_size, Y, B)
    return (Y[0], B[0]) if squeeze else (Y, B)


def matvec_f32(X, q, scales, zeros, K: int, group_size: int) -> np.ndarray:
    X = _c(X, np.float32)
    squeeze = X.ndim == 1
    X2 = X.reshape(1, -1) if squeeze else X
    M = X2.shape[0]
    q = _c(q, np.uint32)
    N = q.shape[0]
    Y = np.empty((M, N), np.float32)
    _load().oracle_matvec_f32(X2, M, q, _c(scales, np.float32), _c(zeros, np.float32),
                              N, K, group_size, Y)
    return Y[0] if squeeze else Y


def split4(x, q, scales, zeros, K: int, group_size: int, n0: int, n1: int, n2: int):
    """Returns ([out0..out3] f64, [b0..b3] f64) routed by the split points."""
    x = _c(x, np.float32)
    q = _c(q, np.uint32)
    N = q.shape[0]
    if not (0 <= n0 <= n1 <= n2 <= N):
        raise ValueError("split points must satisfy 0 <= n0 <= n1 <= n2 <= N")
    sizes = [n0, n1 - n0, n2 - n1, N - n2]
    outs = [np.empty(max(sz, 1), np.float64) for sz in sizes]
    bs = [np.empty(max(sz, 1), np.float64) for sz in sizes]
    _load().oracle_split4(x, q, _c(scales, np.float32), _c(zeros, np.float32), N, K, group_size,
                          n0, n1, n2, *outs, *bs)
    return [o[:sz] for o, sz in zip(outs, sizes)], [b[:sz] for b, sz in zip(bs, sizes)]


def gated(x, q_gate, s_gate, z_gate, q_up, s_up, z_up, K: int, group_size: int):
    """Returns dict with h, g, u, bg, bu (all f64 [N])."""
    x = _c(x, np.float32)
    q_gate = _c(q_gate, np.uint32)
    q_up = _c(q_up, np.uint32)
    N = q_gate.shape[0]
    out = {k: np.empty(N, np.float64) for k in ("h", "g", "u", "bg", "bu")}
    _load().oracle_gated(x, q_gate, _c(s_gate, np.float32), _c(z_gate, np.float32),
                         q_up, _c(s_up, np.float32), _c(z_up, np.float32), N, K, group_size,
                         out["h"], out["g"], out["u"], out["bg"], out["bu"])
    return out


def norm(a_a, a_b, w_norm, eps: float, q, scales, zeros, K: int, group_size: int):
    """Returns dict with y, B (f64 [N]), residual (f32 [K]) and normed (f64 [K])."""
    q = _c(q, np.uint32)
    N = q.shape[0]
    y = np.empty(N, np.float64)
    B = np.empty(N, np.float64)
    residual = np.empty(K, np.float32)
    normed = np.empty(K, np.float64)
    _load().oracle_norm(_c(a_a, np.float32), _c(a_b, np.float32), _c(w_norm, np.float32),
                        ctypes.c_float(eps), q, _c(scales, np.float32), _c(zeros, np.float32),
                        N, K, group_size, y, B, residual, normed)
    return {"y": y, "B": B, "residual": residual, "normed": normed}


def dual(x, q0, s0, z0, q1, s1, z1, K: int, group_size: int):
    """Returns dict with y0, b0, y1, b1 (all f64 [N])."""
    x = _c(x, np.float32)
    q0 = _c(q0, np.uint32)
    q1 = _c(q1, np.uint32)
    N = q0.shape[0]
    _check_shape(K, group_size)
    out = {k: np.empty(N, np.float64) for k in ("y0", "b0", "y1", "b1")}
    _load().oracle_dual(x, q0, _c(s0, np.float32), _c(z0, np.float32),
                        q1, _c(s1, np.float32), _c(z1, np.float32), N, K, group_size,
                        out["y0"], out["b0"], out["y1"], out["b1"])
    return out


def _input_gated(kind: int, a, b, q, scales, zeros, K: int, group_size: int):
    q = _c(q, np.uint32)
    N = q.shape[0]
    _check_shape(K, group_size)
    y = np.empty(N, np.float64)
    B = np.empty(N, np.float64)
    xg = np.empty(K, np.float64)
    _load().oracle_input_gated(kind, _c(a, np.float32), _c(b, np.float32), q,
                               _c(scales, np.float32), _c(zeros, np.float32),
                               N, K, group_size, y, B, xg)
    return {"y": y, "B": B, "xg": xg}


def sigmoid_gated(a, gate, q, scales, zeros, K: int, group_size: int):
    """y = W . (a * sigmoid(gate)); returns dict with y, B (f64 [N]) and xg (f64 [K])."""
    return _input_gated(0, a, gate, q, scales, zeros, K, group_size)


def swiglu_gated(gate, up, q, scales, zeros, K: int, group_size: int):
    """y = W . (silu(gate) * up); returns dict with y, B (f64 [N]) and xg (f64 [K])."""
    return _input_gated(1, gate, up, q, scales, zeros, K, group_size)


def norm_swiglu(a_a, a_b, w_norm, eps: float, q_gate, s_gate, z_gate, q_up, s_up, z_up,
                K: int, group_size: int):
    """Returns dict with h, g, u, bg, bu (f64 [N]) and residual (f32 [K])."""
    q_gate = _c(q_gate, np.uint32)
    q_up = _c(q_up, np.uint32)
    N = q_gate.shape[0]
    _check_shape(K, group_size)
    out = {k: np.empty(N, np.float64) for k in ("h", "g", "u", "bg", "bu")}
    out["residual"] = np.empty(K, np.float32)
    _load().oracle_norm_swiglu(_c(a_a, np.float32), _c(a_b, np.float32), _c(w_norm, np.float32),
                               ctypes.c_float(eps), q_gate, _c(s_gate, np.float32),
                               _c(z_gate, np.float32), q_up, _c(s_up, np.float32),
                               _c(z_up, np.float32), N, K, group_size,
                               out["h"], out["g"], out["u"], out["bg"], out["bu"], out["residual"])
    return out


def embedding(ids, q, scales, zeros, K: int, group_size: int) -> np.ndarray:
    """ids int32 [T] -> out f32 [T, K]: the dequantized table rows (zeros for ids outside [0, N))."""
    ids = _c(ids, np.int32)
    q = _c(q, np.uint32)
    N = q.shape[0]
    _check_shape(K, group_size)
    out = np.empty((ids.shape[0], K), np.float32)
    _load().oracle_embedding(ids, ids.shape[0], q, _c(scales, np.float32), _c(zeros, np.float32),
                             N, K, group_size, out)
    return out


def set_threads(n: int) -> None:
    """Threads the oracle's column loops use (results do not depend on it)."""
    _load().oracle_set_threads(int(n))


def max_threads() -> int:
    """Threads the oracle's column loops use now."""
    return int(_load().oracle_max_threads())


def tolerance(B):
    """Per-output bound on |y_gpu - y_ref| for a dot output: 1e-4 * B + 1e-6."""
    return 1e-4 * np.asarray(B, np.float64) + 1e-6
