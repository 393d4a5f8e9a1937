"""Seeded synthetic inputs shared by the tests, the smoke entry and the bench.

This module holds none of the method's arithmetic: it only draws numbers.
Every value is a pure function of (seed, index), so the result does not depend
on chunking or thread count.

Generator (SplitMix64, Steele, Lea & Flood 2014, used counter-style):
    s_i   = seed + (i + 1) * 0x9E3779B97F4A7C15            (mod 2^64)
    z     = (s_i ^ (s_i >> 30)) * 0xBF58476D1CE4E5B9
    z     = (z ^ (z >> 27)) * 0x94D049BB133111EB
    out_i = z ^ (z >> 31)
Uniform u_i = (out_i >> 11) * 2^-53 in [0, 1).
Normal n_i (Box-Muller, fp64, cosine branch) from the two uniforms 2i, 2i+1:
    n_i = sqrt(-2 ln(1 - u_2i)) * cos(2 pi u_2i+1)
then scaled and rounded once to binary32.

Workload shapes and seeds (decode-shaped activations and weights of the model
family the pages serve; no dataset is involved):
    c1  single matvec   x[1024]           W[1024, 1024]   gs 128   seeds 0x101/0x102
    c2  split4          x[4096]           W[6656, 4096]   gs 128   seeds 0x201/0x202
    c3  gated + down    x[4096]           Wg,Wu[14336,4096], Wd[4096,14336] gs 128
                                                             seeds 0x301..0x304
    c4  norm LM head    a_a,a_b[4096] N(0,1), w_norm U(0.5,1.5), eps 1e-6,
                        W[151936, 4096]   gs 128   seeds 0x401..0x404
    c5  decode lanes    X[M, 5120] (row m = counter offset m*K), M in {1,2,4,8},
                        W[25600, 5120]    gs 64, 1% of groups with one x20 outlier
                                                   seeds 0x501/0x502/0x503
Next-row workloads (fused decode variants around the hot path, same recipe):
    n1  dual q + gate   x[4096]           W0,W1[4096, 4096] gs 128 seeds 0x601..0x603
    n2  sigmoid-gated   a, gate[4096]     W[4096, 4096]     gs 128 seeds 0x701..0x703
        o_proj
    n3  SwiGLU-gated    gate, up[8192]    W[4096, 8192]     gs 128 seeds 0x801..0x803
        out_proj
    n4  norm + SwiGLU   a_a,a_b[4096] N(0,1), w_norm U(0.5,1.5), eps 1e-6,
        MLP front       Wg,Wu[14336, 4096] gs 128         seeds 0x901..0x905
    n5  embedding       ids[T] uniform in [0, 151936) (T = 1 and 4096), table
        gather          [151936, 4096] gs 128               seeds 0xA01/0xA02
    n6  prefill GEMM    X[T, 4096] N(0,1) for T = 512 and 4096, W[4096, 4096] gs 128
                                                            seeds 0xB01/0xB02
Weights are N(0, 0.02^2) (0.02 is the standard deviation), activations N(0, 1).
"""
from __future__ import annotations

import concurrent.futures as _cf
import os

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def splitmix64(seed: int, start: int, count: int) -> np.ndarray:
    """Raw 64-bit outputs out_i for i in [start, start + count)."""
    i = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        s = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + i * _GOLDEN
        z = (s ^ (s >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def uniform(seed: int, start: int, count: int) -> np.ndarray:
    """fp64 uniforms in [0, 1) for counters [start, start + count)."""
    return (splitmix64(seed, start, count) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def _normal_chunk(seed, start, count, sigma, out, off):
    u = uniform(seed, 2 * start, 2 * count).reshape(count, 2)
    r = np.sqrt(-2.0 * np.log1p(-u[:, 0]))
    out[off:off + count] = (sigma * r * np.cos(2.0 * np.pi * u[:, 1])).astype(np.float32)


def normal_f32(seed: int, count: int, sigma: float = 1.0, start: int = 0) -> np.ndarray:
    """binary32 N(0, sigma^2) draws n_i for i in [start, start + count)."""
    out = np.empty(count, np.float32)
    jobs = [(c, min(_CHUNK, count - c)) for c in range(0, count, _CHUNK)]
    if len(jobs) <= 1:
        for c, n in jobs:
            _normal_chunk(seed, start + c, n, sigma, out, c)
        return out
    with _cf.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(lambda j: _normal_chunk(seed, start + j[0], j[1], sigma, out, j[0]), jobs))
    return out


def uniform_f32(seed: int, count: int, lo: float, hi: float, start: int = 0) -> np.ndarray:
    """binary32 U(lo, hi) draws: lo + (hi - lo) * u_i, rounded once."""
    return (lo + (hi - lo) * uniform(seed, start, count)).astype(np.float32)


def weights(seed: int, N: int, K: int, sigma: float = 0.02) -> np.ndarray:
    """W f32 [N, K] row-major (row n is output column n, contiguous along K)."""
    return normal_f32(seed, N * K, sigma).reshape(N, K)


def lanes(seed: int, M: int, K: int) -> np.ndarray:
    """X f32 [M, K]; row m draws counters [m*K, (m+1)*K) so rows are prefix-stable in M."""
    return normal_f32(seed, M * K, 1.0).reshape(M, K)


def add_group_outliers(W: np.ndarray, group_size: int, seed: int, frac: float = 0.01,
                       factor: float = 20.0) -> np.ndarray:
    """Multiply one element in floor(frac * #groups) groups by `factor`, in place.

    Groups are chosen by a seeded partial Fisher-Yates shuffle over all
    (column, group) pairs; the position inside each chosen group is uniform.
    Draw 2t picks the t-th group, draw 2t+1 its position.
    """
    N, K = W.shape
    G = K // group_size
    total = N * G
    count = int(np.floor(frac * total))
    u = uniform(seed, 0, 2 * count)
    perm = np.arange(total, dtype=np.int64)
    for t in range(count):
        j = t + int(u[2 * t] * (total - t))
        perm[t], perm[j] = perm[j], perm[t]
    chosen = perm[:count]
    pos = np.minimum((u[1::2] * group_size).astype(np.int64), group_size - 1)
    n = chosen // G
    g = chosen % G
    flat = W.reshape(-1)
    idx = n * K + g * group_size + pos
    flat[idx] = (flat[idx].astype(np.float64) * factor).astype(np.float32)
    return W


# ----------------------------------------------------------------- workloads

CONFIGS = {
    "c1": dict(name="single int4 matvec N=1024 K=1024 gs=128", N=1024, K=1024, gs=128),
    "c2": dict(name="split4 projection N=6656 K=4096 gs=128 (4096/1024/1024/512)",
               N=6656, K=4096, gs=128, n0=4096, n1=5120, n2=6144),
    "c3": dict(name="SiLU-gated MLP gate/up N=14336 K=4096 + down N=4096 K=14336 gs=128",
               N=14336, K=4096, gs=128, Nd=4096, Kd=14336),
    "c4": dict(name="norm-prefixed LM head N=151936 K=4096 gs=128", N=151936, K=4096, gs=128,
               eps=1e-6),
    "c5": dict(name="decode lanes M in {1,2,4,8} N=25600 K=5120 gs=64", N=25600, K=5120, gs=64,
               Ms=(1, 2, 4, 8)),
}


NEXT = {
    "n1": dict(name="dual q + gate projection 2 x N=4096 K=4096 gs=128", N=4096, K=4096, gs=128),
    "n2": dict(name="sigmoid-gated o_proj N=4096 K=4096 gs=128", N=4096, K=4096, gs=128),
    "n3": dict(name="SwiGLU-gated out_proj N=4096 K=8192 gs=128", N=4096, K=8192, gs=128),
    "n4": dict(name="norm + SwiGLU MLP front 2 x N=14336 K=4096 gs=128", N=14336, K=4096,
               gs=128, eps=1e-6),
    "n5": dict(name="int4 embedding gather from a [151936, 4096] gs=128 table, T = 1 and 4096",
               N=151936, K=4096, gs=128, Ts=(1, 4096)),
    "n6": dict(name="prefill GEMM T=512 (and 4096) N=4096 K=4096 gs=128", T=512, Ts=(512, 4096),
               N=4096, K=4096, gs=128),
    "n7": dict(name="per-layer-embedding gather from a page-locked host table [262144, 8960] gs=64 "
                    "(random codes), T = 1 and 64",
               N=262144, K=8960, gs=64, Ts=(1, 64)),
}


# One GPU's share of each call of the decode step under an 8-way split:
# split4, gate/up, the LM head and the lanes by output columns (each range
# of split4 in eighths), the down projection by K (its partial y would be
# summed across GPUs).  The activations are the full replicated vectors.
SHARD8 = {
    "split4": dict(N=832, K=4096, gs=128, n0=512, n1=640, n2=768),
    "gated": dict(N=1792, K=4096, gs=128),
    "down": dict(N=4096, K=1792, gs=128),
    "lmhead": dict(N=18992, K=4096, gs=128, eps=1e-6),
    "lanes": dict(N=3200, K=5120, gs=64, Ms=(1, 2, 4, 8)),
}


def shard8_inputs():
    """Seeded weights of every shard-shaped call (activations: the configs' own vectors)."""
    s = SHARD8
    return dict(
        W2=weights(0xC01, s["split4"]["N"], s["split4"]["K"]),
        Wg=weights(0xC02, s["gated"]["N"], s["gated"]["K"]),
        Wu=weights(0xC03, s["gated"]["N"], s["gated"]["K"]),
        Wd=weights(0xC04, s["down"]["N"], s["down"]["K"]),
        W4=weights(0xC05, s["lmhead"]["N"], s["lmhead"]["K"]),
        W5=weights(0xC06, s["lanes"]["N"], s["lanes"]["K"]),
    )


def n1_inputs():
    c = NEXT["n1"]
    return dict(x=normal_f32(0x601, c["K"]), W0=weights(0x602, c["N"], c["K"]),
                W1=weights(0x603, c["N"], c["K"]))


def n2_inputs():
    c = NEXT["n2"]
    return dict(a=normal_f32(0x701, c["K"]), gate=normal_f32(0x702, c["K"]),
                W=weights(0x703, c["N"], c["K"]))


def n3_inputs():
    c = NEXT["n3"]
    return dict(gate=normal_f32(0x801, c["K"]), up=normal_f32(0x802, c["K"]),
                W=weights(0x803, c["N"], c["K"]))


def n4_inputs():
    c = NEXT["n4"]
    K = c["K"]
    return dict(a_a=normal_f32(0x901, K), a_b=normal_f32(0x902, K),
                w_norm=uniform_f32(0x903, K, 0.5, 1.5), Wg=weights(0x904, c["N"], K),
                Wu=weights(0x905, c["N"], K), eps=c["eps"])


def token_ids(seed: int, T: int, N: int) -> np.ndarray:
    """int32 ids floor(u_i * N) for i in [0, T)."""
    return np.minimum((uniform(seed, 0, T) * N).astype(np.int64), N - 1).astype(np.int32)


def n5_inputs(N: int | None = None):
    c = NEXT["n5"]
    return dict(ids=token_ids(0xA01, max(c["Ts"]), c["N"]), W=weights(0xA02, N or c["N"], c["K"]))


def ple_table(seed: int, N: int, K: int, group_size: int, pin: bool = True):
    """A random int4 table (q int32 [N, K/8] of uniform 32-bit words, scales
    U(1e-3, 1.1e-2) and integer zero points U{0..15} as fp32 [N, K/gs]) drawn
    from torch's seeded CPU generator straight into page-locked host tensors
    (pin=True): the per-layer-embedding table's shape without its values,
    which a gather does not depend on.  Returns (q, scales, zeros)."""
    import torch
    g = torch.Generator().manual_seed(seed)
    G = K // group_size
    q = torch.empty((N, K // 8), dtype=torch.int32, pin_memory=pin)
    s = torch.empty((N, G), dtype=torch.float32, pin_memory=pin)
    z = torch.empty((N, G), dtype=torch.float32, pin_memory=pin)
    q.copy_(torch.randint(-2**31, 2**31 - 1, (N, K // 8), dtype=torch.int32, generator=g))
    s.copy_(torch.rand((N, G), generator=g) * 1e-2 + 1e-3)
    z.copy_(torch.randint(0, 16, (N, G), generator=g).to(torch.float32))
    return q, s, z


def n7_inputs():
    c = NEXT["n7"]
    return dict(ids=token_ids(0xC01, max(c["Ts"]), c["N"]), table=ple_table(0xC02, c["N"], c["K"], c["gs"]))


def n6_inputs(T: int | None = None):
    c = NEXT["n6"]
    return dict(X=lanes(0xB01, T or c["T"], c["K"]), W=weights(0xB02, c["N"], c["K"]))


def c1_inputs():
    c = CONFIGS["c1"]
    return dict(x=normal_f32(0x101, c["K"]), W=weights(0x102, c["N"], c["K"]))


def c2_inputs():
    c = CONFIGS["c2"]
    return dict(x=normal_f32(0x201, c["K"]), W=weights(0x202, c["N"], c["K"]))


def c3_inputs():
    c = CONFIGS["c3"]
    return dict(x=normal_f32(0x301, c["K"]), Wg=weights(0x302, c["N"], c["K"]),
                Wu=weights(0x303, c["N"], c["K"]), Wd=weights(0x304, c["Nd"], c["Kd"]))


def c4_inputs(N: int | None = None):
    c = CONFIGS["c4"]
    K = c["K"]
    return dict(a_a=normal_f32(0x401, K), a_b=normal_f32(0x402, K),
                w_norm=uniform_f32(0x403, K, 0.5, 1.5),
                W=weights(0x404, N or c["N"], K), eps=c["eps"])


def c5_inputs(M: int = 8):
    c = CONFIGS["c5"]
    W = weights(0x502, c["N"], c["K"])
    add_group_outliers(W, c["gs"], 0x503)
    return dict(X=lanes(0x501, M, c["K"]), W=W)
