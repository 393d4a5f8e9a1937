"""Test helpers: tolerances, independent code packing, adversarial groups.

Nothing here computes the method: tolerances follow the stated error bound
(|err| <= 1e-4 * sum|x_k w_k| + 1e-6 per dot output) and its first-order
propagation through silu(g) * u.
"""
import numpy as np

import oracle


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """codes int [N, K] in 0..15 -> u32 [N, K/8], input k at bits 4*(k%8) of word k/8."""
    N, K = codes.shape
    c = codes.astype(np.uint64).reshape(N, K // 8, 8)
    words = np.zeros((N, K // 8), np.uint64)
    for t in range(8):
        words |= c[:, :, t] << np.uint64(4 * t)
    return words.astype(np.uint32)


def integer_problem(rng, N, K, gs, M=1):
    """Random codes, integer zeros, unit scales and integer X in [-8, 8]: every
    partial sum is an integer below 2^24, so every summation order is exact."""
    codes = rng.integers(0, 16, (N, K))
    zeros = rng.integers(0, 16, (N, K // gs)).astype(np.float32)
    scales = np.ones((N, K // gs), np.float32)
    X = rng.integers(-8, 9, (M, K)).astype(np.float32)
    exact = X.astype(np.int64) @ (codes - np.repeat(zeros.astype(np.int64), gs, axis=1)).T
    return pack_codes(codes), scales, zeros, X, exact


def assert_dot_close(got, ref, B, what=""):
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    tol = oracle.tolerance(B)
    bad = err > tol
    if np.any(bad) or not np.all(np.isfinite(got)):
        i = np.flatnonzero(bad.ravel() | ~np.isfinite(got.ravel()))[:5]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outputs outside 1e-4*B+1e-6; "
            f"first idx {i.tolist()} got {got.ravel()[i]} ref {np.asarray(ref).ravel()[i]} "
            f"max err/tol {float(np.max(err / tol)):.3g}")
    return float(np.max(err / tol)) if err.size else 0.0


def gated_tolerance(ref):
    """First-order bound for h = silu(g) * u from the dot bounds of g and u;
    |silu'| <= 1.0998 is bounded by 1.1."""
    silu_g = ref["g"] / (1.0 + np.exp(-ref["g"]))
    return (1.1 * np.abs(ref["u"]) * oracle.tolerance(ref["bg"])
            + np.abs(silu_g) * oracle.tolerance(ref["bu"]) + 1e-6 * np.abs(ref["h"]) + 1e-6)


def adversarial_groups(rng, n_groups, gs):
    """Groups that stress the quantizer: ties, subnormal ranges, huge values,
    single outliers, all-positive / all-negative, tiny ranges, constants."""
    groups = []
    kinds = ["normal", "ties", "subnormal", "large", "outlier", "positive", "negative",
             "tiny_range", "constant", "zero"]
    for i in range(n_groups):
        kind = kinds[i % len(kinds)]
        if kind == "normal":
            g = rng.normal(0, 0.02, gs)
        elif kind == "ties":
            g = rng.integers(-16, 16, gs) * 0.25
            g[0], g[1] = -2.0, 5.5
        elif kind == "subnormal":
            g = rng.normal(0, 1, gs) * 1e-39
        elif kind == "large":
            g = rng.normal(0, 1, gs) * 1e30
        elif kind == "outlier":
            g = rng.normal(0, 0.02, gs)
            g[rng.integers(gs)] *= 20
        elif kind == "positive":
            g = np.abs(rng.normal(0.5, 0.1, gs)) + 0.1
        elif kind == "negative":
            g = -np.abs(rng.normal(0.5, 0.1, gs)) - 0.1
        elif kind == "tiny_range":
            g = 1.0 + rng.integers(0, 3, gs) * 1e-7
        elif kind == "constant":
            g = np.full(gs, rng.normal(0, 1))
        else:
            g = np.zeros(gs)
            if i % 20 == 9:
                g[::2] = -0.0
        groups.append(np.asarray(g, np.float32))
    return np.stack(groups)
