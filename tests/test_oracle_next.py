"""Pins of the oracle's dual, input-gated and norm-SwiGLU functions (CPU only).

Each function is checked against results fixed outside the oracle:
- exact int64 matrix products on integer problems;
- gate values where the sigmoid is exactly 1/2, 1 or 0 in fp64;
- scipy's logistic function (scipy.special.expit), a routine the oracle does not use,
  and the textbook identity sigma(t) = (1 + tanh(t / 2)) / 2 through numpy's tanh;
- the symmetry sigma(t) + sigma(-t) = 1;
- a power-of-two RMSNorm whose normalized vector is exactly +-1.
A swapped operand, a wrong sign in an exponent or a dropped factor fails at least one of them.
"""
import numpy as np
import pytest

from scipy.special import expit

import oracle
import synth
from test_oracle_matvec import integer_problem


def unpack(q, K):
    """u32 [N, K/8] -> int codes [N, K], input k at bits 4*(k%8) of word k/8."""
    q = np.asarray(q, np.uint32)
    shifts = (4 * np.arange(8, dtype=np.uint32))[None, None, :]
    return ((q[:, :, None] >> shifts) & 15).reshape(q.shape[0], K).astype(np.int64)


def dq64(q, s, z, K, gs):
    """fp64 copy of the binary32 dequantized matrix (code - zero) * scale."""
    codes = unpack(q, K).astype(np.float32)
    zz = np.repeat(np.asarray(z, np.float32), gs, axis=1)
    ss = np.repeat(np.asarray(s, np.float32), gs, axis=1)
    return ((codes - zz) * ss).astype(np.float64)


def sigma_tanh(t):
    """(1 + tanh(t/2)) / 2: accurate to ~1e-16 absolute (not relative for t << 0)."""
    t = np.asarray(t, np.float64)
    return 0.5 * (1.0 + np.tanh(0.5 * t))


def quantized(seed, N, K, gs):
    return oracle.quantize_pack(synth.weights(seed, N, K), gs)


# ------------------------------------------------------------------ dual

def test_dual_integer_exact():
    rng = np.random.default_rng(0x51)
    N, K, gs = 37, 512, 64
    q0, s0, z0, X, e0 = integer_problem(rng, N, K, gs)
    q1, s1, z1, _, _ = integer_problem(rng, N, K, gs)
    x = X[0]
    codes1 = unpack(q1, K)
    e1 = x.astype(np.int64) @ (codes1 - np.repeat(z1.astype(np.int64), gs, axis=1)).T
    r = oracle.dual(x, q0, s0, z0, q1, s1, z1, K, gs)
    np.testing.assert_array_equal(r["y0"], e0[0].astype(np.float64))
    np.testing.assert_array_equal(r["y1"], e1.astype(np.float64))


def test_dual_outputs_are_the_two_plain_products():
    N, K, gs = 29, 1024, 128
    q0, s0, z0 = quantized(0x52, N, K, gs)
    q1, s1, z1 = quantized(0x53, N, K, gs)
    x = synth.normal_f32(0x54, K)
    r = oracle.dual(x, q0, s0, z0, q1, s1, z1, K, gs)
    for y, b, (q, s, z) in ((r["y0"], r["b0"], (q0, s0, z0)), (r["y1"], r["b1"], (q1, s1, z1))):
        d = dq64(q, s, z, K, gs)
        p = d * x.astype(np.float64)[None, :]
        np.testing.assert_allclose(y, p.sum(axis=1), rtol=0, atol=1e-12 * np.max(b))
        np.testing.assert_allclose(b, np.abs(p).sum(axis=1), rtol=1e-12)
    # The same matrix twice gives the same bits twice.
    r2 = oracle.dual(x, q0, s0, z0, q0, s0, z0, K, gs)
    np.testing.assert_array_equal(r2["y0"], r2["y1"])


# ------------------------------------------------------------------ sigmoid-gated input

def test_sigmoid_gate_special_values_are_exact():
    rng = np.random.default_rng(0x61)
    N, K, gs = 23, 256, 32
    q, s, z, X, exact = integer_problem(rng, N, K, gs)
    a = (2 * X[0]).astype(np.float32)  # even integers: a / 2 is exact
    # sigma(0) = 1/2
    r = oracle.sigmoid_gated(a, np.zeros(K, np.float32), q, s, z, K, gs)
    np.testing.assert_array_equal(r["xg"], X[0].astype(np.float64))
    np.testing.assert_array_equal(r["y"], exact[0].astype(np.float64))
    # sigma(100) rounds to 1 in fp64, sigma(-800) is 0 (exp(800) overflows)
    r = oracle.sigmoid_gated(a, np.full(K, 100.0, np.float32), q, s, z, K, gs)
    np.testing.assert_array_equal(r["y"], 2 * exact[0].astype(np.float64))
    r = oracle.sigmoid_gated(a, np.full(K, -800.0, np.float32), q, s, z, K, gs)
    np.testing.assert_array_equal(r["y"], np.zeros(N))


def test_sigmoid_gate_matches_tanh_identity_and_symmetry():
    N, K, gs = 31, 1024, 128
    q, s, z = quantized(0x62, N, K, gs)
    a = synth.normal_f32(0x63, K)
    g = (3.0 * synth.normal_f32(0x64, K)).astype(np.float32)
    r = oracle.sigmoid_gated(a, g, q, s, z, K, gs)
    want = a.astype(np.float64) * expit(g.astype(np.float64))
    np.testing.assert_allclose(r["xg"], want, rtol=1e-15, atol=1e-300)
    assert np.all(np.abs(r["xg"] - a * sigma_tanh(g)) <= 4e-16 * np.abs(a))
    d = dq64(q, s, z, K, gs)
    np.testing.assert_allclose(r["y"], d @ want, rtol=0, atol=1e-12 * np.max(r["B"]))
    np.testing.assert_allclose(r["B"], np.abs(d * want[None, :]).sum(axis=1), rtol=1e-12)
    # sigma(t) + sigma(-t) = 1: the two gated products add up to the ungated one.
    rn = oracle.sigmoid_gated(a, -g, q, s, z, K, gs)
    y_plain, B_plain = oracle.matvec(a, q, s, z, K, gs)
    np.testing.assert_allclose(r["y"] + rn["y"], y_plain, rtol=0, atol=1e-12 * np.max(B_plain))


# ------------------------------------------------------------------ SwiGLU-gated input

def test_swiglu_gate_special_values_are_exact():
    rng = np.random.default_rng(0x71)
    N, K, gs = 19, 256, 64
    q, s, z, X, exact = integer_problem(rng, N, K, gs)
    up = X[0]
    # silu(0) = 0
    r = oracle.swiglu_gated(np.zeros(K, np.float32), up, q, s, z, K, gs)
    np.testing.assert_array_equal(r["y"], np.zeros(N))
    # silu(100) = 100 in fp64, so the input is 100 * up
    r = oracle.swiglu_gated(np.full(K, 100.0, np.float32), up, q, s, z, K, gs)
    np.testing.assert_array_equal(r["xg"], 100.0 * up.astype(np.float64))
    np.testing.assert_array_equal(r["y"], 100.0 * exact[0].astype(np.float64))
    # silu(-800) = -0
    r = oracle.swiglu_gated(np.full(K, -800.0, np.float32), up, q, s, z, K, gs)
    np.testing.assert_array_equal(r["y"], np.zeros(N))


def test_swiglu_gate_matches_tanh_identity():
    N, K, gs = 27, 2048, 64
    q, s, z = quantized(0x72, N, K, gs)
    g = (2.0 * synth.normal_f32(0x73, K)).astype(np.float32)
    u = synth.normal_f32(0x74, K)
    r = oracle.swiglu_gated(g, u, q, s, z, K, gs)
    g64 = g.astype(np.float64)
    want = g64 * expit(g64) * u.astype(np.float64)
    np.testing.assert_allclose(r["xg"], want, rtol=1e-15, atol=1e-300)
    assert np.all(np.abs(r["xg"] - g64 * sigma_tanh(g) * u) <= 4e-16 * np.abs(g64 * u))
    d = dq64(q, s, z, K, gs)
    np.testing.assert_allclose(r["y"], d @ want, rtol=0, atol=1e-12 * np.max(r["B"]))


# ------------------------------------------------------------------ norm + SwiGLU

def test_norm_swiglu_power_of_two():
    rng = np.random.default_rng(0x81)
    N, K, gs = 41, 1024, 128
    qg, sg, zg, _, _ = integer_problem(rng, N, K, gs)
    qu, su, zu, _, _ = integer_problem(rng, N, K, gs)
    signs = rng.choice([-1.0, 1.0], K).astype(np.float32)
    a_a = (8.0 * signs).astype(np.float32)
    zero = np.zeros(K, np.float32)
    one = np.ones(K, np.float32)
    # r = +-8, sum r^2 / K = 64, inv_rms = 1/8: the normalized input is exactly +-1.
    r = oracle.norm_swiglu(a_a, zero, one, 0.0, qg, sg, zg, qu, su, zu, K, gs)
    sg_i = signs.astype(np.int64)
    g_exact = (unpack(qg, K) - np.repeat(zg.astype(np.int64), gs, axis=1)) @ sg_i
    u_exact = (unpack(qu, K) - np.repeat(zu.astype(np.int64), gs, axis=1)) @ sg_i
    np.testing.assert_array_equal(r["g"], g_exact.astype(np.float64))
    np.testing.assert_array_equal(r["u"], u_exact.astype(np.float64))
    g64 = g_exact.astype(np.float64)
    h_want = g64 * expit(g64) * u_exact
    np.testing.assert_allclose(r["h"], h_want, rtol=1e-15, atol=1e-300)
    np.testing.assert_array_equal(r["residual"], a_a)


def test_norm_swiglu_equals_the_unfused_chain():
    N, K, gs = 33, 2048, 128
    qg, sg, zg = quantized(0x82, N, K, gs)
    qu, su, zu = quantized(0x83, N, K, gs)
    a_a = synth.normal_f32(0x84, K)
    a_b = synth.normal_f32(0x85, K)
    w = synth.uniform_f32(0x86, K, 0.5, 1.5)
    r = oracle.norm_swiglu(a_a, a_b, w, 1e-6, qg, sg, zg, qu, su, zu, K, gs)
    # residual: binary32 sum, computed here by numpy
    np.testing.assert_array_equal(r["residual"], (a_a + a_b).astype(np.float32))
    # ResidualRMSNorm -> gate and up matvecs -> SwiGLU, each step by hand in fp64
    res = (a_a + a_b).astype(np.float32).astype(np.float64)
    inv = 1.0 / np.sqrt(np.mean(res * res) + np.float64(np.float32(1e-6)))
    x = res * inv * w.astype(np.float64)
    g = dq64(qg, sg, zg, K, gs) @ x
    u = dq64(qu, su, zu, K, gs) @ x
    np.testing.assert_allclose(r["g"], g, rtol=0, atol=1e-12 * np.max(r["bg"]))
    np.testing.assert_allclose(r["u"], u, rtol=0, atol=1e-12 * np.max(r["bu"]))
    scale = np.abs(u) * np.max(r["bg"]) + np.abs(g) * np.max(r["bu"])
    np.testing.assert_allclose(r["h"], g * expit(g) * u, rtol=0, atol=1e-11 * np.max(scale) + 1e-300)


# ------------------------------------------------------------------ embedding gather

def test_embedding_hand_values():
    # Row 1 holds codes 0..15 in its first two words (low nibble first), codes 0
    # elsewhere; group 0 (inputs 0..31) has scale 0.5 and zero 3, group 1
    # (inputs 32..63) scale -2 and zero 15: values by hand.
    K, gs = 64, 32
    q = np.zeros((3, K // 8), np.uint32)
    q[1, 0] = 0x76543210
    q[1, 1] = 0xFEDCBA98
    s = np.array([[1.0, 1.0], [0.5, -2.0], [1.0, 1.0]], np.float32)
    z = np.array([[0.0, 0.0], [3.0, 15.0], [0.0, 0.0]], np.float32)
    out = oracle.embedding(np.array([1], np.int32), q, s, z, K, gs)
    want = np.zeros(K, np.float32)
    want[:8] = [-1.5, -1.0, -0.5, 0.0, 0.5, 1.0, 1.5, 2.0]
    want[8:16] = [2.5, 3.0, 3.5, 4.0, 4.5, 5.0, 5.5, 6.0]       # (8..15 - 3) * 0.5
    want[16:32] = -1.5                                           # codes 0 in group 0: (0 - 3) * 0.5
    want[32:] = 30.0                                             # codes 0 in group 1: (0 - 15) * -2
    np.testing.assert_array_equal(out[0], want)


def test_embedding_rows_match_an_independent_decode():
    N, K, gs = 50, 512, 128
    q, s, z = quantized(0x91, N, K, gs)
    ids = np.array([0, 49, 7, 7, -1, 50, 3, 2**31 - 1], np.int32)
    out = oracle.embedding(ids, q, s, z, K, gs)
    codes = unpack(q, K).astype(np.float32)
    dq = (codes - np.repeat(z, gs, axis=1)) * np.repeat(s, gs, axis=1)  # binary32, one rounding
    for t, n in enumerate(ids):
        want = dq[n] if 0 <= n < N else np.zeros(K, np.float32)
        np.testing.assert_array_equal(out[t].view(np.uint32), want.astype(np.float32).view(np.uint32))
