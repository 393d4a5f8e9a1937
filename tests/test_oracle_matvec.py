"""Pins of the oracle's matvec family (CPU only).

Closed forms (one-hot inputs, integer-exact weights, codes equal to the zero
point), invariants the pages state (split-4 routing equals one matvec over the
concatenated columns; lanes never interact; fused gated/norm forms equal their
unfused chains), hand-computed RMS values, and a check that the error bound
admits a naive binary32 implementation.
"""
import math

import numpy as np
import pytest

import oracle
import synth


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """codes int [N, K] in 0..15 -> u32 [N, K/8], input k at bits 4*(k%8) of word k/8."""
    N, K = codes.shape
    c = codes.astype(np.uint64).reshape(N, K // 8, 8)
    words = np.zeros((N, K // 8), np.uint64)
    for t in range(8):
        words |= c[:, :, t] << np.uint64(4 * t)
    return words.astype(np.uint32)


def integer_problem(rng, N, K, gs, M=1):
    """Codes, integer zeros, unit scales and integer X in [-8, 8]: every partial
    sum is an integer far below 2^24, so the exact result is an int64 sum."""
    codes = rng.integers(0, 16, (N, K))
    zeros = rng.integers(0, 16, (N, K // gs)).astype(np.float32)
    scales = np.ones((N, K // gs), np.float32)
    X = rng.integers(-8, 9, (M, K)).astype(np.float32)
    exact = X.astype(np.int64) @ (codes - np.repeat(zeros.astype(np.int64), gs, axis=1)).T
    return pack_codes(codes), scales, zeros, X, exact


def random_problem(seed, N, K, gs, M=1):
    W = synth.weights(seed, N, K)
    q, s, z = oracle.quantize_pack(W, gs)
    X = synth.lanes(seed + 1, M, K)
    return W, q, s, z, X


# ------------------------------------------------------------- closed forms

@pytest.mark.parametrize("K,gs", [(256, 32), (512, 128), (384, 64)])
def test_one_hot_returns_the_dequantized_column_entry(K, gs):
    N = 24
    _, q, s, z, _ = random_problem(0x11, N, K, gs)
    dq = oracle.dequant(q, s, z, K, gs)
    for k in (0, 1, 7, 8, gs - 1, gs, K - 1):
        x = np.zeros(K, np.float32)
        x[k] = 1.0
        y, B = oracle.matvec(x, q, s, z, K, gs)
        np.testing.assert_array_equal(y, dq[:, k].astype(np.float64))
        np.testing.assert_array_equal(B, np.abs(dq[:, k]).astype(np.float64))


@pytest.mark.parametrize("M", [1, 3, 8])
def test_integer_exact(M):
    rng = np.random.default_rng(5 + M)
    N, K, gs = 40, 512, 64
    q, s, z, X, exact = integer_problem(rng, N, K, gs, M)
    Y, _ = oracle.matvec(X, q, s, z, K, gs)
    np.testing.assert_array_equal(Y, exact.astype(np.float64))


def test_codes_equal_to_zero_point_give_zero():
    N, K, gs = 16, 256, 32
    zeros = np.tile(np.arange(16, dtype=np.float32)[:, None], (1, K // gs))[:N]
    codes = np.repeat(zeros.astype(np.int64), gs, axis=1)
    q = pack_codes(codes)
    s = np.full((N, K // gs), 0.37, np.float32)
    x = synth.normal_f32(3, K)
    y, B = oracle.matvec(x, q, s, zeros, K, gs)
    assert np.all(y == 0.0) and np.all(B == 0.0)


def test_scale_multiplies_the_group():
    # Doubling one group's scale doubles that group's contribution only.
    rng = np.random.default_rng(9)
    N, K, gs = 8, 256, 64
    q, s, z, X, _ = integer_problem(rng, N, K, gs)
    x = X[0]
    s2 = s.copy()
    s2[:, 2] = 2.0
    y1, _ = oracle.matvec(x, q, s, z, K, gs)
    y2, _ = oracle.matvec(x, q, s2, z, K, gs)
    codes = np.array([[(int(w) >> (4 * t)) & 15 for w in row for t in range(8)] for row in q])
    part = ((codes[:, 2 * gs:3 * gs] - z[:, 2:3]) * x[2 * gs:3 * gs]).sum(axis=1)
    np.testing.assert_array_equal(y2 - y1, part.astype(np.float64))


def test_matches_fp64_dot_of_dequantized_matrix():
    N, K, gs = 33, 640, 64
    _, q, s, z, X = random_problem(0x21, N, K, gs, M=2)
    dq = oracle.dequant(q, s, z, K, gs).astype(np.float64)
    Y, B = oracle.matvec(X, q, s, z, K, gs)
    ref = X.astype(np.float64) @ dq.T
    np.testing.assert_allclose(Y, ref, rtol=0, atol=1e-12 * np.max(B))
    np.testing.assert_allclose(B, np.abs(X.astype(np.float64)) @ np.abs(dq).T, rtol=1e-12)


def test_quantized_matvec_tracks_the_float_matvec():
    # Quantization error per weight is at most half a step, so |y_q - y_f| <= sum |x| * scale / 2.
    N, K, gs = 64, 1024, 128
    W, q, s, z, X = random_problem(0x31, N, K, gs)
    y, _ = oracle.matvec(X[0], q, s, z, K, gs)
    yf = W.astype(np.float64) @ X[0].astype(np.float64)
    bound = (np.abs(X[0]).astype(np.float64)[None, :] * np.repeat(s, gs, axis=1) * 0.5).sum(1)
    assert np.all(np.abs(y - yf) <= bound * (1 + 1e-5))


# -------------------------------------------------------------- invariants

def test_lanes_are_independent():
    N, K, gs = 29, 512, 128
    _, q, s, z, X = random_problem(0x41, N, K, gs, M=5)
    Y, B = oracle.matvec(X, q, s, z, K, gs)
    for m in range(5):
        y, b = oracle.matvec(X[m], q, s, z, K, gs)
        np.testing.assert_array_equal(Y[m], y)
        np.testing.assert_array_equal(B[m], b)


@pytest.mark.parametrize("splits", [(40, 50, 60), (0, 0, 0), (71, 71, 71), (10, 10, 70), (0, 35, 35)])
def test_split4_equals_one_matvec_over_concatenation(splits):
    N, K, gs = 71, 256, 32
    _, q, s, z, X = random_problem(0x51, N, K, gs)
    n0, n1, n2 = splits
    outs, bs = oracle.split4(X[0], q, s, z, K, gs, n0, n1, n2)
    y, b = oracle.matvec(X[0], q, s, z, K, gs)
    assert [len(o) for o in outs] == [n0, n1 - n0, n2 - n1, N - n2]
    np.testing.assert_array_equal(np.concatenate(outs), y)
    np.testing.assert_array_equal(np.concatenate(bs), b)


def test_split4_of_separately_quantized_parts():
    # Quantizing four matrices apart and appending their q/scales/zeros gives
    # the same result as routing one matvec (the quantizer is column-local).
    K, gs = 256, 64
    parts = [synth.weights(0x61 + i, n, K) for i, n in enumerate((12, 5, 7, 3))]
    x = synth.normal_f32(0x66, K)
    qs = [oracle.quantize_pack(W, gs) for W in parts]
    qc = np.concatenate([t[0] for t in qs])
    sc = np.concatenate([t[1] for t in qs])
    zc = np.concatenate([t[2] for t in qs])
    outs, _ = oracle.split4(x, qc, sc, zc, K, gs, 12, 17, 24)
    for o, (q, s, z) in zip(outs, qs):
        y, _ = oracle.matvec(x, q, s, z, K, gs)
        np.testing.assert_array_equal(o, y)


def test_gated_closed_form_integer():
    rng = np.random.default_rng(21)
    N, K, gs = 30, 256, 32
    qg, sg, zg, X, g_exact = integer_problem(rng, N, K, gs)
    qu, su, zu, _, _ = integer_problem(rng, N, K, gs)
    x = X[0]
    codes_u = np.array([[(int(w) >> (4 * t)) & 15 for w in row for t in range(8)] for row in qu])
    u_exact = (codes_u - np.repeat(zu, gs, axis=1)) @ x.astype(np.float64)
    out = oracle.gated(x, qg, sg, zg, qu, su, zu, K, gs)
    np.testing.assert_array_equal(out["g"], g_exact[0].astype(np.float64))
    np.testing.assert_array_equal(out["u"], u_exact)
    for n in range(N):
        g, u = float(g_exact[0, n]), float(u_exact[n])
        # silu(g) = g * sigmoid(g), with the logistic function evaluated stably.
        sig = 1.0 / (1.0 + math.exp(-g)) if g >= 0 else math.exp(g) / (1.0 + math.exp(g))
        assert out["h"][n] == pytest.approx(g * sig * u, rel=1e-13, abs=0.0)


def test_gated_is_not_symmetric_in_gate_and_up():
    N, K, gs = 16, 256, 64
    _, qg, sg, zg, X = random_problem(0x71, N, K, gs)
    _, qu, su, zu, _ = random_problem(0x73, N, K, gs)
    a = oracle.gated(X[0], qg, sg, zg, qu, su, zu, K, gs)
    b = oracle.gated(X[0], qu, su, zu, qg, sg, zg, K, gs)
    np.testing.assert_array_equal(a["g"], b["u"])
    assert not np.allclose(a["h"], b["h"])
    # silu limits: silu(0) = 0, silu(t) -> t for large t, -> 0 for very negative t.
    assert a["h"][np.argmax(a["g"])] == pytest.approx(
        a["g"].max() / (1 + math.exp(-a["g"].max())) * a["u"][np.argmax(a["g"])])


def test_norm_power_of_two_special_case():
    # a_b = 0, w_norm = 1, eps = 0, a_a = +-2^p: mean square is 4^p, inv_rms = 2^-p
    # exactly and the normed vector is +-1, so y is an integer-exact matvec.
    rng = np.random.default_rng(31)
    N, K, gs = 20, 512, 64
    q, s, z, _, _ = integer_problem(rng, N, K, gs)
    signs = rng.choice([-1.0, 1.0], K).astype(np.float32)
    a_a = (signs * 2.0 ** 5).astype(np.float32)
    out = oracle.norm(a_a, np.zeros(K, np.float32), np.ones(K, np.float32), 0.0, q, s, z, K, gs)
    np.testing.assert_array_equal(out["residual"], a_a)
    np.testing.assert_array_equal(out["normed"], signs.astype(np.float64))
    y, _ = oracle.matvec(signs, q, s, z, K, gs)
    np.testing.assert_array_equal(out["y"], y)


def test_norm_hand_computed_rms():
    # r = a_a + a_b = [3, 4, 0, 0, 0, 0, 0, 0]: mean square 25/8, eps 0.
    K = 8
    a_a = np.array([1, 4, 0.5, -0.5, 0, 0, 0, 0], np.float32)
    a_b = np.array([2, 0, -0.5, 0.5, 0, 0, 0, 0], np.float32)
    w = np.array([1, 2, 3, 4, 5, 6, 7, 8], np.float32)
    q = np.zeros((1, 1), np.uint32)
    out = oracle.norm(a_a, a_b, w, 0.0, q, np.ones((1, 1), np.float32),
                      np.zeros((1, 1), np.float32), K, 8)
    np.testing.assert_array_equal(out["residual"], np.array([3, 4, 0, 0, 0, 0, 0, 0], np.float32))
    inv = 1.0 / math.sqrt(25.0 / 8.0)
    np.testing.assert_allclose(out["normed"][:2], [3 * inv * 1, 4 * inv * 2], rtol=1e-15)
    assert np.all(out["normed"][2:] == 0.0)
    # With eps: inv_rms = 1 / sqrt(25/8 + eps).
    out_e = oracle.norm(a_a, a_b, w, 0.875, q, np.ones((1, 1), np.float32),
                        np.zeros((1, 1), np.float32), K, 8)
    np.testing.assert_allclose(out_e["normed"][0], 3 * 0.5, rtol=1e-15)  # 25/8 + 7/8 = 4


def test_norm_equals_matvec_of_normed_vector():
    N, K, gs = 25, 512, 128
    _, q, s, z, _ = random_problem(0x81, N, K, gs)
    a_a = synth.normal_f32(0x82, K)
    a_b = synth.normal_f32(0x83, K)
    w = synth.uniform_f32(0x84, K, 0.5, 1.5)
    out = oracle.norm(a_a, a_b, w, 1e-6, q, s, z, K, gs)
    dq = oracle.dequant(q, s, z, K, gs).astype(np.float64)
    ref = dq @ out["normed"]
    np.testing.assert_allclose(out["y"], ref, rtol=0, atol=1e-12 * out["B"].max())
    # The RMS of the normed vector divided by the gain is 1 (eps is negligible).
    r = out["normed"] / w.astype(np.float64)
    assert abs(math.sqrt(np.mean(r * r)) - 1.0) < 1e-6


# ----------------------------------------------------------- tolerance sanity

@pytest.mark.parametrize("K,gs", [(1024, 128), (4096, 128), (14336, 128), (5120, 64)])
def test_fp32_naive_dot_passes_the_bound(K, gs):
    # The bound 1e-4 * sum|x w| + 1e-6 must admit an ordinary sequential binary32
    # dot product at every configuration's K (sampled columns).
    N = 48
    _, q, s, z, X = random_problem(0x91 + K, N, K, gs)
    Y, B = oracle.matvec(X, q, s, z, K, gs)
    Yf = oracle.matvec_f32(X, q, s, z, K, gs).astype(np.float64)
    assert np.all(np.abs(Yf - Y) <= oracle.tolerance(B))
    # ... and is tight enough to reject a dropped group.
    s_bad = s.copy()
    s_bad[:, 0] = 0.0
    Yb, _ = oracle.matvec(X, q, s_bad, z, K, gs)
    assert np.mean(np.abs(Yb - Y) > oracle.tolerance(B)) > 0.9
