"""Pins of the oracle's quantizer, dequantizer and nibble layout (CPU only).

Each check compares the oracle with something other than itself: hand-worked
groups (tests/golden/quantizer_examples.json), a brute-force search over all
sixteen codes, and bounds that follow from the definition.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quantizer_examples.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _example(name):
    for ex in _golden()["examples"]:
        if ex["name"] == name:
            return ex
    raise KeyError(name)


def _words(hexes):
    return np.array([int(h, 16) for h in hexes], dtype=np.uint32)


def _scale_of(ex):
    if "scale" in ex:
        return np.float32(ex["scale"])
    a, b = ex["scale_expr"].replace("float32(", "").replace(")", "").split(" / ")
    return np.float32(np.float32(float(a)) / np.float32(float(b)))


@pytest.mark.parametrize("name", ["A_ties_to_even", "B_zero_clamped_at_0_code_clamped_at_15",
                                  "C_zero_clamped_at_15", "E_zero_tie_rounds_down_to_even",
                                  "F_zero_tie_rounds_up_to_even"])
def test_worked_examples(name):
    ex = _example(name)
    W = np.array(ex["w"], np.float32).reshape(1, 32)
    q, s, z = oracle.quantize_pack(W, 32)
    assert q.shape == (1, 4) and s.shape == (1, 1) and z.shape == (1, 1)
    assert s[0, 0].tobytes() == _scale_of(ex).tobytes()
    assert z[0, 0].tobytes() == np.float32(ex["zero"]).tobytes()
    np.testing.assert_array_equal(q[0], _words(ex["words"]))


def test_ties_are_not_rounded_half_up():
    ex = _example("A_ties_to_even")
    q, _, _ = oracle.quantize_pack(np.array(ex["w"], np.float32).reshape(1, 32), 32)
    assert not np.array_equal(q[0], _words(ex["words_if_ties_rounded_half_up"]))


@pytest.mark.parametrize("name,alt", [("E_zero_tie_rounds_down_to_even", "words_if_zero_rounded_half_up"),
                                      ("F_zero_tie_rounds_up_to_even", "words_if_zero_truncated")])
def test_zero_point_tie_rule(name, alt):
    # -min/scale is exactly k + 1/2 in both groups: 4.5 -> 4 and 3.5 -> 4 under
    # ties to even.  A half-up zero fails E, a truncated one fails F.
    ex = _example(name)
    q, s, z = oracle.quantize_pack(np.array(ex["w"], np.float32).reshape(1, 32), 32)
    assert z[0, 0] == 4.0
    np.testing.assert_array_equal(q[0], _words(ex["words"]))
    assert not np.array_equal(q[0], _words(ex[alt]))
    np.testing.assert_array_equal(_unpack(q[0], 32), np.array(ex["codes"]))


def _min_subnormal_group(ex):
    units = np.array(ex["w_units_of_min_subnormal"], np.float64)
    return (units * 2.0 ** -149).astype(np.float32)


def test_scale_underflow_group():
    # max > min, but (max - min) / 15 underflows to 0: stored as an all-zero group.
    ex = _example("G_scale_underflows_to_zero")
    w = _min_subnormal_group(ex)
    assert w.min() < 0 < w.max()
    assert np.float32(w.max() - w.min()) / np.float32(15) == 0.0
    q, s, z = oracle.quantize_pack(w.reshape(1, 32), 32)
    assert s[0, 0] == 0.0 and z[0, 0] == 0.0 and z[0, 0] != ex["zero_if_underflow_not_handled"]
    np.testing.assert_array_equal(q[0], _words(ex["words"]))
    assert not np.any(np.isnan(oracle.dequant(q, s, z, 32, 32)))


def test_example_a_dequantizes_onto_the_half_grid():
    ex = _example("A_ties_to_even")
    w = np.array(ex["w"], np.float32)
    q, s, z = oracle.quantize_pack(w.reshape(1, 32), 32)
    dq = oracle.dequant(q, s, z, 32, 32)[0]
    codes = np.array(ex["codes"], np.float64)
    np.testing.assert_array_equal(dq.astype(np.float64), (codes - 4.0) * 0.5)
    assert np.max(np.abs(dq - w)) == 0.25  # only the 0.125 entry is off the grid


@pytest.mark.parametrize("name", ["D_constant_positive", "D_constant_negative", "D_all_zero"])
def test_constant_groups(name):
    ex = _example(name)
    W = np.full((1, 32), ex["w_const"], np.float32)
    q, s, z = oracle.quantize_pack(W, 32)
    assert s[0, 0].tobytes() == _scale_of(ex).tobytes()
    assert z[0, 0].tobytes() == np.float32(ex["zero"]).tobytes()
    word = sum(ex["code"] << (4 * t) for t in range(8))
    np.testing.assert_array_equal(q[0], np.full(4, word, np.uint32))
    dq = oracle.dequant(q, s, z, 32, 32)[0]
    assert np.all(dq == np.float32(ex["dequant"]))
    assert not np.any(np.isnan(dq))


def test_nibble_order_pack_and_unpack():
    nib = _golden()["nibble_order"]
    # min 0, max 15 -> scale 1, zero 0, so codes equal the values.
    w = np.array(nib["codes"] + [15] * 16, np.float32).reshape(1, 32)
    q, s, z = oracle.quantize_pack(w, 32)
    assert s[0, 0] == 1.0 and z[0, 0] == 0.0
    np.testing.assert_array_equal(q[0, :2], _words(nib["words"]))
    np.testing.assert_array_equal(q[0, 2:], np.array([0xFFFFFFFF] * 2, np.uint32))
    # Unpack the hand-written words through the dequantizer (scale 1, zero 0).
    qq = np.array([[0x76543210, 0xFEDCBA98, 0, 0]], np.uint32)
    dq = oracle.dequant(qq, np.ones((1, 1), np.float32), np.zeros((1, 1), np.float32), 32, 32)
    np.testing.assert_array_equal(dq[0, :16], np.arange(16, dtype=np.float32))


def test_group_and_column_indexing():
    # Two columns, two groups each, every group a different constant grid, so
    # a swapped column or group index shows up in scales/zeros.
    K, gs = 64, 32
    W = np.zeros((2, K), np.float32)
    for n in range(2):
        for g in range(2):
            base = 1 + 2 * n + g
            W[n, g * gs:(g + 1) * gs] = np.linspace(-base, 14 * base / 15.0, gs)
            W[n, g * gs] = -base
            W[n, g * gs + 1] = 2 * base  # max - min = 3 * base -> scale = base / 5
    q, s, z = oracle.quantize_pack(W, gs)
    for n in range(2):
        for g in range(2):
            base = 1 + 2 * n + g
            assert s[n, g] == np.float32(np.float32(3 * base) / np.float32(15))
            assert z[n, g] == 5.0
            first = (q[n, g * 4] & 0xF, (q[n, g * 4] >> 4) & 0xF)
            assert first == (0, 15)


def _brute_force_codes(w, scale, zero):
    """argmin over all 16 codes of |fl32(w/scale) - (c - zero)|, ties to the
    code with c - zero even.  Independent of rint and of the clamp."""
    t = (np.float32(w) / np.float32(scale)).astype(np.float64)
    cand = np.arange(16, dtype=np.float64)
    out = []
    for ti in t:
        d = np.abs(ti - (cand - zero))
        best = np.flatnonzero(d == d.min())
        if len(best) > 1:
            even = [c for c in best if (int(c) - int(zero)) % 2 == 0]
            best = even
        out.append(int(best[0]))
    return np.array(out)


def _unpack(words, count):
    codes = []
    for wd in words:
        for t in range(8):
            codes.append((int(wd) >> (4 * t)) & 0xF)
    return np.array(codes[:count])


def _adversarial_groups(rng, n_groups, gs):
    groups = []
    kinds = ["normal", "ties", "subnormal", "large", "outlier", "positive", "negative", "tiny_range"]
    for i in range(n_groups):
        kind = kinds[i % len(kinds)]
        if kind == "normal":
            g = rng.normal(0, 0.02, gs)
        elif kind == "ties":
            g = rng.integers(-16, 16, gs) * 0.25  # many exact .5 quotients
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
        else:
            g = 1.0 + rng.integers(0, 3, gs) * 1e-7
        groups.append(np.asarray(g, np.float32))
    return np.stack(groups)


@pytest.mark.parametrize("gs", [32, 64, 128])
def test_brute_force_codes(gs):
    rng = np.random.default_rng(1234 + gs)
    G = _adversarial_groups(rng, 96, gs)
    W = G.reshape(-1, gs)  # one group per column
    q, s, z = oracle.quantize_pack(W, gs)
    for i in range(W.shape[0]):
        scale, zero = float(s[i, 0]), float(z[i, 0])
        codes = _unpack(q[i], gs)
        assert zero == int(zero) and 0 <= zero <= 15
        if scale == 0.0:
            assert np.all(codes == 0)
            continue
        np.testing.assert_array_equal(codes, _brute_force_codes(W[i], scale, zero),
                                      err_msg=f"group {i}")
        # scale is (hi - lo) / 15 up to the two binary32 roundings (range, quotient).
        lo, hi = float(W[i].min()), float(W[i].max())
        if hi > lo:
            bound = (float(np.spacing(np.float32(scale))) / 2
                     + float(np.spacing(np.float32(hi - lo))) / 30)
            assert abs(scale - (hi - lo) / 15) <= bound


def test_reconstruction_bound_when_unclamped():
    rng = np.random.default_rng(7)
    gs = 128
    W = rng.normal(0, 0.02, (64, 4 * gs)).astype(np.float32)
    W[:, ::gs] = -np.abs(W[:, ::gs]) - 1e-3  # every group straddles zero
    W[:, 1::gs] = np.abs(W[:, 1::gs]) + 1e-3
    q, s, z = oracle.quantize_pack(W, gs)
    dq = oracle.dequant(q, s, z, W.shape[1], gs)
    scale_per_k = np.repeat(s, gs, axis=1).astype(np.float64)
    err = np.abs(W.astype(np.float64) - dq.astype(np.float64))
    # Half a step, plus the few roundings of w/scale, rint and (q-z)*scale.
    assert np.all(err <= scale_per_k * 0.5 * (1 + 2.0 ** -20) + 1e-12)
    assert np.all((z > 0) & (z < 15))


def test_codes_fill_range_for_straddling_groups():
    # With min < 0 < max, the minimum maps to code 0 or 1 and the maximum to 14 or 15.
    rng = np.random.default_rng(11)
    W = rng.normal(0, 0.02, (32, 128)).astype(np.float32)
    q, s, z = oracle.quantize_pack(W, 128)
    for i in range(32):
        codes = _unpack(q[i], 128)
        assert codes[np.argmin(W[i])] <= 1
        assert codes[np.argmax(W[i])] >= 14
