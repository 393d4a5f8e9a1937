"""GPU parity of int4_quantize_pack: codes, scales and zeros bit-exact with
the oracle on hand-worked groups, adversarial groups and random matrices."""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from helpers import adversarial_groups

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quantizer_examples.json")


@pytest.fixture(scope="module")
def q4():
    import torch
    torch.cuda.set_device(0)
    import int4_group_quantized_quant_amd as m
    return m


def gpu_quantize(q4, W, gs):
    import torch
    Wd = torch.from_numpy(np.ascontiguousarray(W, np.float32)).cuda()
    q, s, z = q4.int4_quantize_pack(Wd, gs)
    torch.cuda.synchronize()
    return q.cpu().numpy().view(np.uint32), s.cpu().numpy(), z.cpu().numpy()


def assert_bits_equal(W, gs, got, what):
    q_ref, s_ref, z_ref = oracle.quantize_pack(W, gs)
    q, s, z = got
    for name, a, b in (("q", q, q_ref), ("scales", s.view(np.uint32), s_ref.view(np.uint32)),
                       ("zeros", z.view(np.uint32), z_ref.view(np.uint32))):
        if not np.array_equal(a, b):
            idx = np.argwhere(a != b)[:5]
            raise AssertionError(f"{what}: {name} differs at {idx.tolist()}")


def test_worked_examples(q4):
    ex = json.load(open(GOLDEN))["examples"]
    rows = [np.array(e["w"], np.float32) for e in ex if "w" in e]
    rows += [np.full(32, e["w_const"], np.float32) for e in ex if "w_const" in e]
    # Groups given in units of the smallest subnormal (the scale-underflow case).
    sub = [e for e in ex if "w_units_of_min_subnormal" in e]
    rows += [(np.array(e["w_units_of_min_subnormal"], np.float64) * 2.0 ** -149).astype(np.float32)
             for e in sub]
    W = np.stack(rows)
    got = gpu_quantize(q4, W, 32)
    assert_bits_equal(W, 32, got, "worked examples")
    with_words = [e for e in ex if "w" in e] + [None] * sum("w_const" in e for e in ex) + sub
    for i, e in enumerate(with_words):
        if e is None:
            continue
        words = np.array([int(h, 16) for h in e["words"]], np.uint32)
        np.testing.assert_array_equal(got[0][i], words, err_msg=e["name"])
        np.testing.assert_array_equal(got[2][i], np.float32(e["zero"]), err_msg=e["name"])


@pytest.mark.parametrize("gs", [32, 64, 96, 128, 256, 544])
def test_adversarial_groups(q4, gs):
    rng = np.random.default_rng(100 + gs)
    G = adversarial_groups(rng, 400, gs)
    W = G.reshape(100, 4 * gs)  # four groups per column
    assert_bits_equal(W, gs, gpu_quantize(q4, W, gs), f"adversarial gs={gs}")


@pytest.mark.parametrize("N,K,gs", [(1, 32, 32), (7, 96, 32), (333, 1024, 128), (64, 5120, 64),
                                    (17, 14336, 128), (5, 4096, 4096),
                                    (3, 8192, 8192),  # groups wider than the wave kernel takes
                                    (9, 2880, 160)])  # 20 words per group: lanes padded to 32
def test_random_shapes(q4, N, K, gs):
    W = synth.weights(0xA000 + N + K + gs, N, K)
    assert_bits_equal(W, gs, gpu_quantize(q4, W, gs), f"N={N} K={K} gs={gs}")


def test_million_groups(q4):
    # 2^20 random groups of 32 (N(0, 0.02) with one x20 outlier per 1% of groups).
    W = synth.weights(0xA100, 8192, 4096)
    synth.add_group_outliers(W, 32, 0xA101)
    assert_bits_equal(W, 32, gpu_quantize(q4, W, 32), "1M groups")


def test_empty(q4):
    import torch
    W = torch.empty((0, 256), dtype=torch.float32, device="cuda")
    q, s, z = q4.int4_quantize_pack(W, 64)
    assert q.shape == (0, 32) and s.shape == (0, 4)
