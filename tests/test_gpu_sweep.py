"""A seeded sweep of random shapes through every launch planner: column
counts from 1 up, K from one group to past the register kernel's range,
every lane count, group sizes 32..256.  Each call is checked against the
oracle (codes bit-exact upstream, outputs within 1e-4 * sum|x w| + 1e-6).
The shapes are drawn once from a fixed seed and listed in the test ids, so
a failure names its shape."""
import numpy as np
import pytest

import oracle
import synth
from helpers import assert_dot_close, gated_tolerance

pytestmark = pytest.mark.gpu


def _shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        gs = int(rng.choice([32, 64, 128, 256]))
        K = gs * int(rng.integers(1, max(2, 20480 // gs)))
        if rng.random() < 0.5:  # bias toward decode-sized K
            K = gs * int(rng.integers(1, max(2, 6144 // gs)))
        N = int(rng.choice([1, 2, 15, 16, 17, 63, 100, 256, 257, 511, 512, 1000, 1536, 2049, 4099]))
        M = int(rng.integers(1, 9))
        out.append((N, K, gs, M))
    return out


SHAPES = _shapes(40, 0x5EED)


@pytest.fixture(scope="module")
def q4():
    import torch
    torch.cuda.set_device(0)
    import int4_group_quantized_quant_amd as m
    return m


def dev(*arrs):
    import torch
    return [torch.from_numpy(np.ascontiguousarray(a.view(np.int32) if a.dtype == np.uint32 else a)).cuda()
            for a in arrs]


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


@pytest.mark.parametrize("N,K,gs,M", SHAPES, ids=[f"N{n}-K{k}-gs{g}-M{m}" for n, k, g, m in SHAPES])
def test_sweep(q4, N, K, gs, M):
    seed = (N * 7919 + K * 31 + gs * 3 + M) & 0xFFFFFF
    w = oracle.quantize_pack(synth.weights(seed, N, K), gs)
    X = synth.lanes(seed + 1, M, K)
    wd = dev(*w)
    Y = q4.int4_matvec(*dev(X), *wd)
    Y_ref, B = oracle.matvec(X, *w, K, gs)
    assert_dot_close(host(Y), Y_ref, B, f"matvec N={N} K={K} gs={gs} M={M}")

    x = X[0]
    xd, = dev(x)
    if N >= 4:  # split4 on a split that leaves every range non-empty
        n0, n1, n2 = N // 4, N // 2, (3 * N) // 4
        outs = q4.int4_matvec_split4(xd, *wd, n0, n1, n2)
        y_ref, B1 = oracle.matvec(x, *w, K, gs)
        assert_dot_close(np.concatenate([host(o) for o in outs]), y_ref, B1, "split4")
    w2 = oracle.quantize_pack(synth.weights(seed + 2, N, K), gs)
    w2d = dev(*w2)
    h = q4.int4_matvec_gated(xd, *wd, *w2d)
    ref = oracle.gated(x, *w, *w2, K, gs)
    assert np.all(np.abs(host(h).astype(np.float64) - ref["h"]) <= gated_tolerance(ref)), "gated"
    if M >= 2:
        y0, y1 = q4.int4_matvec_dual(*dev(X), *wd, *w2d)
        y0, y1 = host(y0), host(y1)
        for m in range(M):  # the oracle's dual takes one lane
            r = oracle.dual(X[m], *w, *w2, K, gs)
            assert_dot_close(y0[m], r["y0"], r["b0"], f"dual y0 lane {m}")
            assert_dot_close(y1[m], r["y1"], r["b1"], f"dual y1 lane {m}")
    a_b = synth.normal_f32(seed + 3, K)
    w_n = synth.uniform_f32(seed + 4, K, 0.5, 1.5)
    if K <= 40960:
        y, res, nrm = q4.int4_matvec_norm(*dev(x, a_b, w_n), 1e-6, *wd)
        r = oracle.norm(x, a_b, w_n, 1e-6, *w, K, gs)
        assert_dot_close(host(y), r["y"], r["B"], "norm")
        np.testing.assert_array_equal(host(res), r["residual"])
    if N % gs == 0 and N >= gs:
        # The MLP block with D = K, F = N: gate/up are this shape, down is F x D transposed.
        wdn = oracle.quantize_pack(synth.weights(seed + 5, K, N), gs)
        hm, ym = q4.int4_mlp(xd, *wd, *w2d, *dev(*wdn))
        hh = host(hm)
        assert np.all(np.abs(hh.astype(np.float64) - ref["h"]) <= gated_tolerance(ref)), "mlp h"
        y_ref, B2 = oracle.matvec(hh, *wdn, N, gs)
        assert_dot_close(host(ym), y_ref, B2, "mlp y")
