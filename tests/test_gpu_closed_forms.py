"""GPU closed forms that hold for any valid int4 triplet.

1. Codes equal to their zero points dequantize to exactly 0, so every output
   that is a sum of such products is exactly 0, whatever the scales
   ((code - zero) * scale, gerbil 1.12.0->1.13.0 page 12, WGSL_QUAD_MATVEC_INT4).
   This runs through every entry point, on the one-lane register kernel
   (K = 4096), the LDS kernel (K = 20480), the matrix-core lanes, the
   prefill GEMM and the fused MLP, at non-power-of-two scales and with
   every zero point 0..15 present.
2. Codes equal to their zero points except one per column: each output is
   then a single product x_k * (+-1) * scale, so it must lie within the dot
   bound of the oracle's value although nearly every term cancels.  A
   kernel that folds the zero point out of the per-input work (sum x*code
   minus zero * sum x) fails this at every zero point that is not a power
   of two.
Every output of every call is compared, over ragged column counts.
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import assert_dot_close, pack_codes

pytestmark = pytest.mark.gpu

GS = 128
N = 1000  # several column blocks and a ragged tail


@pytest.fixture(scope="module")
def q4():
    import torch
    torch.cuda.set_device(0)
    import int4_group_quantized_quant_amd as m
    return m


def dev(*arrs):
    import torch
    return [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in arrs]


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def zero_triplet(seed, n, K, scale, off_by_one=False):
    """Codes equal to their group's zero point (every value 0..15 used), with
    all scales `scale`; with off_by_one, one random code per column moved by
    one step (towards the middle of 0..15)."""
    rng = np.random.default_rng(seed)
    G = K // GS
    zeros = rng.integers(0, 16, (n, G))
    zeros.ravel()[:16] = np.arange(16)
    codes = np.repeat(zeros, GS, axis=1)
    if off_by_one:
        ks = rng.integers(0, K, n)
        for i, k in enumerate(ks):
            codes[i, k] += 1 if codes[i, k] < 8 else -1
    q = pack_codes(codes).view(np.int32)
    s = np.full((n, G), scale, np.float32)
    return q, s, zeros.astype(np.float32)


def assert_zero(a, what):
    a = np.asarray(a)
    nz = np.flatnonzero(a.ravel() != 0)
    assert nz.size == 0, f"{what}: {nz.size} of {a.size} outputs non-zero, first {a.ravel()[nz[:4]]}"


@pytest.mark.parametrize("K", [4096, 20480])
@pytest.mark.parametrize("scale", [0.37, 1.0])
def test_one_lane_entry_points_give_zero(q4, K, scale):
    import torch
    w = dev(*zero_triplet(K + int(scale * 100), N, K, scale))
    w2 = dev(*zero_triplet(K + 7, N, K, scale))
    x, a, b = dev(synth.normal_f32(0xC01, K), synth.normal_f32(0xC02, K), synth.normal_f32(0xC03, K))
    g = dev(synth.uniform_f32(0xC04, K, 0.5, 1.5))[0]
    assert_zero(host(q4.int4_matvec(x, *w)), "matvec")
    assert_zero(host(torch.cat(q4.int4_matvec_split4(x, *w, 300, 555, 990))), "split4")
    assert_zero(host(q4.int4_matvec_gated(x, *w, *w2)), "gated")
    assert_zero(host(q4.int4_matvec_norm(a, b, g, 1e-6, *w)[0]), "norm")
    y0, y1 = q4.int4_matvec_dual(x, *w, *w2)
    assert_zero(host(y0), "dual y0")
    assert_zero(host(y1), "dual y1")
    assert_zero(host(q4.int4_matvec_sigmoid_gated(a, b, *w)), "sigmoid-gated")
    assert_zero(host(q4.int4_matvec_swiglu_gated(a, b, *w)), "swiglu-gated")
    assert_zero(host(q4.int4_matvec_norm_swiglu(a, b, g, 1e-6, *w, *w2)[0]), "norm+swiglu")


@pytest.mark.parametrize("M", [2, 4, 8])
def test_lanes_and_gemm_give_zero(q4, M):
    K = 5120
    w = dev(*zero_triplet(0xC10 + M, N, K, 0.37))
    w2 = dev(*zero_triplet(0xC20 + M, N, K, 0.37))
    X, P = dev(synth.lanes(0xC30 + M, M, K), synth.lanes(0xC40 + M, M, K))
    assert_zero(host(q4.int4_matvec(X, *w)), f"lanes M={M}")
    assert_zero(host(q4.int4_matvec_gated_lanes(X, *w, *w2)), f"gated lanes M={M}")
    y0, y1 = q4.int4_matvec_dual(X, *w, *w2)
    assert_zero(host(y0), f"dual lanes M={M}")
    assert_zero(host(q4.int4_matvec_sigmoid_gated(X, P, *w)), f"sigmoid-gated lanes M={M}")
    T = 64 * M
    XT = dev(synth.lanes(0xC50 + M, T, K))[0]
    assert_zero(host(q4.int4_gemm(XT, *w)), f"gemm T={T}")


@pytest.mark.parametrize("D,F", [(1024, 2944), (4096, 14336)])
def test_fused_mlp_gives_zero(q4, D, F):
    # gate/up codes at their zero points: h = silu(0) * 0 = 0, then y = 0.
    # Down codes at their zero points with a non-zero h: y = 0.
    x = dev(synth.normal_f32(0xC60, D))[0]
    zg = dev(*zero_triplet(0xC61, F, D, 0.37))
    zu = dev(*zero_triplet(0xC62, F, D, 0.37))
    zd = dev(*zero_triplet(0xC63, D, F, 0.37))
    qg, sg, zg_ = oracle.quantize_pack(synth.weights(0xC64, F, D), GS)
    qu, su, zu_ = oracle.quantize_pack(synth.weights(0xC65, F, D), GS)
    rg = dev(qg.view(np.int32), sg, zg_)
    ru = dev(qu.view(np.int32), su, zu_)
    h, y = q4.int4_mlp(x, *zg, *zu, *zd)
    assert_zero(host(h), "mlp h")
    assert_zero(host(y), "mlp y")
    h, y = q4.int4_mlp(x, *rg, *ru, *zd)
    assert np.count_nonzero(host(h)) > F // 2
    assert_zero(host(y), "mlp y (non-zero h)")


def test_embedding_rows_give_zero(q4):
    import torch
    K = 4096
    w = dev(*zero_triplet(0xC70, N, K, 0.37))
    ids = torch.arange(0, N, 7, dtype=torch.int32, device="cuda")
    assert_zero(host(q4.int4_embedding_gather(ids, *w)), "embedding")


@pytest.mark.parametrize("K", [4096, 20480])
@pytest.mark.parametrize("scale", [0.37, 3.0])
def test_one_code_off_its_zero_point(q4, K, scale):
    q, s, z = zero_triplet(0xC80 + K, N, K, scale, off_by_one=True)
    x = synth.normal_f32(0xC81, K)
    y_ref, B = oracle.matvec(x, q.view(np.uint32), s, z, K, GS)
    qd, sd, zd = dev(q, s, z)
    xd = dev(x)[0]
    assert_dot_close(host(q4.int4_matvec(xd, qd, sd, zd)), y_ref, B, f"matvec K={K}")
    import torch
    outs = q4.int4_matvec_split4(xd, qd, sd, zd, 111, 600, 777)
    assert_dot_close(host(torch.cat(outs)), y_ref, B, f"split4 K={K}")
    y0, y1 = q4.int4_matvec_dual(xd, qd, sd, zd, qd, sd, zd)
    assert_dot_close(host(y0), y_ref, B, f"dual y0 K={K}")
    X = np.stack([x, -x, 2 * x, x])
    Y_ref, BB = oracle.matvec(X, q.view(np.uint32), s, z, K, GS)
    assert_dot_close(host(q4.int4_matvec(dev(X)[0], qd, sd, zd)), Y_ref, BB, f"lanes M=4 K={K}")
