"""GPU parity of the fused decode variants next to the hot path: the dual
matvec, the sigmoid- and SwiGLU-gated input matvecs and the norm + SwiGLU
MLP front.  Small shapes span several column tiles, ragged tails and both
kernel families (K <= 16384 on the register kernel, longer K on the LDS
kernel); the full workload sizes are checked on sampled columns."""
import numpy as np
import pytest

import oracle
import synth
from helpers import assert_dot_close, gated_tolerance, integer_problem

pytestmark = pytest.mark.gpu

SHAPES = [(129, 1024, 128), (1000, 4096, 128), (33, 2080, 32), (19, 16416, 32), (13, 20480, 64)]


@pytest.fixture(scope="module")
def q4():
    import torch
    torch.cuda.set_device(0)
    import int4_group_quantized_quant_amd as m
    return m


def to_dev(*arrs):
    import torch
    return [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in arrs]


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def quantized(seed, N, K, gs):
    return oracle.quantize_pack(synth.weights(seed, N, K), gs)


def bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def close_ulps(got, want, ulps=8):
    """|got - want| within a few binary32 ulps of want (want fp64)."""
    got = np.asarray(got, np.float64)
    return np.all(np.abs(got - want) <= ulps * np.spacing(np.abs(want).astype(np.float32)) + 1e-37)


# ------------------------------------------------------------------ dual

@pytest.mark.parametrize("N,K,gs", SHAPES)
def test_dual(q4, N, K, gs):
    q0, s0, z0 = quantized(0xF000 + N, N, K, gs)
    q1, s1, z1 = quantized(0xF001 + N, N, K, gs)
    x = synth.normal_f32(0xF002, K)
    ref = oracle.dual(x, q0, s0, z0, q1, s1, z1, K, gs)
    xd, *w = to_dev(x, q0.view(np.int32), s0, z0, q1.view(np.int32), s1, z1)
    y0, y1 = q4.int4_matvec_dual(xd, *w)
    assert_dot_close(host(y0), ref["y0"], ref["b0"], "dual y0")
    assert_dot_close(host(y1), ref["y1"], ref["b1"], "dual y1")
    # Each output is the single-lane matvec of its own matrix, bit for bit.
    np.testing.assert_array_equal(bits(host(y0)), bits(host(q4.int4_matvec(xd, *w[:3]))))
    np.testing.assert_array_equal(bits(host(y1)), bits(host(q4.int4_matvec(xd, *w[3:]))))


def test_dual_integer_exact(q4):
    rng = np.random.default_rng(0xF010)
    N, K, gs = 300, 1024, 64
    q0, s0, z0, X, e0 = integer_problem(rng, N, K, gs)
    q1, s1, z1, _, _ = integer_problem(rng, N, K, gs)
    ref = oracle.dual(X[0], q0, s0, z0, q1, s1, z1, K, gs)
    xd, *w = to_dev(X[0], q0.view(np.int32), s0, z0, q1.view(np.int32), s1, z1)
    y0, y1 = q4.int4_matvec_dual(xd, *w)
    np.testing.assert_array_equal(host(y0), e0[0].astype(np.float32))
    np.testing.assert_array_equal(host(y1), ref["y1"].astype(np.float32))


def test_dual_rejects_mismatched_and_aliased(q4):
    N, K, gs = 20, 512, 64
    q0, s0, z0 = quantized(0xF020, N, K, gs)
    x = synth.normal_f32(0xF021, K)
    xd, qd, sd, zd = to_dev(x, q0.view(np.int32), s0, z0)
    q2, s2, z2 = to_dev(*[a[:10] for a in (q0.view(np.int32), s0, z0)])
    with pytest.raises(ValueError):
        q4.int4_matvec_dual(xd, qd, sd, zd, q2, s2, z2)
    y = host(q4.int4_matvec(xd, qd, sd, zd))
    with pytest.raises(q4.Int4Error):
        q4.int4_matvec_dual(xd, qd, sd, zd, qd, sd, zd, y0=xd[:N], y1=None)
    assert y.shape == (N,)


# ------------------------------------------------------------------ input-gated

@pytest.mark.parametrize("N,K,gs", SHAPES)
def test_sigmoid_gated(q4, N, K, gs):
    q, s, z = quantized(0xF100 + N, N, K, gs)
    a = synth.normal_f32(0xF101, K)
    g = (3.0 * synth.normal_f32(0xF102, K)).astype(np.float32)
    ref = oracle.sigmoid_gated(a, g, q, s, z, K, gs)
    ad, gd, *w = to_dev(a, g, q.view(np.int32), s, z)
    y = q4.int4_matvec_sigmoid_gated(ad, gd, *w)
    assert_dot_close(host(y), ref["y"], ref["B"], "sigmoid-gated")


@pytest.mark.parametrize("N,K,gs", SHAPES)
def test_swiglu_gated(q4, N, K, gs):
    q, s, z = quantized(0xF200 + N, N, K, gs)
    g = (2.0 * synth.normal_f32(0xF201, K)).astype(np.float32)
    u = synth.normal_f32(0xF202, K)
    ref = oracle.swiglu_gated(g, u, q, s, z, K, gs)
    gd, ud, *w = to_dev(g, u, q.view(np.int32), s, z)
    y = q4.int4_matvec_swiglu_gated(gd, ud, *w)
    assert_dot_close(host(y), ref["y"], ref["B"], "swiglu-gated")


def test_input_gates_special_values_exact(q4):
    # sigmoid(0) = 1/2 and silu(t) = t for large t are exact in binary32 too,
    # so integer problems come out exact; very negative gates give zeros.
    rng = np.random.default_rng(0xF300)
    N, K, gs = 150, 2048, 64
    q, s, z, X, exact = integer_problem(rng, N, K, gs)
    w = to_dev(q.view(np.int32), s, z)
    a2 = (2 * X[0]).astype(np.float32)
    zeros_k = np.zeros(K, np.float32)
    ad, zd, xd = to_dev(a2, zeros_k, X[0])
    np.testing.assert_array_equal(host(q4.int4_matvec_sigmoid_gated(ad, zd, *w)),
                                  exact[0].astype(np.float32))
    # e^-32 is below half an ulp of 1, so sigmoid(32) = 1 and silu(32) = 32;
    # |32 * x| <= 256 keeps every partial sum an integer below 2^24.
    big, neg = to_dev(np.full(K, 32.0, np.float32), np.full(K, -200.0, np.float32))
    np.testing.assert_array_equal(host(q4.int4_matvec_sigmoid_gated(ad, big, *w)),
                                  (2 * exact[0]).astype(np.float32))
    np.testing.assert_array_equal(host(q4.int4_matvec_sigmoid_gated(ad, neg, *w)), np.zeros(N, np.float32))
    np.testing.assert_array_equal(host(q4.int4_matvec_swiglu_gated(big, xd, *w)),
                                  (32 * exact[0]).astype(np.float32))
    np.testing.assert_array_equal(host(q4.int4_matvec_swiglu_gated(zd, xd, *w)), np.zeros(N, np.float32))
    np.testing.assert_array_equal(host(q4.int4_matvec_swiglu_gated(neg, xd, *w)), np.zeros(N, np.float32))


# ------------------------------------------------------------------ norm + SwiGLU

def norm_inputs(seed, K):
    return (synth.normal_f32(seed, K), synth.normal_f32(seed + 1, K),
            synth.uniform_f32(seed + 2, K, 0.5, 1.5))


@pytest.mark.parametrize("N,K,gs", SHAPES)
def test_norm_swiglu(q4, N, K, gs):
    qg, sg, zg = quantized(0xF400 + N, N, K, gs)
    qu, su, zu = quantized(0xF401 + N, N, K, gs)
    a_a, a_b, wn = norm_inputs(0xF402, K)
    ref = oracle.norm_swiglu(a_a, a_b, wn, 1e-6, qg, sg, zg, qu, su, zu, K, gs)
    dev = to_dev(a_a, a_b, wn, qg.view(np.int32), sg, zg, qu.view(np.int32), su, zu)
    h, r = q4.int4_matvec_norm_swiglu(*dev[:3], 1e-6, *dev[3:])
    hh = host(h).astype(np.float64)
    tol = gated_tolerance(ref)
    assert np.all(np.abs(hh - ref["h"]) <= tol), f"max err/tol {np.max(np.abs(hh - ref['h']) / tol)}"
    np.testing.assert_array_equal(bits(host(r)), bits(ref["residual"]))
    # g and u are int4_matvec_norm's outputs bit for bit: only silu(g) * u rounds.
    g, _, _ = q4.int4_matvec_norm(*dev[:3], 1e-6, *dev[3:6], want_residual=False, want_norm=False)
    u, _, _ = q4.int4_matvec_norm(*dev[:3], 1e-6, *dev[6:], want_residual=False, want_norm=False)
    g = host(g).astype(np.float64)
    u = host(u).astype(np.float64)
    assert close_ulps(hh, g / (1.0 + np.exp(-g)) * u)


def test_norm_swiglu_optional_residual_and_empty(q4):
    import torch
    N, K, gs = 40, 1024, 64
    qg, sg, zg = quantized(0xF500, N, K, gs)
    qu, su, zu = quantized(0xF501, N, K, gs)
    a_a, a_b, wn = norm_inputs(0xF502, K)
    ref = oracle.norm_swiglu(a_a, a_b, wn, 1e-5, qg, sg, zg, qu, su, zu, K, gs)
    dev = to_dev(a_a, a_b, wn, qg.view(np.int32), sg, zg, qu.view(np.int32), su, zu)
    h, r = q4.int4_matvec_norm_swiglu(*dev[:3], 1e-5, *dev[3:], want_residual=False)
    assert r is None
    assert np.all(np.abs(host(h) - ref["h"]) <= gated_tolerance(ref))
    qe = torch.empty((0, K // 8), dtype=torch.int32, device="cuda")
    se = torch.empty((0, K // gs), dtype=torch.float32, device="cuda")
    h0, r0 = q4.int4_matvec_norm_swiglu(*dev[:3], 1e-5, qe, se, se, qe, se, se)
    assert h0.shape == (0,)
    np.testing.assert_array_equal(host(r0), ref["residual"])


# ------------------------------------------------------------------ embedding gather

@pytest.mark.parametrize("N,K,gs,T", [(1000, 1024, 128, 37), (77, 4096, 64, 300), (5, 2080, 32, 9)])
def test_embedding_gather(q4, N, K, gs, T):
    q, s, z = quantized(0xF600 + N, N, K, gs)
    rng = np.random.default_rng(N)
    ids = rng.integers(0, N, T).astype(np.int32)
    ids[:4] = [0, N - 1, -1, N]          # both ends and two ids out of range
    ids[-1] = 2**31 - 1
    if T > 6:
        ids[5] = ids[4]                  # a repeated token
    ref = oracle.embedding(ids, q, s, z, K, gs)
    idd, qd, sd, zd = to_dev(ids, q.view(np.int32), s, z)
    out = host(q4.int4_embedding_gather(idd, qd, sd, zd))
    np.testing.assert_array_equal(bits(out), bits(ref))


def test_embedding_gather_empty_cases(q4):
    import torch
    K, gs = 512, 64
    q, s, z = quantized(0xF700, 8, K, gs)
    qd, sd, zd = to_dev(q.view(np.int32), s, z)
    ids0 = torch.empty(0, dtype=torch.int32, device="cuda")
    assert q4.int4_embedding_gather(ids0, qd, sd, zd).shape == (0, K)
    # An empty table: every id is out of range, every row is zeros.
    qe = torch.empty((0, K // 8), dtype=torch.int32, device="cuda")
    se = torch.empty((0, K // gs), dtype=torch.float32, device="cuda")
    ids = torch.tensor([0, 3, -2], dtype=torch.int32, device="cuda")
    out = torch.full((3, K), 7.0, device="cuda")
    q4.int4_embedding_gather(ids, qe, se, se, out=out)
    np.testing.assert_array_equal(host(out), np.zeros((3, K), np.float32))


# ------------------------------------------------------------------ full workload sizes

def gpu_quantized(q4, W, gs):
    """GPU and oracle codes of all of W, compared bit for bit over every row."""
    import torch
    qd, sd, zd = q4.int4_quantize_pack(torch.from_numpy(W).cuda(), gs)
    ref = oracle.quantize_pack(W, gs)
    for got, want in zip((qd, sd, zd), ref):
        np.testing.assert_array_equal(bits(host(got)), bits(want))
    return (qd, sd, zd), ref


def test_n1_dual_full(q4):
    import torch
    c = synth.NEXT["n1"]
    inp = synth.n1_inputs()
    (w0, r0) = gpu_quantized(q4, inp["W0"], c["gs"])
    (w1, r1) = gpu_quantized(q4, inp["W1"], c["gs"])
    y0, y1 = q4.int4_matvec_dual(torch.from_numpy(inp["x"]).cuda(), *w0, *w1)
    ref = oracle.dual(inp["x"], *r0, *r1, c["K"], c["gs"])
    assert_dot_close(host(y0), ref["y0"], ref["b0"], "n1 y0")
    assert_dot_close(host(y1), ref["y1"], ref["b1"], "n1 y1")


def test_n2_sigmoid_gated_full(q4):
    import torch
    c = synth.NEXT["n2"]
    inp = synth.n2_inputs()
    w, r = gpu_quantized(q4, inp["W"], c["gs"])
    y = q4.int4_matvec_sigmoid_gated(*to_dev(inp["a"], inp["gate"]), *w)
    ref = oracle.sigmoid_gated(inp["a"], inp["gate"], *r, c["K"], c["gs"])
    assert_dot_close(host(y), ref["y"], ref["B"], "n2")


def test_n3_swiglu_gated_full(q4):
    c = synth.NEXT["n3"]
    inp = synth.n3_inputs()
    w, r = gpu_quantized(q4, inp["W"], c["gs"])
    y = q4.int4_matvec_swiglu_gated(*to_dev(inp["gate"], inp["up"]), *w)
    ref = oracle.swiglu_gated(inp["gate"], inp["up"], *r, c["K"], c["gs"])
    assert_dot_close(host(y), ref["y"], ref["B"], "n3")


def test_n4_norm_swiglu_full(q4):
    c = synth.NEXT["n4"]
    inp = synth.n4_inputs()
    wg, rg = gpu_quantized(q4, inp["Wg"], c["gs"])
    wu, ru = gpu_quantized(q4, inp["Wu"], c["gs"])
    dev = to_dev(inp["a_a"], inp["a_b"], inp["w_norm"])
    h, r = q4.int4_matvec_norm_swiglu(*dev, inp["eps"], *wg, *wu)
    ref = oracle.norm_swiglu(inp["a_a"], inp["a_b"], inp["w_norm"], inp["eps"], *rg, *ru,
                             c["K"], c["gs"])
    hh = host(h).astype(np.float64)
    assert np.all(np.abs(hh - ref["h"]) <= gated_tolerance(ref)), "n4"
    np.testing.assert_array_equal(host(r), ref["residual"])


def test_n5_embedding_gather_full(q4):
    import torch
    c = synth.NEXT["n5"]
    inp = synth.n5_inputs()
    w, r = gpu_quantized(q4, inp["W"], c["gs"])
    del inp["W"]
    # The workload's id stream over the whole table, every row compared.
    T = max(c["Ts"])
    ids = inp["ids"].astype(np.int32)
    assert ids.shape == (T,)
    out = host(q4.int4_embedding_gather(torch.from_numpy(ids).cuda(), *w))
    ref = oracle.embedding(ids, *r, c["K"], c["gs"])
    assert out.shape == (T, c["K"])
    np.testing.assert_array_equal(bits(out), bits(ref))


# ------------------------------------------------------------------ M decode lanes (batch ports)

LANE_SHAPES = [(129, 1024, 128), (300, 5120, 64), (77, 2080, 32), (45, 2304, 96)]


@pytest.mark.parametrize("M", [2, 3, 8])
@pytest.mark.parametrize("N,K,gs", LANE_SHAPES)
def test_dual_lanes(q4, M, N, K, gs):
    q0, s0, z0 = quantized(0xF800 + N, N, K, gs)
    q1, s1, z1 = quantized(0xF801 + N, N, K, gs)
    X = synth.lanes(0xF802 + M, M, K)
    Xd, *w = to_dev(X, q0.view(np.int32), s0, z0, q1.view(np.int32), s1, z1)
    y0, y1 = q4.int4_matvec_dual(Xd, *w)
    y0, y1 = host(y0), host(y1)
    assert y0.shape == (M, N) and y1.shape == (M, N)
    for m in range(M):
        ref = oracle.dual(X[m], q0, s0, z0, q1, s1, z1, K, gs)
        assert_dot_close(y0[m], ref["y0"], ref["b0"], f"dual lanes y0 m={m}")
        assert_dot_close(y1[m], ref["y1"], ref["b1"], f"dual lanes y1 m={m}")
    # Each output is int4_matvec at the same M for its own matrix, bit for bit.
    np.testing.assert_array_equal(bits(y0), bits(host(q4.int4_matvec(Xd, *w[:3]))))
    np.testing.assert_array_equal(bits(y1), bits(host(q4.int4_matvec(Xd, *w[3:]))))


@pytest.mark.parametrize("M", [2, 5, 8])
@pytest.mark.parametrize("N,K,gs", LANE_SHAPES)
def test_input_gated_lanes(q4, M, N, K, gs):
    q, s, z = quantized(0xF900 + N, N, K, gs)
    P = synth.lanes(0xF901 + M, M, K)
    R = (2.0 * synth.lanes(0xF902 + M, M, K)).astype(np.float32)
    Pd, Rd, *w = to_dev(P, R, q.view(np.int32), s, z)
    ys = host(q4.int4_matvec_sigmoid_gated(Pd, Rd, *w))
    yw = host(q4.int4_matvec_swiglu_gated(Pd, Rd, *w))
    assert ys.shape == (M, N) and yw.shape == (M, N)
    for m in range(M):
        rs = oracle.sigmoid_gated(P[m], R[m], q, s, z, K, gs)
        rw = oracle.swiglu_gated(P[m], R[m], q, s, z, K, gs)
        assert_dot_close(ys[m], rs["y"], rs["B"], f"sigmoid-gated lanes m={m}")
        assert_dot_close(yw[m], rw["y"], rw["B"], f"swiglu-gated lanes m={m}")
    # Lanes never interact: the first lane alone (M = 2 with a zero second
    # lane) gives the same bits as lane 0 of the full call.
    P2 = np.stack([P[0], np.zeros(K, np.float32)])
    R2 = np.stack([R[0], np.zeros(K, np.float32)])
    y2 = host(q4.int4_matvec_sigmoid_gated(*to_dev(P2, R2), *w))
    np.testing.assert_array_equal(bits(y2[0]), bits(ys[0]))


def test_lanes_variants_reject_nine_lanes(q4):
    N, K, gs = 20, 512, 64
    q, s, z = quantized(0xFA00, N, K, gs)
    X = synth.lanes(0xFA01, 9, K)
    Xd, *w = to_dev(X, q.view(np.int32), s, z)
    with pytest.raises(q4.Int4Error):
        q4.int4_matvec_dual(Xd, *w, *w)
    with pytest.raises(q4.Int4Error):
        q4.int4_matvec_swiglu_gated(Xd, Xd, *w)


@pytest.mark.parametrize("M", [1, 2, 3, 8])
@pytest.mark.parametrize("N,K,gs", LANE_SHAPES)
def test_gated_lanes(q4, M, N, K, gs):
    qg, sg, zg = quantized(0xFB00 + N, N, K, gs)
    qu, su, zu = quantized(0xFB01 + N, N, K, gs)
    X = synth.lanes(0xFB02 + M, M, K)
    Xd, *w = to_dev(X, qg.view(np.int32), sg, zg, qu.view(np.int32), su, zu)
    H = host(q4.int4_matvec_gated_lanes(Xd, *w))
    assert H.shape == (M, N)
    for m in range(M):
        ref = oracle.gated(X[m], qg, sg, zg, qu, su, zu, K, gs)
        tol = gated_tolerance(ref)
        err = np.abs(H[m].astype(np.float64) - ref["h"])
        assert np.all(err <= tol), f"gated lanes m={m}: max err/tol {np.max(err / tol)}"
    # g and u are int4_matvec's sums at the same M, bit for bit: only
    # silu(g) * u rounds.
    g = host(q4.int4_matvec(Xd, *w[:3])).astype(np.float64)
    u = host(q4.int4_matvec(Xd, *w[3:])).astype(np.float64)
    assert close_ulps(H, g / (1.0 + np.exp(-g)) * u)
    if M == 1:
        np.testing.assert_array_equal(bits(H[0]), bits(host(q4.int4_matvec_gated(Xd[0], *w))))


def test_gated_lanes_table_limit(q4):
    # Both streams' scale / zero tables share the LDS: 512 groups per column
    # fit the plain lanes call but not the gated one.
    N, K, gs = 40, 16384, 32
    rng = np.random.default_rng(0xFB10)
    q = rng.integers(0, 2**32, (N, K // 8), dtype=np.uint64).astype(np.uint32)
    s = np.full((N, K // gs), 1e-3, np.float32)
    z = rng.integers(0, 16, (N, K // gs)).astype(np.float32)
    X = synth.lanes(0xFB11, 2, K)
    Xd, qd, sd, zd = to_dev(X, q.view(np.int32), s, z)
    Y = host(q4.int4_matvec(Xd, qd, sd, zd))
    Y_ref, B = oracle.matvec(X, q, s, z, K, gs)
    assert_dot_close(Y, Y_ref, B, "plain lanes at 512 groups")
    with pytest.raises(q4.Int4Error):
        q4.int4_matvec_gated_lanes(Xd, qd, sd, zd, qd, sd, zd)


def test_lanes_variants_more_blocks_than_resident(q4):
    """Dual and gated lanes whose columns need more tiles than one block per
    CU holds in its LDS tables (9000 columns, 256 groups of 32 per column):
    the grid then has more blocks than the device runs at once.  Every
    output is checked against the oracle, and each stream's sums against
    int4_matvec at the same M."""
    N, K, gs, M = 9000, 8192, 32, 3
    q0, s0, z0 = quantized(0xFC00, N, K, gs)
    q1, s1, z1 = quantized(0xFC01, N, K, gs)
    X = synth.lanes(0xFC02, M, K)
    Xd, *w = to_dev(X, q0.view(np.int32), s0, z0, q1.view(np.int32), s1, z1)
    y0, y1 = q4.int4_matvec_dual(Xd, *w)
    y0, y1 = host(y0), host(y1)
    H = host(q4.int4_matvec_gated_lanes(Xd, *w))
    for m in range(M):
        ref = oracle.dual(X[m], q0, s0, z0, q1, s1, z1, K, gs)
        assert_dot_close(y0[m], ref["y0"], ref["b0"], f"dual lanes y0 m={m}")
        assert_dot_close(y1[m], ref["y1"], ref["b1"], f"dual lanes y1 m={m}")
        rg = oracle.gated(X[m], q0, s0, z0, q1, s1, z1, K, gs)
        err = np.abs(H[m].astype(np.float64) - rg["h"])
        assert np.all(err <= gated_tolerance(rg)), f"gated lanes m={m}"
    g = host(q4.int4_matvec(Xd, *w[:3]))
    u = host(q4.int4_matvec(Xd, *w[3:]))
    np.testing.assert_array_equal(bits(y0), bits(g))
    np.testing.assert_array_equal(bits(y1), bits(u))
    g = g.astype(np.float64)
    u = u.astype(np.float64)
    assert close_ulps(H, g / (1.0 + np.exp(-g)) * u)
