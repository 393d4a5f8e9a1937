"""Captured HIP graphs replay the library's launches exactly: each entry point
(the matvec family, the M-lane matrix-core form, the prefill GEMM with its
split-K adds and the quantizer) is captured once, replayed several times with
eager work between the replays, and every replay is compared bitwise with the
eager call."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q4():
    import torch
    torch.cuda.set_device(0)
    import int4_group_quantized_quant_amd as m
    return m


def dev(*arrs):
    import torch
    return [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in arrs]


def check_graph(fn, outs, replays=4):
    """fn() enqueues the calls writing `outs`; compare each replay with the eager result."""
    import torch
    fn()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for i in range(replays):
        for o in outs:  # eager work between replays
            o.fill_(-1 if o.dtype == torch.int32 else float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o.view(torch.int32), r.view(torch.int32)), f"replay {i} differs"


def test_graph_matvec_family(q4):
    import torch
    N, K, gs = 700, 2048, 128
    W0, W1 = synth.weights(0x7000, N, K), synth.weights(0x7001, N, K)
    q0, s0, z0 = (t for t in dev(*oracle.quantize_pack(W0, gs)))
    q1, s1, z1 = (t for t in dev(*oracle.quantize_pack(W1, gs)))
    q0, q1 = q0.view(torch.int32), q1.view(torch.int32)
    x, a_b, wn = dev(synth.normal_f32(0x7002, K), synth.normal_f32(0x7003, K),
                     synth.uniform_f32(0x7004, K, 0.5, 1.5))
    X4 = dev(synth.lanes(0x7005, 4, K))[0]
    y = torch.empty(N, device="cuda")
    h = torch.empty(N, device="cuda")
    yn, r, nrm = torch.empty(N, device="cuda"), torch.empty(K, device="cuda"), torch.empty(K, device="cuda")
    Y4 = torch.empty((4, N), device="cuda")
    H4 = torch.empty((4, N), device="cuda")
    outs4 = [torch.empty(n, device="cuda") for n in (300, 200, 100, 100)]

    def fn():
        q4.int4_matvec(x, q0, s0, z0, Y=y)
        q4.int4_matvec_gated(x, q0, s0, z0, q1, s1, z1, h=h)
        q4.int4_matvec_norm(x, a_b, wn, 1e-6, q0, s0, z0, y=yn, residual_out=r, norm_out=nrm)
        q4.int4_matvec_split4(x, q0, s0, z0, 300, 500, 600, outs=outs4)
        q4.int4_matvec(X4, q0, s0, z0, Y=Y4)
        q4.int4_matvec_gated_lanes(X4, q0, s0, z0, q1, s1, z1, H=H4)
    check_graph(fn, [y, h, yn, r, nrm, Y4, H4, *outs4])


def test_graph_gemm_and_quantize(q4):
    import torch
    T, N, K, gs = 300, 256, 1024, 64
    W = torch.from_numpy(synth.weights(0x7100, N, K)).cuda()
    X = dev(synth.lanes(0x7101, T, K))[0]
    q, s, z = q4.int4_quantize_pack(W, gs)
    Y = torch.empty((T, N), device="cuda")
    ws = torch.empty(q4.int4_gemm_workspace_bytes(T, N, K, gs), dtype=torch.uint8, device="cuda")
    qq, ss, zz = torch.empty_like(q), torch.empty_like(s), torch.empty_like(z)

    def fn():
        q4.int4_quantize_pack(W, gs, q=qq, scales=ss, zeros=zz)
        q4.int4_gemm(X, q, s, z, Y=Y, workspace=ws)  # K split in two: adds into Y zeroed by the prep
    check_graph(fn, [qq, ss, zz, Y])
