"""GPU parity of the fused decode MLP block, int4_mlp: the gated gate/up
pass and the down projection of its output in one launch, with a grid-wide
wait between them.  h must equal int4_matvec_gated and y int4_matvec on the
GPU's h bit for bit (the fused passes keep the standalone calls' shapes);
h is within the gated bound of the oracle, y within the dot bound of the
oracle's down projection of the GPU's h.  The workspace counts the fused
calls and holds no timeout.
h and y are filled with NaN before each call, so a down pass that read any
part of h before it was written would show."""
import numpy as np
import pytest

import oracle
import synth
from helpers import assert_dot_close, gated_tolerance

pytestmark = pytest.mark.gpu

# (D, F, gs, fused).  The first three run as one launch on this device (both
# passes on the register kernel's one-block-per-CU grid, with 8/6/7/8-wave
# rows and ragged column splits); the next two are small enough that the
# passes' grids differ, and in the last two one pass has more than 16384
# inputs (the LDS kernel), so they run as two launches.
SHAPES = [(1024, 2944, 128, True), (2048, 5632, 64, True), (4096, 1024, 32, True), (256, 512, 32, False),
          (160, 96, 32, False), (20480, 256, 128, False), (1024, 16896, 128, False)]


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


def bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def quantized(seed, N, K, gs):
    return oracle.quantize_pack(synth.weights(seed, N, K), gs)


def weights_dev(w):
    q, s, z = w
    return to_dev(q.view(np.int32), s, z)


def mlp(q4, xd, wg, wu, wd, ws, D, F):
    import torch
    h = torch.full((F,), float("nan"), device=xd.device)
    y = torch.full((D,), float("nan"), device=xd.device)
    q4.int4_mlp(xd, *wg, *wu, *wd, h=h, y=y, workspace=ws)
    return h, y


def workspace(q4):
    import torch
    return torch.zeros(q4.int4_mlp_workspace_bytes() // 4, dtype=torch.int32, device="cuda")


def check_separate(q4, xd, wg, wu, wd, h, y):
    """h and y equal the standalone gated call and the matvec of that h."""
    h2 = q4.int4_matvec_gated(xd, *wg, *wu)
    np.testing.assert_array_equal(bits(host(h)), bits(host(h2)))
    y2 = q4.int4_matvec(h, *wd)
    np.testing.assert_array_equal(bits(host(y)), bits(host(y2)))


def check_workspace(ws, calls):
    """Word 0 counts the fused calls, word 1 (timeout) stays 0, and the
    flags of the blocks that ran hold the last call's count."""
    w = host(ws).view(np.uint32)
    assert w[0] == calls and w[1] == 0, w[:2]
    if calls:
        flags = w[32:]
        nb = int(np.count_nonzero(flags))
        assert nb > 0 and np.all(flags[:nb] == calls) and not flags[nb:].any()


@pytest.mark.parametrize("D,F,gs,fused", SHAPES)
def test_mlp_matches_oracle_and_separate_calls(q4, D, F, gs, fused):
    wg = quantized(0x7100 + F, F, D, gs)
    wu = quantized(0x7101 + F, F, D, gs)
    wd = quantized(0x7102 + D, D, F, gs)
    x = synth.normal_f32(0x7103, D)
    xd, = to_dev(x)
    wg_d, wu_d, wd_d = weights_dev(wg), weights_dev(wu), weights_dev(wd)
    ws = workspace(q4)
    h, y = mlp(q4, xd, wg_d, wu_d, wd_d, ws, D, F)
    print(f"int4_mlp D={D} F={F} gs={gs}", flush=True)
    ref = oracle.gated(x, *wg, *wu, D, gs)
    hh = host(h)
    assert np.all(np.abs(hh.astype(np.float64) - ref["h"]) <= gated_tolerance(ref)), "h"
    y_ref, B = oracle.matvec(hh, *wd, F, gs)
    assert_dot_close(host(y), y_ref, B, "y")
    check_separate(q4, xd, wg_d, wu_d, wd_d, h, y)
    check_workspace(ws, 1 if fused else 0)


def test_mlp_full_size(q4):
    """The SiLU-gated MLP at its workload size (gate/up 14336 x 4096, down
    4096 x 14336, gs 128), the launch the bench times; the down projection
    is checked over every column against the oracle on the GPU's h."""
    import torch
    c = synth.CONFIGS["c3"]
    inp = synth.c3_inputs()
    D, F, gs = c["K"], c["N"], c["gs"]
    wg_d = q4.int4_quantize_pack(torch.from_numpy(inp["Wg"]).cuda(), gs)
    wu_d = q4.int4_quantize_pack(torch.from_numpy(inp["Wu"]).cuda(), gs)
    wd_d = q4.int4_quantize_pack(torch.from_numpy(inp["Wd"]).cuda(), gs)
    xd, = to_dev(inp["x"])
    ws = workspace(q4)
    h, y = mlp(q4, xd, wg_d, wu_d, wd_d, ws, D, F)
    print("int4_mlp full size", flush=True)
    wg = [host(t) for t in wg_d]
    wu = [host(t) for t in wu_d]
    ref = oracle.gated(inp["x"], wg[0].view(np.uint32), wg[1], wg[2], wu[0].view(np.uint32), wu[1], wu[2],
                       D, gs)
    hh = host(h)
    assert np.all(np.abs(hh.astype(np.float64) - ref["h"]) <= gated_tolerance(ref)), "h"
    qd, sd, zd = (host(t) for t in wd_d)
    y_ref, B = oracle.matvec(hh, qd.view(np.uint32), sd, zd, F, gs)
    assert_dot_close(host(y), y_ref, B, "y")
    check_separate(q4, xd, wg_d, wu_d, wd_d, h, y)
    check_workspace(ws, 1)


def test_mlp_calls_in_a_row_and_graph_replays(q4):
    """One workspace across eager calls with new inputs, then across replays
    of a captured call with eager work between them: every result equals the
    separate calls on the same input, and the workspace counts every call."""
    import torch
    D, F, gs = 1024, 2944, 128
    wg_d = weights_dev(quantized(0x7120, F, D, gs))
    wu_d = weights_dev(quantized(0x7121, F, D, gs))
    wd_d = weights_dev(quantized(0x7122, D, F, gs))
    ws = workspace(q4)
    xd = torch.empty(D, device="cuda")
    for i in range(3):
        xd.copy_(torch.from_numpy(synth.normal_f32(0x7130 + i, D)))
        h, y = mlp(q4, xd, wg_d, wu_d, wd_d, ws, D, F)
        check_separate(q4, xd, wg_d, wu_d, wd_d, h, y)
    check_workspace(ws, 3)

    h = torch.empty(F, device="cuda")
    y = torch.empty(D, device="cuda")
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        q4.int4_mlp(xd, *wg_d, *wu_d, *wd_d, h=h, y=y, workspace=ws)  # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        q4.int4_mlp(xd, *wg_d, *wu_d, *wd_d, h=h, y=y, workspace=ws)
    for i in range(3):
        xd.copy_(torch.from_numpy(synth.normal_f32(0x7140 + i, D)))
        h.fill_(float("nan"))
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check_separate(q4, xd, wg_d, wu_d, wd_d, h, y)
    check_workspace(ws, 3 + 1 + 3)  # eager calls, the warm-up, the replays (capture runs nothing)


def test_mlp_timeout_flag_is_reported_and_sticky(q4):
    """The timeout flag, set here from the host (no wait is made to time
    out): the call writes NaN to all of h and y and leaves the call count,
    int4_mlp_timed_out reports the flag, and a zeroed workspace works again."""
    import torch
    D, F, gs = 1024, 2944, 128
    wg_d = weights_dev(quantized(0x7170, F, D, gs))
    wu_d = weights_dev(quantized(0x7171, F, D, gs))
    wd_d = weights_dev(quantized(0x7172, D, F, gs))
    xd, = to_dev(synth.normal_f32(0x7173, D))
    ws = workspace(q4)
    h, y = mlp(q4, xd, wg_d, wu_d, wd_d, ws, D, F)
    check_separate(q4, xd, wg_d, wu_d, wd_d, h, y)
    assert not q4.int4_mlp_timed_out(ws)
    ws[1] = 1
    h = torch.zeros(F, device="cuda")
    y = torch.zeros(D, device="cuda")
    q4.int4_mlp(xd, *wg_d, *wu_d, *wd_d, h=h, y=y, workspace=ws)
    assert np.isnan(host(h)).all() and np.isnan(host(y)).all()
    assert q4.int4_mlp_timed_out(ws)
    assert host(ws).view(np.uint32)[0] == 1
    ws.zero_()
    h, y = mlp(q4, xd, wg_d, wu_d, wd_d, ws, D, F)
    check_separate(q4, xd, wg_d, wu_d, wd_d, h, y)
    assert not q4.int4_mlp_timed_out(ws)
    check_workspace(ws, 1)


def test_mlp_default_workspace_and_shape_errors(q4):
    import torch
    D, F, gs = 256, 512, 32
    wg_d = weights_dev(quantized(0x7150, F, D, gs))
    wu_d = weights_dev(quantized(0x7151, F, D, gs))
    wd_d = weights_dev(quantized(0x7152, D, F, gs))
    xd, = to_dev(synth.normal_f32(0x7153, D))
    h, y = q4.int4_mlp(xd, *wg_d, *wu_d, *wd_d)  # a zeroed workspace is made for the call
    check_separate(q4, xd, wg_d, wu_d, wd_d, h, y)
    with pytest.raises(ValueError):
        q4.int4_mlp(xd, *wg_d, *wu_d, *wg_d)  # down weights of the wrong shape
    small = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(q4.Int4Error):
        q4.int4_mlp(xd, *wg_d, *wu_d, *wd_d, workspace=small)


def test_binding_rejects_short_buffers(q4):
    """The C ABI takes bare pointers, so the binding checks every element
    count: a short output or input raises before any launch."""
    import torch
    N, K, gs = 64, 256, 32
    w = weights_dev(quantized(0x7160, N, K, gs))
    w2 = weights_dev(quantized(0x7161, N, K, gs))
    x = torch.zeros(K, device="cuda")
    short = torch.zeros(N - 1, device="cuda")
    shortK = torch.zeros(K - 4, device="cuda")
    X2 = torch.zeros((2, K), device="cuda")
    cases = [
        lambda: q4.int4_matvec(x, *w, Y=short),
        lambda: q4.int4_matvec(X2, *w, Y=torch.zeros(N, device="cuda")),
        lambda: q4.int4_matvec_split4(shortK, *w, 16, 32, 48),
        lambda: q4.int4_matvec_split4(x, *w, 16, 32, 48,
                                      outs=[torch.zeros(n, device="cuda") for n in (16, 16, 16, 15)]),
        lambda: q4.int4_matvec_gated(x, *w, *w2, h=short),
        lambda: q4.int4_matvec_gated(shortK, *w, *w2),
        lambda: q4.int4_matvec_norm(x, x, shortK, 1e-6, *w),
        lambda: q4.int4_matvec_norm(x, x, x, 1e-6, *w, y=short),
        lambda: q4.int4_matvec_norm(x, x, x, 1e-6, *w, residual_out=shortK),
        lambda: q4.int4_matvec_dual(x, *w, *w2, y1=short),
        lambda: q4.int4_matvec_sigmoid_gated(x, x, *w, y=short),
        lambda: q4.int4_matvec_swiglu_gated(x, x, *w, y=short),
        lambda: q4.int4_matvec_norm_swiglu(x, x, x, 1e-6, *w, *w2, h=short),
        lambda: q4.int4_matvec_gated_lanes(X2, *w, *w2, H=torch.zeros(N, device="cuda")),
        lambda: q4.int4_gemm(X2, *w, Y=torch.zeros((2, N - 1), device="cuda")),
        lambda: q4.int4_quantize_pack(torch.zeros((N, K), device="cuda"), gs,
                                      q=torch.zeros((N, K // 8 - 1), dtype=torch.int32, device="cuda")),
    ]
    for i, case in enumerate(cases):
        with pytest.raises(ValueError):
            case()
        print(f"case {i} rejected", flush=True)
    D, F = 256, 512
    wm = [weights_dev(quantized(0x7162 + i, *shp, gs)) for i, shp in enumerate(((F, D), (F, D), (D, F)))]
    with pytest.raises(ValueError):
        q4.int4_mlp(torch.zeros(D, device="cuda"), *wm[0], *wm[1], *wm[2], y=torch.zeros(D - 1, device="cuda"))
    with pytest.raises(ValueError):
        q4.int4_mlp(torch.zeros(D, device="cuda"), *wm[0], *wm[1], *wm[2], h=torch.zeros(F - 1, device="cuda"))
    torch.cuda.synchronize()
