"""Concurrent calls on different streams: the library keeps no state between
calls (int4_mlp's only state is the caller's workspace), so calls running at
the same time on four streams give the bits each gives alone.  The fused
MLP's grid-wide wait shares the device with the other kernels here; its
timeout word must stay 0."""
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
    return [torch.from_numpy(np.ascontiguousarray(a.view(np.int32) if a.dtype == np.uint32 else a)).cuda()
            for a in arrs]


def test_four_streams_match_serial(q4):
    import torch
    # Norm matvec (register kernel), four lanes (matrix cores), prefill GEMM,
    # and the fused MLP block, each on its own weights.
    wn = dev(*oracle.quantize_pack(synth.weights(0xD001, 20000, 4096), 128))
    an = dev(synth.normal_f32(0xD002, 4096), synth.normal_f32(0xD003, 4096),
             synth.uniform_f32(0xD004, 4096, 0.5, 1.5))
    wl = dev(*oracle.quantize_pack(synth.weights(0xD005, 8000, 5120), 64))
    Xl, = dev(synth.lanes(0xD006, 4, 5120))
    wg = dev(*oracle.quantize_pack(synth.weights(0xD007, 1024, 2048), 128))
    Xg, = dev(synth.lanes(0xD008, 256, 2048))
    D, F = 1024, 2944
    wm = [dev(*oracle.quantize_pack(synth.weights(0xD009 + i, *shp), 128))
          for i, shp in enumerate(((F, D), (F, D), (D, F)))]
    xm, = dev(synth.normal_f32(0xD00C, D))
    ws = torch.zeros(q4.int4_mlp_workspace_bytes() // 4, dtype=torch.int32, device="cuda")
    gws = torch.empty(q4.int4_gemm_workspace_bytes(256, 1024, 2048, 128), dtype=torch.uint8, device="cuda")

    def norm_call(out):
        q4.int4_matvec_norm(*an, 1e-6, *wn, y=out)

    def lanes_call(out):
        q4.int4_matvec(Xl, *wl, Y=out)

    def gemm_call(out):
        q4.int4_gemm(Xg, *wg, Y=out, workspace=gws)

    def mlp_call(out):
        q4.int4_mlp(xm, *wm[0], *wm[1], *wm[2], h=out[0], y=out[1], workspace=ws)

    calls = [
        (norm_call, lambda: torch.empty(20000, device="cuda")),
        (lanes_call, lambda: torch.empty((4, 8000), device="cuda")),
        (gemm_call, lambda: torch.empty((256, 1024), device="cuda")),
        (mlp_call, lambda: (torch.empty(F, device="cuda"), torch.empty(D, device="cuda"))),
    ]
    # Serial references on the default stream.
    refs = []
    for fn, make in calls:
        out = make()
        fn(out)
        refs.append(out)
    torch.cuda.synchronize()
    print("serial references done", flush=True)

    reps = 5
    streams = [torch.cuda.Stream() for _ in calls]
    outs = [[make() for _ in range(reps)] for _, make in calls]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for r in range(reps):
        for (fn, _), s, o in zip(calls, streams, outs):
            with torch.cuda.stream(s):
                fn(o[r])
    torch.cuda.synchronize()
    print("concurrent calls done", flush=True)

    def bits(t):
        return t.cpu().numpy().view(np.uint32)

    for i, (ref, o) in enumerate(zip(refs, outs)):
        for r in range(reps):
            if isinstance(ref, tuple):
                for a, b in zip(ref, o[r]):
                    np.testing.assert_array_equal(bits(b), bits(a), err_msg=f"call {i} rep {r}")
            else:
                np.testing.assert_array_equal(bits(o[r]), bits(ref), err_msg=f"call {i} rep {r}")
    assert ws.cpu().numpy()[1] == 0, "the fused MLP's grid-wide wait timed out"
