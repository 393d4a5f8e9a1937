"""GPU test of int4_gemm_noalloc, the prefill GEMM that takes its workspace
from the library's own scratch array: called through the C ABI, it must
give int4_gemm's bits on two calls in a row (the second smaller, so it
reads a scratch array that still holds the first call's contents), stay
within the dot bound of the oracle, and refuse a problem whose workspace
exceeds the array before launching anything."""
import numpy as np
import pytest

import oracle
import synth
from helpers import assert_dot_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q4():
    import torch
    torch.cuda.set_device(0)
    import int4_group_quantized_quant_amd as m
    return m


def problem(seed, T, N, K, gs):
    W = synth.weights(seed, N, K)
    q, s, z = oracle.quantize_pack(W, gs)
    X = synth.lanes(seed + 1, T, K)
    return X, q, s, z


def run_both(q4, X, q, s, z):
    import torch
    Xd, qd, sd, zd = (torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (X, q.view(np.int32), s, z))
    T, N = X.shape[0], q.shape[0]
    # Outputs filled with NaN, so an output the call did not write shows.
    Y_ws = torch.full((T, N), float("nan"), dtype=torch.float32, device="cuda")
    Y_na = torch.full((T, N), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(q4.int4_gemm_workspace_bytes(T, N, X.shape[1], X.shape[1] // s.shape[1]), 1),
                     dtype=torch.uint8, device="cuda")
    q4.int4_gemm(Xd, qd, sd, zd, Y=Y_ws, workspace=ws)
    q4.int4_gemm_noalloc(Xd, qd, sd, zd, Y=Y_na)
    torch.cuda.synchronize()
    return Y_ws.cpu().numpy(), Y_na.cpu().numpy()


def test_two_calls_in_a_row_match_int4_gemm(q4):
    # First a larger problem (128 x 256 tiles, one K part), then a smaller
    # one (128 x 128 tiles, K split in two, other group size).
    for seed, T, N, K, gs in ((0xD01, 1024, 1000, 4096, 128), (0xD02, 64, 300, 1024, 64)):
        X, q, s, z = problem(seed, T, N, K, gs)
        Y_ws, Y_na = run_both(q4, X, q, s, z)
        assert np.all(np.isfinite(Y_na)), f"T={T}: unwritten outputs"
        np.testing.assert_array_equal(Y_na.view(np.uint32), Y_ws.view(np.uint32),
                                      err_msg=f"T={T} N={N} K={K}: bits differ from int4_gemm")
        rows = slice(0, T) if T <= 64 else slice(0, T, 97)
        y_ref, B = oracle.matvec(X[rows], q, s, z, K, gs)
        assert_dot_close(Y_na[rows], y_ref, B, f"T={T} N={N} K={K}")


def test_refuses_a_workspace_beyond_the_array(q4):
    import torch
    T, N, K, gs = 8192, 256, 4096, 128
    assert q4.int4_gemm_workspace_bytes(T, N, K, gs) > q4.INT4_GEMM_NOALLOC_SCRATCH_BYTES
    X = torch.zeros((T, K), dtype=torch.float32, device="cuda")
    q = torch.zeros((N, K // 8), dtype=torch.int32, device="cuda")
    s = torch.zeros((N, K // gs), dtype=torch.float32, device="cuda")
    Y = torch.full((T, N), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(q4.Int4Error, match="INT4_ERR_SHAPE"):
        q4.int4_gemm_noalloc(X, q, s, s, Y=Y)
    torch.cuda.synchronize()
    assert bool(torch.all(Y == 7.0)), "a refused call wrote its output"
