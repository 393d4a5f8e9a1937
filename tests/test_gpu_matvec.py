"""GPU parity of int4_matvec (one to eight decode lanes) with the oracle.

Ragged shapes (N not a multiple of the column step, K not a multiple of the
64-unit chunk), every group size the kernels accept, one-hot and
integer-exact closed forms (bitwise), lane independence (bitwise: against
calls with every other row replaced, for the matrix-core lanes, M >= 2),
K long enough for several passes over the waves, more columns than one round
of the LDS table, the table's LDS limit, and untouched memory around the
outputs."""
import numpy as np
import pytest

import oracle
import synth
from helpers import assert_dot_close, integer_problem

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q4():
    import torch
    torch.cuda.set_device(0)
    import int4_group_quantized_quant_amd as m
    return m


def to_dev(*arrs):
    import torch
    return [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in arrs]


def quantized(seed, N, K, gs):
    W = synth.weights(seed, N, K)
    return oracle.quantize_pack(W, gs)


def run_matvec(q4, X, q, s, z):
    import torch
    Xd, qd, sd, zd = to_dev(X, q.view(np.int32), s, z)
    Y = q4.int4_matvec(Xd, qd, sd, zd)
    torch.cuda.synchronize()
    return Y.cpu().numpy()


SHAPES = [
    (1, 32, 32), (3, 64, 32), (37, 96, 32), (64, 1024, 128), (1000, 1024, 128),
    (129, 2048, 64), (77, 2080, 32), (250, 4096, 128), (31, 5120, 64), (9, 14336, 128),
    (300, 3072, 256), (5, 8192, 2048),
    # K past 16384 switches the single lane from the register kernel to the
    # LDS kernel; 40960 floats fill the 160 KiB LDS.
    (13, 16384, 128), (11, 16416, 32), (3, 40960, 64),
]


@pytest.mark.parametrize("N,K,gs", SHAPES)
def test_single_lane(q4, N, K, gs):
    q, s, z = quantized(0xB000 + N * 7 + K, N, K, gs)
    x = synth.normal_f32(0xB001 + K, K)
    y_ref, B = oracle.matvec(x, q, s, z, K, gs)
    y = run_matvec(q4, x, q, s, z)
    assert_dot_close(y, y_ref, B, f"matvec N={N} K={K} gs={gs}")


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("N,K,gs", [(203, 1024, 128), (65, 5120, 64),
                                    (77, 2080, 32),    # K/32 not a multiple of 4
                                    (50, 3072, 96)])   # three units per group
def test_lanes(q4, M, N, K, gs):
    q, s, z = quantized(0xB100 + M, N, K, gs)
    X = synth.lanes(0xB101, M, K)
    Y_ref, B = oracle.matvec(X, q, s, z, K, gs)
    Y = run_matvec(q4, X, q, s, z)
    assert Y.shape == (M, N)
    assert_dot_close(Y, Y_ref, B, f"lanes M={M}")
    if M >= 2:
        # Matrix-core lanes never interact: replacing every other row leaves
        # a row's outputs bit-identical.
        for keep in (0, M - 1):
            X2 = synth.lanes(0xB102 + keep, M, K)
            X2[keep] = X[keep]
            Y2 = run_matvec(q4, X2, q, s, z)
            np.testing.assert_array_equal(Y2[keep].view(np.uint32), Y[keep].view(np.uint32))


def check_lanes(q4, X, q, s, z, K, gs, seed):
    Y_ref, B = oracle.matvec(X, q, s, z, K, gs)
    Y = run_matvec(q4, X, q, s, z)
    assert_dot_close(Y, Y_ref, B, f"lanes M={X.shape[0]} K={K} gs={gs}")
    M = X.shape[0]
    for keep in (0, M - 1):
        X2 = synth.lanes(seed + keep, M, K)
        X2[keep] = X[keep]
        Y2 = run_matvec(q4, X2, q, s, z)
        np.testing.assert_array_equal(Y2[keep].view(np.uint32), Y[keep].view(np.uint32))


@pytest.mark.parametrize("M", [2, 3, 8])
@pytest.mark.parametrize("N,K,gs", [(37, 16416, 32),   # 33 slices of 16 units: three passes of 11
                                    (29, 8256, 96),    # 17 slices, three units per group
                                    (23, 9216, 256),   # 18 slices, eight units per group
                                    (40, 7168, 1024),  # every slice inside one group
                                    (19, 25600, 32)])  # 800 groups per column: near the LDS table limit
def test_lanes_long_k(q4, M, N, K, gs):
    q, s, z = quantized(0xB180 + M + K, N, K, gs)
    check_lanes(q4, synth.lanes(0xB181 + K, M, K), q, s, z, K, gs, 0xB182)


def test_lanes_table_limit(q4):
    # 1024 groups per column do not fit the per-block scale/zero table.
    import torch
    q, s, z = quantized(0xB190, 4, 32768, 32)
    _, qd, sd, zd = to_dev(np.zeros(1, np.float32), q.view(np.int32), s, z)
    X = torch.zeros((2, 32768), dtype=torch.float32, device="cuda")
    with pytest.raises(q4.Int4Error):
        q4.int4_matvec(X, qd, sd, zd)


def test_lanes_more_blocks_than_resident(q4):
    """More tiles than one block per CU can hold in its LDS tables (70000
    columns at K = 16416): the grid then has more blocks than the device runs
    at once, each with the tiles its tables hold.  Random packed codes,
    integer zero points; every output is checked."""
    rng = np.random.default_rng(0xB700)
    N, K, gs, M = 70000, 16416, 32, 3
    q = rng.integers(0, 2**32, (N, K // 8), dtype=np.uint32)
    s = (rng.random((N, K // gs), dtype=np.float32) * 0.01 + 1e-3).astype(np.float32)
    z = rng.integers(0, 16, (N, K // gs)).astype(np.float32)
    X = synth.lanes(0xB701, M, K)
    Y = run_matvec(q4, X, q, s, z)
    Y_ref, B = oracle.matvec(X, q, s, z, K, gs)
    assert_dot_close(Y, Y_ref, B, "lanes, two rounds")


@pytest.mark.parametrize("K,gs", [(256, 32), (1024, 128), (2080, 32), (5120, 64)])
def test_one_hot_is_bit_exact(q4, K, gs):
    N = 70
    q, s, z = quantized(0xB200 + K, N, K, gs)
    dq = oracle.dequant(q, s, z, K, gs)
    ks = [0, 1, 2, 3, 7, 31, 32, gs - 1, K // 2 + 5, K - 1]
    X = np.zeros((len(ks), K), np.float32)
    for i, k in enumerate(ks):
        X[i, k] = 1.0
    for lo in range(0, len(ks), 8):
        Y = run_matvec(q4, X[lo:lo + 8], q, s, z)
        for i, k in enumerate(ks[lo:lo + 8]):
            np.testing.assert_array_equal(Y[i].view(np.uint32), dq[:, k].view(np.uint32),
                                          err_msg=f"one-hot k={k}")


@pytest.mark.parametrize("M", [1, 2, 4, 8])
@pytest.mark.parametrize("N,K,gs", [(100, 1024, 32), (41, 4160, 64)])
def test_integer_exact(q4, M, N, K, gs):
    rng = np.random.default_rng(M * 1000 + K)
    q, s, z, X, exact = integer_problem(rng, N, K, gs, M)
    Y = run_matvec(q4, X, q, s, z)
    np.testing.assert_array_equal(Y, exact.astype(np.float32))


def test_scale_and_sign_extremes(q4):
    # Large and tiny scales, negative activations, codes at 0 and 15.
    N, K, gs = 48, 512, 64
    W = synth.weights(0xB300, N, K)
    W[:16] *= 1e6
    W[16:32] *= 1e-6
    q, s, z = oracle.quantize_pack(W, gs)
    x = synth.normal_f32(0xB301, K) * 3
    y_ref, B = oracle.matvec(x, q, s, z, K, gs)
    assert_dot_close(run_matvec(q4, x, q, s, z), y_ref, B, "extremes")


def test_output_guards_untouched(q4):
    import torch
    N, K, gs, M = 333, 1024, 128, 3
    q, s, z = quantized(0xB400, N, K, gs)
    X = synth.lanes(0xB401, M, K)
    Xd, qd, sd, zd = to_dev(X, q.view(np.int32), s, z)
    buf = torch.full((M * N + 64,), 12345.0, dtype=torch.float32, device="cuda")
    Y = buf[32:32 + M * N].view(M, N)
    q4.int4_matvec(Xd, qd, sd, zd, Y=Y)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert np.all(host[:32] == 12345.0) and np.all(host[32 + M * N:] == 12345.0)
    Y_ref, B = oracle.matvec(X, q, s, z, K, gs)
    assert_dot_close(host[32:32 + M * N].reshape(M, N), Y_ref, B, "guarded")


def test_empty_and_zero_lanes(q4):
    import torch
    K, gs = 256, 64
    q = torch.empty((0, K // 8), dtype=torch.int32, device="cuda")
    s = torch.empty((0, K // gs), dtype=torch.float32, device="cuda")
    x = torch.zeros(K, dtype=torch.float32, device="cuda")
    assert q4.int4_matvec(x, q, s, s).shape == (0,)
    q, s, z = quantized(0xB500, 10, K, gs)
    _, qd, sd, zd = to_dev(np.zeros(1, np.float32), q.view(np.int32), s, z)
    X0 = torch.empty((0, K), dtype=torch.float32, device="cuda")
    assert q4.int4_matvec(X0, qd, sd, zd).shape == (0, 10)


def test_rejects_too_many_lanes(q4):
    import torch
    q, s, z = quantized(0xB600, 4, 256, 64)
    _, qd, sd, zd = to_dev(np.zeros(1, np.float32), q.view(np.int32), s, z)
    X = torch.zeros((9, 256), dtype=torch.float32, device="cuda")
    with pytest.raises(q4.Int4Error):
        q4.int4_matvec(X, qd, sd, zd)
