"""GPU parity of the multi-column path (32, 48 or 64 slot columns per weight
block, e.g. several speculative tokens per sequence), through the C ABI:
the slot buffer bit-exact against the oracle's quantiser, outputs within
1e-4 * sum|block terms| + 1e-6 of the oracle, and every column bit-identical
to the 16-slot kernel on the same slot contents and to a one-token call."""

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import gpu_matmul, gpu_pack, sample_rows, to_dev, within_tau

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import quantized_weight_streaming_q8_amd as q8
    assert q8.q8_device_supported(), "device is not gfx950"
    yield
    torch.cuda.synchronize()


def _q8():
    import quantized_weight_streaming_q8_amd as q8
    return q8


def _x(n, K, seed):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((n, K), dtype=np.float32)
    X[:, rng.choice(K, max(1, K // 100), replace=False)] *= np.float32(20)
    X[min(3, n - 1), :64] = 0.0          # zero blocks
    X[min(5, n - 1)] *= np.float32(1e-5)  # binary16-subnormal scales
    return X


def _quantize(X, n_slots, Xq=None):
    q8 = _q8()
    n, K = X.shape
    if Xq is None:
        Xq = q8.empty_act_slots(K, n_slots=n_slots)
    q8.q8_quantize_acts_n(to_dev(X), n, K, Xq, n_slots)
    return Xq


def _slots(Xq, K, n_slots):
    q, d = _q8().read_act_slots(Xq, K, n_slots=n_slots)
    torch.cuda.synchronize()
    return q.cpu().numpy(), d.cpu().numpy().view(np.uint16)


def _multi(Wq, Xq, n_slots, bi, N, K, rows=None):
    q8 = _q8()
    bi_d = to_dev(np.asarray(bi, dtype=np.int32))
    Y = torch.empty((bi_d.numel(), N), dtype=torch.float32, device="cuda")
    q8.q8_matmul_multi(Wq, Xq, n_slots, bi_d, bi_d.numel(), N, K, Y)
    torch.cuda.synchronize()
    Y = Y.cpu().numpy()
    return Y if rows is None else Y[:, rows]


@pytest.mark.parametrize("n_slots", [32, 48, 64])
@pytest.mark.parametrize("K", [288, 5120])
def test_quantize_acts_n_bit_exact(n_slots, K):
    X = _x(n_slots, K, seed=K + n_slots)
    Xq = _quantize(X, n_slots)
    q, d = _slots(Xq, K, n_slots)
    qo, do = oracle.quantize_rows(X)
    assert np.array_equal(q, qo)
    assert np.array_equal(d, do)


def test_quantize_acts_n_partial_rows_leave_other_slots():
    K, n_slots = 768, 64
    X = _x(n_slots, K, seed=4)
    Xq = _quantize(X, n_slots)
    Y2 = _x(40, K, seed=5)
    _quantize(Y2, n_slots, Xq)
    q, d = _slots(Xq, K, n_slots)
    qa, da = oracle.quantize_rows(Y2)
    qb, db = oracle.quantize_rows(X[40:])
    assert np.array_equal(q[:40], qa) and np.array_equal(d[:40], da)
    assert np.array_equal(q[40:], qb) and np.array_equal(d[40:], db)


# (5, 64): one row group holding 5 rows, one super-chunk of which 2 blocks are real
@pytest.mark.parametrize("N,K", [(5, 64), (17, 288), (100, 800), (33, 4128), (40, 17408), (1000, 5120)])
@pytest.mark.parametrize("n_slots", [32, 48, 64])
def test_multi_matches_oracle(N, K, n_slots):
    rng = np.random.default_rng(N * 7 + K + n_slots)
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    X = _x(n_slots, K, seed=K + 3 * n_slots)
    Wq, Xq = gpu_pack(W), _quantize(X, n_slots)
    qw, dw = oracle.quantize_rows(W)
    qx, dx = oracle.quantize_rows(X)
    for bi in (rng.permutation(n_slots), np.array([n_slots - 1]),
               rng.integers(0, n_slots, size=n_slots + 0),  # duplicates
               rng.permutation(n_slots)[: n_slots // 2 + 3]):
        bi = bi.astype(np.int32)
        Yo, Ao = oracle.matmul(qw, dw, qx, dx, bi)
        Y = _multi(Wq, Xq, n_slots, bi, N, K)
        ok, worst = within_tau(Y, Yo, Ao)
        assert ok, (N, K, n_slots, bi[:8], worst)


# The multi-column launch runs a row block's splits as waves of one workgroup,
# where the 16-slot kernel evaluates them in one whole-row wave or as split
# workgroups: (17405, 1056) 1088 row groups, 4 splits; (17981, 2080) 1124 row
# groups, 2 splits; (17500, 768) 3 splits; (18429, 1056) 1152 row groups
# (r = 128), 4 splits; (6555, 8224) 205 two-row-group blocks of long rows,
# four K ranges in one workgroup
@pytest.mark.parametrize("N,K", [(100, 800), (40, 17408), (2304, 5120), (17405, 1056),
                                 (17981, 2080), (17500, 768), (6555, 8224), (18429, 1056)])
def test_multi_columns_equal_the_16_slot_kernel(N, K):
    """Slot 16c + s of a 64-slot buffer gives the bits of slot s of a 16-slot
    buffer holding the same rows; n_slots = 16 is the 16-slot kernel itself."""
    rng = np.random.default_rng(N + K)
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    X = _x(64, K, seed=K)
    Wq = gpu_pack(W)
    Xq64 = _quantize(X, 64)
    for c in range(4):
        Xq16 = _quantize(np.ascontiguousarray(X[16 * c:16 * c + 16]), 16)
        bi16 = rng.permutation(16).astype(np.int32)
        Y16 = gpu_matmul(Wq, Xq16, bi16, N, K)
        Ym = _multi(Wq, Xq64, 64, bi16 + 16 * c, N, K)
        assert np.array_equal(Y16.view(np.uint32), Ym.view(np.uint32)), c
        Y1 = _multi(Wq, Xq16, 16, bi16, N, K)
        assert np.array_equal(Y16.view(np.uint32), Y1.view(np.uint32)), c


# Launch shapes of the multi-column kernels (two row groups per wave; ring
# depth from the weights in flight): (17981, 2080) 1124 row groups with 2
# splits runs two tiles at depth 2 and four at depth 4; (72003, 256) 4501 row
# groups in one split, two tiles at depth 1 and four at depth 2; (18429, 1056)
# 1152 row groups with 4 splits, two tiles at depth 4 and four at depth 2;
# three tiles run at depth 2 everywhere.
@pytest.mark.parametrize("N,K", [(17981, 2080), (72003, 256), (18429, 1056)])
def test_multi_widths_equal_the_16_slot_kernel(N, K):
    """At 32, 48 and 64 slots every 16-slot group of columns gives the bits
    of the 16-slot kernel on the same rows, and sampled rows of the 64-slot
    result match the oracle."""
    rng = np.random.default_rng(N - K)
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    X = _x(64, K, seed=K + 11)
    Wq = gpu_pack(W)
    Y16 = []
    for c in range(4):
        Xq16 = _quantize(np.ascontiguousarray(X[16 * c:16 * c + 16]), 16)
        Y16.append(gpu_matmul(Wq, Xq16, np.arange(16, dtype=np.int32), N, K))
    for n in (32, 48, 64):
        Xq = _quantize(np.ascontiguousarray(X[:n]), n)
        Y = _multi(Wq, Xq, n, np.arange(n, dtype=np.int32), N, K)
        for c in range(n // 16):
            assert np.array_equal(Y[16 * c:16 * c + 16].view(np.uint32), Y16[c].view(np.uint32)), (n, c)
    rows = sample_rows(N, 64, seed=N)
    qw, dw = oracle.quantize_rows(W[rows])
    qx, dx = oracle.quantize_rows(X)
    bi = rng.permutation(64).astype(np.int32)
    Yo, Ao = oracle.matmul(qw, dw, qx, dx, bi)
    ok, worst = within_tau(Y[bi][:, rows], Yo, Ao)
    assert ok, worst


def test_multi_columns_equal_single_token_calls():
    N, K, n_slots = 2304, 5120, 64
    rng = np.random.default_rng(9)
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    Wq, Xq = gpu_pack(W), _quantize(_x(n_slots, K, seed=10), n_slots)
    bi = rng.permutation(n_slots).astype(np.int32)
    Y = _multi(Wq, Xq, n_slots, bi, N, K)
    for t in (0, 1, 17, 31, 32, 47, 63):
        y1 = _multi(Wq, Xq, n_slots, bi[t:t + 1], N, K)
        assert np.array_equal(Y[t].view(np.uint32), y1[0].view(np.uint32)), t
    for n in (5, 33, 50):
        Yn = _multi(Wq, Xq, n_slots, bi[:n], N, K)
        assert np.array_equal(Yn.view(np.uint32), Y[:n].view(np.uint32)), n


def test_multi_bad_slot_gives_nan_row():
    N, K, n_slots = 64, 512, 32
    rng = np.random.default_rng(11)
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    X = _x(n_slots, K, seed=12)
    Wq, Xq = gpu_pack(W), _quantize(X, n_slots)
    bi = np.array([3, 32, 31, -1, 64, 0], dtype=np.int32)
    Y = _multi(Wq, Xq, n_slots, bi, N, K)
    assert np.all(np.isnan(Y[[1, 3, 4]]))
    qw, dw = oracle.quantize_rows(W)
    qx, dx = oracle.quantize_rows(X)
    Yo, Ao = oracle.matmul(qw, dw, qx, dx, bi[[0, 2, 5]])
    assert within_tau(Y[[0, 2, 5]], Yo, Ao)[0]


def test_multi_qwen3_layer_64_columns():
    """The Qwen3-14B-shaped layer with 64 columns (e.g. 16 sequences x 4
    speculative tokens), seeded random batch_index; sampled rows against the
    oracle."""
    w = wl.WORKLOADS["qwen3_layer"]
    rng = np.random.default_rng([0, w.config, 3, 64])
    for i, m in enumerate(w.matrices):
        W = wl.weights(w.config, i, m.N, m.K)
        X = rng.standard_normal((64, m.K), dtype=np.float32)
        Wq, Xq = gpu_pack(W), _quantize(X, 64)
        bi = rng.permutation(64).astype(np.int32)
        rows = sample_rows(m.N, 48, seed=i)
        Y = _multi(Wq, Xq, 64, bi, m.N, m.K)
        qw, dw = oracle.quantize_rows(W[rows])
        qx, dx = oracle.quantize_rows(X)
        Yo, Ao = oracle.matmul(qw, dw, qx, dx, bi)
        ok, worst = within_tau(Y[:, rows], Yo, Ao)
        assert ok, (m.name, worst)
        del Wq, Xq
        torch.cuda.empty_cache()
