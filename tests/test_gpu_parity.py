"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Bars: quantised int8 blocks and binary16 scales bit-exact; per-block int32
sums exact; fp32 outputs within 1e-4 * sum|block terms| + 1e-6 of the
oracle's double sum; per-token columns bit-identical to single-token calls;
the MFMA and DOT4 engines bit-identical to each other.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import (gpu_matmul, gpu_matmul_ws, gpu_pack, gpu_pack_q,
                      gpu_quantize_acts, gpu_unpack, sample_rows, slots_host,
                      split_counters_clear, to_dev, within_tau, write_slots)

pytestmark = pytest.mark.gpu

MFMA, DOT4 = 1, 2


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import quantized_weight_streaming_q8_amd as q8
    assert q8.q8_device_supported(), "device is not gfx950"
    yield
    torch.cuda.synchronize()


def _ragged_x(K, seed, outliers=False):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((16, K), dtype=np.float32)
    if outliers:
        X[:, rng.choice(K, max(1, K // 100), replace=False)] *= np.float32(20)
    X[3, :64] = 0.0            # zero blocks
    X[5] *= np.float32(1e-5)   # binary16-subnormal scales
    return X


# ---------------------------------------------------------------- quantiser

@pytest.mark.parametrize("K", [32, 288, 768, 3072, 4128, 5120, 7168, 17408, 18432])
def test_quantize_acts_bit_exact(K):
    X = _ragged_x(K, seed=K, outliers=True)
    Xq = gpu_quantize_acts(X)
    q, d = slots_host(Xq, K)
    qo, do = oracle.quantize_rows(X)
    assert np.array_equal(q, qo)
    assert np.array_equal(d, do)


def test_quantize_acts_pads_with_zero():
    """Blocks past K inside the last 256-value super-chunk are written as
    zero (q and scale), whatever the buffer held before."""
    import quantized_weight_streaming_q8_amd as q8
    K = 4128  # 129 blocks: 7 padding blocks in the last super-chunk
    Xq = q8.empty_act_slots(K)
    Xq.fill_(0x5A)
    gpu_quantize_acts(_ragged_x(K, seed=2), Xq)
    Kp = 17 * 256
    qp, dp = slots_host(Xq, Kp)  # read the padded width back
    assert not qp[:, K:].any() and not dp[:, K // 32:].any()


def test_quantize_acts_partial_rows_leave_other_slots():
    K = 1024
    import quantized_weight_streaming_q8_amd as q8
    Xq = q8.empty_act_slots(K)
    rng = np.random.default_rng(3)
    q0 = rng.integers(-128, 128, size=(16, K)).astype(np.int8)
    d0 = rng.integers(0, 0x7c00, size=(16, K // 32)).astype(np.uint16)
    write_slots(Xq, K, q0, d0)
    X = _ragged_x(K, seed=1)[:5]
    gpu_quantize_acts(X, Xq)
    q, d = slots_host(Xq, K)
    qo, do = oracle.quantize_rows(X)
    assert np.array_equal(q[:5], qo) and np.array_equal(d[:5], do)
    assert np.array_equal(q[5:], q0[5:]) and np.array_equal(d[5:], d0[5:])


def _edge_rows(n_rows, K, seed):
    """fp32 rows of N(0,1) blocks with the format's edge blocks (a NaN or an
    infinity in the block, scales that underflow to zero or overflow
    binary16; the pins fix their quantisation by hand) placed at seeded
    block positions."""
    import pins
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((n_rows, K), dtype=np.float32)
    KB = K // 32
    for r in range(n_rows):
        for _, x, _, _ in pins.edge_blocks():
            if rng.random() < 0.6:
                b = int(rng.integers(0, KB))
                X[r, 32 * b:32 * b + 32] = x
    return X


@pytest.mark.parametrize("K", [288, 5120])
def test_quantize_edge_blocks_bit_exact(K):
    """NaN and infinity blocks, underflowing and overflowing scales: the
    pre-quantiser and the packer give the oracle's bits."""
    X = _edge_rows(16, K, seed=K)
    Xq = gpu_quantize_acts(X)
    q, d = slots_host(Xq, K)
    qo, do = oracle.quantize_rows(X)
    assert np.array_equal(q, qo)
    assert np.array_equal(d, do)
    W = _edge_rows(37, K, seed=K + 1)
    qw, dw = gpu_unpack(gpu_pack(W), 37, K)
    qwo, dwo = oracle.quantize_rows(W)
    assert np.array_equal(qw, qwo)
    assert np.array_equal(dw, dwo)


def test_matmul_nan_blocks_give_nan_outputs():
    """A weight row or an activation slot holding a NaN or an infinity gives
    NaN outputs exactly where the oracle does; the other outputs stay within
    tolerance."""
    import pins
    N, K = 48, 1024
    rng = np.random.default_rng(9)
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    X = rng.standard_normal((16, K), dtype=np.float32)
    nan_block = pins.edge_blocks()[0][1]
    W[5, 64:96] = nan_block
    X[7, 512:544] = nan_block
    Wq, Xq = gpu_pack(W), gpu_quantize_acts(X)
    bi = rng.permutation(16).astype(np.int32)
    Yo, Ao = _oracle_y(W, X, bi)
    for p in (MFMA, DOT4):
        Y = gpu_matmul(Wq, Xq, bi, N, K, p)
        assert np.array_equal(np.isnan(Y), np.isnan(Yo)), p
        assert np.isnan(Yo[:, 5]).all() and np.isnan(Yo[list(bi).index(7)]).all()
        fin = ~np.isnan(Yo)
        assert within_tau(Y[fin], Yo[fin], Ao[fin])[0], p


# ------------------------------------------------------------------- packer

@pytest.mark.parametrize("N,K", [(1, 32), (17, 288), (100, 800), (768, 768),
                                 (2304, 768), (768, 3072), (33, 4128)])
def test_pack_weights_bit_exact_small(N, K):
    rng = np.random.default_rng(N * 7 + K)
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    W[0, :32] = 0.0
    Wq = gpu_pack(W)
    q, d = gpu_unpack(Wq, N, K)
    qo, do = oracle.quantize_rows(W)
    assert np.array_equal(q, qo) and np.array_equal(d, do)


@pytest.mark.parametrize("key,idx", [("qwen3_layer", 0), ("qwen3_layer", 1),
                                     ("qwen3_layer", 2), ("qwen3_layer", 3),
                                     ("large_dense", 0), ("large_dense", 1)])
def test_pack_weights_bit_exact_full(key, idx):
    w = wl.WORKLOADS[key]
    m = w.matrices[idx]
    W = wl.weights(w.config, idx, m.N, m.K)
    Wq = gpu_pack(W)
    q, d = gpu_unpack(Wq, m.N, m.K)
    qo, do = oracle.quantize_rows(W)
    assert np.array_equal(q, qo) and np.array_equal(d, do)


def test_pack_q_round_trip_any_int8():
    rng = np.random.default_rng(5)
    N, K = 37, 1056
    q = rng.integers(-128, 128, size=(N, K)).astype(np.int8)
    d = rng.integers(0, 0x7c00, size=(N, K // 32)).astype(np.uint16)
    Wq = gpu_pack_q(q, d)
    q2, d2 = gpu_unpack(Wq, N, K)
    assert np.array_equal(q, q2) and np.array_equal(d, d2)


# ------------------------------------------------------------------- matmul

def _oracle_y(W, X, bi, rows=None):
    Wr = W if rows is None else W[rows]
    qw, dw = oracle.quantize_rows(Wr)
    qx, dx = oracle.quantize_rows(X)
    return oracle.matmul(qw, dw, qx, dx, bi)


@pytest.mark.parametrize("N,K", [(1, 32), (17, 288), (15, 2080), (100, 800),
                                 (16, 256), (33, 4128), (768, 768), (40, 17408),
                                 (17, 8224), (100, 9024), (1000, 5120), (5120, 2080)])
def test_matmul_ragged_shapes(N, K):
    rng = np.random.default_rng(N + K)
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    X = _ragged_x(K, seed=K + 1)
    Wq, Xq = gpu_pack(W), gpu_quantize_acts(X)
    import quantized_weight_streaming_q8_amd as q8
    ws = q8.zeroed_workspace(N, K)
    for bi in (np.array([0]), np.array([3, 3, 9]), rng.permutation(16),
               np.array([15, 2, 2, 7, 0, 11, 5])):
        bi = bi.astype(np.int32)
        Yo, Ao = _oracle_y(W, X, bi)
        Ym = gpu_matmul(Wq, Xq, bi, N, K, MFMA)
        ok, worst = within_tau(Ym, Yo, Ao)
        assert ok, (N, K, bi, worst)
        Yd = gpu_matmul(Wq, Xq, bi, N, K, DOT4)
        assert np.array_equal(Ym.view(np.uint32), Yd.view(np.uint32)), (N, K, bi)
        Yw = gpu_matmul_ws(Wq, Xq, bi, N, K, ws)
        assert np.array_equal(Ym.view(np.uint32), Yw.view(np.uint32)), (N, K, bi)


# Large ragged shapes that reach each tiling the default rule picks for 1024+
# row groups: one row group per wave with 4 (G <= 1466), 2 (G <= 2933) or 1
# (G <= 4400) chunks in flight, and two row groups per wave past 4400; N is
# not a multiple of 16 and K leaves the last super-chunk partly empty.  For
# G mod 256 = r in 1..128 the tree has min(4, 256 / r, NSC) splits, and the
# workspace entry point runs only the last r row groups as split workgroups:
# r = 1 (4 splits), 100 (2 splits), 64 (4 splits), 128 (4 splits, two pieces
# per CU); 209 and 185 are not split.
# r = 70 gives 3 splits (K = 1312: folds at super-chunks 2 and 4 of 6; K = 768:
# at 1 and 2 of 3, the second on the last super-chunk); r = 100 with K = 512
# folds on the last of its 2 super-chunks.  18992 x 5120 is one of eight
# column shards of the 151936-row head (1187 row groups, r = 163: not split).
@pytest.mark.parametrize("N,K", [(16391, 4128), (32005, 800), (48003, 1056), (72009, 800),
                                 (17981, 2080), (17405, 1056), (17500, 1312), (17500, 768),
                                 (17981, 512), (18992, 5120), (18429, 1056)])
def test_matmul_large_ragged_shapes(N, K):
    rng = np.random.default_rng(N - K)
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    X = _ragged_x(K, seed=K + 2)
    Wq, Xq = gpu_pack(W), gpu_quantize_acts(X)
    import quantized_weight_streaming_q8_amd as q8
    ws = q8.zeroed_workspace(N, K)
    rows = sample_rows(N, 96, seed=N)
    for bi in (rng.permutation(16), np.array([5, 5, 0, 12])):
        bi = bi.astype(np.int32)
        Yo, Ao = _oracle_y(W, X, bi, rows)
        Ym = gpu_matmul(Wq, Xq, bi, N, K, MFMA)
        ok, worst = within_tau(Ym[:, rows], Yo, Ao)
        assert ok, (N, K, bi, worst)
        Yw = gpu_matmul_ws(Wq, Xq, bi, N, K, ws)
        assert np.array_equal(Ym.view(np.uint32), Yw.view(np.uint32)), (N, K, bi)
        Yd = gpu_matmul(Wq, Xq, bi, N, K, DOT4)
        assert np.array_equal(Ym.view(np.uint32), Yd.view(np.uint32)), (N, K, bi)
    # every column is its slot's column of the full 16-slot call
    full = gpu_matmul(Wq, Xq, np.arange(16, dtype=np.int32), N, K, MFMA)
    bi = np.array([7, 3, 3, 14], dtype=np.int32)
    Yb = gpu_matmul(Wq, Xq, bi, N, K, MFMA)
    assert np.array_equal(Yb.view(np.uint32), full[bi].view(np.uint32))
    del Wq
    torch.cuda.empty_cache()


# Long rows (K >= 8192) whose two-row-group blocks number 205..256 run their
# four K ranges as four wave slices of one workgroup; 204 or fewer blocks, or
# more than 256, run them as four split workgroups.  Both evaluate the same
# ranges and add them in the same order, so a row's bits do not depend on
# which side of the boundary its matrix falls: 6555 rows (410 row groups, 205
# blocks, the last group ragged) against their first 6528 (204 blocks), and
# 8192 rows (256 blocks) against 8208 (257 blocks).  K = 8224 leaves the last
# of its 33 super-chunks one block long.
@pytest.mark.parametrize("N_wg,N_split", [(6555, 6528), (8192, 8208)])
def test_long_rows_same_bits_either_side_of_the_workgroup_rule(N_wg, N_split):
    import quantized_weight_streaming_q8_amd as q8
    K = 8224
    N = max(N_wg, N_split)
    assert q8.q8_matmul_workspace_bytes(N_wg, K) == 0
    assert q8.q8_matmul_workspace_bytes(N_split, K) > 0
    rng = np.random.default_rng(N_wg)
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    X = _ragged_x(K, seed=K + 3, outliers=True)
    Xq = gpu_quantize_acts(X)
    Y = {}
    for n in (N_wg, N_split):
        Wq = gpu_pack(np.ascontiguousarray(W[:n]))
        ws = q8.zeroed_workspace(n, K)
        rows = sample_rows(n, 96, seed=n)
        for bi in (rng.permutation(16), np.array([2, 11, 11])):
            bi = bi.astype(np.int32)
            Yo, Ao = _oracle_y(W[:n], X, bi, rows)
            Ym = gpu_matmul(Wq, Xq, bi, n, K, MFMA)
            ok, worst = within_tau(Ym[:, rows], Yo, Ao)
            assert ok, (n, K, bi, worst)
            Yw = gpu_matmul_ws(Wq, Xq, bi, n, K, ws)
            assert np.array_equal(Ym.view(np.uint32), Yw.view(np.uint32)), (n, bi)
            Yd = gpu_matmul(Wq, Xq, bi, n, K, DOT4)
            assert np.array_equal(Ym.view(np.uint32), Yd.view(np.uint32)), (n, bi)
        Y[n] = gpu_matmul_ws(Wq, Xq, np.arange(16, dtype=np.int32), n, K, ws)
        del Wq, ws
    m = min(N_wg, N_split)
    assert np.array_equal(Y[N_wg][:, :m].view(np.uint32), Y[N_split][:, :m].view(np.uint32))
    torch.cuda.empty_cache()


def test_largest_k():
    """The largest K the boundary takes, 2^24 - 32: 65536 super-chunks, the
    last of them 7 blocks long, split 4 ways across workgroups; N = 17 (a
    ragged second row group).  Packed weights and slots bit-exact, outputs
    within tolerance of the oracle, and the plain, workspace and DOT4
    paths bit-identical.  (Each wave here adds ~131k terms in order, past
    the length for which the tolerance bounds every order; the error of
    these sums stays far inside it all the same.)"""
    import quantized_weight_streaming_q8_amd as q8
    N, K = 17, (1 << 24) - 32
    assert q8.q8_packed_weight_bytes(N, K) > 0 and q8.q8_matmul_workspace_bytes(N, K) > 0
    rng = np.random.default_rng(2024)
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    X = rng.standard_normal((16, K), dtype=np.float32)
    Wq, Xq = gpu_pack(W), gpu_quantize_acts(X)
    qw, dw = oracle.quantize_rows(W)
    qx, dx = oracle.quantize_rows(X)
    q, d = gpu_unpack(Wq, N, K)
    assert np.array_equal(q, qw) and np.array_equal(d, dw)
    del q, d
    qs, ds = slots_host(Xq, K)
    assert np.array_equal(qs, qx) and np.array_equal(ds, dx)
    del qs, ds
    ws = q8.zeroed_workspace(N, K)
    for bi in (rng.permutation(16), np.array([9, 0, 9])):
        bi = bi.astype(np.int32)
        Yo, Ao = oracle.matmul(qw, dw, qx, dx, bi)
        Ym = gpu_matmul(Wq, Xq, bi, N, K, MFMA)
        ok, worst = within_tau(Ym, Yo, Ao)
        assert ok, (bi, worst)
        Yw = gpu_matmul_ws(Wq, Xq, bi, N, K, ws)
        assert np.array_equal(Ym.view(np.uint32), Yw.view(np.uint32)), bi
        Yd = gpu_matmul(Wq, Xq, bi, N, K, DOT4)
        assert np.array_equal(Ym.view(np.uint32), Yd.view(np.uint32)), bi
    del Wq, Xq, ws
    torch.cuda.empty_cache()


def test_largest_n():
    """The most rows the boundary takes at K = 32, 2^26: K pads to one
    256-value super-chunk, so the padded matrix holds the limit of 2^34
    values (an 18 GB packed buffer, 2^31 threads to pack it, 2^21
    workgroups to stream it).  The weights come in as canonical q8_0
    (random codes, fp16 scales); sampled rows, the first and the last
    included, are checked against the oracle on the device's outputs, and
    the DOT4 engine must give the same bits."""
    import quantized_weight_streaming_q8_amd as q8
    N, K = 1 << 26, 32
    assert q8.q8_packed_weight_bytes(N, K) > 0 and q8.q8_packed_weight_bytes(N + 1, K) == 0
    rng = np.random.default_rng(26)
    q = rng.integers(-127, 128, size=(N, K), dtype=np.int8)
    d16 = rng.uniform(1e-4, 1e-3, size=(N, 1)).astype(np.float16).view(np.uint16)
    Wq = gpu_pack_q(q, d16)
    X = rng.standard_normal((16, K), dtype=np.float32)
    Xq = gpu_quantize_acts(X)
    qx, dx = oracle.quantize_rows(X)
    rows = sample_rows(N, 96, seed=26)
    rows_d = torch.from_numpy(rows).cuda()
    for bi in (rng.permutation(16), np.array([4])):
        bi = bi.astype(np.int32)
        bi_d = to_dev(bi)
        Y = torch.empty((bi.size, N), dtype=torch.float32, device="cuda")
        q8.q8_matmul_narrow(Wq, Xq, bi_d, bi.size, N, K, Y)
        Yd = torch.empty_like(Y)
        q8.q8_matmul_narrow_path(Wq, Xq, bi_d, bi.size, N, K, Yd, DOT4)
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int32), Yd.view(torch.int32)), bi
        Ys = Y[:, rows_d].cpu().numpy()
        Yo, Ao = oracle.matmul(q, d16, qx, dx, bi, rows)
        ok, worst = within_tau(Ys, Yo, Ao)
        assert ok, (bi, worst)
        del Y, Yd
    del Wq
    torch.cuda.empty_cache()


@pytest.mark.parametrize("n_live", [1, 2, 4])
def test_single_768(n_live):
    w = wl.WORKLOADS["single"]
    W, X = wl.workload_inputs("single", 0)
    bi = wl.batch_index(w.config, n_live, random=False)
    Wq, Xq = gpu_pack(W), gpu_quantize_acts(X)
    Yo, Ao = _oracle_y(W, X, bi)
    for path in (0, MFMA, DOT4):
        ok, worst = within_tau(gpu_matmul(Wq, Xq, bi, 768, 768, path), Yo, Ao)
        assert ok, (path, worst)


def test_llama68m_stack():
    w = wl.WORKLOADS["llama68m"]
    for idx, m in enumerate(w.matrices):
        W, X = wl.workload_inputs("llama68m", idx)
        Wq, Xq = gpu_pack(W), gpu_quantize_acts(X)
        for n_live in w.n_live:
            bi = wl.batch_index(w.config, n_live, random=False)
            Yo, Ao = _oracle_y(W, X, bi)
            Y = gpu_matmul(Wq, Xq, bi, m.N, m.K)
            ok, worst = within_tau(Y, Yo, Ao)
            assert ok, (m.name, n_live, worst)


def test_block_sums_exact_through_the_kernel():
    """With weight scale 1 on block b0 and +0 elsewhere, and activation scale
    1, Y[t,n] is exactly the int32 block sum S_b0 (every other term is +0 and
    S < 2^24 is exact in fp32)."""
    rng = np.random.default_rng(19)
    N, K = 48, 2080  # 65 blocks: a partial last super-chunk
    KB = K // 32
    qw = rng.integers(-128, 128, size=(N, K)).astype(np.int8)
    qx = rng.integers(-128, 128, size=(16, K)).astype(np.int8)
    qw[0, :] = -128
    qx[4, :] = -128  # S = 2^19 for row 0, slot 4
    import quantized_weight_streaming_q8_amd as q8
    Xq = q8.empty_act_slots(K)
    write_slots(Xq, K, qx, np.full((16, KB), 0x3c00, dtype=np.uint16))
    bi = np.array([4, 0, 15, 7, 4], dtype=np.int32)
    S = oracle.block_dots(qw, qx, bi)
    for b0 in (0, 1, 7, 8, 31, 63, 64):
        d = np.zeros((N, KB), dtype=np.uint16)
        d[:, b0] = 0x3c00
        Wq = gpu_pack_q(qw, d)
        for path in (MFMA, DOT4):
            Y = gpu_matmul(Wq, Xq, bi, N, K, path)
            assert np.array_equal(Y, S[:, :, b0].astype(np.float32)), (b0, path)
    assert S[0, 0, 0] == 1 << 19


def test_pad_slots_do_not_leak():
    """Slots that are not live may hold anything (here random bytes and
    infinite / NaN scales): the live outputs do not change by a bit."""
    rng = np.random.default_rng(23)
    N, K = 64, 1024
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    X = rng.standard_normal((16, K), dtype=np.float32)
    Wq = gpu_pack(W)
    Xq = gpu_quantize_acts(X)
    bi = np.array([2, 9, 5], dtype=np.int32)
    clean = {p: gpu_matmul(Wq, Xq, bi, N, K, p) for p in (MFMA, DOT4)}
    q, d = slots_host(Xq, K)
    for s in range(16):
        if s in bi:
            continue
        q[s] = rng.integers(-128, 128, size=K).astype(np.int8)
        d[s] = rng.integers(0, 1 << 16, size=K // 32).astype(np.uint16)
    d[0] = 0x7c00  # +inf
    d[1] = 0x7e00  # NaN
    write_slots(Xq, K, q, d)
    for p in (MFMA, DOT4):
        assert np.array_equal(gpu_matmul(Wq, Xq, bi, N, K, p).view(np.uint32),
                              clean[p].view(np.uint32))


def test_bad_batch_index_gives_nan_row():
    rng = np.random.default_rng(29)
    N, K = 40, 512
    W = rng.standard_normal((N, K), dtype=np.float32)
    X = rng.standard_normal((16, K), dtype=np.float32)
    Wq, Xq = gpu_pack(W), gpu_quantize_acts(X)
    bi = np.array([1, 16, -1, 3, 1 << 30], dtype=np.int32)
    Yo, Ao = _oracle_y(W, X, np.array([1, 3], dtype=np.int32))
    for p in (MFMA, DOT4):
        Y = gpu_matmul(Wq, Xq, bi, N, K, p)
        assert np.all(np.isnan(Y[[1, 2, 4]]))
        assert within_tau(Y[[0, 3]], Yo, Ao)[0]


def test_workspace_is_rearmed_by_every_call():
    """A workspace used by many calls in a row (and by calls with different
    live batches) keeps giving the plain entry point's bits, and has every
    row block's arrival counter back at zero after each call."""
    import quantized_weight_streaming_q8_amd as q8
    rng = np.random.default_rng(37)
    N, K = 5120, 17408  # long rows: the workspace entry point splits K across workgroups
    assert q8.q8_matmul_workspace_bytes(N, K) > 0
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    X = rng.standard_normal((16, K), dtype=np.float32)
    Wq, Xq = gpu_pack(W), gpu_quantize_acts(X)
    ws = q8.zeroed_workspace(N, K)
    for rep in range(3):
        for n in (16, 1, 5):
            bi = rng.permutation(16)[:n].astype(np.int32)
            Yp = gpu_matmul(Wq, Xq, bi, N, K)
            Yw = gpu_matmul_ws(Wq, Xq, bi, N, K, ws)
            assert np.array_equal(Yp.view(np.uint32), Yw.view(np.uint32)), (rep, n)
            assert split_counters_clear(ws, N, K), (rep, n)


def test_one_workspace_serves_every_shape():
    """One workspace shared by split matrices of different row-block counts,
    in turns: each call gives the plain entry point's bits.  The partial sums
    a call leaves behind must never sit where another shape keeps a counter
    (with the counters of all row blocks first and the partials after them,
    a shape with more row blocks would find them there)."""
    import quantized_weight_streaming_q8_amd as q8
    rng = np.random.default_rng(41)
    # 188, 38, 125 row groups, all split; then 1088 and 1124 row groups whose
    # last 64 and 100 are split (4 and 2 splits)
    shapes = [(3000, 8448), (600, 9024), (2000, 8192), (17405, 1056), (17981, 2080)]
    mats = []
    for N, K in shapes:
        assert q8.q8_matmul_workspace_bytes(N, K) > 0, (N, K)
        W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
        X = rng.standard_normal((16, K), dtype=np.float32)
        mats.append((N, K, gpu_pack(W), gpu_quantize_acts(X)))
    nbytes = max(q8.q8_matmul_workspace_bytes(N, K) for N, K in shapes)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    for rep, i in enumerate((0, 1, 3, 2, 4, 0, 3, 1, 2, 4, 1)):
        N, K, Wq, Xq = mats[i]
        bi = rng.permutation(16)[: 1 + rep * 2].astype(np.int32)
        Yp = gpu_matmul(Wq, Xq, bi, N, K)
        Yw = gpu_matmul_ws(Wq, Xq, bi, N, K, ws)
        assert np.array_equal(Yp.view(np.uint32), Yw.view(np.uint32)), (rep, N, K)
        assert split_counters_clear(ws, N, K), (rep, N, K)


def test_columns_equal_single_token_calls():
    """Row t of a batched call is bit-identical to the call with n_live = 1
    and batch_index = {batch_index[t]}, for every t, on both engines."""
    N, K = 2304, 5120
    rng = np.random.default_rng(31)
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    X = _ragged_x(K, seed=3, outliers=True)
    Wq, Xq = gpu_pack(W), gpu_quantize_acts(X)
    bi = rng.permutation(16).astype(np.int32)
    for p in (MFMA, DOT4):
        Y = gpu_matmul(Wq, Xq, bi, N, K, p)
        for t in range(16):
            y1 = gpu_matmul(Wq, Xq, bi[t:t + 1], N, K, p)
            assert np.array_equal(Y[t].view(np.uint32), y1[0].view(np.uint32)), (p, t)
        for n in (3, 8, 13):
            Yn = gpu_matmul(Wq, Xq, bi[:n], N, K, p)
            assert np.array_equal(Yn.view(np.uint32), Y[:n].view(np.uint32)), (p, n)


# -------------------------------------------- full-size model-shaped layers

def test_qwen3_layer_every_live_batch():
    """Qwen3-14B decode layer, every live batch 1..16 with a seeded random
    batch_index, in the launch configuration the benchmark times: every row
    against the oracle at n_live 1 and 16, sampled rows at the others, and
    the two engines bit-identical on all rows."""
    w = wl.WORKLOADS["qwen3_layer"]
    for idx, m in enumerate(w.matrices):
        W, X = wl.workload_inputs("qwen3_layer", idx)
        Wq, Xq = gpu_pack(W), gpu_quantize_acts(X)
        import quantized_weight_streaming_q8_amd as q8
        ws = q8.zeroed_workspace(m.N, m.K)
        rows = sample_rows(m.N, 96, seed=idx)
        qw_all, dw_all = oracle.quantize_rows(W)
        qw, dw = qw_all[rows], dw_all[rows]
        qx, dx = oracle.quantize_rows(X)
        del W
        for n_live in w.n_live:
            bi = wl.batch_index(w.config, n_live, random=True)
            Y = gpu_matmul(Wq, Xq, bi, m.N, m.K)
            if n_live in (1, 16):  # every row
                Yo, Ao = oracle.matmul(qw_all, dw_all, qx, dx, bi)
                ok, worst = within_tau(Y, Yo, Ao)
            else:
                Yo, Ao = oracle.matmul(qw, dw, qx, dx, bi)
                ok, worst = within_tau(Y[:, rows], Yo, Ao)
            assert ok, (m.name, n_live, worst)
            Yw = gpu_matmul_ws(Wq, Xq, bi, m.N, m.K, ws)
            assert np.array_equal(Y.view(np.uint32), Yw.view(np.uint32)), (m.name, n_live)
            if n_live in (1, 7, 16):
                Yd = gpu_matmul(Wq, Xq, bi, m.N, m.K, DOT4)
                assert np.array_equal(Y.view(np.uint32), Yd.view(np.uint32)), (m.name, n_live)
        del Wq
        torch.cuda.empty_cache()


def test_qwen3_head_columns():
    """The Qwen3-14B head 5120 -> 151936: the packer bit-exact on the whole
    matrix, every row against the oracle at n_live 16 and sampled rows at
    1, 2, 4 and 8, and every column bit-identical to its single-token call."""
    w = wl.WORKLOADS["qwen3_head"]
    m = w.matrices[0]
    W, X = wl.workload_inputs("qwen3_head", 0)
    Wq, Xq = gpu_pack(W), gpu_quantize_acts(X)
    rows = sample_rows(m.N, 128, seed=4)
    qw_all, dw_all = oracle.quantize_rows(W)
    del W
    q, d = gpu_unpack(Wq, m.N, m.K)
    assert np.array_equal(q, qw_all) and np.array_equal(d, dw_all)
    del q, d
    qw, dw = qw_all[rows], dw_all[rows]
    qx, dx = oracle.quantize_rows(X)
    Y16 = None
    for n_live in w.n_live:
        bi = wl.batch_index(w.config, n_live, random=False)
        Y = gpu_matmul(Wq, Xq, bi, m.N, m.K)
        if n_live == 16:  # every row
            Yo, Ao = oracle.matmul(qw_all, dw_all, qx, dx, bi)
            ok, worst = within_tau(Y, Yo, Ao)
        else:
            Yo, Ao = oracle.matmul(qw, dw, qx, dx, bi)
            ok, worst = within_tau(Y[:, rows], Yo, Ao)
        assert ok, (n_live, worst)
        if n_live == 16:
            Y16 = Y
    for t in range(16):
        y1 = gpu_matmul(Wq, Xq, np.array([t], dtype=np.int32), m.N, m.K)
        assert np.array_equal(y1[0].view(np.uint32), Y16[t].view(np.uint32)), t


@pytest.mark.parametrize("idx", [0, 1])
def test_large_dense_schedule(idx):
    """A 1000-step decode schedule with n_live uniform on 1..16: every step's
    rows are the 16-slot result's rows gathered by batch_index, bit for bit;
    the 16-slot result matches the oracle on sampled rows."""
    w = wl.WORKLOADS["large_dense"]
    m = w.matrices[idx]
    W, X = wl.workload_inputs("large_dense", idx)
    Wq, Xq = gpu_pack(W), gpu_quantize_acts(X)
    rows = sample_rows(m.N, 96, seed=5 + idx)
    ident = np.arange(16, dtype=np.int32)
    Yo, Ao = _oracle_y(W, X, ident, rows)
    del W
    Y16 = gpu_matmul(Wq, Xq, ident, m.N, m.K)
    ok, worst = within_tau(Y16[:, rows], Yo, Ao)
    assert ok, worst
    import quantized_weight_streaming_q8_amd as q8
    sched = wl.schedule(w.config, steps=1000)
    Y = torch.empty((16, m.N), dtype=torch.float32, device="cuda")
    ref = torch.from_numpy(Y16).cuda()
    bad = torch.zeros((), dtype=torch.int64, device="cuda")
    ws = q8.zeroed_workspace(m.N, m.K)
    for i, bi in enumerate(sched):
        bi_d = to_dev(bi)
        n = bi.size
        if i % 2:  # alternate the two entry points; both must give the same bits
            q8.q8_matmul_narrow_ws(Wq, Xq, bi_d, n, m.N, m.K, Y, ws)
        else:
            q8.q8_matmul_narrow(Wq, Xq, bi_d, n, m.N, m.K, Y)
        bad += (Y[:n].view(torch.int32) != ref[bi_d.long()].view(torch.int32)).sum()
    assert int(bad) == 0
