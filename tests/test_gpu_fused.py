"""GPU parity of the fused pre-quantise + matmul entry point: the slot buffer
and Y bit-identical to q8_quantize_acts followed by q8_matmul_narrow_ws, on
ragged and model-shaped matrices (the long-K ones split across workgroups),
over repeated calls with new activations on the same buffers (the slots and
the counters are rearmed every time), and against the oracle."""

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import gpu_pack, sample_rows, split_counters_clear, to_dev, within_tau

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
    if n > 3:
        X[3, :64] = 0.0
    return X


def _counters_clear(ws, N, K):
    """The fused counters and flags (the first 64 KB, but the timeout word)
    and, for split shapes, every row block's split counter are back to zero;
    the partial sums may hold anything."""
    t = _q8().Q8_FUSED_TIMEOUTS_OFFSET
    if ws[:t].any() or ws[t + 4:65536].any():
        return False
    if _q8().q8_matmul_workspace_bytes(N, K) > 0:
        return split_counters_clear(ws, N, K, offset=65536)
    return True


def _separate(Wq, X, Xq, bi, N, K):
    """q8_quantize_acts then q8_matmul_narrow_ws: (Y, slot buffer bytes)."""
    q8 = _q8()
    q8.q8_quantize_acts(to_dev(X), X.shape[0], K, Xq)
    bi_d = to_dev(bi)
    Y = torch.empty((bi.size, N), dtype=torch.float32, device="cuda")
    q8.q8_matmul_narrow_ws(Wq, Xq, bi_d, bi.size, N, K, Y, q8.zeroed_workspace(N, K))
    torch.cuda.synchronize()
    return Y.cpu().numpy(), Xq.cpu().numpy()


def _fused(Wq, X, Xq, bi, N, K, ws):
    q8 = _q8()
    bi_d = to_dev(bi)
    Y = torch.empty((bi.size, N), dtype=torch.float32, device="cuda")
    q8.q8_matmul_narrow_fused(Wq, to_dev(X), X.shape[0], Xq, bi_d, bi.size, N, K, Y, ws)
    torch.cuda.synchronize()
    return Y.cpu().numpy(), Xq.cpu().numpy()


@pytest.mark.parametrize("N,K", [(1, 32), (17, 288), (100, 800), (33, 4128), (40, 17408),
                                 (768, 768), (1000, 5120), (5120, 2080), (7168, 5120),
                                 (5120, 17408), (17405, 1056), (17981, 2080), (17500, 768)])
def test_fused_equals_quantize_then_matmul(N, K):
    q8 = _q8()
    rng = np.random.default_rng(N + 3 * K)
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    Wq = gpu_pack(W)
    ws = q8.zeroed_fused_workspace(N, K)
    for n_rows, bi in ((16, rng.permutation(16)), (5, np.array([4, 0, 0, 2])),
                       (16, rng.permutation(16)[:7])):
        X = _x(n_rows, K, seed=int(bi.sum()) + n_rows)
        bi = bi.astype(np.int32)
        base = rng.integers(0, 256, q8.q8_act_buffer_bytes(K), dtype=np.uint8)  # prior slot contents
        Xa = to_dev(base)
        Xb = to_dev(base)
        Ys, slots_s = _separate(Wq, X, Xa, bi, N, K)
        Yf, slots_f = _fused(Wq, X, Xb, bi, N, K, ws)
        assert np.array_equal(slots_s, slots_f), (N, K, n_rows)
        assert np.array_equal(Ys.view(np.uint32), Yf.view(np.uint32)), (N, K, n_rows)
        assert _counters_clear(ws, N, K)


def test_fused_repeated_calls_see_new_activations():
    """Calls in a row on the same slot buffer and workspace, each with new
    activations: every call's outputs follow its own inputs."""
    q8 = _q8()
    N, K = 5120, 5120
    rng = np.random.default_rng(71)
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    Wq = gpu_pack(W)
    ws = q8.zeroed_fused_workspace(N, K)
    Xq = q8.empty_act_slots(K)
    rows = sample_rows(N, 40, seed=3)
    qw, dw = oracle.quantize_rows(W[rows])
    for rep in range(4):
        X = _x(16, K, seed=100 + rep)
        bi = rng.permutation(16)[: 4 + 4 * rep].astype(np.int32)
        Y, _ = _fused(Wq, X, Xq, bi, N, K, ws)
        qx, dx = oracle.quantize_rows(X)
        Yo, Ao = oracle.matmul(qw, dw, qx, dx, bi)
        ok, worst = within_tau(Y[:, rows], Yo, Ao)
        assert ok, (rep, worst)


def test_fused_qwen3_layer():
    """The Qwen3-14B-shaped layer through the fused entry point, n_live=16,
    seeded random batch_index: sampled rows against the oracle."""
    q8 = _q8()
    w = wl.WORKLOADS["qwen3_layer"]
    bi = wl.batch_index(w.config, 16, random=True)
    for i, m in enumerate(w.matrices):
        W = wl.weights(w.config, i, m.N, m.K)
        X = wl.activations(w.config, m.K, outliers=w.outliers)
        Wq = gpu_pack(W)
        Y, _ = _fused(Wq, X, q8.empty_act_slots(m.K), bi, m.N, m.K,
                      q8.zeroed_fused_workspace(m.N, m.K))
        rows = sample_rows(m.N, 48, seed=i)
        qw, dw = oracle.quantize_rows(W[rows])
        qx, dx = oracle.quantize_rows(X)
        Yo, Ao = oracle.matmul(qw, dw, qx, dx, bi)
        ok, worst = within_tau(Y[:, rows], Yo, Ao)
        assert ok, (m.name, worst)
        del Wq
        torch.cuda.empty_cache()


def test_fused_graph_replays():
    """Fused calls captured in a HIP graph: every replay, with new
    activations copied in between, matches the eager call."""
    q8 = _q8()
    N, K = 7168, 5120
    rng = np.random.default_rng(5)
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    Wq = gpu_pack(W)
    ws = q8.zeroed_fused_workspace(N, K)
    Xq = q8.empty_act_slots(K)
    Xd = torch.empty((16, K), dtype=torch.float32, device="cuda")
    bi = to_dev(rng.permutation(16).astype(np.int32))
    Y = torch.empty((16, N), dtype=torch.float32, device="cuda")
    Xd.copy_(to_dev(_x(16, K, seed=1)))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        q8.q8_matmul_narrow_fused(Wq, Xd, 16, Xq, bi, 16, N, K, Y, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q8.q8_matmul_narrow_fused(Wq, Xd, 16, Xq, bi, 16, N, K, Y, ws)
    for rep in range(4):
        X = _x(16, K, seed=20 + rep)
        Xd.copy_(to_dev(X))
        g.replay()
        torch.cuda.synchronize()
        got = Y.clone()
        q8.q8_matmul_narrow_fused(Wq, Xd, 16, Xq, bi, 16, N, K, Y, ws)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int32), Y.view(torch.int32)), rep
        assert _counters_clear(ws, N, K)


@pytest.mark.parametrize("N,K", [(100, 800), (40, 17408), (5120, 5120), (5120, 17408)])
def test_fused_wait_that_runs_out_is_loud(N, K):
    """Forced from the host: no quantising workgroups and a small bound on
    the wait.  Every kernel finishes, every output row is quiet NaN, the
    workspace's timeout word counts the matmul workgroups, the counters are
    rearmed, and the next normal call on the same workspace is right."""
    q8 = _q8()
    rng = np.random.default_rng(N + K)
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    Wq = gpu_pack(W)
    ws = q8.zeroed_fused_workspace(N, K)
    X = _x(16, K, seed=7)
    Xd = to_dev(X)
    Xq = q8.empty_act_slots(K)
    bi = rng.permutation(16)[:9].astype(np.int32)
    bi_d = to_dev(bi)
    counts = []
    for rep in range(2):
        Y = torch.zeros((bi.size, N), dtype=torch.float32, device="cuda")
        q8.q8_matmul_narrow_fused_bounded(Wq, Xd, 16, Xq, bi_d, bi.size, N, K, Y, ws,
                                          max_spins=8, quantize=0)
        torch.cuda.synchronize()
        assert torch.isnan(Y).all(), rep
        assert _counters_clear(ws, N, K), rep
        counts.append(q8.fused_timeouts(ws))
    assert counts[0] >= 1 and counts[1] == 2 * counts[0], counts
    assert not Xq.any(), "no slot may be written without quantising workgroups"
    Ys, slots_s = _separate(Wq, X, q8.empty_act_slots(K), bi, N, K)
    Yf, slots_f = _fused(Wq, X, Xq, bi, N, K, ws)
    assert np.array_equal(slots_s, slots_f)
    assert np.array_equal(Ys.view(np.uint32), Yf.view(np.uint32))
    assert _counters_clear(ws, N, K)
    assert q8.fused_timeouts(ws) == counts[1], "a normal call adds no timeout"


def test_fused_bounded_with_quantisation_is_the_fused_call():
    """quantize = 1 with a generous bound is q8_matmul_narrow_fused."""
    q8 = _q8()
    N, K = 1000, 5120
    rng = np.random.default_rng(3)
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    Wq = gpu_pack(W)
    X = _x(16, K, seed=9)
    bi = rng.permutation(16)[:11].astype(np.int32)
    Yf, slots_f = _fused(Wq, X, q8.empty_act_slots(K), bi, N, K, q8.zeroed_fused_workspace(N, K))
    ws = q8.zeroed_fused_workspace(N, K)
    Xq = q8.empty_act_slots(K)
    Y = torch.empty((bi.size, N), dtype=torch.float32, device="cuda")
    q8.q8_matmul_narrow_fused_bounded(Wq, to_dev(X), 16, Xq, to_dev(bi), bi.size, N, K, Y, ws,
                                      max_spins=1 << 22, quantize=1)
    torch.cuda.synchronize()
    assert np.array_equal(Y.cpu().numpy().view(np.uint32), Yf.view(np.uint32))
    assert np.array_equal(Xq.cpu().numpy(), slots_f)
    assert q8.fused_timeouts(ws) == 0
