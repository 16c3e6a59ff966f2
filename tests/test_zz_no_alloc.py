"""q8_matmul_narrow_noalloc: the split workspace in the library's static
device array instead of a caller's buffer.  Its output must be bit-identical
to q8_matmul_narrow_ws on the same arguments, call after call on the shared
array, with the second call on a smaller shape than the first; and within
the parity tolerance of the oracle."""

import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import gpu_pack, gpu_quantize_acts, q8, sample_rows, to_dev, within_tau

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _inputs(N, K, seed):
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    X = rng.standard_normal((16, K), dtype=np.float32)
    return W, X, gpu_pack(W), gpu_quantize_acts(X)


def _both(Wq, Xq, bi, N, K):
    m = q8()
    bi_d = to_dev(np.asarray(bi, dtype=np.int32))
    n = bi_d.numel()
    Yn = torch.full((n, N), float("nan"), dtype=torch.float32, device="cuda")
    Yw = torch.full((n, N), float("nan"), dtype=torch.float32, device="cuda")
    m.q8_matmul_narrow_noalloc(Wq, Xq, bi_d, n, N, K, Yn)
    ws = m.zeroed_workspace(N, K)
    m.q8_matmul_narrow_ws(Wq, Xq, bi_d, n, N, K, Yw, ws)
    torch.cuda.synchronize()
    return Yn.cpu().numpy(), Yw.cpu().numpy()


def _oracle_rows(W, X, bi, rows):
    import oracle
    qw, dw = oracle.quantize_rows(W[rows])
    qx, dx = oracle.quantize_rows(X)
    return oracle.matmul(qw, dw, qx, dx, np.asarray(bi, dtype=np.int32))


def test_noalloc_equals_workspace_entry_point_on_two_calls():
    """A Qwen3-14B down projection (17408 -> 5120, 16 live tokens), then a
    smaller split shape (8448 -> 1000, 3 live tokens) on the same array."""
    m = q8()
    rng = np.random.default_rng(2024)
    cases = [(5120, 17408, rng.permutation(16).astype(np.int32)),
             (1000, 8448, rng.permutation(16)[:3].astype(np.int32))]
    sizes = [m.q8_matmul_workspace_bytes(N, K) for N, K, _ in cases]
    assert 0 < sizes[1] < sizes[0] <= m.Q8_NOALLOC_SCRATCH_BYTES
    for i, (N, K, bi) in enumerate(cases):
        W, X, Wq, Xq = _inputs(N, K, seed=100 + i)
        Yn, Yw = _both(Wq, Xq, bi, N, K)
        assert np.array_equal(Yn.view(np.uint32), Yw.view(np.uint32)), (N, K)
        rows = sample_rows(N, 64, seed=i)
        Yo, Ao = _oracle_rows(W, X, bi, rows)
        ok, worst = within_tau(Yn[:, rows], Yo, Ao)
        assert ok, (N, K, worst)


def test_noalloc_repeated_and_unsplit_shapes():
    """Calls on split and unsplit shapes in turn, each with its own live
    batch, keep giving the workspace entry point's bits."""
    rng = np.random.default_rng(77)
    # split, unsplit, split, unsplit, and two shapes whose last 64 / 100 row
    # groups are split (1088 and 1124 row groups)
    mats = [(40, 17408), (2304, 5120), (600, 9024), (17, 288), (17405, 1056), (17981, 2080)]
    data = [(N, K) + _inputs(N, K, seed=300 + j)[2:] for j, (N, K) in enumerate(mats)]
    for rep, j in enumerate((0, 1, 4, 2, 3, 5, 2, 0, 4)):
        N, K, Wq, Xq = data[j]
        bi = rng.permutation(16)[: 1 + (rep * 5) % 16].astype(np.int32)
        Yn, Yw = _both(Wq, Xq, bi, N, K)
        assert np.array_equal(Yn.view(np.uint32), Yw.view(np.uint32)), (rep, N, K)


def test_noalloc_qwen3_down_every_live_batch():
    """The workload's down projection at every live batch 1..16 with the
    seeded random batch_index, each call against the workspace entry point."""
    w = wl.WORKLOADS["qwen3_layer"]
    i = [k for k, mm in enumerate(w.matrices) if mm.name == "down"][0]
    mm = w.matrices[i]
    W = wl.weights(w.config, i, mm.N, mm.K)
    X = wl.activations(w.config, mm.K, outliers=w.outliers)
    Wq, Xq = gpu_pack(W), gpu_quantize_acts(X)
    for n in range(1, 17):
        bi = wl.batch_index(w.config, n, random=True)
        Yn, Yw = _both(Wq, Xq, bi, mm.N, mm.K)
        assert np.array_equal(Yn.view(np.uint32), Yw.view(np.uint32)), n
