"""GPU parity of the pos-vector RoPE (q8_rope_multi) through the C ABI: the
rotated values within one fp32 rounding of the oracle's double result
(|delta| <= 2^-23 * (|a| + |b|) for the pair (a, b)), the other columns
untouched bit for bit, and every row bitwise equal to a single-row call."""

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import gpu_matmul, gpu_pack, gpu_quantize_acts, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import quantized_weight_streaming_q8_amd as q8
    assert q8.q8_device_supported(), "device is not gfx950"
    yield
    torch.cuda.synchronize()


def _rope_gpu(Y, pos, n_heads, head_dim, base):
    import quantized_weight_streaming_q8_amd as q8
    Yd = to_dev(np.ascontiguousarray(Y, dtype=np.float32))
    q8.q8_rope_multi(Yd, Y.shape[0], Y.shape[1], to_dev(np.asarray(pos, dtype=np.int32)),
                     n_heads, head_dim, base)
    torch.cuda.synchronize()
    return Yd.cpu().numpy()


def _check(Y, pos, n_heads, head_dim, base):
    out = _rope_gpu(Y, pos, n_heads, head_dim, base)
    ref, mag = oracle.rope(Y, pos, n_heads, head_dim, base)
    w = n_heads * head_dim
    err = np.abs(out[:, :w].astype(np.float64) - ref)
    bound = 2.0 ** -23 * mag + 1e-37
    assert np.all(err <= bound), float(np.max(err / bound))
    assert np.array_equal(out[:, w:].view(np.uint32), Y[:, w:].view(np.uint32))
    return out


@pytest.mark.parametrize("n_rows,stride,n_heads,head_dim,base", [
    (16, 7168, 48, 128, 1e6),      # Qwen3-14B QKV rows: 40 query + 8 key heads, values untouched
    (1, 128, 1, 128, 1e4),
    (3, 2 * 96 + 7, 2, 96, 5e5),
    (64, 512, 4, 64, 1e4),        # 64 rows (multi-column width)
    (5, 10, 5, 2, 1e4),           # one pair per head
])
def test_rope_matches_oracle(n_rows, stride, n_heads, head_dim, base):
    rng = np.random.default_rng(n_rows * 131 + head_dim)
    Y = rng.standard_normal((n_rows, stride), dtype=np.float32) * np.float32(3.0)
    pos = rng.integers(-50, 40000, size=n_rows).astype(np.int32)
    pos[0] = 0
    if n_rows > 2:
        pos[1] = (1 << 20) + 17   # far into a long context
        pos[2] = -(1 << 18)
    _check(Y, pos, n_heads, head_dim, base)


def test_rope_rows_equal_single_row_calls():
    rng = np.random.default_rng(4)
    Y = rng.standard_normal((16, 7168), dtype=np.float32)
    pos = rng.permutation(40000)[:16].astype(np.int32)
    all_rows = _rope_gpu(Y, pos, 48, 128, 1e6)
    for t in range(16):
        one = _rope_gpu(Y[t:t + 1], pos[t:t + 1], 48, 128, 1e6)
        assert np.array_equal(all_rows[t].view(np.uint32), one[0].view(np.uint32)), t
    for n in (3, 9):
        part = _rope_gpu(Y[:n], pos[:n], 48, 128, 1e6)
        assert np.array_equal(part.view(np.uint32), all_rows[:n].view(np.uint32)), n


def test_rope_after_the_qkv_matmul():
    """The QKV projection of the Qwen3 layer for 16 live tokens, then RoPE on
    its query and key heads with each token's own position."""
    w = wl.WORKLOADS["qwen3_layer"]
    m = w.matrices[0]
    assert m.name == "qkv" and m.N == 7168
    W = wl.weights(w.config, 0, m.N, m.K)
    X = wl.activations(w.config, m.K, outliers=w.outliers)
    bi = wl.batch_index(w.config, 16, random=True)
    Y = gpu_matmul(gpu_pack(W), gpu_quantize_acts(X), bi, m.N, m.K)
    pos = np.arange(1000, 1016, dtype=np.int32) * 37
    _check(Y, pos, 48, 128, 1e6)
