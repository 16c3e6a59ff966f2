"""GPU checks of the read-ceiling kernel behind bench.py's read_ceiling
figure: it reads the first and the last 16-byte unit of the buffer (a unit
whose words XOR to the marker makes exactly its reader write its sink entry),
and otherwise writes nothing."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

MAGIC = 0x9E3779B9
GRID_THREADS = 2048 * 256


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import quantized_weight_streaming_q8_amd as q8
    assert q8.q8_device_supported(), "device is not gfx950"
    yield
    torch.cuda.synchronize()


def _read(words: torch.Tensor) -> np.ndarray:
    import quantized_weight_streaming_q8_amd as q8
    sink = torch.full((1024,), -1, dtype=torch.int32, device="cuda")
    q8.q8_stream_read(words, words.numel() * 4, sink)
    torch.cuda.synchronize()
    return sink.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("nbytes", [64 << 20, (64 << 20) + 48])
def test_stream_read_reaches_first_and_last_unit(nbytes):
    n16 = nbytes // 16
    words = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    marker = int(np.uint32(MAGIC).view(np.int32))
    assert (_read(words) == 0xFFFFFFFF).all()   # nothing marked: nothing written
    words[0] = marker                             # the first unit: thread 0 reads it
    s = _read(words)
    assert s[0] == MAGIC and (s[1:] == 0xFFFFFFFF).all()
    words[0] = 0
    words[4 * (n16 - 1) + 2] = marker             # the last unit
    s = _read(words)
    t = ((n16 - 1) % GRID_THREADS) & 1023
    others = np.ones(1024, dtype=bool)
    others[t] = False
    assert s[t] == MAGIC and (s[others] == 0xFFFFFFFF).all()
