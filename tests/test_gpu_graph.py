"""The library's calls captured in a HIP graph (through torch's graph API)
give the eager results on every replay, with eager work and synchronisation
between replays.  Nothing the library enqueues is a memset."""

import numpy as np
import pytest
import torch

from gpu_util import gpu_pack, q8, to_dev

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    m = q8()
    rng = np.random.default_rng(41)
    N, K = 2304, 3072
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    X1 = to_dev(rng.standard_normal((16, K), dtype=np.float32))
    X2 = to_dev(rng.standard_normal((16, K), dtype=np.float32))
    Wq = gpu_pack(W)
    Xq = m.empty_act_slots(K)
    bi = to_dev(np.array([7, 1, 12, 3, 3, 0], dtype=np.int32))
    X = X1.clone()
    Y = torch.empty((6, N), dtype=torch.float32, device="cuda")

    def step():
        m.q8_quantize_acts(X, 16, K, Xq)
        m.q8_matmul_narrow(Wq, Xq, bi, 6, N, K, Y)

    # eager references for both inputs
    refs = []
    for src in (X1, X2):
        X.copy_(src)
        step()
        torch.cuda.synchronize()
        refs.append(Y.clone())
    assert not torch.equal(refs[0], refs[1])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for i in range(6):
        which = i % 2
        X.copy_(X1 if which == 0 else X2)
        Y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int32), refs[which].view(torch.int32)), i
        # eager work between replays, on the same buffers
        X.copy_(X2 if which == 0 else X1)
        step()
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int32), refs[1 - which].view(torch.int32)), i
