"""The timeline build (libq8narrow_timeline.so, include/q8timeline.h) on the
GPU, called through its C ABI next to the product library: the same Y bits,
and one well-formed record per wave of the launch plan (stamps in order, one
last split per split row block, nothing past max_waves)."""

import ctypes

import numpy as np
import pytest
import torch

from gpu_util import gpu_pack, gpu_quantize_acts, q8, to_dev

pytestmark = pytest.mark.gpu

MAX_WAVES = 1 << 16


@pytest.fixture(scope="module")
def tl():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    m = q8()
    from quantized_weight_streaming_q8_amd import build
    lib = ctypes.CDLL(build.TIMELINE_LIB_PATH)
    for name, (args, res) in dict(m._SIGNATURES, **m._TIMELINE_SIGNATURES).items():
        fn = getattr(lib, name)
        fn.argtypes, fn.restype = args, res
    assert lib.q8_device_supported() == 1
    yield lib
    lib.q8_timeline_set(None, 0)
    torch.cuda.synchronize()


def _timeline_ws(tl, Wq, Xq, bi, n, N, K, Y, ws, ws_bytes, rec, max_waves):
    stream = torch.cuda.current_stream().cuda_stream
    assert tl.q8_timeline_set(rec.data_ptr(), max_waves) == 0
    st = tl.q8_matmul_narrow_ws(Wq.data_ptr(), Xq.data_ptr(), bi.data_ptr(), n, N, K,
                                Y.data_ptr(), ws.data_ptr() if ws_bytes else None, ws_bytes,
                                stream)
    assert tl.q8_timeline_set(None, 0) == 0
    assert st == 0
    torch.cuda.synchronize()
    return rec.view(-1, 8).cpu().numpy()


# a split shape (K >= 8192: 4 one-wave workgroups per row group), a small
# single-workgroup tree with a ragged row group, one with many row blocks,
# a balanced one (1152 row groups: 1024 whole-row waves, the last 128 row
# groups as 4 split pieces each) and long rows in 205 four-wave workgroups
@pytest.mark.parametrize("N,K", [(256, 8192), (100, 512), (1040, 2048), (18432, 2048),
                                 (6555, 8224)])
def test_timeline_build_same_bits_and_wellformed_records(tl, N, K):
    m = q8()
    print(f"timeline build N={N} K={K}", flush=True)
    rng = np.random.default_rng(N * 7 + K)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    X = rng.standard_normal((16, K)).astype(np.float32)
    Wq, Xq = gpu_pack(W), gpu_quantize_acts(X)
    bi = to_dev(np.array([5, 0, 11, 3], dtype=np.int32))
    n = 4
    ws_bytes = m.q8_matmul_workspace_bytes(N, K)
    ws1 = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    ws2 = torch.zeros_like(ws1)
    Y1 = torch.full((n, N), 7.0, device="cuda")
    Y2 = torch.full_like(Y1, 7.0)
    m.q8_matmul_narrow_ws(Wq, Xq, bi, n, N, K, Y1, ws1 if ws_bytes else None)
    rec = torch.zeros(MAX_WAVES * 8, dtype=torch.int64, device="cuda")
    torch.cuda.synchronize()
    r = _timeline_ws(tl, Wq, Xq, bi, n, N, K, Y2, ws2, ws_bytes, rec, MAX_WAVES)
    assert torch.equal(Y1.view(torch.int32), Y2.view(torch.int32))

    written = r[:, 0] > 0
    nw = int(written.sum())
    assert nw >= 1 and written[:nw].all() and not written[nw:].any()
    # one record per wave of the launch the plan reports
    plan = m.q8_matmul_launch_info(N, K, 16, ws_bytes > 0)
    assert nw == plan["workgroups"] * plan["waves_per_workgroup"], (nw, plan)
    t = r[:nw]
    for a, b in ((0, 1), (1, 2), (2, 3), (3, 4), (4, 5)):
        assert (t[:, b] >= t[:, a]).all(), (a, b)
    split = ws_bytes > 0
    if split:
        # one last split per split row block (every row block of a long-row
        # shape; only the last G mod 256 of a balanced one)
        last = t[:, 6] > 0
        split_blocks = (plan["workgroups"] - plan["whole_row_workgroups"]) // plan["k_splits"]
        assert int(last.sum()) == split_blocks
        assert (t[last, 6] >= t[last, 5]).all()
    else:
        assert (t[:, 6] == 0).all()
    assert (((t[:, 7] >> 32) & 0xF) < 8).all()
    assert (t[:, 6:7].max(initial=0) if split else t[:, 5].max()) - t[:, 0].min() < 10**8  # < 1 s

    # the counters are back at zero and records stop at max_waves
    if nw > 3:
        rec.zero_()
        r = _timeline_ws(tl, Wq, Xq, bi, n, N, K, Y2, ws2, ws_bytes, rec, 3)
        assert (r[:3, 0] > 0).all() and not (r[3:] != 0).any()
        assert torch.equal(Y1.view(torch.int32), Y2.view(torch.int32))


@pytest.mark.parametrize("N,K,n_slots", [(18432, 2048, 64), (1040, 2048, 32), (6555, 8224, 48)])
def test_timeline_build_multi_column_waves_match_the_plan(tl, N, K, n_slots):
    """The multi-column launch records one wave per wave of the plan and
    gives the product library's bits."""
    m = q8()
    print(f"timeline build multi N={N} K={K} n_slots={n_slots}", flush=True)
    rng = np.random.default_rng(N + K + n_slots)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    X = rng.standard_normal((n_slots, K)).astype(np.float32)
    Wq = gpu_pack(W)
    Xq = m.empty_act_slots(K, n_slots=n_slots)
    m.q8_quantize_acts_n(to_dev(X), n_slots, K, Xq, n_slots)
    bi = to_dev(rng.permutation(n_slots).astype(np.int32))
    Y1 = torch.empty((n_slots, N), dtype=torch.float32, device="cuda")
    Y2 = torch.full_like(Y1, 7.0)
    m.q8_matmul_multi(Wq, Xq, n_slots, bi, n_slots, N, K, Y1)
    rec = torch.zeros(MAX_WAVES * 8, dtype=torch.int64, device="cuda")
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    assert tl.q8_timeline_set(rec.data_ptr(), MAX_WAVES) == 0
    st = tl.q8_matmul_multi(Wq.data_ptr(), Xq.data_ptr(), n_slots, bi.data_ptr(), n_slots, N, K,
                            Y2.data_ptr(), stream)
    assert tl.q8_timeline_set(None, 0) == 0
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(Y1.view(torch.int32), Y2.view(torch.int32))
    r = rec.view(-1, 8).cpu().numpy()
    written = r[:, 0] > 0
    nw = int(written.sum())
    assert written[:nw].all() and not written[nw:].any()
    plan = m.q8_matmul_launch_info(N, K, n_slots)
    assert nw == plan["workgroups"] * plan["waves_per_workgroup"], (nw, plan)
    t = r[:nw]
    for a, b in ((0, 1), (1, 2), (2, 3), (3, 4), (4, 5)):
        assert (t[:, b] >= t[:, a]).all(), (a, b)
