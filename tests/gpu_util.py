"""Helpers for the GPU tests: run the HIP path through the C ABI and compare
with the CPU oracle.  Inputs come from ``workloads`` (seeded, synthetic)."""

from __future__ import annotations

import numpy as np
import torch

BLOCK = 32


def q8():
    import quantized_weight_streaming_q8_amd as m
    return m


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def gpu_pack(W: np.ndarray) -> torch.Tensor:
    m = q8()
    N, K = W.shape
    Wd = to_dev(W.astype(np.float32))
    Wq = m.empty_packed_weights(N, K)
    m.q8_pack_weights(Wd, N, K, Wq)
    del Wd
    return Wq


def gpu_pack_q(q: np.ndarray, d16: np.ndarray) -> torch.Tensor:
    m = q8()
    N, K = q.shape
    Wq = m.empty_packed_weights(N, K)
    m.q8_pack_weights_q(to_dev(q.astype(np.int8)), to_dev(d16.astype(np.uint16).view(np.int16)),
                        N, K, Wq)
    return Wq


def gpu_unpack(Wq: torch.Tensor, N: int, K: int):
    m = q8()
    q = torch.empty((N, K), dtype=torch.int8, device="cuda")
    d = torch.empty((N, K // BLOCK), dtype=torch.int16, device="cuda")
    m.q8_unpack_weights(Wq, N, K, q, d)
    torch.cuda.synchronize()
    return q.cpu().numpy(), d.cpu().numpy().view(np.uint16)


def gpu_quantize_acts(X: np.ndarray, Xq: torch.Tensor | None = None) -> torch.Tensor:
    m = q8()
    R, K = X.shape
    if Xq is None:
        Xq = m.empty_act_slots(K)
    m.q8_quantize_acts(to_dev(X.astype(np.float32)), R, K, Xq)
    return Xq


def slots_host(Xq: torch.Tensor, K: int):
    """(q int8 [16][K], d16 uint16 [16][K/32]) of every slot, read back
    through the library's unpack kernel."""
    q, d = q8().read_act_slots(Xq, K)
    torch.cuda.synchronize()
    return q.cpu().numpy(), d.cpu().numpy().view(np.uint16)


def write_slots(Xq: torch.Tensor, K: int, q: np.ndarray, d16: np.ndarray) -> None:
    """Write all 16 slots from canonical q8_0 arrays."""
    q8().write_act_slots(Xq, K, to_dev(q.astype(np.int8)),
                         to_dev(d16.astype(np.uint16).view(np.int16)))
    torch.cuda.synchronize()


def gpu_matmul(Wq, Xq, bi: np.ndarray, N: int, K: int, path: int = 0) -> np.ndarray:
    m = q8()
    bi_d = to_dev(np.asarray(bi, dtype=np.int32))
    Y = torch.empty((bi_d.numel(), N), dtype=torch.float32, device="cuda")
    m.q8_matmul_narrow_path(Wq, Xq, bi_d, bi_d.numel(), N, K, Y, path)
    torch.cuda.synchronize()
    return Y.cpu().numpy()


def gpu_matmul_ws(Wq, Xq, bi: np.ndarray, N: int, K: int, ws) -> np.ndarray:
    """The workspace entry point (split execution) on a given workspace."""
    m = q8()
    bi_d = to_dev(np.asarray(bi, dtype=np.int32))
    Y = torch.empty((bi_d.numel(), N), dtype=torch.float32, device="cuda")
    m.q8_matmul_narrow_ws(Wq, Xq, bi_d, bi_d.numel(), N, K, Y, ws)
    torch.cuda.synchronize()
    return Y.cpu().numpy()


def within_tau(Y: np.ndarray, Yo: np.ndarray, Ao: np.ndarray):
    """|Y - Y_oracle| <= 1e-4 * sum|block terms| + 1e-6, elementwise.
    Returns (ok, worst ratio of error to bound)."""
    Y = Y.astype(np.float64)
    tau = 1e-4 * Ao + 1e-6
    err = np.abs(Y - Yo)
    ratio = np.max(err / tau) if err.size else 0.0
    return bool(np.all(err <= tau)), float(ratio)


def sample_rows(N: int, n: int, seed: int) -> np.ndarray:
    """First, last, the last row group and random rows in between."""
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 15, 16, N - 1, N - 2, N - 16, N - 17]
    rest = rng.choice(N, size=min(N, n), replace=False)
    rows = np.unique(np.clip(np.concatenate([fixed, rest]), 0, N - 1))
    return rows.astype(np.int64)


RECORD_BYTES = 256 + 4 * 1024  # counter line + room for 4 partial 16x16 fp32 tiles


def split_counters_clear(ws, N: int, K: int, offset: int = 0) -> bool:
    """True if every split row block's arrival counter in a split workspace
    (from byte `offset` on) is zero.  The workspace is one record of
    RECORD_BYTES per row block of 16 rows that runs as split workgroups,
    each starting with its counter's 256-byte line."""
    nbytes = q8().q8_matmul_workspace_bytes(N, K)
    n_rec = nbytes // RECORD_BYTES
    assert n_rec * RECORD_BYTES == nbytes and 1 <= n_rec <= -(-N // 16)
    heads = ws[offset:offset + nbytes].view(n_rec, RECORD_BYTES)[:, :256]
    return not heads.any()
