"""Seeded synthetic inputs for the narrow-batch q8_0 decode matmul.

This module only draws random numbers and describes shapes.  It holds none
of the method's arithmetic (no quantisation, no dot products), so that both
the CPU oracle and the HIP path can consume the very same fp32 arrays.

Workloads (the shapes of the pages' models; no weights or datasets are used):

* ``single``      one 768x768 matmul, live batch 1, 2, 4.
* ``llama68m``    the dense stack of a llama-68m-shaped decoder (hidden 768),
                  the model the "[feature] Enable Dynamic Batching" page times
                  (section "Experiment 1"), live batch 1, 2, 4, 8.
* ``qwen3_layer`` one Qwen3-14B-shaped decode layer (hidden 5120), the model
                  of "dynamic public batch (1..16) for Qwen3-14B decode"; a
                  16-slot padded buffer and live batches 1..16 gathered through
                  a seeded random batch_index; 1% of activation channels are
                  outliers scaled by 20.
* ``qwen3_head``  the Qwen3-14B output head 5120 -> 151936, live 1..16.
* ``large_dense`` 7168 -> 18432 and 18432 -> 7168, with a 1000-step schedule
                  whose live batch is uniform on 1..16.

Weights are fp32 N(0, 0.02) [N][K]; activations fp32 N(0, 1) [16][K].  Every
array comes from its own numpy PCG64 stream keyed by
``(0, config, purpose, id)``: purpose 0 = weights (id = matrix index in the
listed order), 1 = activations (id = K), 2 = outlier channels (id = K),
3 = batch_index / schedule (id = live batch, or 0 for the schedule).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

N_SLOTS = 16
WEIGHT_STD = 0.02
OUTLIER_FRACTION = 0.01
OUTLIER_SCALE = 20.0


@dataclass(frozen=True)
class Matrix:
    name: str
    K: int  # input features (reduction length)
    N: int  # output features (rows of W)


@dataclass(frozen=True)
class Workload:
    key: str
    config: int  # seed component
    matrices: tuple
    n_live: tuple
    outliers: bool = False
    random_batch_index: bool = False
    # pos-vector RoPE on the QKV output: (rotated heads, head_dim, base), the
    # query and key heads that lead the QKV rows; None where there is none
    rope: tuple | None = None


WORKLOADS = {
    "single": Workload("single", 1, (Matrix("w", 768, 768),), (1, 2, 4)),
    "llama68m": Workload(
        "llama68m", 2,
        (Matrix("qkv", 768, 2304), Matrix("o", 768, 768),
         Matrix("gate_up", 768, 6144), Matrix("down", 3072, 768),
         Matrix("head", 768, 32000)),
        (1, 2, 4, 8), rope=(24, 64, 1e4)),
    "qwen3_layer": Workload(
        "qwen3_layer", 3,
        (Matrix("qkv", 5120, 7168), Matrix("o", 5120, 5120),
         Matrix("gate_up", 5120, 34816), Matrix("down", 17408, 5120)),
        tuple(range(1, 17)), outliers=True, random_batch_index=True, rope=(48, 128, 1e6)),
    "qwen3_head": Workload(
        "qwen3_head", 4, (Matrix("head", 5120, 151936),), (1, 2, 4, 8, 16)),
    "large_dense": Workload(
        "large_dense", 5,
        (Matrix("up", 7168, 18432), Matrix("down", 18432, 7168)),
        tuple(range(1, 17)), random_batch_index=True),
}


def _rng(config: int, purpose: int, ident: int) -> np.random.Generator:
    return np.random.default_rng([0, int(config), int(purpose), int(ident)])


def weights(config: int, matrix_id: int, N: int, K: int,
            std: float = WEIGHT_STD) -> np.ndarray:
    """fp32 [N][K] weights, N(0, std)."""
    g = _rng(config, 0, matrix_id)
    w = g.standard_normal((N, K), dtype=np.float32)
    w *= np.float32(std)
    return w


def outlier_channels(config: int, K: int,
                     fraction: float = OUTLIER_FRACTION) -> np.ndarray:
    """round(fraction*K) distinct channels, drawn without replacement."""
    n = int(round(fraction * K))
    g = _rng(config, 2, K)
    return np.sort(g.choice(K, size=n, replace=False)).astype(np.int64)


def activations(config: int, K: int, n_slots: int = N_SLOTS,
                outliers: bool = False) -> np.ndarray:
    """fp32 [n_slots][K] activations, N(0, 1); with ``outliers`` the same 1%
    of channels in every slot is multiplied by 20."""
    g = _rng(config, 1, K)
    x = g.standard_normal((n_slots, K), dtype=np.float32)
    if outliers:
        ch = outlier_channels(config, K)
        x[:, ch] *= np.float32(OUTLIER_SCALE)
    return x


def batch_index(config: int, n_live: int, random: bool,
                n_slots: int = N_SLOTS) -> np.ndarray:
    """int32 [n_live] slot indices: identity, or a seeded random prefix of a
    permutation of the slots."""
    if not random:
        return np.arange(n_live, dtype=np.int32)
    g = _rng(config, 3, n_live)
    return g.permutation(n_slots)[:n_live].astype(np.int32)


def schedule(config: int, steps: int = 1000, n_slots: int = N_SLOTS):
    """A decode schedule: ``steps`` batch_index arrays whose live batch is
    uniform on 1..n_slots, each a random prefix of a slot permutation."""
    g = _rng(config, 3, 0)
    out = []
    for _ in range(steps):
        n = int(g.integers(1, n_slots + 1))
        out.append(g.permutation(n_slots)[:n].astype(np.int32))
    return out


def workload_inputs(key: str, matrix: int):
    """(W fp32 [N][K], X fp32 [16][K]) for one matrix of a workload."""
    wl = WORKLOADS[key]
    m = wl.matrices[matrix]
    return (weights(wl.config, matrix, m.N, m.K),
            activations(wl.config, m.K, outliers=wl.outliers))
