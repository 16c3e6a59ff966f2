"""Python binding of libq8narrow.so, the narrow-batch q8_0 decode matmul for
MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/q8narrow.h``; torch supplies
device memory and the current stream.  The functions keep the C names and
raise ``Q8Error`` on a non-OK status.  There is no fallback: if the library
is not built, importing this package raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

from . import build as _build

LIB_PATH = _build.LIB_PATH

Q8_BLOCK = 32
Q8_MAX_SLOTS = 16
Q8_MAX_COLUMNS = 64

Q8_OK = 0
Q8_ERR_INVALID_ARG = 1
Q8_ERR_UNSUPPORTED = 2
Q8_ERR_HIP = 3
Q8_ERR_TOO_LARGE = 4
Q8_NOALLOC_SCRATCH_BYTES = 8 << 20

Q8_PATH_AUTO = 0
Q8_PATH_MFMA = 1
Q8_PATH_DOT4 = 2

# Every symbol the header declares, with its ctypes signature.
_vp, _i64, _i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
_SIGNATURES = {
    "q8_packed_weight_bytes": ([_i64, _i64], ctypes.c_size_t),
    "q8_act_buffer_bytes": ([_i64], ctypes.c_size_t),
    "q8_pack_weights": ([_vp, _i64, _i64, _vp, _vp], _i32),
    "q8_pack_weights_q": ([_vp, _vp, _i64, _i64, _vp, _vp], _i32),
    "q8_unpack_weights": ([_vp, _i64, _i64, _vp, _vp, _vp], _i32),
    "q8_quantize_acts": ([_vp, _i32, _i64, _vp, _vp], _i32),
    "q8_matmul_narrow": ([_vp, _vp, _vp, _i32, _i64, _i64, _vp, _vp], _i32),
    "q8_matmul_narrow_path": ([_vp, _vp, _vp, _i32, _i64, _i64, _vp, _vp, _i32], _i32),
    "q8_matmul_workspace_bytes": ([_i64, _i64], ctypes.c_size_t),
    "q8_matmul_narrow_ws": ([_vp, _vp, _vp, _i32, _i64, _i64, _vp, _vp, ctypes.c_size_t, _vp], _i32),
    "q8_matmul_narrow_noalloc": ([_vp, _vp, _vp, _i32, _i64, _i64, _vp, _vp], _i32),
    "q8_matmul_fused_workspace_bytes": ([_i64, _i64], ctypes.c_size_t),
    "q8_matmul_narrow_fused": ([_vp, _vp, _i32, _vp, _vp, _i32, _i64, _i64, _vp, _vp,
                                ctypes.c_size_t, _vp], _i32),
    "q8_act_buffer_bytes_n": ([_i64, _i32], ctypes.c_size_t),
    "q8_quantize_acts_n": ([_vp, _i32, _i64, _vp, _i32, _vp], _i32),
    "q8_matmul_multi": ([_vp, _vp, _i32, _vp, _i32, _i64, _i64, _vp, _vp], _i32),
    "q8_rope_multi": ([_vp, _i32, _i64, _vp, _i32, _i32, ctypes.c_double, _vp], _i32),
    "q8_stream_read": ([_vp, ctypes.c_size_t, _vp, _vp], _i32),
    "q8_device_supported": ([], _i32),
    "q8_status_str": ([_i32], ctypes.c_char_p),
}


class Q8Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)}")


def _load_library():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
            "or `python quantized_weight_streaming_q8_amd/build.py` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (args, res) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = _load_library()


def library() -> ctypes.CDLL:
    return _lib


# ------------------------------------------------------------------ helpers

def _ptr(x) -> int | None:
    """Device address of a tensor (or an int address, or None for NULL)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, torch.Tensor):
        if not x.is_cuda:
            raise ValueError("expected a device tensor")
        if not x.is_contiguous():
            raise ValueError("expected a contiguous tensor")
        return x.data_ptr()
    raise TypeError(f"cannot pass {type(x).__name__} as a device pointer")


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(rc: int, where: str) -> None:
    if rc != Q8_OK:
        raise Q8Error(rc, where)


def status_str(status: int) -> str:
    return _lib.q8_status_str(int(status)).decode()


# ----------------------------------------------------------------- the ABI

def q8_packed_weight_bytes(N: int, K: int) -> int:
    return int(_lib.q8_packed_weight_bytes(N, K))


def q8_act_buffer_bytes(K: int) -> int:
    return int(_lib.q8_act_buffer_bytes(K))


def q8_pack_weights(W, N: int, K: int, Wq, stream=None) -> None:
    _check(_lib.q8_pack_weights(_ptr(W), N, K, _ptr(Wq), _stream(stream)),
           "q8_pack_weights")


def q8_pack_weights_q(q, d16, N: int, K: int, Wq, stream=None) -> None:
    _check(_lib.q8_pack_weights_q(_ptr(q), _ptr(d16), N, K, _ptr(Wq), _stream(stream)),
           "q8_pack_weights_q")


def q8_unpack_weights(Wq, N: int, K: int, q, d16, stream=None) -> None:
    _check(_lib.q8_unpack_weights(_ptr(Wq), N, K, _ptr(q), _ptr(d16), _stream(stream)),
           "q8_unpack_weights")


def q8_quantize_acts(X, n_rows: int, K: int, Xq, stream=None) -> None:
    _check(_lib.q8_quantize_acts(_ptr(X), n_rows, K, _ptr(Xq), _stream(stream)),
           "q8_quantize_acts")


def q8_matmul_narrow(Wq, Xq, batch_index, n_live: int, N: int, K: int, Y,
                     stream=None) -> None:
    _check(_lib.q8_matmul_narrow(_ptr(Wq), _ptr(Xq), _ptr(batch_index), n_live,
                                 N, K, _ptr(Y), _stream(stream)),
           "q8_matmul_narrow")


def q8_matmul_narrow_path(Wq, Xq, batch_index, n_live: int, N: int, K: int, Y,
                          path: int, stream=None) -> None:
    _check(_lib.q8_matmul_narrow_path(_ptr(Wq), _ptr(Xq), _ptr(batch_index), n_live,
                                      N, K, _ptr(Y), _stream(stream), int(path)),
           "q8_matmul_narrow_path")


def q8_matmul_workspace_bytes(N: int, K: int) -> int:
    return int(_lib.q8_matmul_workspace_bytes(N, K))


def q8_matmul_narrow_ws(Wq, Xq, batch_index, n_live: int, N: int, K: int, Y,
                        workspace, workspace_bytes: int | None = None,
                        stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.q8_matmul_narrow_ws(_ptr(Wq), _ptr(Xq), _ptr(batch_index), n_live, N, K,
                                    _ptr(Y), _ptr(workspace), workspace_bytes, _stream(stream)),
           "q8_matmul_narrow_ws")


def q8_matmul_narrow_noalloc(Wq, Xq, batch_index, n_live: int, N: int, K: int, Y,
                             stream=None) -> None:
    _check(_lib.q8_matmul_narrow_noalloc(_ptr(Wq), _ptr(Xq), _ptr(batch_index), n_live, N, K,
                                         _ptr(Y), _stream(stream)),
           "q8_matmul_narrow_noalloc")


def q8_matmul_fused_workspace_bytes(N: int, K: int) -> int:
    return int(_lib.q8_matmul_fused_workspace_bytes(N, K))


def q8_matmul_narrow_fused(Wq, X, n_rows: int, Xq, batch_index, n_live: int, N: int, K: int,
                           Y, workspace, workspace_bytes: int | None = None,
                           stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.q8_matmul_narrow_fused(_ptr(Wq), _ptr(X), n_rows, _ptr(Xq), _ptr(batch_index),
                                       n_live, N, K, _ptr(Y), _ptr(workspace), workspace_bytes,
                                       _stream(stream)), "q8_matmul_narrow_fused")


def q8_act_buffer_bytes_n(K: int, n_slots: int) -> int:
    return int(_lib.q8_act_buffer_bytes_n(K, n_slots))


def q8_quantize_acts_n(X, n_rows: int, K: int, Xq, n_slots: int, stream=None) -> None:
    _check(_lib.q8_quantize_acts_n(_ptr(X), n_rows, K, _ptr(Xq), n_slots, _stream(stream)),
           "q8_quantize_acts_n")


def q8_matmul_multi(Wq, Xq, n_slots: int, batch_index, n_live: int, N: int, K: int, Y,
                    stream=None) -> None:
    _check(_lib.q8_matmul_multi(_ptr(Wq), _ptr(Xq), n_slots, _ptr(batch_index), n_live, N, K,
                                _ptr(Y), _stream(stream)), "q8_matmul_multi")


def q8_rope_multi(Y, n_rows: int, row_stride: int, pos, n_heads: int, head_dim: int,
                  base: float, stream=None) -> None:
    _check(_lib.q8_rope_multi(_ptr(Y), n_rows, row_stride, _ptr(pos), n_heads, head_dim,
                              float(base), _stream(stream)), "q8_rope_multi")


def q8_stream_read(buf, nbytes: int, sink, stream=None) -> None:
    _check(_lib.q8_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(stream)), "q8_stream_read")


def q8_device_supported() -> bool:
    return bool(_lib.q8_device_supported())


# ------------------------------------------------- torch allocation helpers

def empty_packed_weights(N: int, K: int, device="cuda") -> torch.Tensor:
    nbytes = q8_packed_weight_bytes(N, K)
    if nbytes == 0:
        raise ValueError(f"invalid shape N={N} K={K}")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def zeroed_workspace(N: int, K: int, device="cuda") -> torch.Tensor | None:
    """A zero-filled workspace for q8_matmul_narrow_ws (None if the shape
    needs none)."""
    nbytes = q8_matmul_workspace_bytes(N, K)
    if nbytes == 0:
        return None
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def zeroed_fused_workspace(N: int, K: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace for q8_matmul_narrow_fused."""
    nbytes = q8_matmul_fused_workspace_bytes(N, K)
    if nbytes == 0:
        raise ValueError(f"invalid shape N={N} K={K}")
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def empty_act_slots(K: int, device="cuda", n_slots: int = Q8_MAX_SLOTS) -> torch.Tensor:
    nbytes = q8_act_buffer_bytes_n(K, n_slots)
    if nbytes == 0:
        raise ValueError(f"invalid K={K} or n_slots={n_slots}")
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def read_act_slots(Xq: torch.Tensor, K: int, stream=None, n_slots: int = Q8_MAX_SLOTS):
    """All slots of a slot buffer in canonical q8_0 form:
    (q int8 [n_slots][K], d16 int16 [n_slots][K/32]) device tensors."""
    q = torch.empty((n_slots, K), dtype=torch.int8, device=Xq.device)
    d = torch.empty((n_slots, K // Q8_BLOCK), dtype=torch.int16, device=Xq.device)
    q8_unpack_weights(Xq, n_slots, K, q, d, stream)
    return q, d


def write_act_slots(Xq: torch.Tensor, K: int, q: torch.Tensor, d16: torch.Tensor,
                    stream=None, n_slots: int = Q8_MAX_SLOTS) -> None:
    """Write all slots from canonical q8_0 (q int8 [n_slots][K], d16 int16
    [n_slots][K/32] binary16 bits)."""
    q8_pack_weights_q(q, d16, n_slots, K, Xq, stream)
