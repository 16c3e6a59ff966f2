"""Python binding of libq8narrow.so, the narrow-batch q8_0 decode matmul for
MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/q8narrow.h``; torch supplies
device memory and the current stream.  The functions keep the C names and
raise ``Q8Error`` on a non-OK status.  There is no fallback: if the library
is not built, importing this package raises.

With the environment variable Q8_LIBRARY=timeline set before the first
import, the package loads the timeline build, libq8narrow_timeline.so, instead
(same entry points and results, plus ``q8_timeline_set`` of
``include/q8timeline.h``: per-wave real-time counter records for profiling).
"""

from __future__ import annotations

import ctypes
import os

import torch

from . import build as _build

_VARIANT = os.environ.get("Q8_LIBRARY", "")
if _VARIANT not in ("", "timeline"):
    raise ImportError(f"Q8_LIBRARY={_VARIANT!r}: only 'timeline' (or unset) is known")
TIMELINE = _VARIANT == "timeline"
LIB_PATH = _build.TIMELINE_LIB_PATH if TIMELINE else _build.LIB_PATH

Q8_BLOCK = 32
Q8_MAX_SLOTS = 16
Q8_MAX_COLUMNS = 64

Q8_OK = 0
Q8_ERR_INVALID_ARG = 1
Q8_ERR_UNSUPPORTED = 2
Q8_ERR_HIP = 3
Q8_ERR_TOO_LARGE = 4
Q8_NOALLOC_SCRATCH_BYTES = 8 << 20
Q8_FUSED_TIMEOUTS_OFFSET = 256

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
    "q8_matmul_launch_info": ([_i64, _i64, _i32, _i32, _vp], _i32),
    "q8_matmul_narrow_ws": ([_vp, _vp, _vp, _i32, _i64, _i64, _vp, _vp, ctypes.c_size_t, _vp], _i32),
    "q8_matmul_narrow_noalloc": ([_vp, _vp, _vp, _i32, _i64, _i64, _vp, _vp], _i32),
    "q8_matmul_fused_workspace_bytes": ([_i64, _i64], ctypes.c_size_t),
    "q8_matmul_narrow_fused": ([_vp, _vp, _i32, _vp, _vp, _i32, _i64, _i64, _vp, _vp,
                                ctypes.c_size_t, _vp], _i32),
    "q8_matmul_narrow_fused_bounded": ([_vp, _vp, _i32, _vp, _vp, _i32, _i64, _i64, _vp, _vp,
                                        ctypes.c_size_t, _i32, _i32, _vp], _i32),
    "q8_act_buffer_bytes_n": ([_i64, _i32], ctypes.c_size_t),
    "q8_quantize_acts_n": ([_vp, _i32, _i64, _vp, _i32, _vp], _i32),
    "q8_matmul_multi": ([_vp, _vp, _i32, _vp, _i32, _i64, _i64, _vp, _vp], _i32),
    "q8_rope_multi": ([_vp, _i32, _i64, _vp, _i32, _i32, ctypes.c_double, _vp], _i32),
    "q8_stream_read": ([_vp, ctypes.c_size_t, _vp, _vp], _i32),
    "q8_device_supported": ([], _i32),
    "q8_status_str": ([_i32], ctypes.c_char_p),
}
# The timeline build's own symbol (include/q8timeline.h).
_TIMELINE_SIGNATURES = {
    "q8_timeline_set": ([_vp, _i64], _i32),
}
Q8_STAMP_WORDS = 8


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
    sigs = dict(_SIGNATURES, **(_TIMELINE_SIGNATURES if TIMELINE else {}))
    for name, (args, res) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = _load_library()


def library() -> ctypes.CDLL:
    return _lib


# ------------------------------------------------------------------ helpers

_F32 = (torch.float32,)
_I32 = (torch.int32,)
_I8 = (torch.int8,)
_H16 = (torch.int16, torch.float16)  # binary16 bits
_ANY = None


def _arg(x, name: str, dtypes=_ANY, need_bytes: int = 0):
    """First check of argument `name` for the C ABI: a tensor's dtype (when
    the argument has one), that it holds at least `need_bytes` bytes (0: no
    size check, e.g. when the shape itself is invalid and the library will
    reject the call) and that it is contiguous.  An int is a raw device
    address and None is NULL; both pass unchecked (the library's own host
    checks still apply).  Returns (name, x) for _dev."""
    if x is None or isinstance(x, int):
        return name, x
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name}: cannot pass {type(x).__name__} as a device pointer")
    if dtypes is not None and x.dtype not in dtypes:
        want = " or ".join(str(d).replace("torch.", "") for d in dtypes)
        raise ValueError(f"{name}: expected {want}, got {str(x.dtype).replace('torch.', '')}")
    have = x.numel() * x.element_size()
    if have < need_bytes:
        raise ValueError(f"{name}: holds {have} bytes, the call needs at least {need_bytes}")
    if not x.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    return name, x


def _dev(*checked):
    """Second check, once every argument has passed _arg: each tensor lives
    on the current device.  Returns the device addresses, in order."""
    out = []
    for name, x in checked:
        if isinstance(x, torch.Tensor):
            if not x.is_cuda:
                raise ValueError(f"{name}: expected a device tensor, got one on {x.device}")
            if x.device.index != torch.cuda.current_device():
                raise ValueError(f"{name}: on {x.device}, but the current device is "
                                 f"cuda:{torch.cuda.current_device()}")
            x = x.data_ptr()
        out.append(x)
    return out


def _ptr(x) -> int | None:
    """Device address of a tensor (or an int address, or None for NULL)."""
    return _dev(_arg(x, "argument"))[0]


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


def _n(count: int, size: int) -> int:
    """Bytes of `count` elements of `size` bytes (0 for a non-positive count,
    which the library rejects itself)."""
    return count * size if count > 0 else 0


# ----------------------------------------------------------------- the ABI

def q8_packed_weight_bytes(N: int, K: int) -> int:
    return int(_lib.q8_packed_weight_bytes(N, K))


def q8_act_buffer_bytes(K: int) -> int:
    return int(_lib.q8_act_buffer_bytes(K))


def q8_pack_weights(W, N: int, K: int, Wq, stream=None) -> None:
    w, wq = _dev(_arg(W, "W", _F32, _n(N * K, 4)),
                 _arg(Wq, "Wq", _ANY, q8_packed_weight_bytes(N, K)))
    _check(_lib.q8_pack_weights(w, N, K, wq, _stream(stream)), "q8_pack_weights")


def q8_pack_weights_q(q, d16, N: int, K: int, Wq, stream=None) -> None:
    qq, dd, wq = _dev(_arg(q, "q", _I8, _n(N * K, 1)),
                      _arg(d16, "d16", _H16, _n(N * (K // Q8_BLOCK), 2)),
                      _arg(Wq, "Wq", _ANY, q8_packed_weight_bytes(N, K)))
    _check(_lib.q8_pack_weights_q(qq, dd, N, K, wq, _stream(stream)), "q8_pack_weights_q")


def q8_unpack_weights(Wq, N: int, K: int, q, d16, stream=None) -> None:
    wq, qq, dd = _dev(_arg(Wq, "Wq", _ANY, q8_packed_weight_bytes(N, K)),
                      _arg(q, "q", _I8, _n(N * K, 1)),
                      _arg(d16, "d16", _H16, _n(N * (K // Q8_BLOCK), 2)))
    _check(_lib.q8_unpack_weights(wq, N, K, qq, dd, _stream(stream)), "q8_unpack_weights")


def q8_quantize_acts(X, n_rows: int, K: int, Xq, stream=None) -> None:
    x, xq = _dev(_arg(X, "X", _F32, _n(n_rows * K, 4)),
                 _arg(Xq, "Xq", _ANY, q8_act_buffer_bytes(K)))
    _check(_lib.q8_quantize_acts(x, n_rows, K, xq, _stream(stream)), "q8_quantize_acts")


def _mm_checked(Wq, Xq, batch_index, n_live: int, N: int, K: int, Y, xq_bytes: int | None = None):
    return [_arg(Wq, "Wq", _ANY, q8_packed_weight_bytes(N, K)),
            _arg(Xq, "Xq", _ANY, q8_act_buffer_bytes(K) if xq_bytes is None else xq_bytes),
            _arg(batch_index, "batch_index", _I32, _n(n_live, 4)),
            _arg(Y, "Y", _F32, _n(n_live * N, 4))]


def q8_matmul_narrow(Wq, Xq, batch_index, n_live: int, N: int, K: int, Y,
                     stream=None) -> None:
    wq, xq, bi, y = _dev(*_mm_checked(Wq, Xq, batch_index, n_live, N, K, Y))
    _check(_lib.q8_matmul_narrow(wq, xq, bi, n_live, N, K, y, _stream(stream)), "q8_matmul_narrow")


def q8_matmul_narrow_path(Wq, Xq, batch_index, n_live: int, N: int, K: int, Y,
                          path: int, stream=None) -> None:
    wq, xq, bi, y = _dev(*_mm_checked(Wq, Xq, batch_index, n_live, N, K, Y))
    _check(_lib.q8_matmul_narrow_path(wq, xq, bi, n_live, N, K, y, _stream(stream), int(path)),
           "q8_matmul_narrow_path")


def q8_matmul_workspace_bytes(N: int, K: int) -> int:
    return int(_lib.q8_matmul_workspace_bytes(N, K))


class _LaunchInfo(ctypes.Structure):
    _fields_ = [("row_groups_per_wave", ctypes.c_int32), ("column_tiles", ctypes.c_int32),
                ("chunks_in_flight", ctypes.c_int32), ("k_splits", ctypes.c_int32),
                ("slices_per_split", ctypes.c_int32), ("split_workgroups", ctypes.c_int32),
                ("whole_row_workgroups", ctypes.c_int32), ("waves_per_workgroup", ctypes.c_int32),
                ("workgroups", ctypes.c_int64), ("lds_bytes", ctypes.c_int64)]


def q8_matmul_launch_info(N: int, K: int, n_slots: int = Q8_MAX_SLOTS,
                          with_workspace: bool = False) -> dict:
    """The MFMA engine's launch for an N x K matrix (host only)."""
    info = _LaunchInfo()
    _check(_lib.q8_matmul_launch_info(N, K, n_slots, int(with_workspace), ctypes.byref(info)),
           "q8_matmul_launch_info")
    return {name: int(getattr(info, name)) for name, _ in _LaunchInfo._fields_}


def _ws_bytes(workspace, workspace_bytes):
    if workspace_bytes is not None:
        return workspace_bytes
    if isinstance(workspace, torch.Tensor):
        return workspace.numel() * workspace.element_size()
    return 0


def q8_matmul_narrow_ws(Wq, Xq, batch_index, n_live: int, N: int, K: int, Y,
                        workspace, workspace_bytes: int | None = None,
                        stream=None) -> None:
    wq, xq, bi, y, ws = _dev(*_mm_checked(Wq, Xq, batch_index, n_live, N, K, Y),
                             _arg(workspace, "workspace", _ANY, q8_matmul_workspace_bytes(N, K)))
    _check(_lib.q8_matmul_narrow_ws(wq, xq, bi, n_live, N, K, y, ws,
                                    _ws_bytes(workspace, workspace_bytes), _stream(stream)),
           "q8_matmul_narrow_ws")


def q8_matmul_narrow_noalloc(Wq, Xq, batch_index, n_live: int, N: int, K: int, Y,
                             stream=None) -> None:
    wq, xq, bi, y = _dev(*_mm_checked(Wq, Xq, batch_index, n_live, N, K, Y))
    _check(_lib.q8_matmul_narrow_noalloc(wq, xq, bi, n_live, N, K, y, _stream(stream)),
           "q8_matmul_narrow_noalloc")


def q8_matmul_fused_workspace_bytes(N: int, K: int) -> int:
    return int(_lib.q8_matmul_fused_workspace_bytes(N, K))


def _fused_ptrs(Wq, X, n_rows, Xq, batch_index, n_live, N, K, Y, workspace):
    mm = _mm_checked(Wq, Xq, batch_index, n_live, N, K, Y)
    return _dev(mm[0], _arg(X, "X", _F32, _n(n_rows * K, 4)), mm[1], mm[2], mm[3],
                _arg(workspace, "workspace", _ANY, q8_matmul_fused_workspace_bytes(N, K)))


def q8_matmul_narrow_fused(Wq, X, n_rows: int, Xq, batch_index, n_live: int, N: int, K: int,
                           Y, workspace, workspace_bytes: int | None = None,
                           stream=None) -> None:
    wq, x, xq, bi, y, ws = _fused_ptrs(Wq, X, n_rows, Xq, batch_index, n_live, N, K, Y, workspace)
    _check(_lib.q8_matmul_narrow_fused(wq, x, n_rows, xq, bi, n_live, N, K, y, ws,
                                       _ws_bytes(workspace, workspace_bytes), _stream(stream)),
           "q8_matmul_narrow_fused")


def q8_matmul_narrow_fused_bounded(Wq, X, n_rows: int, Xq, batch_index, n_live: int, N: int,
                                   K: int, Y, workspace, max_spins: int, quantize: int,
                                   workspace_bytes: int | None = None, stream=None) -> None:
    wq, x, xq, bi, y, ws = _fused_ptrs(Wq, X, n_rows, Xq, batch_index, n_live, N, K, Y, workspace)
    _check(_lib.q8_matmul_narrow_fused_bounded(wq, x, n_rows, xq, bi, n_live, N, K, y, ws,
                                               _ws_bytes(workspace, workspace_bytes),
                                               int(max_spins), int(quantize), _stream(stream)),
           "q8_matmul_narrow_fused_bounded")


def fused_timeouts(workspace) -> int:
    """The fused workspace's count of matmul workgroups whose wait ran out
    (reads 4 bytes back from the device; synchronises)."""
    w = workspace[Q8_FUSED_TIMEOUTS_OFFSET:Q8_FUSED_TIMEOUTS_OFFSET + 4]
    return int.from_bytes(bytes(w.cpu().numpy().tobytes()), "little")


def q8_act_buffer_bytes_n(K: int, n_slots: int) -> int:
    return int(_lib.q8_act_buffer_bytes_n(K, n_slots))


def q8_quantize_acts_n(X, n_rows: int, K: int, Xq, n_slots: int, stream=None) -> None:
    x, xq = _dev(_arg(X, "X", _F32, _n(n_rows * K, 4)),
                 _arg(Xq, "Xq", _ANY, q8_act_buffer_bytes_n(K, n_slots)))
    _check(_lib.q8_quantize_acts_n(x, n_rows, K, xq, n_slots, _stream(stream)),
           "q8_quantize_acts_n")


def q8_matmul_multi(Wq, Xq, n_slots: int, batch_index, n_live: int, N: int, K: int, Y,
                    stream=None) -> None:
    wq, xq, bi, y = _dev(*_mm_checked(Wq, Xq, batch_index, n_live, N, K, Y,
                                      xq_bytes=q8_act_buffer_bytes_n(K, n_slots)))
    _check(_lib.q8_matmul_multi(wq, xq, n_slots, bi, n_live, N, K, y, _stream(stream)),
           "q8_matmul_multi")


def q8_rope_multi(Y, n_rows: int, row_stride: int, pos, n_heads: int, head_dim: int,
                  base: float, stream=None) -> None:
    need = _n((n_rows - 1) * row_stride + n_heads * head_dim, 4) if n_rows > 0 else 0
    y, p = _dev(_arg(Y, "Y", _F32, need), _arg(pos, "pos", _I32, _n(n_rows, 4)))
    _check(_lib.q8_rope_multi(y, n_rows, row_stride, p, n_heads, head_dim, float(base),
                              _stream(stream)), "q8_rope_multi")


def q8_stream_read(buf, nbytes: int, sink, stream=None) -> None:
    b, sk = _dev(_arg(buf, "buf", _ANY, max(nbytes, 0)), _arg(sink, "sink", _I32, 4 * 1024))
    _check(_lib.q8_stream_read(b, nbytes, sk, _stream(stream)), "q8_stream_read")


def q8_device_supported() -> bool:
    return bool(_lib.q8_device_supported())


def q8_timeline_set(records, max_waves: int) -> None:
    """Timeline build only: the record buffer (int64, Q8_STAMP_WORDS per
    wave) of the following matmul launches; None or max_waves 0 switches
    recording off."""
    if not TIMELINE:
        raise Q8Error(Q8_ERR_UNSUPPORTED, "q8_timeline_set (set Q8_LIBRARY=timeline before the "
                      "first import to load the timeline build)")
    (r,) = _dev(_arg(records, "records", (torch.int64,), 8 * Q8_STAMP_WORDS * max(max_waves, 0)))
    _check(_lib.q8_timeline_set(r, max_waves), "q8_timeline_set")


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
