"""The C ABI on the host: the library loads, exports every symbol the header
declares, reports layout sizes, and rejects invalid arguments before making
any HIP call (so these tests need no GPU and launch nothing)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q8narrow.h")


@pytest.fixture(scope="module")
def q8():
    import quantized_weight_streaming_q8_amd as q8
    return q8


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b(q8_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_abi():
    names = header_functions()
    for core in ("q8_pack_weights", "q8_quantize_acts", "q8_matmul_narrow"):
        assert core in names
    assert len(names) == 22, names


def test_every_declared_symbol_is_exported(q8):
    lib = ctypes.CDLL(q8.LIB_PATH)
    for name in header_functions():
        assert hasattr(lib, name), name
    assert set(header_functions()) == set(q8._SIGNATURES)


TIMELINE_HEADER = os.path.join(ROOT, "include", "q8timeline.h")


def timeline_functions():
    text = re.sub(r"/\*.*?\*/", "", open(TIMELINE_HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(q8_\w+)\s*\(", text, flags=re.M)))


def test_timeline_build_exports_both_headers_and_product_build_only_its_own(q8):
    """The timeline build exports every q8narrow.h entry point plus
    q8_timeline_set; the product library does not export the latter."""
    from quantized_weight_streaming_q8_amd import build
    assert timeline_functions() == ["q8_timeline_set"]
    assert set(timeline_functions()) == set(q8._TIMELINE_SIGNATURES)
    tl = ctypes.CDLL(build.TIMELINE_LIB_PATH)
    for name in header_functions() + timeline_functions():
        assert hasattr(tl, name), name
    prod = ctypes.CDLL(build.LIB_PATH)
    assert not hasattr(prod, "q8_timeline_set")
    text = open(TIMELINE_HEADER).read()
    assert int(re.search(r"#define Q8_STAMP_WORDS (\d+)", text).group(1)) == q8.Q8_STAMP_WORDS


def test_timeline_set_rejects_invalid_buffers():
    """Host checks only (no device pointer is dereferenced): a negative
    count, or a null or misaligned buffer with a positive count."""
    from quantized_weight_streaming_q8_amd import build
    tl = ctypes.CDLL(build.TIMELINE_LIB_PATH)
    fn = tl.q8_timeline_set
    fn.argtypes, fn.restype = [ctypes.c_void_p, ctypes.c_int64], ctypes.c_int
    assert fn(None, -1) == 1
    assert fn(None, 5) == 1
    assert fn(0x1004, 5) == 1
    assert fn(None, 0) == 0   # recording off
    assert fn(0x1000, 0) == 0


def test_product_binding_refuses_timeline_calls(q8):
    if q8.TIMELINE:
        pytest.skip("this process loaded the timeline build")
    with pytest.raises(q8.Q8Error):
        q8.q8_timeline_set(None, 0)


def test_constants_agree_with_header(q8):
    text = open(HEADER).read()
    assert int(re.search(r"#define Q8_MAX_SLOTS (\d+)", text).group(1)) == q8.Q8_MAX_SLOTS == 16
    assert int(re.search(r"#define Q8_BLOCK (\d+)", text).group(1)) == q8.Q8_BLOCK == 32
    assert int(re.search(r"#define Q8_MAX_COLUMNS (\d+)", text).group(1)) == q8.Q8_MAX_COLUMNS == 64
    assert int(re.search(r"#define Q8_NOALLOC_SCRATCH_BYTES \((\d+)u << 20\)", text).group(1)) << 20 \
        == q8.Q8_NOALLOC_SCRATCH_BYTES
    for name in ("Q8_OK", "Q8_ERR_INVALID_ARG", "Q8_ERR_UNSUPPORTED", "Q8_ERR_HIP",
                 "Q8_ERR_TOO_LARGE", "Q8_PATH_AUTO", "Q8_PATH_MFMA", "Q8_PATH_DOT4"):
        val = int(re.search(name + r"\s*=\s*(\d+)", text).group(1))
        assert getattr(q8, name) == val, name


def test_status_strings(q8):
    assert q8.status_str(0) == "Q8_OK"
    assert q8.status_str(1) == "Q8_ERR_INVALID_ARG"
    assert q8.status_str(2) == "Q8_ERR_UNSUPPORTED"
    assert q8.status_str(3) == "Q8_ERR_HIP"
    assert q8.status_str(4) == "Q8_ERR_TOO_LARGE"
    assert q8.status_str(99) == "Q8_ERR_UNKNOWN"


@pytest.mark.parametrize("N,K", [(768, 768), (7168, 5120), (5120, 17408),
                                 (151936, 5120), (1, 32), (17, 288)])
def test_layout_sizes(q8, N, K):
    G = -(-N // 16)
    NSC = -(-K // 256)
    assert q8.q8_packed_weight_bytes(N, K) == G * NSC * (4096 + 256)
    # the slot buffer is the packed form of a 16-row matrix
    assert q8.q8_act_buffer_bytes(K) == q8.q8_packed_weight_bytes(16, K) == NSC * 4352


def test_packed_size_is_weight_bytes_plus_padding(q8):
    # 34 bytes per 32 weights when N % 16 == 0 and K % 256 == 0
    assert q8.q8_packed_weight_bytes(7168, 5120) == 7168 * 5120 * 34 // 32


@pytest.mark.parametrize("N,K", [(0, 32), (-1, 32), (4, 0), (4, 31), (4, 48),
                                 (4, 1 << 24), (1 << 30, 1 << 12)])
def test_invalid_shapes_have_no_size(q8, N, K):
    assert q8.q8_packed_weight_bytes(N, K) == 0


def test_shape_limit_is_the_padded_size(q8):
    # the matrix padded to whole 16-row groups and 256-value super-chunks may
    # hold 2^34 values (every launch then stays below 2^32 threads)
    assert q8.q8_packed_weight_bytes(1 << 26, 256) == (1 << 26) * 256 * 34 // 32
    assert q8.q8_packed_weight_bytes((1 << 26) + 1, 256) == 0   # pads to 2^26 + 16 rows
    assert q8.q8_packed_weight_bytes(1 << 26, 32) > 0            # 32 values pad to 256
    assert q8.q8_packed_weight_bytes((1 << 26) + 1, 32) == 0
    assert q8.q8_packed_weight_bytes(1 << 13, (1 << 21) - 32) > 0
    assert q8.q8_packed_weight_bytes((1 << 13) + 1, (1 << 21) - 32) == 0
    assert q8.q8_packed_weight_bytes(151936, 5120) > 0           # the largest matrix here


@pytest.mark.parametrize("K", [32, 288, 768, 5120, 17408, 18432])
def test_slot_buffer_is_the_packed_16_row_matrix(q8, K):
    """The slot buffer's layout is the packed layout of a 16 x K matrix
    (row s = slot s): its size is exactly that matrix's packed size, at any
    slot count the multi-column calls take, and the library exports no slot
    stride.  Slots are crafted and read through the canonical q8_0
    import/export with N = 16 (the binding's write_act_slots and
    read_act_slots)."""
    assert q8.q8_act_buffer_bytes(K) == q8.q8_packed_weight_bytes(16, K)
    for n in (16, 32, 48, 64):
        assert q8.q8_act_buffer_bytes_n(K, n) == q8.q8_packed_weight_bytes(n, K)
    assert not hasattr(q8.library(), "q8_act_slot_stride")
    import inspect
    assert "q8_pack_weights_q(q, d16, n_slots, K, Xq" in inspect.getsource(q8.write_act_slots)
    assert "q8_unpack_weights(Xq, n_slots, K, q, d" in inspect.getsource(q8.read_act_slots)


def test_invalid_k_has_no_slot_buffer(q8):
    assert q8.q8_act_buffer_bytes(0) == 0
    assert q8.q8_act_buffer_bytes(33) == 0


# Fake but well-aligned addresses: every call below must be rejected by the
# host-side checks before any pointer is used or any HIP call is made.
P = 1 << 20


def _rc(fn, *args):
    return fn(*args)


@pytest.mark.parametrize("args", [
    (None, P, P, 4, 64, 64, P, None),       # Wq null
    (P, None, P, 4, 64, 64, P, None),       # Xq null
    (P, P, None, 4, 64, 64, P, None),       # batch_index null
    (P, P, P, 4, 64, 64, None, None),       # Y null
    (P, P, P, 0, 64, 64, P, None),          # n_live 0
    (P, P, P, 17, 64, 64, P, None),         # n_live beyond the slots
    (P, P, P, -3, 64, 64, P, None),
    (P, P, P, 4, 0, 64, P, None),           # N = 0
    (P, P, P, 4, 64, 48, P, None),          # K % 32 != 0
    (P, P, P, 4, 64, 16, P, None),          # K < 32
    (P + 8, P, P, 4, 64, 64, P, None),      # Wq misaligned
    (P, P + 4, P, 4, 64, 64, P, None),      # Xq misaligned
    (P, P, P + 2, 4, 64, 64, P, None),      # batch_index misaligned
    (P, P, P, 4, 64, 64, P + 1, None),      # Y misaligned
])
def test_matmul_rejects_invalid_arguments(q8, args):
    assert q8.library().q8_matmul_narrow(*args) == q8.Q8_ERR_INVALID_ARG
    assert q8.library().q8_matmul_narrow_noalloc(*args) == q8.Q8_ERR_INVALID_ARG


def test_noalloc_rejects_shapes_beyond_its_array(q8):
    """The no-allocation entry point's static array holds the split records
    of up to 1927 row groups; a split shape needing more is refused before
    any HIP call, one that fits is not refused for its size."""
    lib = q8.library()
    cap = q8.Q8_NOALLOC_SCRATCH_BYTES
    rec = 256 + 4 * 1024
    assert cap // rec == 1927
    fits, over = 1927 * 16, 1928 * 16
    assert q8.q8_matmul_workspace_bytes(fits, 17408) <= cap < q8.q8_matmul_workspace_bytes(over, 17408)
    assert lib.q8_matmul_narrow_noalloc(P, P, P, 4, over, 17408, P, None) == q8.Q8_ERR_TOO_LARGE
    assert lib.q8_matmul_narrow_noalloc(P, P, P, 4, 10 ** 6, 8192, P, None) == q8.Q8_ERR_TOO_LARGE
    # shapes that fit (or are not split) get past the size check; with no
    # gfx950 device the call then stops at the device check
    if not q8.q8_device_supported():
        for N, K in ((fits, 17408), (151936, 5120)):
            assert lib.q8_matmul_narrow_noalloc(P, P, P, 4, N, K, P, None) == q8.Q8_ERR_UNSUPPORTED


def test_matmul_path_rejects_unknown_engine(q8):
    lib = q8.library()
    assert lib.q8_matmul_narrow_path(P, P, P, 4, 64, 64, P, None, 3) == q8.Q8_ERR_INVALID_ARG
    assert lib.q8_matmul_narrow_path(P, P, P, 4, 64, 64, P, None, -1) == q8.Q8_ERR_INVALID_ARG


def test_other_entry_points_reject_invalid_arguments(q8):
    lib = q8.library()
    bad = q8.Q8_ERR_INVALID_ARG
    assert lib.q8_pack_weights(None, 4, 64, P, None) == bad
    assert lib.q8_pack_weights(P, 4, 64, None, None) == bad
    assert lib.q8_pack_weights(P + 4, 4, 64, P, None) == bad
    assert lib.q8_pack_weights(P, 4, 40, P, None) == bad
    assert lib.q8_pack_weights_q(P, P, 4, 64, P + 8, None) == bad
    assert lib.q8_pack_weights_q(P + 4, P, 4, 64, P, None) == bad
    assert lib.q8_pack_weights_q(P, P + 1, 4, 64, P, None) == bad
    assert lib.q8_unpack_weights(P, 0, 64, P, P, None) == bad
    assert lib.q8_unpack_weights(None, 4, 64, P, P, None) == bad
    assert lib.q8_quantize_acts(P, 0, 64, P, None) == bad
    assert lib.q8_quantize_acts(P, 17, 64, P, None) == bad
    assert lib.q8_quantize_acts(P, 4, 65, P, None) == bad
    assert lib.q8_quantize_acts(P + 4, 4, 64, P, None) == bad
    assert lib.q8_quantize_acts(P, 4, 64, None, None) == bad


def test_workspace_sizes(q8):
    # long rows (K >= 8192) are split across workgroups and need a workspace:
    # one record per row group, its counter's 256-byte line then 4 partial
    # tiles of 16 x 16 fp32, the same record size for every split shape;
    # shorter rows are not split
    rec = 256 + 4 * 1024
    assert q8.q8_matmul_workspace_bytes(5120, 17408) == (5120 // 16) * rec
    # 224 two-row-group blocks fill 88% of the 256 CUs: the K ranges run in one workgroup
    assert q8.q8_matmul_workspace_bytes(7168, 18432) == 0
    assert q8.q8_matmul_workspace_bytes(16 * 2 * 204, 18432) == 2 * 204 * rec  # 80% not reached
    assert q8.q8_matmul_workspace_bytes(16 * 2 * 205, 18432) == 0
    assert q8.q8_matmul_workspace_bytes(16 * 2 * 257, 18432) == 2 * 257 * rec  # more blocks than CUs
    assert q8.q8_matmul_workspace_bytes(1000, 8224) == 63 * rec
    assert q8.q8_matmul_workspace_bytes(5120, 5120) == 0
    assert q8.q8_matmul_workspace_bytes(151936, 5120) == 0
    assert q8.q8_matmul_workspace_bytes(0, 5120) == 0
    assert q8.q8_matmul_workspace_bytes(16, 32) == 0  # one super-chunk: no split
    # 1024..4400 row groups, not a multiple of the 256 CUs: only the last
    # (G mod 256) row groups run as split workgroups, one record each
    assert q8.q8_matmul_workspace_bytes(34816, 5120) == 128 * rec   # gate+up: 2176 = 8*256 + 128
    assert q8.q8_matmul_workspace_bytes(18432, 7168) == 128 * rec   # 1152 = 4*256 + 128
    assert q8.q8_matmul_workspace_bytes(17408, 5120) == 64 * rec    # 1088: 64 row groups, 4 splits
    assert q8.q8_matmul_workspace_bytes(16391, 5120) == 1 * rec     # 1025: one ragged row group
    assert q8.q8_matmul_workspace_bytes(32768, 5120) == 0           # 2048 = 8*256
    assert q8.q8_matmul_workspace_bytes(16 * (1024 + 129), 5120) == 0  # r = 129: one split only


# (N, K, n_slots, with_workspace) -> row groups per wave, column tiles,
# chunks in flight, K splits, slices per split, split workgroups, whole-row
# workgroups, waves per workgroup, workgroups.  The Qwen3-14B layer and head,
# the large dense pair, and a one-row-group matrix; their grids (workgroups x
# waves x 64 lanes) are the ones the kernel traces record.
LAUNCH_PLANS = {
    (7168, 5120, 16, 0): (2, 1, 4, 1, 4, 0, 0, 4, 224),      # QKV: 4 K slices in one workgroup
    (5120, 5120, 16, 0): (2, 1, 4, 1, 4, 0, 0, 4, 160),      # O
    (34816, 5120, 16, 0): (1, 1, 2, 4, 1, 0, 2176, 1, 2176),  # gate+up: whole rows, 4 splits in turn
    (34816, 5120, 16, 1): (1, 1, 2, 4, 1, 1, 2048, 1, 2560),  # ... the last 128 as 4 pieces each
    (5120, 17408, 16, 0): (2, 1, 4, 4, 1, 0, 0, 4, 160),     # down: 4 splits as waves
    (5120, 17408, 16, 1): (1, 1, 4, 4, 1, 1, 0, 1, 1280),    # ... as one-wave workgroups
    (151936, 5120, 16, 0): (2, 1, 1, 1, 1, 0, 0, 1, 4748),   # head: two row groups, one chunk
    (18432, 7168, 16, 1): (1, 1, 4, 4, 1, 1, 1024, 1, 1536),  # 7168->18432
    (7168, 18432, 16, 1): (2, 1, 4, 1, 4, 0, 0, 4, 224),     # 18432->7168: 205..256 blocks, no split
    (34816, 5120, 32, 0): (2, 2, 4, 4, 1, 0, 0, 4, 1088),    # multi-column: two row groups per wave
    (34816, 5120, 48, 0): (2, 3, 2, 4, 1, 0, 0, 4, 1088),
    (34816, 5120, 64, 0): (2, 4, 2, 4, 1, 0, 0, 4, 1088),
    (7168, 5120, 64, 0): (2, 4, 4, 1, 4, 0, 0, 4, 224),
    (151936, 5120, 32, 0): (2, 2, 1, 1, 1, 0, 0, 1, 4748),
    (151936, 5120, 64, 0): (2, 4, 2, 1, 1, 0, 0, 1, 4748),
    (5, 64, 64, 0): (1, 4, 2, 1, 1, 0, 0, 1, 1),              # one row group
}
_PLAN_KEYS = ("row_groups_per_wave", "column_tiles", "chunks_in_flight", "k_splits",
              "slices_per_split", "split_workgroups", "whole_row_workgroups",
              "waves_per_workgroup", "workgroups")


@pytest.mark.parametrize("key", list(LAUNCH_PLANS))
def test_launch_plans(q8, key):
    N, K, n_slots, ws = key
    info = q8.q8_matmul_launch_info(N, K, n_slots, bool(ws))
    assert tuple(info[k] for k in _PLAN_KEYS) == LAUNCH_PLANS[key]
    # one float4 per lane, row group and column tile of every wave
    assert info["lds_bytes"] == (info["waves_per_workgroup"] * info["row_groups_per_wave"]
                                 * info["column_tiles"] * 64 * 16)


def test_launch_plan_tree_does_not_depend_on_width_or_workspace(q8):
    """The summation tree (K splits, slices per split) is the same for every
    slot width and with or without a workspace, so a column's bits never
    depend on how the call was made; the launch stays within 8 waves and
    64 KB of LDS per workgroup, and a split execution exactly when the shape
    needs a workspace."""
    rng = __import__("random").Random(7)
    shapes = [(34816, 5120), (5120, 17408), (18432, 7168), (7168, 18432), (17405, 1056),
              (17981, 2080), (72003, 256), (6555, 8224), (6528, 8224), (1, 32), (17, 288)]
    shapes += [(rng.randrange(1, 80000), 32 * rng.randrange(1, 700)) for _ in range(40)]
    for N, K in shapes:
        need = q8.q8_matmul_workspace_bytes(N, K)
        plans = [q8.q8_matmul_launch_info(N, K, 16, True)]
        plans += [q8.q8_matmul_launch_info(N, K, n, False) for n in (16, 32, 48, 64)]
        assert len({(p["k_splits"], p["slices_per_split"]) for p in plans}) == 1, (N, K)
        assert plans[0]["split_workgroups"] == (1 if need > 0 else 0), (N, K)
        G = -(-N // 16)
        for p in plans:
            assert 1 <= p["waves_per_workgroup"] <= 8 and p["lds_bytes"] <= 64 * 1024, (N, K, p)
            assert p["chunks_in_flight"] in (1, 2, 4)
            rg = p["row_groups_per_wave"]
            assert rg in (1, 2) and G >= rg
            blocks = -(-G // rg)
            pieces = (blocks - p["whole_row_workgroups"]) * p["k_splits"] if p["split_workgroups"] else 0
            assert p["workgroups"] == (p["whole_row_workgroups"] + pieces if p["split_workgroups"]
                                       else blocks), (N, K, p)


@pytest.mark.parametrize("args", [(0, 32, 16, 0), (16, 48, 16, 0), (16, 32, 8, 0), (16, 32, 80, 0),
                                  (16, 32, 17, 0), (16, 32, 32, 1), (16, 32, 16, 2),
                                  (16, 32, 16, -1)])
def test_launch_info_rejects_invalid_arguments(q8, args):
    info = q8._LaunchInfo()
    assert q8._lib.q8_matmul_launch_info(*args, ctypes.byref(info)) == q8.Q8_ERR_INVALID_ARG
    assert q8._lib.q8_matmul_launch_info(16, 32, 16, 0, None) == q8.Q8_ERR_INVALID_ARG


def test_ws_entry_point_rejects_a_missing_or_small_workspace(q8):
    lib = q8.library()
    bad = q8.Q8_ERR_INVALID_ARG
    need = q8.q8_matmul_workspace_bytes(5120, 17408)
    assert need > 0
    assert lib.q8_matmul_narrow_ws(P, P, P, 4, 5120, 17408, P, None, need, None) == bad
    assert lib.q8_matmul_narrow_ws(P, P, P, 4, 5120, 17408, P, P, need - 1, None) == bad
    assert lib.q8_matmul_narrow_ws(P, P, P, 4, 5120, 17408, P, P + 16, need, None) == bad
    assert lib.q8_matmul_narrow_ws(P, P, P, 0, 5120, 17408, P, P, need, None) == bad


def test_binding_raises_on_rejected_call(q8):
    with pytest.raises(q8.Q8Error) as e:
        q8.q8_matmul_narrow(P, P, P, 0, 64, 64, P, stream=0)
    assert e.value.status == q8.Q8_ERR_INVALID_ARG
    assert "Q8_ERR_INVALID_ARG" in str(e.value)


@pytest.mark.parametrize("K", [32, 768, 5120, 17408])
def test_multi_column_buffer_sizes(q8, K):
    for n in (16, 32, 48, 64):
        assert q8.q8_act_buffer_bytes_n(K, n) == q8.q8_packed_weight_bytes(n, K)
        assert q8.q8_act_buffer_bytes_n(K, n) == (n // 16) * q8.q8_act_buffer_bytes(K)
    for bad in (0, 8, 17, 24, 80, -16):
        assert q8.q8_act_buffer_bytes_n(K, bad) == 0


def test_multi_column_calls_reject_invalid_arguments(q8):
    lib = q8.library()
    bad = q8.Q8_ERR_INVALID_ARG
    # slot counts that are not 16, 32, 48 or 64
    for n_slots in (0, 8, 24, 80):
        assert lib.q8_quantize_acts_n(P, 4, 64, P, n_slots, None) == bad
        assert lib.q8_matmul_multi(P, P, n_slots, P, 4, 64, 64, P, None) == bad
    # more rows or live tokens than slots
    assert lib.q8_quantize_acts_n(P, 33, 64, P, 32, None) == bad
    assert lib.q8_quantize_acts_n(P, 0, 64, P, 32, None) == bad
    assert lib.q8_matmul_multi(P, P, 32, P, 33, 64, 64, P, None) == bad
    assert lib.q8_matmul_multi(P, P, 64, P, 0, 64, 64, P, None) == bad
    # shapes, null and misaligned pointers
    assert lib.q8_matmul_multi(P, P, 64, P, 4, 64, 48, P, None) == bad
    assert lib.q8_matmul_multi(None, P, 64, P, 4, 64, 64, P, None) == bad
    assert lib.q8_matmul_multi(P, P + 8, 64, P, 4, 64, 64, P, None) == bad
    assert lib.q8_matmul_multi(P, P, 64, P + 2, 4, 64, 64, P, None) == bad
    assert lib.q8_matmul_multi(P, P, 64, P, 4, 64, 64, P + 1, None) == bad
    assert lib.q8_quantize_acts_n(P + 4, 4, 64, P, 64, None) == bad


def test_fused_workspace_sizes(q8):
    for N, K in ((5120, 5120), (5120, 17408), (151936, 5120), (16, 32)):
        assert q8.q8_matmul_fused_workspace_bytes(N, K) == 65536 + q8.q8_matmul_workspace_bytes(N, K)
    assert q8.q8_matmul_fused_workspace_bytes(0, 5120) == 0


def test_fused_bounded_rejects_invalid_bounds(q8):
    lib = q8.library()
    bad = q8.Q8_ERR_INVALID_ARG
    need = q8.q8_matmul_fused_workspace_bytes(64, 256)
    for spins, quantize in ((0, 1), (-1, 1), ((1 << 30) + 1, 1), (8, 2), (8, -1)):
        assert lib.q8_matmul_narrow_fused_bounded(P, P, 16, P, P, 4, 64, 256, P, P, need, spins,
                                                  quantize, None) == bad, (spins, quantize)
    assert lib.q8_matmul_narrow_fused_bounded(P, P, 16, P, P, 4, 64, 256, P, P, need - 1, 8, 1,
                                              None) == bad


def test_fused_call_rejects_invalid_arguments(q8):
    lib = q8.library()
    bad = q8.Q8_ERR_INVALID_ARG
    need = q8.q8_matmul_fused_workspace_bytes(64, 64)
    ok = (P, P, 4, P, P, 4, 64, 64, P, P, need, None)
    def call(**kw):
        args = list(ok)
        for i, v in kw.items():
            args[int(i[1:])] = v
        return lib.q8_matmul_narrow_fused(*args)
    assert call(a2=0) == bad and call(a2=17) == bad          # n_rows
    assert call(a5=0) == bad and call(a5=17) == bad          # n_live
    assert call(a7=48) == bad                                # K % 32
    assert call(a0=None) == bad and call(a1=P + 4) == bad    # Wq null, X misaligned
    assert call(a3=P + 8) == bad and call(a4=P + 2) == bad   # Xq, batch_index misaligned
    assert call(a9=None) == bad and call(a9=P + 16) == bad   # workspace missing, misaligned
    assert call(a10=need - 1) == bad                         # workspace too small


def test_rope_rejects_invalid_arguments(q8):
    lib = q8.library()
    bad = q8.Q8_ERR_INVALID_ARG
    ok = [P, 4, 7168, P, 48, 128, 1e6, None]
    def call(i, v):
        a = list(ok)
        a[i] = v
        return lib.q8_rope_multi(*a)
    assert call(1, 0) == bad and call(1, 65) == bad          # n_rows
    assert call(2, 48 * 128 - 1) == bad                      # heads do not fit the row
    assert call(4, 0) == bad                                 # n_heads
    assert call(5, 127) == bad and call(5, 0) == bad and call(5, 2048) == bad  # head_dim
    assert call(6, 1.0) == bad and call(6, float("nan")) == bad and call(6, -5.0) == bad
    assert call(0, None) == bad and call(0, P + 2) == bad    # Y null, misaligned
    assert call(3, None) == bad and call(3, P + 1) == bad    # pos null, misaligned
    # more than 2^32 rotated values (the launch would pass 2^32 threads)
    a = [P, 64, 65537 * 1024, P, 65537, 1024, 1e6, None]
    assert lib.q8_rope_multi(*a) == bad


def test_stream_read_rejects_invalid_arguments(q8):
    lib = q8.library()
    bad = q8.Q8_ERR_INVALID_ARG
    assert lib.q8_stream_read(None, 1024, P, None) == bad          # no buffer
    assert lib.q8_stream_read(P, 1024, None, None) == bad          # no sink
    assert lib.q8_stream_read(P, 0, P, None) == bad                # empty
    assert lib.q8_stream_read(P, 1000, P, None) == bad             # not whole 16-byte units
    assert lib.q8_stream_read(P + 8, 1024, P, None) == bad         # misaligned buffer
    assert lib.q8_stream_read(P, 1024, P + 2, None) == bad         # misaligned sink
    assert lib.q8_stream_read(P, (1 << 40) + 16, P, None) == bad   # too large


# --------------------------------------------- binding argument checks
#
# The binding checks tensors before any call: dtype, size against the
# library's own size functions and n_live * N, contiguity, and that the
# tensor is on the current device.  These run on the CPU: the checks come in
# that order, so host tensors of a wrong dtype or size fail before the device
# check, and correct host tensors fail at the device check.

def _t(n, dtype):
    import torch
    return torch.zeros(n, dtype=dtype)


def test_binding_rejects_wrong_dtypes(q8):
    import torch
    N, K = 32, 256
    wq = _t(q8.q8_packed_weight_bytes(N, K), torch.uint8)
    xq = _t(q8.q8_act_buffer_bytes(K), torch.uint8)
    Y = _t(4 * N, torch.float32)
    bi = _t(4, torch.int32)
    cases = [
        (lambda: q8.q8_pack_weights(_t(N * K, torch.float64), N, K, wq, stream=0), "W: expected float32"),
        (lambda: q8.q8_pack_weights_q(_t(N * K, torch.uint8), _t(N * K // 32, torch.int16), N, K, wq,
                                      stream=0), "q: expected int8"),
        (lambda: q8.q8_pack_weights_q(_t(N * K, torch.int8), _t(N * K // 32, torch.float32), N, K, wq,
                                      stream=0), "d16: expected int16 or float16"),
        (lambda: q8.q8_quantize_acts(_t(16 * K, torch.float16), 16, K, xq, stream=0), "X: expected float32"),
        (lambda: q8.q8_matmul_narrow(wq, xq, _t(4, torch.int64), 4, N, K, Y, stream=0),
         "batch_index: expected int32"),
        (lambda: q8.q8_matmul_narrow(wq, xq, bi, 4, N, K, _t(4 * N, torch.float64), stream=0),
         "Y: expected float32"),
        (lambda: q8.q8_rope_multi(Y, 4, N, _t(4, torch.int64), 1, 8, 1e4, stream=0),
         "pos: expected int32"),
    ]
    for fn, msg in cases:
        with pytest.raises(ValueError, match=msg):
            fn()


def test_binding_rejects_undersized_tensors(q8):
    import torch
    N, K = 48, 512
    pw = q8.q8_packed_weight_bytes(N, K)
    ab = q8.q8_act_buffer_bytes(K)
    wq, xq = _t(pw, torch.uint8), _t(ab, torch.uint8)
    bi, Y = _t(5, torch.int32), _t(5 * N, torch.float32)
    cases = [
        (lambda: q8.q8_pack_weights(_t(N * K - 1, torch.float32), N, K, wq, stream=0), "W: holds"),
        (lambda: q8.q8_pack_weights(_t(N * K, torch.float32), N, K, _t(pw - 1, torch.uint8), stream=0),
         "Wq: holds"),
        (lambda: q8.q8_unpack_weights(wq, N, K, _t(N * K, torch.int8), _t(N * K // 32 - 1, torch.int16),
                                      stream=0), "d16: holds"),
        (lambda: q8.q8_quantize_acts(_t(16 * K, torch.float32), 16, K, _t(ab - 16, torch.uint8),
                                     stream=0), "Xq: holds"),
        (lambda: q8.q8_matmul_narrow(wq, xq, _t(4, torch.int32), 5, N, K, Y, stream=0),
         "batch_index: holds"),
        (lambda: q8.q8_matmul_narrow(wq, xq, bi, 5, N, K, _t(5 * N - 1, torch.float32), stream=0),
         "Y: holds"),
        (lambda: q8.q8_matmul_narrow_noalloc(_t(pw - 16, torch.uint8), xq, bi, 5, N, K, Y, stream=0),
         "Wq: holds"),
        (lambda: q8.q8_matmul_multi(wq, xq, 32, bi, 5, N, K, Y, stream=0), "Xq: holds"),
        (lambda: q8.q8_matmul_narrow_fused(wq, _t(16 * K - 1, torch.float32), 16, xq, bi, 5, N, K, Y,
                                           _t(q8.q8_matmul_fused_workspace_bytes(N, K), torch.uint8),
                                           stream=0), "X: holds"),
        (lambda: q8.q8_matmul_narrow_fused(wq, _t(16 * K, torch.float32), 16, xq, bi, 5, N, K, Y,
                                           _t(1024, torch.uint8), stream=0), "workspace: holds"),
        (lambda: q8.q8_matmul_narrow_ws(wq, xq, bi, 5, 5120, 17408, _t(5 * 5120, torch.float32),
                                        _t(100, torch.uint8), stream=0), "holds"),
        (lambda: q8.q8_rope_multi(_t(3 * 100, torch.float32), 4, 100, _t(4, torch.int32), 2, 8, 1e4,
                                  stream=0), "Y: holds"),
        (lambda: q8.q8_stream_read(_t(1000, torch.uint8), 1024, _t(1024, torch.int32), stream=0),
         "buf: holds"),
    ]
    for fn, msg in cases:
        with pytest.raises(ValueError, match=msg):
            fn()


def test_binding_rejects_host_tensors_and_non_tensors(q8):
    import torch
    N, K = 16, 256
    wq = _t(q8.q8_packed_weight_bytes(N, K), torch.uint8)
    xq = _t(q8.q8_act_buffer_bytes(K), torch.uint8)
    with pytest.raises(ValueError, match="expected a device tensor"):
        q8.q8_matmul_narrow(wq, xq, _t(2, torch.int32), 2, N, K, _t(2 * N, torch.float32), stream=0)
    with pytest.raises(ValueError, match="contiguous"):
        q8.q8_matmul_narrow(wq, xq, _t(4, torch.int32)[::2], 2, N, K, _t(2 * N, torch.float32),
                            stream=0)
    with pytest.raises(TypeError):
        q8.q8_matmul_narrow(wq, xq, [0, 1], 2, N, K, _t(2 * N, torch.float32), stream=0)
