"""Host-side pieces of bench.py (no GPU)."""

import os

import numpy as np
import pytest

import bench
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "ds4_measured.txt")


def _rows():
    for line in open(GOLDEN):
        if line.strip() and not line.startswith("#"):
            path, n, ms, sp = line.split()
            yield path, int(n), (None if ms == "-" else float(ms)), float(sp)


def test_speedup_formula_reproduces_the_printed_table():
    rows = list(_rows())
    t1 = [r for r in rows if r[0] == "single"][0][2]
    checked = 0
    for path, n, ms, sp in rows:
        if ms is None:
            continue
        # printed to two decimals (0.6252 is printed 0.62 on the page)
        assert abs(bench.speedup_vs_single(t1, ms, n) - sp) <= 0.01, (path, n)
        checked += 1
    assert checked == 5


def test_matmul_bytes_match_the_packed_format():
    # weights 34 B per 32, activations 34 B per block per token
    assert bench.matmul_bytes(7168, 5120, 1) == 7168 * 160 * 34 + 160 * 34 + 4 + 4 * 7168
    b16 = bench.matmul_bytes(151936, 5120, 16)
    assert abs(b16 / 1e6 - 836.34) < 0.01
    assert abs(bench.matmul_bytes(5120, 17408, 16) / 1e6 - 95.32) < 0.01


def test_step_bytes_of_the_qwen3_layer():
    mats = wl.WORKLOADS["qwen3_layer"].matrices
    mm = sum(bench.matmul_bytes(m.N, m.K, 16) for m in mats)
    assert abs(mm / 1e6 - (39.54 + 28.27 + 191.71 + 95.32)) < 0.05
    assert bench.step_bytes(mats, 16) > mm


def test_more_than_one_gpu_is_refused():
    assert bench.main(["--gpus", "2"]) == 2


def test_steps_per_graph_divides_the_timed_steps():
    import bench
    assert bench.steps_per_graph(400) == 40
    assert bench.steps_per_graph(100) == 25
    assert bench.steps_per_graph(20) == 20
    assert bench.steps_per_graph(7) == 7
    assert bench.steps_per_graph(41) == 1
    for steps in (400, 100, 30, 7, 97):
        n = bench.steps_per_graph(steps)
        assert steps % n == 0 and 1 <= n <= 40


def test_each_matrix_rotates_at_least_a_gib():
    """Per-matrix rotations of packed copies: every Qwen3-14B layer matrix
    covers at least 1 GiB on its own (QKV 28 copies, O 39, gate+up 6, down
    12), so per-matrix timings stream from HBM, not the 256 MB cache."""
    import bench
    want = {"qkv": 28, "o": 39, "gate_up": 6, "down": 12}
    for m in wl.WORKLOADS["qwen3_layer"].matrices:
        nbytes = m.N * (m.K // 32) * 34  # no padding on these shapes
        c = bench.copies_for(nbytes)
        assert c == want[m.name] and c * nbytes >= 1 << 30 > (c - 1) * nbytes, m.name
    assert bench.copies_for(1 << 20) == bench.MAX_COPIES  # tiny matrices are capped
    assert bench.copies_for(4 << 30) == 2


def test_schedule_draws_every_live_batch_uniformly():
    """The large dense shapes' 1000-step schedule: every live batch 1..16
    occurs, each about 1000/16 times, and every step's batch_index is a
    prefix of a slot permutation (distinct slots in 0..15)."""
    import numpy as np
    sched = wl.schedule(wl.WORKLOADS["large_dense"].config, 1000)
    counts = np.bincount([b.size for b in sched], minlength=17)
    assert counts[0] == 0 and counts[1:].sum() == 1000
    assert counts[1:].min() >= 30 and counts[1:].max() <= 100
    for b in sched:
        assert b.dtype == np.int32 and len(set(b.tolist())) == b.size
        assert b.min() >= 0 and b.max() < 16
    bytes_total = sum(bench.step_bytes(wl.WORKLOADS["large_dense"].matrices, b.size) for b in sched)
    assert bytes_total > 1000 * 2 * 140_000_000


def test_rope_configurations_fit_their_qkv_rows():
    """Each workload's pos-vector RoPE heads (query + key) fit the QKV
    matrix's output rows; Qwen3-14B rotates 40 + 8 heads of 128."""
    for key, w in wl.WORKLOADS.items():
        if w.rope is None:
            continue
        heads, head_dim, base = w.rope
        qkv = [m for m in w.matrices if m.name == "qkv"]
        assert qkv, key
        assert head_dim % 2 == 0 and heads * head_dim <= qkv[0].N and base > 1, key
    assert wl.WORKLOADS["qwen3_layer"].rope == (48, 128, 1e6)


def test_traffic_is_reported_only_for_the_matrix_it_was_counted_on():
    """Each committed counter summary covers one workload's matrix (the four
    matrices of the Qwen3-14B layer, the Qwen3-14B head): no other matrix
    borrows its traffic, and each moves at least its own algorithmic bytes
    and at most a few percent more."""
    assert bench.measured_traffic("large_dense", "up", 16, False) is None
    assert bench.measured_traffic("qwen3_layer", "gate_up", 16, True) is None
    for key, name, N, K in (("qwen3_layer", "qkv", 7168, 5120),
                            ("qwen3_layer", "o", 5120, 5120),
                            ("qwen3_layer", "gate_up", 34816, 5120),
                            ("qwen3_layer", "down", 5120, 17408),
                            ("qwen3_head", "head", 151936, 5120)):
        t = bench.measured_traffic(key, name, 16, False)
        if t is not None:  # only while the summary matches the kernel source
            alg = bench.matmul_bytes(N, K, 16)
            assert 0.995 * alg <= t <= 1.08 * alg, (key, name, t / alg)


def _records(nw, split, ncu=256):
    """Synthetic timeline records: wave i starts at i % 7 ticks, its phases
    last 100, 1200, 40, 60 and 40 ticks (and 90 for the combine of every
    fourth wave of a split shape); wave i runs on CU i % ncu."""
    t = np.zeros((nw + 5, 8), dtype=np.int64)
    w = np.arange(nw)
    t[:nw, 0] = 10**9 + w % 7
    for k, d in enumerate((100, 1200, 40, 60, 40)):
        t[:nw, k + 1] = t[:nw, k] + d
    if split:
        t[:nw, 6] = np.where(w % 4 == 3, t[:nw, 5] + 90, 0)
    cu = w % ncu
    t[:nw, 7] = ((cu % 8) << 32) | ((cu // 8) << 8)
    return t


def test_timeline_summary_of_known_records():
    s = bench.timeline_summary([_records(1280, True), _records(1280, True)], True)
    assert s["launches"] == 2 and s["waves"] == 1280 and s["cus_used"] == 256
    ph = s["phases_us"]
    assert ph["first_chunk"] == [1.0] * 5 and ph["stream"] == [12.0] * 5
    assert ph["reduce"] == [0.4] * 5 and ph["publish"] == [0.6] * 5
    assert ph["arrive"] == [0.4] * 5 and ph["combine"] == [0.9] * 5
    assert ph["last_tail"] == [2.3] * 5
    assert ph["start"][0] == 0.0 and ph["start"][-1] == 0.06
    assert s["span_us"] == [15.36, 15.36]  # latest start 6 + 100 + 1200 + 40 + 60 + 40 + 90 ticks
    # each CU's last end, by a plain loop over the waves
    last = {}
    for w in range(1280):
        end = w % 7 + 1440 + (90 if w % 4 == 3 else 0)
        last[w % 256] = max(last.get(w % 256, 0), end)
    med = float(np.median(list(last.values()))) / 100
    assert s["waves_per_cu"] == {5: {"cus": 256, "last_end_us_median": round(med, 3)}}
    assert {x: v["waves"] for x, v in s["per_xcc"].items()} == {x: 160 for x in range(8)}
    assert s["per_xcc"][3]["end_us_max"] == 15.36 and s["per_xcc"][0]["end_us_max"] == 14.46
    p = bench.timeline_summary([_records(2176, False)], False)
    assert p["waves_per_cu"][8]["cus"] == 128 and p["waves_per_cu"][9]["cus"] == 128
    assert p["phases_us"]["y_issue"] == [0.6] * 5 and p["phases_us"]["y_done"] == [0.4] * 5
    assert p["span_us_median"] == 14.46  # latest start 6 + 1440 ticks


def test_timeline_cu_end_rank_correlation():
    # one wave per CU; CU c streams for a time set by a per-launch order of the CUs
    def launch(order):
        t = _records(256, False)
        extra = 10 * np.asarray(order, dtype=np.int64)  # ticks of streaming added to CU c
        for k in (2, 3, 4, 5):
            t[:256, k] += extra
        return t
    same = np.arange(256)
    rev = same[::-1].copy()
    perm = np.random.default_rng(5).permutation(256)
    assert bench.timeline_summary([launch(same), launch(same)], False)["cu_end_rank_corr_median"] == 1.0
    assert bench.timeline_summary([launch(same), launch(rev)], False)["cu_end_rank_corr_median"] == -1.0
    from scipy.stats import spearmanr
    # the record's start offsets (i % 7 ticks) are part of each CU's end time
    ends_a = np.arange(256) % 7 + 1440 + 10 * same
    ends_b = np.arange(256) % 7 + 1440 + 10 * perm
    want = spearmanr(ends_a, ends_b).correlation
    got = bench.timeline_summary([launch(same), launch(perm)], False)["cu_end_rank_corr_median"]
    assert abs(got - want) < 1e-3
    assert bench.timeline_summary([launch(same)], False)["cu_end_rank_corr_median"] is None


def test_kernel_hash_ignores_comments_not_code():
    a = "int f(int x) {\n    return x + 1;  // one more\n}\n"
    b = "/* block\n   comment */\nint f(int x) {\n\n    // a comment line\n    return x + 1;\n}\n"
    c = "int f(int x) {\n    return x + 2;\n}\n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)
