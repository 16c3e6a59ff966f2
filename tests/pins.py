"""Pins for the CPU oracle: checks against facts fixed by the number formats
and by mathematics, never against the oracle itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` instance and raises
``AssertionError`` when the oracle disagrees.  ``test_oracle_pins.py`` runs
them on the real oracle; ``test_oracle_mutants.py`` runs them on oracle
builds with planted mistakes and expects a failure each time.

What pins what:
  * binary16 conversion -- a library routine (torch's CPU float->half, which
    is IEEE round-to-nearest-even), exhaustively or on a boundary sample;
  * block quantisation -- hand-derived closed forms in
    ``golden/q8_0_closed_forms.txt``, invariants that hold for every block,
    and two constructed blocks that separate the readings the pages leave
    open (divide vs multiply by a reciprocal; quantise with the binary32
    scale vs with its binary16 rounding);
  * the matmul -- brute force in exact rational arithmetic on tiny inputs,
    agreement with a float64 dense matmul of the dequantised operands, the
    invariant that each batched column equals its single-token result, and
    exact per-block integer sums against a numpy int64 reduction.
"""

from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
BLOCK = 32


# --------------------------------------------------------------------------
# library references
# --------------------------------------------------------------------------

def f16_bits_reference(x: np.ndarray) -> np.ndarray:
    """binary32 -> binary16 bits with torch's CPU conversion (IEEE RNE)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float16).view(torch.int16).numpy().view(np.uint16)


def f16_value(bits) -> np.ndarray:
    """binary16 bits -> float64 value (numpy's conversion, exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def half_away(v) -> np.ndarray:
    """Round to nearest integer, ties away from zero (float64 in, exact)."""
    v = np.asarray(v, dtype=np.float64)
    return np.sign(v) * np.floor(np.abs(v) + 0.5)


# --------------------------------------------------------------------------
# golden closed forms
# --------------------------------------------------------------------------

def load_closed_forms(path: str | None = None):
    path = path or os.path.join(GOLDEN, "q8_0_closed_forms.txt")
    cases, cur = [], None
    with open(path) as fh:
        for raw in fh:
            line = raw.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(" ") if line.startswith("case ") else line.partition(":")
            val = val.strip()
            if key == "case":
                cur = {"name": val}
                cases.append(cur)
            elif key == "unit":
                cur["unit"] = float.fromhex(val)
            elif key == "k":
                cur["k"] = [int(v) for v in val.split()]
            elif key == "q":
                cur["q"] = np.array([int(v) for v in val.split()], dtype=np.int8)
            elif key == "d16":
                cur["d16"] = int(val, 16)
            elif key == "why":
                cur["why"] = val
    for c in cases:
        x = np.array([k * c["unit"] for k in c["k"]], dtype=np.float64)
        assert np.all(x.astype(np.float32).astype(np.float64) == x), c["name"]
        c["x"] = x.astype(np.float32)
        assert c["x"].size == BLOCK and c["q"].size == BLOCK, c["name"]
    return cases


def pin_closed_forms(orc):
    cases = load_closed_forms()
    for c in cases:
        q, d16 = orc.quantize_rows(c["x"][None, :])
        assert np.array_equal(q[0], c["q"]), (c["name"], q[0], c["q"])
        assert int(d16[0, 0]) == c["d16"], (c["name"], hex(int(d16[0, 0])))
    # The same blocks side by side in one row and across rows: each block is
    # quantised on its own, wherever it sits.
    X = np.concatenate([c["x"] for c in cases])[None, :]
    X = np.concatenate([X, X[:, ::-1].copy()], axis=0)
    q, d16 = orc.quantize_rows(X)
    for i, c in enumerate(cases):
        assert np.array_equal(q[0, BLOCK * i:BLOCK * (i + 1)], c["q"]), c["name"]
        assert int(d16[0, i]) == c["d16"], c["name"]
        j = len(cases) - 1 - i  # reversed row: block j holds case i reversed
        assert np.array_equal(q[1, BLOCK * j:BLOCK * (j + 1)], c["q"][::-1]), c["name"]
        assert int(d16[1, j]) == c["d16"], c["name"]


# --------------------------------------------------------------------------
# binary16 conversion
# --------------------------------------------------------------------------

def _f16_boundary_sample() -> np.ndarray:
    """binary32 values at and around every binary16 value and every midpoint
    between consecutive binary16 values, both signs, plus the overflow edge."""
    h = np.arange(0, 0x7c00, dtype=np.uint16)          # finite non-negative
    v = h.view(np.float16).astype(np.float64)
    nxt = np.append(v[1:], 65536.0)                    # next value (inf edge)
    mid = (v + nxt) / 2                                # exact in float64
    pts = np.concatenate([v, mid]).astype(np.float32)  # exact in float32
    up = np.nextafter(pts, np.float32(np.inf))
    dn = np.nextafter(pts, np.float32(0))
    extra = np.array([65504, 65519.99, 65520, 65536, 1e30, 2.0 ** -25,
                      np.nextafter(np.float32(2.0 ** -25), np.float32(1)),
                      2.0 ** -26, 1e-40, 0.0], dtype=np.float32)
    s = np.concatenate([pts, up, dn, extra])
    return np.concatenate([s, -s])


def pin_f16_boundaries(orc):
    x = _f16_boundary_sample()
    got = orc.f32_to_f16_bits(x)
    ref = f16_bits_reference(x)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]


def pin_f16_exhaustive(orc, chunk_bits: int = 26):
    """All 2^32 binary32 patterns (NaNs only need to stay NaN)."""
    step = 1 << chunk_bits
    base = np.arange(step, dtype=np.uint32)
    for c in range(1 << (32 - chunk_bits)):
        bits = base + np.uint32(c * step)
        x = bits.view(np.float32)
        got = orc.f32_to_f16_bits(x)
        ref = f16_bits_reference(x)
        nan = (bits & 0x7f800000) == 0x7f800000
        nan &= (bits & 0x007fffff) != 0
        bad = np.nonzero((got != ref) & ~nan)[0]
        assert bad.size == 0, (hex(int(bits[bad[0]])), hex(got[bad[0]]), hex(ref[bad[0]]))
        gn = got[nan]
        assert np.all(((gn & 0x7c00) == 0x7c00) & ((gn & 0x3ff) != 0))


def pin_f16_to_f32(orc):
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = orc.f16_bits_to_f32(h)
    ref = torch.from_numpy(h.view(np.int16)).view(torch.float16).to(torch.float32).numpy()
    nan = np.isnan(ref)
    assert np.all(np.isnan(got[nan]))
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


# --------------------------------------------------------------------------
# quantisation invariants and the open readings
# --------------------------------------------------------------------------

def pin_quant_invariants(orc, X: np.ndarray):
    X = np.ascontiguousarray(X, dtype=np.float32)
    q, d16, d32 = orc.quantize_rows(X, return_d32=True)
    R, K = X.shape
    xb = X.reshape(R, K // BLOCK, BLOCK).astype(np.float64)
    qb = q.reshape(R, K // BLOCK, BLOCK).astype(np.float64)
    d = d32.astype(np.float64)[..., None]
    a = np.abs(xb).max(axis=-1)
    assert np.all(np.abs(qb) <= 127)
    zero = a == 0
    assert np.all(qb[zero] == 0) and np.all(d16[zero] == 0) and np.all(d32[zero] == 0)
    nz = ~zero
    # d is the correctly rounded a/127: |127 d - a| <= 127 * ulp(d) / 2
    ulp = np.spacing(d32.astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(127.0 * d32.astype(np.float64) - a)[nz] <= 63.5 * ulp[nz])
    # the stored scale is binary16(d), round to nearest even
    assert np.array_equal(d16, f16_bits_reference(d32))
    # signs agree, the largest magnitude maps to +-127
    assert np.all(qb * xb >= 0)
    assert np.all((qb != 0) | zero[..., None] | (np.abs(xb) < d * (0.5 + 2.0 ** -16)))
    j = np.abs(xb).argmax(axis=-1)[..., None]
    qa = np.take_along_axis(qb, j, axis=-1)[..., 0]
    xa = np.take_along_axis(xb, j, axis=-1)[..., 0]
    assert np.all(qa[nz] == 127 * np.sign(xa[nz]))
    # q*d is the nearest grid point up to the rounding of x/d
    err = np.abs(xb - qb * d)
    assert np.all(err[nz] <= (d * (0.5 + 2.0 ** -16))[nz])


def constructed_reading_block():
    """One block whose quantisation separates the open readings.

    absmax = 1, so d = fl(1/127).  The other values were found by a search
    with numpy float32 arithmetic; each one quantises differently under the
    alternative readings, which this function re-verifies before returning.
    Returns (x float32[32], expected q int8[32]).
    """
    f32 = np.float32
    x = np.zeros(BLOCK, dtype=np.float32)
    x[0] = 1.0
    # division vs multiplication by the rounded reciprocal
    recip_cases = [float.fromhex("0x1.60c182p-1")]
    # binary32 scale vs its binary16 rounding
    f16_cases = [0.91729766, 0.4606225, 0.9409342, 0.3503813, 0.6259593]
    vals = recip_cases + f16_cases
    x[1:1 + len(vals)] = np.array(vals, dtype=np.float32)
    x[10:10 + len(vals)] = -x[1:1 + len(vals)]
    d = f32(f32(1.0) / f32(127.0))
    q = half_away(x / d).astype(np.int8)  # numpy float32 division is IEEE
    # the alternatives really differ on these values
    r = f32(f32(1.0) / d)
    q_recip = half_away(x * r)
    d16 = np.float32(np.float16(d))
    q_f16 = half_away(x / d16)
    assert q_recip[1] != q[1] and q_recip[10] != q[10]
    for i in range(2, 1 + len(vals)):
        assert q_f16[i] != q[i] and q_f16[i + 9] != q[i + 9]
    return x, q


def pin_open_readings(orc):
    x, q_expect = constructed_reading_block()
    q, _ = orc.quantize_rows(x[None, :])
    assert np.array_equal(q[0], q_expect), (q[0], q_expect)


# --------------------------------------------------------------------------
# the matmul
# --------------------------------------------------------------------------

def _random_f16_bits(rng, shape):
    """Finite binary16 bit patterns of any sign, subnormals and zero included."""
    h = rng.integers(0, 1 << 16, size=shape, dtype=np.uint32).astype(np.uint16)
    inf_nan = (h & 0x7c00) == 0x7c00
    h[inf_nan] &= 0xbfff  # clear the top exponent bit: finite
    return h


def exact_matmul(qw, dw, qx, dx, batch_index):
    """Y and A in exact rational arithmetic with Python integers."""
    N, K = qw.shape
    KB = K // BLOCK
    wv = f16_value(dw)
    xv = f16_value(dx)
    Y, A = [], []
    for s in batch_index:
        yr, ar = [], []
        for n in range(N):
            y = Fraction(0)
            a = Fraction(0)
            for b in range(KB):
                S = sum(int(qw[n, BLOCK * b + i]) * int(qx[s, BLOCK * b + i])
                        for i in range(BLOCK))
                term = Fraction(S) * Fraction(float(wv[n, b])) * Fraction(float(xv[s, b]))
                y += term
                a += abs(term)
            yr.append(y)
            ar.append(a)
        Y.append(yr)
        A.append(ar)
    return Y, A


def pin_matmul_bruteforce(orc, seed: int = 7):
    rng = np.random.default_rng(seed)
    for K in (32, 64, 96):
        for N in (1, 3, 8):
            n_slots = 5
            qw = rng.integers(-128, 128, size=(N, K), dtype=np.int64).astype(np.int8)
            qx = rng.integers(-128, 128, size=(n_slots, K), dtype=np.int64).astype(np.int8)
            dw = _random_f16_bits(rng, (N, K // BLOCK))
            dx = _random_f16_bits(rng, (n_slots, K // BLOCK))
            bi = np.array([3, 0, 3, 4], dtype=np.int32)[: 1 + (K // 32) % 4 + (N > 1)]
            Y, A = orc.matmul(qw, dw, qx, dx, bi)
            Ye, Ae = exact_matmul(qw, dw, qx, dx, bi)
            KB = K // BLOCK
            for t in range(bi.size):
                for n in range(N):
                    # a double sum of KB exact terms: |error| <= KB 2^-53 A
                    bound = float(Ae[t][n]) * KB * 2.0 ** -52 + 1e-300
                    assert abs(Fraction(Y[t, n]) - Ye[t][n]) <= Fraction(bound), (K, N, t, n)
                    assert abs(Fraction(A[t, n]) - Ae[t][n]) <= Fraction(bound), (K, N, t, n)


def dequantize(q, d16):
    R, K = q.shape
    scale = np.repeat(f16_value(d16), BLOCK, axis=1)
    return q.astype(np.float64) * scale


def pin_matmul_dense(orc, seed: int = 11, K: int = 768, N: int = 96):
    """sum_b dw dx S_b is exactly the dot product of the dequantised rows, so a
    float64 dense matmul must agree to float64 rounding."""
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02))
    X = rng.standard_normal((16, K), dtype=np.float32)
    X[:, rng.choice(K, 8, replace=False)] *= np.float32(20.0)
    qw, dw = orc.quantize_rows(W)
    qx, dx = orc.quantize_rows(X)
    bi = rng.permutation(16)[:9].astype(np.int32)
    Y, A = orc.matmul(qw, dw, qx, dx, bi)
    Wd, Xd = dequantize(qw, dw), dequantize(qx, dx)
    Yd = Xd[bi] @ Wd.T
    mag = np.abs(Xd[bi]) @ np.abs(Wd).T
    assert np.all(np.abs(Y - Yd) <= 1e-10 * mag + 1e-300)
    assert np.all(A <= mag * (1 + 1e-12)) and np.all(A >= np.abs(Y) * (1 - 1e-12))
    # and the quantised product tracks the unquantised one (a sanity check of
    # the encoding, not a parity bound)
    Yf = X[bi].astype(np.float64) @ W.T.astype(np.float64)
    rel = np.linalg.norm(Y - Yf) / np.linalg.norm(Yf)
    assert rel < 0.02, rel


def pin_column_invariance(orc, seed: int = 13, K: int = 256, N: int = 40):
    rng = np.random.default_rng(seed)
    qw = rng.integers(-127, 128, size=(N, K), dtype=np.int64).astype(np.int8)
    qx = rng.integers(-127, 128, size=(16, K), dtype=np.int64).astype(np.int8)
    dw = _random_f16_bits(rng, (N, K // BLOCK)) & 0x7fff
    dx = _random_f16_bits(rng, (16, K // BLOCK)) & 0x7fff
    bi = np.array([5, 2, 15, 2, 0, 9], dtype=np.int32)
    Y, A = orc.matmul(qw, dw, qx, dx, bi)
    for t, s in enumerate(bi):
        y1, a1 = orc.matmul(qw, dw, qx, dx, np.array([s], dtype=np.int32))
        assert np.array_equal(Y[t], y1[0]) and np.array_equal(A[t], a1[0])
    # a row subset returns those rows
    rows = np.array([N - 1, 0, 17, 17], dtype=np.int64)
    Ys, As = orc.matmul(qw, dw, qx, dx, bi, rows=rows)
    assert np.array_equal(Ys, Y[:, rows]) and np.array_equal(As, A[:, rows])
    # the scales enter each term linearly: doubling one row's scales doubles
    # exactly that row
    dw2 = dw.copy()
    v = f16_value(dw2[3])
    ok = np.abs(v) < 30000
    dw2[3, ok] = (v[ok] * 2).astype(np.float16).view(np.uint16)
    Y2, _ = orc.matmul(qw, dw2, qx, dx, bi)
    keep = np.arange(N) != 3
    assert np.array_equal(Y2[:, keep], Y[:, keep])
    if ok.all():
        assert np.array_equal(Y2[:, 3], 2 * Y[:, 3])


def pin_block_dots(orc, seed: int = 17, K: int = 160, N: int = 12):
    rng = np.random.default_rng(seed)
    qw = rng.integers(-128, 128, size=(N, K), dtype=np.int64).astype(np.int8)
    qx = rng.integers(-128, 128, size=(16, K), dtype=np.int64).astype(np.int8)
    bi = np.array([7, 7, 1, 14, 0], dtype=np.int32)
    S = orc.block_dots(qw, qx, bi)
    KB = K // BLOCK
    ref = (qx[bi].reshape(bi.size, 1, KB, BLOCK).astype(np.int64) *
           qw.reshape(1, N, KB, BLOCK).astype(np.int64)).sum(-1)
    assert np.array_equal(S.astype(np.int64), ref)
    # extremes: all -128 gives 32 * 128^2 = 2^19 per block
    qm = np.full((2, 64), -128, dtype=np.int8)
    S2 = orc.block_dots(qm, qm, np.array([1, 0], dtype=np.int32))
    assert np.all(S2 == 1 << 19)
    # and the matmul is the scaled sum of exactly these integers
    dw = _random_f16_bits(rng, (N, KB)) & 0x7fff
    dx = _random_f16_bits(rng, (16, KB)) & 0x7fff
    Y, _ = orc.matmul(qw, dw, qx, dx, bi)
    terms = ref.astype(np.float64) * f16_value(dw)[None] * f16_value(dx)[bi][:, None, :]
    assert np.all(np.abs(Y - terms.sum(-1)) <= 1e-12 * np.abs(terms).sum(-1) + 1e-300)


def pin_bad_slot(orc):
    qw = np.ones((3, 64), dtype=np.int8)
    dw = np.full((3, 2), 0x3c00, dtype=np.uint16)
    qx = np.ones((4, 64), dtype=np.int8)
    dx = np.full((4, 2), 0x3c00, dtype=np.uint16)
    Y, A = orc.matmul(qw, dw, qx, dx, np.array([1, 4, -1, 3], dtype=np.int32))
    assert np.all(Y[[0, 3]] == 64.0) and np.all(A[[0, 3]] == 64.0)
    assert np.all(np.isnan(Y[[1, 2]])) and np.all(np.isnan(A[[1, 2]]))


def edge_blocks():
    """Blocks at the edges of the format, each with the q and binary16 bits
    the stated rules give by hand: (name, x float32 [32], q int8 [32], d16).

    * a NaN or an infinity anywhere in the block: q = 0 and the quiet NaN
      0x7E00 as scale (so every output using the block is NaN);
    * absmax 63 * 2^-149: absmax/127 is below half the smallest subnormal,
      so the scale rounds to +0 and the block is the zero block;
    * absmax 64 * 2^-149: absmax/127 rounds up to 2^-149 (64/127 > 1/2), so
      x = k * 2^-149 gives x/d = k exactly, and binary16(2^-149) = +0;
    * absmax 127 * 2^20: d = 2^20 exactly, beyond binary16's range, so the
      stored scale is +infinity 0x7C00 while q = k."""
    rng = np.random.default_rng(5)
    out = []
    base = (rng.standard_normal(BLOCK) * 3).astype(np.float32)
    zero_q = np.zeros(BLOCK, dtype=np.int8)
    for name, pos, val in (("nan", 7, np.nan), ("neg_nan", 0, -np.nan), ("inf", 31, np.inf),
                           ("neg_inf", 12, -np.inf), ("nan_and_inf", 3, np.nan)):
        x = base.copy()
        x[pos] = np.float32(val)
        if name == "nan_and_inf":
            x[20] = np.float32(-np.inf)
        out.append((name, x, zero_q, 0x7E00))
    k = np.array([(-1) ** i * (i * 2 % 64) for i in range(BLOCK)], dtype=np.int64)
    k63 = k.copy()
    k63[5] = -63
    out.append(("underflow_63", (k63 * 2.0 ** -149).astype(np.float32), zero_q, 0x0000))
    k64 = k.copy()
    k64[9] = 64
    out.append(("smallest_nonzero_scale", (k64 * 2.0 ** -149).astype(np.float32),
                k64.astype(np.int8), 0x0000))
    kb = np.array([(i * 37) % 255 - 127 for i in range(BLOCK)], dtype=np.int64)
    kb[0] = 127
    out.append(("scale_overflows_binary16", (kb * 2.0 ** 20).astype(np.float32),
                kb.astype(np.int8), 0x7C00))
    for name, x, q, _ in out:
        assert x.dtype == np.float32 and x.size == BLOCK and q.size == BLOCK, name
    return out


def pin_edge_blocks(orc):
    cases = edge_blocks()
    for name, x, q, d16 in cases:
        qo, do = orc.quantize_rows(x[None, :])
        assert np.array_equal(qo[0], q), (name, qo[0])
        assert int(do[0, 0]) == d16, (name, hex(int(do[0, 0])))
    # side by side with ordinary blocks: each block keeps its own result
    normal = (np.arange(BLOCK, dtype=np.float32) - 16) * np.float32(0.25)
    row = np.concatenate([np.concatenate([normal, x]) for _, x, _, _ in cases])[None, :]
    qo, do = orc.quantize_rows(row)
    qn, dn = orc.quantize_rows(normal[None, :])
    for i, (name, _, q, d16) in enumerate(cases):
        assert np.array_equal(qo[0, 64 * i:64 * i + 32], qn[0]), name
        assert int(do[0, 2 * i]) == int(dn[0, 0]), name
        assert np.array_equal(qo[0, 64 * i + 32:64 * i + 64], q), name
        assert int(do[0, 2 * i + 1]) == d16, name
    # a NaN-scaled block turns its outputs into NaN, the others stay finite
    qw = np.ones((2, 64), dtype=np.int8)
    dw = np.array([[0x3C00, 0x3C00], [0x3C00, 0x7E00]], dtype=np.uint16)
    qx = np.ones((1, 64), dtype=np.int8)
    dx = np.full((1, 2), 0x3C00, dtype=np.uint16)
    Y, _ = orc.matmul(qw, dw, qx, dx, np.array([0], dtype=np.int32))
    assert Y[0, 0] == 64.0 and np.isnan(Y[0, 1]), Y


FAST_PINS = [
    pin_closed_forms,
    pin_edge_blocks,
    pin_f16_boundaries,
    pin_f16_to_f32,
    pin_open_readings,
    pin_matmul_bruteforce,
    pin_matmul_dense,
    pin_column_invariance,
    pin_block_dots,
    pin_bad_slot,
]


def quant_invariant_inputs(seed: int = 3) -> np.ndarray:
    """Rows with the value mixes the workloads use, plus zero and tiny blocks."""
    rng = np.random.default_rng(seed)
    K = 2048
    X = rng.standard_normal((8, K), dtype=np.float32)
    X[0] *= np.float32(0.02)
    X[1, rng.choice(K, 20, replace=False)] *= np.float32(20.0)
    X[2, :64] = 0.0                                  # two zero blocks
    X[3] *= np.float32(1e-4)                         # binary16-subnormal scales
    X[4] = np.round(X[4] * 8) / 8                    # many exact grid points
    X[5, 32:64] = np.float32(3.5)                    # constant block
    X[6] *= np.float32(1e4)
    X[7, ::2] = -X[7, ::2]
    return X


def pin_quant_invariants_default(orc):
    pin_quant_invariants(orc, quant_invariant_inputs())


FAST_PINS.append(pin_quant_invariants_default)


# --------------------------------------------------------------------------
# pos-vector RoPE
# --------------------------------------------------------------------------

def load_rope_closed_forms(path: str | None = None):
    path = path or os.path.join(GOLDEN, "rope_closed_forms.txt")
    cases = []
    with open(path) as fh:
        for raw in fh:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            head, xs, ys = (p.strip() for p in line.split("|"))
            base, d, pos = head.split()
            cases.append((float(base), int(d), int(pos),
                          np.array([float(v) for v in xs.split()], dtype=np.float32),
                          np.array([float(v) for v in ys.split()], dtype=np.float64)))
    return cases


def pin_rope_closed_forms(orc):
    """Hand-derived rotations: which values pair up, by what angle, which
    signs, and the row's own position (rows of one call carry different
    positions)."""
    cases = load_rope_closed_forms()
    for base, d, pos, x, y in cases:
        out, mag = orc.rope(x[None, :], np.array([pos], dtype=np.int32), 1, d, base)
        assert np.allclose(out[0], y, rtol=0, atol=4e-16), (base, d, pos)
        half = d // 2
        assert np.allclose(mag[0, :half], np.abs(x[:half]) + np.abs(x[half:])), (base, d, pos)
    # several rows of one call, each with its own position
    groups = {}
    for c in cases:
        groups.setdefault((c[0], c[1]), []).append(c)
    mixed = 0
    for (base, d), same in groups.items():
        if len(same) < 2:
            continue
        mixed += len({c[2] for c in same}) > 1
        Y = np.stack([c[3] for c in same])
        out, _ = orc.rope(Y, np.array([c[2] for c in same], dtype=np.int32), 1, d, base)
        for r, c in enumerate(same):
            assert np.allclose(out[r], c[4], rtol=0, atol=4e-16), (base, d, r)
    assert mixed, "no call mixes positions"


def pin_rope_group(orc, seed: int = 23):
    """Rotation-group identities on random heads: the pair norms are kept,
    turning back by -pos restores the input, two turns add their positions,
    and the dot product of two rotated heads depends only on the position
    difference (the relative-position property)."""
    rng = np.random.default_rng(seed)
    H, d, base = 3, 16, 10000.0
    x = rng.standard_normal((4, H * d + 5), dtype=np.float32)  # extra columns are not heads
    pos = np.array([0, 5, 123, 40000], dtype=np.int32)
    out, mag = orc.rope(x, pos, H, d, base)
    half = d // 2
    xa = x[:, :H * d].reshape(4, H, 2, half).astype(np.float64)
    oa = out.reshape(4, H, 2, half)
    assert np.allclose(np.hypot(oa[:, :, 0], oa[:, :, 1]), np.hypot(xa[:, :, 0], xa[:, :, 1]),
                       rtol=1e-12, atol=0)
    back, _ = orc.rope(out.astype(np.float32), -pos, H, d, base)
    assert np.allclose(back, x[:, :H * d], rtol=0, atol=1e-6 * np.max(mag))
    p1, p2 = np.array([3, 7, 11, 2], np.int32), np.array([5, 1, 100, 9], np.int32)
    once, _ = orc.rope(x, p1 + p2, H, d, base)
    twice, _ = orc.rope(orc.rope(x, p1, H, d, base)[0].astype(np.float32), p2, H, d, base)
    assert np.allclose(once, twice, rtol=0, atol=1e-6 * np.max(mag))
    q, k = x[0:1, :H * d], x[1:2, :H * d]
    def dots(m, n):
        rq, _ = orc.rope(q, np.array([m], np.int32), H, d, base)
        rk, _ = orc.rope(k, np.array([n], np.int32), H, d, base)
        return (rq.reshape(H, d) * rk.reshape(H, d)).sum(axis=1)
    assert np.allclose(dots(10, 3), dots(1007, 1000), rtol=1e-9, atol=1e-12)
    assert not np.allclose(dots(10, 3), dots(10, 4), rtol=1e-6)


FAST_PINS += [pin_rope_closed_forms, pin_rope_group]
