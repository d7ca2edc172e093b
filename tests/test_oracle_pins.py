"""Pins of the CPU oracle to facts fixed by the pages or by mathematics.

Each test checks the oracle against something other than itself: numbers the
blog prints for a worked example (fixtures under tests/golden, each with its
citation), crafted cases whose answer follows from the definitions, closed-form
special cases, invariants, an error bound, and pure-Python brute force on tiny
inputs.
"""
import itertools
import math
import struct

import numpy as np
import pytest

from conftest import read_golden
from oracle import int8_oracle as O

INF = float("inf")


# --------------------------------------------------------------------------
# fp16 helpers for the printed tensors (values shown to 4 decimals)
# --------------------------------------------------------------------------
def _all_fp16_nonneg():
    bits = np.arange(0, 0x7C00, dtype=np.uint16)
    return bits.view(np.float16).astype(np.float64)


_FP16 = _all_fp16_nonneg()


def fp16_candidates(shown: float, decimals: int = 4):
    """Every fp16 value that prints as ``shown`` when rounded to ``decimals``."""
    half = 0.5 * 10.0 ** (-decimals)
    mag = abs(shown)
    lo, hi = mag - half, mag + half
    c = _FP16[(_FP16 >= lo - 1e-12) & (_FP16 <= hi + 1e-12)]
    c = c[np.round(c, decimals) == round(mag, decimals)]
    return np.sign(shown) * c if shown != 0 else c


# --------------------------------------------------------------------------
# Worked examples printed on the pages
# --------------------------------------------------------------------------
def test_absmax_vector_example_fp32_and_fp16():
    g = read_golden("absmax_vector.txt")
    v = np.array([float(x) for x in g["input"]], dtype=np.float64)
    want = np.array([int(x) for x in g["codes"]], dtype=np.int8)
    # exact decimal inputs held in fp32
    v32 = v.astype(np.float32)
    got = O.absmax_codes(v32, np.abs(v32).max())
    np.testing.assert_array_equal(got, want)
    # the same vector as an fp16 activation row (decomposition off)
    Xq, sx, idx, X_O = O.quantize_activation(v.astype(np.float16)[None, :], INF)
    np.testing.assert_array_equal(Xq[0], want)
    assert sx[0] == np.float32(np.float16(5.4)) and len(idx) == 0
    # ... and as one column of an fp16 weight
    Wq, sw = O.quantize_weight(v.astype(np.float16)[:, None])
    np.testing.assert_array_equal(Wq[0], want)


def test_fixed_range_example():
    g = read_golden("fixed_range_example.txt")
    absmax = float(g["absmax"][0])
    v = float(g["value"][0])
    code = O.absmax_codes(np.array([v, absmax], np.float32), np.float32(absmax))[0]
    assert code == int(g["code"][0])
    back = code / 127.0
    assert round(back, 4) == float(g["dequant_4dp"][0])
    # the page's stated error is off by 10x; the real error is 7.87e-4
    assert abs(abs(v - back) - float(g["error"][0])) < 1e-12
    assert abs(v - back) < 1e-3
    # fp16 storage of 0.3 does not change the code
    code16 = O.absmax_codes(np.array([np.float16(v)], np.float32), np.float32(1.0))[0]
    assert code16 == 38


def _usage_printout():
    g = read_golden("usage_weight_printout.txt")
    rows = [0, 1, 2, 61, 62, 63]
    w = {r: [float(x) for x in g[f"fp16 {r}"]] for r in rows}
    q = {r: [int(x) for x in g[f"int8 {r}"]] for r in rows}
    d = {r: [float(x) for x in g[f"dequant {r}"]] for r in rows}
    return rows, w, q, d


def test_usage_weight_row2_full_pin():
    """Row 2 shows its own absmax (-0.1227 -> -127): every fp16 value consistent
    with the printout, with that absmax, gives exactly the printed codes."""
    rows, w, q, _ = _usage_printout()
    vals, codes = w[2], q[2]
    amax_cands = fp16_candidates(-0.1227)
    assert len(amax_cands) >= 1
    for a in amax_cands:
        for v, c in zip(vals, codes):
            cands = fp16_candidates(v)
            cands = cands[np.abs(cands) <= abs(a)]
            assert len(cands) >= 1
            # one weight column per candidate, holding the absmax element as well
            K = 2
            W = np.zeros((K, len(cands)), dtype=np.float16)
            W[0, :] = cands.astype(np.float16)
            W[1, :] = np.float16(a)
            Wq, sw = O.quantize_weight(W)
            assert np.all(sw == np.float32(abs(np.float16(a))))
            np.testing.assert_array_equal(Wq[:, 0], np.full(len(cands), c, np.int8))
            np.testing.assert_array_equal(Wq[:, 1], np.full(len(cands), -127, np.int8))


def _feasible_absmax(vals, codes):
    """fp16 absmax values (>= every visible |v|) under which the oracle reproduces
    the printed codes for at least one fp16 reading of each visible value."""
    lo = max(abs(v) for v in vals)
    cands_s = _FP16[(_FP16 >= lo - 1e-4) & (_FP16 <= 0.2)]
    ok = []
    for s in cands_s:
        good = True
        for v, c in zip(vals, codes):
            cv = fp16_candidates(v)
            cv = cv[np.abs(cv) <= s]
            if len(cv) == 0:
                good = False
                break
            got = O.absmax_codes(cv.astype(np.float32), np.float32(s))
            if not np.any(got == c):
                good = False
                break
        if good:
            ok.append(s)
    return np.array(ok)


def test_usage_weight_rows_share_one_absmax():
    """For each printed row the visible codes are reproduced by a single absmax."""
    rows, w, q, _ = _usage_printout()
    for r in rows:
        feas = _feasible_absmax(w[r], q[r])
        assert len(feas) > 0, r


def test_usage_dequant_printout_broadcasts_scale_on_the_input_axis():
    """The printed CB*SCB/127 tensor scales column j by row j's absmax (a
    transposed broadcast on a square layer); the oracle scales by the output row.

    The factor implied by the printed dequant, D*127/CB, is constant down each
    printed column and lies in the absmax range feasible for the row with the
    same index; it is not constant along rows.
    """
    rows, w, q, d = _usage_printout()
    feas = {r: _feasible_absmax(w[r], q[r]) for r in rows}
    for j, col in enumerate(rows):
        lo, hi = -np.inf, np.inf
        for r in rows:
            c = q[r][j]
            D = d[r][j]
            a, b = 127 * (D - 5e-5) / c, 127 * (D + 5e-5) / c
            lo, hi = max(lo, min(a, b)), min(hi, max(a, b))
        assert lo <= hi, (col, lo, hi)
        f = feas[col]
        assert np.any((f >= lo - 1e-4) & (f <= hi + 1e-4)), (col, lo, hi, f.min(), f.max())
    # row-wise reading: row 2's implied factors differ between its columns
    f2 = [127 * d[2][j] / q[2][j] for j in range(6)]
    assert max(f2) - min(f2) > 5e-3
    # the oracle's dequant uses the output-row scale: row 2 of CB with the
    # row's own absmax comes back close to the printed fp16 row, not to the
    # printed dequant row
    s2 = np.float32(np.float16(0.1227))
    back = O.dequantize_weight(np.array([q[2]], np.int8), np.array([s2]))[:, 0]
    assert np.all(np.abs(back.astype(np.float64) - np.array(w[2])) <= s2 / 254 + 1e-4)
    assert np.any(np.abs(back.astype(np.float64) - np.array(d[2])) > 2e-3)


# --------------------------------------------------------------------------
# Crafted cases fixed by the definitions
# --------------------------------------------------------------------------
def test_round_half_away_from_zero_ties():
    # absmax 127/32 makes the scale exactly 32, so k/64 lands on k/2
    s = 127.0 / 32.0
    assert float(np.float16(s)) == s
    vals = np.array([5, -5, 3, 7, 9, -9, 1, 0], dtype=np.float64) / 64.0
    row = np.concatenate([vals, [s]]).astype(np.float16)
    want = np.array([3, -3, 2, 4, 5, -5, 1, 0, 127], dtype=np.int8)   # RNE would give 2,-2,2,4,4,-4,0
    Xq, sx, _, _ = O.quantize_activation(row[None, :], 6.0)
    np.testing.assert_array_equal(Xq[0], want)
    Wq, sw = O.quantize_weight(row[:, None])
    np.testing.assert_array_equal(Wq[0], want)


def test_threshold_boundary_is_inclusive():
    X = np.zeros((3, 5), dtype=np.float16)
    X[:, :] = 0.25
    X[1, 1] = 6.0                       # exactly the threshold: outlier
    X[2, 2] = np.float16(5.99609375)    # largest fp16 below 6: not an outlier
    X[0, 3] = -6.0                      # magnitude counts
    idx = O.outlier_columns(X, 6.0)
    np.testing.assert_array_equal(idx, [1, 3])
    Xq, sx, idx2, X_O = O.quantize_activation(X, 6.0)
    np.testing.assert_array_equal(X_O, X[:, [1, 3]])
    assert np.all(Xq[:, [1, 3]] == 0)
    # the whole column goes to fp16, also for rows whose entry there is small
    assert X_O[0, 0] == np.float16(0.25) and X_O[2, 1] == np.float16(0.25)
    # 5.996 stays in the int8 part and sets row 2's scale
    assert sx[2] == np.float32(np.float16(5.99609375)) and Xq[2, 2] == 127


def test_nan_and_inf_columns():
    """r12: a column is an outlier when some entry has |x| >= t; NaN >= t is
    false, so a NaN alone never makes an outlier and does not hide a large
    entry beside it; an infinity reaches any finite t."""
    X = np.full((3, 6), 0.5, dtype=np.float16)
    X[0, 1] = np.nan                  # NaN alone
    X[1, 2] = np.nan                  # NaN beside an outlier-sized value
    X[2, 2] = 9.0
    X[2, 3] = 9.0                     # a plain outlier column
    X[1, 4] = -np.inf                 # infinity: an outlier for finite thresholds
    X[0, 5] = np.float16(-np.nan)     # a negative NaN pattern (sign bit set)
    np.testing.assert_array_equal(O.outlier_columns(X, 6.0), [2, 3, 4])
    np.testing.assert_array_equal(O.outlier_columns(X, 60000.0), [4])
    assert len(O.outlier_columns(X, np.inf)) == 0


def test_threshold_disabled_values():
    X = np.full((2, 4), 7.0, dtype=np.float16)
    for t in (0.0, -1.0, INF):
        assert len(O.outlier_columns(X, t)) == 0
    with pytest.raises(ValueError):
        O.outlier_columns(X, float("nan"))


def test_zero_rows_and_columns():
    X = np.zeros((3, 8), dtype=np.float16)
    X[1, :] = np.linspace(-1, 1, 8)
    W = np.zeros((8, 4), dtype=np.float16)
    W[:, 2] = np.linspace(-0.5, 0.5, 8)
    Wq, sw = O.quantize_weight(W)
    assert np.all(Wq[[0, 1, 3]] == 0) and np.all(sw[[0, 1, 3]] == 0)
    r = O.int8_linear(X, Wq, sw, W, 6.0)
    assert np.all(r["Xq"][[0, 2]] == 0) and np.all(r["sx"][[0, 2]] == 0)
    assert np.all(r["Y"][[0, 2]] == 0) and np.all(r["Y"][:, [0, 1, 3]] == 0)


def test_all_columns_outliers_equals_fp16_matmul():
    """With a threshold at the smallest fp16 subnormal every nonzero column is an
    outlier: the int8 part vanishes and Y is the plain matrix product."""
    rng = np.random.default_rng(7)
    M, K, N = 5, 24, 7
    X = rng.standard_normal((M, K)).astype(np.float16)
    W = (0.02 * rng.standard_normal((K, N))).astype(np.float16)
    Wq, sw = O.quantize_weight(W)
    r = O.int8_linear(X, Wq, sw, W, 2.0**-24)
    np.testing.assert_array_equal(r["idx"], np.arange(K))
    assert np.all(r["Xq"] == 0) and np.all(r["sx"] == 0) and np.all(r["acc"] == 0)
    exact = X.astype(np.float64) @ W.astype(np.float64)
    np.testing.assert_allclose(r["Y64"], exact, rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(r["Y"], exact.astype(np.float16))


# --------------------------------------------------------------------------
# Brute force on tiny inputs (pure Python, independent arithmetic)
# --------------------------------------------------------------------------
def _f32(x: float) -> float:
    return struct.unpack("f", struct.pack("f", x))[0]


def _bf_code(x: float, s: float) -> int:
    """Pure-Python absmax code: fp32 quotient, fp32 product (both correctly
    rounded through fp64, which is exact for these fp32 operands), ties away."""
    if s == 0.0:
        return 0
    inv = _f32(127.0 / s)
    v = _f32(x * inv)
    r = math.floor(abs(v) + 0.5)
    r = min(r, 127)
    return int(math.copysign(r, v)) if r else 0


def _bf_linear(X, W, t):
    M, K = len(X), len(X[0])
    N = len(W[0])
    outl = [k for k in range(K) if t > 0 and t != INF and max(abs(X[i][k]) for i in range(M)) >= t]
    reg = [k for k in range(K) if k not in outl]
    sw = [max(abs(W[k][n]) for k in range(K)) for n in range(N)]
    Wq = [[_bf_code(W[k][n], sw[n]) for k in range(K)] for n in range(N)]
    sx = [max([abs(X[i][k]) for k in reg], default=0.0) for i in range(M)]
    Xq = [[_bf_code(X[i][k], sx[i]) if k in reg else 0 for k in range(K)] for i in range(M)]
    acc = [[sum(Xq[i][k] * Wq[n][k] for k in range(K)) for n in range(N)] for i in range(M)]
    Y = [[0.0] * N for _ in range(M)]
    for i in range(M):
        for n in range(N):
            y = acc[i][n] * sx[i] * sw[n] / 16129.0
            y += math.fsum(X[i][k] * W[k][n] for k in outl)
            Y[i][n] = y
    return outl, sx, Xq, sw, Wq, acc, Y


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_bruteforce_tiny(seed):
    rng = np.random.default_rng(100 + seed)
    M, K, N = 3 + seed, 16, 5
    X = rng.standard_normal((M, K)).astype(np.float16)
    X[:, rng.choice(K, seed, replace=False)] = np.float16(7.5)
    X[0, 3] = np.float16(-6.0) if seed % 2 else X[0, 3]
    W = (0.05 * rng.standard_normal((K, N))).astype(np.float16)
    Xl = X.astype(np.float64).tolist()
    Wl = W.astype(np.float64).tolist()
    outl, sx, Xq, sw, Wq, acc, Y = _bf_linear(Xl, Wl, 6.0)
    oWq, osw = O.quantize_weight(W)
    np.testing.assert_array_equal(oWq, np.array(Wq, np.int8))
    np.testing.assert_array_equal(osw, np.array(sw, np.float32))
    r = O.int8_linear(X, oWq, osw, W, 6.0)
    np.testing.assert_array_equal(r["idx"], outl)
    np.testing.assert_array_equal(r["sx"], np.array(sx, np.float32))
    np.testing.assert_array_equal(r["Xq"], np.array(Xq, np.int8))
    np.testing.assert_array_equal(r["acc"], np.array(acc, np.int64))
    np.testing.assert_allclose(r["Y64"], np.array(Y), rtol=1e-12, atol=1e-14)


def test_int8_matmul_bruteforce_extremes():
    """acc is exact for extreme codes (K*127^2 accumulations, signs mixed)."""
    K = 4096
    Xq = np.full((2, K), 127, np.int8)
    Xq[1, ::2] = -127
    Wq = np.full((3, K), -127, np.int8)
    Wq[2, 1::3] = 127
    acc = O.int8_matmul(Xq, Wq)
    want = [[sum(int(a) * int(b) for a, b in zip(Xq[i], Wq[n])) for n in range(3)] for i in range(2)]
    np.testing.assert_array_equal(acc, np.array(want))


# --------------------------------------------------------------------------
# Invariants and the error bound
# --------------------------------------------------------------------------
def _case(seed, M=12, K=96, N=20, n_out=3):
    rng = np.random.default_rng(seed)
    X = np.clip(rng.standard_normal((M, K)), -5.75, 5.75).astype(np.float16)
    cols = rng.choice(K, n_out, replace=False)
    X[:, cols] = (rng.uniform(8, 20, (M, n_out)) * rng.choice([-1, 1], (M, n_out))).astype(np.float16)
    W = (0.02 * rng.standard_normal((K, N)) * rng.uniform(0.2, 3.0, N)).astype(np.float16)
    return X, W, np.sort(cols)


@pytest.mark.parametrize("seed", [11, 12, 13])
def test_error_bound_against_exact_product(seed):
    """Every code is within half a step of its scaled value, so
    |Y64 - X@W| <= sum over regular k of (|X| sw/254 + sx |W|/254 + 3 sx sw/254^2)."""
    X, W, cols = _case(seed)
    Wq, sw = O.quantize_weight(W)
    r = O.int8_linear(X, Wq, sw, W, 6.0)
    np.testing.assert_array_equal(r["idx"], cols)
    Xf, Wf = X.astype(np.float64), W.astype(np.float64)
    exact = Xf @ Wf
    reg = np.ones(X.shape[1], bool)
    reg[cols] = False
    sx = r["sx"].astype(np.float64)[:, None]
    swv = sw.astype(np.float64)[None, :]
    bound = (np.abs(Xf[:, reg]) @ np.ones((reg.sum(), 1))) * swv / 254 \
        + sx * (np.ones((1, reg.sum())) @ np.abs(Wf[reg])) / 254 \
        + reg.sum() * 3 * sx * swv / 254**2
    err = np.abs(r["Y64"] - exact)
    assert np.all(err <= bound * (1 + 1e-3) + 1e-12)
    # the outlier part is carried exactly: drop it and the bound breaks
    assert np.any(np.abs(r["Y64"] - r["Yo"] - exact) > bound)
    # row scales never include an outlier column
    assert np.all(r["sx"] < 6.0)


def test_square_nonsymmetric_weight_axis():
    """Scales belong to output features: on a square weight whose columns have
    very different ranges, dequantized codes come back within half a step."""
    rng = np.random.default_rng(5)
    K = N = 32
    W = (rng.standard_normal((K, N)) * np.logspace(-3, 0, N)[None, :]).astype(np.float16)
    Wq, sw = O.quantize_weight(W)
    np.testing.assert_array_equal(sw, np.abs(W.astype(np.float32)).max(axis=0))
    back = O.dequantize_weight(Wq, sw).astype(np.float64)
    step = sw.astype(np.float64)[None, :] / 254
    assert np.all(np.abs(back - W.astype(np.float64)) <= step * 1.01 + 1e-3 * np.abs(W) + 1e-7)


def test_zero_outliers_equals_pure_vectorwise_int8():
    """With no column reaching the threshold the layer is plain vector-wise int8:
    threshold 6 and a disabled decomposition give identical results."""
    X, W, _ = _case(21, n_out=0)
    Wq, sw = O.quantize_weight(W)
    a = O.int8_linear(X, Wq, sw, W, 6.0)
    b = O.int8_linear(X, Wq, sw, W, INF)
    assert len(a["idx"]) == 0
    for k in ("Xq", "sx", "acc"):
        np.testing.assert_array_equal(a[k], b[k])
    np.testing.assert_array_equal(a["Y"], b["Y"])


def test_power_of_two_scaling():
    X, W, cols = _case(31, n_out=0)
    X = (X.astype(np.float32) * 0.5).astype(np.float16)      # |x| <= 2.875 < 3
    Wq, sw = O.quantize_weight(W)
    a = O.int8_linear(X, Wq, sw, W, 6.0)
    X2 = X.copy()
    X2[4] = (X2[4].astype(np.float32) * 2).astype(np.float16)
    b = O.int8_linear(X2, Wq, sw, W, 6.0)
    np.testing.assert_array_equal(a["Xq"], b["Xq"])
    assert b["sx"][4] == 2 * a["sx"][4]
    np.testing.assert_array_equal(b["Y64"][4], 2 * a["Y64"][4])
    W2 = W.copy()
    W2[:, 3] = (W2[:, 3].astype(np.float32) * 4).astype(np.float16)
    Wq2, sw2 = O.quantize_weight(W2)
    np.testing.assert_array_equal(Wq, Wq2)
    assert sw2[3] == 4 * sw[3]


def test_joint_k_permutation():
    X, W, cols = _case(41)
    Wq, sw = O.quantize_weight(W)
    a = O.int8_linear(X, Wq, sw, W, 6.0)
    perm = np.random.default_rng(3).permutation(X.shape[1])
    Xp, Wp = X[:, perm], W[perm]
    Wqp, swp = O.quantize_weight(Wp)
    b = O.int8_linear(Xp, Wqp, swp, Wp, 6.0)
    inv = np.argsort(perm)
    np.testing.assert_array_equal(np.sort(inv[a["idx"]]), b["idx"])
    np.testing.assert_array_equal(a["acc"], b["acc"])
    np.testing.assert_array_equal(a["Xq"][:, perm], b["Xq"])
    np.testing.assert_allclose(a["Y64"], b["Y64"], rtol=1e-12)


def test_rows_independent_given_outlier_set():
    X, W, cols = _case(51)
    Wq, sw = O.quantize_weight(W)
    a = O.int8_linear(X, Wq, sw, W, 6.0)
    b = O.int8_linear(X[3:7], Wq, sw, W, 6.0)
    np.testing.assert_array_equal(a["idx"], b["idx"])
    np.testing.assert_array_equal(a["Y"][3:7], b["Y"])


def test_sampled_entries_match_full():
    X, W, cols = _case(61, M=9, K=64, N=33)
    Wq, sw = O.quantize_weight(W)
    full = O.int8_linear(X, Wq, sw, W, 6.0)
    rng = np.random.default_rng(0)
    rows = rng.integers(0, 9, 50)
    cs = rng.integers(0, 33, 50)
    Wq_r, sw_r = O.quantize_weight_rows(W, cs)
    acc, Y64 = O.int8_linear_entries(X, Wq_r, sw_r, W, 6.0, rows, cs)
    np.testing.assert_array_equal(acc, full["acc"][rows, cs])
    np.testing.assert_allclose(Y64, full["Y64"][rows, cs], rtol=1e-12, atol=1e-15)


def test_dequantize_weight_closed_forms():
    """Rebuilt weight rows (no fp16 copy kept): fp16(fl32(q * s) / 127), indexed
    by the output feature.  Scales that make the result exact pin the formula."""
    q = np.array([[127, -127, 1, 0, -64, 5],
                  [127, -1, 32, 64, -32, 96]], dtype=np.int8)        # Wq [N=2][K=6]
    sw = np.array([127.0, 127.0 / 32.0], dtype=np.float32)          # both fp16-exact
    W = O.dequantize_weight(q, sw)                                    # [K][N]
    assert W.shape == (6, 2) and W.dtype == np.float16
    np.testing.assert_array_equal(W[:, 0], q[0].astype(np.float16))   # s = 127: w = q
    np.testing.assert_array_equal(W[:, 1], (q[1] / 32.0).astype(np.float16))   # q / 32
    # an inexact case: 1 * 0.1 / 127 in fp32, then fp16
    w = O.dequantize_weight(np.array([[1]], np.int8), np.array([np.float32(np.float16(0.1))]))
    want = np.float16(np.float32(np.float32(np.float16(0.1)) / np.float32(127)))
    assert w[0, 0] == want
    # round trip: within half a code step of the original weight
    rng = np.random.default_rng(5)
    W0 = (rng.standard_normal((40, 9)) * 0.02).astype(np.float16)
    Wq, s = O.quantize_weight(W0)
    back = O.dequantize_weight(Wq, s).astype(np.float64)
    assert np.all(np.abs(back - W0) <= s.astype(np.float64)[None, :] / 254 * 1.001
                  + np.abs(W0) * 2.0 ** -11 + 1e-8)


def test_bias_added_before_the_single_rounding():
    rng = np.random.default_rng(8)
    K, N = 64, 24
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float16)
    b = (rng.standard_normal(N) * 3).astype(np.float16)
    Wq, sw = O.quantize_weight(W)
    # X = 0: every product vanishes and Y is the bias itself
    r = O.int8_linear(np.zeros((3, K), np.float16), Wq, sw, W, 6.0, bias=b)
    np.testing.assert_array_equal(r["Y"], np.broadcast_to(b, (3, N)))
    # otherwise Y64 moves by exactly the bias, and Y is one rounding of the sum
    X = (rng.standard_normal((5, K))).astype(np.float16)
    X[:, 3] = 9.0
    a0 = O.int8_linear(X, Wq, sw, W, 6.0)
    a1 = O.int8_linear(X, Wq, sw, W, 6.0, bias=b)
    np.testing.assert_allclose(a1["Y64"] - a0["Y64"], np.broadcast_to(b, (5, N)).astype(np.float64),
                               rtol=0, atol=1e-12)
    np.testing.assert_array_equal(a1["Y"], a1["Y64"].astype(np.float16))
    _, y = O.int8_linear_entries(X, Wq[[2, 7]], sw[[2, 7]], W, 6.0, [1, 4], [2, 7], bias=b)
    np.testing.assert_allclose(y, a1["Y64"][[1, 4], [2, 7]], rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# Zero-point variant (unsigned codes with a zero point)
# --------------------------------------------------------------------------
def test_zero_point_codes_closed_forms():
    # range [-1, 1]: inv = 127.5, zp = RHAZ(127.5) = 128; 0 maps to the zero point
    X = np.array([[-1.0, 0.5, 0.25, 1.0, 0.0]], np.float16)
    Xq, zp, xs, idx, _ = O.quantize_activation_zp(X, 6.0)
    q = Xq.astype(np.int32) + 128
    assert len(idx) == 0 and zp[0] == 128
    np.testing.assert_array_equal(q[0], [0, 192, 160, 255, 128])      # 1.0 -> 256 -> 255
    assert xs[0] == np.float32(2.0) / np.float32(255)
    # all-positive row: the range is widened to 0, so zp = 0
    Xq, zp, xs, _, _ = O.quantize_activation_zp(np.array([[0.5, 2.0]], np.float16), 6.0)
    assert zp[0] == 0
    np.testing.assert_array_equal(Xq[0].astype(np.int32) + 128, [64, 255])
    # zero row: every code is the zero point 0
    Xq, zp, xs, _, _ = O.quantize_activation_zp(np.zeros((1, 4), np.float16), 6.0)
    assert zp[0] == 0 and xs[0] == 0 and np.all(Xq == -128)
    # outlier column: excluded from the range, its code is the zero point
    X = np.array([[-0.5, 7.0, 1.5], [0.25, -8.0, 0.75]], np.float16)
    Xq, zp, xs, idx, X_O = O.quantize_activation_zp(X, 6.0)
    np.testing.assert_array_equal(idx, [1])
    np.testing.assert_array_equal(Xq[:, 1].astype(np.int32) + 128, zp)
    np.testing.assert_array_equal(X_O[:, 0], X[:, 1])
    assert xs[0] == np.float32(2.0) / np.float32(255)                 # [-0.5, 1.5]
    assert xs[1] == np.float32(0.75) / np.float32(255)                # [0, 0.75]


def test_zero_point_round_trip_and_layer_identity():
    rng = np.random.default_rng(17)
    M, K, N = 6, 96, 20
    X = (rng.standard_normal((M, K)) * 1.5 + 0.7).astype(np.float16)    # off-centre rows
    X[:, 9] = 9.0
    W = (rng.standard_normal((K, N)) * 0.05).astype(np.float16)
    b = (rng.standard_normal(N)).astype(np.float16)
    Wq, sw = O.quantize_weight(W)
    Xq, zp, xs, idx, X_O = O.quantize_activation_zp(X, 6.0)
    reg = np.ones(K, bool)
    reg[idx] = False
    deq = (Xq.astype(np.float64) + 128 - zp[:, None]) * xs.astype(np.float64)[:, None]
    err = np.abs(deq - X.astype(np.float64))[:, reg]
    step = np.broadcast_to(xs.astype(np.float64)[:, None], (M, K))[:, reg]
    # q - zp is RHAZ(fl(x * inv)): half a step, plus the three fp32 roundings in
    # inv = fl(255 / range), fl(x * inv) and xscale = fl(range / 255), each at
    # most 2^-24 relative to |x|; where the clamp to [0, 255] bites at the ends of
    # the range, one step more
    ax = np.abs(X.astype(np.float64))[:, reg]
    fp = 4 * 2.0 ** -24 * ax
    q = Xq.astype(np.int32)[:, reg] + 128
    inner = (q > 0) & (q < 255)
    assert inner.sum() > 0.9 * inner.size
    assert np.all(err[inner] <= (0.5 * step + fp)[inner])
    assert np.all(err <= 1.5 * step + fp)
    # signed storage: sum (q-128) w + (128 - zp) S = sum (q - zp) w, exactly
    S = O.weight_code_sums(Wq)
    lhs = Xq.astype(np.int64) @ Wq.astype(np.int64).T + (128 - zp.astype(np.int64))[:, None] * S
    r = O.int8_linear_zp(X, Wq, sw, W, 6.0, bias=b)
    np.testing.assert_array_equal(lhs, r["acc"])
    # the layer equals the product of the dequantized operands (plus outliers, bias)
    Wd = Wq.astype(np.float64).T * sw.astype(np.float64)[None, :] / 127
    ref = deq[:, reg] @ Wd[reg] + X[:, idx].astype(np.float64) @ W[idx].astype(np.float64) + b
    np.testing.assert_allclose(r["Y64"], ref, rtol=1e-12, atol=1e-12)


def test_zero_point_sampled_entries_match_full():
    rng = np.random.default_rng(23)
    M, K, N = 9, 160, 24
    X = (rng.standard_normal((M, K)) + 0.8).astype(np.float16)
    X[:, [3, 77]] = np.float16(7.5)
    W = (rng.standard_normal((K, N)) * 0.04).astype(np.float16)
    b = rng.standard_normal(N).astype(np.float16)
    Wq, sw = O.quantize_weight(W)
    full = O.int8_linear_zp(X, Wq, sw, W, 6.0, bias=b)
    rows, cols = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    rows, cols = rows.ravel(), cols.ravel()
    act = O.quantize_activation_zp(X, 6.0)
    acc, y = O.int8_linear_zp_entries(act, Wq[cols], sw[cols], W, rows, cols, bias=b)
    np.testing.assert_array_equal(acc, full["acc"][rows, cols])
    np.testing.assert_allclose(y, full["Y64"][rows, cols], rtol=1e-13, atol=1e-13)
