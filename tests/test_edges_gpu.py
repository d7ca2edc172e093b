"""The method's edge cases through every launch path of the layer, on MI355X.

Each path decides outliers and rounds codes with its own code: the fused
small-M kernel (M <= 16, K <= 4096), the small-M activation kernels before the
streaming kernel (M <= 16, K > 4096), the column scan with one row block
(16 < M <= 64) and with several (M > 64, before the GEMM).  So every path gets
  * entries of exactly +/-6.0 (outliers: [blog, "A closer look at the MatMul"],
    magnitude 6 or more) and of 5.99609375, the largest fp16 below 6 (not);
  * rows on which the codes are rounding ties ([blog, "Introduction to model
    quantization"]: round half away from zero): absmax 127/32 = 3.96875 makes
    the scale exactly 32, so an entry k/64 with k odd scales to k/2; for
    zero-point codes the range [-3.96875, 4] makes the scale exactly 32 too;
  * NaN entries, which never reach the threshold (a column is an outlier when
    some entry has |x| >= t).
Codes, scales, zero points, the outlier list and X_O must match the oracle bit
for bit, Y within max(2e-3 |Y64|, 1e-2).  Also: the split-K path of the int8
GEMM against the exact integer product.
"""
import zlib

import numpy as np
import pytest

from mixed_precision_quantized_int8_amd import workloads as wl
from oracle import int8_oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

RTOL, ATOL = 2e-3, 1e-2
BELOW6 = np.float16(5.99609375)
TIE_ABSMAX = np.float16(127.0 / 32.0)


@pytest.fixture(scope="module")
def lib(i8l):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    return i8l


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def say(*a):
    print(*a, flush=True)


def assert_y(Yg, Y64, what="", rows=None):
    y = np.asarray(Yg).astype(np.float64)
    if rows is not None:
        y, Y64 = y[rows], Y64[rows]
    err = np.abs(y - Y64)
    tol = np.maximum(RTOL * np.abs(Y64), ATOL)
    bad = ~(err <= tol)
    if bad.any():
        k = np.unravel_index(np.argmax(np.where(bad, err - tol, -np.inf)), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst "
                             f"gpu={y[k]!r} ref={Y64[k]!r} at {k}")


def tie_values(rng, n):
    """n values k/64 with k odd, |k| <= 253: ties once the scale is 32."""
    k = 2 * rng.integers(0, 127, n) + 1
    return (np.where(rng.integers(0, 2, n) == 1, k, -k) / 64.0).astype(np.float16)


def edge_x(M, K, zp, seed):
    """X with threshold-edge columns and tie rows (see the module docstring).

    Returns (X, tie_rows).  Column c6 holds 6.0 in row 0 and column c6n holds
    -6.0 in the last row (both outliers); columns cb, cb + 1 hold +/-5.99609375
    in row 1 (not outliers) when M >= 3; the tie rows are the others."""
    rng = np.random.default_rng(seed)
    X, _ = wl.make_x(M, K, 1.0, 0, 8, 20, seed)
    c6, c6n, cb = K // 3, K // 3 + 37, K // 2 + 5
    tie_rows = [r for r in range(M) if M < 3 or r != 1]
    for r in tie_rows:
        X[r, :] = tie_values(rng, K)
        if zp:
            X[r, 3] = -TIE_ABSMAX          # lo = -3.96875, hi = 4: range 255/32
            X[r, 4] = np.float16(4.0)
        else:
            X[r, 3] = TIE_ABSMAX if r % 2 else -TIE_ABSMAX
    if M >= 3:
        X[1, cb] = BELOW6
        X[1, cb + 1] = -BELOW6
    X[0, c6] = np.float16(6.0)
    X[M - 1, c6n] = np.float16(-6.0)
    return X, tie_rows


# (name, M, K, N): one case per launch path, and the fused kernel's register
# packings (R = 1, 2, 4, 8 k-steps per register set for M = 16, 8, 3 and 1)
PATHS = [
    ("fused_m8_k1024", 8, 1024, 320),
    ("fused_m1_k512", 1, 512, 200),
    ("fused_m16_k4096", 16, 4096, 192),
    ("fused_m3_k2048", 3, 2048, 130),
    ("small_act_m8_k4160", 8, 4160, 256),
    ("stream_m24_k1024", 24, 1024, 300),
    ("gemm_m80_k1040", 80, 1040, 260),
    ("gemm_m300_k272", 300, 272, 520),
]


def _check_absmax(lib, ws, M, K, r, what, rows=None):
    v = lib.workspace_views(ws, M, K)
    n = int(host(v["n_out"])[0])
    assert n == len(r["idx"]), f"{what}: n_out {n} != {len(r['idx'])}"
    np.testing.assert_array_equal(host(v["idx"])[:n], r["idx"], err_msg=f"{what}: idx")
    sel = slice(None) if rows is None else rows
    np.testing.assert_array_equal(host(v["sx"])[sel].view(np.uint32),
                                  r["sx"][sel].view(np.uint32), err_msg=f"{what}: sx")
    np.testing.assert_array_equal(host(v["Xq"])[sel], r["Xq"][sel], err_msg=f"{what}: Xq")
    if n:
        np.testing.assert_array_equal(host(v["X_O"])[:, :n][sel].view(np.uint16),
                                      r["X_O"][sel].view(np.uint16), err_msg=f"{what}: X_O")


def _check_zp(lib, ws, M, K, r, what, rows=None):
    v = lib.workspace_views(ws, M, K)
    n = int(host(v["n_out"])[0])
    assert n == len(r["idx"]), f"{what}: n_out {n} != {len(r['idx'])}"
    np.testing.assert_array_equal(host(v["idx"])[:n], r["idx"], err_msg=f"{what}: idx")
    sel = slice(None) if rows is None else rows
    np.testing.assert_array_equal(host(v["zp"])[sel], r["zp"][sel], err_msg=f"{what}: zp")
    np.testing.assert_array_equal(host(v["sx"])[sel].view(np.uint32),
                                  r["xscale"][sel].view(np.uint32), err_msg=f"{what}: xscale")
    np.testing.assert_array_equal(host(v["Xq"])[sel], r["Xq"][sel], err_msg=f"{what}: Xq")
    if n:
        np.testing.assert_array_equal(host(v["X_O"])[:, :n][sel].view(np.uint16),
                                      r["X_O"][sel].view(np.uint16), err_msg=f"{what}: X_O")


@pytest.mark.parametrize("zp", [False, True], ids=["absmax", "zero_point"])
@pytest.mark.parametrize("case", PATHS, ids=lambda c: c[0])
def test_threshold_and_tie_edges(lib, case, zp):
    name, M, K, N = case
    what = f"{name} {'zero-point' if zp else 'absmax'}"
    say(f"edges {what} M={M} K={K} N={N}")
    seed = zlib.crc32(name.encode()) % 1000
    X, tie_rows = edge_x(M, K, zp, seed)
    W = wl.make_w(K, N, 0.02, seed)
    Xd, Wd = dev(X), dev(W)
    Wq, sw = lib.quantize_weight(Wd)
    ws = lib.new_workspace(M, K, N, Xd.device)
    Wq_o, sw_o = O.quantize_weight(W)
    if zp:
        S = lib.weight_code_sums(Wq)
        Y = lib.linear_zp(Xd, Wq, sw, S, Wd, 6.0, workspace=ws)
        r = O.int8_linear_zp(X, Wq_o, sw_o, W, 6.0)
        # the crafted rows really are ties: scale 32 and half-integer products
        for t in tie_rows:
            assert r["xscale"][t] == np.float32(np.float16(4.0) + TIE_ABSMAX) / np.float32(255)
            assert r["zp"][t] == 127
        _check_zp(lib, ws, M, K, r, what)
    else:
        Y = lib.linear(Xd, Wq, sw, Wd, 6.0, workspace=ws)
        r = O.int8_linear(X, Wq_o, sw_o, W, 6.0)
        for t in tie_rows:
            assert r["sx"][t] == np.float32(TIE_ABSMAX)
        _check_absmax(lib, ws, M, K, r, what)
    expect = sorted({K // 3, K // 3 + 37})
    np.testing.assert_array_equal(r["idx"], expect)   # 6.0 in, 5.99609375 out
    assert_y(host(Y), r["Y64"], what)


# (name, M, K, N): M >= 3 so that the NaN and the large entry sit in other rows;
# the GEMM case puts them 200 rows apart, in different row blocks of the scan
NAN_PATHS = [
    ("fused_m3_k1024", 3, 1024, 256),
    ("fused_m16_k2048", 16, 2048, 128),
    ("small_act_m4_k4160", 4, 4160, 128),
    ("stream_m24_k1024", 24, 1024, 128),
    ("gemm_m300_k1040", 300, 1040, 260),
]


@pytest.mark.parametrize("zp", [False, True], ids=["absmax", "zero_point"])
@pytest.mark.parametrize("case", NAN_PATHS, ids=lambda c: c[0])
def test_nan_entries_never_reach_the_threshold(lib, case, zp):
    """A column with a NaN and a 9.0 in other rows is an outlier (the 9.0 reaches
    6); a column whose only large-looking entry is a NaN is not.  The NaN
    lands in X_O (an outlier column) or in a regular column of its row; rows
    without a NaN in a regular column are compared whole."""
    name, M, K, N = case
    what = f"nan {name} {'zero-point' if zp else 'absmax'}"
    say(f"{what} M={M} K={K} N={N}")
    seed = zlib.crc32(name.encode()) % 1000 + 3
    X, _ = wl.make_x(M, K, 1.0, 0, 8, 20, seed)
    far = min(M - 1, 201)
    ca, cb, cc = 17, K // 2 + 1, K - 9
    X[1, ca] = np.float16(np.nan)
    X[far, ca] = np.float16(9.0)          # outlier column despite the NaN
    X[0, cb] = np.float16(-9.0)           # plain outlier column
    X[2, cc] = np.float16(-np.nan)        # NaN in a regular column: row 2 unspecified
    Xd = dev(X)
    W = wl.make_w(K, N, 0.02, seed)
    Wd = dev(W)
    Wq, sw = lib.quantize_weight(Wd)
    ws = lib.new_workspace(M, K, N, Xd.device)
    Wq_o, sw_o = O.quantize_weight(W)
    clean = np.array([i for i in range(M) if i != 2])
    with np.errstate(invalid="ignore"):
        if zp:
            Y = lib.linear_zp(Xd, Wq, sw, lib.weight_code_sums(Wq), Wd, 6.0, workspace=ws)
            r = O.int8_linear_zp(X, Wq_o, sw_o, W, 6.0)
            _check_zp(lib, ws, M, K, r, what, rows=clean)
        else:
            Y = lib.linear(Xd, Wq, sw, Wd, 6.0, workspace=ws)
            r = O.int8_linear(X, Wq_o, sw_o, W, 6.0)
            _check_absmax(lib, ws, M, K, r, what, rows=clean)
    np.testing.assert_array_equal(r["idx"], sorted([ca, cb]))
    # row 1's NaN sits in an outlier column: its outputs are NaN on both sides
    y = host(Y)
    assert np.isnan(y[1]).all() and np.isnan(r["Y64"][1]).all()
    assert_y(y, r["Y64"], what, rows=np.array([i for i in clean if i != 1]))


# ---------------------------------------------------------------------------------
# the int8 GEMM's split-K path, exact
# ---------------------------------------------------------------------------------
# (M, K, N): 18 tiles split 2 ways; 256 whole tiles + 128 split 2 ways; 30 tiles
# split 4 ways; 32 tiles split 8 ways; 12 tiles split 2 ways with a K tail
@pytest.mark.parametrize("M,K,N", [(520, 2048, 1300), (2048, 2048, 12200), (768, 4096, 2560),
                                   (512, 8192, 4096), (600, 2064, 1000)])
def test_gemm_i32_split_k_bitexact(lib, M, K, N):
    L = lib.workspace_layout(M, K, N)
    say(f"gemm_i32 split-K M={M} K={K} N={N} partial tiles={L['gemm_slices']}")
    assert L["gemm_slices"] > 0
    rng = np.random.default_rng(M + 3 * K + 7 * N)
    Xq = rng.integers(-127, 128, (M, K), dtype=np.int8)
    Wq = rng.integers(-127, 128, (N, K), dtype=np.int8)
    Xq[0, :] = 127                                       # extremes in row 0 / feature 0
    Wq[0, :] = -127
    ws = lib.new_workspace(M, K, N, torch.device("cuda:0"))
    ws.fill_(0xA5)                                       # stale partials must not leak
    Xd, Wd = dev(Xq), dev(Wq)
    acc = lib.gemm_i32(Xd, Wd, workspace=ws)
    ref = O.int8_matmul(Xq, Wq)
    np.testing.assert_array_equal(host(acc), ref)
    # without a workspace: the whole-tile path, the same integers
    np.testing.assert_array_equal(host(lib.gemm_i32(Xd, Wd)), ref)
