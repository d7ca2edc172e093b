"""Parity of the HIP path (through the C ABI) with the CPU oracle on MI355X.

Integer work (outlier sets, codes, scales, int32 accumulators) must match
bit-exactly; fp16 outputs must satisfy |Y - Y64| <= max(2e-3 |Y64|, 1e-2)
against the oracle's fp64 value, with infinities matching exactly.
"""
import math
import zlib

import numpy as np
import pytest

from mixed_precision_quantized_int8_amd import workloads as wl
from oracle import int8_oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

RTOL, ATOL = 2e-3, 1e-2


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


def assert_y(Yg, Y64, Y16=None, what=""):
    Yg = np.asarray(Yg)
    y = Yg.astype(np.float64)
    if Y16 is None:
        with np.errstate(over="ignore"):
            Y16 = Y64.astype(np.float16)
    inf = np.isinf(Y16)
    np.testing.assert_array_equal(Yg[inf], Y16[inf], err_msg=f"{what}: infinities differ")
    fin = ~inf
    err = np.abs(y[fin] - Y64[fin])
    tol = np.maximum(RTOL * np.abs(Y64[fin]), ATOL)
    bad = ~(err <= tol)
    if bad.any():
        k = np.argmax(err - tol)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst "
                             f"gpu={y[fin][k]!r} ref={Y64[fin][k]!r}")


def check_workspace(lib, ws, M, K, act, what=""):
    Xq_o, sx_o, idx_o, XO_o = act
    v = lib.workspace_views(ws, M, K)
    n = int(host(v["n_out"])[0])
    assert n == len(idx_o), f"{what}: n_out {n} != {len(idx_o)}"
    np.testing.assert_array_equal(host(v["idx"])[:n], idx_o, err_msg=f"{what}: idx")
    np.testing.assert_array_equal(host(v["sx"]).view(np.uint32), sx_o.view(np.uint32),
                                  err_msg=f"{what}: sx")
    np.testing.assert_array_equal(host(v["Xq"]), Xq_o, err_msg=f"{what}: Xq")
    if n:
        np.testing.assert_array_equal(host(v["X_O"])[:, :n].view(np.uint16),
                                      XO_o.view(np.uint16), err_msg=f"{what}: X_O")


def run_linear(lib, X, W, t, pass_w=True):
    Xd, Wd = dev(X), dev(W)
    Wq, sw = lib.quantize_weight(Wd)
    M, K = X.shape
    N = W.shape[1]
    ws = lib.new_workspace(M, K, N, Xd.device)
    Y = lib.linear(Xd, Wq, sw, Wd if pass_w else None, t, workspace=ws)
    return Y, Wq, sw, ws


# ---------------------------------------------------------------------------------
# weight quantization
# ---------------------------------------------------------------------------------
@pytest.mark.parametrize("K,N,seed", [(1024, 4096, 1), (4096, 16384, 2), (272, 520, 3),
                                      (64, 7, 4), (16, 1, 5), (1040, 33, 6)])
def test_quantize_weight_bitexact(lib, K, N, seed):
    say(f"quantize_weight K={K} N={N}")
    W = wl.make_w(K, N, 0.02, seed)
    if N > 3:
        W[:, 1] = 0                                  # absmax 0
        W[:, 2] = 0
        W[0, 2] = np.float16(127 / 32)               # scale exactly 32: ties
        W[1:6, 2] = np.array([5, -5, 7, 9, -9], np.float16) / np.float16(64)
    Wq, sw = lib.quantize_weight(dev(W))
    Wq_o, sw_o = O.quantize_weight(W)
    np.testing.assert_array_equal(host(sw).view(np.uint32), sw_o.view(np.uint32))
    np.testing.assert_array_equal(host(Wq), Wq_o)


# ---------------------------------------------------------------------------------
# activation stage (stage export)
# ---------------------------------------------------------------------------------
def _rowpass_x(M, K, seed):
    """X with whole outlier columns plus rows whose largest entry below the
    threshold lies in a column that another row makes an outlier."""
    X, c = wl.make_x(M, K, 0.5, 3, 8, 20, seed)
    p, p2, q = 11, 40, 41            # partial outlier columns p, p2; regular column q
    X[:, [p, p2, q]] = np.clip(X[:, [p, p2, q]], -1, 1)
    X[0, p] = 7.0                    # p is an outlier column because of row 0 ...
    X[5, p] = np.float16(5.9)        # ... and holds row 5's largest entry below 6
    X[1, p2] = -9.0
    X[6, p2] = np.float16(5.5)       # a tie: 5.5 in outlier column p2 and regular q
    X[6, q] = np.float16(-5.5)
    X[7, p] = np.nan                 # a NaN in an outlier column
    X[9, q] = np.float16(5.99609375)  # largest in a regular column: exact provisional scale
    X[10, p] = 6.0                   # exactly the threshold, in an outlier column
    X[M - 1, K - 1] = 6.0            # a last outlier column, set by the last row only
    X[M - 2, K - 1] = np.float16(5.8)
    return X, sorted(set(c) | {p, p2, K - 1})


def _act_cases():
    yield "tiny", *wl.make_x(16, 1024, 1.0, 2, 8, 20, 1), 6.0
    yield "decode", *wl.make_x(8, 4096, 1.0, 4, 6.5, 40, 2), 6.0
    yield "ragged", *wl.make_x(300, 272, 1.0, 5, 8, 20, 3), 6.0
    yield "one_row", *wl.make_x(1, 16, 1.0, 0, 8, 20, 4), 6.0
    yield "k_mod32_16", *wl.make_x(17, 1040, 1.0, 3, 8, 20, 5), 6.0
    yield "many_outliers", *wl.make_x(40, 512, 1.0, 45, 8, 20, 6), 6.0
    # wide rows at M <= 16 (512-column slices)
    yield "k_24576", *wl.make_x(5, 24576, 1.0, 3, 8, 20, 11), 6.0
    yield "k_60000", *wl.make_x(3, 60000, 1.0, 4, 8, 20, 12), 6.0
    yield "k_max", *wl.make_x(2, 133136, 1.0, 5, 8, 20, 13), 6.0
    # 17-256 rows (strip scan, then one row-quantizer workgroup per row): one
    # case per wide launch shape of the row quantizer (16-byte chunks per
    # thread up to 4, 7, 8, 16 and 17), then the same quantizer after the
    # full-column flag pass (more than 256 rows, decomposition off)
    for M, K, seed in ((40, 24576, 31), (100, 57344, 32), (65, 61456, 33), (200, 99984, 34),
                       (33, 133136, 35)):
        X, c = wl.make_x(M, K, 1.0, 5, 8, 20, seed)
        X[M - 1, K - 1] = 6.0
        X[M // 2, K // 2] = np.float16(5.99609375)
        yield f"rowquant_{M}x{K}", X, sorted(set(c) | {K - 1}), 6.0
    yield "rowquant_disabled_300x99984", *wl.make_x(300, 99984, 1.0, 3, 8, 20, 36), math.inf
    X, c = wl.make_x(33, 256, 1.0, 0, 8, 20, 7)
    yield "all_outliers", X, c, 2.0 ** -24
    yield "disabled_inf", X, c, math.inf
    yield "disabled_zero", X, c, 0.0
    # small M (<= 16): 512-column slices; outliers on both sides of slice edges,
    # K ending in the middle of a flag word, a zero row, many outliers
    X, c = wl.make_x(16, 1552, 1.0, 0, 8, 20, 14)
    for k in (0, 511, 512, 1023, 1024, 1535, 1536, 1551):
        X[:, k] = np.float16(7.0)
    X[9, :] = 0
    X[2, 700] = 6.0
    X[4, 701] = np.float16(5.99609375)
    yield "small_slice_edges", X, [0, 511, 512, 700, 1023, 1024, 1535, 1536, 1551], 6.0
    yield "small_many_outliers", *wl.make_x(7, 2048, 1.0, 300, 8, 20, 15), 6.0
    X, c = wl.make_x(6, 256, 1.0, 0, 8, 20, 16)
    yield "small_all_outliers", X, c, 2.0 ** -24
    yield "small_disabled", *wl.make_x(10, 1040, 1.0, 3, 8, 20, 17), math.inf
    yield "rows64_wide_k", *wl.make_x(64, 24592, 1.0, 7, 8, 20, 18), 6.0   # strip scan, 2 rows/thread
    # 64-column strip scan, one launch shape per rows-per-thread count (up to 32,
    # 64, 128, 256 rows): threshold edges in the last row block, a K that ends
    # inside a strip (K % 64 == 16) and one on a strip edge
    for M, K, seed in ((32, 1040, 19), (65, 4096, 20), (128, 1104, 21), (255, 2064, 22),
                       (256, 4096, 23)):
        X, c = wl.make_x(M, K, 0.5, 3, 8, 20, seed)
        X[M - 1, K - 1] = 6.0
        X[M - 2, K - 17] = np.float16(5.99609375)
        X[M - 1, 63] = -6.0
        X[M // 2, 64] = np.float16(-5.99609375)
        yield f"strip_{M}x{K}", X, sorted(set(c) | {K - 1, 63}), 6.0
    # more than 256 rows, absmax codes: one pass over each row with a provisional
    # scale (its largest entry below the threshold), then a fix-up that zeroes and
    # gathers the outlier columns and recomputes a row whose provisional maximum
    # sits in an outlier column
    yield "rowpass_fallback", *_rowpass_x(300, 1040, 24), 6.0
    yield "rowpass_fallback_k_mod64", *_rowpass_x(513, 2064, 25), 6.0
    X, c = wl.make_x(260, 64, 1.0, 0, 8, 20, 26)
    X[:, 7] = 0
    yield "rowpass_all_outliers", X, c, 2.0 ** -24
    X, c = wl.make_x(24, 128, 0.25, 0, 8, 20, 8)
    X[3, 5] = 6.0
    X[7, 9] = np.float16(5.99609375)
    X[11, 100] = -6.0
    X[5, :] = 0
    yield "boundary", X, c, 6.0


def _partial_outliers(X, rng, ncols, nan=True):
    """Entries at or above the threshold in a few rows of `ncols` random
    columns, entries just below it in a few other rows of the same columns,
    and (with `nan`) a NaN in some of those columns."""
    M, K = X.shape
    partial = []
    for _ in range(ncols):
        col = int(rng.integers(0, K))
        rows = rng.choice(M, size=int(rng.integers(1, 4)), replace=False)
        X[rows, col] = np.float16(rng.choice([6.0, -6.0, 7.5, -40.0]))
        near = rng.choice(M, size=int(rng.integers(0, 6)), replace=False)
        X[near, col] = np.float16(rng.choice([5.99609375, -5.9, 5.5]))
        partial.append((col, set(rows.tolist())))
    if nan:
        for col, rows in partial[:int(rng.integers(0, 3))]:
            r = int(rng.integers(0, M))
            if r not in rows:
                X[r, col] = np.nan
    return X


def _rowpass_random(n=12, seed=77):
    """More than 256 rows with partial outlier columns: entries at or above
    the threshold in some rows only, so that other rows hold entries below it
    in those columns (zeroed by the fix-up, or, when one is a row's largest,
    recomputed), plus values exactly at the threshold and NaNs in outlier
    columns (a row with a NaN in a regular column has no defined scale).
    The last cases take the wide launch shapes of the row pass (K up to
    32768, 65536, 131072 and the largest K, the last two recomputing the
    per-chunk threshold masks instead of keeping them)."""
    rng = np.random.default_rng(seed)
    shapes = [(int(rng.integers(257, 700)), int(16 * rng.integers(2, 400))) for _ in range(n)]
    shapes += [(257, 24592), (300, 61456), (261, 99984), (258, 133136)]
    for i, (M, K) in enumerate(shapes):
        X, _ = wl.make_x(M, K, float(rng.choice([0.25, 1.0, 2.0])), 0, 8, 20, 100 + i)
        _partial_outliers(X, rng, int(rng.integers(0, 12)))
        yield f"rp{i}_{M}x{K}", X


@pytest.mark.parametrize("case", list(_rowpass_random()), ids=lambda c: c[0])
def test_rowpass_random_bitexact(lib, case):
    name, X = case
    say(f"quantize_activation (row pass) {name}")
    r = lib.quantize_activation(dev(X), 6.0)
    Xq_o, sx_o, idx_o, XO_o = O.quantize_activation(X, 6.0)
    n = int(host(r["n_out"])[0])
    assert n == len(idx_o), name
    np.testing.assert_array_equal(host(r["idx"])[:n], idx_o, err_msg=name)
    np.testing.assert_array_equal(host(r["sx"]).view(np.uint32), sx_o.view(np.uint32), err_msg=name)
    np.testing.assert_array_equal(host(r["Xq"]), Xq_o, err_msg=name)
    np.testing.assert_array_equal(host(r["X_O"])[:, :n].view(np.uint16), XO_o.view(np.uint16),
                                  err_msg=name)


@pytest.mark.parametrize("case", list(_act_cases()), ids=lambda c: c[0])
def test_quantize_activation_bitexact(lib, case):
    name, X, _, t = case
    say(f"quantize_activation {name} M={X.shape[0]} K={X.shape[1]} t={t}")
    r = lib.quantize_activation(dev(X), t)
    Xq_o, sx_o, idx_o, XO_o = O.quantize_activation(X, t)
    n = int(host(r["n_out"])[0])
    assert n == len(idx_o)
    np.testing.assert_array_equal(host(r["idx"])[:n], idx_o)
    np.testing.assert_array_equal(host(r["sx"]).view(np.uint32), sx_o.view(np.uint32))
    np.testing.assert_array_equal(host(r["Xq"]), Xq_o)
    np.testing.assert_array_equal(host(r["X_O"])[:, :n].view(np.uint16), XO_o.view(np.uint16))


def test_quantize_activation_reused_workspace(lib):
    """One workspace through calls whose outlier sets shrink: no column flag
    of an earlier call may survive (rows <= 256 store every flag word; more
    rows clear the flags first; the threshold off stores zeros)."""
    K = 1040
    ws = lib.new_workspace(300, K, 0, torch.device("cuda:0"))
    ws.fill_(0xff)
    calls = [("m40_many", wl.make_x(40, K, 1.0, 60, 8, 20, 21)[0], 6.0),
             ("m40_none", wl.make_x(40, K, 1.0, 0, 8, 20, 22)[0], 6.0),
             ("m300_many", wl.make_x(300, K, 1.0, 50, 8, 20, 23)[0], 6.0),
             ("m64_few", wl.make_x(64, K, 1.0, 2, 8, 20, 24)[0], 6.0),
             ("m200_many", wl.make_x(200, K, 1.0, 40, 8, 20, 27)[0], 6.0),
             ("m130_none", wl.make_x(130, K, 1.0, 0, 8, 20, 28)[0], 6.0),
             ("m300_off", wl.make_x(300, K, 1.0, 9, 8, 20, 25)[0], math.inf),
             ("m20_off", wl.make_x(20, K, 1.0, 9, 8, 20, 26)[0], math.inf)]
    for name, X, t in calls:
        say(f"quantize_activation reused workspace {name} M={X.shape[0]} K={K} t={t}")
        r = lib.quantize_activation(dev(X), t, workspace=ws)
        Xq_o, sx_o, idx_o, XO_o = O.quantize_activation(X, t)
        n = int(host(r["n_out"])[0])
        assert n == len(idx_o), name
        np.testing.assert_array_equal(host(r["idx"])[:n], idx_o, err_msg=name)
        np.testing.assert_array_equal(host(r["sx"]).view(np.uint32), sx_o.view(np.uint32),
                                      err_msg=name)
        np.testing.assert_array_equal(host(r["Xq"]), Xq_o, err_msg=name)


def test_quantize_activation_reused_outputs(lib):
    """The same output tensors written again by a second call (the `out`
    argument): the second call's results, bit-exact, nothing left of the first
    (its outlier set is larger), and an out tensor of the wrong shape raises."""
    K = 1040
    ws = lib.new_workspace(64, K, 0, torch.device("cuda:0"))
    X1 = wl.make_x(40, K, 1.0, 60, 8, 20, 31)[0]
    X2 = wl.make_x(40, K, 1.0, 3, 8, 20, 32)[0]
    say(f"quantize_activation reused outputs M=40 K={K}")
    out = lib.quantize_activation(dev(X1), 6.0, workspace=ws)
    r = lib.quantize_activation(dev(X2), 6.0, workspace=ws, out=out)
    assert all(r[k] is out[k] for k in out)
    Xq_o, sx_o, idx_o, XO_o = O.quantize_activation(X2, 6.0)
    n = int(host(r["n_out"])[0])
    assert n == len(idx_o)
    np.testing.assert_array_equal(host(r["idx"])[:n], idx_o)
    np.testing.assert_array_equal(host(r["sx"]).view(np.uint32), sx_o.view(np.uint32))
    np.testing.assert_array_equal(host(r["Xq"]), Xq_o)
    np.testing.assert_array_equal(host(r["X_O"])[:, :n], XO_o)
    bad = dict(out, sx=torch.empty(39, dtype=torch.float32, device="cuda:0"))
    with pytest.raises(ValueError):
        lib.quantize_activation(dev(X2), 6.0, workspace=ws, out=bad)


# ---------------------------------------------------------------------------------
# exact int8 GEMM (stage export)
# ---------------------------------------------------------------------------------
@pytest.mark.parametrize("M,K,N", [(16, 1024, 4096), (300, 272, 520), (513, 1040, 257),
                                   (256, 128, 256), (1, 16, 1), (257, 80, 300), (40, 144, 600),
                                   (300, 48, 270), (1024, 4096, 1024)])
def test_gemm_i32_bitexact(lib, M, K, N):
    say(f"gemm_i32 M={M} K={K} N={N}")
    rng = np.random.default_rng(M * 7 + K + N)
    Xq = rng.integers(-127, 128, (M, K), dtype=np.int8)
    Wq = rng.integers(-127, 128, (N, K), dtype=np.int8)
    acc = lib.gemm_i32(dev(Xq), dev(Wq))
    np.testing.assert_array_equal(host(acc), O.int8_matmul(Xq, Wq))


def test_gemm_i32_extremes(lib):
    say("gemm_i32 extremes")
    M, N, K = 64, 80, 8192
    Xq = np.full((M, K), 127, np.int8)
    Xq[1::2] = -127
    Wq = np.full((N, K), 127, np.int8)
    Wq[::3, ::2] = -127
    acc = lib.gemm_i32(dev(Xq), dev(Wq))
    np.testing.assert_array_equal(host(acc), O.int8_matmul(Xq, Wq))


# The largest K the library accepts, every code at +-127: the accumulators
# reach +-127^2 * K = +-2147350544, just inside int32 (the bound that fixes
# that K).  One row and one weight row of random codes catch misplaced
# k-steps.  M = 8 and 100: 128-row skinny tiles; 200: 256-row skinny tiles;
# 300: the 256 x 256 GEMM, whole tiles or (with a workspace) split along K.
@pytest.mark.parametrize("M,N,split", [(8, 40, False), (100, 72, False), (200, 64, False),
                                       (300, 64, False), (300, 64, True)])
def test_gemm_i32_max_k(lib, M, N, split):
    K = lib.MAX_K
    say(f"gemm_i32 max K M={M} K={K} N={N} split={split}")
    Xq = np.full((M, K), 127, np.int8)
    Xq[1::2] = -127
    Wq = np.full((N, K), 127, np.int8)
    Wq[1::3] = -127
    Wq[2::3, ::2] = -127
    rng = np.random.default_rng(M + N)
    Xq[-1] = rng.integers(-127, 128, K, dtype=np.int8)
    Wq[-1] = rng.integers(-127, 128, K, dtype=np.int8)
    ws = lib.new_workspace(M, K, N, torch.device("cuda:0")) if split else None
    acc = host(lib.gemm_i32(dev(Xq), dev(Wq), workspace=ws))
    np.testing.assert_array_equal(acc, O.int8_matmul(Xq, Wq))
    assert acc[0, 0] == 127 * 127 * K == 2147350544
    assert acc[1, 0] == -2147350544 and acc[0, 1] == -2147350544 and acc[1, 1] == 2147350544
    assert acc[0, 2] == 0


# ---------------------------------------------------------------------------------
# the whole layer through int8_linear (small M: fused decode kernel; larger M: GEMM)
# ---------------------------------------------------------------------------------
def _linear_cases():
    # name, M, K, N, n_out, threshold, x_sigma
    yield "decode_small", 8, 1024, 4096, 2, 6.0, 1.0
    yield "decode_m1", 1, 512, 1000, 1, 6.0, 1.0
    yield "decode_m16", 16, 4096, 512, 3, 6.0, 1.0
    yield "decode_m12_k2048", 12, 2048, 300, 2, 6.0, 1.0
    yield "decode_k8192", 8, 8192, 256, 5, 6.0, 1.0
    yield "decode_k_mod64", 5, 1040, 200, 2, 6.0, 1.0
    yield "decode_unfused_bigk", 8, 16384, 256, 4, 6.0, 1.0
    yield "decode_bigk_many_outliers", 3, 4112, 200, 90, 6.0, 1.0
    yield "decode_bigk_m16_ragged_n", 16, 6160, 777, 3, 6.0, 1.0
    yield "decode_bigk_m1", 1, 8192, 1000, 2, 6.0, 1.0
    # the largest K the library accepts: small-M activation kernels and the
    # streaming kernel; the 256 x 256 GEMM (two tiles, split along K)
    yield "decode_max_k", 8, 133136, 300, 5, 6.0, 1.0
    yield "prefill_max_k", 300, 133136, 64, 5, 6.0, 1.0
    # 17 <= M <= 64: activation kernels + the streaming kernel with 2 or 4 row groups
    yield "stream_m17", 17, 1024, 600, 2, 6.0, 1.0
    yield "stream_m24_k4112", 24, 4112, 300, 3, 6.0, 1.0
    yield "stream_m32", 32, 4096, 1000, 3, 6.0, 1.0
    yield "stream_m33", 33, 272, 130, 1, 6.0, 1.0
    yield "stream_m48_k8192", 48, 8192, 777, 5, 6.0, 1.0
    yield "stream_m64", 64, 2048, 520, 4, 6.0, 1.0
    yield "stream_m64_many_outliers", 64, 1024, 200, 90, 6.0, 1.0
    yield "decode_many_outliers", 4, 1024, 130, 70, 6.0, 1.0
    # the fused kernel with many outlier columns per wave (batched reads)
    yield "decode_m16_300_outliers", 16, 4096, 320, 300, 6.0, 1.0
    yield "decode_m1_100_outliers", 1, 512, 200, 100, 6.0, 1.0
    yield "decode_m8_41_outliers", 8, 4096, 520, 41, 6.0, 1.0
    # many outlier columns per wave with 4 and 8 k-steps packed per register set
    yield "decode_m4_70_outliers", 4, 4096, 520, 70, 6.0, 1.0
    yield "decode_m2_60_outliers", 2, 4096, 300, 60, 6.0, 1.0
    yield "decode_m3_k2048_40_outliers", 3, 2048, 260, 40, 6.0, 1.0
    yield "prefill_m17", 17, 1024, 600, 2, 6.0, 1.0
    # 64 < M <= 256: the 256 x 64 tiles (one or two outlier staging rounds,
    # ragged N with element stores)
    yield "skinny_m65", 65, 1040, 520, 5, 6.0, 1.0
    yield "skinny_m128", 128, 4096, 1000, 3, 6.0, 1.0
    yield "skinny_m200_ragged_n", 200, 272, 70, 2, 6.0, 1.0
    yield "skinny_m256_40_outliers", 256, 2048, 264, 40, 6.0, 1.0
    yield "prefill_ragged", 300, 272, 520, 5, 6.0, 1.0
    yield "prefill_tiles", 513, 1040, 769, 8, 6.0, 1.0
    yield "prefill_chunks", 64, 512, 300, 45, 6.0, 1.0
    yield "prefill_many_outliers", 70, 1024, 300, 130, 6.0, 1.0   # 256 x 64 tiles
    yield "prefill_many_outliers_big", 300, 1024, 300, 130, 6.0, 1.0   # > 96: unstaged path
    yield "prefill_split_k", 520, 2048, 1300, 6, 6.0, 1.0         # 18 tiles, K split in 2
    yield "prefill_no_outliers", 260, 512, 512, 0, 6.0, 1.0
    yield "prefill_disabled", 260, 512, 512, 3, math.inf, 1.0
    yield "prefill_all_outliers", 70, 256, 96, 0, 2.0 ** -24, 1.0
    yield "decode_all_outliers", 6, 256, 96, 0, 2.0 ** -24, 1.0


@pytest.mark.parametrize("case", list(_linear_cases()), ids=lambda c: c[0])
def test_linear_parity(lib, case):
    name, M, K, N, n_out, t, xs = case
    say(f"int8_linear {name} M={M} K={K} N={N} n_out={n_out} t={t}")
    X, W, _ = wl.make_small(M, K, N, seed=zlib.crc32(name.encode()) % 1000, n_out=n_out, x_sigma=xs)
    if name.startswith("prefill_ragged") or name.startswith("decode_m12"):
        X[2, :] = 0                                   # zero row
        W[:, 5] = 0                                   # zero output column
    pass_w = not math.isinf(t)
    Y, Wq, sw, ws = run_linear(lib, X, W, t, pass_w)
    Wq_o, sw_o = O.quantize_weight(W)
    np.testing.assert_array_equal(host(Wq), Wq_o)
    r = O.int8_linear(X, Wq_o, sw_o, W, t)
    check_workspace(lib, ws, M, K, (r["Xq"], r["sx"], r["idx"], r["X_O"]), name)
    assert_y(host(Y), r["Y64"], r["Y"], name)


@pytest.mark.parametrize("M,K,N,seed", [(300, 1040, 520, 24), (513, 2064, 300, 25)])
def test_linear_rowpass_fallback(lib, M, K, N, seed):
    """The whole layer on rows whose provisional scale must be recomputed
    (their largest entry below the threshold, or a NaN, in an outlier column)."""
    say(f"int8_linear rowpass fallback M={M} K={K} N={N}")
    X, _ = _rowpass_x(M, K, seed)
    W = wl.make_w(K, N, 0.02, seed)
    Y, Wq, sw, ws = run_linear(lib, X, W, 6.0)
    Wq_o, sw_o = O.quantize_weight(W)
    r = O.int8_linear(X, Wq_o, sw_o, W, 6.0)
    check_workspace(lib, ws, M, K, (r["Xq"], r["sx"], r["idx"], r["X_O"]), "rowpass")
    # row 7 holds a NaN in an outlier column: its outputs are NaN on both sides
    nan = np.isnan(r["Y64"])
    assert np.array_equal(np.isnan(host(Y).astype(np.float64)), nan)
    assert_y(np.where(nan, 0, host(Y)), np.where(nan, 0, r["Y64"]), None, "rowpass")


def test_linear_overflow_to_inf(lib):
    say("int8_linear overflow")
    M, K, N = 20, 64, 32
    X = np.full((M, K), 5.0, np.float16)
    X[::2] = -5.0
    W = np.full((K, N), 300.0, np.float16)
    W[:, ::3] = 1.0
    Y, *_ = run_linear(lib, X, W, 6.0)
    Wq_o, sw_o = O.quantize_weight(W)
    r = O.int8_linear(X, Wq_o, sw_o, W, 6.0)
    assert np.isinf(r["Y"]).any()
    assert_y(host(Y), r["Y64"], r["Y"], "overflow")


def test_linear_empty(lib):
    say("int8_linear empty")
    W = np.zeros((64, 8), np.float16)
    Wd = dev(W)
    Wq, sw = lib.quantize_weight(Wd)
    Y = lib.linear(dev(np.zeros((0, 64), np.float16)), Wq, sw, Wd, 6.0)
    assert tuple(Y.shape) == (0, 8)
    Wq0 = torch.empty((0, 64), dtype=torch.int8, device="cuda:0")
    sw0 = torch.empty((0,), dtype=torch.float32, device="cuda:0")
    Y0 = lib.linear(dev(np.ones((4, 64), np.float16)), Wq0, sw0, None, math.inf)
    assert tuple(Y0.shape) == (4, 0)


def test_linear_deterministic(lib):
    say("int8_linear determinism")
    for (M, K, N) in [(8, 4096, 2048), (300, 1024, 700)]:
        X, W, _ = wl.make_small(M, K, N, seed=9, n_out=3)
        Y1, *_ = run_linear(lib, X, W, 6.0)
        Y2, *_ = run_linear(lib, X, W, 6.0)
        np.testing.assert_array_equal(host(Y1).view(np.uint16), host(Y2).view(np.uint16))


def test_linear_concurrent_host_threads(lib):
    """The library keeps no per-call state: host threads, each with its own
    stream and workspace, get the results a single thread gets (fused kernel,
    streaming kernel for 8 and 40 rows, GEMM with a split tail)."""
    import threading
    say("int8_linear from 4 host threads")
    shapes = [(8, 4096, 2048), (8, 8192, 512), (40, 1024, 700), (520, 2048, 1300)]
    jobs = []
    for i, (M, K, N) in enumerate(shapes):
        X, W, _ = wl.make_small(M, K, N, seed=40 + i, n_out=3)
        Xd, Wd = dev(X), dev(W)
        Wq, sw = lib.quantize_weight(Wd)
        ref = lib.linear(Xd, Wq, sw, Wd, 6.0)
        ws = lib.new_workspace(M, K, N, Xd.device)
        out = torch.empty((M, N), dtype=torch.float16, device=Xd.device)
        jobs.append((Xd, Wq, sw, Wd, ws, out, ref))
    torch.cuda.synchronize()
    errors = []

    def work(job):
        Xd, Wq, sw, Wd, ws, out, ref = job
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(5):
                    lib.linear(Xd, Wq, sw, Wd, 6.0, workspace=ws, out=out)
            s.synchronize()
        except Exception as e:   # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(j,)) for j in jobs]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for (M, K, N), (*_, out, ref) in zip(shapes, jobs):
        np.testing.assert_array_equal(host(out).view(np.uint16), host(ref).view(np.uint16),
                                      err_msg=f"{M}x{K}x{N}")


# ---------------------------------------------------------------------------------
# the benchmark workloads at full size, in the launch configuration bench.py times
# ---------------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny", "decode", "decode_1pct", "decode_m128"])
def test_workload_full_oracle(lib, name):
    w = wl.WORKLOADS[name]
    say(f"workload {name} (full oracle)")
    X, W, cols = wl.make_inputs(w)
    Y, Wq, sw, ws = run_linear(lib, X, W, w.threshold)
    Wq_o, sw_o = O.quantize_weight(W)
    np.testing.assert_array_equal(host(Wq), Wq_o)
    np.testing.assert_array_equal(host(sw).view(np.uint32), sw_o.view(np.uint32))
    r = O.int8_linear(X, Wq_o, sw_o, W, w.threshold)
    np.testing.assert_array_equal(r["idx"], np.sort(cols))
    check_workspace(lib, ws, w.M, w.K, (r["Xq"], r["sx"], r["idx"], r["X_O"]), name)
    assert_y(host(Y), r["Y64"], r["Y"], name)


@pytest.mark.parametrize("name", ["qkv_prefill", "mlp_down_prefill", "square_0pct",
                                  "square_0.1pct", "square_1pct", "decode_qkv",
                                  "decode_mlp_down", "decode_m32", "decode_m256"])
def test_workload_full_sampled(lib, name):
    w = wl.WORKLOADS[name]
    say(f"workload {name} (sampled): generating inputs")
    X, W, cols = wl.make_inputs(w)
    say(f"workload {name}: running GPU")
    Xd, Wd = dev(X), dev(W)
    Wq, sw = lib.quantize_weight(Wd)
    ws = lib.new_workspace(w.M, w.K, w.N, Xd.device)
    # NaN-filled output: an entry the layer never writes stays NaN
    Y = torch.full((w.M, w.N), float("nan"), dtype=torch.float16, device=Xd.device)
    lib.linear(Xd, Wq, sw, Wd, w.threshold, workspace=ws, out=Y)
    torch.cuda.synchronize()
    assert not torch.isnan(Y).any().item(), f"{name}: output entries left unwritten"
    assert torch.isfinite(Y).all().item()
    say(f"workload {name}: activation stage, full")
    act = O.quantize_activation(X, w.threshold)
    np.testing.assert_array_equal(act[2], np.sort(cols))
    check_workspace(lib, ws, w.M, w.K, act, name)

    # sampled outputs: one random entry in every 256 x 256 output tile (the
    # GEMM's tile; whole tiles, split-K tail tiles and ragged edge tiles),
    # plus random entries and the tile edges and last row / column
    rng = np.random.default_rng(1234)
    T0, T1 = np.meshgrid(np.arange(0, w.M, 256), np.arange(0, w.N, 256), indexing="ij")
    t_rows = np.minimum(T0.ravel() + rng.integers(0, 256, T0.size), w.M - 1)
    t_cols = np.minimum(T1.ravel() + rng.integers(0, 256, T1.size), w.N - 1)
    S = 3000
    edges = [r for r in (0, 255, 256, w.M - 1) if r < w.M]
    r_cols = np.concatenate([rng.integers(0, w.N, 48), [0, 255, 256, w.N - 1]])
    r_cols = r_cols[r_cols < w.N]
    ns = np.unique(np.concatenate([r_cols, t_cols]))
    say(f"workload {name}: {len(ns)} weight rows, {T0.size} output tiles")
    Wq_r, sw_r = O.quantize_weight_rows(W, ns)
    nsd = torch.as_tensor(ns, device="cuda:0")
    np.testing.assert_array_equal(host(Wq[nsd]), Wq_r)
    np.testing.assert_array_equal(host(sw[nsd]).view(np.uint32), sw_r.view(np.uint32))
    rr = np.concatenate([rng.integers(0, w.M, S), edges])
    rows = np.concatenate([rr, t_rows])
    colsel = np.concatenate([r_cols[rng.integers(0, len(r_cols), len(rr))], t_cols])
    pick = np.searchsorted(ns, colsel)
    acc_o = np.empty(len(rows), np.int32)
    Y64 = np.empty(len(rows))
    for a in range(0, len(rows), 512):        # bounded host memory at K = 57344
        b = slice(a, a + 512)
        acc_o[b], Y64[b] = O.int8_linear_entries(X, Wq_r[pick[b]], sw_r[pick[b]], W,
                                                 w.threshold, rows[b], colsel[b], act=act)
    ri = torch.as_tensor(rows, device="cuda:0")
    ci = torch.as_tensor(colsel, device="cuda:0")
    assert_y(host(Y[ri, ci]), Y64, what=name)
    # exact int32 accumulators at the same entries via the GEMM stage, split
    # along K as in the layer
    v = lib.workspace_views(ws, w.M, w.K)
    ws2 = lib.new_workspace(w.M, w.K, w.N, Xd.device)
    acc = lib.gemm_i32(v["Xq"].contiguous(), Wq, workspace=ws2)
    np.testing.assert_array_equal(host(acc[ri, ci]), acc_o)
    del acc, Y, Wq, ws, ws2, Xd, Wd
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------------
# graph capture: replays of a captured int8_linear equal the eager call
# ---------------------------------------------------------------------------------
# (520, 2048, 1300): 18 tiles, split in 2 along K (partials, then the fix-up
# launch, inside the graph); (8, 8192, 300): small-M activation kernels
# and the stream kernel; (40, 4096, 1000): the stream kernel with 4 row groups
@pytest.mark.parametrize("M,K,N", [(8, 1024, 4096), (300, 272, 520), (520, 2048, 1300),
                                   (8, 8192, 300), (40, 4096, 1000)])
def test_linear_graph_replay(lib, M, K, N):
    say(f"int8_linear graph replay M={M} K={K} N={N}")
    X, W, _ = wl.make_small(M, K, N, seed=M + K, n_out=3, x_sigma=1.0)
    X2, _, _ = wl.make_small(M, K, N, seed=M + K + 1, n_out=2, x_sigma=1.0)
    Xd, Wd, X2d = dev(X), dev(W), dev(X2)
    Wq, sw = lib.quantize_weight(Wd)
    ws = lib.new_workspace(M, K, N, Xd.device)
    Y_eager = lib.linear(Xd, Wq, sw, Wd, 6.0, workspace=ws).clone()
    Yg = torch.empty_like(Y_eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        lib.linear(Xd, Wq, sw, Wd, 6.0, workspace=ws, out=Yg)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lib.linear(Xd, Wq, sw, Wd, 6.0, workspace=ws, out=Yg)
    for rep in range(3):
        Yg.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(Yg).view(np.uint16), host(Y_eager).view(np.uint16),
                                      err_msg=f"replay {rep}")
        # eager work on other inputs (same workspace) between the replays
        lib.linear(X2d, Wq, sw, Wd, 6.0, workspace=ws)
        torch.cuda.synchronize()


# ---------------------------------------------------------------------------------
# GEMM split-K tail: 384 tiles = 256 whole + 128 split along K (sampled outputs)
# ---------------------------------------------------------------------------------
def test_linear_split_tail_sampled(lib):
    M, K, N = 2048, 2048, 12200
    say(f"int8_linear split tail M={M} K={K} N={N}")
    assert lib.workspace_layout(M, K, N)["gemm_slices"] == 128 * 2
    X, W, _ = wl.make_small(M, K, N, seed=77, n_out=5, x_sigma=1.0)
    Xd, Wd = dev(X), dev(W)
    Wq, sw = lib.quantize_weight(Wd)
    ws = lib.new_workspace(M, K, N, Xd.device)
    Y = lib.linear(Xd, Wq, sw, Wd, 6.0, workspace=ws)
    torch.cuda.synchronize()
    act = O.quantize_activation(X, 6.0)
    check_workspace(lib, ws, M, K, act, "split tail")
    rng = np.random.default_rng(99)
    # columns of the split tiles (tile columns 32..47) and elsewhere
    ns = np.unique(np.concatenate([rng.integers(8192, N, 24), rng.integers(0, 8192, 16),
                                   [0, 8191, 8192, N - 1]]))
    Wq_r, sw_r = O.quantize_weight_rows(W, ns)
    S = 2500
    rows = np.concatenate([rng.integers(0, M, S), [0, 255, 256, M - 1]])
    pick = rng.integers(0, len(ns), len(rows))
    cols = ns[pick]
    acc_o, Y64 = O.int8_linear_entries(X, Wq_r[pick], sw_r[pick], W, 6.0, rows, cols, act=act)
    ri = torch.as_tensor(rows, device="cuda:0")
    ci = torch.as_tensor(cols, device="cuda:0")
    assert_y(host(Y[ri, ci]), Y64, what="split tail")
    # a second call on the same workspace (counters are re-armed per call)
    Y2 = lib.linear(Xd, Wq, sw, Wd, 6.0, workspace=ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(Y2).view(np.uint16), host(Y).view(np.uint16))


# ---------------------------------------------------------------------------------
# no fp16 weight kept: outlier rows rebuilt from the codes (W_outlier_rows NULL)
# ---------------------------------------------------------------------------------
@pytest.mark.parametrize("name,M,K,N,n_out", [
    ("decode", 8, 4096, 1000, 3),            # fused decode kernel
    ("decode_m1", 1, 1040, 300, 2),
    ("decode_many", 4, 1024, 130, 9),        # more outliers than a wave preloads
    ("decode_many_lds", 8, 1024, 520, 60),   # columns 5-8 of a wave fetched into LDS, and beyond
    ("decode_m2_many", 2, 4096, 300, 60),    # 8 k-steps per register set
    ("decode_bigk", 8, 16384, 256, 4),       # activation kernels + streaming kernel
    ("stream_m32", 32, 4096, 520, 3),        # streaming kernel, 2 row groups
    ("stream_m64_many", 64, 1024, 200, 70),  # 4 row groups, outliers past the LDS copy
    ("prefill", 300, 1040, 520, 5),          # GEMM, staged outlier rows
    ("prefill_many", 300, 1024, 300, 130),   # GEMM, rows straight from memory
    ("skinny_many", 70, 1024, 300, 130),     # 256 x 64 tiles, five staging rounds
    ("prefill_split", 520, 2048, 1300, 6),   # GEMM split-K tail
])
def test_linear_rebuilt_outlier_rows(lib, name, M, K, N, n_out):
    say(f"int8_linear without fp16 weight: {name} M={M} K={K} N={N} n_out={n_out}")
    X, W, _ = wl.make_small(M, K, N, seed=zlib.crc32(name.encode()) % 1000 + 7, n_out=n_out,
                            x_sigma=1.0)
    Xd, Wd = dev(X), dev(W)
    Wq, sw = lib.quantize_weight(Wd)
    del Wd
    ws = lib.new_workspace(M, K, N, Xd.device)
    Y = lib.linear(Xd, Wq, sw, None, 6.0, workspace=ws)
    torch.cuda.synchronize()
    Wq_o, sw_o = O.quantize_weight(W)
    np.testing.assert_array_equal(host(Wq), Wq_o)
    W_deq = O.dequantize_weight(Wq_o, sw_o)
    r = O.int8_linear(X, Wq_o, sw_o, W_deq, 6.0)
    assert len(r["idx"]) == n_out
    check_workspace(lib, ws, M, K, (r["Xq"], r["sx"], r["idx"], r["X_O"]), name)
    assert_y(host(Y), r["Y64"], r["Y"], name)
    # and it differs from the result with the original fp16 rows only by the
    # rebuilt weight values (a sanity check that the rebuilt path is used)
    r16 = O.int8_linear(X, Wq_o, sw_o, W, 6.0)
    assert not np.array_equal(r16["Y64"], r["Y64"])


# ---------------------------------------------------------------------------------
# a sweep of seeded random shapes through both activation codes
# ---------------------------------------------------------------------------------
def _random_cases(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    for i in range(n):
        M = int(rng.choice([1, 2, 3, 5, 8, 11, 16, 17, 33, 100, 257, 300]))
        K = int(16 * rng.integers(1, 160))            # 16 .. 2544, ragged against 64 and 128
        N = int(rng.integers(1, 700))
        n_out = int(min(K, rng.choice([0, 1, 2, 5, 20])))
        yield (f"r{i}_{M}x{K}x{N}_o{n_out}", M, K, N, n_out, bool(rng.integers(0, 2)),
               bool(rng.integers(0, 2)), bool(rng.integers(0, 2)), int(rng.integers(0, 1000)))


@pytest.mark.parametrize("case", list(_random_cases()), ids=lambda c: c[0])
def test_linear_random_shapes(lib, case):
    name, M, K, N, n_out, with_bias, pass_w, zp, seed = case
    say(f"random {name} bias={with_bias} W={'fp16' if pass_w else 'rebuilt'} zp={zp}")
    X, W, _ = wl.make_small(M, K, N, seed=seed, n_out=n_out)
    b = (np.random.default_rng(seed).standard_normal(N) * 0.5).astype(np.float16) \
        if with_bias else None
    Xd, Wd = dev(X), dev(W)
    Wq, sw = lib.quantize_weight(Wd)
    bd = dev(b) if b is not None else None
    Wq_o, sw_o = O.quantize_weight(W)
    np.testing.assert_array_equal(host(Wq), Wq_o)
    W_rows = W if pass_w else O.dequantize_weight(Wq_o, sw_o)
    if zp:
        S = lib.weight_code_sums(Wq)
        Y = lib.linear_zp(Xd, Wq, sw, S, Wd if pass_w else None, 6.0, bias=bd)
        r = O.int8_linear_zp(X, Wq_o, sw_o, W_rows, 6.0, bias=b)
    else:
        Y = lib.linear(Xd, Wq, sw, Wd if pass_w else None, 6.0, bias=bd)
        r = O.int8_linear(X, Wq_o, sw_o, W_rows, 6.0, bias=b)
    assert_y(host(Y), r["Y64"], what=name)
