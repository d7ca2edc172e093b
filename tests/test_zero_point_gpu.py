"""Zero-point (unsigned) activation codes on MI355X against the CPU oracle.

[blog, "Introduction to model quantization"]: the unsigned int8 scheme maps a
row's range onto [0, 255] with an integer zero point.  Codes, zero points,
scales, outlier lists and the weight code sums must match bit-exactly; fp16
outputs to |Y - Y64| <= max(2e-3 |Y64|, 1e-2) against the oracle's fp64 value,
the same bar as the absmax layer.
"""
import math
import zlib

import numpy as np
import pytest

from mixed_precision_quantized_int8_amd import workloads as wl
from oracle import int8_oracle as O
from test_parity_gpu import _partial_outliers

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


def assert_y(Yg, Y64, what=""):
    y = np.asarray(Yg).astype(np.float64)
    with np.errstate(over="ignore"):
        Y16 = Y64.astype(np.float16)
    inf = np.isinf(Y16)
    np.testing.assert_array_equal(np.asarray(Yg)[inf], Y16[inf], err_msg=f"{what}: infinities")
    err = np.abs(y[~inf] - Y64[~inf])
    tol = np.maximum(RTOL * np.abs(Y64[~inf]), ATOL)
    bad = ~(err <= tol)
    if bad.any():
        k = np.argmax(err - tol)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst "
                             f"gpu={y[~inf][k]!r} ref={Y64[~inf][k]!r}")


def check_act(got, act, what):
    """got: dict of device tensors Xq, zp, sx (xscale), idx, n_out, X_O."""
    Xq_o, zp_o, xs_o, idx_o, XO_o = act
    n = int(host(got["n_out"])[0])
    assert n == len(idx_o), f"{what}: n_out {n} != {len(idx_o)}"
    np.testing.assert_array_equal(host(got["idx"])[:n], idx_o, err_msg=f"{what}: idx")
    np.testing.assert_array_equal(host(got["zp"]), zp_o, err_msg=f"{what}: zp")
    np.testing.assert_array_equal(host(got["sx"]).view(np.uint32), xs_o.view(np.uint32),
                                  err_msg=f"{what}: xscale")
    np.testing.assert_array_equal(host(got["Xq"]), Xq_o, err_msg=f"{what}: Xq")
    if n:
        np.testing.assert_array_equal(host(got["X_O"])[:, :n].view(np.uint16),
                                      XO_o.view(np.uint16), err_msg=f"{what}: X_O")


def shaped_x(kind, M, K, n_out, seed):
    """Activations of the workload recipe, shifted or folded so that rows are
    off-centre (zero point inside the range), one-signed (zero point 0 or 255)
    or zero."""
    X, cols = wl.make_x(M, K, 1.0, n_out, 8.0, 20.0, seed)
    reg = np.ones(K, bool)
    reg[cols] = False
    Xr = X[:, reg].astype(np.float32)
    if kind == "offset":
        Xr = Xr + np.linspace(-2.0, 2.0, M, dtype=np.float32)[:, None]
    elif kind == "positive":
        Xr = np.abs(Xr)
    elif kind == "negative":
        Xr = -np.abs(Xr) * 0.5
    X[:, reg] = np.clip(Xr, -5.5, 5.5).astype(np.float16)   # below the threshold
    if kind in ("offset", "positive") and M > 2:
        X[1, :] = 0                                          # a zero row
    return X, cols


def _rowpass_zp_x(M, K, seed):
    """Rows whose largest or smallest entry below the threshold lies in a column
    that another row makes an outlier (and one tie), on off-centre rows."""
    X, c = shaped_x("offset", M, K, 3, seed)
    p, p2, q = 11, 40, 41            # partial outlier columns p, p2; regular column q
    X[:, [p, p2, q]] = np.clip(X[:, [p, p2, q]], -1, 1)
    X[0, p] = 7.0                    # p is an outlier column because of row 0 ...
    X[5, p] = np.float16(5.9)        # ... and holds row 5's largest entry below 6
    X[1, p2] = -9.0
    X[6, p2] = np.float16(-5.75)     # row 6's smallest entry, in outlier column p2
    X[8, p] = np.float16(-5.25)      # a tie for row 8's smallest: outlier p, regular q
    X[8, q] = np.float16(-5.25)
    X[7, p] = np.nan                 # a NaN in an outlier column
    X[9, q] = np.float16(5.99609375)  # largest in a regular column
    X[M - 1, K - 1] = -6.0           # a last outlier column, set by the last row only
    X[M - 2, K - 1] = np.float16(-5.8)
    return X, sorted(set(c) | {p, p2, K - 1})


# ---------------------------------------------------------------------------------
# weight code sums
# ---------------------------------------------------------------------------------
@pytest.mark.parametrize("N,K", [(4096, 1024), (7, 64), (1, 16), (1000, 14336), (3, 66304)])
def test_weight_code_sums_bitexact(lib, N, K):
    say(f"weight_code_sums N={N} K={K}")
    rng = np.random.default_rng(N + K)
    Wq = rng.integers(-127, 128, (N, K), dtype=np.int8)
    Wq[0, :] = 127
    S = lib.weight_code_sums(dev(Wq))
    np.testing.assert_array_equal(host(S), O.weight_code_sums(Wq))


# ---------------------------------------------------------------------------------
# activation stage
# ---------------------------------------------------------------------------------
def _act_cases():
    yield "tiny", *shaped_x("normal", 16, 1024, 2, 1), 6.0
    yield "decode_offset", *shaped_x("offset", 8, 4096, 4, 2), 6.0
    yield "ragged_positive", *shaped_x("positive", 300, 272, 5, 3), 6.0
    yield "negative", *shaped_x("negative", 40, 512, 3, 4), 6.0
    yield "one_row", *shaped_x("offset", 1, 16, 0, 5), 6.0
    yield "k_mod32_16", *shaped_x("offset", 17, 1040, 3, 6), 6.0
    yield "wide_k", *shaped_x("offset", 3, 40000, 6, 7), 6.0
    yield "max_k", *shaped_x("positive", 2, O.ZP_MAX_K, 2, 8), 6.0
    # small M (<= 16): 512-column slices
    X, c = shaped_x("offset", 16, 1552, 0, 10)
    for k in (0, 511, 512, 1023, 1024, 1535, 1536, 1551):
        X[:, k] = np.float16(-7.0)
    X[9, :] = 0
    yield "small_slice_edges", X, [0, 511, 512, 1023, 1024, 1535, 1536, 1551], 6.0
    yield "small_many_outliers", *shaped_x("negative", 7, 2048, 300, 11), 6.0
    X, c = shaped_x("positive", 6, 256, 0, 12)
    yield "small_all_outliers", X, c, 2.0 ** -24
    yield "small_disabled", *shaped_x("offset", 10, 1040, 3, 13), math.inf
    yield "rows64_wide_k", *shaped_x("offset", 64, 24592, 7, 14), 6.0
    # 17-256 rows: the wide launch shapes of the row quantizer up to the
    # largest K of zero-point codes, and the same quantizer after the
    # full-column flag pass (more than 256 rows, decomposition off)
    for M, K, seed in ((100, 57344, 31), (65, 61456, 32), (200, O.ZP_MAX_K, 33)):
        yield f"rowquant_{M}x{K}", *shaped_x("offset", M, K, 5, seed), 6.0
    yield "rowquant_disabled_300x66304", *shaped_x("offset", 300, O.ZP_MAX_K, 3, 34), math.inf
    # more than 256 rows: one pass per row with a provisional range (its
    # smallest and largest entry below the threshold), then the fix-up, which
    # recomputes a row whose range end sits in an outlier column
    yield "rowpass_offset", *shaped_x("offset", 300, 1040, 3, 15), 6.0
    yield "rowpass_fallback", *_rowpass_zp_x(300, 1040, 16), 6.0
    yield "rowpass_fallback_k_mod64", *_rowpass_zp_x(513, 2064, 17), 6.0
    X, c = shaped_x("negative", 260, 64, 0, 18)
    X[:, 7] = 0
    yield "rowpass_all_outliers", X, c, 2.0 ** -24
    X, c = shaped_x("offset", 33, 256, 0, 9)
    yield "all_outliers", X, c, 2.0 ** -24
    yield "disabled_inf", X, c, math.inf
    yield "disabled_zero", X, c, 0.0


def _rowpass_random(n=8, seed=78):
    """More than 256 rows, zero-point codes, with partial outlier columns (see
    the absmax sweep in test_parity_gpu.py) on off-centre rows; the last cases
    take the wide launch shapes of the row pass up to the largest K of
    zero-point codes (where the per-chunk masks are recomputed)."""
    rng = np.random.default_rng(seed)
    shapes = [(int(rng.integers(257, 600)), int(16 * rng.integers(2, 300))) for _ in range(n)]
    shapes += [(259, 24592), (300, 61456), (257, O.ZP_MAX_K)]
    for i, (M, K) in enumerate(shapes):
        X, _ = shaped_x(str(rng.choice(["offset", "positive", "negative", "normal"])), M, K, 0,
                        200 + i)
        _partial_outliers(X, rng, int(rng.integers(0, 10)), nan=False)
        yield f"rpzp{i}_{M}x{K}", X


@pytest.mark.parametrize("case", list(_rowpass_random()), ids=lambda c: c[0])
def test_rowpass_random_zp_bitexact(lib, case):
    name, X = case
    say(f"quantize_activation_zp (row pass) {name}")
    r = lib.quantize_activation_zp(dev(X), 6.0)
    r["sx"] = r["xscale"]
    check_act(r, O.quantize_activation_zp(X, 6.0), name)


@pytest.mark.parametrize("case", list(_act_cases()), ids=lambda c: c[0])
def test_quantize_activation_zp_bitexact(lib, case):
    name, X, _, t = case
    say(f"quantize_activation_zp {name} M={X.shape[0]} K={X.shape[1]} t={t}")
    r = lib.quantize_activation_zp(dev(X), t)
    r["sx"] = r["xscale"]
    act = O.quantize_activation_zp(X, t)
    check_act(r, act, name)
    if name == "ragged_positive":
        assert (act[1][2:] == 0).all()                    # one-signed rows: zero point 0
    if name == "negative":
        assert (act[1] == 255).all()


# ---------------------------------------------------------------------------------
# the layer
# ---------------------------------------------------------------------------------
def _linear_cases():
    # name, M, K, N, n_out, threshold, kind, bias, pass_w
    yield "decode_small", 8, 1024, 4096, 2, 6.0, "offset", False, True
    yield "decode_m1_bias", 1, 512, 1000, 1, 6.0, "positive", True, True
    yield "decode_m16", 16, 4096, 512, 3, 6.0, "offset", True, False
    yield "decode_k8192", 8, 8192, 256, 5, 6.0, "negative", False, True
    yield "decode_bigk_many_outliers", 3, 4112, 200, 90, 6.0, "offset", True, True
    # the fused kernel with up to and beyond eight outlier columns per wave
    yield "decode_many_outliers", 8, 2048, 520, 50, 6.0, "offset", True, True
    yield "decode_many_outliers_rebuilt", 4, 1024, 200, 60, 6.0, "negative", False, False
    yield "decode_m4_many_outliers", 4, 4096, 520, 70, 6.0, "offset", True, True
    yield "decode_m2_many_outliers", 2, 4096, 300, 60, 6.0, "positive", False, True
    yield "stream_m17_bias", 17, 1024, 600, 2, 6.0, "offset", True, True
    yield "stream_m40_k4112", 40, 4112, 300, 3, 6.0, "negative", False, False
    yield "stream_m64", 64, 2048, 520, 4, 6.0, "positive", True, True
    yield "decode_k_mod64", 5, 1040, 200, 2, 6.0, "offset", False, False
    yield "decode_m3_k272", 3, 272, 130, 1, 6.0, "negative", True, True
    yield "decode_m12_k2048", 12, 2048, 300, 2, 6.0, "positive", False, True
    yield "decode_m4_k4096", 4, 4096, 520, 3, 6.0, "offset", True, False
    yield "decode_m1_k16", 1, 16, 64, 0, 6.0, "offset", False, True
    yield "decode_m2_k3088", 2, 3088, 70, 1, 6.0, "offset", True, True
    yield "prefill_m17", 17, 1024, 600, 2, 6.0, "positive", True, True
    yield "skinny_m100", 100, 1024, 520, 3, 6.0, "offset", True, True
    yield "skinny_m256_rebuilt", 256, 2048, 264, 40, 6.0, "negative", False, False
    yield "prefill_ragged", 300, 272, 520, 5, 6.0, "offset", True, True
    yield "prefill_tiles", 513, 1040, 769, 8, 6.0, "offset", False, False
    yield "prefill_split_k", 520, 2048, 1300, 6, 6.0, "positive", True, True
    yield "prefill_many_outliers", 70, 1024, 300, 130, 6.0, "offset", False, True
    yield "prefill_normal", 260, 512, 512, 3, 6.0, "normal", False, True
    yield "prefill_disabled", 260, 512, 512, 3, math.inf, "offset", False, False
    yield "prefill_all_outliers", 70, 256, 96, 0, 2.0 ** -24, "offset", False, True
    yield "decode_all_outliers", 6, 256, 96, 0, 2.0 ** -24, "offset", True, True


@pytest.mark.parametrize("case", list(_linear_cases()), ids=lambda c: c[0])
def test_linear_zp_parity(lib, case):
    name, M, K, N, n_out, t, kind, with_bias, pass_w = case
    say(f"int8_linear_zp {name} M={M} K={K} N={N} n_out={n_out} t={t} bias={with_bias} "
        f"W={'fp16' if pass_w else 'rebuilt'}")
    seed = zlib.crc32(name.encode()) % 1000
    X, _ = shaped_x(kind, M, K, n_out, seed)
    W = wl.make_w(K, N, 0.02, seed)
    b = (np.random.default_rng(seed).standard_normal(N) * 0.5).astype(np.float16) \
        if with_bias else None
    Xd, Wd = dev(X), dev(W)
    Wq, sw = lib.quantize_weight(Wd)
    S = lib.weight_code_sums(Wq)
    ws = lib.new_workspace(M, K, N, Xd.device)
    Y = lib.linear_zp(Xd, Wq, sw, S, Wd if pass_w else None, t, workspace=ws,
                      bias=dev(b) if b is not None else None)
    Wq_o, sw_o = O.quantize_weight(W)
    np.testing.assert_array_equal(host(Wq), Wq_o)
    W_rows = W if pass_w else O.dequantize_weight(Wq_o, sw_o)
    r = O.int8_linear_zp(X, Wq_o, sw_o, W_rows, t, bias=b)
    check_act(lib.workspace_views(ws, M, K), (r["Xq"], r["zp"], r["xscale"], r["idx"], r["X_O"]),
              name)
    assert_y(host(Y), r["Y64"], name)


def test_linear_zp_int32_limit(lib):
    """K at the zero-point limit with every product at its largest: the exact
    sum 255 * 127 * K is just below 2^31."""
    say("int8_linear_zp int32 limit")
    M, K, N = 20, O.ZP_MAX_K, 16
    X = np.ones((M, K), np.float16)                   # lo = 0: zp = 0, every code 255
    X[1::2] = -1.0                                    # hi = 0: zp = 255, every code 0
    W = np.full((K, N), 0.001, np.float16)            # every weight code 127
    W[:, 1::2] = -0.001
    Xd, Wd = dev(X), dev(W)
    Wq, sw = lib.quantize_weight(Wd)
    S = lib.weight_code_sums(Wq)
    for M_ in (M, 4):                                 # GEMM and small-M paths
        Y = lib.linear_zp(Xd[:M_].contiguous(), Wq, sw, S, Wd, 6.0)
        Wq_o, sw_o = O.quantize_weight(W)
        r = O.int8_linear_zp(X[:M_], Wq_o, sw_o, W, 6.0)
        assert np.abs(r["acc"]).max() == 255 * 127 * K
        assert_y(host(Y), r["Y64"], f"int32 limit M={M_}")


def test_linear_zp_rejects_large_k(lib):
    M, K, N = 4, O.ZP_MAX_K + 16, 8
    X = torch.zeros((M, K), dtype=torch.float16, device="cuda:0")
    Wq = torch.zeros((N, K), dtype=torch.int8, device="cuda:0")
    sw = torch.ones((N,), dtype=torch.float32, device="cuda:0")
    S = torch.zeros((N,), dtype=torch.int32, device="cuda:0")
    with pytest.raises(lib.Int8LinError, match="K_TOO_LARGE"):
        lib.linear_zp(X, Wq, sw, S, None, 6.0)
    with pytest.raises(lib.Int8LinError, match="K_TOO_LARGE"):
        lib.quantize_activation_zp(X, 6.0)


@pytest.mark.parametrize("name", ["decode", "qkv_prefill", "mlp_down_prefill",
                                  "decode_mlp_down"])
def test_workload_zp_sampled(lib, name):
    """The benchmark workloads at full size through int8_linear_zp: the whole
    activation stage bit-exact, sampled outputs against the oracle."""
    w = wl.WORKLOADS[name]
    say(f"workload {name} zero-point (sampled): generating inputs")
    X, W, cols = wl.make_inputs(w)
    say(f"workload {name}: running GPU")
    Xd, Wd = dev(X), dev(W)
    Wq, sw = lib.quantize_weight(Wd)
    S = lib.weight_code_sums(Wq)
    ws = lib.new_workspace(w.M, w.K, w.N, Xd.device)
    Y = lib.linear_zp(Xd, Wq, sw, S, Wd, w.threshold, workspace=ws)
    torch.cuda.synchronize()
    say(f"workload {name}: activation stage, full")
    act = O.quantize_activation_zp(X, w.threshold)
    np.testing.assert_array_equal(act[3], np.sort(cols))
    check_act(lib.workspace_views(ws, w.M, w.K), act, name)

    rng = np.random.default_rng(4321)
    ns = np.unique(np.concatenate([rng.integers(0, w.N, 48), [0, 255, 256, w.N - 1]]))
    Wq_r, sw_r = O.quantize_weight_rows(W, ns)
    np.testing.assert_array_equal(host(Wq[torch.as_tensor(ns, device="cuda:0")]), Wq_r)
    np.testing.assert_array_equal(host(S[torch.as_tensor(ns, device="cuda:0")]),
                                  O.weight_code_sums(Wq_r))
    n_s = 3000
    rows = np.concatenate([rng.integers(0, w.M, n_s), [0, w.M - 1, min(255, w.M - 1)]])
    pick = rng.integers(0, len(ns), len(rows))
    colsel = ns[pick]
    _, Y64 = O.int8_linear_zp_entries(act, Wq_r[pick], sw_r[pick], W, rows, colsel)
    ri = torch.as_tensor(rows, device="cuda:0")
    ci = torch.as_tensor(colsel, device="cuda:0")
    assert_y(host(Y[ri, ci]), Y64, name)
    assert torch.isfinite(Y).all().item()
    del Y, Wq, ws, Xd, Wd, S
    torch.cuda.empty_cache()
