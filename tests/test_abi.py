"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import math
import os
import re
import subprocess

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "int8lin.h")
OK, INVALID, K_TOO_LARGE, WORKSPACE = 0, 1, 2, 3
P16 = 0x10000      # fake, 16-byte aligned, never dereferenced: every call below fails
                   # validation (or is an empty no-op) before touching the device


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"^#.*$", "", src, flags=re.M)        # preprocessor lines
    return sorted(set(re.findall(r"\b(\w+)\s*\([^;{]*\)\s*;", src)))


def test_header_matches_binding(i8l):
    assert declared_functions() == sorted(i8l.EXPORTS)


def test_library_exports_every_declared_symbol(i8l):
    from mixed_precision_quantized_int8_amd import _binding

    out = subprocess.run(["nm", "-D", "--defined-only", _binding.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    text = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for name in declared_functions():
        assert name in text, name
        assert hasattr(i8l.lib(), name)


def test_build_info(i8l):
    info = i8l.build_info()
    assert "gfx950" in info


def _linear(L, X=P16, M=32, K=64, Wq=P16, sw=P16, N=32, W=P16, t=6.0, Y=P16, ws=P16,
            wsb=1 << 40):
    return L.int8_linear(X, M, K, Wq, sw, N, W, t, Y, ws, wsb, None)


def test_linear_validation(i8l):
    L = i8l.lib()
    assert _linear(L, X=None) == INVALID and "X is NULL" in i8l.last_error()
    assert _linear(L, Wq=None) == INVALID
    assert _linear(L, sw=None) == INVALID
    assert _linear(L, Y=None) == INVALID
    assert _linear(L, ws=None) == INVALID
    # W_outlier_rows may be NULL (rows rebuilt from Wq, sw): a bad shape is still
    # caught before any HIP call
    assert _linear(L, W=None, K=8) == INVALID
    assert _linear(L, K=0) == INVALID
    assert _linear(L, K=8) == INVALID
    assert _linear(L, K=72) == INVALID
    assert _linear(L, K=-16) == INVALID
    assert _linear(L, M=-1) == INVALID
    assert _linear(L, N=-1) == INVALID
    assert _linear(L, K=133152) == K_TOO_LARGE
    assert _linear(L, K=133136, M=0) == OK          # largest K accepted (empty call)
    assert _linear(L, t=math.nan) == INVALID and "NaN" in i8l.last_error()
    assert _linear(L, X=P16 + 8) == INVALID and "aligned" in i8l.last_error()
    assert _linear(L, Y=P16 + 2) == INVALID
    assert _linear(L, sw=P16 + 2) == INVALID
    assert _linear(L, W=P16 + 1) == INVALID and "W_outlier_rows" in i8l.last_error()
    assert _linear(L, ws=P16 + 4) == INVALID
    need = i8l.workspace_bytes(32, 64, 32)
    assert _linear(L, wsb=need - 1) == WORKSPACE and str(need) in i8l.last_error()


def test_linear_empty_calls_are_noops(i8l):
    L = i8l.lib()
    assert _linear(L, M=0) == OK and i8l.last_error() == ""
    assert _linear(L, N=0) == OK
    # decomposition disabled: W may be NULL
    for t in (0.0, -1.0, math.inf):
        assert _linear(L, M=0, W=None, t=t) == OK


def test_other_entry_points_validate(i8l):
    L = i8l.lib()
    assert L.int8_quantize_weight(None, 64, 32, P16, P16, None) == INVALID
    assert L.int8_quantize_weight(P16, 64, 32, P16 + 8, P16, None) == INVALID
    assert L.int8_quantize_weight(P16, 70, 32, P16, P16, None) == INVALID
    assert L.int8_quantize_weight(P16, 200000, 32, P16, P16, None) == K_TOO_LARGE
    assert L.int8_quantize_weight(P16, 64, 0, P16, P16, None) == OK
    assert L.int8_gemm_i32(P16, P16, 4, 4, 24, P16, None, 0, None) == INVALID
    assert L.int8_gemm_i32(None, P16, 4, 4, 32, P16, None, 0, None) == INVALID
    assert L.int8_gemm_i32(P16, P16, 0, 4, 32, P16, None, 0, None) == OK
    # a workspace must be aligned and large enough for the split tail
    assert L.int8_gemm_i32(P16, P16, 520, 1300, 2048, P16, P16 + 8, 1 << 40, None) == INVALID
    assert L.int8_gemm_i32(P16, P16, 520, 1300, 2048, P16, P16, 16, None) == WORKSPACE
    args = [P16, 8, 64, 6.0, P16, P16, P16, P16, P16, P16, 1 << 40, None]
    for i in (0, 4, 5, 6, 7, 8, 9):
        bad = list(args)
        bad[i] = None
        assert L.int8_quantize_activation(*bad) == INVALID, i
    bad = list(args)
    bad[3] = math.nan
    assert L.int8_quantize_activation(*bad) == INVALID
    bad = list(args)
    bad[10] = 16
    assert L.int8_quantize_activation(*bad) == WORKSPACE


def test_zero_point_entry_points_validate(i8l):
    L = i8l.lib()

    def lin(X=P16, M=32, K=64, Wq=P16, sw=P16, S=P16, N=32, W=P16, b=None, t=6.0, Y=P16,
            ws=P16, wsb=1 << 40):
        return L.int8_linear_zp(X, M, K, Wq, sw, S, N, W, b, t, Y, ws, wsb, None)

    assert lin(S=None) == INVALID and "wsum is NULL" in i8l.last_error()
    assert lin(S=P16 + 2) == INVALID and "aligned" in i8l.last_error()
    assert lin(X=None) == INVALID
    assert lin(b=P16 + 1) == INVALID and "bias" in i8l.last_error()
    assert lin(t=math.nan) == INVALID
    assert lin(K=72) == INVALID
    # zero-point codes: 255 * 127 * K must fit in int32
    assert lin(K=66320) == K_TOO_LARGE and "66304" in i8l.last_error()
    assert lin(K=66304, M=0) == OK
    assert lin(M=0) == OK and lin(N=0) == OK
    need = i8l.workspace_bytes(32, 64, 32)
    assert lin(wsb=need - 1) == WORKSPACE

    args = [P16, 8, 64, 6.0, P16, P16, P16, P16, P16, P16, P16, 1 << 40, None]
    for i in (0, 4, 5, 6, 7, 8, 9, 10):
        bad = list(args)
        bad[i] = None
        assert L.int8_quantize_activation_zp(*bad) == INVALID, i
    bad = list(args)
    bad[2] = 66320
    assert L.int8_quantize_activation_zp(*bad) == K_TOO_LARGE
    bad = list(args)
    bad[11] = 16
    assert L.int8_quantize_activation_zp(*bad) == WORKSPACE

    assert L.int8_weight_code_sums(None, 8, 64, P16, None) == INVALID
    assert L.int8_weight_code_sums(P16, 8, 64, None, None) == INVALID
    assert L.int8_weight_code_sums(P16 + 4, 8, 64, P16, None) == INVALID
    assert L.int8_weight_code_sums(P16, 8, 70, P16, None) == INVALID
    assert L.int8_weight_code_sums(P16, 0, 64, P16, None) == OK
    assert i8l.MAX_K_ZP == 66304


def test_workspace_layout(i8l):
    for (M, K) in [(1, 16), (16, 1024), (2048, 14336), (4096, 57344), (300, 272)]:
        L = i8l.workspace_layout(M, K, 123)
        offs = [L[k] for k in ("n_outliers", "outlier_idx", "sx", "flags", "Xq", "X_outliers")]
        assert all(o % 256 == 0 for o in offs)
        assert offs == sorted(offs)
        assert L["outlier_idx"] - L["n_outliers"] >= 4
        assert L["sx"] - L["outlier_idx"] >= 4 * K
        assert L["flags"] - L["sx"] >= 4 * M
        assert L["Xq"] - L["flags"] >= 4 * ((K + 31) // 32)
        assert L["X_outliers"] - L["Xq"] >= M * K
        assert L["zero_points"] - L["X_outliers"] >= 2 * M * K
        assert L["act_partials"] - L["zero_points"] >= 4 * M
        assert L["act_partials"] % 256 == 0
        act_words = -(-K // 512) * 33 if 1 <= M <= 16 else 0
        assert L["gemm_counters"] - L["act_partials"] >= 4 * act_words
        assert L["act_partials"] == i8l.workspace_layout(M, K, 0)["act_partials"]
        assert L["zero_points"] % 256 == 0
        assert L["zero_points"] == i8l.workspace_layout(M, K, 0)["zero_points"]
        assert L["gemm_partials"] >= L["gemm_counters"]
        assert L["total"] - L["gemm_partials"] >= L["gemm_slices"] * 256 * 256 * 4
        if L["gemm_slices"]:
            assert L["gemm_partials"] - L["gemm_counters"] >= 4 * 256
        assert i8l.workspace_bytes(M, K, 123) == L["total"]
    # split-K tail of the GEMM: the tiles of a partial last round over 256
    # compute units, split along K into S = min(256 / tiles, k-steps / 8) >= 2
    # parts; none for decode shapes
    assert i8l.workspace_layout(16, 4096, 16384)["gemm_slices"] == 0
    assert i8l.workspace_layout(2048, 14336, 43008)["gemm_slices"] == 64 * 4   # 1344 tiles
    assert i8l.workspace_layout(2048, 2048, 12200)["gemm_slices"] == 128 * 2   # 384 tiles
    assert i8l.workspace_layout(4096, 57344, 14336)["gemm_slices"] == 128 * 2  # 896 tiles
    assert i8l.workspace_layout(8192, 8192, 8192)["gemm_slices"] == 0         # 1024 tiles
    assert i8l.workspace_layout(520, 2048, 1300)["gemm_slices"] == 18 * 2     # 18 tiles
    # M <= 256 never reaches the 256 x 256 GEMM (M <= 64: the small-M kernels;
    # 64 < M <= 256: 256 x 64 tiles, never split), so no partial tiles there
    assert i8l.workspace_layout(32, 4096, 16384)["gemm_slices"] == 0
    assert i8l.workspace_layout(64, 4096, 16384)["gemm_slices"] == 0
    assert i8l.workspace_layout(65, 4096, 16384)["gemm_slices"] == 0
    assert i8l.workspace_layout(256, 4096, 16384)["gemm_slices"] == 0
    assert i8l.workspace_layout(257, 4096, 16384)["gemm_slices"] == 128 * 2   # 128 tiles
    assert i8l.workspace_bytes(4, 70, 4) == 0
    with pytest.raises(i8l.Int8LinError):
        i8l.workspace_layout(4, 70)


def test_missing_library_fails_loudly(monkeypatch):
    from mixed_precision_quantized_int8_amd import _binding

    monkeypatch.setattr(_binding, "_lib", None)
    monkeypatch.setattr(_binding, "LIB_PATH", "/nonexistent/libint8lin.so")
    with pytest.raises(RuntimeError, match="missing"):
        _binding.lib()


def test_static_entry_point_validates(i8l):
    """int8_linear_static checks its arguments and the scratch size on the host,
    before it looks up the scratch array or enqueues anything."""
    L = i8l.lib()
    hdr = open(HEADER).read()
    m = re.search(r"#define I8L_STATIC_SCRATCH_BYTES \((\d+)u << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == i8l.STATIC_SCRATCH_BYTES

    def call(X=P16, M=8, K=64, N=32, Y=P16, t=6.0):
        return L.int8_linear_static(X, M, K, P16, P16, N, None, None, t, Y, None)

    assert call(X=None) == INVALID and "X is NULL" in i8l.last_error()
    assert call(Y=None) == INVALID
    assert call(K=24) == INVALID
    assert call(t=math.nan) == INVALID
    assert call(M=0) == OK and call(N=0) == OK
    # 3 * 4096 * 4096 bytes of codes and outlier values: beyond the scratch
    assert call(M=4096, K=4096, N=256) == WORKSPACE
    assert "static scratch" in i8l.last_error()
    assert call(M=64, K=200000) == K_TOO_LARGE
