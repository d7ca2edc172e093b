"""CPU oracle for the LLM.int8() linear layer -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The product (the HIP library and its Python binding)
never calls it and shares no code with it.

It is a plain, slow, step-by-step restatement of the method described in the
blog "A Gentle Introduction to 8-bit Matrix Multiplication for transformers at
scale using Hugging Face Transformers, Accelerate and bitsandbytes" (cited
below as [blog]; the three translated pages carry the same text):

  * [blog, "Introduction to model quantization"]: absmax quantization maps a
    vector onto [-127, 127] by scaling with 127 / absmax and rounding;
    vector-wise quantization uses one absmax per row of the left operand and
    one per column of the right operand, multiplies the int8 matrices, and
    denormalises by the outer product of the two absmax vectors.
  * [blog, "A gentle summary of LLM.int8()"]: three steps -- pull out outlier
    columns of the hidden states by a threshold; multiply the outliers in fp16
    and the rest in int8; dequantize the int8 result and add both in fp16.
  * [blog, "A closer look at the MatMul" (MatMul 内部)]: threshold 6 (values of
    magnitude 6 or more are outliers), hidden states quantized per row, weight
    per column, int8 result dequantized and added to the fp16 outlier product.
  * [blog, "Usage"]: the weight is quantized once when the module is moved to
    the GPU; CB is the int8 weight in nn.Linear layout [out][in], SCB holds one
    absmax per output feature, and CB * SCB / 127 recovers the fp16 weight.

Readings taken where the text is silent or garbled (each is also listed with
its reason in the design notes of the repository):
  r1  outlier test is |x| >= t (the MatMul section says "6 or more"; the summary
      says "greater than"); t <= 0 or t = +inf disables the decomposition.
  r2  an outlier is a whole column of X over all rows of the call.
  r3  outlier columns do not take part in the row absmax of X.
  r4  the weight absmax runs over all K input features (quantized at load time,
      before any activation is seen).
  r5  rounding is round-half-away-from-zero, then clamp to [-127, 127].
  r6  the scale is computed as fl32(127 / absmax) (IEEE fp32 division) and the
      element is scaled by one fp32 multiply; fp16 -> fp32 is exact.  The
      quantized codes are integers decided by floating point, so the oracle
      takes that decision in the same fp32 precision as the kernels.
  r7  absmax == 0 gives an all-zero code vector.
  r8  dequantization and the add are done in fp64 here with one final rounding
      to fp16 (round to nearest even, overflow to +/-inf).
  r9  the dequantization scale of the weight indexes the OUTPUT feature; the
      Usage section's printed dequantization broadcasts it along the other axis
      of a square matrix, which is a display artefact, not the method.
  r10 when no fp16 weight is kept, the outlier rows are rebuilt from the codes
      as the Usage section does, on fp32 values (code x scale, then / 127),
      and rounded to fp16 for the fp16 outlier product.
  r11 zero-point variant (the unsigned int8 scheme of "Introduction to model
      quantization": subtract the minimum, scale by the range, zero exact):
      per row of X over the regular columns lo = min(0, min x), hi = max(0,
      max x); inv = fl32(255 / fl32(hi - lo)); zp = RHAZ(fl32(-lo * inv));
      q = clamp(RHAZ(fl32(x * inv)) + zp, 0, 255); outlier columns take q = zp;
      the row's dequantization factor is xscale = fl32(fl32(hi - lo) / 255).
      Codes are kept as q - 128 (int8) and the weight stays absmax per
      column, so sum_k (q - zp) w = sum_k (q - 128) w + (128 - zp) S[n] with
      S[n] = sum_k Wq[n][k]; K <= 66304 keeps every such sum inside int32.
  r13 mixed int8/fp16 training mode ([blog, "Usage"]: has_fp16_weights=True,
      the default, is for training in mixed Int8/FP16 precision; the pages
      describe no gradient path).  Reading: the fp16 weight is the trained
      parameter; every forward call re-quantizes it (its codes follow each
      update) and runs the layer as above; the backward pass treats the
      quantization as the identity, so the gradients are those of the exact
      product X @ W: dX = dY @ W^T, dW = X^T @ dY, dbias = sum over rows of dY,
      each formed in fp64 here and rounded once to fp16.
  r12 non-finite X (outside the layer's contract, but the outlier set is still
      defined once): a column is an outlier when some entry has |x| >= t; a
      NaN entry never satisfies that (NaN >= t is false), so it neither makes
      its column an outlier nor keeps a large entry beside it from doing so;
      +/-inf reaches every finite t.

Layouts (row-major numpy arrays):
  X  fp16 [M][K]        W  fp16 [K][N]  (math layout, Y = X @ W)
  Wq int8 [N][K]        sw fp32 [N]     (CB / SCB layout: one row per output)
  Xq int8 [M][K]        sx fp32 [M]     idx int32 [n_out] ascending
  X_O fp16 [M][n_out]   acc int32 [M][N]   Y fp16 [M][N]

Everything that is not a quantization decision is computed in fp64.
"""
from __future__ import annotations

import numpy as np

INT8_MAX = 127

__all__ = [
    "rhaz",
    "absmax_codes",
    "quantize_weight",
    "quantize_weight_rows",
    "outlier_columns",
    "quantize_activation",
    "int8_matmul",
    "outlier_matmul",
    "dequantize_add",
    "int8_linear",
    "int8_linear_entries",
    "dequantize_weight",
    "decomposition_enabled",
    "zero_point_codes",
    "quantize_activation_zp",
    "weight_code_sums",
    "int8_linear_zp",
    "train_forward",
    "linear_backward_input",
    "linear_backward_weight",
    "linear_backward_bias",
    "linear_backward_entries",
]


def rhaz(v) -> np.ndarray:
    """Round half away from zero, evaluated in fp64 (r5).

    For the fp32 inputs used here |v| < 2^8, so |v| + 0.5 is exact in fp64 and
    floor() gives the exact rounding.
    """
    v = np.asarray(v, dtype=np.float64)
    return np.sign(v) * np.floor(np.abs(v) + 0.5)


def absmax_codes(values_f32: np.ndarray, absmax_f32: np.ndarray) -> np.ndarray:
    """Absmax quantization of fp32 values with a given fp32 absmax (r5, r6, r7).

    [blog, "Introduction to model quantization"]: divide 127 by the absolute
    maximum to get the scaling factor, multiply, round, stay inside
    [-127, 127].  ``absmax_f32`` broadcasts against ``values_f32``.
    """
    values = np.asarray(values_f32, dtype=np.float32)
    absmax = np.asarray(absmax_f32, dtype=np.float32)
    safe = np.where(absmax > 0, absmax, np.float32(1.0)).astype(np.float32)
    inv = (np.float32(INT8_MAX) / safe).astype(np.float32)          # fl32(127 / absmax)
    scaled = (values * inv).astype(np.float32)                      # one fp32 multiply
    codes = np.clip(rhaz(scaled), -INT8_MAX, INT8_MAX)
    codes = np.where(absmax > 0, codes, 0.0)                        # r7
    return codes.astype(np.int8)


def quantize_weight(W16: np.ndarray):
    """Column-wise absmax quantization of the weight (r4, r5, r6, r7).

    [blog, "A closer look at the MatMul"]: the weight matrix is quantized per
    column (one absmax per output feature of Y = X @ W).  [blog, "Usage"]: the
    int8 weight keeps nn.Linear's [out][in] layout, so Wq is [N][K] here, and
    the per-output absmax is kept next to it.

    Returns (Wq int8 [N][K], sw fp32 [N]).
    """
    W = np.asarray(W16, dtype=np.float16)
    assert W.ndim == 2
    return quantize_weight_rows(W, np.arange(W.shape[1]))


def quantize_weight_rows(W16: np.ndarray, cols) -> tuple:
    """Rows ``cols`` of Wq (= columns of W) and their scales, one column at a time
    stacked -- used to check sampled outputs of the full-size weights."""
    W = np.asarray(W16, dtype=np.float16)
    cols = np.asarray(cols, dtype=np.int64)
    Wt = W[:, cols].astype(np.float32).T                 # [len(cols)][K], exact fp16 -> fp32
    sw = np.abs(Wt).max(axis=1) if Wt.shape[1] else np.zeros(len(cols), np.float32)
    sw = sw.astype(np.float32)
    Wq = absmax_codes(Wt, sw[:, None])
    return Wq, sw


def decomposition_enabled(threshold: float) -> bool:
    """r1: a finite, positive threshold enables the outlier decomposition."""
    t = float(threshold)
    if np.isnan(t):
        raise ValueError("threshold is NaN")
    return 0.0 < t < np.inf


def outlier_columns(X16: np.ndarray, threshold: float) -> np.ndarray:
    """Ascending indices of the outlier columns of X (r1, r2).

    [blog, "A gentle summary of LLM.int8()"], step 1: outliers are taken out of
    the hidden states column by column; [blog, "A closer look at the MatMul"]:
    magnitude 6 or more.  A column is an outlier when some entry of it, in any
    row, has magnitude at least the threshold (r12: a NaN entry never does).
    """
    X = np.asarray(X16, dtype=np.float16)
    if not decomposition_enabled(threshold) or X.shape[0] == 0:
        return np.zeros(0, dtype=np.int32)
    with np.errstate(invalid="ignore"):
        hit = np.abs(X.astype(np.float32)) >= np.float32(threshold)
    return np.nonzero(hit.any(axis=0))[0].astype(np.int32)


def quantize_activation(X16: np.ndarray, threshold: float):
    """Decompose X and quantize its regular part row by row (r1-r3, r5-r7).

    [blog, "A closer look at the MatMul"]: after the outlier columns are split
    off, the hidden states are quantized per row.  The outlier columns are
    zero in Xq and are copied, in ascending column order, to X_O.

    Returns (Xq int8 [M][K], sx fp32 [M], idx int32 [n_out], X_O fp16 [M][n_out]).
    """
    X = np.asarray(X16, dtype=np.float16)
    M, K = X.shape
    idx = outlier_columns(X, threshold)
    regular = np.ones(K, dtype=bool)
    regular[idx] = False
    Xf = X.astype(np.float32)
    Xr = np.where(regular[None, :], Xf, np.float32(0.0))
    sx = (np.abs(Xr).max(axis=1) if K else np.zeros(M)).astype(np.float32)   # r3
    Xq = absmax_codes(Xr, sx[:, None])
    Xq[:, ~regular] = 0
    X_O = X[:, idx].copy()
    return Xq, sx, idx, X_O


def int8_matmul(Xq: np.ndarray, Wq: np.ndarray, block: int = 2048) -> np.ndarray:
    """acc[i, n] = sum_k Xq[i, k] * Wq[n, k], exactly, as int32.

    [blog, "Introduction to model quantization"]: the normalised int8 matrices
    are multiplied.  The product is formed by an fp64 matrix multiply of the
    int8 values: every partial sum is an integer of magnitude at most
    K * 127^2 < 2^53, so any summation order gives the exact integer.
    Blocked over N only to bound host memory.
    """
    Xq = np.asarray(Xq, dtype=np.int8)
    Wq = np.asarray(Wq, dtype=np.int8)
    M, K = Xq.shape
    N = Wq.shape[0]
    assert Wq.shape[1] == K
    assert K * INT8_MAX * INT8_MAX < 2**31
    acc = np.empty((M, N), dtype=np.int32)
    A = Xq.astype(np.float64)
    for n0 in range(0, N, block):
        B = Wq[n0:n0 + block].astype(np.float64)
        acc[:, n0:n0 + block] = (A @ B.T).astype(np.int32)
    return acc


def outlier_matmul(X_O: np.ndarray, W16: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Yo = X_O @ W[idx, :] in fp64 (fp16 x fp16 products are exact in fp64).

    [blog, "A gentle summary of LLM.int8()"], step 2: the outlier part is an
    ordinary fp16 matrix product against the matching rows of the weight.
    """
    X_O = np.asarray(X_O, dtype=np.float16).astype(np.float64)
    W = np.asarray(W16, dtype=np.float16)
    WO = W[np.asarray(idx, dtype=np.int64), :].astype(np.float64)
    return X_O @ WO


def dequantize_add(acc, sx, sw, Yo, bias=None):
    """Y64 = acc * sx[i] * sw[n] / 127^2 + Yo (+ bias[n]); Y16 = fp16(Y64) (r8, r9).

    [blog, "Introduction to model quantization"]: denormalise by the outer
    product of the row and column absmax vectors (each code carries a factor
    127 / absmax, hence the 127^2).  [blog, "A gentle summary of LLM.int8()"],
    step 3: add the outlier product.  [blog, "Usage"]: the 8-bit layer keeps
    nn.Linear's bias, added to the output (before the one rounding, r8).
    """
    acc = np.asarray(acc, dtype=np.float64)
    sx = np.asarray(sx, dtype=np.float64)
    sw = np.asarray(sw, dtype=np.float64)
    Y64 = acc * np.multiply.outer(sx, sw) / float(INT8_MAX * INT8_MAX) + Yo
    if bias is not None:
        Y64 = Y64 + np.asarray(bias, dtype=np.float16).astype(np.float64)[None, :]
    with np.errstate(over="ignore"):
        Y16 = Y64.astype(np.float16)
    return Y64, Y16


def int8_linear(X16, Wq, sw, W16, threshold, bias=None):
    """The whole LLM.int8() linear layer on the CPU.

    Returns a dict with every intermediate: Xq, sx, idx, X_O, acc, Yo, Y64, Y.
    ``W16`` supplies the fp16 rows used for the outlier product; it may be a
    dequantized weight (see ``dequantize_weight``) when no fp16 copy is kept.
    """
    Xq, sx, idx, X_O = quantize_activation(X16, threshold)
    acc = int8_matmul(Xq, Wq)
    M, N = acc.shape
    if len(idx):
        Yo = outlier_matmul(X_O, W16, idx)
    else:
        Yo = np.zeros((M, N))
    Y64, Y = dequantize_add(acc, sx, sw, Yo, bias)
    return dict(Xq=Xq, sx=sx, idx=idx, X_O=X_O, acc=acc, Yo=Yo, Y64=Y64, Y=Y)


def int8_linear_entries(X16, Wq_rows, sw_rows, W16, threshold, rows, cols, act=None,
                        bias=None):
    """Y64 at sampled (rows[j], cols[j]) pairs, each computed on its own.

    ``Wq_rows`` / ``sw_rows`` hold the quantized weight rows for ``cols`` (in the
    same order), e.g. from ``quantize_weight_rows``; ``act`` may pass a
    precomputed ``quantize_activation`` result.
    """
    if act is None:
        act = quantize_activation(X16, threshold)
    Xq, sx, idx, X_O = act
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    acc = np.einsum(
        "jk,jk->j", Xq[rows].astype(np.float64), np.asarray(Wq_rows, np.int8).astype(np.float64)
    )
    Y64 = acc * sx[rows].astype(np.float64) * np.asarray(sw_rows, np.float64) / float(INT8_MAX**2)
    if len(idx):
        W = np.asarray(W16, dtype=np.float16)
        WO = W[idx.astype(np.int64)][:, cols].astype(np.float64)    # [n_out][len]
        Y64 = Y64 + np.einsum("jo,oj->j", X_O[rows].astype(np.float64), WO)
    if bias is not None:
        Y64 = Y64 + np.asarray(bias, dtype=np.float16).astype(np.float64)[cols]
    return acc.astype(np.int32), Y64


def dequantize_weight(Wq, sw) -> np.ndarray:
    """fp16 weight rebuilt from its codes: W[k, n] ~ Wq[n, k] * sw[n] / 127 (r9, r10).

    [blog, "Usage"]: the int8 weight times its per-output scale over 127 gives
    the fp16 weight back; the page forms it on fp32 tensors (code times scale,
    exact in fp32; then one IEEE fp32 division by 127) and the outlier product
    uses it as an fp16 operand, so the value is rounded once more, to fp16
    (round to nearest even).  Returned in math layout [K][N].
    """
    q = np.asarray(Wq, dtype=np.int8).astype(np.float32)
    s = np.asarray(sw, dtype=np.float32)
    prod = q * s[:, None]                       # exact: 8-bit integer x fp16 value
    return (prod / np.float32(INT8_MAX)).T.astype(np.float16)


# ---------------------------------------------------------------------------
# Zero-point (unsigned) variant of the activation quantizer (r11)
# ---------------------------------------------------------------------------
UINT8_MAX = 255
ZP_MAX_K = 66304          # 255 * 127 * K < 2^31


def zero_point_codes(values_f32, lo_f32, hi_f32):
    """Unsigned 8-bit codes with a zero point (r11).

    [blog, "Introduction to model quantization"]: for unsigned int8 the minimum
    is subtracted and the values scaled to the range; with the range widened
    to contain 0, the value 0 maps to an integer (the zero point) exactly.
    Returns (q int32 in [0, 255], zp int32, xscale fp32); broadcasts like
    ``absmax_codes``.
    """
    x = np.asarray(values_f32, dtype=np.float32)
    lo = np.minimum(np.asarray(lo_f32, dtype=np.float32), np.float32(0))
    hi = np.maximum(np.asarray(hi_f32, dtype=np.float32), np.float32(0))
    rng = (hi - lo).astype(np.float32)                                   # fl32
    safe = np.where(rng > 0, rng, np.float32(1.0)).astype(np.float32)
    inv = np.where(rng > 0, (np.float32(UINT8_MAX) / safe).astype(np.float32),
                   np.float32(0.0)).astype(np.float32)
    zp = rhaz((-lo * inv).astype(np.float32))
    q = np.clip(rhaz((x * inv).astype(np.float32)) + zp, 0, UINT8_MAX)
    xscale = (rng / np.float32(UINT8_MAX)).astype(np.float32)
    return q.astype(np.int32), zp.astype(np.int32), xscale


def quantize_activation_zp(X16: np.ndarray, threshold: float):
    """Decomposition as in ``quantize_activation``, then zero-point codes per row
    over the regular columns (r11).

    Returns (Xq int8 [M][K] = q - 128 (zp - 128 in outlier columns), zp int32 [M],
    xscale fp32 [M], idx int32 [n_out], X_O fp16 [M][n_out]).
    """
    X = np.asarray(X16, dtype=np.float16)
    M, K = X.shape
    idx = outlier_columns(X, threshold)
    regular = np.ones(K, dtype=bool)
    regular[idx] = False
    Xf = X.astype(np.float32)
    big = np.float32(np.inf)
    lo = np.where(regular[None, :], Xf, big).min(axis=1) if K else np.zeros(M, np.float32)
    hi = np.where(regular[None, :], Xf, -big).max(axis=1) if K else np.zeros(M, np.float32)
    lo = np.where(np.isfinite(lo), lo, 0).astype(np.float32)       # no regular column: 0
    hi = np.where(np.isfinite(hi), hi, 0).astype(np.float32)
    q, zp, xscale = zero_point_codes(Xf, lo[:, None], hi[:, None])
    zp = zp[:, 0]
    xscale = xscale[:, 0]
    q = np.where(regular[None, :], q, zp[:, None])
    return (q - 128).astype(np.int8), zp.astype(np.int32), xscale, idx, X[:, idx].copy()


def weight_code_sums(Wq) -> np.ndarray:
    """S[n] = sum_k Wq[n, k] as int32 (r11: the zero-point correction)."""
    return np.asarray(Wq, dtype=np.int8).astype(np.int64).sum(axis=1).astype(np.int32)


def int8_linear_zp(X16, Wq, sw, W16, threshold, bias=None):
    """The LLM.int8() layer with zero-point activation codes (r11):
    Y64 = sum_k (q - zp) w * xscale[i] * sw[n] / 127 + outlier product (+ bias)."""
    Xq, zp, xscale, idx, X_O = quantize_activation_zp(X16, threshold)
    qd = Xq.astype(np.float64) + 128.0 - zp.astype(np.float64)[:, None]    # q - zp, exact
    acc = qd @ np.asarray(Wq, np.int8).astype(np.float64).T                 # exact integers
    M, N = acc.shape
    Yo = outlier_matmul(X_O, W16, idx) if len(idx) else np.zeros((M, N))
    Y64 = acc * np.multiply.outer(xscale.astype(np.float64),
                                  np.asarray(sw, np.float64)) / float(INT8_MAX) + Yo
    if bias is not None:
        Y64 = Y64 + np.asarray(bias, dtype=np.float16).astype(np.float64)[None, :]
    with np.errstate(over="ignore"):
        Y = Y64.astype(np.float16)
    return dict(Xq=Xq, zp=zp, xscale=xscale, idx=idx, X_O=X_O, acc=acc.astype(np.int64),
                Y64=Y64, Y=Y)


def int8_linear_zp_entries(act_zp, Wq_rows, sw_rows, W16, rows, cols, bias=None):
    """Y64 of ``int8_linear_zp`` at sampled (rows[j], cols[j]) pairs (r11), each
    computed on its own from a ``quantize_activation_zp`` result; ``Wq_rows`` /
    ``sw_rows`` hold the weight rows for ``cols`` in the same order.
    Returns (acc int64 = sum_k (q - zp) w, Y64)."""
    Xq, zp, xscale, idx, X_O = act_zp
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    qd = Xq[rows].astype(np.float64) + 128.0 - zp[rows].astype(np.float64)[:, None]
    acc = np.einsum("jk,jk->j", qd, np.asarray(Wq_rows, np.int8).astype(np.float64))
    Y64 = acc * xscale[rows].astype(np.float64) * np.asarray(sw_rows, np.float64) / float(INT8_MAX)
    if len(idx):
        W = np.asarray(W16, dtype=np.float16)
        WO = W[idx.astype(np.int64)][:, cols].astype(np.float64)
        Y64 = Y64 + np.einsum("jo,oj->j", X_O[rows].astype(np.float64), WO)
    if bias is not None:
        Y64 = Y64 + np.asarray(bias, dtype=np.float16).astype(np.float64)[cols]
    return acc.astype(np.int64), Y64


# ---------------------------------------------------------------------------
# Mixed int8/fp16 training mode (r13)
# ---------------------------------------------------------------------------
def train_forward(X16, W16, threshold, bias=None):
    """Forward pass of the training mode (r13): the current fp16 weight is
    quantized afresh ([blog, "Usage"]: the codes are made from the fp16 weight)
    and the layer runs with that weight's own rows for the outlier product."""
    Wq, sw = quantize_weight(W16)
    r = int8_linear(X16, Wq, sw, W16, threshold, bias=bias)
    r["Wq"], r["sw"] = Wq, sw
    return r


def _to_fp16(Y64):
    with np.errstate(over="ignore"):
        return Y64.astype(np.float16)


def linear_backward_input(dY16, W16):
    """dX = dY @ W^T (r13): dY fp16 [M][N], W fp16 [K][N] (math layout).

    Returns (dX64 fp64 [M][K], dX fp16)."""
    dY = np.asarray(dY16, dtype=np.float16).astype(np.float64)
    W = np.asarray(W16, dtype=np.float16).astype(np.float64)
    dX64 = dY @ W.T
    return dX64, _to_fp16(dX64)


def linear_backward_weight(X16, dY16):
    """dW = X^T @ dY (r13): X fp16 [M][K], dY fp16 [M][N] -> [K][N], the
    weight's math layout.  Returns (dW64 fp64, dW fp16)."""
    X = np.asarray(X16, dtype=np.float16).astype(np.float64)
    dY = np.asarray(dY16, dtype=np.float16).astype(np.float64)
    dW64 = X.T @ dY
    return dW64, _to_fp16(dW64)


def linear_backward_bias(dY16):
    """dbias[n] = sum_i dY[i, n] (r13).  Returns (db64 fp64 [N], db fp16)."""
    db64 = np.asarray(dY16, dtype=np.float16).astype(np.float64).sum(axis=0)
    return db64, _to_fp16(db64)


def linear_backward_entries(A16, B16, rows, cols, transpose_a=False):
    """Entries (rows[j], cols[j]) of the two gradient products (r13), each one
    dot product in fp64, with the matching dot product of magnitudes:
      transpose_a False: dX[i, k] = sum_n dY[i, n] W[k, n]    (A = dY, B = W)
      transpose_a True:  dW[k, n] = sum_i X[i, k] dY[i, n]     (A = X,  B = dY)
    Returns (values fp64, magnitudes fp64)."""
    A = np.asarray(A16, dtype=np.float16)
    B = np.asarray(B16, dtype=np.float16)
    vals = np.empty(len(rows))
    mags = np.empty(len(rows))
    for j, (r, c) in enumerate(zip(rows, cols)):
        if transpose_a:
            a, b = A[:, r].astype(np.float64), B[:, c].astype(np.float64)
        else:
            a, b = A[r].astype(np.float64), B[c].astype(np.float64)
        vals[j] = a @ b
        mags[j] = np.abs(a) @ np.abs(b)
    return vals, mags
