"""Pins of the oracle's training-mode functions (no GPU).

[blog, "Usage"]: has_fp16_weights=True keeps the fp16 weight for training in
mixed int8/fp16 precision.  The reading (the oracle's r13): every forward
re-quantizes the current fp16 weight, and the backward pass is that of the
exact product X @ W.  These tests pin the oracle against things other than
itself: pure-Python integer brute force, the chain rule as torch's autograd
computes it in float64 on the CPU, one-hot closed forms, and the re-quantization
invariant.
"""
import itertools

import numpy as np
import pytest

from oracle import int8_oracle as O


def _dyadic(rng, shape, scale=16):
    """fp16 values k/scale with |k| <= 64: exactly representable, and every
    product and sum below is exact in fp64."""
    return (rng.integers(-64, 65, shape) / scale).astype(np.float16)


@pytest.mark.parametrize("M,K,N", [(3, 4, 5), (4, 4, 4), (1, 6, 2), (5, 2, 7)])
def test_backward_bruteforce(M, K, N):
    rng = np.random.default_rng(M * 100 + K * 10 + N)
    X, W, dY = _dyadic(rng, (M, K)), _dyadic(rng, (K, N)), _dyadic(rng, (M, N))
    x = [[float(v) for v in r] for r in X]
    w = [[float(v) for v in r] for r in W]
    g = [[float(v) for v in r] for r in dY]
    dX = [[sum(g[i][n] * w[k][n] for n in range(N)) for k in range(K)] for i in range(M)]
    dW = [[sum(x[i][k] * g[i][n] for i in range(M)) for n in range(N)] for k in range(K)]
    db = [sum(g[i][n] for i in range(M)) for n in range(N)]
    np.testing.assert_array_equal(O.linear_backward_input(dY, W)[0], np.array(dX))
    np.testing.assert_array_equal(O.linear_backward_weight(X, dY)[0], np.array(dW))
    np.testing.assert_array_equal(O.linear_backward_bias(dY)[0], np.array(db))
    # the fp16 results are the one rounding of those exact values
    np.testing.assert_array_equal(O.linear_backward_input(dY, W)[1],
                                  np.array(dX).astype(np.float16))


def test_backward_matches_autograd_float64():
    """The chain rule through L = sum(dY * (X @ W + b)), as torch's autograd
    computes it in float64 on the CPU, gives the oracle's three gradients."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    M, K, N = 7, 12, 9
    X = (rng.standard_normal((M, K))).astype(np.float16)
    W = (rng.standard_normal((K, N)) * 0.1).astype(np.float16)
    b = (rng.standard_normal(N)).astype(np.float16)
    dY = (rng.standard_normal((M, N))).astype(np.float16)
    tX = torch.tensor(X.astype(np.float64), requires_grad=True)
    tW = torch.tensor(W.astype(np.float64), requires_grad=True)
    tb = torch.tensor(b.astype(np.float64), requires_grad=True)
    L = (torch.tensor(dY.astype(np.float64)) * (tX @ tW + tb)).sum()
    gX, gW, gb = torch.autograd.grad(L, [tX, tW, tb])
    np.testing.assert_allclose(O.linear_backward_input(dY, W)[0], gX.numpy(), rtol=1e-12,
                               atol=1e-12)
    np.testing.assert_allclose(O.linear_backward_weight(X, dY)[0], gW.numpy(), rtol=1e-12,
                               atol=1e-12)
    np.testing.assert_allclose(O.linear_backward_bias(dY)[0], gb.numpy(), rtol=1e-12, atol=1e-12)


def test_backward_one_hot_closed_forms():
    """dY = e_(i, n): dX is zero but row i, which is column n of W; dW is zero
    but column n, which is row i of X; dbias is e_n.  A square, non-symmetric
    W catches a transposed operand."""
    rng = np.random.default_rng(9)
    M = K = N = 6
    X = _dyadic(rng, (M, K))
    W = _dyadic(rng, (K, N))
    assert not np.array_equal(W, W.T)
    for i, n in itertools.product((0, 3, 5), (1, 4)):
        dY = np.zeros((M, N), np.float16)
        dY[i, n] = 1.0
        dX = O.linear_backward_input(dY, W)[0]
        want = np.zeros((M, K))
        want[i] = W[:, n]
        np.testing.assert_array_equal(dX, want)
        dW = O.linear_backward_weight(X, dY)[0]
        want = np.zeros((K, N))
        want[:, n] = X[i]
        np.testing.assert_array_equal(dW, want)
        want = np.zeros(N)
        want[n] = 1.0
        np.testing.assert_array_equal(O.linear_backward_bias(dY)[0], want)


def test_train_forward_requantizes_the_current_weight():
    """r13: the codes follow the fp16 weight -- after an update the forward uses
    the codes of the new weight, not those it was built with."""
    rng = np.random.default_rng(11)
    M, K, N = 8, 64, 24
    X = (rng.standard_normal((M, K))).astype(np.float16)
    X[:, 5] = 9.0                                        # one outlier column
    W = (rng.standard_normal((K, N)) * 0.05).astype(np.float16)
    dY = (rng.standard_normal((M, N))).astype(np.float16)
    r0 = O.train_forward(X, W, 6.0)
    Wq0, sw0 = O.quantize_weight(W)
    np.testing.assert_array_equal(r0["Wq"], Wq0)
    np.testing.assert_array_equal(r0["Y64"], O.int8_linear(X, Wq0, sw0, W, 6.0)["Y64"])
    W1 = (W.astype(np.float32) - 0.5 * O.linear_backward_weight(X, dY)[1].astype(np.float32)
          ).astype(np.float16)
    r1 = O.train_forward(X, W1, 6.0)
    Wq1, sw1 = O.quantize_weight(W1)
    np.testing.assert_array_equal(r1["Wq"], Wq1)
    assert not np.array_equal(Wq1, Wq0)
    # the outlier column's product uses the new fp16 rows
    np.testing.assert_array_equal(r1["Y64"], O.int8_linear(X, Wq1, sw1, W1, 6.0)["Y64"])


def test_backward_entries_match_full():
    rng = np.random.default_rng(21)
    M, K, N = 9, 24, 16
    X = rng.standard_normal((M, K)).astype(np.float16)
    W = rng.standard_normal((K, N)).astype(np.float16)
    dY = rng.standard_normal((M, N)).astype(np.float16)
    r, c = rng.integers(0, M, 30), rng.integers(0, K, 30)
    v, mag = O.linear_backward_entries(dY, W, r, c)
    np.testing.assert_allclose(v, O.linear_backward_input(dY, W)[0][r, c], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(mag, (np.abs(dY.astype(np.float64)) @
                                     np.abs(W.astype(np.float64)).T)[r, c], rtol=1e-13)
    r, c = rng.integers(0, K, 30), rng.integers(0, N, 30)
    v, _ = O.linear_backward_entries(X, dY, r, c, transpose_a=True)
    np.testing.assert_allclose(v, O.linear_backward_weight(X, dY)[0][r, c], rtol=1e-13,
                               atol=1e-13)
