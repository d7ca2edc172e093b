"""The mixed int8/fp16 training mode on MI355X against the CPU oracle.

[blog, "Usage"]: has_fp16_weights=True keeps the fp16 weight for training in
mixed int8/fp16 precision.  Reading (the oracle's r13): each forward
re-quantizes the current fp16 weight; the gradients are those of X . W + b.
The GPU forms them from fp16 operands with fp32 accumulation and rounds once
to fp16, so against the oracle's fp64 value g64 an entry may differ by

    |g - g64| <= 2^-11 |g64| + L 2^-24 (|A| |B|) + 2^-24

(half an fp16 ulp of the result, relative, plus the worst-case growth of an
fp32 sum of L products -- each product of two fp16 values is exact in fp32 --
for the contraction length L, where (|A| |B|) is the same product formed from
the magnitudes; the last term covers fp16 subnormal spacing).  The bias
gradient is the same bound with B = 1.
"""
import zlib

import numpy as np
import pytest

from mixed_precision_quantized_int8_amd import workloads as wl
from oracle import int8_oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lib(i8l):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    return i8l


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def say(*a):
    print(*a, flush=True)


def assert_grad(g, g64, mag, L, what):
    """g: fp16 result; g64: fp64 oracle value; mag: the product of magnitudes."""
    g = np.asarray(g).astype(np.float64)
    tol = 2.0 ** -11 * np.abs(g64) + L * 2.0 ** -24 * mag + 2.0 ** -24
    err = np.abs(g - g64)
    bad = ~(err <= tol)
    if bad.any():
        k = np.unravel_index(np.argmax(np.where(bad, err - tol, -np.inf)), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside the bound; worst "
                             f"at {k}: gpu={g[k]!r} ref={g64[k]!r} tol={tol[k]!r}")


def grads_inputs(M, K, N, seed):
    """X, W of the workload recipe (with outlier columns) and an upstream
    gradient dY ~ N(0, 1) in fp16."""
    X, W, _ = wl.make_small(M, K, N, seed=seed, n_out=min(3, K))
    rng = np.random.default_rng(seed + 1)
    dY = rng.standard_normal((M, N), dtype=np.float32).astype(np.float16)
    return X, W, dY


SHAPES = [(300, 1040, 520), (1, 64, 8), (17, 256, 136), (64, 16, 8), (513, 272, 264),
          (1024, 4096, 2048), (8, 4096, 16384)]


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_backward_input(lib, M, K, N):
    say(f"backward_input M={M} K={K} N={N}")
    X, W, dY = grads_inputs(M, K, N, M + K + N)
    dX = lib.backward_input(dev(dY), dev(W))
    g64, _ = O.linear_backward_input(dY, W)
    mag = np.abs(dY.astype(np.float64)) @ np.abs(W.astype(np.float64)).T
    assert_grad(host(dX), g64, mag, N, f"dX {M}x{K}x{N}")


@pytest.mark.parametrize("M,K,N", SHAPES)
@pytest.mark.parametrize("with_bias", [True, False], ids=["bias", "nobias"])
def test_backward_weight(lib, M, K, N, with_bias):
    say(f"backward_weight M={M} K={K} N={N} bias={with_bias}")
    X, W, dY = grads_inputs(M, K, N, M + 2 * K + N)
    ws = torch.full((lib.lib().i8l_backward_weight_workspace_bytes(M, K, N),), 0x7f,
                    dtype=torch.uint8, device="cuda:0")   # stale bytes must not leak
    dW, db = lib.backward_weight(dev(X), dev(dY), with_bias=with_bias, workspace=ws)
    g64, _ = O.linear_backward_weight(X, dY)
    mag = np.abs(X.astype(np.float64)).T @ np.abs(dY.astype(np.float64))
    assert_grad(host(dW), g64, mag, M, f"dW {M}x{K}x{N}")
    if with_bias:
        b64, _ = O.linear_backward_bias(dY)
        assert_grad(host(db), b64, np.abs(dY.astype(np.float64)).sum(axis=0), M, "dbias")
    else:
        assert db is None


def test_backward_empty(lib):
    say("backward with M = 0 and N = 0")
    K, N = 64, 24
    X = torch.zeros((0, K), dtype=torch.float16, device="cuda:0")
    dY = torch.zeros((0, N), dtype=torch.float16, device="cuda:0")
    dW, db = lib.backward_weight(X, dY, with_bias=True)
    assert (host(dW) == 0).all() and (host(db) == 0).all()
    W = torch.ones((K, 0), dtype=torch.float16, device="cuda:0")
    dYe = torch.ones((5, 0), dtype=torch.float16, device="cuda:0")
    out = torch.full((5, K), 3.0, dtype=torch.float16, device="cuda:0")
    dX = lib.backward_input(dYe, W, out=out)
    assert (host(dX) == 0).all()


def test_backward_rejects_bad_n(lib):
    with pytest.raises(lib.Int8LinError, match="multiple of 8"):
        lib.backward_input(torch.zeros((4, 12), dtype=torch.float16, device="cuda:0"),
                           torch.zeros((64, 12), dtype=torch.float16, device="cuda:0"))


def test_backward_deterministic(lib):
    say("backward determinism")
    M, K, N = 300, 1040, 520
    X, W, dY = (dev(a) for a in grads_inputs(M, K, N, 5))
    a = [lib.backward_input(dY, W) for _ in range(2)]
    b = [lib.backward_weight(X, dY, with_bias=True) for _ in range(2)]
    np.testing.assert_array_equal(host(a[0]).view(np.uint16), host(a[1]).view(np.uint16))
    np.testing.assert_array_equal(host(b[0][0]).view(np.uint16), host(b[1][0]).view(np.uint16))
    np.testing.assert_array_equal(host(b[0][1]).view(np.uint16), host(b[1][1]).view(np.uint16))


@pytest.mark.parametrize("name", ["mlp_down_prefill", "qkv_prefill"])
def test_backward_full_size_sampled(lib, name):
    """The BLOOM-176B prefill layers' gradients at full size: one entry in every
    256 x 256 output tile of dX and dW (plus random ones), the bias gradient
    whole; the outputs are filled with NaN first, so an unwritten entry
    cannot pass."""
    w = wl.WORKLOADS[name]
    say(f"backward full size {name}: inputs")
    X, W, _ = wl.make_inputs(w)
    rng = np.random.default_rng(77)
    dY = rng.standard_normal((w.M, w.N), dtype=np.float32).astype(np.float16)
    Xd, Wd, dYd = dev(X), dev(W), dev(dY)
    say(f"backward full size {name}: GPU")
    dX = torch.full((w.M, w.K), float("nan"), dtype=torch.float16, device="cuda:0")
    lib.backward_input(dYd, Wd, out=dX)
    dW, db = lib.backward_weight(Xd, dYd, with_bias=True)
    torch.cuda.synchronize()
    assert not torch.isnan(dX).any().item() and not torch.isnan(dW).any().item()
    del Xd, Wd
    for (what, out, R, C, L, A, B, ta) in [("dX", dX, w.M, w.K, w.N, dY, W, False),
                                           ("dW", dW, w.K, w.N, w.M, X, dY, True)]:
        T0, T1 = np.meshgrid(np.arange(0, R, 256), np.arange(0, C, 256), indexing="ij")
        rows = np.concatenate([np.minimum(T0.ravel() + rng.integers(0, 256, T0.size), R - 1),
                               rng.integers(0, R, 500)])
        cols = np.concatenate([np.minimum(T1.ravel() + rng.integers(0, 256, T1.size), C - 1),
                               rng.integers(0, C, 500)])
        got = host(out[torch.as_tensor(rows, device="cuda:0"), torch.as_tensor(cols, device="cuda:0")])
        g64, mag = O.linear_backward_entries(A, B, rows, cols, transpose_a=ta)
        assert_grad(got, g64, mag, L, f"{name} {what} sampled")
    b64, _ = O.linear_backward_bias(dY)
    assert_grad(host(db), b64, np.abs(dY.astype(np.float64)).sum(axis=0), w.M, f"{name} dbias")
    del dX, dW, db
    torch.cuda.empty_cache()


@pytest.mark.parametrize("M,K,N,bias", [(300, 1040, 520, True), (8, 1024, 4096, True),
                                        (40, 2048, 264, False)])
def test_module_training_step(lib, M, K, N, bias):
    """Int8Linear with fp16 weights through autograd: the forward equals the
    oracle's training forward, the three gradients equal the oracle's within the
    bound above, and after an SGD step the next forward uses the codes of the
    updated weight (bit-exact against the oracle's quantization of it)."""
    from mixed_precision_quantized_int8_amd.module import Int8Linear

    say(f"Int8Linear training step M={M} K={K} N={N} bias={bias}")
    seed = zlib.crc32(f"{M}{K}{N}".encode()) % 1000
    X, W, dY = grads_inputs(M, K, N, seed)
    b = (np.random.default_rng(seed).standard_normal(N) * 0.5).astype(np.float16)
    lin = torch.nn.Linear(K, N, bias=bias)
    with torch.no_grad():
        lin.weight.copy_(torch.from_numpy(W.T.astype(np.float32)))
        if bias:
            lin.bias.copy_(torch.from_numpy(b.astype(np.float32)))
    m = Int8Linear.from_linear(lin, has_fp16_weights=True, threshold=6.0, device="cuda:0")
    assert m.weight16.requires_grad and (m.bias is None or m.bias.requires_grad)
    x = dev(X).requires_grad_(True)
    y = m(x)
    r = O.train_forward(X, W, 6.0, bias=b if bias else None)
    from test_parity_gpu import assert_y
    assert_y(host(y), r["Y64"], r["Y"], "training forward")
    y.backward(dev(dY))
    gx64, _ = O.linear_backward_input(dY, W)
    assert_grad(host(x.grad), gx64,
                np.abs(dY.astype(np.float64)) @ np.abs(W.astype(np.float64)).T, N, "x.grad")
    gw64, _ = O.linear_backward_weight(X, dY)
    assert_grad(host(m.weight16.grad), gw64,
                np.abs(X.astype(np.float64)).T @ np.abs(dY.astype(np.float64)), M, "weight.grad")
    if bias:
        gb64, _ = O.linear_backward_bias(dY)
        assert_grad(host(m.bias.grad), gb64, np.abs(dY.astype(np.float64)).sum(axis=0), M,
                    "bias.grad")
    # one SGD step on the fp16 parameters, then the codes follow the weight
    opt = torch.optim.SGD(m.parameters(), lr=0.05)
    opt.step()
    W1 = host(m.weight16).astype(np.float16)
    b1 = host(m.bias).astype(np.float16) if bias else None
    y1 = m(dev(X))
    Wq1, sw1 = O.quantize_weight(W1)
    np.testing.assert_array_equal(host(m.Wq), Wq1)
    np.testing.assert_array_equal(host(m.sw).view(np.uint32), sw1.view(np.uint32))
    assert not np.array_equal(Wq1, O.quantize_weight(W)[0])
    r1 = O.train_forward(X, W1, 6.0, bias=b1)
    assert_y(host(y1), r1["Y64"], r1["Y"], "forward after the step")
