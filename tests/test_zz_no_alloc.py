"""int8_linear_static (no workspace argument: the library's static scratch
array) against int8_linear_bias with a caller workspace, through the C ABI.

The two entry points run the same kernels on the same inputs, so their outputs
must be identical bit for bit; each pair of calls below runs back to back on
the one scratch array, the second with a smaller input, so a stale
intermediate of the first call would show up in the second.
"""
import numpy as np
import pytest

from mixed_precision_quantized_int8_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lib(i8l):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    return i8l


def say(*a):
    print(*a, flush=True)


def layer(lib, M, K, N, seed, n_out, bias, pass_w):
    X, W, _ = wl.make_small(M, K, N, seed=seed, n_out=n_out)
    Xd = torch.from_numpy(X).to("cuda:0")
    Wd = torch.from_numpy(W).to("cuda:0")
    Wq, sw = lib.quantize_weight(Wd)
    b = (torch.randn(N, device="cuda:0") * 0.5).half() if bias else None
    return Xd, Wq, sw, (Wd if pass_w else None), b


# pairs of (M, K, N, n_out, bias, fp16 rows): the first call, then a smaller one
PAIRS = [
    ("decode_then_m1", (8, 4096, 16384, 4, False, True), (1, 512, 1000, 1, True, True)),
    ("stream_then_fused", (40, 8192, 700, 5, True, False), (16, 1024, 300, 2, False, True)),
    ("gemm_then_stream", (300, 1040, 520, 6, True, True), (24, 1040, 520, 3, False, False)),
    # with its split-K partials the workspace (70 MB) exceeds the scratch: the
    # static call computes every tile whole, the same exact integers
    ("gemm_unsplit_then_gemm", (512, 4096, 16384, 3, False, True), (80, 2048, 1300, 2, True, True)),
]


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: p[0])
def test_static_scratch_matches_workspace_entry(lib, pair):
    name, first, second = pair
    for i, (M, K, N, n_out, bias, pass_w) in enumerate((first, second)):
        say(f"int8_linear_static {name} call {i + 1}: M={M} K={K} N={N} n_out={n_out}")
        X, Wq, sw, W, b = layer(lib, M, K, N, 100 * i + M, n_out, bias, pass_w)
        ref = lib.linear(X, Wq, sw, W, 6.0, bias=b)
        out = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda:0")
        y = lib.linear_static(X, Wq, sw, W, 6.0, out=out, bias=b)
        assert y.data_ptr() == out.data_ptr()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y.cpu().numpy().view(np.uint16),
                                      ref.cpu().numpy().view(np.uint16), err_msg=f"{name} {i}")


def test_static_scratch_rejects_large_shapes(lib):
    """A workspace that does not fit the scratch even without split-K partials
    is refused on the host, with nothing enqueued and a message naming the
    sizes."""
    say("int8_linear_static rejects a shape beyond the scratch")
    M, K, N = 4096, 4096, 256          # 3 * M * K = 48 MB of codes and outlier values
    assert lib.workspace_layout(M, K, N)["total"] > lib.STATIC_SCRATCH_BYTES
    X = torch.zeros((M, K), dtype=torch.float16, device="cuda:0")
    Wq = torch.zeros((N, K), dtype=torch.int8, device="cuda:0")
    sw = torch.ones((N,), dtype=torch.float32, device="cuda:0")
    out = torch.full((M, N), 7.0, dtype=torch.float16, device="cuda:0")
    with pytest.raises(lib.Int8LinError, match="WORKSPACE.*static scratch"):
        lib.linear_static(X, Wq, sw, None, 6.0, out=out)
    torch.cuda.synchronize()
    assert (out == 7.0).all().item()   # nothing ran
