"""Int8Linear / replace_linear (the nn.Linear replacement) against the CPU oracle."""
import zlib

import numpy as np
import pytest
import torch

import mixed_precision_quantized_int8_amd.workloads as wl
from oracle import int8_oracle as O

from test_parity_gpu import assert_y, host, lib, say  # noqa: F401  (fixture and helpers)


@pytest.mark.gpu
@pytest.mark.parametrize("name,lead,K,N,n_out,fp16w", [
    ("decode", (2, 7), 1040, 300, 2, False),        # 14 rows: fused decode kernel
    ("decode_fp16w", (3, 5), 1024, 520, 3, True),
    ("prefill", (4, 75), 1040, 520, 5, False),      # 300 rows: GEMM
    ("prefill_fp16w", (300,), 512, 300, 4, True),
    ("bigk", (8,), 16384, 256, 3, False),           # streaming decode kernel
])
def test_int8linear_matches_oracle(lib, name, lead, K, N, n_out, fp16w):
    from mixed_precision_quantized_int8_amd.module import Int8Linear

    M = int(np.prod(lead))
    say(f"Int8Linear {name} x{lead + (K,)} -> {N} fp16 weights={fp16w}")
    X, W, _ = wl.make_small(M, K, N, seed=zlib.crc32(name.encode()) % 997, n_out=n_out,
                            x_sigma=1.0)
    rng = np.random.default_rng(3)
    b = (rng.standard_normal(N) * 0.5).astype(np.float16)
    lin = torch.nn.Linear(K, N, bias=True)
    with torch.no_grad():
        lin.weight.copy_(torch.from_numpy(W.T.astype(np.float32)))   # nn.Linear: [out][in]
        lin.bias.copy_(torch.from_numpy(b.astype(np.float32)))
    m = Int8Linear.from_linear(lin, has_fp16_weights=fp16w, threshold=6.0, device="cuda:0")
    x = torch.from_numpy(X).to("cuda:0").reshape(*lead, K)
    y = m(x)
    torch.cuda.synchronize()
    assert y.shape == (*lead, N) and y.dtype == torch.float16
    Wq_o, sw_o = O.quantize_weight(W)
    np.testing.assert_array_equal(host(m.Wq), Wq_o)
    W_out = W if fp16w else O.dequantize_weight(Wq_o, sw_o)
    r = O.int8_linear(X, Wq_o, sw_o, W_out, 6.0, bias=b)
    assert len(r["idx"]) == n_out
    assert_y(host(y.detach().reshape(M, N)), r["Y64"], r["Y"], name)


@pytest.mark.gpu
def test_replace_linear_and_state_dict(lib):
    from mixed_precision_quantized_int8_amd.module import Int8Linear, replace_linear

    say("replace_linear on a small model; state dict round trip")
    torch.manual_seed(0)

    class Block(torch.nn.Module):
        def __init__(self):
            super().__init__()
            self.up = torch.nn.Linear(256, 512)
            self.down = torch.nn.Linear(512, 256, bias=False)

        def forward(self, x):
            return self.down(torch.nn.functional.gelu(self.up(x)))

    class Model(torch.nn.Module):
        def __init__(self):
            super().__init__()
            self.blocks = torch.nn.ModuleList([Block(), Block()])
            self.lm_head = torch.nn.Linear(256, 1000, bias=False)

        def forward(self, x):
            for blk in self.blocks:
                x = x + blk(x)
            return self.lm_head(x)

    model = Model().half().to("cuda:0")
    replace_linear(model, has_fp16_weights=False, threshold=6.0)
    assert isinstance(model.blocks[0].up, Int8Linear) and isinstance(model.blocks[1].down, Int8Linear)
    assert model.blocks[0].up.bias is not None and model.blocks[1].down.bias is None
    assert type(model.lm_head) is torch.nn.Linear                  # kept in full precision
    x = (torch.randn(4, 9, 256, device="cuda:0") * 0.5).half()
    x[..., 17] = 12.0                                              # an outlier column
    y = model(x)
    assert y.shape == (4, 9, 1000) and torch.isfinite(y).all()
    # state dict: codes, scales, bias; a fresh layer loaded from it computes the same
    up = model.blocks[0].up
    sd = up.state_dict()
    assert set(sd) == {"Wq", "sw", "bias"}
    fresh = Int8Linear(256, 512, bias=True, device="cuda:0")
    fresh.load_state_dict(sd)
    a = up(x)
    b = fresh(x)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(a).view(np.uint16), host(b).view(np.uint16))
