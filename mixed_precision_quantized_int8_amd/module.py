"""Drop-in replacement for torch.nn.Linear built on the LLM.int8() library.

[blog, "Usage"]: the 8-bit layer takes nn.Linear's arguments plus
``has_fp16_weights`` and ``threshold``; the weight is quantized once, when the
layer is put on the GPU, and kept as int8 codes (CB, [out][in]) with one absmax
per output feature (SCB).  Without fp16 weights the outlier rows are rebuilt
from the codes.  Every model layer except the output head is replaced
(the blog keeps ``lm_head`` in full precision).

The module only holds tensors and calls the library: quantization, the layer
itself and the bias all run in the HIP kernels.
"""
from __future__ import annotations

import torch

from . import _binding  # noqa: F401  (loads the library; fails loudly when missing)
from . import linear as _linear
from . import quantize_weight as _quantize_weight


class Int8Linear(torch.nn.Module):
    """y = LLM.int8()(x @ W) + b for fp16 x [..., in_features] on a GPU.

    Buffers (saved in the state dict): ``Wq`` int8 [out][in], ``sw`` fp32 [out],
    ``bias`` fp16 [out] (if any) and, with ``has_fp16_weights``, ``weight16``
    fp16 [in][out] (the math-layout weight whose rows serve the outlier
    columns).
    """

    def __init__(self, in_features: int, out_features: int, bias: bool = True,
                 has_fp16_weights: bool = False, threshold: float = 6.0, device=None):
        super().__init__()
        self.in_features = in_features
        self.out_features = out_features
        self.has_fp16_weights = has_fp16_weights
        self.threshold = float(threshold)
        dev = torch.device(device) if device is not None else torch.device("cuda")
        self.register_buffer("Wq", torch.zeros((out_features, in_features), dtype=torch.int8,
                                               device=dev))
        self.register_buffer("sw", torch.zeros((out_features,), dtype=torch.float32, device=dev))
        self.register_buffer("bias", torch.zeros((out_features,), dtype=torch.float16, device=dev)
                             if bias else None)
        self.register_buffer("weight16", torch.zeros((in_features, out_features),
                                                     dtype=torch.float16, device=dev)
                             if has_fp16_weights else None)

    @classmethod
    def from_linear(cls, lin: torch.nn.Linear, has_fp16_weights: bool = False,
                    threshold: float = 6.0, device=None) -> "Int8Linear":
        """Quantize an nn.Linear (its weight is [out][in]) on the GPU."""
        dev = torch.device(device) if device is not None else (
            lin.weight.device if lin.weight.is_cuda else torch.device("cuda"))
        m = cls(lin.in_features, lin.out_features, lin.bias is not None, has_fp16_weights,
                threshold, dev)
        with torch.no_grad():
            W = lin.weight.detach().to(dev, torch.float16).t().contiguous()   # [in][out]
            _quantize_weight(W, m.Wq, m.sw)
            if has_fp16_weights:
                m.weight16.copy_(W)
            if lin.bias is not None:
                m.bias.copy_(lin.bias.detach().to(dev, torch.float16))
        return m

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if x.shape[-1] != self.in_features:
            raise ValueError(f"expected last dimension {self.in_features}, got {x.shape[-1]}")
        lead = x.shape[:-1]
        x2 = x.reshape(-1, self.in_features)
        if x2.dtype != torch.float16:
            raise TypeError(f"Int8Linear takes fp16 input (got {x2.dtype})")
        if not x2.is_contiguous():
            x2 = x2.contiguous()
        y = _linear(x2, self.Wq, self.sw, self.weight16, self.threshold, bias=self.bias)
        return y.reshape(*lead, self.out_features)

    def extra_repr(self) -> str:
        return (f"in_features={self.in_features}, out_features={self.out_features}, "
                f"bias={self.bias is not None}, has_fp16_weights={self.has_fp16_weights}, "
                f"threshold={self.threshold}")


def replace_linear(model: torch.nn.Module, skip=("lm_head",), has_fp16_weights: bool = False,
                   threshold: float = 6.0, device=None) -> torch.nn.Module:
    """Swap every nn.Linear of ``model`` (recursively, in place) for an Int8Linear,
    except modules whose name is in ``skip``.  Returns ``model``."""
    for name, child in list(model.named_children()):
        if name in skip:
            continue
        if isinstance(child, torch.nn.Linear):
            setattr(model, name, Int8Linear.from_linear(child, has_fp16_weights, threshold, device))
        else:
            replace_linear(child, skip, has_fp16_weights, threshold, device)
    return model
