"""LLM.int8() quantized linear layer for AMD MI355X (gfx950).

Python face of the C ABI in include/int8lin.h: same operation names, torch
tensors in and out.  Marshalling only -- every step runs in the HIP kernels of
libint8lin.so; torch supplies device memory and the current stream.

    Wq, sw = quantize_weight(W)              # W fp16 [K][N] (Y = X @ W)
    Y = linear(X, Wq, sw, W, threshold=6.0)  # X fp16 [M][K] -> Y fp16 [M][N]
"""
from __future__ import annotations

from ._binding import (  # noqa: F401
    EXPORTS,
    Int8LinError,
    MAX_K,
    MAX_K_ZP,
    STATIC_SCRATCH_BYTES,
    build_info,
    check,
    last_error,
    lib,
    workspace_bytes,
    workspace_layout,
)

__all__ = [
    "quantize_weight",
    "linear",
    "linear_static",
    "quantize_activation",
    "gemm_i32",
    "weight_code_sums",
    "linear_zp",
    "quantize_activation_zp",
    "backward_input",
    "backward_weight",
    "workspace_layout",
    "workspace_bytes",
    "workspace_views",
    "Int8LinError",
    "build_info",
]


def _torch():
    import torch

    return torch


def _stream(t):
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def _require(t, dtype, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def quantize_weight(W, Wq=None, sw=None):
    """W fp16 [K][N] -> (Wq int8 [N][K], sw fp32 [N]); column-wise absmax codes."""
    torch = _torch()
    _require(W, torch.float16, "W")
    K, N = W.shape
    if Wq is None:
        Wq = torch.empty((N, K), dtype=torch.int8, device=W.device)
    if sw is None:
        sw = torch.empty((N,), dtype=torch.float32, device=W.device)
    with torch.cuda.device(W.device):
        check(lib().int8_quantize_weight(W.data_ptr(), K, N, Wq.data_ptr(), sw.data_ptr(),
                                         _stream(W)))
    return Wq, sw


def new_workspace(M, K, N, device):
    torch = _torch()
    return torch.empty((max(workspace_bytes(M, K, N), 1),), dtype=torch.uint8, device=device)


def _linear_args(X, Wq, sw, W, bias, workspace, out, need_workspace=True):
    torch = _torch()
    _require(X, torch.float16, "X")
    _require(Wq, torch.int8, "Wq")
    _require(sw, torch.float32, "sw")
    M, K = X.shape
    N = Wq.shape[0]
    if Wq.shape[1] != K or sw.shape != (N,):
        raise ValueError(f"shape mismatch: X {tuple(X.shape)}, Wq {tuple(Wq.shape)}, sw {tuple(sw.shape)}")
    if W is not None:
        _require(W, torch.float16, "W")
        if tuple(W.shape) != (K, N):
            raise ValueError(f"W must be [K][N] = [{K}][{N}], got {tuple(W.shape)}")
    if bias is not None:
        _require(bias, torch.float16, "bias")
        if tuple(bias.shape) != (N,):
            raise ValueError(f"bias must be [{N}], got {tuple(bias.shape)}")
    if not need_workspace:
        workspace = None
    elif workspace is None:
        workspace = new_workspace(M, K, N, X.device)
    else:
        _require(workspace, torch.uint8, "workspace")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=X.device)
    else:
        _require(out, torch.float16, "out")
        if tuple(out.shape) != (M, N):
            raise ValueError(f"out must be [{M}][{N}], got {tuple(out.shape)}")
    return M, K, N, workspace, out


def linear(X, Wq, sw, W=None, threshold=6.0, workspace=None, out=None, bias=None):
    """LLM.int8() linear layer: X fp16 [M][K] -> Y fp16 [M][N].

    W (fp16 [K][N]) supplies the weight rows of the outlier columns.  With
    W None no fp16 weight is kept: those rows are rebuilt from the codes as
    fp16(Wq[n][k] * sw[n] / 127).  ``bias`` (fp16 [N]) is added before the
    final rounding.
    """
    torch = _torch()
    M, K, N, workspace, out = _linear_args(X, Wq, sw, W, bias, workspace, out)
    with torch.cuda.device(X.device):
        check(lib().int8_linear_bias(
            X.data_ptr(), M, K, Wq.data_ptr(), sw.data_ptr(), N,
            W.data_ptr() if W is not None else None,
            bias.data_ptr() if bias is not None else None, float(threshold),
            out.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(X)))
    return out


def linear_static(X, Wq, sw, W=None, threshold=6.0, out=None, bias=None):
    """``linear`` without a workspace: the intermediates go to the library's
    static scratch array on the current GPU (``STATIC_SCRATCH_BYTES``), so the
    call allocates nothing when ``out`` is given.  Calls that overlap on one
    GPU race on that array; shapes whose workspace does not fit it raise."""
    torch = _torch()
    M, K, N, _, out = _linear_args(X, Wq, sw, W, bias, None, out, need_workspace=False)
    with torch.cuda.device(X.device):
        check(lib().int8_linear_static(
            X.data_ptr(), M, K, Wq.data_ptr(), sw.data_ptr(), N,
            W.data_ptr() if W is not None else None,
            bias.data_ptr() if bias is not None else None, float(threshold),
            out.data_ptr(), _stream(X)))
    return out


def weight_code_sums(Wq, out=None):
    """Wq int8 [N][K] -> S int32 [N], S[n] = sum_k Wq[n][k] (zero-point variant)."""
    torch = _torch()
    _require(Wq, torch.int8, "Wq")
    N, K = Wq.shape
    if out is None:
        out = torch.empty((N,), dtype=torch.int32, device=Wq.device)
    with torch.cuda.device(Wq.device):
        check(lib().int8_weight_code_sums(Wq.data_ptr(), N, K, out.data_ptr(), _stream(Wq)))
    return out


def linear_zp(X, Wq, sw, wsum, W=None, threshold=6.0, workspace=None, out=None, bias=None):
    """The layer with zero-point (unsigned) activation codes per row of X; the
    weight keeps its absmax codes.  ``wsum`` comes from ``weight_code_sums(Wq)``;
    the other arguments as for ``linear``."""
    torch = _torch()
    M, K, N, workspace, out = _linear_args(X, Wq, sw, W, bias, workspace, out)
    _require(wsum, torch.int32, "wsum")
    if tuple(wsum.shape) != (N,):
        raise ValueError(f"wsum must be [{N}], got {tuple(wsum.shape)}")
    with torch.cuda.device(X.device):
        check(lib().int8_linear_zp(
            X.data_ptr(), M, K, Wq.data_ptr(), sw.data_ptr(), wsum.data_ptr(), N,
            W.data_ptr() if W is not None else None,
            bias.data_ptr() if bias is not None else None, float(threshold),
            out.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(X)))
    return out


def workspace_views(workspace, M, K):
    """Typed views of the intermediates an int8_linear call leaves in its workspace."""
    torch = _torch()
    L = workspace_layout(M, K, 0)
    b = workspace

    def view(off, nbytes, dtype, shape):
        return b[off:off + nbytes].view(dtype).view(shape)

    return {
        "zp": view(L["zero_points"], 4 * M, torch.int32, (M,)),
        "n_out": view(L["n_outliers"], 4, torch.int32, (1,)),
        "idx": view(L["outlier_idx"], 4 * K, torch.int32, (K,)),
        "sx": view(L["sx"], 4 * M, torch.float32, (M,)),
        "Xq": view(L["Xq"], M * K, torch.int8, (M, K)),
        "X_O": view(L["X_outliers"], 2 * M * K, torch.float16, (M, K)),
    }


def _act_outputs(M, K, dev, out, zp):
    """The activation stage's output tensors: ``out``'s (checked) or new ones."""
    torch = _torch()
    spec = [("Xq", (M, K), torch.int8)]
    spec += [("zp", (M,), torch.int32), ("xscale", (M,), torch.float32)] if zp else \
        [("sx", (M,), torch.float32)]
    spec += [("idx", (K,), torch.int32), ("n_out", (1,), torch.int32),
             ("X_O", (M, K), torch.float16)]
    if out is None:
        return {name: torch.empty(shape, dtype=dt, device=dev) for name, shape, dt in spec}
    for name, shape, dt in spec:
        t = out[name]
        _require(t, dt, name)
        if tuple(t.shape) != shape or t.device != dev:
            raise ValueError(f"out[{name!r}] must be {shape} on {dev}")
    return {name: out[name] for name, _, _ in spec}


def quantize_activation(X, threshold=6.0, workspace=None, out=None):
    """Activation stage alone: dict of Xq [M][K], sx [M], idx [K] (first n_out
    valid), n_out [1], X_O [M][K] (first n_out columns valid).  ``out``: a dict
    of such tensors from an earlier call, written again instead of new ones."""
    torch = _torch()
    _require(X, torch.float16, "X")
    M, K = X.shape
    dev = X.device
    o = _act_outputs(M, K, dev, out, zp=False)
    Xq, sx, idx, n_out, X_O = o["Xq"], o["sx"], o["idx"], o["n_out"], o["X_O"]
    if workspace is None:
        workspace = new_workspace(M, K, 0, dev)
    else:
        _require(workspace, torch.uint8, "workspace")
    with torch.cuda.device(dev):
        check(lib().int8_quantize_activation(
            X.data_ptr(), M, K, float(threshold), Xq.data_ptr(), sx.data_ptr(), idx.data_ptr(),
            n_out.data_ptr(), X_O.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(X)))
    return {"Xq": Xq, "sx": sx, "idx": idx, "n_out": n_out, "X_O": X_O}


def quantize_activation_zp(X, threshold=6.0, workspace=None, out=None):
    """Zero-point activation stage alone: dict of Xq [M][K] (codes - 128), zp [M],
    xscale [M], idx [K] (first n_out valid), n_out [1], X_O [M][K].  ``out``: a
    dict of such tensors from an earlier call, written again instead of new ones."""
    torch = _torch()
    _require(X, torch.float16, "X")
    M, K = X.shape
    dev = X.device
    o = _act_outputs(M, K, dev, out, zp=True)
    Xq, zp, xscale, idx, n_out, X_O = (o["Xq"], o["zp"], o["xscale"], o["idx"], o["n_out"],
                                      o["X_O"])
    if workspace is None:
        workspace = new_workspace(M, K, 0, dev)
    else:
        _require(workspace, torch.uint8, "workspace")
    with torch.cuda.device(dev):
        check(lib().int8_quantize_activation_zp(
            X.data_ptr(), M, K, float(threshold), Xq.data_ptr(), zp.data_ptr(), xscale.data_ptr(),
            idx.data_ptr(), n_out.data_ptr(), X_O.data_ptr(), workspace.data_ptr(),
            workspace.numel(), _stream(X)))
    return {"Xq": Xq, "zp": zp, "xscale": xscale, "idx": idx, "n_out": n_out, "X_O": X_O}


def gemm_i32(Xq, Wq, workspace=None):
    """Exact int8 GEMM: Xq int8 [M][K], Wq int8 [N][K] -> int32 [M][N].

    With ``workspace`` (uint8, at least ``workspace_bytes(M, K, N)``) the
    output tiles of a partial last round are split along K and summed as in
    ``linear``; without it every tile is computed whole."""
    torch = _torch()
    _require(Xq, torch.int8, "Xq")
    _require(Wq, torch.int8, "Wq")
    M, K = Xq.shape
    N = Wq.shape[0]
    if Wq.shape[1] != K:
        raise ValueError("Xq and Wq must share K")
    acc = torch.empty((M, N), dtype=torch.int32, device=Xq.device)
    if workspace is not None:
        _require(workspace, torch.uint8, "workspace")
    ws_ptr, ws_bytes = (workspace.data_ptr(), workspace.numel()) if workspace is not None \
        else (None, 0)
    with torch.cuda.device(Xq.device):
        check(lib().int8_gemm_i32(Xq.data_ptr(), Wq.data_ptr(), M, N, K, acc.data_ptr(),
                                  ws_ptr, ws_bytes, _stream(Xq)))
    return acc


def backward_input(dY, W, out=None):
    """Training mode: dX = dY . W^T; dY fp16 [M][N], W fp16 [K][N] -> fp16 [M][K]."""
    torch = _torch()
    _require(dY, torch.float16, "dY")
    _require(W, torch.float16, "W")
    M, N = dY.shape
    K = W.shape[0]
    if W.shape[1] != N:
        raise ValueError(f"W must be [K][{N}], got {tuple(W.shape)}")
    if out is None:
        out = torch.empty((M, K), dtype=torch.float16, device=dY.device)
    else:
        _require(out, torch.float16, "out")
        if tuple(out.shape) != (M, K):
            raise ValueError(f"out must be [{M}][{K}], got {tuple(out.shape)}")
    with torch.cuda.device(dY.device):
        check(lib().int8_linear_backward_input(dY.data_ptr(), W.data_ptr(), M, K, N,
                                               out.data_ptr(), _stream(dY)))
    return out


def backward_weight(X, dY, with_bias=False, workspace=None):
    """Training mode: (dW = X^T . dY fp16 [K][N], dbias fp16 [N] or None)."""
    torch = _torch()
    _require(X, torch.float16, "X")
    _require(dY, torch.float16, "dY")
    M, K = X.shape
    if dY.shape[0] != M:
        raise ValueError(f"dY must have {M} rows, got {tuple(dY.shape)}")
    N = dY.shape[1]
    dW = torch.empty((K, N), dtype=torch.float16, device=X.device)
    db = torch.empty((N,), dtype=torch.float16, device=X.device) if with_bias else None
    if workspace is None:
        nbytes = int(lib().i8l_backward_weight_workspace_bytes(M, K, N))
        workspace = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=X.device)
    else:
        _require(workspace, torch.uint8, "workspace")
    with torch.cuda.device(X.device):
        check(lib().int8_linear_backward_weight(
            X.data_ptr(), dY.data_ptr(), M, K, N, dW.data_ptr(),
            db.data_ptr() if db is not None else None, workspace.data_ptr(), workspace.numel(),
            _stream(X)))
    return dW, db
