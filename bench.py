#!/usr/bin/env python3
"""Throughput of the LLM.int8() linear layer on one MI355X.

One step = one int8_linear call (outlier scan, row quantization, int8 GEMM,
outlier fp16 product, dequantize + add) on synthetic seeded inputs already
resident in HBM; the weight is quantized once, untimed, as the layer does when
it is placed on the GPU.  Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload mlp_down_prefill]
    python bench.py --copy-calibration 512   # plain 512 MiB device copy only

The default (headline) workload is the largest single-GPU configuration, the
BLOOM-176B MLP down-projection prefill: X 4096x57344 . W 57344x14336 with 16
outlier columns, bound by the int8 matrix cores.  The same line carries, under
"decode", the decode configuration X 8x4096 . W 4096x16384 with 4 outlier
columns (bound by HBM), timed the same way in the same process
(--no-decode skips it).

Under "train" it also carries one step of the mixed int8/fp16 training mode
on the headline layer (re-quantize the fp16 weight, the forward, the
gradients dX, dW and dbias), whose fp16 GEMMs are priced against the fp16
matrix-core peak (--no-train skips it).

The K timed steps are captured into one HIP graph and replayed (--no-graph
launches each step from Python instead).  `value` is the whole call's rate;
`roofline` prices the call's dominant kernel: for the GEMM paths, the call's
time less that of its activation stage, which is timed alone (the same
kernels, in a graph of its own, on the same inputs).  To keep the 256 MB Infinity Cache
from serving the weight, steps rotate over several copies of (X, Wq, sw, W, Y,
workspace) totalling more than 512 MB.

--copy-calibration runs nothing but torch's device-to-device copy of a buffer
of known size; under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE it gives the
factor that turns those counters into bytes.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published peaks.
PEAK_HBM_GBS = 8000.0
PEAK_INT8_TOPS = 5000.0

# Secondary (decode) measurement: a step is ~17 us, so it is timed over more
# steps than the headline.
DECODE_STEPS, DECODE_WARMUP = 200, 20

# HBM traffic per call of the priced kernel (the GEMM's three launches; the
# fused decode kernel's one) from rocprofv3 FETCH_SIZE / WRITE_SIZE counter
# runs, scaled by the copy-kernel calibration factor
# (profiles/traffic-mlp_down_prefill_and_decode.md); valid only for the kernel
# sources it was measured on (sha256 of the listed files).
TRAFFIC = {
    ("gemm_i8_kernel", "mlp_down_prefill"): {"bytes": 5555191473, "src": "16060831513ff7ee"},
    ("decode_kernel", "decode"): {"bytes": 68483640, "src": "0cc9611719cb8aeb"},
}


def kernel_source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "mixed_precision_quantized_int8_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w):
    """Bytes the method must move once: X, Wq, the outlier weight rows, Y, scales."""
    return (2 * w.M * w.K + w.N * w.K + 2 * w.n_out * w.N + 2 * w.M * w.N
            + 4 * w.N + 4 * w.M + 4 * w.n_out)


def dominant_kernel(w):
    """The kernel that carries the call: the fused small-M kernel (M <= 16,
    K <= 4096), the streaming kernel (M <= 64 otherwise), the skinny GEMM
    (M <= 256) or the GEMM."""
    if w.M <= 64:
        name = "decode_kernel" if w.M <= 16 and w.K <= 4096 else "decode_stream_kernel"
        return name, "hbm", ["decode.hip", "common.h"]
    if w.M <= 256:
        return "gemm_skinny_kernel", "mfma", ["skinny.hip", "act.hip", "common.h"]
    return "gemm_i8_kernel", "mfma", ["gemm.hip", "act.hip", "common.h"]


def blas_threads():
    """Threads the host BLAS (which carries the oracle's matrix products) uses."""
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        return max((i.get("num_threads") or 0) for i in info) if info else None
    except Exception:
        return None


def cpu_baseline(w, X, W, budget_s=12.0):
    """Time the CPU oracle (as it stands) on a bounded sample of the workload.

    Small workloads (M*N*K <= 2^31) run whole.  Larger ones: the first 64 rows
    of X against the first 2048 output columns of the weight (every row of X
    carries the same injected outlier columns, so the sample's outlier set is
    the workload's); the rate is scaled by the sample's share of the ops."""
    import numpy as np
    from oracle import int8_oracle as O

    threads = blas_threads()
    whole = w.M * w.N * w.K <= 2**31
    rows = w.M if whole else min(w.M, 64)
    cols = w.N if whole else min(w.N, 2048)
    Ws = W if cols == w.N else np.ascontiguousarray(W[:, :cols])
    Wq, sw = O.quantize_weight(Ws)            # untimed, as on the GPU side
    Xs = X[:rows]
    reps, t_total, out = 0, 0.0, None
    t0 = time.perf_counter()
    while reps < 100 and (time.perf_counter() - t0) < budget_s:
        s = time.perf_counter()
        out = O.int8_linear(Xs, Wq, sw, Ws, w.threshold)
        t_total += time.perf_counter() - s
        reps += 1
    per_call = t_total / reps
    what = (f"full {w.name} call ({w.M}x{w.K}x{w.N})" if whole else
            f"first {rows} rows x first {cols} output columns of the {w.name} call "
            f"({rows}x{w.K}x{cols}), rate scaled by the op share")
    return {
        "value": round(2.0 * rows * cols * w.K / per_call / 1e12, 6),
        "unit": "TOPS",
        "cores": threads or os.cpu_count(),
        "kind": "oracle",
        "sample": f"{what}, weight pre-quantized, {reps} calls, {per_call * 1e3:.1f} ms/call; "
                  f"host has {os.cpu_count()} cpus",
    }, out, Wq, rows, cols


def copy_ceiling(torch, dev, mib=1024, reps=10):
    """Device-to-device copy rate (bytes read + written per second) of torch's copy kernel."""
    src = torch.empty((mib << 20,), dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = None
    for _ in range(reps):
        a.record()
        dst.copy_(src)
        b.record()
        b.synchronize()
        ms = a.elapsed_time(b)
        best = ms if best is None else min(best, ms)
    del src, dst
    return 2 * (mib << 20) / (best * 1e-3) / 1e9


def fp16_context(torch, w, sets, int8_ms, reps):
    """Context only, not part of the library: the plain fp16 product X.W at the
    same shape through torch.matmul (the vendor BLAS), over the same rotated
    buffer sets, timed with events around `reps` back-to-back calls."""
    out = torch.empty((w.M, w.N), dtype=torch.float16, device=sets[0][0].device)
    R = len(sets)
    for i in range(3):
        torch.matmul(sets[i % R][0], sets[i % R][3], out=out)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(reps):
        torch.matmul(sets[i % R][0], sets[i % R][3], out=out)
    b.record()
    b.synchronize()
    ms = a.elapsed_time(b) / reps
    del out
    return {"op": "torch.matmul fp16 X.W (vendor BLAS), eager launches, same buffer sets",
            "ms_per_call": round(ms, 5),
            "tflops": round(2.0 * w.M * w.N * w.K / (ms * 1e-3) / 1e12, 2),
            "int8_layer_speedup": round(ms / int8_ms, 3)}


def copy_calibration(mib):
    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    src = torch.empty((mib << 20,), dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": mib << 20,
                      "copy_calibration_bytes_written": mib << 20, "launches": 3}))


def time_steps(torch, step, K, graph, eager=True):
    """Time exactly K steps: captured once into a HIP graph and replayed
    (events around the replay), or launched eagerly with events per step.
    Returns (ms per step, eager ms per step or None, per-step ms array or None);
    eager=False skips the reference eager timing after a graph replay."""
    import numpy as np
    if graph:
        # The K steps are captured once into a HIP graph and replayed: the
        # kernels then run back to back, as in a serving loop, instead of
        # waiting on the Python launch path.  The graph holds no memset nodes
        # (the library clears its flags with a fill kernel).
        s_cap = torch.cuda.Stream()
        s_cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s_cap):
            for i in range(3):
                step(i)
        torch.cuda.current_stream().wait_stream(s_cap)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(K):
                step(i)
        g.replay()   # untimed first replay
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        g.replay()
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / K
        if not eager:
            del g
            return ms, None, None
        # eager launches, for reference (Python launch path included)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(K):
            step(i)
        e1.record()
        torch.cuda.synchronize()
        del g
        return ms, e0.elapsed_time(e1) / K, None
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(K):
        starts[i].record()
        step(i)
        ends[i].record()
    t1.record()
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])
    return t0.elapsed_time(t1) / K, None, per


def measure(torch, pkg, workloads, w, args, steps, warmup, with_fp16_context):
    """Set up one workload's rotated buffer sets, warm up, time `steps` steps.

    Returns (result dict, X, W, the first set's Y and Wq) -- the caller checks
    parity on them and frees them."""
    import numpy as np

    dev = torch.device("cuda:0")
    X, W, _ = workloads.make_inputs(w)
    Xd = torch.from_numpy(X).to(dev)
    Wd = torch.from_numpy(W).to(dev)
    Wq, sw = pkg.quantize_weight(Wd)
    ws_bytes = pkg.workspace_bytes(w.M, w.K, w.N)
    # bytes a step streams: X, Wq, Y (the fp16 weight is only read at outlier rows)
    set_bytes = Xd.numel() * 2 + Wq.numel() + 2 * w.M * w.N
    R = args.rotate or max(1, min(16, -(-512 * 2**20 // set_bytes)))
    sets = []
    for r in range(R):
        s = (Xd, Wq, sw, Wd) if r == 0 else (Xd.clone(), Wq.clone(), sw.clone(), Wd.clone())
        ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)
        Y = torch.empty((w.M, w.N), dtype=torch.float16, device=dev)
        S = pkg.weight_code_sums(s[1]) if args.zero_point else None   # once per layer
        sets.append((*s, ws, Y, S))
    bias_t = (torch.randn(w.N, device=dev) * 0.1).half() if args.bias else None

    def step(i):
        x, q, s, wf, ws, y, S = sets[i % R]
        rows = None if args.rebuilt_rows else wf
        if args.zero_point:
            pkg.linear_zp(x, q, s, S, rows, w.threshold, workspace=ws, out=y, bias=bias_t)
        else:
            pkg.linear(x, q, s, rows, w.threshold, workspace=ws, out=y, bias=bias_t)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ms, eager_ms, per = time_steps(torch, step, steps, not args.no_graph)

    kname, bound, files = dominant_kernel(w)
    src_hash = kernel_source_hash(files)
    if bound == "hbm":
        alg = algorithmic_bytes(w)
        achieved = alg / (ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
        # one call is exactly one launch of the fused kernel
        launch = ("one launch of decode_kernel per call" if kname == "decode_kernel" else
                  "activation kernels + decode_stream_kernel per call")
    else:
        # The GEMM's own launches: the call's time less that of its activation
        # stage (flag clear, column scan, row quantization), which runs the very
        # same kernels when timed alone, in a graph of its own, on the same
        # rotated inputs and workspaces.
        act_ms = activation_ms(torch, pkg, w, sets, R, steps, args)
        kernel_ms = ms - act_ms
        achieved = w.int_ops / (kernel_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_INT8_TOPS,
                "unit": "TOPS", "frac": round(achieved / PEAK_INT8_TOPS, 4),
                "kernel_ms": round(kernel_ms, 5), "activation_ms": round(act_ms, 5)}
        if kname == "gemm_skinny_kernel":
            launch = ("gemm_skinny_kernel (one launch per call): the call's time less its "
                      "activation stage timed alone")
        else:
            launch = ("gemm_i8_kernel whole tiles, split-K tail and fix-up: the call's time "
                      "less its activation stage (flag clear, rowpass_kernel, rowfix_kernel, "
                      "for both code types; decomposition off: colflags_kernel, "
                      "rowquant_kernel) timed alone")
    # counter figures were taken on the default layer (fp16 outlier rows, absmax codes)
    tr = None if (args.zero_point or args.rebuilt_rows or args.bias) else TRAFFIC.get((kname, w.name))
    roof["traffic"] = tr["bytes"] if tr and tr["src"] == src_hash else None
    roof["kernel"] = kname
    roof["timed"] = launch
    roof["step_ms"] = round(ms, 5)
    if per is not None:
        roof["step_ms_p10_p50_p90"] = [round(float(np.percentile(per, q)), 5) for q in (10, 50, 90)]
    roof["kernel_src"] = src_hash

    res = {
        "value": round(w.int_ops / (ms * 1e-3) / 1e12, 3),
        "unit": "TOPS",
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 5),
        "config": {"workload": w.name, "M": w.M, "K": w.K, "N": w.N,
                   "outlier_columns": w.n_out, "threshold": w.threshold,
                   "buffer_sets": R, "x_dtype": "fp16", "y_dtype": "fp16",
                   "outlier_rows": "rebuilt from codes" if args.rebuilt_rows else "fp16 weight",
                   "bias": bool(args.bias),
                   "activation_codes": "zero-point" if args.zero_point else "absmax",
                   "ops_int8": 2 * w.M * w.N * (w.K - w.n_out),
                   "ops_fp16": 2 * w.M * w.N * w.n_out,
                   "algorithmic_bytes": algorithmic_bytes(w),
                   "launch": "eager" if args.no_graph else "hip_graph"},
        "roofline": roof,
    }
    if eager_ms is not None:
        res["eager_ms_per_step"] = round(eager_ms, 5)
    if with_fp16_context:
        res["fp16_context"] = fp16_context(torch, w, sets, ms, min(steps, 50))
    Y0, Wq0 = sets[0][5], sets[0][1]
    del sets, Xd, Wd
    return res, X, W, Y0, Wq0


def activation_ms(torch, pkg, w, sets, R, K, args):
    """Per-call time of the layer's activation stage alone (the kernels the call
    runs before its GEMM), K calls over the same rotated buffer sets captured
    into one HIP graph; the outputs go to buffers allocated once."""
    import numpy as np
    x0, ws0 = sets[0][0], sets[0][4]
    if args.zero_point:
        out = pkg.quantize_activation_zp(x0, w.threshold, workspace=ws0)
        fn = lambda x, ws: pkg.quantize_activation_zp(x, w.threshold, workspace=ws, out=out)
    else:
        out = pkg.quantize_activation(x0, w.threshold, workspace=ws0)
        fn = lambda x, ws: pkg.quantize_activation(x, w.threshold, workspace=ws, out=out)
    ms, _, _ = time_steps(torch, lambda i: fn(sets[i % R][0], sets[i % R][4]), K,
                          not args.no_graph, eager=False)
    del out
    return ms


def graph_ms(torch, fn, K):
    """Per-call time of `fn` captured K times into one HIP graph and replayed
    (events around the replay, after an untimed replay)."""
    s_cap = torch.cuda.Stream()
    s_cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s_cap):
        fn()
    torch.cuda.current_stream().wait_stream(s_cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(K):
            fn()
    g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    g.replay()
    t1.record()
    torch.cuda.synchronize()
    del g
    return t0.elapsed_time(t1) / K


PEAK_FP16_TFLOPS = 2500.0


def measure_train(torch, pkg, w, X, W, steps, warmup, with_cpu):
    """One step of the mixed int8/fp16 training mode on the workload's layer,
    the fp16 weight being the trained parameter: re-quantize it, the int8
    forward with its fp16 rows for the outlier columns and a bias, then the
    gradients dX = dY W^T, dW = X^T dY and dbias.  Each part is also timed on
    its own (one graph per part)."""
    import numpy as np

    dev = torch.device("cuda:0")
    rng = np.random.default_rng(1000 + w.seed)
    dY = rng.standard_normal((w.M, w.N), dtype=np.float32).astype(np.float16)
    bias = (rng.standard_normal(w.N) * 0.1).astype(np.float16)
    Xd, Wd = torch.from_numpy(X).to(dev), torch.from_numpy(W).to(dev)
    dYd, bd = torch.from_numpy(dY).to(dev), torch.from_numpy(bias).to(dev)
    Wq = torch.empty((w.N, w.K), dtype=torch.int8, device=dev)
    sw = torch.empty((w.N,), dtype=torch.float32, device=dev)
    Y = torch.empty((w.M, w.N), dtype=torch.float16, device=dev)
    dX = torch.empty((w.M, w.K), dtype=torch.float16, device=dev)
    ws = pkg.new_workspace(w.M, w.K, w.N, dev)
    nbw = int(pkg.lib().i8l_backward_weight_workspace_bytes(w.M, w.K, w.N))
    wsb = torch.empty((nbw,), dtype=torch.uint8, device=dev)

    def forward():
        pkg.quantize_weight(Wd, Wq, sw)
        pkg.linear(Xd, Wq, sw, Wd, w.threshold, workspace=ws, out=Y, bias=bd)

    def back_in():
        pkg.backward_input(dYd, Wd, out=dX)

    def back_w():
        return pkg.backward_weight(Xd, dYd, with_bias=True, workspace=wsb)

    def step():
        forward()
        back_in()
        back_w()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ms = {"step": graph_ms(torch, step, steps), "forward": graph_ms(torch, forward, steps),
          "backward_input": graph_ms(torch, back_in, steps),
          "backward_weight": graph_ms(torch, back_w, steps)}
    mnk2 = 2.0 * w.M * w.N * w.K
    back_ms = ms["backward_input"] + ms["backward_weight"]
    achieved = 2 * mnk2 / (back_ms * 1e-3) / 1e12
    res = {
        "value": round(3 * mnk2 / (ms["step"] * 1e-3) / 1e12, 3),
        "unit": "TOPS (2MNK int8 forward + 4MNK fp16 backward per step)",
        "ms_per_step": round(ms["step"], 5),
        "steps": steps,
        "config": {"workload": w.name, "M": w.M, "K": w.K, "N": w.N, "bias": True,
                   "weight": "fp16 parameter, re-quantized every step",
                   "step": "quantize_weight, linear, backward_input, backward_weight (+bias)"},
        "parts_ms": {k: round(v, 5) for k, v in ms.items() if k != "step"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_FP16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP16_TFLOPS, 4),
                     "traffic": None, "kernel": "gemm_i8_kernel (fp16 instantiation)",
                     "timed": "backward_input + backward_weight: the two fp16 GEMMs, the "
                              "two transposes and the bias sum",
                     "backward_input_frac": round(mnk2 / (ms["backward_input"] * 1e-3) / 1e12
                                                  / PEAK_FP16_TFLOPS, 4),
                     "backward_weight_frac": round(mnk2 / (ms["backward_weight"] * 1e-3) / 1e12
                                                   / PEAK_FP16_TFLOPS, 4)},
    }
    if with_cpu:
        res["cpu_baseline"] = cpu_baseline_train(w, X, W, dY, bias)
    del Xd, Wd, dYd, Wq, Y, dX, ws, wsb
    torch.cuda.empty_cache()
    return res


def cpu_baseline_train(w, X, W, dY, bias, budget_s=10.0):
    """The oracle's training step (forward with fresh codes, the three
    gradients) on a bounded sample: the first 64 rows and the first 2048
    output features of the layer; the rate is scaled by the op share."""
    from oracle import int8_oracle as O
    import numpy as np

    rows, cols = min(w.M, 64), min(w.N, 2048)
    Xs = X[:rows]
    Ws = np.ascontiguousarray(W[:, :cols])
    dYs = np.ascontiguousarray(dY[:rows, :cols])
    reps, t_total = 0, 0.0
    t0 = time.perf_counter()
    while reps < 100 and (time.perf_counter() - t0) < budget_s:
        s = time.perf_counter()
        O.train_forward(Xs, Ws, w.threshold, bias=bias[:cols])
        O.linear_backward_input(dYs, Ws)
        O.linear_backward_weight(Xs, dYs)
        O.linear_backward_bias(dYs)
        t_total += time.perf_counter() - s
        reps += 1
    per = t_total / reps
    return {"value": round(3 * 2.0 * rows * cols * w.K / per / 1e12, 6), "unit": "TOPS",
            "cores": blas_threads() or os.cpu_count(), "kind": "oracle",
            "sample": f"first {rows} rows x first {cols} output features of the {w.name} "
                      f"layer ({rows}x{w.K}x{cols}), {reps} steps, {per * 1e3:.1f} ms/step"}


def parity_of(w, y_dev, wq_dev, ref, Wq_o, rows, cols):
    """The benchmark's own output against the oracle on the sampled block."""
    import numpy as np
    y = y_dev[:rows, :cols].cpu().numpy().astype(np.float64)
    err = np.abs(y - ref["Y64"])
    tol = np.maximum(2e-3 * np.abs(ref["Y64"]), 1e-2)
    return {"checked": f"Y[:{rows}, :{cols}], Wq[:{cols}]",
            "Y_within_tol": bool(np.all(err <= tol)),
            "Wq_bitexact": bool(np.array_equal(wq_dev[:cols].cpu().numpy(), Wq_o)),
            "max_abs_err": float(err.max())}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mlp_down_prefill")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the secondary decode measurement")
    ap.add_argument("--no-train", action="store_true",
                    help="skip the training-mode step (fp16 weight, backward pass)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rotate", type=int, default=0, help="buffer sets (0: auto, >512 MB)")
    ap.add_argument("--rebuilt-rows", action="store_true",
                    help="keep no fp16 weight: outlier rows rebuilt from the codes")
    ap.add_argument("--bias", action="store_true", help="add an fp16 bias [N]")
    ap.add_argument("--zero-point", action="store_true",
                    help="zero-point (unsigned) activation codes: int8_linear_zp")
    ap.add_argument("--no-fp16-context", action="store_true",
                    help="skip timing torch.matmul in fp16 at the same shape")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch every step from Python instead of replaying a captured graph")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-MiB buffer three times (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one MI355X: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import torch

    import mixed_precision_quantized_int8_amd as pkg
    from mixed_precision_quantized_int8_amd import _binding, workloads

    if not os.path.exists(_binding.LIB_PATH):
        from mixed_precision_quantized_int8_amd import build
        build.build_library()

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = workloads.WORKLOADS[args.workload]
    res, X, W, Y0, Wq0 = measure(torch, pkg, workloads, w, args, args.steps, args.warmup,
                                 not args.no_fp16_context)
    result = {
        "metric": "int8_linear TOPS and % of int8-MFMA / HBM roofline on one MI355X",
        "value": res["value"],
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": res["config"],
        "roofline": res["roofline"],
    }
    for k in ("eager_ms_per_step", "fp16_context"):
        if k in res:
            result[k] = res[k]
    result["roofline"]["measured_copy_GBs"] = round(copy_ceiling(torch, dev), 1)

    default_layer = not (args.rebuilt_rows or args.bias or args.zero_point)
    if not args.no_cpu_baseline:
        if not default_layer:
            raise SystemExit("the CPU baseline and parity check cover the default layer only "
                             "(run with --no-cpu-baseline)")
        cb, ref, Wq_o, rows, cols = cpu_baseline(w, X, W)
        result["cpu_baseline"] = cb
        result["parity"] = parity_of(w, Y0, Wq0, ref, Wq_o, rows, cols)
    del Y0, Wq0
    torch.cuda.empty_cache()
    if not args.no_train and default_layer:
        result["train"] = measure_train(torch, pkg, w, X, W, args.steps, args.warmup,
                                        not args.no_cpu_baseline)
    del X, W

    if not args.no_decode and w.name != "decode":
        wd = workloads.WORKLOADS["decode"]
        dres, *_ = measure(torch, pkg, workloads, wd, args, DECODE_STEPS, DECODE_WARMUP,
                           not args.no_fp16_context)
        result["decode"] = dres
    print(json.dumps(result))


if __name__ == "__main__":
    main()
