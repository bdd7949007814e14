#!/usr/bin/env python3
"""Benchmark of the FP8 fine-grained quantization + block-scaled GEMM hot path
on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic inputs:
  linear layer X [4096,7168] bf16, W [2048,7168] fp32, dY [4096,2048] bf16
    quant_batch[quant_weight(W, +q_t), quant_act_transpose(X)] -> Fprop Y = X W^T (bf16)
    quant_act_transpose(dY) -> Dgrad dX = dY W (bf16)
    Wgrad dW = dY^T X (fp32) on the transposed codes kept from both
  MoE layer X [16384,7168] bf16 routed to 32 experts W_e [2048,7168] fp32
    quant_act(X) -> quant_weight(W stacked) -> grouped Fprop (bf16)
The same step with every quantizer as its own launch (quant_act X, quant_weight
W, quant_act dY, quant_transpose X and dY) is timed and reported beside it.
Inputs are generated and resident in HBM before the timed region.

Reported beside the step (not part of its value): the microscaling (MXFP8)
variant of the linear layer's three products with its quantizers; the MoE
layer's backward,
dY [16384,2048] bf16 -> quant_act(dY), quant_weight(W stacked, +q_t) ->
grouped Dgrad (bf16); grouped quant_transpose(X), (dY) -> grouped Wgrad
(dW [32,2048,7168] fp32), timed the same way over its own passes.

Prints one JSON line on stdout; progress goes to stderr.
"""

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 MFMA
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense BF16 MFMA (the exact-accumulation GEMMs)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ["quant_kernels.hip", "gemm_fp8.hip", "gemm_tile.h", "device_common.h",
                  "quant_mx.hip", "gemm_mx.hip"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# --launch-log: the ops in launch order, each with the number of kernels it
# launches, so that a rocprofv3 trace of the same run can be attributed to
# ops (several ops share a kernel; see profile_summary)
LAUNCHES = []
KERNELS_PER_OP = {"gemm_fprop + quant_act Y": 2, "gemm_dgrad + quant_act dX": 2}


def launch(op):
    LAUNCHES.append((op[0], KERNELS_PER_OP.get(op[0], 1)))
    op[1]()


def cdiv(a, b):
    return (a + b - 1) // b


def host_inputs():
    """The step's seeded synthetic inputs on the host (CPU tensors)."""
    import synth

    t0 = time.time()
    x, w = synth.linear_x_w()
    dy = synth.linear_dy()
    xm, wm, off = synth.moe_fprop()
    dym = synth.moe_dy()
    log(f"inputs generated in {time.time() - t0:.1f}s")
    return dict(x=x, w=w, dy=dy, xm=xm, wm=wm, off=off, dym=dym)


def build_workload(H, dev):
    g = lambda t: t.to(dev)
    return dict(x=g(H["x"]), w=g(H["w"]), dy=g(H["dy"]), xm=g(H["xm"]),
                wm=g(H["wm"]).reshape(-1, H["wm"].shape[2]), off=g(H["off"]), dym=g(H["dym"]))


def make_ops(L, dev, form="batched"):
    """The step's kernels as (name, launch, kind, algorithmic work per launch).

    form "batched" (the step): the layer input X is quantized once into its
    row and transposed codes (the transposed ones are kept for the weight
    gradient), in the same grid as the weight W; dY likewise once into both
    layouts.  form "separate": every quantizer of the path is its own launch
    (1x128 X, 128x128 W, 1x128 dY, then the two transposing quantizers for
    the weight gradient), as the path's steps are listed."""
    import torch
    import fp8_fine_grained_quant_amd as fq

    u8, f32 = torch.uint8, torch.float32
    E = 32
    M, K, N = L["x"].shape[0], L["x"].shape[1], L["w"].shape[0]
    Mm, Nm = L["xm"].shape[0], L["wm"].shape[0] // E
    e = lambda *s, dt=u8: torch.empty(*s, dtype=dt, device=dev)
    O = dict(
        xq=e(M, K), xs=e(M, K // 128, dt=f32), wq=e(N, K), wq_t=e(K, N), ws=e(N // 128, K // 128, dt=f32),
        y=e(M, N, dt=torch.bfloat16), dyq=e(M, N), dys=e(M, N // 128, dt=f32), dx=e(M, K, dt=torch.bfloat16),
        xq_t=e(K, M), xs_t=e(K, M // 128, dt=f32), dyq_t=e(N, M), dys_t=e(N, M // 128, dt=f32),
        dw=e(N, K, dt=f32),
        xmq=e(Mm, K), xms=e(Mm, K // 128, dt=f32), wmq=e(E * Nm, K), wms=e(E * Nm // 128, K // 128, dt=f32),
        ym=e(Mm, Nm, dt=torch.bfloat16),
    )
    act_bytes = lambda r, c, es: r * c * (es + 1) + r * cdiv(c, 128) * 4
    w_bytes = N * K * 6 + cdiv(N, 128) * cdiv(K, 128) * 4
    dual_bytes = lambda r, c: r * c * 4 + (r * cdiv(c, 128) + c * cdiv(r, 128)) * 4
    moe = [
        ("quant_act X_moe", lambda: fq.fp8q_quant_act_1x128(L["xm"], O["xmq"], O["xms"]), "hbm",
         act_bytes(Mm, K, 2)),
        ("quant_weight W_moe", lambda: fq.fp8q_quant_weight_128x128(L["wm"], O["wmq"], None, O["wms"]), "hbm",
         E * Nm * K * 5 + cdiv(E * Nm, 128) * cdiv(K, 128) * 4),
        ("grouped_gemm", lambda: fq.fp8q_grouped_gemm(O["xmq"], O["xms"], O["wmq"].view(E, Nm, K),
                                                      O["wms"].view(E, Nm // 128, K // 128), L["off"], O["ym"]),
         "mfma", 2.0 * Mm * Nm * K),
    ]
    if form == "batched":
        ops = [
            ("quant_batch W (+q_t) + X (rows + cols)",
             lambda: fq.fp8q_quant_batch([("weight", L["w"], O["wq"], O["wq_t"], O["ws"]),
                                          ("act_transpose", L["x"], O["xq"], O["xs"], O["xq_t"], O["xs_t"])]),
             "hbm", w_bytes + dual_bytes(M, K)),
            ("gemm_fprop", lambda: fq.fp8q_gemm_fprop(O["xq"], O["xs"], O["wq"], O["ws"], O["y"]), "mfma",
             2.0 * M * N * K),
            ("quant_act_transpose dY", lambda: fq.fp8q_quant_act_transpose(L["dy"], O["dyq"], O["dys"], O["dyq_t"],
                                                                          O["dys_t"]), "hbm", dual_bytes(M, N)),
            ("gemm_dgrad", lambda: fq.fp8q_gemm_dgrad(O["dyq"], O["dys"], O["wq_t"], O["ws"], O["dx"]), "mfma",
             2.0 * M * N * K),
            ("gemm_wgrad", lambda: fq.fp8q_gemm_wgrad(O["dyq_t"], O["dys_t"], O["xq_t"], O["xs_t"], O["dw"]),
             "mfma", 2.0 * M * N * K),
        ] + moe
        return ops, O
    ops = [
        ("quant_act X", lambda: fq.fp8q_quant_act_1x128(L["x"], O["xq"], O["xs"]), "hbm", act_bytes(M, K, 2)),
        ("quant_weight W (+q_t)", lambda: fq.fp8q_quant_weight_128x128(L["w"], O["wq"], O["wq_t"], O["ws"]),
         "hbm", N * K * 6 + cdiv(N, 128) * cdiv(K, 128) * 4),
        ("gemm_fprop", lambda: fq.fp8q_gemm_fprop(O["xq"], O["xs"], O["wq"], O["ws"], O["y"]), "mfma",
         2.0 * M * N * K),
        ("quant_act dY", lambda: fq.fp8q_quant_act_1x128(L["dy"], O["dyq"], O["dys"]), "hbm", act_bytes(M, N, 2)),
        ("gemm_dgrad", lambda: fq.fp8q_gemm_dgrad(O["dyq"], O["dys"], O["wq_t"], O["ws"], O["dx"]), "mfma",
         2.0 * M * N * K),
        ("quant_transpose X", lambda: fq.fp8q_quant_transpose(L["x"], O["xq_t"], O["xs_t"]), "hbm",
         act_bytes(M, K, 2)),
        ("quant_transpose dY", lambda: fq.fp8q_quant_transpose(L["dy"], O["dyq_t"], O["dys_t"]), "hbm",
         act_bytes(M, N, 2)),
        ("gemm_wgrad", lambda: fq.fp8q_gemm_wgrad(O["dyq_t"], O["dys_t"], O["xq_t"], O["xs_t"], O["dw"]), "mfma",
         2.0 * M * N * K),
    ] + moe
    return ops, O


def make_moe_bwd_ops(L, dev):
    """The MoE layer's backward kernels, as make_ops."""
    import torch
    import fp8_fine_grained_quant_amd as fq

    u8, f32 = torch.uint8, torch.float32
    E = 32
    Mm, K = L["xm"].shape
    Nm = L["wm"].shape[0] // E
    cap = fq.token_capacity(Mm, E)
    e = lambda *s, dt=u8: torch.empty(*s, dtype=dt, device=dev)
    B = dict(dyq=e(Mm, Nm), dys=e(Mm, Nm // 128, dt=f32), wq=e(E * Nm, K), wq_t=e(K, E * Nm),
             ws=e(E * Nm // 128, K // 128, dt=f32), dx=e(Mm, K, dt=torch.bfloat16),
             xq_t=e(K, cap), xs_t=e(K, cap // 128, dt=f32), dyq_t=e(Nm, cap), dys_t=e(Nm, cap // 128, dt=f32),
             dw=e(E, Nm, K, dt=f32))
    act_bytes = lambda r, c, es: r * c * (es + 1) + r * cdiv(c, 128) * 4
    ops = [
        ("quant_act dY_moe", lambda: fq.fp8q_quant_act_1x128(L["dym"], B["dyq"], B["dys"]), "hbm",
         act_bytes(Mm, Nm, 2)),
        ("quant_weight W_moe (+q_t)", lambda: fq.fp8q_quant_weight_128x128(L["wm"], B["wq"], B["wq_t"], B["ws"]),
         "hbm", E * Nm * K * 6 + cdiv(E * Nm, 128) * cdiv(K, 128) * 4),
        ("grouped_gemm_dgrad", lambda: fq.fp8q_grouped_gemm_dgrad(B["dyq"], B["dys"], B["wq_t"], B["ws"], L["off"],
                                                                  B["dx"]), "mfma", 2.0 * Mm * Nm * K),
        ("quant_transpose_grouped X_moe", lambda: fq.fp8q_quant_transpose_grouped(L["xm"], L["off"], B["xq_t"],
                                                                                 B["xs_t"]), "hbm",
         act_bytes(Mm, K, 2)),
        ("quant_transpose_grouped dY_moe", lambda: fq.fp8q_quant_transpose_grouped(L["dym"], L["off"], B["dyq_t"],
                                                                                  B["dys_t"]), "hbm",
         act_bytes(Mm, Nm, 2)),
        ("grouped_gemm_wgrad", lambda: fq.fp8q_grouped_gemm_wgrad(B["dyq_t"], B["dys_t"], B["xq_t"], B["xs_t"],
                                                                  L["off"], Mm, B["dw"]), "mfma",
         2.0 * Mm * Nm * K),
    ]
    return ops, B


def make_dual_ops(L, dev):
    """The dual-output quantizer on the linear layer's X and dY (each feeds a
    row-quantized GEMM and the weight-gradient GEMM), as make_ops."""
    import torch
    import fp8_fine_grained_quant_amd as fq

    ops = []
    for name, x in (("X", L["x"]), ("dY", L["dy"])):
        m, c = x.shape
        e = lambda *s, dt=torch.uint8: torch.empty(*s, dtype=dt, device=dev)
        bufs = (e(m, c), e(m, cdiv(c, 128), dt=torch.float32), e(c, m), e(c, cdiv(m, 128), dt=torch.float32))
        work = m * c * 4 + (m * cdiv(c, 128) + c * cdiv(m, 128)) * 4
        ops.append((f"quant_act_transpose {name}",
                    (lambda x=x, b=bufs: fq.fp8q_quant_act_transpose(x, *b)), "hbm", work))
    return ops


def make_mx_ops(L, dev):
    """The linear layer's step in the microscaling variant (MXFP8 E4M3, 1x32
    blocks along each product's contraction axis, E8M0 scales): one dual
    quantizer per tensor (row blocks and transposed column blocks from one
    read), then Fprop, Dgrad and Wgrad through the block-scaled MFMA GEMM."""
    import torch
    import fp8_fine_grained_quant_amd as fq

    u8 = torch.uint8
    e = lambda *s, dt=u8: torch.empty(*s, dtype=dt, device=dev)
    M, K = L["x"].shape
    N = L["w"].shape[0]
    Q = {}
    for name, t in (("x", L["x"]), ("w", L["w"]), ("dy", L["dy"])):
        r, c = t.shape
        Q[name] = (e(r, c), e(r, cdiv(c, 32)), e(c, r), e(c, cdiv(r, 32)))
    y, dx, dw = e(M, N, dt=torch.bfloat16), e(M, K, dt=torch.bfloat16), e(N, K, dt=torch.float32)
    qbytes = lambda r, c, es: r * c * (es + 2) + (r * cdiv(c, 32) + c * cdiv(r, 32))
    xq, xs, xq_t, xs_t = Q["x"]
    wq, ws, wq_t, ws_t = Q["w"]
    dyq, dys, dyq_t, dys_t = Q["dy"]
    ops = [
        ("mx quant X (rows + cols)", lambda: fq.fp8q_quant_mx_transpose(L["x"], xq_t, xs_t, xq, xs), "hbm",
         qbytes(M, K, 2)),
        ("mx quant W (rows + cols)", lambda: fq.fp8q_quant_mx_transpose(L["w"], wq_t, ws_t, wq, ws), "hbm",
         qbytes(N, K, 4)),
        ("mx gemm fprop", lambda: fq.fp8q_gemm_mx(xq, xs, wq, ws, y), "mfma", 2.0 * M * N * K),
        ("mx quant dY (rows + cols)", lambda: fq.fp8q_quant_mx_transpose(L["dy"], dyq_t, dys_t, dyq, dys), "hbm",
         qbytes(M, N, 2)),
        ("mx gemm dgrad", lambda: fq.fp8q_gemm_mx(dyq, dys, wq_t, ws_t, dx), "mfma", 2.0 * M * N * K),
        ("mx gemm wgrad", lambda: fq.fp8q_gemm_mx(dyq_t, dys_t, xq_t, xs_t, dw), "mfma", 2.0 * M * N * K),
    ]
    return ops


def make_exact_ops(L, O):
    """The exact-accumulation GEMMs (BF16 matrix instruction on exactly
    converted codes, FP32 promotion per 128-K chunk) on the step's own
    quantized operands: the linear layer's three products and the grouped
    Fprop, as make_ops."""
    import torch
    import fp8_fine_grained_quant_amd as fq

    E = 32
    M, K, N = L["x"].shape[0], L["x"].shape[1], L["w"].shape[0]
    Mm, Nm = L["xm"].shape[0], L["wm"].shape[0] // E
    dev = L["x"].device
    y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    dx = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
    dw = torch.empty(N, K, dtype=torch.float32, device=dev)
    ym = torch.empty(Mm, Nm, dtype=torch.bfloat16, device=dev)
    ops = [
        ("gemm_fprop_exact", lambda: fq.fp8q_gemm_fprop(O["xq"], O["xs"], O["wq"], O["ws"], y, exact=True),
         "mfma_bf16", 2.0 * M * N * K),
        ("gemm_dgrad_exact", lambda: fq.fp8q_gemm_dgrad(O["dyq"], O["dys"], O["wq_t"], O["ws"], dx, exact=True),
         "mfma_bf16", 2.0 * M * N * K),
        ("gemm_wgrad_exact", lambda: fq.fp8q_gemm_wgrad(O["dyq_t"], O["dys_t"], O["xq_t"], O["xs_t"], dw,
                                                        exact=True), "mfma_bf16", 2.0 * M * N * K),
        ("grouped_gemm_exact", lambda: fq.fp8q_grouped_gemm(O["xmq"], O["xms"], O["wmq"].view(E, Nm, K),
                                                            O["wms"].view(E, Nm // 128, K // 128), L["off"], ym,
                                                            exact=True), "mfma_bf16", 2.0 * Mm * Nm * K),
    ]
    return ops, dict(y=y, dx=dx, dw=dw, ym=ym)


def make_fused_ops(L, O):
    """Fprop and Dgrad of the linear layer with the next layer's 1x128
    quantization of their BF16 output fused into the GEMM epilogue, beside
    the same GEMMs followed by the separate quantizer, as make_ops."""
    import torch
    import fp8_fine_grained_quant_amd as fq

    M, K, N = L["x"].shape[0], L["x"].shape[1], L["w"].shape[0]
    dev = L["x"].device
    e = lambda *s, dt=torch.uint8: torch.empty(*s, dtype=dt, device=dev)
    F = dict(y=e(M, N, dt=torch.bfloat16), yq=e(M, N), ys=e(M, N // 128, dt=torch.float32),
             dx=e(M, K, dt=torch.bfloat16), dxq=e(M, K), dxs=e(M, K // 128, dt=torch.float32))
    flop = 2.0 * M * N * K
    ops = [
        ("gemm_fprop + quant_act Y", lambda: (fq.fp8q_gemm_fprop(O["xq"], O["xs"], O["wq"], O["ws"], F["y"]),
                                              fq.fp8q_quant_act_1x128(F["y"], F["yq"], F["ys"])), "mfma", flop),
        ("gemm_fprop_quant", lambda: fq.fp8q_gemm_fprop_quant(O["xq"], O["xs"], O["wq"], O["ws"], F["y"], F["yq"],
                                                               F["ys"]), "mfma", flop),
        ("gemm_dgrad + quant_act dX", lambda: (fq.fp8q_gemm_dgrad(O["dyq"], O["dys"], O["wq_t"], O["ws"], F["dx"]),
                                               fq.fp8q_quant_act_1x128(F["dx"], F["dxq"], F["dxs"])), "mfma", flop),
        ("gemm_dgrad_quant", lambda: fq.fp8q_gemm_dgrad_quant(O["dyq"], O["dys"], O["wq_t"], O["ws"], F["dx"],
                                                               F["dxq"], F["dxs"]), "mfma", flop),
    ]
    return ops


def tiny_gemm_latency(dev, reps=200):
    """The tiny Fprop (X bf16 [128,256], W fp32 [128,256], bf16 Y [128,128]):
    one launch, so its figure is latency.  Returns the median of single
    launches bracketed by HIP events, and the per-launch time of `reps`
    launches back to back."""
    import torch
    import fp8_fine_grained_quant_amd as fq
    import synth

    x, w = synth.tiny_fprop()
    xg, wg = x.to(dev), w.to(dev)
    xq = torch.empty(128, 256, dtype=torch.uint8, device=dev)
    xs = torch.empty(128, 2, dtype=torch.float32, device=dev)
    wq = torch.empty(128, 256, dtype=torch.uint8, device=dev)
    ws = torch.empty(1, 2, dtype=torch.float32, device=dev)
    y = torch.empty(128, 128, dtype=torch.bfloat16, device=dev)
    launch(("tiny quant_act X", lambda: fq.fp8q_quant_act_1x128(xg, xq, xs)))
    launch(("tiny quant_weight W", lambda: fq.fp8q_quant_weight_128x128(wg, wq, None, ws)))
    op = ("tiny gemm_fprop", lambda: fq.fp8q_gemm_fprop(xq, xs, wq, ws, y))
    stream = torch.cuda.current_stream()
    for _ in range(20):
        launch(op)
    torch.cuda.synchronize()
    single = []
    for _ in range(50):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        launch(op)
        b.record(stream)
        b.synchronize()
        single.append(a.elapsed_time(b) * 1e3)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        launch(op)
    b.record(stream)
    torch.cuda.synchronize()
    single.sort()
    # the same launches captured once in a HIP graph and replayed: the entry
    # points allocate nothing and never wait, so a caller can capture them;
    # a replay costs no host work per launch, so this is the GPU-side latency
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(reps):
            op[1]()
    torch.cuda.synchronize()
    times = []
    for _ in range(3):
        c, d = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c.record(stream)
        graph.replay()
        d.record(stream)
        torch.cuda.synchronize()
        LAUNCHES.extend([(op[0], 1)] * reps)  # the replay's dispatches, for the trace's attribution
        times.append(c.elapsed_time(d) * 1e3 / reps)
    return {"workload": "tiny Fprop X [128,256] . W [128,256]^T, bf16 out (8.39 MFLOP)",
            "single_launch_us_median": round(single[len(single) // 2], 2),
            "back_to_back_us_per_launch": round(a.elapsed_time(b) * 1e3 / reps, 2),
            "graph_replay_us_per_launch": round(min(times), 2),
            "launches": reps}


def telemetry(ops, seconds=3.0, settle=1.2):
    """GPU clock, power and activity while the step runs back to back for
    `seconds` (amdsmi, sampled every 20 ms from a thread), and the step time
    of that sustained loop.  The device's metrics table trails the hardware
    by about a second (measured: a busy GPU still read 214 MHz and 1%
    activity for the first ~1 s of a loop, then ~1.9-2.0 GHz and 100%), so
    only samples taken `settle` seconds or more after the loop started are
    reported.  Every device amdsmi lists is sampled; the one reported is the
    one whose PCI bus matches cuda:0, else the busiest.  Returns the reason
    instead if telemetry is unavailable."""
    import threading
    import torch
    try:
        import amdsmi
        amdsmi.amdsmi_init()
    except Exception as ex:  # pragma: no cover - depends on the host
        return {"unavailable": f"amdsmi: {ex}"}
    try:
        handles = amdsmi.amdsmi_get_processor_handles()
        bus = []
        for h in handles:
            try:
                bus.append(amdsmi.amdsmi_get_gpu_device_bdf(h))
            except Exception:
                bus.append("?")
        samples = [{"clk": [], "pwr": [], "act": []} for _ in handles]
        stop = threading.Event()
        t_keep = [float("inf")]  # samples before this time are dropped

        def sample():
            while not stop.is_set():
                if time.perf_counter() < t_keep[0]:
                    time.sleep(0.02)
                    continue
                for h, smp in zip(handles, samples):
                    try:
                        c = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX)
                        smp["clk"].append(float(c.get("clk", c.get("cur_clk"))))
                    except Exception:
                        pass
                    try:
                        p = amdsmi.amdsmi_get_power_info(h)
                        v = p.get("current_socket_power", "N/A")
                        if v in ("N/A", None):
                            v = p.get("average_socket_power", "N/A")
                        if v not in ("N/A", None):
                            smp["pwr"].append(float(v))
                    except Exception:
                        pass
                    try:
                        smp["act"].append(float(amdsmi.amdsmi_get_gpu_activity(h)["gfx_activity"]))
                    except Exception:
                        pass
                time.sleep(0.02)

        th = threading.Thread(target=sample, daemon=True)
        th.start()
        torch.cuda.synchronize()
        t0, n = time.perf_counter(), 0
        t_keep[0] = t0 + settle
        while time.perf_counter() - t0 < seconds:
            for _ in range(10):
                for op in ops:
                    launch(op)
            n += 10
            torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        stop.set()
        th.join()
        med = lambda v: sorted(v)[len(v) // 2] if v else None
        pick, how = None, "busiest"
        try:
            want = torch.cuda.get_device_properties(0).pci_bus_id
            for k, b in enumerate(bus):
                if b != "?" and int(b.split(":")[1], 16) == want:
                    pick, how = k, "pci bus of cuda:0"
        except Exception:
            pass
        if pick is None:
            pick = max(range(len(handles)), key=lambda k: med(samples[k]["act"]) or 0.0)
        smp = samples[pick]
        return {"device": {"bdf": bus[pick], "chosen_by": how, "devices_listed": len(handles)},
                "sclk_mhz": {"median": med(smp["clk"]), "min": min(smp["clk"]) if smp["clk"] else None,
                             "max": max(smp["clk"]) if smp["clk"] else None, "samples": len(smp["clk"])},
                "power_w": {"median": med(smp["pwr"]), "max": max(smp["pwr"]) if smp["pwr"] else None,
                            "samples": len(smp["pwr"])},
                "gfx_activity_pct": {"median": med(smp["act"]), "samples": len(smp["act"])},
                "sustained_ms_per_step": round(dt * 1e3 / n, 4), "steps": n,
                "note": f"sampled every 20 ms over the last {seconds - settle:.1f} s of {seconds:.1f} s of the step "
                        "running back to back, right before the timed region (the metrics table trails the "
                        f"hardware by about a second, so the first {settle:.1f} s are not sampled)"}
    finally:
        try:
            amdsmi.amdsmi_shut_down()
        except Exception:
            pass


def context_error(H, outs, samples=64, seed=7):
    """Error of the GPU outputs against the unquantized product in FP64 (the
    inputs before quantization: X and dY in BF16, W in FP32), on sampled
    output rows: relative Frobenius norm and max |y - Y_true| / S_true with
    S_true = sum_k |a_k b_k|.  Plain NumPy on the host inputs."""
    import numpy as np

    rng = np.random.Generator(np.random.PCG64(seed))
    x = H["x"].float().numpy().astype(np.float64)
    dy = H["dy"].float().numpy().astype(np.float64)
    w = H["w"].numpy().astype(np.float64)
    M, K = x.shape
    N = w.shape[0]
    rows = np.sort(rng.choice(M, samples, replace=False))
    chans = np.sort(rng.choice(N, samples, replace=False))
    cases = {
        "fprop": (x[rows], w, lambda o: o["y"][rows]),
        "dgrad": (dy[rows], w.T, lambda o: o["dx"][rows]),
        "wgrad": (dy[:, chans].T, x.T, lambda o: o["dw"][chans]),
    }
    out = {}
    for name, (a, b, pick) in cases.items():
        y_true = a @ b.T
        s_true = np.abs(a) @ np.abs(b).T
        d = {}
        for path, o in outs.items():
            y = pick(o).float().cpu().numpy().astype(np.float64)
            err = y - y_true
            d[path] = {"rel_frobenius": float(np.linalg.norm(err) / np.linalg.norm(y_true)),
                       "max_err_over_S_true": float((np.abs(err) / s_true).max())}
        out[name] = d
    out["sample"] = f"{samples} seeded output rows of each product (dW: {samples} rows = output channels)"
    return out


def _algorithmic_mbytes():
    """Operand + scale + output bytes of each GEMM op of the step and its side
    sections (the quantizers' bytes are their `mbytes`)."""
    M, K, N, Mm, E = 4096, 7168, 2048, 16384, 32
    g = lambda m, n, k, out_es: (m * k + n * k + (m + n) * (k // 128) * 4 + m * n * out_es) / 1e6
    fp, dg, wg = g(M, N, K, 2), g(M, K, N, 2), g(N, K, M, 4)
    gr = (Mm * K + E * N * K + (Mm + E * N) * (K // 128) * 4 + Mm * N * 2) / 1e6
    grd = (Mm * N + E * N * K + (Mm + E * N) * (K // 128) * 4 + Mm * K * 2) / 1e6
    grw = (Mm * (N + K) + Mm // 128 * (N + K) * 4 + E * N * K * 4) / 1e6
    return {"gemm_fprop": fp, "gemm_dgrad": dg, "gemm_wgrad": wg, "grouped_gemm": gr, "grouped_gemm_dgrad": grd,
            "grouped_gemm_wgrad": grw, "gemm_fprop_exact": fp, "gemm_dgrad_exact": dg, "gemm_wgrad_exact": wg,
            "grouped_gemm_exact": gr, "gemm_fprop_quant": fp + M * N / 1e6 + M * N / 128 * 4 / 1e6,
            "gemm_dgrad_quant": dg + M * K / 1e6 + M * K / 128 * 4 / 1e6, "mx gemm fprop": fp, "mx gemm dgrad": dg,
            "mx gemm wgrad": wg}


def _csv_rows(d, suffix):
    import csv
    import glob
    paths = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not paths:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    with open(paths[0]) as f:
        return list(csv.DictReader(f))


def _attribute(rows, log_path):
    """rows: one per library kernel dispatch; the launch log names the op of
    each dispatch in order.  Returns {op: [rows]} (asserts the counts match)."""
    from collections import defaultdict
    with open(log_path) as f:
        seq = [name for name, nk in json.load(f) for _ in range(nk)]
    rows = sorted((r for r in rows if "fp8q::" in r["Kernel_Name"]), key=lambda r: int(r["Dispatch_Id"]))
    if len(rows) != len(seq):
        raise AssertionError(f"{len(rows)} library dispatches in the trace, {len(seq)} in the launch log")
    by = defaultdict(list)
    for r, op in zip(rows, seq):
        by[op].append(r)
    return by


def _short(name):
    import re
    m = re.match(r"void fp8q::(\w+(<[^(]*>)?)\(", name)
    return (m.group(1) if m else name).replace("fp8q::", "")


def profile_summary(prof, bench_json=None):
    """Summaries of rocprofv3 runs of this bench (each run made with
    --launch-log <its dir>/launches.json and --no-telemetry): prof/kt (the
    kernel trace), prof/FETCH_SIZE and prof/WRITE_SIZE (one counter each),
    prof/cal_FETCH_SIZE and prof/cal_WRITE_SIZE (--copy-calibration 1024).
    Prints the per-op kernel-trace table and the per-op HBM traffic table
    (markdown) and writes profiles/traffic.json for the current kernel
    sources."""
    ev = {}
    if bench_json:
        with open(bench_json) as f:
            bj = json.loads(f.read().strip().splitlines()[-1])
        for sec in (None, "step_separate_quantizers", "moe_backward", "dual_output_quantizer", "microscaling_variant",
                    "exact_variant", "fused_output_quant"):
            ev.update((bj if sec is None else bj[sec])["kernels"])
    by = _attribute(_csv_rows(os.path.join(prof, "kt"), "kernel_trace.csv"), os.path.join(prof, "kt", "launches.json"))
    print("| op | kernel | launches | mean us | median us | min us | bench.py HIP-event avg us |")
    print("|---|---|---|---|---|---|---|")
    for op, rows in by.items():
        d = sorted((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows)
        ks = sorted({_short(r["Kernel_Name"]) for r in rows})
        print(f"| {op} | {', '.join('`' + k + '`' for k in ks)} | {len(d)} | {sum(d) / len(d):.2f} | "
              f"{d[len(d) // 2]:.2f} | {d[0]:.2f} | {ev.get(op, {}).get('avg_us', '')} |")

    def counter(c, sub):
        rows = [r for r in _csv_rows(os.path.join(prof, sub), "counter_collection.csv") if r["Counter_Name"] == c]
        return rows

    def per_op(c):
        b = _attribute(counter(c, c), os.path.join(prof, c, "launches.json"))
        return {op: sum(float(r["Counter_Value"]) for r in v) / len(v) for op, v in b.items()}

    def calib(c):
        big = [float(r["Counter_Value"]) for r in counter(c, "cal_" + c) if "copyBuffer" in r["Kernel_Name"]]
        if not big:
            raise AssertionError(f"no copy kernel in the {c} calibration run")
        return sum(big) / len(big)

    nbytes = 1024000000
    ff, wf = nbytes / 1024 / calib("FETCH_SIZE"), nbytes / 1024 / calib("WRITE_SIZE")
    fc, wc = per_op("FETCH_SIZE"), per_op("WRITE_SIZE")
    alg = _algorithmic_mbytes()
    out = {"source_sha": kernel_source_hash(), "copy_calibration": {"bytes": float(nbytes), "fetch_factor": ff,
                                                                    "write_factor": wf}, "kernels": {}}
    print()
    print(f"Calibration: FETCH_SIZE x {ff:.4f}, WRITE_SIZE x {wf:.4f} (a plain copy of {nbytes} bytes)")
    print()
    print("| op | FETCH KiB (counted) | WRITE KiB (counted) | traffic MB (scaled) | algorithmic MB | traffic / algorithmic |")
    print("|---|---|---|---|---|---|")
    for op in fc:
        b = (fc[op] * ff + wc.get(op, 0.0) * wf) * 1024
        a = ev.get(op, {}).get("mbytes") or alg.get(op)
        ratio = f"{b / 1e6 / a:.2f}" if a else ""
        print(f"| {op} | {fc[op]:.0f} | {wc.get(op, 0.0):.0f} | {b / 1e6:.1f} | {a or ''} | {ratio} |")
        out["kernels"][op] = {"fetch_kib_counted": fc[op], "write_kib_counted": wc.get(op, 0.0),
                              "bytes_per_launch": int(b)}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)


def counters_summary(prof):
    """Per-op means of every counter collected under prof/pmc*/ (one rocprofv3
    --pmc run per directory, each with its launch log), for the GEMM ops, as a
    markdown table (ops as columns)."""
    import glob
    from collections import defaultdict
    vals = defaultdict(dict)
    for d in sorted(p for p in glob.glob(os.path.join(prof, "pmc*")) if os.path.isdir(p)):
        rows = _csv_rows(d, "counter_collection.csv")
        names = sorted({r["Counter_Name"] for r in rows})
        for c in names:
            b = _attribute([r for r in rows if r["Counter_Name"] == c], os.path.join(d, "launches.json"))
            for op, v in b.items():
                vals[op][c] = sum(float(r["Counter_Value"]) for r in v) / len(v)
    ops = [op for op in vals if "gemm" in op and "+" not in op and not op.startswith("tiny")]
    counters = sorted({c for op in ops for c in vals[op]})
    print("| counter | " + " | ".join(ops) + " |")
    print("|---|" + "---|" * len(ops))
    for c in counters:
        print(f"| {c} | " + " | ".join(f"{vals[op].get(c, float('nan')):.4g}" for op in ops) + " |")
    # matrix-core busy: busy cycles per SIMD (1024 SIMDs) over active cycles per XCD (8 XCDs)
    print()
    print("| op | MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES / 1024) / (GRBM_GUI_ACTIVE / 8) |")
    print("|---|---|")
    for op in ops:
        v = vals[op]
        if "SQ_VALU_MFMA_BUSY_CYCLES" in v and "GRBM_GUI_ACTIVE" in v:
            print(f"| {op} | {v['SQ_VALU_MFMA_BUSY_CYCLES'] / 1024 / (v['GRBM_GUI_ACTIVE'] / 8):.1%} |")


def time_ops(ops, steps, warmup, stream, flush=None):
    """Run `warmup` untimed passes, then time `steps` passes back to back
    (HIP events on `stream` before the first and after the last launch only),
    then `steps` more passes with HIP events around every launch for the
    per-kernel breakdown; returns (ms per pass, per-kernel summaries).

    flush: a callable run before every pass, outside the timed launches (a
    read of a buffer larger than the 256 MB MALL), for sections whose
    whole working set would otherwise stay cache-resident from pass to pass,
    unlike in a training step.  The pass time is then the mean over the
    instrumented passes of first launch start to last launch end."""
    import torch

    for _ in range(warmup):
        if flush:
            flush()
        for op in ops:
            launch(op)
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in ops]
          for _ in range(steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ms_pass = None
    if not flush:
        # the passes back to back, with no instrumentation between launches
        torch.cuda.synchronize()
        t_start.record(stream)
        for s in range(steps):
            for op in ops:
                launch(op)
        t_end.record(stream)
        torch.cuda.synchronize()
        ms_pass = t_start.elapsed_time(t_end) / steps
    # the per-kernel breakdown: the same passes again, with HIP events around every launch
    torch.cuda.synchronize()
    for s in range(steps):
        if flush:
            flush()
        for i, op in enumerate(ops):
            ev[s][i][0].record(stream)
            launch(op)
            ev[s][i][1].record(stream)
    torch.cuda.synchronize()
    if flush:
        ms_pass = sum(ev[s][0][0].elapsed_time(ev[s][-1][1]) for s in range(steps)) / steps
    kernels = {}
    for i, (name, _, kind, work) in enumerate(ops):
        times = sorted(ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(steps))
        avg_ms = sum(times) / len(times)
        d = {"avg_us": round(avg_ms * 1e3, 2), "median_us": round(times[len(times) // 2] * 1e3, 2)}
        if kind in ("mfma", "mfma_bf16"):
            a = work / (avg_ms * 1e-3) / 1e12
            peak = PEAK_FP8_TFLOPS if kind == "mfma" else PEAK_BF16_TFLOPS
            d.update(gflop=round(work / 1e9, 3), tflops=round(a, 1), frac_peak=round(a / peak, 4))
        else:
            a = work / (avg_ms * 1e-3) / 1e9
            d.update(mbytes=round(work / 1e6, 3), gbs=round(a, 1), frac_peak=round(a / PEAK_HBM_GBS, 4))
        kernels[name] = d
        log(f"{name:32s} {d}")
    return ms_pass, kernels


def cpu_baseline(H, frac):
    """The CPU oracle, as it stands, on a token sample of one step: the first
    `frac` of the tokens (rounded to 128) of the linear layer (quantizers,
    Fprop, Dgrad, and Wgrad over those tokens) and of the MoE layer (its
    quantizer over those tokens, the weights of the experts they reach, the
    grouped Fprop).  Returns its GEMM throughput in the bench's unit."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
                           or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    x, w, dy, xm, wm, off = H["x"], H["w"], H["dy"], H["xm"], H["wm"], H["off"]
    M, K = x.shape
    N = w.shape[0]
    rs = max(128, int(M * frac) // 128 * 128)
    ts = max(128, int(xm.shape[0] * frac) // 128 * 128)
    x_s = x[:rs].float().numpy()
    dy_s = dy[:rs].float().numpy()
    xm_s = xm[:ts].float().numpy()
    offs = np.minimum(off.numpy().astype(np.int64), ts)
    experts = [e for e in range(len(offs) - 1) if offs[e + 1] > offs[e]]
    per_op = {}

    def timed(name, fn, kind, work):
        t = time.perf_counter()
        r = fn()
        dt = time.perf_counter() - t
        d = {"s": round(dt, 3)}
        if kind == "gemm":
            d["gflops"] = round(work / dt / 1e9, 2)
        else:
            d["gbs"] = round(work / dt / 1e9, 4)
        per_op[name] = d
        return r

    act_bytes = lambda r, c: r * c * 3 + r * cdiv(c, 128) * 4
    flops = 0.0
    t0 = time.perf_counter()
    xq, xsc = timed("quant_act X", lambda: oracle.quant_act_1x128(x_s), "quant", act_bytes(rs, K))
    wq, wsc, _ = timed("quant_weight W (+q_t)", lambda: oracle.quant_weight_128x128(w.numpy()), "quant",
                       N * K * 6 + cdiv(N, 128) * cdiv(K, 128) * 4)
    timed("gemm_fprop", lambda: oracle.fprop_ref(xq, xsc, wq, wsc), "gemm", 2.0 * rs * N * K)
    dyq, dysc = timed("quant_act dY", lambda: oracle.quant_act_1x128(dy_s), "quant", act_bytes(rs, N))
    timed("gemm_dgrad", lambda: oracle.dgrad_ref(dyq, dysc, wq, wsc), "gemm", 2.0 * rs * N * K)
    xq_t, xs_t = timed("quant_transpose X", lambda: oracle.quant_transpose(x_s), "quant", act_bytes(rs, K))
    dq_t, ds_t = timed("quant_transpose dY", lambda: oracle.quant_transpose(dy_s), "quant", act_bytes(rs, N))
    timed("gemm_wgrad", lambda: oracle.wgrad_ref(dq_t, ds_t, xq_t, xs_t), "gemm", 2.0 * rs * N * K)
    flops += 3 * 2.0 * rs * N * K
    xmq, xmsc = timed("quant_act X_moe", lambda: oracle.quant_act_1x128(xm_s), "quant", act_bytes(ts, K))
    wmq = np.zeros(wm.shape, dtype=np.uint8)
    wms = np.zeros((wm.shape[0], N // 128, K // 128), dtype=np.float32)

    def quant_experts():
        for e in experts:
            wmq[e], wms[e], _ = oracle.quant_weight_128x128(wm[e].numpy())

    timed("quant_weight W_moe", quant_experts, "quant", len(experts) * (N * K * 5 + (N // 128) * (K // 128) * 4))
    timed("grouped_gemm", lambda: oracle.grouped_ref(xmq, xmsc, wmq, wms, offs), "gemm", 2.0 * ts * N * K)
    flops += 2.0 * ts * N * K
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"one step on a token sample: linear layer on the first {rs} of {M} tokens (all three "
                      f"GEMMs, all quantizers, full W), MoE layer on the first {ts} of {xm.shape[0]} tokens "
                      f"({len(experts)} experts reached, their weights quantized); {dt:.1f}s wall; FP64 BLAS "
                      f"GEMMs on {blas_threads} threads, NumPy quantizers on one",
            "per_op": per_op,
            "per_op_note": "quantizers: NumPy on one core, GB/s of the same algorithmic bytes as the GPU's; "
                           "GEMMs: the FP64 product of the dequantized operands plus the sum|a*b| normaliser "
                           f"(two BLAS GEMMs) on {blas_threads} threads, GFLOP/s of the useful 2MNK"}


def kernel_source_hash():
    """SHA-256 over the kernel sources' code (comments and whitespace
    removed): measured HBM traffic is reported only while the kernels are
    the ones the counters were taken on, and an edit of a comment does not
    change them."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "fp8_fine_grained_quant_amd", "csrc", name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel calibration), or None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha") != kernel_source_hash():
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


def copy_calibration(mbytes, reps):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch
    n = int(mbytes * 1e6) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "reps": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-frac", type=float, default=1 / 2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=float, default=0.0, metavar="MB",
                    help="only run a plain device copy of MB megabytes (counter calibration) and exit")
    ap.add_argument("--no-telemetry", action="store_true",
                    help="skip the sustained-load telemetry loop (profiling runs: a deterministic launch sequence)")
    ap.add_argument("--launch-log", metavar="JSON", help="write the ops in launch order (for --profile-summary)")
    ap.add_argument("--profile-summary", metavar="DIR",
                    help="only summarize rocprofv3 runs of this bench under DIR (see profile_summary) and exit")
    ap.add_argument("--bench-json", metavar="FILE", help="with --profile-summary: a bench line to compare against")
    ap.add_argument("--counters-summary", metavar="DIR",
                    help="only summarize the rocprofv3 --pmc runs under DIR/pmc* (see counters_summary) and exit")
    args = ap.parse_args()
    if args.profile_summary:
        profile_summary(args.profile_summary, args.bench_json)
        return
    if args.counters_summary:
        counters_summary(args.counters_summary)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the path is built and timed on a single MI355X; "
              "multi-GPU runs are not part of this library", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration, 5)
        return

    import torch
    import fp8_fine_grained_quant_amd as fq

    fq.load_library()
    dev = "cuda:0"
    H = host_inputs()
    L = build_workload(H, dev)
    ops, O = make_ops(L, dev)
    names = [o[0] for o in ops]

    stream = torch.cuda.current_stream()
    # the step under sustained load first: clock, power and activity, and the
    # GPU at its working clocks before the timed region
    tele = None
    if not args.no_telemetry:
        log("telemetry: the step back to back for ~1.5 s")
        tele = telemetry(ops)
        log(f"telemetry {tele}")
    log(f"warmup {args.warmup} steps, timing {args.steps} steps")
    ms_step, kernels = time_ops(ops, args.steps, args.warmup, stream)
    sops, _ = make_ops(L, dev, form="separate")
    log(f"the step with separate quantizer launches: warmup {args.warmup}, timing {args.steps} steps")
    ms_sep, skernels = time_ops(sops, args.steps, args.warmup, stream)

    # the MoE backward, beside the step
    bops, _ = make_moe_bwd_ops(L, dev)
    log(f"MoE backward: warmup {args.warmup}, timing {args.steps} passes")
    ms_bwd, bkernels = time_ops(bops, args.steps, args.warmup, stream)
    bwd_flops = sum(w for _, _, k, w in bops if k == "mfma")

    # sections beside the step whose passes would fit the MALL: flushed between passes
    # (a read of 1 GiB: the lines it evicts are clean, so the next kernel pays
    # no write-back for it)
    flush_buf = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
    flush = flush_buf.sum

    # the dual-output quantizer, beside the step (the step keeps the separate ones)
    dops = make_dual_ops(L, dev)
    log(f"dual-output quantizer: warmup {args.warmup}, timing {args.steps} passes")
    _, dkernels = time_ops(dops, args.steps, args.warmup, stream, flush)

    # the microscaling variant of the linear layer's step, beside the step
    mops = make_mx_ops(L, dev)
    log(f"microscaling variant: warmup {args.warmup}, timing {args.steps} passes")
    ms_mx, mkernels = time_ops(mops, args.steps, args.warmup, stream, flush)
    del flush_buf
    mx_flops = sum(w for _, _, k, w in mops if k == "mfma")

    # the exact-accumulation GEMMs on the step's quantized operands, beside the step
    flush_buf = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
    flush = flush_buf.sum
    xops, X = make_exact_ops(L, O)
    log(f"exact-accumulation GEMMs: warmup {args.warmup}, timing {args.steps} passes")
    _, xkernels = time_ops(xops, args.steps, args.warmup, stream, flush)
    fops = make_fused_ops(L, O)
    log(f"fused output quantization: warmup {args.warmup}, timing {args.steps} passes")
    _, fkernels = time_ops(fops, args.steps, args.warmup, stream, flush)
    del flush_buf

    log("tiny GEMM latency")
    tiny = tiny_gemm_latency(dev)
    log(f"tiny {tiny}")

    log("context error against the unquantized FP64 products")
    ctx = context_error(H, {"fp8": {"y": O["y"], "dx": O["dx"], "dw": O["dw"]},
                            "exact": {"y": X["y"], "dx": X["dx"], "dw": X["dw"]}})
    log(f"context {ctx}")
    lin = ["quant_act X", "quant_weight W (+q_t)", "gemm_fprop", "quant_act dY", "gemm_dgrad", "quant_transpose X",
           "quant_transpose dY", "gemm_wgrad"]
    lin_us = sum(skernels[n]["avg_us"] for n in lin)
    lin_batched_us = sum(kernels[n]["avg_us"] for n in ("quant_batch W (+q_t) + X (rows + cols)", "gemm_fprop",
                                                        "quant_act_transpose dY", "gemm_dgrad", "gemm_wgrad"))
    quant_lin = {"batched": round(kernels["quant_batch W (+q_t) + X (rows + cols)"]["avg_us"]
                                  + kernels["quant_act_transpose dY"]["avg_us"], 2),
                 "separate": round(sum(skernels[n]["avg_us"] for n in lin if n.startswith("quant")), 2)}

    gemm_flops = sum(w for _, _, k, w in ops if k == "mfma")
    value = gemm_flops / (ms_step * 1e-3) / 1e12
    dom = max(range(len(ops)), key=lambda i: kernels[names[i]]["avg_us"])
    dname, _, dkind, dwork = ops[dom]
    dk = kernels[dname]
    traffic = measured_traffic(dname)
    if dkind == "mfma":
        roof = {"kernel": dname, "bound": "mfma", "achieved": dk["tflops"], "peak": PEAK_FP8_TFLOPS,
                "unit": "TFLOP/s", "frac": dk["frac_peak"], "traffic": traffic}
    else:
        roof = {"kernel": dname, "bound": "hbm", "achieved": dk["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": dk["frac_peak"], "traffic": traffic}

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(H, args.cpu_frac)
        log(f"cpu baseline {cpu}")

    out = {
        "metric": "FP8 blockwise GEMM TFLOP/s & % FP8 MFMA peak; quantize GB/s & % HBM peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 x fp8e4m3 -> f32 (bf16/f32 out)",
        "data": "synthetic",
        "config": {
            "workload": "FP8 linear layer Fprop+Dgrad+Wgrad (X [4096,7168] bf16, W [2048,7168] fp32, dY [4096,2048] "
                        "bf16) + MoE grouped Fprop (X [16384,7168] bf16, 32 experts of [2048,7168] fp32, Zipf "
                        "token counts), each with its online 1x128 / 128x128 E4M3 quantization",
            "gemm_gflop_per_step": round(gemm_flops / 1e9, 2),
            "value_definition": "useful GEMM FLOPs of the step / step time (quantizers inside the timed step)",
        },
        "roofline": roof,
        "kernel_source_sha": kernel_source_hash(),
        "kernels": kernels,
        "linear_layer_quantization_us": quant_lin,
        "linear_layer_quantization_note": "all quantization of the linear layer's step (X, W with its transposed "
                                          "codes, dY, and the token-grouped transposed codes of X and dY): the step's "
                                          "two batched/dual launches against the five separate quantizer launches; "
                                          "316.9 MB of algorithmic bytes (70% of HBM peak = 56.6 us)",
        "step_separate_quantizers": {
            "ms_per_step": round(ms_sep, 4),
            "value": round(sum(w for _, _, k, w in sops if k == "mfma") / (ms_sep * 1e-3) / 1e12, 2),
            "kernels": skernels,
        },
        "moe_backward": {
            "workload": "MoE layer backward: dY [16384,2048] bf16 (Student-t(3), 1% token rows x100), X and the "
                        "32 experts' W as the step's MoE layer; grouped Dgrad (bf16 dX) and grouped Wgrad "
                        "(fp32 dW [32,2048,7168]) with their online quantization",
            "ms_per_pass": round(ms_bwd, 4),
            "gemm_gflop_per_pass": round(bwd_flops / 1e9, 2),
            "gemm_tflops": round(bwd_flops / (ms_bwd * 1e-3) / 1e12, 2),
            "kernels": bkernels,
        },
        "dual_output_quantizer": {
            "workload": "quant_act_1x128 + quant_transpose of the linear layer's X [4096,7168] and dY [4096,2048] "
                        "(bf16) in one pass each",
            "kernels": dkernels,
            "separate_us": {n: round(skernels[f"quant_act {n}"]["avg_us"]
                                     + skernels[f"quant_transpose {n}"]["avg_us"], 2) for n in ("X", "dY")},
        },
        "microscaling_variant": {
            "workload": "the linear layer's Fprop+Dgrad+Wgrad (shapes as the step) in MXFP8 E4M3: 1x32 blocks "
                        "along each product's contraction axis, E8M0 scales applied by the block-scaled MFMA; "
                        "one dual quantizer per tensor",
            "ms_per_pass": round(ms_mx, 4),
            "gemm_tflops": round(mx_flops / (ms_mx * 1e-3) / 1e12, 2),
            "method_linear_layer_us": {"separate_quantizers": round(lin_us, 2), "as_step": round(lin_batched_us, 2)},
            "kernels": mkernels,
        },
        "exact_variant": {
            "workload": "the step's GEMMs (linear Fprop, Dgrad, Wgrad; MoE grouped Fprop) on the same quantized "
                        "operands through the *_exact entry points: codes converted exactly to BF16, BF16 matrix "
                        "instruction (exact products, FP32 sums), FP32 promotion per 128-K chunk; the path that "
                        "stays within 1e-5 * sum|a*b| of the exact contraction",
            "peak_tflops": PEAK_BF16_TFLOPS,
            "kernels": xkernels,
        },
        "fused_output_quant": {
            "workload": "the linear layer's Fprop (Y [4096,2048]) and Dgrad (dX [4096,7168]) writing BF16 output "
                        "and, fused into the epilogue, its 1x128 E4M3 codes and scales (the next layer's FP8 "
                        "input), against the same GEMM followed by quant_act_1x128 of its output; each entry is "
                        "one launch pair or one launch between HIP events",
            "kernels": fkernels,
            "saved_us": {
                "fprop": round(fkernels["gemm_fprop + quant_act Y"]["avg_us"] - fkernels["gemm_fprop_quant"]["avg_us"], 2),
                "dgrad": round(fkernels["gemm_dgrad + quant_act dX"]["avg_us"] - fkernels["gemm_dgrad_quant"]["avg_us"],
                               2)},
        },
        "tiny_gemm": tiny,
        "telemetry": tele,
        "context_error": ctx,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    if args.launch_log:
        os.makedirs(os.path.dirname(os.path.abspath(args.launch_log)), exist_ok=True)
        with open(args.launch_log, "w") as f:
            json.dump(LAUNCHES, f)


if __name__ == "__main__":
    main()
