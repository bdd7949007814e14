#!/usr/bin/env python3
"""Benchmark of the FP8 fine-grained quantization + block-scaled GEMM hot path
on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic inputs:
  linear layer X [4096,7168] bf16, W [2048,7168] fp32, dY [4096,2048] bf16
    quant_act(X) -> quant_weight(W, +q_t) -> Fprop Y = X W^T (bf16)
    quant_act(dY) -> Dgrad dX = dY W (bf16)
    quant_transpose(X), quant_transpose(dY) -> Wgrad dW = dY^T X (fp32)
  MoE layer X [16384,7168] bf16 routed to 32 experts W_e [2048,7168] fp32
    quant_act(X) -> quant_weight(W stacked) -> grouped Fprop (bf16)
Inputs are generated and resident in HBM before the timed region.

Prints one JSON line on stdout; progress goes to stderr.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cdiv(a, b):
    return (a + b - 1) // b


def build_workload(dev):
    import torch
    import synth

    t0 = time.time()
    x, w = synth.linear_x_w()
    dy = synth.linear_dy()
    xm, wm, off = synth.moe_fprop()
    log(f"inputs generated in {time.time() - t0:.1f}s; moving to {dev}")
    g = lambda t: t.to(dev)
    L = dict(x=g(x), w=g(w), dy=g(dy), xm=g(xm), wm=g(wm).reshape(-1, wm.shape[2]), off=g(off))
    del x, w, dy, xm, wm
    return L


def make_ops(L, dev):
    """The step's kernels as (name, launch, kind, algorithmic work per launch)."""
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
        ("quant_act X_moe", lambda: fq.fp8q_quant_act_1x128(L["xm"], O["xmq"], O["xms"]), "hbm",
         act_bytes(Mm, K, 2)),
        ("quant_weight W_moe", lambda: fq.fp8q_quant_weight_128x128(L["wm"], O["wmq"], None, O["wms"]), "hbm",
         E * Nm * K * 5 + cdiv(E * Nm, 128) * cdiv(K, 128) * 4),
        ("grouped_gemm", lambda: fq.fp8q_grouped_gemm(O["xmq"], O["xms"], O["wmq"].view(E, Nm, K),
                                                      O["wms"].view(E, Nm // 128, K // 128), L["off"], O["ym"]),
         "mfma", 2.0 * Mm * Nm * K),
    ]
    return ops, O


def cpu_baseline(frac):
    """The CPU oracle, as it stands, on a row sample (fraction `frac`) of
    every op of one step; returns its GEMM throughput."""
    import numpy as np
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
                           or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    x, w = synth.linear_x_w()
    dy = synth.linear_dy()
    M, K = x.shape
    N = w.shape[0]
    rs = max(1, int(M * frac))
    ns = max(128, int(N * frac) // 128 * 128)
    xs_ = x[:rs].float().numpy()
    dys_ = dy[:rs].float().numpy()
    wf = w.numpy()
    flops = 0.0
    t0 = time.perf_counter()
    xq, xsc = oracle.quant_act_1x128(xs_)
    wq, wsc, _ = oracle.quant_weight_128x128(wf[:ns])            # a slice of the weight rows
    wq_full, wsc_full, _ = oracle.quant_weight_128x128(wf)        # the GEMMs need all of W
    y, _ = oracle.fprop_ref(xq, xsc, wq_full, wsc_full)
    flops += 2.0 * rs * N * K
    dyq, dysc = oracle.quant_act_1x128(dys_)
    dx, _ = oracle.dgrad_ref(dyq, dysc, wq_full, wsc_full)
    flops += 2.0 * rs * N * K
    xq_t, xs_t = oracle.quant_transpose(x.float().numpy()[:, : max(128, int(K * frac))])
    dq_t, ds_t = oracle.quant_transpose(dy.float().numpy()[:, :ns])
    dw, _ = oracle.wgrad_ref(dq_t, ds_t, xq_t, xs_t)
    flops += 2.0 * ns * xq_t.shape[0] * M
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"linear-layer step on a {frac:g} row sample (X/dY rows {rs}, W rows {ns} quantized "
                      f"plus full W for the GEMM operands, Wgrad {ns}x{xq_t.shape[0]} outputs over {M} tokens); "
                      f"{dt:.1f}s wall, FP64 BLAS GEMMs + NumPy quantizers"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-frac", type=float, default=1 / 32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the path is built and timed on a single MI355X; "
              "multi-GPU runs are not part of this library", file=sys.stderr)
        sys.exit(2)

    import torch
    import fp8_fine_grained_quant_amd as fq

    fq.load_library()
    dev = "cuda:0"
    L = build_workload(dev)
    ops, O = make_ops(L, dev)
    names = [o[0] for o in ops]

    def step():
        for _, fn, _, _ in ops:
            fn()

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in ops]
          for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t_start.record(stream)
    for s in range(args.steps):
        for i, (_, fn, _, _) in enumerate(ops):
            ev[s][i][0].record(stream)
            fn()
            ev[s][i][1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps

    kernels = {}
    for i, (name, _, kind, work) in enumerate(ops):
        times = sorted(ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(args.steps))
        avg_ms = sum(times) / len(times)
        d = {"avg_us": round(avg_ms * 1e3, 2), "median_us": round(times[len(times) // 2] * 1e3, 2)}
        if kind == "mfma":
            a = work / (avg_ms * 1e-3) / 1e12
            d.update(gflop=round(work / 1e9, 3), tflops=round(a, 1), frac_peak=round(a / PEAK_FP8_TFLOPS, 4))
        else:
            a = work / (avg_ms * 1e-3) / 1e9
            d.update(mbytes=round(work / 1e6, 3), gbs=round(a, 1), frac_peak=round(a / PEAK_HBM_GBS, 4))
        kernels[name] = d
        log(f"{name:24s} {d}")

    gemm_flops = sum(w for _, _, k, w in ops if k == "mfma")
    value = gemm_flops / (ms_step * 1e-3) / 1e12
    dom = max(range(len(ops)), key=lambda i: kernels[names[i]]["avg_us"])
    dname, _, dkind, dwork = ops[dom]
    dk = kernels[dname]
    if dkind == "mfma":
        roof = {"kernel": dname, "bound": "mfma", "achieved": dk["tflops"], "peak": PEAK_FP8_TFLOPS,
                "unit": "TFLOP/s", "frac": dk["frac_peak"], "traffic": None}
    else:
        roof = {"kernel": dname, "bound": "hbm", "achieved": dk["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": dk["frac_peak"], "traffic": None}

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(args.cpu_frac)
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
            "workload": "fp8 linear-layer fwd+dgrad+wgrad (M=4096 tokens, K=7168, N=2048) + MoE grouped fprop "
                        "(16384 tokens, 32 experts, 2048x7168), incl. all online quantization",
            "gemm_gflop_per_step": round(gemm_flops / 1e9, 2),
            "value_definition": "useful GEMM FLOPs of the step / step time (quantizers inside the timed step)",
        },
        "roofline": roof,
        "kernels": kernels,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
