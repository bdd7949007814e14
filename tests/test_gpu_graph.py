"""The entry points inside a captured HIP graph: they allocate nothing and
never wait, so a caller can capture a quantize-then-GEMM sequence once and
replay it (serving loops, launch-bound inner loops).  The graph's input is
overwritten between replays by ordinary eager work, and every replay's
outputs must equal, bit for bit, the same calls made eagerly on that input."""

import numpy as np
import pytest
import torch

import fp8_fine_grained_quant_amd as fq
import synth
from gpu_util import gpu, log

pytestmark = pytest.mark.gpu

M, N, K = 304, 256, 512  # M ragged against 128; q_t rows of M bytes need 16-byte strides


def _inputs(seed):
    x = synth.to_bf16(synth.general(M, K, seed=seed, kind="t3", outlier_frac=0.005, outlier_mul=30.0))
    return gpu(x)


def _sequence(x, w, o):
    """quantize X (both layouts) and W, then Fprop and a Dgrad-form product."""
    fq.fp8q_quant_act_transpose(x, o["xq"], o["xs"], o["xq_t"], o["xs_t"])
    fq.fp8q_quant_weight_128x128(w, o["wq"], o["wq_t"], o["ws"])
    fq.fp8q_gemm_fprop(o["xq"], o["xs"], o["wq"], o["ws"], o["y"])
    fq.fp8q_gemm_dgrad(o["yq"], o["ys"], o["wq_t"], o["ws"], o["dx"])


def _outputs(dev):
    e = lambda *s, dt=torch.uint8: torch.zeros(*s, dtype=dt, device=dev)
    o = dict(xq=e(M, K), xs=e(M, K // 128, dt=torch.float32), xq_t=e(K, M), xs_t=e(K, (M + 127) // 128, dt=torch.float32),
             wq=e(N, K), wq_t=e(K, N), ws=e(N // 128, K // 128, dt=torch.float32), y=e(M, N, dt=torch.bfloat16),
             dx=e(M, K, dt=torch.bfloat16))
    # the Dgrad-form product consumes fixed codes of a [M, N] tensor
    yq, ys = fq.quant_act_1x128(gpu(synth.to_bf16(synth.general(M, N, seed=5, kind="normal"))))
    o["yq"], o["ys"] = yq, ys
    return o


def _bits(t):
    return t.view(torch.uint8).cpu().numpy()


def test_graph_replays_match_eager():
    dev = torch.device("cuda:0")
    w = gpu(torch.from_numpy((synth.general(N, K, seed=3) * 0.02).astype(np.float32)))
    x_static = _inputs(10)
    g_out, e_out = _outputs(dev), _outputs(dev)
    _sequence(x_static, w, g_out)  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _sequence(x_static, w, g_out)
    torch.cuda.synchronize()
    for rep, seed in enumerate((11, 12, 13)):
        x_new = _inputs(seed)
        x_static.copy_(x_new)          # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _sequence(x_new, w, e_out)     # the same calls, eagerly
        torch.cuda.synchronize()
        for name in ("xq", "xs", "xq_t", "xs_t", "wq", "wq_t", "ws", "y", "dx"):
            assert np.array_equal(_bits(g_out[name]), _bits(e_out[name])), (rep, name)
        log(f"graph replay {rep}: every output equals the eager calls")
