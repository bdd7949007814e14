"""Batched quantization (fp8q_quant_batch): several independent quantizations
in one grid.  Every job must give, bit for bit, what its single entry point
gives (which the other quantizer tests hold to the oracle), whatever the mix
of kinds, dtypes, shapes and strides in the batch."""

import numpy as np
import pytest
import torch

import fp8_fine_grained_quant_amd as fq
import synth
from gpu_util import DEV, gpu, log
from special_values import special_matrix

pytestmark = pytest.mark.gpu


def _same(a, b, what):
    if a.dtype == torch.float32:
        a, b = a.view(torch.int32), b.view(torch.int32)
    bad = int((a != b).sum())
    assert bad == 0, f"{what}: {bad} of {a.numel()} differ"


def _strided(rows, cols, dtype, fill, extra=16):
    """A [rows, cols] view with a wider, 16-byte-multiple row stride inside a guard-filled buffer."""
    esz = torch.tensor([], dtype=dtype).element_size()
    ld = cols + extra
    ld += (-(ld * esz)) % 16 // esz
    buf = torch.full((rows + 1, ld), fill, dtype=dtype, device=DEV)
    return buf, buf[:rows, :cols]


def _input(rows, cols, dtype, seed, special=False):
    a = special_matrix(rows, cols, seed, for_bf16=dtype == torch.bfloat16) if special else \
        synth.general(rows, cols, seed=seed, kind="t3", outlier_frac=0.01, outlier_mul=80.0).astype(np.float32)
    t = synth.to_bf16(a) if dtype == torch.bfloat16 else torch.from_numpy(a)
    return gpu(t)


def _outputs(kind, rows, cols, strided):
    """Output tensors of one job (views into guard-filled buffers when strided)."""
    mk = (lambda r, c, dt, fill: _strided(r, c, dt, fill)) if strided else \
        (lambda r, c, dt, fill: (None, torch.full((r, c), fill, dtype=dt, device=DEV)))
    out = {}
    if kind in ("act", "act_transpose"):
        out["q"] = mk(rows, cols, torch.uint8, 0x5A)
        out["scale"] = mk(rows, (cols + 127) // 128, torch.float32, -9.0)
    if kind == "weight":
        out["q"] = mk(rows, cols, torch.uint8, 0x5A)
        out["q_t"] = mk(cols, rows, torch.uint8, 0x5A)
        out["scale"] = mk((rows + 127) // 128, (cols + 127) // 128, torch.float32, -9.0)
    if kind in ("transpose", "act_transpose"):
        out["q_t"] = mk(cols, rows, torch.uint8, 0x5A)
        out["scale_t"] = mk(cols, (rows + 127) // 128, torch.float32, -9.0)
    return out


def _job_tuple(kind, x, o):
    v = lambda k: o[k][1]
    if kind == "act":
        return (kind, x, v("q"), v("scale"))
    if kind == "weight":
        return (kind, x, v("q"), v("q_t"), v("scale"))
    if kind == "transpose":
        return (kind, x, v("q_t"), v("scale_t"))
    return (kind, x, v("q"), v("scale"), v("q_t"), v("scale_t"))


def _single(kind, x):
    if kind == "act":
        q, s = fq.quant_act_1x128(x)
        return {"q": q, "scale": s}
    if kind == "weight":
        q, s, q_t = fq.quant_weight_128x128(x)
        return {"q": q, "q_t": q_t, "scale": s}
    if kind == "transpose":
        q_t, s_t = fq.quant_transpose(x)
        return {"q_t": q_t, "scale_t": s_t}
    q, s, q_t, s_t = fq.quant_act_transpose(x)
    return {"q": q, "scale": s, "q_t": q_t, "scale_t": s_t}


def _run(specs, strided=False):
    """specs: (kind, rows, cols, dtype, seed, special).  Runs them as one batch
    and each alone; compares every output bitwise and the guards."""
    xs = [_input(r, c, dt, seed, sp) for _, r, c, dt, seed, sp in specs]
    outs = [_outputs(sp[0], sp[1], sp[2], strided) for sp in specs]
    fq.fp8q_quant_batch([_job_tuple(sp[0], x, o) for sp, x, o in zip(specs, xs, outs)])
    refs = [_single(sp[0], x) for sp, x in zip(specs, xs)]
    torch.cuda.synchronize()
    for i, (sp, o, ref) in enumerate(zip(specs, outs, refs)):
        for k, (buf, view) in o.items():
            _same(view, ref[k], f"job {i} ({sp[0]} {sp[1]}x{sp[2]}) {k}")
            if buf is not None:
                fill = 0x5A if buf.dtype == torch.uint8 else -9.0
                r, c = view.shape
                assert torch.all(buf[r] == fill) and torch.all(buf[:r, c:] == fill), f"job {i} {k} guards"


def test_batch_linear_layer_forward_inputs():
    """The step's forward pair: X [4096,7168] bf16 (row and transposed codes)
    with W [2048,7168] fp32 (codes and transposed codes)."""
    x, w = synth.linear_x_w()
    xg, wg = gpu(x), gpu(w)
    o = dict(q=torch.empty(4096, 7168, dtype=torch.uint8, device=DEV),
             s=torch.empty(4096, 56, device=DEV), q_t=torch.empty(7168, 4096, dtype=torch.uint8, device=DEV),
             s_t=torch.empty(7168, 32, device=DEV), wq=torch.empty(2048, 7168, dtype=torch.uint8, device=DEV),
             wq_t=torch.empty(7168, 2048, dtype=torch.uint8, device=DEV), ws=torch.empty(16, 56, device=DEV))
    log("batch: X dual + W")
    fq.fp8q_quant_batch([("act_transpose", xg, o["q"], o["s"], o["q_t"], o["s_t"]),
                         ("weight", wg, o["wq"], o["wq_t"], o["ws"])])
    q, s, q_t, s_t = fq.quant_act_transpose(xg)
    wq, ws, wq_t = fq.quant_weight_128x128(wg)
    torch.cuda.synchronize()
    for a, b, what in ((o["q"], q, "X codes"), (o["s"], s, "X scales"), (o["q_t"], q_t, "X^T codes"),
                       (o["s_t"], s_t, "X^T scales"), (o["wq"], wq, "W codes"), (o["wq_t"], wq_t, "W^T codes"),
                       (o["ws"], ws, "W scales")):
        _same(a, b, what)


def test_batch_every_kind_dense():
    _run([("act", 4096, 2048, torch.bfloat16, 1, False), ("transpose", 4096, 2048, torch.bfloat16, 2, False),
          ("weight", 384, 1024, torch.float32, 3, False), ("act_transpose", 512, 768, torch.float32, 4, False)])


@pytest.mark.parametrize("strided", [False, True], ids=["dense", "strided"])
def test_batch_ragged_mixed(strided):
    # ragged against the 128 groups; row lengths stay 16-byte multiples as the quantizers require
    _run([("act", 257, 1008, torch.bfloat16, 5, False), ("weight", 144, 144, torch.float32, 6, False),
          ("transpose", 304, 80, torch.bfloat16, 7, False), ("act_transpose", 144, 16, torch.float32, 8, False),
          ("act", 1, 128, torch.float32, 9, False), ("weight", 304, 16, torch.bfloat16, 10, False)],
         strided=strided)


def test_batch_eight_jobs_special_values():
    _run([(k, 304, 13 * 128 + 48, dt, 20 + i, True)
          for i, (k, dt) in enumerate([("act", torch.float32), ("act", torch.bfloat16), ("weight", torch.float32),
                                       ("weight", torch.bfloat16), ("transpose", torch.float32),
                                       ("transpose", torch.bfloat16), ("act_transpose", torch.float32),
                                       ("act_transpose", torch.bfloat16)])])


def test_batch_moe_sized_act_and_weights():
    """Above 64 MB the codes are written non-temporally: X [16384,7168] with 3
    stacked experts of [2048,7168] (75 M codes) in one batch."""
    rng = np.random.Generator(np.random.PCG64(91))
    xm = gpu(synth.to_bf16(rng.standard_normal((16384, 7168), dtype=np.float32)))
    wm = gpu(torch.from_numpy(rng.standard_normal((3 * 2048, 7168), dtype=np.float32) * np.float32(0.02)))
    q = torch.empty(16384, 7168, dtype=torch.uint8, device=DEV)
    s = torch.empty(16384, 56, device=DEV)
    wq = torch.empty(3 * 2048, 7168, dtype=torch.uint8, device=DEV)
    ws = torch.empty(48, 56, device=DEV)
    log("batch: X_moe + 3 experts")
    fq.fp8q_quant_batch([("act", xm, q, s), ("weight", wm, wq, None, ws)])
    q1, s1 = fq.quant_act_1x128(xm)
    wq1, ws1, _ = fq.quant_weight_128x128(wm, transpose=False)
    torch.cuda.synchronize()
    _same(q, q1, "X codes")
    _same(s, s1, "X scales")
    _same(wq, wq1, "W codes")
    _same(ws, ws1, "W scales")
