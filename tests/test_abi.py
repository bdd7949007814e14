"""C-ABI checks that need no GPU: the library loads, exports every entry point
the header declares, and rejects bad arguments on the host (validation happens
before any launch, so these calls never reach the device)."""

import ctypes
import os
import re
import subprocess

import pytest

import fp8_fine_grained_quant_amd as fq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8q.h")

OK, NULL, SHAPE, STRIDE, ALIGN, DTYPE = 0, 1, 2, 3, 4, 5
A16 = 1 << 20          # a fake, 16-byte-aligned address (never dereferenced)


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(fp8q_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fq.LIB_PATH):
        pytest.fail("libfp8q.so is not built: run __graft_entry__.build()")
    return fq.load_library()


BOTH = pytest.mark.parametrize("path", [fq.LIB_PATH, fq.DEBUG_LIB_PATH], ids=["product", "debug"])


@BOTH
def test_exports_every_declared_symbol(lib, path):
    """Both builds (the product library and its FP8Q_DEBUG twin) load and
    export every entry point the header declares."""
    handle = lib if path == fq.LIB_PATH else fq.load_debug_library()
    names = declared_functions()
    assert set(names) == set(fq.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (fp8q_\w+)", out))
    for n in names:
        assert n in exported, n
        assert getattr(handle, n) is not None


@BOTH
def test_every_kernel_launch_stub_is_defined(lib, path):
    """A kernel whose host-side launch stub is missing makes dlopen fail on the
    GPU machine only; catch it here."""
    out = subprocess.run(["nm", "-D", path], capture_output=True, text=True).stdout
    undefined = [l for l in out.splitlines() if " U " in l and "__device_stub__" in l]
    assert not undefined, undefined[:3]
    # quantizers (1x128, 128x128, transposing, grouped, dual; MX rows and
    # transposing), FP8, exact and MX GEMM instantiations
    assert sum(1 for l in out.splitlines() if "__device_stub__" in l) >= 25


def test_gemm_tile_setting(lib):
    assert lib.fp8q_set_gemm_tile(3) == SHAPE
    assert lib.fp8q_set_gemm_tile(-1) == SHAPE
    for t in (1, 2, 0):
        assert lib.fp8q_set_gemm_tile(t) == OK


def test_status_strings(lib):
    for code, name in enumerate(fq._STATUS):
        assert fq.status_string(code).startswith(name)
    assert "unknown" in fq.status_string(99)


def test_quantizer_argument_errors(lib):
    f = lib.fp8q_quant_act_1x128
    assert f(A16, 0, -1, 128, 128, A16, 128, A16, 1, None) == SHAPE
    assert f(A16, 7, 4, 128, 128, A16, 128, A16, 1, None) == DTYPE
    assert f(None, 0, 4, 128, 128, A16, 128, A16, 1, None) == NULL
    assert f(A16, 0, 4, 128, 100, A16, 128, A16, 1, None) == STRIDE       # ld_x < cols
    assert f(A16, 0, 4, 128, 128, A16, 128, A16, 0, None) == STRIDE       # ld_s < groups
    assert f(A16 + 2, 0, 4, 128, 128, A16, 128, A16, 1, None) == ALIGN
    assert f(A16, 0, 4, 100, 100, A16, 112, A16, 1, None) == ALIGN        # 200-byte rows
    assert f(A16, 0, 0, 128, 128, None, 128, None, 1, None) == OK         # empty: no-op
    g = lib.fp8q_quant_weight_128x128
    assert g(A16, 1, 256, 256, 256, A16, 256, A16, 100, A16, 2, None) == STRIDE  # ld_qt < rows
    assert g(A16, 1, 256, 256, 256, A16, 256, A16 + 4, 256, A16, 2, None) == ALIGN
    assert g(A16, 1, 256, 256, 256, A16, 256, None, 0, A16, 1, None) == STRIDE   # ld_s < 2
    h = lib.fp8q_quant_transpose
    assert h(A16, 0, 300, 64, 64, A16, 256, A16, 3, None) == STRIDE      # ld_qt < rows
    assert h(A16, 0, 300, 64, 64, A16, 304, A16, 2, None) == STRIDE      # ld_st < 3


def test_gemm_argument_errors(lib):
    fp = lib.fp8q_gemm_fprop
    assert fp(A16, A16, A16, A16, 64, 128, 200, A16, 0, 128, None) == SHAPE  # K % 128
    assert fp(A16, A16, A16, A16, 64, 100, 256, A16, 0, 128, None) == SHAPE  # N % 128
    assert fp(A16, A16, A16, A16, 64, 128, 256, A16, 3, 128, None) == DTYPE
    assert fp(A16, None, A16, A16, 64, 128, 256, A16, 0, 128, None) == NULL
    assert fp(A16, A16, A16, A16, 64, 128, 256, A16, 0, 120, None) == STRIDE
    assert fp(A16, A16, A16, A16, 64, 128, 256, A16, 0, 132, None) == ALIGN  # 264-byte rows
    assert fp(A16 + 8, A16, A16, A16, 64, 128, 256, A16, 0, 128, None) == ALIGN
    assert fp(A16, A16, A16, A16, 0, 128, 256, None, 0, 128, None) == OK     # M = 0
    # outputs whose launch grid (ceil(rows / 256) x cols / 128 tiles) exceeds 2^31 - 1: rejected on the host
    big_m, big_n = (1 << 31) - 1, (1 << 31) - 128
    assert fp(A16, A16, A16, A16, big_m, big_n, 128, A16, 0, big_n, None) == SHAPE
    assert lib.fp8q_gemm_dgrad(A16, A16, A16, A16, big_m, 128, big_n, A16, 0, big_n, None) == SHAPE
    assert lib.fp8q_gemm_wgrad(A16, A16, A16, A16, 128, big_m, big_n, A16, big_n, 0, None) == SHAPE
    assert lib.fp8q_gemm_mx(A16, A16, 128, 4, A16, A16, 128, 4, big_m, big_n, 128, A16, 0, big_n, 0,
                            None) == SHAPE
    kmax = 1024 * 128  # every chunk's block scale is kept in LDS
    assert fp(A16, A16, A16, A16, 64, 128, kmax + 128, A16, 0, 128, None) == SHAPE
    assert fp(A16, A16, A16, A16, 64, 256, kmax + 128, A16, 0, 256, None) == SHAPE
    dg = lib.fp8q_gemm_dgrad
    assert dg(A16, A16, A16, A16, 64, kmax + 128, 256, A16, 0, 256, None) == SHAPE
    assert lib.fp8q_gemm_wgrad(A16, A16, A16, A16, kmax + 128, 64, 256, A16, 256, 0, None) == SHAPE
    assert dg(A16, A16, A16, A16, 64, 200, 256, A16, 0, 256, None) == SHAPE  # contraction % 128
    wg = lib.fp8q_gemm_wgrad
    assert wg(A16, A16, A16, A16, 200, 64, 256, A16, 256, 0, None) == SHAPE  # T % 128
    assert wg(A16, A16, A16, A16, 256, 64, 256, A16, 256, 2, None) == SHAPE  # accumulate flag
    assert wg(A16, A16, A16, A16, 256, 64, 256, A16, 254, 0, None) == STRIDE
    gg = lib.fp8q_grouped_gemm
    assert gg(A16, A16, A16, A16, A16, 0, 64, 128, 256, A16, 0, 128, None) == SHAPE  # E = 0
    assert gg(A16, A16, A16, A16, None, 4, 64, 128, 256, A16, 0, 128, None) == NULL
    assert gg(A16, A16, A16, A16, A16 + 2, 4, 64, 128, 256, A16, 0, 128, None) == ALIGN


def test_fused_quant_argument_errors(lib):
    fq_ = lib.fp8q_gemm_fprop_quant
    #          xq   xs   wq   ws   M   N    K    y    ldy  yq   ldyq ys  ldys ex
    assert fq_(A16, A16, A16, A16, 64, 256, 256, A16, 256, None, 256, A16, 2, 0, None) == NULL
    assert fq_(A16, A16, A16, A16, 64, 256, 256, A16, 256, A16, 256, None, 2, 0, None) == NULL
    assert fq_(A16, A16, A16, A16, 64, 256, 256, A16, 256, A16, 248, A16, 2, 0, None) == STRIDE  # ld_yq < N
    assert fq_(A16, A16, A16, A16, 64, 256, 256, A16, 256, A16, 256, A16, 1, 0, None) == STRIDE  # ld_ys < N/128
    assert fq_(A16, A16, A16, A16, 64, 256, 256, A16, 256, A16, 264, A16, 2, 0, None) == ALIGN   # ld_yq % 16
    assert fq_(A16, A16, A16, A16, 64, 256, 256, A16, 256, A16 + 8, 256, A16, 2, 0, None) == ALIGN
    assert fq_(A16, A16, A16, A16, 64, 256, 256, A16, 250, A16, 256, A16, 2, 0, None) == STRIDE  # ld_y < N
    assert fq_(A16, A16, A16, A16, 64, 256, 256, A16, 256, A16, 256, A16, 2, 2, None) == SHAPE   # exact flag
    assert fq_(A16, A16, A16, A16, 64, 200, 256, A16, 256, A16, 256, A16, 2, 0, None) == SHAPE   # N % 128
    assert fq_(A16, A16, A16, A16, 0, 256, 256, None, 256, None, 256, None, 2, 0, None) == OK    # M = 0
    dq = lib.fp8q_gemm_dgrad_quant
    #         dyq  dys  wq_t ws   M   N    K    dx   ldx  dxq  ldq  dxs lds ex
    assert dq(A16, A16, A16, A16, 64, 256, 384, A16, 384, None, 384, A16, 3, 0, None) == NULL
    assert dq(A16, A16, A16, A16, 64, 256, 384, A16, 384, A16, 256, A16, 3, 0, None) == STRIDE  # ld_dxq < K
    assert dq(A16, A16, A16, A16, 64, 256, 384, A16, 384, A16, 384, A16, 2, 0, None) == STRIDE  # ld_dxs < K/128
    assert dq(A16, A16, A16, A16, 64, 256, 384, A16, 384, A16, 384, A16, 3, -1, None) == SHAPE


def test_interval_study_argument_errors(lib):
    f = lib.fp8q_gemm_fprop_interval
    #        xq   xs   wq   ws   M   N    K    y    ldy  interval
    assert f(A16, A16, A16, A16, 64, 128, 512, A16, 128, 384, None) == SHAPE    # not a supported interval
    assert f(A16, A16, A16, A16, 64, 128, 512, A16, 128, 2048, None) == SHAPE
    assert f(A16, A16, A16, A16, 64, 128, 384, A16, 128, 128, None) == SHAPE    # K % 512
    assert f(A16, A16 + 4, A16, A16, 64, 128, 512, A16, 128, 0, None) == ALIGN  # xs 16-byte
    assert f(A16, A16, A16, A16, 64, 128, 512, A16, 120, 256, None) == STRIDE
    assert f(A16, None, A16, A16, 64, 128, 512, A16, 128, 512, None) == NULL
    assert f(A16, A16, A16, A16, 0, 128, 512, None, 128, 1024, None) == OK      # M = 0


def _job(kind, rows, cols, ld_x=None, **kw):
    j = fq.QuantJob()
    j.kind, j.xt, j.x, j.rows, j.cols = kind, 0, A16, rows, cols
    j.ld_x = cols if ld_x is None else ld_x
    j.q, j.ld_q, j.scale, j.ld_s = A16, cols, A16, (cols + 127) // 128
    j.q_t, j.ld_qt, j.scale_t, j.ld_st = A16, rows, A16, (rows + 127) // 128
    for k, v in kw.items():
        setattr(j, k, v)
    return j


def _batch(lib, *jobs):
    arr = (fq.QuantJob * max(1, len(jobs)))(*jobs)
    return lib.fp8q_quant_batch(ctypes.cast(arr, ctypes.c_void_p), len(jobs), None)


def test_quant_batch_argument_errors(lib):
    import ctypes as C
    assert lib.fp8q_quant_batch(None, 0, None) == OK
    assert lib.fp8q_quant_batch(None, 1, None) == NULL
    assert lib.fp8q_quant_batch(None, 9, None) == SHAPE                       # more than 8 jobs
    assert lib.fp8q_quant_batch(None, -1, None) == SHAPE
    assert C.sizeof(fq.QuantJob) == 4 + 4 + 8 * 12
    assert _batch(lib, _job(4, 128, 128)) == SHAPE                            # unknown kind
    assert _batch(lib, _job(0, 128, 128, xt=9)) == DTYPE
    # the first invalid job decides; nothing is launched
    assert _batch(lib, _job(0, 128, 128, ld_x=100), _job(1, 128, 128, q=None)) == STRIDE
    assert _batch(lib, _job(0, 128, 128, q=None), _job(1, 128, 128, ld_x=100)) == NULL
    assert _batch(lib, _job(1, 256, 256, ld_qt=100)) == STRIDE                # weight q_t narrower than rows
    assert _batch(lib, _job(2, 300, 64, ld_qt=256)) == STRIDE                 # transpose: ld_qt < rows
    assert _batch(lib, _job(3, 300, 64, ld_qt=304, ld_st=2)) == STRIDE        # dual: ld_st < 3
    assert _batch(lib, _job(3, 300, 64, ld_q=64, ld_s=1, scale=A16 + 2)) == ALIGN
    assert _batch(lib, _job(0, 0, 128, x=None, q=None, scale=None)) == OK     # empty jobs are skipped


def test_grouped_backward_argument_errors(lib):
    tg = lib.fp8q_quant_transpose_grouped
    # rows 300, E 4: capacity 128 * (2 + 4) = 768 token columns, 6 scale columns
    assert tg(A16, 0, 300, 64, 64, A16, 0, A16, 768, A16, 6, None) == SHAPE    # E = 0
    assert tg(A16, 0, 300, 64, 64, A16, 4, A16, 640, A16, 6, None) == STRIDE   # ld_qt < capacity
    assert tg(A16, 0, 300, 64, 64, A16, 4, A16, 768, A16, 5, None) == STRIDE   # ld_st < capacity/128
    assert tg(A16, 0, 300, 64, 64, None, 4, A16, 768, A16, 6, None) == NULL
    assert tg(A16, 0, 0, 64, 64, None, 4, None, 768, None, 6, None) == OK      # empty: no-op
    gd = lib.fp8q_grouped_gemm_dgrad
    assert gd(A16, A16, A16, A16, A16, 4, 64, 200, 256, A16, 0, 256, None) == SHAPE  # N % 128
    assert gd(A16, A16, A16, A16, None, 4, 64, 256, 256, A16, 0, 256, None) == NULL
    assert gd(A16, A16, A16, A16, A16, 0, 64, 256, 256, A16, 0, 256, None) == SHAPE  # E = 0
    # launch grid (ceil(M_total / 256) + E) * (N / 128) one past 2^31 - 1: rejected before any launch
    m_edge = 256 * 8388606 + 1
    assert gd(A16, A16, A16, A16, A16, 1, m_edge, 128, 32768, A16, 0, 32768, None) == SHAPE
    assert lib.fp8q_grouped_gemm(A16, A16, A16, A16, A16, 1, m_edge, 32768, 128, A16, 0, 32768, None) == SHAPE
    assert lib.fp8q_grouped_gemm_mx(A16, A16, A16, A16, A16, 1, m_edge, 32768, 128, A16, 0, 32768, None) == SHAPE
    # stacked transposed weights wider than 32-bit buffer offsets cover for 256 rows: one step past the bound
    # (E*N = 2^23, against the bound (2^31 - 1) / 256 = 2^23 - 1)
    assert gd(A16, A16, A16, A16, A16, 64, 64, 1 << 17, 256, A16, 0, 256, None) == SHAPE
    assert gd(A16, A16, A16, A16, A16, 65536, 64, 128, 256, A16, 0, 256, None) == SHAPE
    gw = lib.fp8q_grouped_gemm_wgrad
    assert gw(A16, A16, A16, A16, A16, 4, 300, 128, 256, 640, A16, 0, None) == STRIDE  # ld_t < 768
    # a padded token stride past what 32-bit buffer offsets cover for 256 rows (the next multiple of 128)
    ld_big = (((1 << 31) - 1) // 256 // 128 + 1) * 128
    assert gw(A16, A16, A16, A16, A16, 4, 300, 128, 256, ld_big, A16, 0, None) == SHAPE
    assert gw(A16, A16, A16, A16, A16, 4, 300, 128, 256, 800, A16, 0, None) == ALIGN   # ld_t % 128
    assert gw(A16, A16, A16, A16, A16, 4, 300, 128, 200, 768, A16, 0, None) == SHAPE   # K % 128
    assert gw(A16, A16, A16, A16, A16, 4, 300, 128, 256, 768, A16, 2, None) == SHAPE   # accumulate flag
    assert gw(A16, A16, A16, A16, A16, 4, 300, 0, 256, 768, A16, 0, None) == OK        # N = 0


def test_mx_argument_errors(lib):
    q = lib.fp8q_quant_mx_1x32
    assert q(A16, 0, 4, 128, 128, A16, 128, A16, 3, None) == STRIDE       # ld_s < 4 blocks
    assert q(A16, 0, 4, 100, 100, A16, 112, A16, 4, None) == ALIGN        # 200-byte rows
    assert q(A16, 2, 4, 128, 128, A16, 128, A16, 4, None) == DTYPE
    assert q(A16, 0, 0, 128, 128, None, 128, None, 4, None) == OK         # empty: no-op
    t = lib.fp8q_quant_mx_transpose
    assert t(A16, 0, 300, 64, 64, A16, 304, A16, 9, None, 0, None, 0, None) == STRIDE    # ld_st < 10
    assert t(A16, 0, 300, 64, 64, A16, 304, A16, 10, A16, 64, None, 0, None) == NULL     # q without s
    assert t(A16, 0, 300, 64, 64, A16, 304, A16, 10, A16, 64, A16, 1, None) == STRIDE    # ld_s < 2
    g = lib.fp8q_gemm_mx
    #        aq   as   lda  ldsa bq   bs   ldb  ldsb M   N    K    c    ct ldc acc
    assert g(A16, A16, 256, 8, A16, A16, 256, 8, 64, 128, 200, A16, 0, 128, 0, None) == SHAPE   # K % 128
    assert g(A16, A16, 256, 8, A16, A16, 256, 8, 64, 100, 256, A16, 0, 128, 0, None) == SHAPE   # N % 128
    assert g(A16, A16, 256, 8, A16, A16, 256, 8, 64, 128, 256, A16, 0, 128, 1, None) == DTYPE   # += into BF16
    assert g(A16, A16, 256, 8, A16, A16, 256, 8, 64, 128, 256, A16, 1, 128, 2, None) == SHAPE   # flag
    assert g(A16, A16, 256, 7, A16, A16, 256, 8, 64, 128, 256, A16, 0, 128, 0, None) == STRIDE  # ld_sa < K/32
    assert g(A16, A16, 248, 8, A16, A16, 256, 8, 64, 128, 256, A16, 0, 128, 0, None) == STRIDE  # lda < K
    assert g(A16, A16, 264, 8, A16, A16, 256, 8, 64, 128, 256, A16, 0, 128, 0, None) == ALIGN   # lda % 16
    assert g(A16, A16, 256, 10, A16, A16, 256, 8, 64, 128, 256, A16, 0, 128, 0, None) == ALIGN  # ld_sa % 4
    assert g(A16, A16 + 2, 256, 8, A16, A16, 256, 8, 64, 128, 256, A16, 0, 128, 0, None) == ALIGN
    assert g(A16, None, 256, 8, A16, A16, 256, 8, 64, 128, 256, A16, 0, 128, 0, None) == NULL
    assert g(A16, A16, 256, 8, A16, A16, 256, 8, 0, 128, 256, None, 0, 128, 0, None) == OK      # M = 0
    gg = lib.fp8q_grouped_gemm_mx
    #         xq   xs   wq   ws   off  E  M   N    K    y    yt ldy
    assert gg(A16, A16, A16, A16, A16, 0, 64, 128, 256, A16, 0, 128, None) == SHAPE     # E = 0
    assert gg(A16, A16, A16, A16, A16, 4, 64, 100, 256, A16, 0, 128, None) == SHAPE     # N % 128
    assert gg(A16, A16, A16, A16, A16, 4, 64, 128, 200, A16, 0, 128, None) == SHAPE     # K % 128
    assert gg(A16, A16, A16, A16, A16, 4, 64, 128, 1024 * 128 + 128, A16, 0, 128, None) == SHAPE  # K max
    assert gg(A16, A16, A16, A16, A16, 4, 64, 128, 256, A16, 2, 128, None) == DTYPE
    assert gg(A16, A16, A16, A16, None, 4, 64, 128, 256, A16, 0, 128, None) == NULL     # offsets
    assert gg(A16 + 4, A16, A16, A16, A16, 4, 64, 128, 256, A16, 0, 128, None) == ALIGN  # codes 16-byte
    assert gg(A16, A16 + 2, A16, A16, A16, 4, 64, 128, 256, A16, 0, 128, None) == ALIGN  # scales 4-byte
    assert gg(None, None, None, None, None, 4, 0, 128, 256, None, 0, 128, None) == OK    # M_total = 0
    gd = lib.fp8q_grouped_gemm_mx_dgrad
    #         dyq  dys  wq_t ws_t off  E  M   N    K    dx   t  ldx
    assert gd(A16, A16, A16, A16, A16, 0, 64, 128, 256, A16, 0, 256, None) == SHAPE     # E = 0
    assert gd(A16, A16, A16, A16, A16, 4, 64, 200, 256, A16, 0, 256, None) == SHAPE     # N % 128
    assert gd(A16, A16, A16, A16, A16, 4, 64, 128, 200, A16, 0, 256, None) == SHAPE     # K % 128
    assert gd(A16, A16, A16, A16, A16, 65536, 64, 1 << 15, 256, A16, 0, 256, None) == SHAPE  # E*N too large
    assert gd(A16, A16, A16, A16, A16, 4, 64, 128, 256, A16, 0, 128, None) == STRIDE    # ld_dx < K
    assert gd(A16, A16, None, A16, A16, 4, 64, 128, 256, A16, 0, 256, None) == NULL
    assert gd(A16, A16, A16, A16 + 1, A16, 4, 64, 128, 256, A16, 0, 256, None) == ALIGN
    assert gd(None, None, None, None, None, 4, 0, 128, 256, None, 0, 256, None) == OK    # M_total = 0


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(4, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fq.quant_act_1x128(x)


def test_header_compiles_as_c(tmp_path):
    src = tmp_path / "t.c"
    src.write_text('#include "fp8q.h"\nint main(void){ return (int)FP8Q_OK; }\n')
    res = subprocess.run(["gcc", "-std=c99", "-fsyntax-only", "-I", os.path.join(ROOT, "include"),
                          "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__", str(src)],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
