// C ABI of libfp8q: host-side argument validation, then the asynchronous
// launch on the caller's stream.  Nothing here allocates, synchronises,
// prints or throws.  The entry points and their rules are documented in
// include/fp8q.h.  (Built with FP8Q_DEBUG, as libfp8q_debug.so, the grouped
// entry points also read the expert offsets back and check them, which
// synchronises the stream.)

#include "../../include/fp8q.h"
#include "launch.h"

#include <atomic>
#include <stdint.h>
#ifdef FP8Q_DEBUG
#include <vector>
#endif

namespace fp8q {

namespace {
std::atomic<int> g_gemm_tile{0};  // fp8q_set_gemm_tile
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];  // compute units per device, 0 = not yet queried
}  // namespace

int gemm_tile_setting() { return g_gemm_tile.load(std::memory_order_relaxed); }

int device_cu_count() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  cus = g_cus[dev].load(std::memory_order_relaxed);
  if (cus > 0) return cus;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  g_cus[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

}  // namespace fp8q

namespace {

using fp8q::GemmArgs;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int esize(fp8q_dtype t) { return t == FP8Q_BF16 ? 2 : 4; }
inline bool valid_dtype(fp8q_dtype t) { return t == FP8Q_BF16 || t == FP8Q_F32; }
inline fp8q_status launched(hipError_t e) { return e == hipSuccess ? FP8Q_OK : FP8Q_ERR_LAUNCH; }

constexpr int64_t kMaxGroups = (int64_t(1) << 31) - 1;

// Expert offsets live on the device and the product library never reads
// them: malformed offsets are undefined behaviour there.  The FP8Q_DEBUG
// build copies them to the host (after the work already on the stream) and
// rejects any that break the rule offsets[0] = 0, non-decreasing,
// offsets[E] = M_total, with FP8Q_ERR_SHAPE and nothing enqueued.
fp8q_status debug_check_offsets(const int32_t* offsets, int64_t E, int64_t M_total, hipStream_t stream) {
#ifdef FP8Q_DEBUG
  std::vector<int32_t> h((size_t)E + 1);
  if (hipMemcpyAsync(h.data(), offsets, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return FP8Q_ERR_LAUNCH;
  if (h[0] != 0 || h[(size_t)E] != M_total) return FP8Q_ERR_SHAPE;
  for (size_t e = 0; e < (size_t)E; ++e)
    if (h[e + 1] < h[e]) return FP8Q_ERR_SHAPE;
#else
  (void)offsets; (void)E; (void)M_total; (void)stream;
#endif
  return FP8Q_OK;
}
constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxContraction = 1024 * 128;  // the GEMM keeps one scale per chunk in LDS

// Checks shared by the three quantizers: input [rows, cols] with stride ld_in
// (elements of size in_es), code output with stride ld_out bytes covering
// out_len bytes per row, scale array of scale_rows x scale_cols with stride
// ld_s.
fp8q_status check_quant(const void* in, int in_es, int64_t rows, int64_t cols, int64_t ld_in,
                        const void* out, int64_t ld_out, int64_t out_len, const void* s, int64_t ld_s,
                        int64_t scale_cols) {
  if (rows < 0 || cols < 0 || rows > kMaxDim || cols > kMaxDim) return FP8Q_ERR_SHAPE;
  if (rows == 0 || cols == 0) return FP8Q_OK;
  if (!in || !out || !s) return FP8Q_ERR_NULL;
  if (ld_in < cols || ld_out < out_len || ld_s < scale_cols) return FP8Q_ERR_STRIDE;
  if (!aligned16(in) || !aligned16(out) || !aligned4(s)) return FP8Q_ERR_ALIGN;
  if ((ld_in * in_es) % 16 != 0 || ld_out % 16 != 0) return FP8Q_ERR_ALIGN;
  return FP8Q_OK;
}

fp8q_status check_gemm_out(const void* y, fp8q_dtype yt, int64_t ld_y, int64_t ncols) {
  if (!valid_dtype(yt)) return FP8Q_ERR_DTYPE;
  if (!y) return FP8Q_ERR_NULL;
  if (ld_y < ncols) return FP8Q_ERR_STRIDE;
  if (!aligned16(y) || (ld_y * esize(yt)) % 16 != 0) return FP8Q_ERR_ALIGN;
  return FP8Q_OK;
}

}  // namespace

extern "C" {

fp8q_status fp8q_set_gemm_tile(int tile) {
  if (tile < 0 || tile > 2) return FP8Q_ERR_SHAPE;
  fp8q::g_gemm_tile.store(tile, std::memory_order_relaxed);
  return FP8Q_OK;
}

const char* fp8q_status_string(fp8q_status s) {
  switch (s) {
    case FP8Q_OK: return "FP8Q_OK";
    case FP8Q_ERR_NULL: return "FP8Q_ERR_NULL: required pointer is NULL";
    case FP8Q_ERR_SHAPE: return "FP8Q_ERR_SHAPE: negative size or size rule broken";
    case FP8Q_ERR_STRIDE: return "FP8Q_ERR_STRIDE: leading dimension smaller than the row length";
    case FP8Q_ERR_ALIGN: return "FP8Q_ERR_ALIGN: pointer or row stride not aligned as required";
    case FP8Q_ERR_DTYPE: return "FP8Q_ERR_DTYPE: unsupported element type";
    case FP8Q_ERR_LAUNCH: return "FP8Q_ERR_LAUNCH: the HIP runtime refused a launch";
  }
  return "FP8Q: unknown status";
}

fp8q_status fp8q_quant_act_1x128(const void* x, fp8q_dtype xt, int64_t rows, int64_t cols, int64_t ld_x,
                                 uint8_t* q, int64_t ld_q, float* scale, int64_t ld_s, hipStream_t stream) {
  if (!valid_dtype(xt)) return FP8Q_ERR_DTYPE;
  const fp8q_status c = check_quant(x, esize(xt), rows, cols, ld_x, q, ld_q, cols, scale, ld_s, cdiv(cols, 128));
  if (c != FP8Q_OK || rows == 0 || cols == 0) return c;
  if (rows * cdiv(cols, 128) > kMaxGroups) return FP8Q_ERR_SHAPE;
  return launched(fp8q::launch_quant_act(x, xt == FP8Q_BF16, rows, cols, ld_x, q, ld_q, scale, ld_s, stream));
}

fp8q_status fp8q_quant_weight_128x128(const void* w, fp8q_dtype wt, int64_t rows, int64_t cols, int64_t ld_w,
                                      uint8_t* q, int64_t ld_q, uint8_t* q_t, int64_t ld_qt,
                                      float* scale, int64_t ld_s, hipStream_t stream) {
  if (!valid_dtype(wt)) return FP8Q_ERR_DTYPE;
  fp8q_status c = check_quant(w, esize(wt), rows, cols, ld_w, q, ld_q, cols, scale, ld_s, cdiv(cols, 128));
  if (c != FP8Q_OK || rows == 0 || cols == 0) return c;
  if (q_t) {
    if (ld_qt < rows) return FP8Q_ERR_STRIDE;
    if (!aligned16(q_t) || ld_qt % 16 != 0) return FP8Q_ERR_ALIGN;
  }
  if (cdiv(rows, 128) > 65535) return FP8Q_ERR_SHAPE;  // grid y limit
  return launched(fp8q::launch_quant_weight(w, wt == FP8Q_BF16, rows, cols, ld_w, q, ld_q, q_t, ld_qt, scale,
                                            ld_s, stream));
}

fp8q_status fp8q_quant_transpose(const void* x, fp8q_dtype xt, int64_t rows, int64_t cols, int64_t ld_x,
                                 uint8_t* q_t, int64_t ld_qt, float* scale_t, int64_t ld_st, hipStream_t stream) {
  if (!valid_dtype(xt)) return FP8Q_ERR_DTYPE;
  const fp8q_status c =
      check_quant(x, esize(xt), rows, cols, ld_x, q_t, ld_qt, rows, scale_t, ld_st, cdiv(rows, 128));
  if (c != FP8Q_OK || rows == 0 || cols == 0) return c;
  if (cdiv(rows, 128) > 65535) return FP8Q_ERR_SHAPE;
  return launched(
      fp8q::launch_quant_transpose(x, xt == FP8Q_BF16, rows, cols, ld_x, q_t, ld_qt, scale_t, ld_st, stream));
}

fp8q_status fp8q_quant_act_transpose(const void* x, fp8q_dtype xt, int64_t rows, int64_t cols, int64_t ld_x,
                                     uint8_t* q, int64_t ld_q, float* scale, int64_t ld_s, uint8_t* q_t,
                                     int64_t ld_qt, float* scale_t, int64_t ld_st, hipStream_t stream) {
  if (!valid_dtype(xt)) return FP8Q_ERR_DTYPE;
  fp8q_status c = check_quant(x, esize(xt), rows, cols, ld_x, q, ld_q, cols, scale, ld_s, cdiv(cols, 128));
  if (c != FP8Q_OK || rows == 0 || cols == 0) return c;
  c = check_quant(x, esize(xt), rows, cols, ld_x, q_t, ld_qt, rows, scale_t, ld_st, cdiv(rows, 128));
  if (c != FP8Q_OK) return c;
  if (cdiv(rows, 128) > 65535) return FP8Q_ERR_SHAPE;
  return launched(fp8q::launch_quant_act_transpose(x, xt == FP8Q_BF16, rows, cols, ld_x, q, ld_q, scale, ld_s,
                                                   q_t, ld_qt, scale_t, ld_st, stream));
}

fp8q_status fp8q_quant_transpose_grouped(const void* x, fp8q_dtype xt, int64_t rows, int64_t cols, int64_t ld_x,
                                         const int32_t* offsets, int64_t E, uint8_t* q_t, int64_t ld_qt,
                                         float* scale_t, int64_t ld_st, hipStream_t stream) {
  if (!valid_dtype(xt)) return FP8Q_ERR_DTYPE;
  if (E < 1 || E > 65536) return FP8Q_ERR_SHAPE;
  if (rows < 0 || rows > kMaxDim) return FP8Q_ERR_SHAPE;
  const int64_t cap = 128 * (rows / 128 + E);  // padded token capacity
  const fp8q_status c = check_quant(x, esize(xt), rows, cols, ld_x, q_t, ld_qt, cap, scale_t, ld_st, cap / 128);
  if (c != FP8Q_OK || rows == 0 || cols == 0) return c;
  if (!offsets) return FP8Q_ERR_NULL;
  if (!aligned4(offsets)) return FP8Q_ERR_ALIGN;
  if (cap / 128 > 65535) return FP8Q_ERR_SHAPE;  // grid y limit
  if (const fp8q_status d = debug_check_offsets(offsets, E, rows, stream); d != FP8Q_OK) return d;
  return launched(fp8q::launch_quant_transpose_grouped(x, xt == FP8Q_BF16, rows, cols, ld_x, offsets, E, q_t, ld_qt,
                                                       scale_t, ld_st, stream));
}

fp8q_status fp8q_quant_batch(const fp8q_quant_job* jobs, int n_jobs, hipStream_t stream) {
  if (n_jobs < 0 || n_jobs > FP8Q_MAX_QUANT_JOBS) return FP8Q_ERR_SHAPE;
  if (n_jobs == 0) return FP8Q_OK;
  if (!jobs) return FP8Q_ERR_NULL;
  fp8q::QuantJob qj[FP8Q_MAX_QUANT_JOBS];
  for (int i = 0; i < n_jobs; ++i) {
    const fp8q_quant_job& J = jobs[i];
    const fp8q_dtype xt = (fp8q_dtype)J.xt;
    if (J.kind < FP8Q_QUANT_ACT_1X128 || J.kind > FP8Q_QUANT_ACT_TRANSPOSE) return FP8Q_ERR_SHAPE;
    if (!valid_dtype(xt)) return FP8Q_ERR_DTYPE;
    fp8q_status c = FP8Q_OK;
    const int64_t rows = J.rows, cols = J.cols;
    if (J.kind != FP8Q_QUANT_TRANSPOSE)
      c = check_quant(J.x, esize(xt), rows, cols, J.ld_x, J.q, J.ld_q, cols, J.scale, J.ld_s, cdiv(cols, 128));
    if (c == FP8Q_OK && (J.kind == FP8Q_QUANT_TRANSPOSE || J.kind == FP8Q_QUANT_ACT_TRANSPOSE))
      c = check_quant(J.x, esize(xt), rows, cols, J.ld_x, J.q_t, J.ld_qt, rows, J.scale_t, J.ld_st, cdiv(rows, 128));
    if (c == FP8Q_OK && J.kind == FP8Q_QUANT_WEIGHT_128X128 && rows > 0 && cols > 0 && J.q_t) {
      if (J.ld_qt < rows) c = FP8Q_ERR_STRIDE;
      else if (!aligned16(J.q_t) || J.ld_qt % 16 != 0) c = FP8Q_ERR_ALIGN;
    }
    if (c == FP8Q_OK && rows > 0 && cols > 0 && rows * cdiv(cols, 128) > kMaxGroups) c = FP8Q_ERR_SHAPE;
    if (c != FP8Q_OK) return c;
    fp8q::QuantJob& q = qj[i];
    q.kind = J.kind; q.x_bf16 = xt == FP8Q_BF16; q.x = J.x; q.rows = rows; q.cols = cols; q.ld_x = J.ld_x;
    const bool rows_out = J.kind != FP8Q_QUANT_TRANSPOSE, t_out = J.kind != FP8Q_QUANT_ACT_1X128;
    q.q = rows_out ? J.q : nullptr; q.ld_q = J.ld_q; q.s = rows_out ? J.scale : nullptr; q.ld_s = J.ld_s;
    q.q_t = t_out ? J.q_t : nullptr; q.ld_qt = J.ld_qt;
    q.s_t = t_out ? J.scale_t : nullptr; q.ld_st = J.ld_st;
  }
  if (fp8q::quant_batch_blocks(qj, n_jobs) > kMaxGroups) return FP8Q_ERR_SHAPE;  // one grid dimension
  return launched(fp8q::launch_quant_batch(qj, n_jobs, stream));
}

}  // extern "C"

// The fused output quantization's arguments: codes [rows, ncols] (row stride
// ld_q bytes) and scales [rows, ncols/128] (row stride ld_s).
static fp8q_status check_quant_out(const uint8_t* q, int64_t ld_q, const float* s, int64_t ld_s, int64_t ncols) {
  if (!q || !s) return FP8Q_ERR_NULL;
  if (ld_q < ncols || ld_s < ncols / 128) return FP8Q_ERR_STRIDE;
  if (!aligned16(q) || ld_q % 16 != 0 || !aligned4(s)) return FP8Q_ERR_ALIGN;
  return FP8Q_OK;
}

static fp8q_status fp8q_gemm_fprop_impl(int exact, const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                            int64_t M, int64_t N, int64_t K, void* y, fp8q_dtype yt, int64_t ld_y,
                            hipStream_t stream, uint8_t* qo = nullptr, int64_t ld_qo = 0, float* so = nullptr,
                            int64_t ld_so = 0, bool quant_out = false) {
  if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return FP8Q_ERR_SHAPE;
  if (N % 128 != 0 || K % 128 != 0 || K > kMaxContraction) return FP8Q_ERR_SHAPE;
  if (!valid_dtype(yt)) return FP8Q_ERR_DTYPE;
  if (M == 0 || N == 0) return FP8Q_OK;
  if (K == 0) return FP8Q_ERR_SHAPE;  // an empty contraction would leave Y undefined
  if (!xq || !xs || !wq || !ws) return FP8Q_ERR_NULL;
  if (quant_out) {
    const fp8q_status c = check_quant_out(qo, ld_qo, so, ld_so, N);
    if (c != FP8Q_OK) return c;
  }
  if (!quant_out || y != nullptr) {
    const fp8q_status c = check_gemm_out(y, yt, ld_y, N);
    if (c != FP8Q_OK) return c;
  }
  if (!aligned16(xq) || !aligned16(wq) || !aligned4(xs) || !aligned4(ws)) return FP8Q_ERR_ALIGN;
  if (cdiv(M, 256) * (N / 128) > kMaxGroups) return FP8Q_ERR_SHAPE;  // the launch grid
  GemmArgs a{};
  a.A = xq; a.B = wq; a.sa = xs; a.sb = ws; a.C = y;
  a.lda = K; a.ldb = K; a.ld_sa = K / 128; a.sb_rs = K / 128; a.sb_cs = 1; a.ldc = ld_y;
  a.M = M; a.N = N; a.K = K;
  a.sb_mode = fp8q::kSbBlock; a.out_f32 = yt == FP8Q_F32; a.accumulate = 0; a.exact = exact;
  a.qo = qo; a.ld_qo = ld_qo; a.so = so; a.ld_so = ld_so;
  return launched(fp8q::launch_gemm(a, stream));
}

static fp8q_status fp8q_gemm_dgrad_impl(int exact, const uint8_t* dyq, const float* dys, const uint8_t* wq_t, const float* ws,
                            int64_t M, int64_t N, int64_t K, void* dx, fp8q_dtype dxt, int64_t ld_dx,
                            hipStream_t stream, uint8_t* qo = nullptr, int64_t ld_qo = 0, float* so = nullptr,
                            int64_t ld_so = 0, bool quant_out = false) {
  if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return FP8Q_ERR_SHAPE;
  if (N % 128 != 0 || K % 128 != 0 || N > kMaxContraction) return FP8Q_ERR_SHAPE;
  if (!valid_dtype(dxt)) return FP8Q_ERR_DTYPE;
  if (M == 0 || K == 0) return FP8Q_OK;
  if (N == 0) return FP8Q_ERR_SHAPE;
  if (!dyq || !dys || !wq_t || !ws) return FP8Q_ERR_NULL;
  if (quant_out) {
    const fp8q_status c = check_quant_out(qo, ld_qo, so, ld_so, K);
    if (c != FP8Q_OK) return c;
  }
  if (!quant_out || dx != nullptr) {
    const fp8q_status c = check_gemm_out(dx, dxt, ld_dx, K);
    if (c != FP8Q_OK) return c;
  }
  if (!aligned16(dyq) || !aligned16(wq_t) || !aligned4(dys) || !aligned4(ws)) return FP8Q_ERR_ALIGN;
  if (cdiv(M, 256) * (K / 128) > kMaxGroups) return FP8Q_ERR_SHAPE;  // the launch grid
  // NT form over the contraction axis N: A = dY [M, N], B = W^T codes [K, N];
  // the block scale of (output column k, chunk kb over N) is ws[kb, k/128].
  GemmArgs a{};
  a.A = dyq; a.B = wq_t; a.sa = dys; a.sb = ws; a.C = dx;
  a.lda = N; a.ldb = N; a.ld_sa = N / 128; a.sb_rs = 1; a.sb_cs = K / 128; a.ldc = ld_dx;
  a.M = M; a.N = K; a.K = N;
  a.sb_mode = fp8q::kSbBlock; a.out_f32 = dxt == FP8Q_F32; a.accumulate = 0; a.exact = exact;
  a.qo = qo; a.ld_qo = ld_qo; a.so = so; a.ld_so = ld_so;
  return launched(fp8q::launch_gemm(a, stream));
}

static fp8q_status fp8q_gemm_wgrad_impl(int exact, const uint8_t* dyq_t, const float* dys_t, const uint8_t* xq_t, const float* xs_t,
                            int64_t T, int64_t N, int64_t K, float* dw, int64_t ld_dw, int accumulate,
                            hipStream_t stream) {
  if (T < 0 || N < 0 || K < 0 || T > kMaxDim || N > kMaxDim || K > kMaxDim) return FP8Q_ERR_SHAPE;
  if (T % 128 != 0 || K % 128 != 0 || T > kMaxContraction) return FP8Q_ERR_SHAPE;
  if (accumulate != 0 && accumulate != 1) return FP8Q_ERR_SHAPE;
  if (N == 0 || K == 0) return FP8Q_OK;
  if (T == 0) return FP8Q_ERR_SHAPE;
  if (!dyq_t || !dys_t || !xq_t || !xs_t) return FP8Q_ERR_NULL;
  const fp8q_status c = check_gemm_out(dw, FP8Q_F32, ld_dw, K);
  if (c != FP8Q_OK) return c;
  if (!aligned16(dyq_t) || !aligned16(xq_t) || !aligned4(dys_t) || !aligned4(xs_t)) return FP8Q_ERR_ALIGN;
  if (cdiv(N, 256) * (K / 128) > kMaxGroups) return FP8Q_ERR_SHAPE;  // the launch grid
  // NT form over the tokens: A = dY^T codes [N, T], B = X^T codes [K, T], one
  // scale per row of each per 128 tokens.
  GemmArgs a{};
  a.A = dyq_t; a.B = xq_t; a.sa = dys_t; a.sb = xs_t; a.C = dw;
  a.lda = T; a.ldb = T; a.ld_sa = T / 128; a.sb_rs = T / 128; a.sb_cs = 1; a.ldc = ld_dw;
  a.M = N; a.N = K; a.K = T;
  a.sb_mode = fp8q::kSbRow; a.out_f32 = 1; a.accumulate = accumulate; a.exact = exact;
  return launched(fp8q::launch_gemm(a, stream));
}

static fp8q_status fp8q_grouped_gemm_impl(int exact, const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                              const int32_t* offsets, int64_t E, int64_t M_total, int64_t N, int64_t K,
                              void* y, fp8q_dtype yt, int64_t ld_y, hipStream_t stream) {
  if (E < 1 || E > 65536) return FP8Q_ERR_SHAPE;
  if (M_total < 0 || N < 0 || K < 0 || M_total > kMaxDim || N > kMaxDim || K > kMaxDim) return FP8Q_ERR_SHAPE;
  if (N % 128 != 0 || K % 128 != 0) return FP8Q_ERR_SHAPE;
  if (!valid_dtype(yt)) return FP8Q_ERR_DTYPE;
  if (M_total == 0 || N == 0) return FP8Q_OK;
  if (K == 0) return FP8Q_ERR_SHAPE;
  if (!xq || !xs || !wq || !ws || !offsets) return FP8Q_ERR_NULL;
  const fp8q_status c = check_gemm_out(y, yt, ld_y, N);
  if (c != FP8Q_OK) return c;
  if (!aligned16(xq) || !aligned16(wq) || !aligned4(xs) || !aligned4(ws) || !aligned4(offsets))
    return FP8Q_ERR_ALIGN;
  // the launch grid: a partial m-tile per expert on top of ceil(M_total / 256)
  if (((M_total + 255) / 256 + E) * (N / 128) > kMaxGroups) return FP8Q_ERR_SHAPE;
  if (const fp8q_status d = debug_check_offsets(offsets, E, M_total, stream); d != FP8Q_OK) return d;
  GemmArgs a{};
  a.A = xq; a.B = wq; a.sa = xs; a.sb = ws; a.C = y;
  a.lda = K; a.ldb = K; a.ld_sa = K / 128; a.sb_rs = K / 128; a.sb_cs = 1; a.ldc = ld_y;
  a.M = M_total; a.N = N; a.K = K;
  a.sb_mode = fp8q::kSbBlock; a.out_f32 = yt == FP8Q_F32; a.accumulate = 0; a.exact = exact;
  a.offsets = offsets; a.E = E; a.b_estride = N * K; a.sb_estride = (N / 128) * (K / 128);
  return launched(fp8q::launch_gemm(a, stream));
}


extern "C" {

fp8q_status fp8q_grouped_gemm_dgrad(const uint8_t* dyq, const float* dys, const uint8_t* wq_t, const float* ws,
                                    const int32_t* offsets, int64_t E, int64_t M_total, int64_t N, int64_t K,
                                    void* dx, fp8q_dtype dxt, int64_t ld_dx, hipStream_t stream) {
  if (E < 1 || E > 65536) return FP8Q_ERR_SHAPE;
  if (M_total < 0 || N < 0 || K < 0 || M_total > kMaxDim || N > kMaxDim || K > kMaxDim) return FP8Q_ERR_SHAPE;
  if (N % 128 != 0 || K % 128 != 0 || N > kMaxContraction) return FP8Q_ERR_SHAPE;
  // the kernels address 256 rows of the stacked transposed codes (E*N bytes
  // each) with 32-bit buffer offsets
  if (E * N > INT32_MAX / 256) return FP8Q_ERR_SHAPE;
  if (!valid_dtype(dxt)) return FP8Q_ERR_DTYPE;
  if (M_total == 0 || K == 0) return FP8Q_OK;
  if (N == 0) return FP8Q_ERR_SHAPE;
  if (!dyq || !dys || !wq_t || !ws || !offsets) return FP8Q_ERR_NULL;
  const fp8q_status c = check_gemm_out(dx, dxt, ld_dx, K);
  if (c != FP8Q_OK) return c;
  if (!aligned16(dyq) || !aligned16(wq_t) || !aligned4(dys) || !aligned4(ws) || !aligned4(offsets))
    return FP8Q_ERR_ALIGN;
  if (((M_total + 255) / 256 + E) * (K / 128) > kMaxGroups) return FP8Q_ERR_SHAPE;
  if (const fp8q_status d = debug_check_offsets(offsets, E, M_total, stream); d != FP8Q_OK) return d;
  // Per expert: the Dgrad NT form (A = dY rows of the expert, contraction N)
  // with B = W_e^T = columns [eN, (e+1)N) of the stacked transposed codes
  // [K, E*N], and the block scale of (output column k, chunk kb) at
  // ws[e*N/128 + kb, k/128].
  GemmArgs a{};
  a.A = dyq; a.B = wq_t; a.sa = dys; a.sb = ws; a.C = dx;
  a.lda = N; a.ldb = E * N; a.ld_sa = N / 128; a.sb_rs = 1; a.sb_cs = K / 128; a.ldc = ld_dx;
  a.M = M_total; a.N = K; a.K = N;
  a.sb_mode = fp8q::kSbBlock; a.out_f32 = dxt == FP8Q_F32; a.accumulate = 0; a.exact = 0;
  a.offsets = offsets; a.E = E; a.b_estride = N; a.sb_estride = (N / 128) * (K / 128);
  return launched(fp8q::launch_gemm(a, stream));
}

fp8q_status fp8q_grouped_gemm_wgrad(const uint8_t* dyq_t, const float* dys_t, const uint8_t* xq_t,
                                    const float* xs_t, const int32_t* offsets, int64_t E, int64_t M_total,
                                    int64_t N, int64_t K, int64_t ld_t, float* dw, int accumulate,
                                    hipStream_t stream) {
  if (E < 1 || E > 65536) return FP8Q_ERR_SHAPE;
  if (M_total < 0 || N < 0 || K < 0 || M_total > kMaxDim || N > kMaxDim || K > kMaxDim) return FP8Q_ERR_SHAPE;
  if (K % 128 != 0 || M_total > kMaxContraction) return FP8Q_ERR_SHAPE;
  if (accumulate != 0 && accumulate != 1) return FP8Q_ERR_SHAPE;
  if (N == 0 || K == 0) return FP8Q_OK;
  if (!dyq_t || !dys_t || !xq_t || !xs_t || !offsets || !dw) return FP8Q_ERR_NULL;
  const int64_t cap = 128 * (M_total / 128 + E);
  if (ld_t < cap) return FP8Q_ERR_STRIDE;
  if (ld_t % 128 != 0) return FP8Q_ERR_ALIGN;
  // the kernels address 256 operand rows (ld_t bytes each) with 32-bit buffer offsets
  if (ld_t > INT32_MAX / 256) return FP8Q_ERR_SHAPE;
  if (!aligned16(dyq_t) || !aligned16(xq_t) || !aligned16(dw) || !aligned4(dys_t) || !aligned4(xs_t) ||
      !aligned4(offsets))
    return FP8Q_ERR_ALIGN;
  if (E * ((N + 255) / 256) * (K / 128) > kMaxGroups) return FP8Q_ERR_SHAPE;
  if (const fp8q_status d = debug_check_offsets(offsets, E, M_total, stream); d != FP8Q_OK) return d;
  // Per expert: the Wgrad NT form over the expert's padded token chunks
  // (A = dY^T codes [N, ld_t], B = X^T codes [K, ld_t], one scale per row
  // per chunk), written to dw + e*N*K.
  GemmArgs a{};
  a.A = dyq_t; a.B = xq_t; a.sa = dys_t; a.sb = xs_t; a.C = dw;
  a.lda = ld_t; a.ldb = ld_t; a.ld_sa = ld_t / 128; a.sb_rs = ld_t / 128; a.sb_cs = 1; a.ldc = K;
  a.M = N; a.N = K; a.K = ld_t;
  a.sb_mode = fp8q::kSbRow; a.out_f32 = 1; a.accumulate = accumulate; a.exact = 0;
  a.offsets = offsets; a.E = E; a.b_estride = 0; a.sb_estride = 0;
  a.k_grouped = 1; a.c_estride = N * K;
  return launched(fp8q::launch_gemm(a, stream));
}

fp8q_status fp8q_gemm_fprop_quant(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws, int64_t M,
                                  int64_t N, int64_t K, void* y, int64_t ld_y, uint8_t* yq, int64_t ld_yq, float* ys,
                                  int64_t ld_ys, int exact, hipStream_t stream) {
  if (exact != 0 && exact != 1) return FP8Q_ERR_SHAPE;
  return fp8q_gemm_fprop_impl(exact, xq, xs, wq, ws, M, N, K, y, FP8Q_BF16, ld_y, stream, yq, ld_yq, ys, ld_ys, true);
}
fp8q_status fp8q_gemm_dgrad_quant(const uint8_t* dyq, const float* dys, const uint8_t* wq_t, const float* ws,
                                  int64_t M, int64_t N, int64_t K, void* dx, int64_t ld_dx, uint8_t* dxq,
                                  int64_t ld_dxq, float* dxs, int64_t ld_dxs, int exact, hipStream_t stream) {
  if (exact != 0 && exact != 1) return FP8Q_ERR_SHAPE;
  return fp8q_gemm_dgrad_impl(exact, dyq, dys, wq_t, ws, M, N, K, dx, FP8Q_BF16, ld_dx, stream, dxq, ld_dxq, dxs,
                              ld_dxs, true);
}
fp8q_status fp8q_gemm_fprop_interval(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                                     int64_t M, int64_t N, int64_t K, float* y, int64_t ld_y, int64_t interval,
                                     hipStream_t stream) {
  int chunks = -1;
  if (interval == 0) chunks = 0;
  else if (interval == 128 || interval == 256 || interval == 512 || interval == 1024) chunks = (int)(interval / 128);
  if (chunks < 0) return FP8Q_ERR_SHAPE;
  if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return FP8Q_ERR_SHAPE;
  if (N % 128 != 0 || K % 512 != 0 || K > kMaxContraction) return FP8Q_ERR_SHAPE;
  if (M == 0 || N == 0) return FP8Q_OK;
  if (K == 0) return FP8Q_ERR_SHAPE;
  if (!xq || !xs || !wq || !ws) return FP8Q_ERR_NULL;
  const fp8q_status c = check_gemm_out(y, FP8Q_F32, ld_y, N);
  if (c != FP8Q_OK) return c;
  if (!aligned16(xq) || !aligned16(wq) || !aligned16(xs) || !aligned4(ws)) return FP8Q_ERR_ALIGN;
  if (cdiv(M, 256) * (N / 128) > kMaxGroups) return FP8Q_ERR_SHAPE;
  GemmArgs a{};
  a.A = xq; a.B = wq; a.sa = xs; a.sb = ws; a.C = y;
  a.lda = K; a.ldb = K; a.ld_sa = K / 128; a.sb_rs = K / 128; a.sb_cs = 1; a.ldc = ld_y;
  a.M = M; a.N = N; a.K = K;
  a.sb_mode = fp8q::kSbBlock; a.out_f32 = 1;
  return launched(fp8q::launch_gemm_interval(a, chunks, stream));
}

fp8q_status fp8q_gemm_fprop(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws, int64_t M,
                            int64_t N, int64_t K, void* y, fp8q_dtype yt, int64_t ld_y, hipStream_t stream) {
  return fp8q_gemm_fprop_impl(0, xq, xs, wq, ws, M, N, K, y, yt, ld_y, stream);
}
fp8q_status fp8q_gemm_fprop_exact(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                                  int64_t M, int64_t N, int64_t K, void* y, fp8q_dtype yt, int64_t ld_y,
                                  hipStream_t stream) {
  return fp8q_gemm_fprop_impl(1, xq, xs, wq, ws, M, N, K, y, yt, ld_y, stream);
}
fp8q_status fp8q_gemm_dgrad(const uint8_t* dyq, const float* dys, const uint8_t* wq_t, const float* ws, int64_t M,
                            int64_t N, int64_t K, void* dx, fp8q_dtype dxt, int64_t ld_dx, hipStream_t stream) {
  return fp8q_gemm_dgrad_impl(0, dyq, dys, wq_t, ws, M, N, K, dx, dxt, ld_dx, stream);
}
fp8q_status fp8q_gemm_dgrad_exact(const uint8_t* dyq, const float* dys, const uint8_t* wq_t, const float* ws,
                                  int64_t M, int64_t N, int64_t K, void* dx, fp8q_dtype dxt, int64_t ld_dx,
                                  hipStream_t stream) {
  return fp8q_gemm_dgrad_impl(1, dyq, dys, wq_t, ws, M, N, K, dx, dxt, ld_dx, stream);
}
fp8q_status fp8q_gemm_wgrad(const uint8_t* dyq_t, const float* dys_t, const uint8_t* xq_t, const float* xs_t,
                            int64_t T, int64_t N, int64_t K, float* dw, int64_t ld_dw, int accumulate,
                            hipStream_t stream) {
  return fp8q_gemm_wgrad_impl(0, dyq_t, dys_t, xq_t, xs_t, T, N, K, dw, ld_dw, accumulate, stream);
}
fp8q_status fp8q_gemm_wgrad_exact(const uint8_t* dyq_t, const float* dys_t, const uint8_t* xq_t, const float* xs_t,
                                  int64_t T, int64_t N, int64_t K, float* dw, int64_t ld_dw, int accumulate,
                                  hipStream_t stream) {
  return fp8q_gemm_wgrad_impl(1, dyq_t, dys_t, xq_t, xs_t, T, N, K, dw, ld_dw, accumulate, stream);
}
fp8q_status fp8q_grouped_gemm(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                              const int32_t* offsets, int64_t E, int64_t M_total, int64_t N, int64_t K, void* y,
                              fp8q_dtype yt, int64_t ld_y, hipStream_t stream) {
  return fp8q_grouped_gemm_impl(0, xq, xs, wq, ws, offsets, E, M_total, N, K, y, yt, ld_y, stream);
}
fp8q_status fp8q_grouped_gemm_exact(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                                    const int32_t* offsets, int64_t E, int64_t M_total, int64_t N, int64_t K,
                                    void* y, fp8q_dtype yt, int64_t ld_y, hipStream_t stream) {
  return fp8q_grouped_gemm_impl(1, xq, xs, wq, ws, offsets, E, M_total, N, K, y, yt, ld_y, stream);
}

}  // extern "C"

extern "C" {

fp8q_status fp8q_quant_mx_1x32(const void* x, fp8q_dtype xt, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q,
                               int64_t ld_q, uint8_t* s, int64_t ld_s, hipStream_t stream) {
  if (!valid_dtype(xt)) return FP8Q_ERR_DTYPE;
  const fp8q_status c = check_quant(x, esize(xt), rows, cols, ld_x, q, ld_q, cols, s, ld_s, cdiv(cols, 32));
  if (c != FP8Q_OK || rows == 0 || cols == 0) return c;
  if (rows * cdiv(cols, 128) > kMaxGroups) return FP8Q_ERR_SHAPE;
  return launched(fp8q::launch_quant_mx(x, xt == FP8Q_BF16, rows, cols, ld_x, q, ld_q, s, ld_s, stream));
}

fp8q_status fp8q_quant_mx_transpose(const void* x, fp8q_dtype xt, int64_t rows, int64_t cols, int64_t ld_x,
                                    uint8_t* q_t, int64_t ld_qt, uint8_t* s_t, int64_t ld_st, uint8_t* q,
                                    int64_t ld_q, uint8_t* s, int64_t ld_s, hipStream_t stream) {
  if (!valid_dtype(xt)) return FP8Q_ERR_DTYPE;
  if ((q == nullptr) != (s == nullptr)) return FP8Q_ERR_NULL;
  fp8q_status c = check_quant(x, esize(xt), rows, cols, ld_x, q_t, ld_qt, rows, s_t, ld_st, cdiv(rows, 32));
  if (c != FP8Q_OK || rows == 0 || cols == 0) return c;
  if (q) {
    c = check_quant(x, esize(xt), rows, cols, ld_x, q, ld_q, cols, s, ld_s, cdiv(cols, 32));
    if (c != FP8Q_OK) return c;
  }
  if (cdiv(rows, 128) > 65535) return FP8Q_ERR_SHAPE;
  return launched(fp8q::launch_quant_mx_transpose(x, xt == FP8Q_BF16, rows, cols, ld_x, q_t, ld_qt, s_t, ld_st, q,
                                                  ld_q, s, ld_s, stream));
}

fp8q_status fp8q_gemm_mx(const uint8_t* aq, const uint8_t* as, int64_t lda, int64_t ld_sa, const uint8_t* bq,
                         const uint8_t* bs, int64_t ldb, int64_t ld_sb, int64_t M, int64_t N, int64_t K, void* c,
                         fp8q_dtype ct, int64_t ld_c, int accumulate, hipStream_t stream) {
  if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return FP8Q_ERR_SHAPE;
  if (N % 128 != 0 || K % 128 != 0 || K > kMaxContraction) return FP8Q_ERR_SHAPE;
  if (accumulate != 0 && accumulate != 1) return FP8Q_ERR_SHAPE;
  if (!valid_dtype(ct)) return FP8Q_ERR_DTYPE;
  if (accumulate && ct != FP8Q_F32) return FP8Q_ERR_DTYPE;
  if (M == 0 || N == 0) return FP8Q_OK;
  if (K == 0) return FP8Q_ERR_SHAPE;
  if (!aq || !as || !bq || !bs) return FP8Q_ERR_NULL;
  const fp8q_status st = check_gemm_out(c, ct, ld_c, N);
  if (st != FP8Q_OK) return st;
  if (lda < K || ldb < K || ld_sa < K / 32 || ld_sb < K / 32) return FP8Q_ERR_STRIDE;
  if (!aligned16(aq) || !aligned16(bq) || lda % 16 != 0 || ldb % 16 != 0) return FP8Q_ERR_ALIGN;
  if (!aligned4(as) || !aligned4(bs) || ld_sa % 4 != 0 || ld_sb % 4 != 0) return FP8Q_ERR_ALIGN;
  // the kernel's buffer descriptors address one tile's rows with 32-bit offsets
  if (256 * lda > INT32_MAX || 128 * ldb > INT32_MAX) return FP8Q_ERR_SHAPE;
  if (cdiv(M, 256) * (N / 128) > kMaxGroups) return FP8Q_ERR_SHAPE;  // the launch grid
  fp8q::MxArgs a{};
  a.g.A = aq; a.g.B = bq; a.g.C = c;
  a.g.lda = lda; a.g.ldb = ldb; a.g.ldc = ld_c;
  a.g.M = M; a.g.N = N; a.g.K = K;
  a.g.out_f32 = ct == FP8Q_F32; a.g.accumulate = accumulate;
  a.sa = as; a.sb = bs; a.ld_sa = ld_sa; a.ld_sb = ld_sb;
  return launched(fp8q::launch_gemm_mx(a, stream));
}

fp8q_status fp8q_grouped_gemm_mx(const uint8_t* xq, const uint8_t* xs, const uint8_t* wq, const uint8_t* ws,
                                 const int32_t* offsets, int64_t E, int64_t M_total, int64_t N, int64_t K, void* y,
                                 fp8q_dtype yt, int64_t ld_y, hipStream_t stream) {
  if (E < 1 || E > 65536) return FP8Q_ERR_SHAPE;
  if (M_total < 0 || N < 0 || K < 0 || M_total > kMaxDim || N > kMaxDim || K > kMaxDim) return FP8Q_ERR_SHAPE;
  if (N % 128 != 0 || K % 128 != 0 || K > kMaxContraction) return FP8Q_ERR_SHAPE;
  if (!valid_dtype(yt)) return FP8Q_ERR_DTYPE;
  if (M_total == 0 || N == 0) return FP8Q_OK;
  if (K == 0) return FP8Q_ERR_SHAPE;
  if (!xq || !xs || !wq || !ws || !offsets) return FP8Q_ERR_NULL;
  const fp8q_status c = check_gemm_out(y, yt, ld_y, N);
  if (c != FP8Q_OK) return c;
  // scale rows are K/32 bytes, a multiple of 4 since K % 128 == 0
  if (!aligned16(xq) || !aligned16(wq) || !aligned4(xs) || !aligned4(ws) || !aligned4(offsets))
    return FP8Q_ERR_ALIGN;
  if (((M_total + 255) / 256 + E) * (N / 128) > kMaxGroups) return FP8Q_ERR_SHAPE;
  if (const fp8q_status d = debug_check_offsets(offsets, E, M_total, stream); d != FP8Q_OK) return d;
  fp8q::MxArgs a{};
  a.g.A = xq; a.g.B = wq; a.g.C = y;
  a.g.lda = K; a.g.ldb = K; a.g.ldc = ld_y;
  a.g.M = M_total; a.g.N = N; a.g.K = K;
  a.g.out_f32 = yt == FP8Q_F32; a.g.accumulate = 0;
  a.g.offsets = offsets; a.g.E = E; a.g.b_estride = N * K;
  a.sa = xs; a.sb = ws; a.ld_sa = K / 32; a.ld_sb = K / 32; a.sb_estride = N * (K / 32);
  return launched(fp8q::launch_gemm_mx(a, stream));
}

fp8q_status fp8q_grouped_gemm_mx_dgrad(const uint8_t* dyq, const uint8_t* dys, const uint8_t* wq_t,
                                       const uint8_t* ws_t, const int32_t* offsets, int64_t E, int64_t M_total,
                                       int64_t N, int64_t K, void* dx, fp8q_dtype dxt, int64_t ld_dx,
                                       hipStream_t stream) {
  if (E < 1 || E > 65536) return FP8Q_ERR_SHAPE;
  if (M_total < 0 || N < 0 || K < 0 || M_total > kMaxDim || N > kMaxDim || K > kMaxDim) return FP8Q_ERR_SHAPE;
  if (N % 128 != 0 || K % 128 != 0 || N > kMaxContraction) return FP8Q_ERR_SHAPE;
  // the kernel addresses 128 rows of the stacked transposed codes (E*N bytes each) with 32-bit offsets
  if (E * N > INT32_MAX / 128) return FP8Q_ERR_SHAPE;
  if (!valid_dtype(dxt)) return FP8Q_ERR_DTYPE;
  if (M_total == 0 || K == 0) return FP8Q_OK;
  if (N == 0) return FP8Q_ERR_SHAPE;
  if (!dyq || !dys || !wq_t || !ws_t || !offsets) return FP8Q_ERR_NULL;
  const fp8q_status c = check_gemm_out(dx, dxt, ld_dx, K);
  if (c != FP8Q_OK) return c;
  if (!aligned16(dyq) || !aligned16(wq_t) || !aligned4(dys) || !aligned4(ws_t) || !aligned4(offsets))
    return FP8Q_ERR_ALIGN;
  if (((M_total + 255) / 256 + E) * (K / 128) > kMaxGroups) return FP8Q_ERR_SHAPE;
  if (const fp8q_status d = debug_check_offsets(offsets, E, M_total, stream); d != FP8Q_OK) return d;
  // Per expert: C = dY rows . B^T with B = W_e^T = columns [eN, (e+1)N) of
  // the stacked transposed codes (row stride E*N) and of their scales (E*N/32)
  fp8q::MxArgs a{};
  a.g.A = dyq; a.g.B = wq_t; a.g.C = dx;
  a.g.lda = N; a.g.ldb = E * N; a.g.ldc = ld_dx;
  a.g.M = M_total; a.g.N = K; a.g.K = N;
  a.g.out_f32 = dxt == FP8Q_F32; a.g.accumulate = 0;
  a.g.offsets = offsets; a.g.E = E; a.g.b_estride = N;
  a.sa = dys; a.sb = ws_t; a.ld_sa = N / 32; a.ld_sb = E * N / 32; a.sb_estride = N / 32;
  return launched(fp8q::launch_gemm_mx(a, stream));
}

}  // extern "C"
