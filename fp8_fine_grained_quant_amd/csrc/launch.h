// Host-side launchers of the HIP kernels (internal to libfp8q; the C ABI in
// include/fp8q.h validates arguments and calls these).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

hipError_t launch_quant_act(const void* x, bool x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                            uint8_t* q, int64_t ld_q, float* s, int64_t ld_s, hipStream_t st);

hipError_t launch_quant_weight(const void* w, bool w_bf16, int64_t rows, int64_t cols, int64_t ld_w,
                               uint8_t* q, int64_t ld_q, uint8_t* q_t, int64_t ld_qt,
                               float* s, int64_t ld_s, hipStream_t st);

hipError_t launch_quant_transpose(const void* x, bool x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                                  uint8_t* q_t, int64_t ld_qt, float* s_t, int64_t ld_st, hipStream_t st);

// quant_act_1x128 and quant_transpose of the same x from one read of it.
hipError_t launch_quant_act_transpose(const void* x, bool x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                                      uint8_t* q, int64_t ld_q, float* s, int64_t ld_s, uint8_t* q_t,
                                      int64_t ld_qt, float* s_t, int64_t ld_st, hipStream_t st);

// Per expert e (rows [offsets[e], offsets[e+1]) of x), the quantize-transpose
// of that block alone, written at padded token column 128*(offsets[e]/128 + e);
// the tail of an expert's last 128-token chunk is written as code 0.
hipError_t launch_quant_transpose_grouped(const void* x, bool x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                                          const int32_t* offsets, int64_t E, uint8_t* q_t, int64_t ld_qt,
                                          float* s_t, int64_t ld_st, hipStream_t st);

// One quantization of a batched launch (kinds as fp8q_quant_kind: 0 act 1x128,
// 1 weight 128x128 (q_t optional), 2 transpose, 3 act + transpose); arguments
// as the single entry points, already validated.
struct QuantJob {
  int kind;
  bool x_bf16;
  const void* x;
  int64_t rows, cols, ld_x;
  uint8_t* q;
  int64_t ld_q;
  float* s;
  int64_t ld_s;
  uint8_t* q_t;
  int64_t ld_qt;
  float* s_t;
  int64_t ld_st;
};
constexpr int kMaxQuantJobs = 8;
// All jobs in one grid (each job's blocks form one contiguous range of it).
hipError_t launch_quant_batch(const QuantJob* jobs, int n, hipStream_t st);
// Workgroups that grid has (all must fit one grid dimension).
int64_t quant_batch_blocks(const QuantJob* jobs, int n);

// How the scale of the B operand (rows = output columns) is indexed.
enum SbMode : int {
  kSbBlock = 0,  // one scale per 128 output columns per chunk: sb[(n/128)*sb_rs + kb*sb_cs]
  kSbRow = 1     // one scale per output column per chunk:      sb[n*sb_rs + kb]
};

// C[m, n] = sum_kb P_kb[m, n] * sa[m*ld_sa + kb] * sB(n, kb), P_kb the FP8
// product of the 128-long chunk kb of A[m, :] and B[n, :] (both row-major
// with the contraction axis contiguous).
struct GemmArgs {
  const uint8_t* A;     // [M, K] codes, row stride lda bytes
  const uint8_t* B;     // [N, K] codes, row stride ldb bytes
  const float* sa;      // [M, K/128]
  const float* sb;      // see SbMode
  void* C;              // [M, N], BF16 or FP32, row stride ldc elements
  int64_t lda, ldb, ld_sa, sb_rs, sb_cs, ldc;
  int64_t M, N, K;
  int sb_mode;          // SbMode
  int out_f32;          // 0 = BF16 output, 1 = FP32 output
  int accumulate;       // FP32 output only: C += result
  int exact;            // 0: FP8 MFMA per chunk; 1: exact BF16 MFMA on the converted codes
  // grouped: rows [offsets[e], offsets[e+1]) use B + e*b_estride, sb + e*sb_estride
  const int32_t* offsets;  // NULL for a plain GEMM
  int64_t E, b_estride, sb_estride;
  // grouped contraction (k_grouped = 1): expert e contracts over the padded
  // chunks [offsets[e]/128 + e, + ceil(m_e/128)) of A and B (token-padded
  // operands), and writes its own output C + e*c_estride; M, N are per expert
  int k_grouped;
  int64_t c_estride;
  // fused output quantization (BF16 output only; qo == NULL: none): the 1x128
  // E4M3 codes qo [M, N] (row stride ld_qo bytes) and scales so [M, N/128]
  // (row stride ld_so) of the BF16-rounded output, as quant_act_1x128 would
  // produce them from C; C may then be NULL (codes only)
  uint8_t* qo;
  float* so;
  int64_t ld_qo, ld_so;
};

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st);

// Workgroup tile of the block-scaled GEMMs: 0 = chosen by problem size,
// 1 = 256 x 128, 2 = 256 x 256 (fp8q_set_gemm_tile; both tiles give the same
// result bits).
int gemm_tile_setting();
// Compute units of the current device, queried once per device.
int device_cu_count();
// the FP8 matrix-instruction kernel (a.exact == 0)
hipError_t launch_gemm_fp8(const GemmArgs& a, hipStream_t st);
// the promotion-interval study (block scales, FP32 output): partials chained
// through the matrix instruction over `chunks` chunks (1, 2, 4, 8; 0 = all)
hipError_t launch_gemm_interval(const GemmArgs& a, int chunks, hipStream_t st);

// Microscaling (MXFP8 E4M3) quantizers: one E8M0 scale byte per 32
// consecutive elements, along rows (quant_mx) or along columns with the
// codes transposed (quant_mx_transpose; q, s optional row outputs of the same
// read, NULL to skip).
hipError_t launch_quant_mx(const void* x, bool x_bf16, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q,
                           int64_t ld_q, uint8_t* s, int64_t ld_s, hipStream_t st);
hipError_t launch_quant_mx_transpose(const void* x, bool x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                                     uint8_t* q_t, int64_t ld_qt, uint8_t* s_t, int64_t ld_st, uint8_t* q,
                                     int64_t ld_q, uint8_t* s, int64_t ld_s, hipStream_t st);

// MX GEMM: C = A . B^T, both operands blocked along K with E8M0 bytes
// sa[m*ld_sa + k/32], sb[n*ld_sb + k/32] (strides in bytes).  g carries A, B,
// C, their strides, M, N, K, out_f32 and accumulate; its scale fields are unused.
struct MxArgs {
  GemmArgs g;
  const uint8_t* sa;
  const uint8_t* sb;
  int64_t ld_sa, ld_sb;
  int64_t sb_estride;  // grouped: bytes between experts' B scales (g.b_estride for the codes)
};
hipError_t launch_gemm_mx(const MxArgs& a, hipStream_t st);

}  // namespace fp8q
