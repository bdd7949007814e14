// Microscaling (MXFP8, E4M3 elements) quantizers for gfx950.
//
// The pages contrast the method's FP32 group scales with the microscaling
// formats that newer hardware supports natively: small groups sharing a
// power-of-two scale (the innerforce.co.kr excerpt of the DeepSeek-V3 report,
// paragraph on Figure 7 (a)).  The variant here follows the OCP Microscaling
// v1.0 definition of MXFP8 with E4M3 elements:
//
//   block    32 consecutive elements along the contraction axis;
//   scale    X = 2^(floor(log2 amax) - 8), stored as the E8M0 byte
//            clamp(floor(log2 amax) - 8 + 127, 0, 254); 0 for an all-zero block;
//   codes    E4M3(x / X), round-to-nearest-even, saturating at +-448.
//
// For a finite FP32 amax with exponent field E, floor(log2 amax) = E - 127
// (normal) and the byte is max(E - 8, 0) (a subnormal or zero amax gives 0).
// 1/X = 2^(127 - byte) is a normal FP32 power of two for every byte in
// [0, 246], so x * (1/X) is the exact quotient (or, far below E4M3's range,
// its correctly rounded FP32 value, which encodes to a signed zero either
// way) and |x / X| < 512.
//
// Both kernels stream: every input byte is read once, every code and scale
// byte written once, reductions stay in registers and DPP.

#include "device_common.h"
#include <type_traits>
#include "launch.h"

namespace fp8q {

namespace {

// Max over the 4 lanes of a DPP quad (lanes 4k .. 4k+3); all four receive it.
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)0, (int)v, 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)0, (int)v, 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
  return v;
}

// E8M0 byte of a block whose max-abs has the FP32 bits `amax_bits`, and the
// block's inverse scale 2^(127 - byte).
__device__ __forceinline__ uint32_t mx_scale(uint32_t amax_bits, float& inv) {
  const int e = (int)(amax_bits >> 23);
  const uint32_t byte = (uint32_t)max(e - 8, 0);
  inv = __uint_as_float((254u - byte) << 23);
  return byte;
}

}  // namespace

// ---------------------------------------------------------------------------
// 1x32 blocks along rows: 16 lanes (one DPP row) cover 128 consecutive columns
// of one row, 8 elements per lane, so each DPP quad is one 32-block; a wave
// covers 4 such 128-column spans per step and U steps.  Inputs are read
// non-temporally (each byte once; measured faster for tensors that are not
// cache-resident).
constexpr int kMxU = 2;

template <class In>
__global__ __launch_bounds__(256) void k_quant_mx(const typename In::elem* __restrict__ x, int64_t ld_x,
                                                  uint8_t* __restrict__ q, int64_t ld_q,
                                                  uint8_t* __restrict__ s, int64_t ld_s,
                                                  int cols, int ngr, int total) {
  const int lane = threadIdx.x & 63;
  const int wave = (int)((blockIdx.x * (uint32_t)blockDim.x + threadIdx.x) >> 6);
  const int team = lane >> 4, lig = lane & 15;
  float v[kMxU][8];
  int grow[kMxU], gcol[kMxU];
#pragma unroll
  for (int u = 0; u < kMxU; ++u) {
    const int gi = (wave * kMxU + u) * 4 + team;
    grow[u] = -1;
    gcol[u] = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[u][e] = 0.f;
    if (gi < total) {
      const int r = gi / ngr, j = gi - r * ngr;
      const int c0 = j * 128 + lig * 8;
      grow[u] = r;
      gcol[u] = c0;
      const typename In::elem* p = x + (int64_t)r * ld_x + c0;
      if (c0 + 8 <= cols) {
        In::template load8<1>(p, v[u]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (c0 + e < cols) v[u][e] = In::load1(p + e);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kMxU; ++u) {
    uint32_t m = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) m = max(m, abs_bits(v[u][e]));
    m = quad_max_u32(m);  // the quad's 32 elements form one block
    const int r = grow[u], c0 = gcol[u];
    if (r < 0 || c0 >= cols) continue;
    float inv;
    const uint32_t byte = mx_scale(m, inv);
    const uint32_t w0 = pack4_e4m3(v[u][0] * inv, v[u][1] * inv, v[u][2] * inv, v[u][3] * inv);
    const uint32_t w1 = pack4_e4m3(v[u][4] * inv, v[u][5] * inv, v[u][6] * inv, v[u][7] * inv);
    uint8_t* qp = q + (int64_t)r * ld_q + c0;
    if (c0 + 8 <= cols) {
      *reinterpret_cast<uint2*>(qp) = make_uint2(w0, w1);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (c0 + e < cols) qp[e] = (uint8_t)(((e < 4 ? w0 : w1) >> (8 * (e & 3))) & 0xFF);
    }
    if ((lig & 3) == 0) s[(int64_t)r * ld_s + (c0 >> 5)] = (uint8_t)byte;
  }
}

hipError_t launch_quant_mx(const void* x, bool x_bf16, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q,
                           int64_t ld_q, uint8_t* s, int64_t ld_s, hipStream_t st) {
  const int64_t ngr = (cols + 127) / 128;
  const int64_t total = rows * ngr;
  const int64_t waves = (total + 4 * kMxU - 1) / (4 * kMxU);
  const int64_t blocks = (waves + 3) / 4;
  if (x_bf16)
    hipLaunchKernelGGL(k_quant_mx<BF16In>, dim3((uint32_t)blocks), dim3(256), 0, st, (const uint16_t*)x, ld_x, q,
                       ld_q, s, ld_s, (int)cols, (int)ngr, (int)total);
  else
    hipLaunchKernelGGL(k_quant_mx<F32In>, dim3((uint32_t)blocks), dim3(256), 0, st, (const float*)x, ld_x, q, ld_q,
                       s, ld_s, (int)cols, (int)ngr, (int)total);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 32x1 blocks along columns, codes written transposed: one workgroup per
// 128-row x 128-column tile.  Thread t owns 8 consecutive rows (8*(t/16) ..)
// of 8 consecutive columns (8*(t%16) ..), so wave w holds rows
// [32w, 32w + 32) of the tile: a column's 32-block is reduced over the four
// lanes l%16 + 16k of one wave (xor 16, xor 32), without LDS.  Each column's
// 8 codes are converted pairwise down the column into an LDS copy of the
// tile's transposed codes, which leaves as whole 128-byte q_t row segments.
//
// D (dual output): the tile's rows also yield the 1x32 row blocks (a DPP
// quad of lanes spans 32 consecutive columns of one row), so x is read once
// for both the row codes q [rows, cols] and the transposed ones.
//
// F (full tiles): rows and cols are multiples of 128, so every tile is whole
// and the per-row and per-column bounds checks drop out (with them in, the
// loads sat in separate branches and could not be issued together).
template <class In, bool D, bool F>
__global__ __launch_bounds__(256) void k_quant_mx_t(const typename In::elem* __restrict__ x, int64_t ld_x,
                                                    int rows, int cols,
                                                    uint8_t* __restrict__ qt, int64_t ld_qt,
                                                    uint8_t* __restrict__ st, int64_t ld_st,
                                                    uint8_t* __restrict__ q, int64_t ld_q,
                                                    uint8_t* __restrict__ s, int64_t ld_s) {
  __shared__ __attribute__((aligned(16))) uint8_t tq[128 * 128];  // [channel][token] codes of the tile
  const int t = threadIdx.x, wv = t >> 6;
  const int c8 = t & 15, rblk = t >> 4;
  const int bi = blockIdx.y, bj = blockIdx.x;
  const int r0 = bi * 128 + rblk * 8;
  const int c0 = bj * 128 + c8 * 8;
  float v[8][8];
  // row and column addresses advance by pointer increments (a 64-bit
  // multiply per row or column was a large share of the vector work)
  const typename In::elem* p = x + (int64_t)r0 * ld_x + c0;
#pragma unroll
  for (int i = 0; i < 8; ++i, p += ld_x) {
    const int r = r0 + i;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[i][e] = 0.f;
    if (F || r < rows) {
      if (F || c0 + 8 <= cols) {
        In::template load8<1>(p, v[i]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (c0 + e < cols) v[i][e] = In::load1(p + e);
      }
    }
  }
  if (D) {
    uint8_t* qp = q + (int64_t)r0 * ld_q + c0;
    uint8_t* sp = s + (int64_t)r0 * ld_s + (c0 >> 5);
#pragma unroll
    for (int i = 0; i < 8; ++i, qp += ld_q, sp += ld_s) {
      uint32_t a = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) a = max(a, abs_bits(v[i][e]));
      a = quad_max_u32(a);
      const int r = r0 + i;
      if (!F && (r >= rows || c0 >= cols)) continue;
      float iv;
      const uint32_t byte = mx_scale(a, iv);
      const uint32_t w0 = pack4_e4m3(v[i][0] * iv, v[i][1] * iv, v[i][2] * iv, v[i][3] * iv);
      const uint32_t w1 = pack4_e4m3(v[i][4] * iv, v[i][5] * iv, v[i][6] * iv, v[i][7] * iv);
      if (F || c0 + 8 <= cols) {
        *reinterpret_cast<uint2*>(qp) = make_uint2(w0, w1);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (c0 + e < cols) qp[e] = (uint8_t)(((e < 4 ? w0 : w1) >> (8 * (e & 3))) & 0xFF);
      }
      if ((c8 & 3) == 0) *sp = (uint8_t)byte;
    }
  }
  // column maxima over the wave's 32 rows: all 16 cross-lane exchanges are
  // issued before any of them is waited for
  uint32_t m[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    uint32_t a = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = max(a, abs_bits(v[i][e]));
    m[e] = a;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) m[e] = max(m[e], (uint32_t)__shfl_xor((int)m[e], 16));
#pragma unroll
  for (int e = 0; e < 8; ++e) m[e] = max(m[e], (uint32_t)__shfl_xor((int)m[e], 32));
  const bool block_present = F || bi * 128 + wv * 32 < rows;  // this wave's 32-row block has rows
  const bool full_r = F || r0 + 8 <= rows;
  const int oc0 = bi * 128 + rblk * 8;  // output token column of this thread's rows
  // A tile of 128 whole tokens stages its transposed codes in LDS (channel
  // cl's 128 token codes at tq[128 cl], 8-byte token chunk k at slot
  // k ^ (2 (c8 & 7))) so that 8 lanes write each 128-byte q_t row segment
  // together; a partial last token tile stores from registers.
  const bool staged = F || bi * 128 + 128 <= rows;
  const int swz = 2 * (c8 & 7);
  uint8_t* stp = st + (int64_t)c0 * ld_st + bi * 4 + wv;
  uint8_t* tp = qt + (int64_t)c0 * ld_qt + oc0;
#pragma unroll
  for (int e = 0; e < 8; ++e, stp += ld_st, tp += ld_qt) {
    if (!F && c0 + e >= cols) continue;
    float iv;
    const uint32_t byte = mx_scale(m[e], iv);
    if ((t & 63) < 16 && block_present) *stp = (uint8_t)byte;
    const uint32_t d0 = pack4_e4m3(v[0][e] * iv, v[1][e] * iv, v[2][e] * iv, v[3][e] * iv);
    const uint32_t d1 = pack4_e4m3(v[4][e] * iv, v[5][e] * iv, v[6][e] * iv, v[7][e] * iv);
    if (staged) {
      *reinterpret_cast<uint2*>(tq + (c8 * 8 + e) * 128 + (rblk ^ swz) * 8) = make_uint2(d0, d1);
      continue;
    }
    if (full_r) {
      *reinterpret_cast<uint2*>(tp) = make_uint2(d0, d1);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (r0 + i < rows) tp[i] = (uint8_t)((((i < 4) ? d0 : d1) >> (8 * (i & 3))) & 0xFF);
    }
  }
  if (!staged) return;
  __syncthreads();
  // lane t writes bytes [16 k, 16 k + 16) of channel 32 pass + t/8, k = t%8
  const int k16 = t & 7;
  uint8_t* pq = qt + (int64_t)(bj * 128 + (t >> 3)) * ld_qt + bi * 128 + k16 * 16;
  const int64_t pass_step = 32 * ld_qt;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass, pq += pass_step) {
    const int cl = pass * 32 + (t >> 3);
    if (!F && bj * 128 + cl >= cols) break;  // channels ascend with the pass
    const u32x4 w = *reinterpret_cast<const u32x4*>(tq + cl * 128 + (k16 ^ ((cl >> 3) & 7)) * 16);
    *reinterpret_cast<u32x4*>(pq) = w;
  }
}

hipError_t launch_quant_mx_transpose(const void* x, bool x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                                     uint8_t* q_t, int64_t ld_qt, uint8_t* s_t, int64_t ld_st, uint8_t* q,
                                     int64_t ld_q, uint8_t* s, int64_t ld_s, hipStream_t st) {
  const dim3 grid((uint32_t)((cols + 127) / 128), (uint32_t)((rows + 127) / 128));
  const bool dual = q != nullptr, full = rows % 128 == 0 && cols % 128 == 0;
  auto go = [&](auto in, auto d, auto f) {
    typedef decltype(in) In;
    constexpr bool D = decltype(d)::value, F = decltype(f)::value;
    hipLaunchKernelGGL((k_quant_mx_t<In, D, F>), grid, dim3(256), 0, st, (const typename In::elem*)x, ld_x,
                       (int)rows, (int)cols, q_t, ld_qt, s_t, ld_st, D ? q : nullptr, D ? ld_q : 0,
                       D ? s : nullptr, D ? ld_s : 0);
  };
  using T = std::true_type;
  using N = std::false_type;
  if (x_bf16) {
    if (dual) full ? go(BF16In{}, T{}, T{}) : go(BF16In{}, T{}, N{});
    else full ? go(BF16In{}, N{}, T{}) : go(BF16In{}, N{}, N{});
  } else {
    if (dual) full ? go(F32In{}, T{}, T{}) : go(F32In{}, T{}, N{});
    else full ? go(F32In{}, N{}, T{}) : go(F32In{}, N{}, N{});
  }
  return hipGetLastError();
}

}  // namespace fp8q
