// Online fine-grained E4M3 quantizers for gfx950.
//
// Group rule ("How does the unified E4M3 format contribute to the efficiency
// of DeepSeek-V3", sections "Fine-Grained Quantization Strategy" and "Dynamic
// Scaling and Online Quantization"; innerforce.co.kr excerpt, paragraph on
// Figure 7 (a)): amax = max |x| over the group, s = fl32(max(amax,2^-100)/448)
// is stored, and each element becomes E4M3(fl32(x * fl32(448/max(amax,2^-100)))),
// round-to-nearest-even, saturating, sign of zero kept.
//
// All three kernels are HBM-bound streaming kernels: every input byte is read
// once and every code/scale written once, with 16-byte loads and coalesced
// stores; reductions stay in registers, DPP and (for cross-wave) a few bytes of
// LDS.

#include "device_common.h"
#include "launch.h"

#include <type_traits>

namespace fp8q {

// Non-temporal choices per access (see ld_stream16).  Inputs are read once,
// non-temporally.  Row codes of up to kNtCodeBytes are written cached: the
// GEMM that consumes them runs next and finds them in the 256 MB MALL
// (written non-temporally, X's 29 MB of codes cost Fprop 5-6 us of its 62).
// Larger code arrays (the MoE layer's activations and stacked experts) are
// written non-temporally, which measured faster for them and for the grouped
// GEMM after them.  Measured on MI355X with inputs that are not
// cache-resident, as in a training step.
constexpr int kNtWeightLoad = 1, kNtWeightTStore = 0, kNtTransLoad = 1, kNtTransStore = 0;
constexpr int kNtActLoad = 1;
constexpr int64_t kNtCodeBytes = 64ll << 20;

// ---------------------------------------------------------------------------
// 1x128 activation tiles: 16 lanes (one DPP row) own one group, 8 elements per
// lane; a wave covers 4 consecutive groups per step and U steps, so each lane
// keeps U 16-byte loads in flight.  Two steps per wave measured fastest for
// 25-360 MB tensors: more waves, each short, keep the read and write streams
// overlapped better than fewer, longer ones.
//
// FLAT: the tensor is dense (cols a multiple of 128, ld_x = ld_q = cols,
// ld_s = cols/128), so group g starts at element 128 g of x and q and its
// scale is s[g]; no row/column split is needed.
constexpr int kActU = 2;

// One 256-thread block `vb` of the activation quantizer (the kernel below, and
// activation jobs of the batched launch).
template <class In, bool FLAT, int NTS>
__device__ __forceinline__ void quant_act_block(int vb, const typename In::elem* __restrict__ x, int64_t ld_x,
                                                uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ s,
                                                int64_t ld_s, int cols, int ngr, int total) {
  const int lane = threadIdx.x & 63;
  const int wave = (int)((vb * 256u + threadIdx.x) >> 6);
  const int team = lane >> 4, lig = lane & 15;
  float v[kActU][8];
  int grow[kActU], gcol[kActU];
#pragma unroll
  for (int u = 0; u < kActU; ++u) {
    const int g = (wave * kActU + u) * 4 + team;
    grow[u] = -1;
    gcol[u] = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[u][e] = 0.f;
    if (FLAT && g < total) {
      grow[u] = g;
      In::template load8<kNtActLoad>(x + (int64_t)g * 128 + lig * 8, v[u]);
    } else if (g < total) {
      const int r = g / ngr, j = g - r * ngr;
      const int c0 = j * 128 + lig * 8;
      grow[u] = r;
      gcol[u] = c0;
      const typename In::elem* p = x + (int64_t)r * ld_x + c0;
      if (c0 + 8 <= cols) {
        In::template load8<kNtActLoad>(p, v[u]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (c0 + e < cols) v[u][e] = In::load1(p + e);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kActU; ++u) {
    uint32_t m = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) m = max(m, abs_bits(v[u][e]));
    m = row16_max_u32(m);  // all 16 lanes of the team share one group
    const int r = grow[u];
    if (r < 0) continue;
    float sc, inv;
    group_scale(__uint_as_float(m), sc, inv);
    const uint32_t w0 = pack4_e4m3_grp(v[u][0] * inv, v[u][1] * inv, v[u][2] * inv, v[u][3] * inv);
    const uint32_t w1 = pack4_e4m3_grp(v[u][4] * inv, v[u][5] * inv, v[u][6] * inv, v[u][7] * inv);
    if (FLAT) {
      st_stream8<NTS>(q + (int64_t)r * 128 + lig * 8, w0, w1);
      if (lig == 0) s[r] = sc;
      continue;
    }
    const int c0 = gcol[u];
    uint8_t* qp = q + (int64_t)r * ld_q + c0;
    if (c0 + 8 <= cols) {
      st_stream8<NTS>(qp, w0, w1);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (c0 + e < cols) qp[e] = (uint8_t)(((e < 4 ? w0 : w1) >> (8 * (e & 3))) & 0xFF);
    }
    if (lig == 0) s[(int64_t)r * ld_s + (c0 >> 7)] = sc;
  }
}

template <class In, bool FLAT, int NTS>
__global__ __launch_bounds__(256) void k_quant_act(const typename In::elem* __restrict__ x, int64_t ld_x,
                                                   uint8_t* __restrict__ q, int64_t ld_q,
                                                   float* __restrict__ s, int64_t ld_s,
                                                   int cols, int ngr, int total) {
  quant_act_block<In, FLAT, NTS>((int)blockIdx.x, x, ld_x, q, ld_q, s, ld_s, cols, ngr, total);
}

hipError_t launch_quant_act(const void* x, bool x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                            uint8_t* q, int64_t ld_q, float* s, int64_t ld_s, hipStream_t st) {
  const int64_t ngr = (cols + 127) / 128;
  const int64_t total = rows * ngr;
  const int64_t waves = (total + 4 * kActU - 1) / (4 * kActU);
  const int64_t blocks = (waves + 3) / 4;
  const bool flat = cols % 128 == 0 && ld_x == cols && ld_q == cols && ld_s == ngr;
  const bool nt = rows * cols > kNtCodeBytes;
  const dim3 grid((uint32_t)blocks), block(256);
  const int c = (int)cols, ng = (int)ngr, tot = (int)total;
#define FP8Q_ACT(T, F, N) \
  hipLaunchKernelGGL((k_quant_act<T, F, N>), grid, block, 0, st, (const T::elem*)x, ld_x, q, ld_q, s, ld_s, c, ng, tot)
  if (x_bf16) {
    if (flat) { if (nt) FP8Q_ACT(BF16In, true, 1); else FP8Q_ACT(BF16In, true, 0); }
    else { if (nt) FP8Q_ACT(BF16In, false, 1); else FP8Q_ACT(BF16In, false, 0); }
  } else {
    if (flat) { if (nt) FP8Q_ACT(F32In, true, 1); else FP8Q_ACT(F32In, true, 0); }
    else { if (nt) FP8Q_ACT(F32In, false, 1); else FP8Q_ACT(F32In, false, 0); }
  }
#undef FP8Q_ACT
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 128x128 weight blocks: one workgroup per block.  Thread t owns 16
// consecutive rows (16*(t/32) ..) of 4 consecutive columns (4*(t%32) ..), so
// row-wise codes go out as 128-byte row segments and the transposed codes as
// 16-byte column segments without an LDS transpose.
template <class In>
__device__ __forceinline__ void load4(const typename In::elem* p, float v[4]);
template <>
__device__ __forceinline__ void load4<F32In>(const float* p, float v[4]) {
  const u32x4 a = ld_stream16<kNtWeightLoad>(p);
  v[0] = __uint_as_float(a[0]); v[1] = __uint_as_float(a[1]); v[2] = __uint_as_float(a[2]); v[3] = __uint_as_float(a[3]);
}
template <>
__device__ __forceinline__ void load4<BF16In>(const uint16_t* p, float v[4]) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  v[0] = bf16_to_f32(u.x & 0xFFFFu); v[1] = bf16_to_f32(u.x >> 16);
  v[2] = bf16_to_f32(u.y & 0xFFFFu); v[3] = bf16_to_f32(u.y >> 16);
}

// One 128 x 128 block (bi, bj) of the weight quantizer; red (4 words) and tq
// (16 KB, 16-byte aligned) are the block's LDS.  F (full blocks): rows and
// cols are multiples of 128, so the per-row and per-column checks drop out
// (with them in, each row's load sat in a branch of its own).
template <class In, int NTS, bool F>
__device__ __forceinline__ void quant_weight_block(int bi, int bj, const typename In::elem* __restrict__ w,
                                                   int64_t ld_w, int rows, int cols, uint8_t* __restrict__ q,
                                                   int64_t ld_q, uint8_t* __restrict__ qt, int64_t ld_qt,
                                                   float* __restrict__ s, int64_t ld_s, uint32_t* red,
                                                   uint8_t* tq) {
  const int t = threadIdx.x;
  const int c4 = t & 31, rb = t >> 5;
  const int r0 = bi * 128 + rb * 16;
  const int c0 = bj * 128 + c4 * 4;
  const bool full_c = F || c0 + 4 <= cols;
  float v[16][4];
  // row addresses by pointer increments (no 64-bit multiply per row)
  const typename In::elem* p = w + (int64_t)r0 * ld_w + c0;
#pragma unroll
  for (int i = 0; i < 16; ++i, p += ld_w) {
    const int r = r0 + i;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[i][e] = 0.f;
    if (F || r < rows) {
      if (full_c) {
        load4<In>(p, v[i]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (c0 + e < cols) v[i][e] = In::load1(p + e);
      }
    }
  }
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) m = max(m, abs_bits(v[i][e]));
  m = wave_max_u32(m);
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  m = max(max(red[0], red[1]), max(red[2], red[3]));
  float sc, inv;
  group_scale(__uint_as_float(m), sc, inv);
  if (t == 0) s[(int64_t)bi * ld_s + bj] = sc;

  // row-wise codes: one dword (4 columns) per row
  uint8_t* qp = q + (int64_t)r0 * ld_q + c0;
#pragma unroll
  for (int i = 0; i < 16; ++i, qp += ld_q) {
    if (!F && r0 + i >= rows) continue;  // (a break here kept the loop from unrolling)
    const uint32_t wd = pack4_e4m3_grp(v[i][0] * inv, v[i][1] * inv, v[i][2] * inv, v[i][3] * inv);
    if (full_c) {
      st_stream4<NTS>(qp, wd);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (c0 + e < cols) qp[e] = (uint8_t)((wd >> (8 * e)) & 0xFF);
    }
  }
  if (qt == nullptr) return;
  // transposed codes: 16 consecutive rows of one column -> 16 bytes of q_t.
  // A block of 128 whole rows stages them in LDS (column cl's 128 row codes
  // at tq[128 cl], 16-byte row chunk k at slot k ^ ((cl / 4) % 8)), so that 8
  // lanes write each 128-byte q_t row segment together instead of four waves
  // writing 32 bytes of it each.
  if (F || bi * 128 + 128 <= rows) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t d[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        d[k] = pack4_e4m3_grp(v[4 * k][e] * inv, v[4 * k + 1][e] * inv, v[4 * k + 2][e] * inv, v[4 * k + 3][e] * inv);
      *reinterpret_cast<u32x4*>(tq + (c4 * 4 + e) * 128 + (rb ^ (c4 & 7)) * 16) = u32x4{d[0], d[1], d[2], d[3]};
    }
    __syncthreads();
    const int k16 = t & 7;
    uint8_t* pq = qt + (int64_t)(bj * 128 + (t >> 3)) * ld_qt + bi * 128 + k16 * 16;
    const int64_t pass_step = 32 * ld_qt;
#pragma unroll
    for (int pass = 0; pass < 4; ++pass, pq += pass_step) {
      const int cl = pass * 32 + (t >> 3);
      if (!F && bj * 128 + cl >= cols) break;  // columns ascend with the pass
      const u32x4 w4 = *reinterpret_cast<const u32x4*>(tq + cl * 128 + (k16 ^ ((cl >> 2) & 7)) * 16);
      st_stream16<kNtWeightTStore>(pq, w4[0], w4[1], w4[2], w4[3]);
    }
    return;
  }
  const bool full_r = r0 + 16 <= rows;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int c = c0 + e;
    if (c >= cols) break;
    uint32_t d[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      d[k] = pack4_e4m3_grp(v[4 * k][e] * inv, v[4 * k + 1][e] * inv, v[4 * k + 2][e] * inv, v[4 * k + 3][e] * inv);
    uint8_t* tp = qt + (int64_t)c * ld_qt + r0;
    if (full_r) {
      st_stream16<kNtWeightTStore>(tp, d[0], d[1], d[2], d[3]);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (r0 + i < rows) tp[i] = (uint8_t)((d[i >> 2] >> (8 * (i & 3))) & 0xFF);
    }
  }
}

template <class In, int NTS, bool F>
__global__ __launch_bounds__(256) void k_quant_weight(const typename In::elem* __restrict__ w, int64_t ld_w,
                                                      int rows, int cols,
                                                      uint8_t* __restrict__ q, int64_t ld_q,
                                                      uint8_t* __restrict__ qt, int64_t ld_qt,
                                                      float* __restrict__ s, int64_t ld_s) {
  __shared__ uint32_t red[4];
  __shared__ __attribute__((aligned(16))) uint8_t tq[128 * 128];  // [column][row] codes of the block
  quant_weight_block<In, NTS, F>((int)blockIdx.y, (int)blockIdx.x, w, ld_w, rows, cols, q, ld_q, qt, ld_qt, s,
                                 ld_s, red, tq);
}

hipError_t launch_quant_weight(const void* w, bool w_bf16, int64_t rows, int64_t cols, int64_t ld_w,
                               uint8_t* q, int64_t ld_q, uint8_t* q_t, int64_t ld_qt,
                               float* s, int64_t ld_s, hipStream_t st) {
  const dim3 grid((uint32_t)((cols + 127) / 128), (uint32_t)((rows + 127) / 128));
  const bool nt = rows * cols > kNtCodeBytes, full = rows % 128 == 0 && cols % 128 == 0;
  auto go = [&](auto in, auto n, auto f) {
    typedef decltype(in) In;
    hipLaunchKernelGGL((k_quant_weight<In, decltype(n)::value, decltype(f)::value>), grid, dim3(256), 0, st,
                       (const typename In::elem*)w, ld_w, (int)rows, (int)cols, q, ld_q, q_t, ld_qt, s, ld_s);
  };
  using N0 = std::integral_constant<int, 0>;
  using N1 = std::integral_constant<int, 1>;
  using T = std::true_type;
  using Fa = std::false_type;
  if (w_bf16) {
    if (nt) full ? go(BF16In{}, N1{}, T{}) : go(BF16In{}, N1{}, Fa{});
    else full ? go(BF16In{}, N0{}, T{}) : go(BF16In{}, N0{}, Fa{});
  } else {
    if (nt) full ? go(F32In{}, N1{}, T{}) : go(F32In{}, N1{}, Fa{});
    else full ? go(F32In{}, N0{}, T{}) : go(F32In{}, N0{}, Fa{});
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fused quantize + transpose: one workgroup per 128-token x 128-channel tile.
// Thread t owns 8 consecutive tokens (8*(t/16) ..) of 8 consecutive channels
// (8*(t%16) ..): loads are 16-byte row segments, the per-channel max-abs is
// reduced over the 16 threads of a channel (xor 16/32 inside the wave, LDS
// across the 4 waves), and each channel's 8 codes are converted pairwise
// down the column, so they leave as one 8-byte segment of the q_t row.
//
// D (dual output): the same tile also yields the 1x128 row quantization -- a
// tile's 128 channels of one token are exactly one 1x128 group -- so X is
// read once for both the row codes q [rows, cols] and the transposed ones.
//
// F (full tiles): cols is a multiple of 128, and (not grouped) so is rows, so
// every tile is whole and the per-row and per-column bounds checks drop out.
// Grouped with F: the columns are whole; the rows past the expert's end load
// the expert's first row of the tile instead and are zeroed by a select, so
// no load sits in a branch of its own (in branches they were issued and
// waited for one by one).
//
// The transposed codes of a tile that spans 128 whole tokens are staged in
// LDS (one 128-byte row per channel), so that every global store writes 16
// bytes and 8 lanes together one whole 128-byte q_t row segment: written
// straight from registers, each segment would arrive as four 32-byte pieces
// from four waves (measured 26.5 -> 22 us for X [4096,7168], 95 -> 80 us for
// [16384,7168]).
//
// Each group's scale is computed once, not by every thread that holds part
// of the group (the correctly rounded divisions of group_scale dominated the
// kernel's vector work): a row group's by one lane of its 16-lane DPP row,
// then broadcast along the row; a column group's by one thread, handed to the
// others through LDS.  Row addresses advance by pointer increments, not by
// 64-bit multiplies per row.
//
// One 128-token x 128-channel tile (bi, bj) of the transposing quantizer;
// red (5 x 128 words: 4 rows of per-wave column maxima, then the column
// inverse scales) and tq (16 KB, 16-byte aligned) are the tile's LDS.
template <class In, bool G, bool D, bool F>
__device__ __forceinline__ void quant_transpose_block(int bi, int bj, const typename In::elem* __restrict__ x,
                                                      int64_t ld_x, int rows, int cols, uint8_t* __restrict__ qt,
                                                      int64_t ld_qt, float* __restrict__ st, int64_t ld_st,
                                                      const int32_t* __restrict__ offsets, int E,
                                                      uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ s,
                                                      int64_t ld_s, uint32_t (*red)[128], uint8_t* tq) {
  const int t = threadIdx.x;
  const int c8 = t & 15, rblk = t >> 4;
  // Output chunk bi (token columns [128 bi, 128 bi + 128) of q_t) comes from
  // input rows [rlo, rlo + 128), of which those below rhi exist.
  int rlo = bi * 128, rhi = rows;
  if (G) {
    // the expert whose padded chunks [start_e, start_e + ceil(m_e/128)) hold
    // bi, start_e = offsets[e]/128 + e (strictly increasing in e)
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (offsets[mid] / 128 + mid <= bi) lo = mid;
      else hi = mid - 1;
    }
    const int o0 = offsets[lo], o1 = offsets[lo + 1], start = o0 / 128 + lo;
    if (bi < start || bi >= start + (o1 - o0 + 127) / 128) return;  // a chunk no expert owns
    rlo = o0 + 128 * (bi - start);
    rhi = o1;
  }
  const int r0 = rlo + rblk * 8;           // first input row of this thread
  const int oc0 = bi * 128 + rblk * 8;     // its output token column
  const int c0 = bj * 128 + c8 * 8;
  float v[8][8];
  const typename In::elem* p = x + (int64_t)r0 * ld_x + c0;
  const typename In::elem* const p_first = x + (int64_t)rlo * ld_x + c0;  // a valid row of the tile
#pragma unroll
  for (int i = 0; i < 8; ++i, p += ld_x) {
    const int r = r0 + i;
    if (G && F) {
      const bool ok = r < rhi;
      In::template load8<kNtTransLoad>(ok ? p : p_first, v[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[i][e] = ok ? v[i][e] : 0.f;
      continue;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) v[i][e] = 0.f;
    if ((F && !G) || r < rhi) {
      if (F || c0 + 8 <= cols) {
        In::template load8<kNtTransLoad>(p, v[i]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (c0 + e < cols) v[i][e] = In::load1(p + e);
      }
    }
  }
  if (D) {
    // row groups: the 16 threads holding the tile's 8 rows r0..r0+7 form one
    // DPP row of a wave; lane c8 < 8 computes the scale of row r0 + c8 (lanes
    // 8-15 repeat rows 0-7), and lane i hands row i's inverse scale to the
    // whole DPP row
    uint32_t am[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t a = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) a = max(a, abs_bits(v[i][e]));
      am[i] = row16_max_u32(a);
    }
    uint32_t mine = am[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mine = (c8 & 7) == i ? am[i] : mine;
    float sc_m, iv_m;
    group_scale(__uint_as_float(mine), sc_m, iv_m);
    if (c8 < 8 && (F || r0 + c8 < rows)) s[(int64_t)(r0 + c8) * ld_s + bj] = sc_m;
    float ivr[8];
    ivr[0] = row_bcast<0>(iv_m); ivr[1] = row_bcast<1>(iv_m); ivr[2] = row_bcast<2>(iv_m);
    ivr[3] = row_bcast<3>(iv_m); ivr[4] = row_bcast<4>(iv_m); ivr[5] = row_bcast<5>(iv_m);
    ivr[6] = row_bcast<6>(iv_m); ivr[7] = row_bcast<7>(iv_m);
    uint8_t* qp = q + (int64_t)r0 * ld_q + c0;
#pragma unroll
    for (int i = 0; i < 8; ++i, qp += ld_q) {
      if (!F && r0 + i >= rows) break;
      const float iv = ivr[i];
      const uint32_t w0 = pack4_e4m3_grp(v[i][0] * iv, v[i][1] * iv, v[i][2] * iv, v[i][3] * iv);
      const uint32_t w1 = pack4_e4m3_grp(v[i][4] * iv, v[i][5] * iv, v[i][6] * iv, v[i][7] * iv);
      if (F || c0 + 8 <= cols) {
        *reinterpret_cast<uint2*>(qp) = make_uint2(w0, w1);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (c0 + e < cols) qp[e] = (uint8_t)(((e < 4 ? w0 : w1) >> (8 * (e & 3))) & 0xFF);
      }
    }
  }
  uint32_t m[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    uint32_t a = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = max(a, abs_bits(v[i][e]));
    a = max(a, (uint32_t)__shfl_xor((int)a, 16));
    a = max(a, (uint32_t)__shfl_xor((int)a, 32));
    m[e] = a;
  }
  const int wv = t >> 6;
  if ((t & 63) < 16) {
#pragma unroll
    for (int e = 0; e < 8; ++e) red[wv][c8 * 8 + e] = m[e];
  }
  __syncthreads();
  {
    // column group cl's scale, once: threads 0-127 take one column each
    // (128-255 compute the same values and store none)
    const int cl = t & 127;
    const uint32_t a = max(max(red[0][cl], red[1][cl]), max(red[2][cl], red[3][cl]));
    float sc, iv;
    group_scale(__uint_as_float(a), sc, iv);
    if (t < 128) {
      red[4][cl] = __float_as_uint(iv);
      if (F || bj * 128 + cl < cols) st[(int64_t)(bj * 128 + cl) * ld_st + bi] = sc;
    }
  }
  __syncthreads();
  float inv[8];
  {
    const u32x4 i0 = *reinterpret_cast<const u32x4*>(&red[4][c8 * 8]);
    const u32x4 i1 = *reinterpret_cast<const u32x4*>(&red[4][c8 * 8 + 4]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      inv[e] = __uint_as_float(i0[e]);
      inv[4 + e] = __uint_as_float(i1[e]);
    }
  }
  // grouped: rows past the expert's end are padding, stored as code 0 (their
  // values were loaded as 0)
  if (F || G || rlo + 128 <= rows) {
    // LDS: channel cl's 128 token codes at tq[128 cl]; its 8-byte token chunk
    // k at slot k ^ (2 (c8 & 7)), which spreads one wave's writes over the
    // banks and keeps chunk pairs (2k, 2k+1) adjacent and in order
    const int swz = 2 * (c8 & 7);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t d0 = pack4_e4m3_grp(v[0][e] * inv[e], v[1][e] * inv[e], v[2][e] * inv[e], v[3][e] * inv[e]);
      const uint32_t d1 = pack4_e4m3_grp(v[4][e] * inv[e], v[5][e] * inv[e], v[6][e] * inv[e], v[7][e] * inv[e]);
      *reinterpret_cast<uint2*>(tq + (c8 * 8 + e) * 128 + (rblk ^ swz) * 8) = make_uint2(d0, d1);
    }
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
      st_stream16<kNtTransStore>(pq, w[0], w[1], w[2], w[3]);
    }
    return;
  }
  // a partial last token tile: each channel's 8 codes straight from registers
  const bool full_r = r0 + 8 <= rows;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = c0 + e;
    if (!F && c >= cols) break;
    const uint32_t d0 = pack4_e4m3_grp(v[0][e] * inv[e], v[1][e] * inv[e], v[2][e] * inv[e], v[3][e] * inv[e]);
    const uint32_t d1 = pack4_e4m3_grp(v[4][e] * inv[e], v[5][e] * inv[e], v[6][e] * inv[e], v[7][e] * inv[e]);
    uint8_t* tp = qt + (int64_t)c * ld_qt + oc0;
    if (full_r) {
      st_stream8<kNtTransStore>(tp, d0, d1);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (r0 + i < rows) tp[i] = (uint8_t)((((i < 4) ? d0 : d1) >> (8 * (i & 3))) & 0xFF);
    }
  }
}

template <class In, bool G, bool D, bool F>
__global__ __launch_bounds__(256) void k_quant_transpose(const typename In::elem* __restrict__ x, int64_t ld_x,
                                                         int rows, int cols,
                                                         uint8_t* __restrict__ qt, int64_t ld_qt,
                                                         float* __restrict__ st, int64_t ld_st,
                                                         const int32_t* __restrict__ offsets, int E,
                                                         uint8_t* __restrict__ q, int64_t ld_q,
                                                         float* __restrict__ s, int64_t ld_s) {
  __shared__ __attribute__((aligned(16))) uint32_t red[5][128];
  __shared__ __attribute__((aligned(16))) uint8_t tq[128 * 128];  // [channel][token] codes of the tile
  quant_transpose_block<In, G, D, F>((int)blockIdx.y, (int)blockIdx.x, x, ld_x, rows, cols, qt, ld_qt, st, ld_st,
                                     offsets, E, q, ld_q, s, ld_s, red, tq);
}

template <class In, bool D>
static void launch_transpose_tiles(const void* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q_t,
                                   int64_t ld_qt, float* s_t, int64_t ld_st, uint8_t* q, int64_t ld_q, float* s,
                                   int64_t ld_s, hipStream_t st) {
  typedef typename In::elem T;
  const dim3 grid((uint32_t)((cols + 127) / 128), (uint32_t)((rows + 127) / 128));
  if (rows % 128 == 0 && cols % 128 == 0)
    hipLaunchKernelGGL((k_quant_transpose<In, false, D, true>), grid, dim3(256), 0, st, (const T*)x, ld_x, (int)rows,
                       (int)cols, q_t, ld_qt, s_t, ld_st, nullptr, 0, q, ld_q, s, ld_s);
  else
    hipLaunchKernelGGL((k_quant_transpose<In, false, D, false>), grid, dim3(256), 0, st, (const T*)x, ld_x,
                       (int)rows, (int)cols, q_t, ld_qt, s_t, ld_st, nullptr, 0, q, ld_q, s, ld_s);
}

hipError_t launch_quant_transpose(const void* x, bool x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                                  uint8_t* q_t, int64_t ld_qt, float* s_t, int64_t ld_st, hipStream_t st) {
  if (x_bf16)
    launch_transpose_tiles<BF16In, false>(x, rows, cols, ld_x, q_t, ld_qt, s_t, ld_st, nullptr, 0, nullptr, 0, st);
  else
    launch_transpose_tiles<F32In, false>(x, rows, cols, ld_x, q_t, ld_qt, s_t, ld_st, nullptr, 0, nullptr, 0, st);
  return hipGetLastError();
}

hipError_t launch_quant_act_transpose(const void* x, bool x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                                      uint8_t* q, int64_t ld_q, float* s, int64_t ld_s, uint8_t* q_t,
                                      int64_t ld_qt, float* s_t, int64_t ld_st, hipStream_t st) {
  if (x_bf16)
    launch_transpose_tiles<BF16In, true>(x, rows, cols, ld_x, q_t, ld_qt, s_t, ld_st, q, ld_q, s, ld_s, st);
  else
    launch_transpose_tiles<F32In, true>(x, rows, cols, ld_x, q_t, ld_qt, s_t, ld_st, q, ld_q, s, ld_s, st);
  return hipGetLastError();
}

hipError_t launch_quant_transpose_grouped(const void* x, bool x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                                          const int32_t* offsets, int64_t E, uint8_t* q_t, int64_t ld_qt,
                                          float* s_t, int64_t ld_st, hipStream_t st) {
  // one block per padded 128-token chunk of the capacity 128*(rows/128 + E)
  const dim3 grid((uint32_t)((cols + 127) / 128), (uint32_t)(rows / 128 + E));
  const bool fc = cols % 128 == 0;  // whole column tiles
  if (x_bf16) {
    if (fc)
      hipLaunchKernelGGL((k_quant_transpose<BF16In, true, false, true>), grid, dim3(256), 0, st, (const uint16_t*)x,
                         ld_x, (int)rows, (int)cols, q_t, ld_qt, s_t, ld_st, offsets, (int)E, nullptr, 0, nullptr, 0);
    else
      hipLaunchKernelGGL((k_quant_transpose<BF16In, true, false, false>), grid, dim3(256), 0, st, (const uint16_t*)x,
                         ld_x, (int)rows, (int)cols, q_t, ld_qt, s_t, ld_st, offsets, (int)E, nullptr, 0, nullptr, 0);
  } else {
    if (fc)
      hipLaunchKernelGGL((k_quant_transpose<F32In, true, false, true>), grid, dim3(256), 0, st, (const float*)x, ld_x,
                         (int)rows, (int)cols, q_t, ld_qt, s_t, ld_st, offsets, (int)E, nullptr, 0, nullptr, 0);
    else
      hipLaunchKernelGGL((k_quant_transpose<F32In, true, false, false>), grid, dim3(256), 0, st, (const float*)x, ld_x,
                         (int)rows, (int)cols, q_t, ld_qt, s_t, ld_st, offsets, (int)E, nullptr, 0, nullptr, 0);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Batched launch: several independent quantizations in one grid.  Each launch
// of a 25-90 MB quantizer pays the ramp-up and drain of its own HBM stream
// (a few us); in one grid the next job's blocks start while the previous
// job's last blocks drain.  Every block runs exactly the code of the single
// kernel it stands for (the block bodies above), so outputs are bit for bit
// those of the separate calls.  Jobs go to one of two grids by resource
// class: the activation quantizer needs ~30 VGPRs and no LDS and runs 8
// waves per SIMD, the tile quantizers (weight, transpose, dual) up to ~154
// VGPRs and 18.5 KB of LDS; one grid for both would hold the activation blocks
// to the tile blocks' occupancy (measured: X and W in one grid 44.7 us
// against 36.2 us for the two launches).
struct QBody {
  int variant;  // body and template arguments (see k_quant_batch)
  int gx;       // weight / transpose: tiles along the columns
  const void* x;
  int64_t ld_x;
  int rows, cols;
  uint8_t* q;
  int64_t ld_q;
  float* s;
  int64_t ld_s;
  uint8_t* qt;
  int64_t ld_qt;
  float* st;
  int64_t ld_st;
  int ngr, total;  // activation jobs: groups per row, groups in all
};
struct QBatch {
  QBody job[kMaxQuantJobs];
  int start[kMaxQuantJobs + 1];  // first block of each job, start[n] = grid size
  int n;
};

enum : int { kVAct = 0, kVWeight = 8, kVTrans = 16, kVDual = 20 };

template <bool TILES>
__global__ __launch_bounds__(256) void k_quant_batch(QBatch b) {
  __shared__ __attribute__((aligned(16))) uint32_t red[TILES ? 5 : 1][128];
  __shared__ __attribute__((aligned(16))) uint8_t tq[TILES ? 128 * 128 : 16];
  const int bid = (int)blockIdx.x;
  int j = 0;
  while (j + 1 < b.n && bid >= b.start[j + 1]) ++j;
  const QBody& J = b.job[j];
  const int vb = bid - b.start[j];
  const int bi = vb / J.gx, bj = vb - (vb / J.gx) * J.gx;
  const uint16_t* xb = (const uint16_t*)J.x;
  const float* xf = (const float*)J.x;
#define FP8Q_ACT_CASE(V, T, F, N, XP)                                                                     \
  case V: quant_act_block<T, F, N>(vb, XP, J.ld_x, J.q, J.ld_q, J.s, J.ld_s, J.cols, J.ngr, J.total); break;
#define FP8Q_W_CASE(V, T, N, F, XP)                                                                          \
  case V: quant_weight_block<T, N, F>(bi, bj, XP, J.ld_x, J.rows, J.cols, J.q, J.ld_q, J.qt, J.ld_qt, J.s,      \
                                      J.ld_s, &red[0][0], tq); break;
#define FP8Q_T_CASE(V, T, D, F, XP)                                                                      \
  case V: quant_transpose_block<T, false, D, F>(bi, bj, XP, J.ld_x, J.rows, J.cols, J.qt, J.ld_qt, J.st,   \
                                                J.ld_st, nullptr, 0, J.q, J.ld_q, J.s, J.ld_s, red, tq); break;
  if (!TILES) {
    switch (J.variant) {
    FP8Q_ACT_CASE(kVAct + 0, F32In, false, 0, xf)
    FP8Q_ACT_CASE(kVAct + 1, F32In, false, 1, xf)
    FP8Q_ACT_CASE(kVAct + 2, F32In, true, 0, xf)
    FP8Q_ACT_CASE(kVAct + 3, F32In, true, 1, xf)
    FP8Q_ACT_CASE(kVAct + 4, BF16In, false, 0, xb)
    FP8Q_ACT_CASE(kVAct + 5, BF16In, false, 1, xb)
    FP8Q_ACT_CASE(kVAct + 6, BF16In, true, 0, xb)
    FP8Q_ACT_CASE(kVAct + 7, BF16In, true, 1, xb)
    default: break;
    }
    return;
  }
  switch (J.variant) {
    FP8Q_W_CASE(kVWeight + 0, F32In, 0, false, xf)
    FP8Q_W_CASE(kVWeight + 1, F32In, 1, false, xf)
    FP8Q_W_CASE(kVWeight + 2, BF16In, 0, false, xb)
    FP8Q_W_CASE(kVWeight + 3, BF16In, 1, false, xb)
    FP8Q_W_CASE(kVWeight + 4, F32In, 0, true, xf)
    FP8Q_W_CASE(kVWeight + 5, F32In, 1, true, xf)
    FP8Q_W_CASE(kVWeight + 6, BF16In, 0, true, xb)
    FP8Q_W_CASE(kVWeight + 7, BF16In, 1, true, xb)
    FP8Q_T_CASE(kVTrans + 0, F32In, false, false, xf)
    FP8Q_T_CASE(kVTrans + 1, F32In, false, true, xf)
    FP8Q_T_CASE(kVTrans + 2, BF16In, false, false, xb)
    FP8Q_T_CASE(kVTrans + 3, BF16In, false, true, xb)
    FP8Q_T_CASE(kVDual + 0, F32In, true, false, xf)
    FP8Q_T_CASE(kVDual + 1, F32In, true, true, xf)
    FP8Q_T_CASE(kVDual + 2, BF16In, true, false, xb)
    FP8Q_T_CASE(kVDual + 3, BF16In, true, true, xb)
    default: break;
  }
#undef FP8Q_ACT_CASE
#undef FP8Q_W_CASE
#undef FP8Q_T_CASE
}

int64_t quant_batch_blocks(const QuantJob* jobs, int n) {
  int64_t blocks = 0;
  for (int i = 0; i < n; ++i) {
    const QuantJob& J = jobs[i];
    if (J.rows == 0 || J.cols == 0) continue;
    if (J.kind == 0) blocks += ((J.rows * ((J.cols + 127) / 128) + 4 * kActU - 1) / (4 * kActU) + 3) / 4;
    else blocks += ((J.cols + 127) / 128) * ((J.rows + 127) / 128);
  }
  return blocks;
}

template <bool TILES>
static hipError_t launch_batch_class(const QuantJob* jobs, int n, hipStream_t st) {
  QBatch b{};
  int m = 0;
  int64_t blocks = 0;
  for (int i = 0; i < n; ++i) {
    const QuantJob& J = jobs[i];
    if (J.rows == 0 || J.cols == 0 || (J.kind != 0) != TILES) continue;
    QBody& B = b.job[m];
    B.x = J.x; B.ld_x = J.ld_x; B.rows = (int)J.rows; B.cols = (int)J.cols;
    B.q = J.q; B.ld_q = J.ld_q; B.s = J.s; B.ld_s = J.ld_s;
    B.qt = J.q_t; B.ld_qt = J.ld_qt; B.st = J.s_t; B.ld_st = J.ld_st;
    B.gx = (int)((J.cols + 127) / 128);
    const int gy = (int)((J.rows + 127) / 128);
    const int bf = J.x_bf16 ? 1 : 0;
    const bool full = J.rows % 128 == 0 && J.cols % 128 == 0;
    int64_t nb = 0;
    if (J.kind == 0) {
      const int64_t ngr = (J.cols + 127) / 128, total = J.rows * ngr;
      const bool flat = J.cols % 128 == 0 && J.ld_x == J.cols && J.ld_q == J.cols && J.ld_s == ngr;
      const bool nt = J.rows * J.cols > kNtCodeBytes;
      B.variant = kVAct + 4 * bf + (flat ? 2 : 0) + (nt ? 1 : 0);
      B.ngr = (int)ngr;
      B.total = (int)total;
      B.gx = 1;
      nb = ((total + 4 * kActU - 1) / (4 * kActU) + 3) / 4;
    } else if (J.kind == 1) {
      B.variant = kVWeight + (full ? 4 : 0) + 2 * bf + (J.rows * J.cols > kNtCodeBytes ? 1 : 0);
      nb = (int64_t)B.gx * gy;
    } else {
      B.variant = (J.kind == 2 ? kVTrans : kVDual) + 2 * bf + (full ? 1 : 0);
      nb = (int64_t)B.gx * gy;
    }
    b.start[m] = (int)blocks;
    blocks += nb;
    ++m;
  }
  if (m == 0) return hipSuccess;
  b.start[m] = (int)blocks;
  b.n = m;
  hipLaunchKernelGGL(k_quant_batch<TILES>, dim3((uint32_t)blocks), dim3(256), 0, st, b);
  return hipGetLastError();
}

hipError_t launch_quant_batch(const QuantJob* jobs, int n, hipStream_t st) {
  if (quant_batch_blocks(jobs, n) > INT32_MAX) return hipErrorInvalidConfiguration;
  const hipError_t e = launch_batch_class<false>(jobs, n, st);
  if (e != hipSuccess) return e;
  return launch_batch_class<true>(jobs, n, st);
}

}  // namespace fp8q
