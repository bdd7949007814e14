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

template <class In, bool FLAT, int NTS>
__global__ __launch_bounds__(256) void k_quant_act(const typename In::elem* __restrict__ x, int64_t ld_x,
                                                   uint8_t* __restrict__ q, int64_t ld_q,
                                                   float* __restrict__ s, int64_t ld_s,
                                                   int cols, int ngr, int total) {
  const int lane = threadIdx.x & 63;
  const int wave = (int)((blockIdx.x * (uint32_t)blockDim.x + threadIdx.x) >> 6);
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
    const uint32_t w0 = pack4_e4m3(v[u][0] * inv, v[u][1] * inv, v[u][2] * inv, v[u][3] * inv);
    const uint32_t w1 = pack4_e4m3(v[u][4] * inv, v[u][5] * inv, v[u][6] * inv, v[u][7] * inv);
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

template <class In, int NTS>
__global__ __launch_bounds__(256) void k_quant_weight(const typename In::elem* __restrict__ w, int64_t ld_w,
                                                      int rows, int cols,
                                                      uint8_t* __restrict__ q, int64_t ld_q,
                                                      uint8_t* __restrict__ qt, int64_t ld_qt,
                                                      float* __restrict__ s, int64_t ld_s) {
  __shared__ uint32_t red[4];
  __shared__ __attribute__((aligned(16))) uint8_t tq[128 * 128];  // [column][row] codes of the block
  const int t = threadIdx.x;
  const int c4 = t & 31, rb = t >> 5;
  const int bi = blockIdx.y, bj = blockIdx.x;
  const int r0 = bi * 128 + rb * 16;
  const int c0 = bj * 128 + c4 * 4;
  const bool full_c = c0 + 4 <= cols;
  float v[16][4];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = r0 + i;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[i][e] = 0.f;
    if (r < rows) {
      const typename In::elem* p = w + (int64_t)r * ld_w + c0;
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
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = r0 + i;
    if (r >= rows) break;
    const uint32_t wd = pack4_e4m3(v[i][0] * inv, v[i][1] * inv, v[i][2] * inv, v[i][3] * inv);
    uint8_t* qp = q + (int64_t)r * ld_q + c0;
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
  if (bi * 128 + 128 <= rows) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t d[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        d[k] = pack4_e4m3(v[4 * k][e] * inv, v[4 * k + 1][e] * inv, v[4 * k + 2][e] * inv, v[4 * k + 3][e] * inv);
      *reinterpret_cast<u32x4*>(tq + (c4 * 4 + e) * 128 + (rb ^ (c4 & 7)) * 16) = u32x4{d[0], d[1], d[2], d[3]};
    }
    __syncthreads();
    const int k16 = t & 7;
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int cl = pass * 32 + (t >> 3);
      const int c = bj * 128 + cl;
      if (c >= cols) break;  // columns ascend with the pass
      const u32x4 w4 = *reinterpret_cast<const u32x4*>(tq + cl * 128 + (k16 ^ ((cl >> 2) & 7)) * 16);
      st_stream16<kNtWeightTStore>(qt + (int64_t)c * ld_qt + bi * 128 + k16 * 16, w4[0], w4[1], w4[2], w4[3]);
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
      d[k] = pack4_e4m3(v[4 * k][e] * inv, v[4 * k + 1][e] * inv, v[4 * k + 2][e] * inv, v[4 * k + 3][e] * inv);
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

hipError_t launch_quant_weight(const void* w, bool w_bf16, int64_t rows, int64_t cols, int64_t ld_w,
                               uint8_t* q, int64_t ld_q, uint8_t* q_t, int64_t ld_qt,
                               float* s, int64_t ld_s, hipStream_t st) {
  const dim3 grid((uint32_t)((cols + 127) / 128), (uint32_t)((rows + 127) / 128));
  const bool nt = rows * cols > kNtCodeBytes;
  if (w_bf16) {
    const uint16_t* wb = (const uint16_t*)w;
    if (nt)
      hipLaunchKernelGGL((k_quant_weight<BF16In, 1>), grid, dim3(256), 0, st, wb, ld_w, (int)rows, (int)cols, q,
                         ld_q, q_t, ld_qt, s, ld_s);
    else
      hipLaunchKernelGGL((k_quant_weight<BF16In, 0>), grid, dim3(256), 0, st, wb, ld_w, (int)rows, (int)cols, q,
                         ld_q, q_t, ld_qt, s, ld_s);
  } else {
    const float* wf = (const float*)w;
    if (nt)
      hipLaunchKernelGGL((k_quant_weight<F32In, 1>), grid, dim3(256), 0, st, wf, ld_w, (int)rows, (int)cols, q,
                         ld_q, q_t, ld_qt, s, ld_s);
    else
      hipLaunchKernelGGL((k_quant_weight<F32In, 0>), grid, dim3(256), 0, st, wf, ld_w, (int)rows, (int)cols, q,
                         ld_q, q_t, ld_qt, s, ld_s);
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
// F (full tiles, not grouped): rows and cols are multiples of 128, so every
// tile is whole and the per-row and per-column bounds checks drop out.
//
// The transposed codes of a tile that spans 128 whole tokens are staged in
// LDS (one 128-byte row per channel), so that every global store writes 16
// bytes and 8 lanes together one whole 128-byte q_t row segment: written
// straight from registers, each segment would arrive as four 32-byte pieces
// from four waves (measured 26.5 -> 22 us for X [4096,7168], 95 -> 80 us for
// [16384,7168]).
template <class In, bool G, bool D, bool F>
__global__ __launch_bounds__(256) void k_quant_transpose(const typename In::elem* __restrict__ x, int64_t ld_x,
                                                         int rows, int cols,
                                                         uint8_t* __restrict__ qt, int64_t ld_qt,
                                                         float* __restrict__ st, int64_t ld_st,
                                                         const int32_t* __restrict__ offsets, int E,
                                                         uint8_t* __restrict__ q, int64_t ld_q,
                                                         float* __restrict__ s, int64_t ld_s) {
  __shared__ uint32_t red[4][128];
  __shared__ __attribute__((aligned(16))) uint8_t tq[128 * 128];  // [channel][token] codes of the tile
  const int t = threadIdx.x;
  const int c8 = t & 15, rblk = t >> 4;
  const int bi = blockIdx.y, bj = blockIdx.x;
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
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = r0 + i;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[i][e] = 0.f;
    if (F || r < rhi) {
      const typename In::elem* p = x + (int64_t)r * ld_x + c0;
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
    // row groups: the 16 threads of a token row form one DPP row of a wave
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t a = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) a = max(a, abs_bits(v[i][e]));
      a = row16_max_u32(a);
      const int r = r0 + i;
      if (!F && r >= rows) continue;
      float sc, iv;
      group_scale(__uint_as_float(a), sc, iv);
      const uint32_t w0 = pack4_e4m3(v[i][0] * iv, v[i][1] * iv, v[i][2] * iv, v[i][3] * iv);
      const uint32_t w1 = pack4_e4m3(v[i][4] * iv, v[i][5] * iv, v[i][6] * iv, v[i][7] * iv);
      uint8_t* qp = q + (int64_t)r * ld_q + c0;
      if (F || c0 + 8 <= cols) {
        *reinterpret_cast<uint2*>(qp) = make_uint2(w0, w1);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (c0 + e < cols) qp[e] = (uint8_t)(((e < 4 ? w0 : w1) >> (8 * (e & 3))) & 0xFF);
      }
      if (c8 == 0) s[(int64_t)r * ld_s + bj] = sc;
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
  float inv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int cl = c8 * 8 + e;
    const uint32_t a = max(max(red[0][cl], red[1][cl]), max(red[2][cl], red[3][cl]));
    float sc;
    group_scale(__uint_as_float(a), sc, inv[e]);
    if (rblk == 0 && (F || c0 + e < cols)) st[(int64_t)(c0 + e) * ld_st + bi] = sc;
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
      const uint32_t d0 = pack4_e4m3(v[0][e] * inv[e], v[1][e] * inv[e], v[2][e] * inv[e], v[3][e] * inv[e]);
      const uint32_t d1 = pack4_e4m3(v[4][e] * inv[e], v[5][e] * inv[e], v[6][e] * inv[e], v[7][e] * inv[e]);
      *reinterpret_cast<uint2*>(tq + (c8 * 8 + e) * 128 + (rblk ^ swz) * 8) = make_uint2(d0, d1);
    }
    __syncthreads();
    // lane t writes bytes [16 k, 16 k + 16) of channel 32 pass + t/8, k = t%8
    const int k16 = t & 7;
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int cl = pass * 32 + (t >> 3);
      const int c = bj * 128 + cl;
      if (!F && c >= cols) break;  // channels ascend with the pass
      const u32x4 w = *reinterpret_cast<const u32x4*>(tq + cl * 128 + (k16 ^ ((cl >> 3) & 7)) * 16);
      st_stream16<kNtTransStore>(qt + (int64_t)c * ld_qt + bi * 128 + k16 * 16, w[0], w[1], w[2], w[3]);
    }
    return;
  }
  // a partial last token tile: each channel's 8 codes straight from registers
  const bool full_r = r0 + 8 <= rows;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = c0 + e;
    if (!F && c >= cols) break;
    const uint32_t d0 = pack4_e4m3(v[0][e] * inv[e], v[1][e] * inv[e], v[2][e] * inv[e], v[3][e] * inv[e]);
    const uint32_t d1 = pack4_e4m3(v[4][e] * inv[e], v[5][e] * inv[e], v[6][e] * inv[e], v[7][e] * inv[e]);
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
  if (x_bf16)
    hipLaunchKernelGGL((k_quant_transpose<BF16In, true, false, false>), grid, dim3(256), 0, st, (const uint16_t*)x, ld_x,
                       (int)rows, (int)cols, q_t, ld_qt, s_t, ld_st, offsets, (int)E, nullptr, 0, nullptr, 0);
  else
    hipLaunchKernelGGL((k_quant_transpose<F32In, true, false, false>), grid, dim3(256), 0, st, (const float*)x, ld_x,
                       (int)rows, (int)cols, q_t, ld_qt, s_t, ld_st, offsets, (int)E, nullptr, 0, nullptr, 0);
  return hipGetLastError();
}

}  // namespace fp8q
