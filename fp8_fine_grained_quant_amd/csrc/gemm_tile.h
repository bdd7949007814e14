// Output-tile assignment and LDS-staged epilogue shared by the GEMM kernels.
#pragma once

#include "device_common.h"
#include "launch.h"

namespace fp8q {

constexpr int kGroupM = 4;  // m-tiles per band of the tile order

struct TileCoord {
  int64_t m0;    // first output row of the tile
  int64_t mend;  // end of the rows this tile may write (M, or the expert's end)
  int n0;        // first output column
  int e;         // expert (grouped launches), else 0
};

// Maps this workgroup to an output tile; false when it has none (grouped
// launches size the grid for the worst case).
//
// Dispatch hands consecutive workgroup ids to the 8 XCDs in turn, so the ids
// are first renumbered to give each XCD one contiguous run of tile numbers;
// tile numbers then walk bands of kGroupM m-tiles column by column.  The
// workgroups of one XCD thus cover a compact block of the output and share
// their A rows and B columns in that XCD's L2.
// The coordinates depend only on the workgroup id, the launch arguments and
// the expert offsets, so they are the same in every lane; the compiler cannot
// always prove that through the expert walks below, and then keeps them in
// vector registers and wraps every buffer load that uses them in a loop over
// lanes (measured: 52 such loops in the grouped weight-gradient kernel).
// Reading them back from lane 0 makes them scalar again.
__device__ __forceinline__ int64_t uniform_i64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void make_uniform(TileCoord& tc) {
  tc.m0 = uniform_i64(tc.m0);
  tc.mend = uniform_i64(tc.mend);
  tc.n0 = __builtin_amdgcn_readfirstlane(tc.n0);
  tc.e = __builtin_amdgcn_readfirstlane(tc.e);
}

template <int BM, int BN, bool GROUPED>
__device__ __forceinline__ bool tile_coord(const GemmArgs& p, TileCoord& tc) {
  const int G = gridDim.x, bid = blockIdx.x;
  const int xcd = bid & 7, q8 = G >> 3, r8 = G & 7;
  const int t = xcd * q8 + min(xcd, r8) + (bid >> 3);
  const int tiles_n = (int)(p.N / BN);
  if (!GROUPED) {
    const int tiles_m = (int)((p.M + BM - 1) / BM);
    const int band = kGroupM * tiles_n;
    const int b = t / band, first_m = b * kGroupM;
    const int gm = min(tiles_m - first_m, kGroupM);
    const int in_band = t - b * band;
    tc.m0 = (int64_t)(first_m + in_band % gm) * BM;
    tc.n0 = (in_band / gm) * BN;
    tc.mend = p.M;
    tc.e = 0;
    return true;
  }
  if (p.k_grouped) {
    // grouped contraction: every expert owns a full M x N grid of tiles, and
    // tiles of different experts differ in work (the expert's token count).
    // Each XCD takes an equal share of every expert: the expert's tiles in
    // n-major order (m-tiles innermost) are cut into 8 contiguous runs whose
    // lengths differ by at most one, run x on XCD x, walked expert by expert,
    // so an XCD reads about 1/8 of each expert's X^T column blocks once and
    // shares the expert's dY^T rows among its workgroups.  (Taking the
    // experts in turns tile by tile instead measured 1.6x slower: the XCD's
    // L2 then holds no expert's operands long enough.  Whole n-slices per
    // XCD leave an XCD idle when the n-tile count is not a multiple of 8, as
    // with 28 tiles of 256 columns.)
    const int tiles_m = (int)((p.M + BM - 1) / BM);
    const int per_ex = tiles_m * tiles_n;
    const int slots = (per_ex + 7) / 8;  // workgroups per expert per XCD
    const int ew = (bid >> 3) / slots;   // position in this XCD's walk over the experts
    if (ew >= (int)p.E) return false;
    const int tl = (bid >> 3) - ew * slots;
    // each XCD starts its walk E/8 experts after the previous one, so that
    // at any moment the XCDs work on different experts (some storing a small
    // expert's gradient while others compute a large one's; measured 626 ->
    // 618 us for the 32-expert weight gradient)
    const int e = (int)((ew + (int64_t)xcd * ((p.E + 7) / 8)) % p.E);
    const int q = per_ex >> 3, r = per_ex & 7;
    if (tl >= q + (xcd < r ? 1 : 0)) return false;
    const int t = xcd * q + min(xcd, r) + tl;
    tc.m0 = (int64_t)(t % tiles_m) * BM;
    tc.n0 = (t / tiles_m) * BN;
    tc.mend = p.M;
    tc.e = e;
    make_uniform(tc);
    return true;
  }
  // grouped rows: tiles never straddle experts.  The grid is sized for the
  // worst case (a partial m-tile per expert), so the real tiles are counted
  // first and cut into 8 contiguous runs of near-equal length, run x on XCD x
  // (cutting the whole grid instead left the last XCDs without work: 616 real
  // tiles of 768 slots filled XCDs 0-5 and part of 6).
  int64_t total = 0;
  for (int e = 0; e < (int)p.E; ++e) total += (p.offsets[e + 1] - p.offsets[e] + BM - 1) / BM;
  total *= tiles_n;
  const int64_t q = total >> 3, rem = total & 7, slot = bid >> 3;
  if (slot >= q + (xcd < rem ? 1 : 0)) return false;
  const int64_t tg = xcd * q + min((int64_t)xcd, rem) + slot;
  int64_t base = 0, lo = 0, hi = 0, mt = 0;
  int e = 0;
  for (; e < (int)p.E; ++e) {
    lo = p.offsets[e];
    hi = p.offsets[e + 1];
    mt = (hi - lo + BM - 1) / BM;
    const int64_t cnt = mt * tiles_n;
    if (tg < base + cnt) break;
    base += cnt;
  }
  if (e >= (int)p.E) return false;
  const int64_t local = tg - base;
  tc.m0 = lo + (local % mt) * BM;
  tc.n0 = (int)(local / mt) * BN;
  tc.mend = hi;
  tc.e = e;
  make_uniform(tc);
  return true;
}

// NTS = 1 writes non-temporally: for outputs that are written once and read
// much later (the weight gradients), so they do not fill the caches with
// dirty lines that the kernels after them must write back (measured:
// grouped Wgrad 796 -> 618 us, and the kernel after it 521 -> 465 us).
//
// Writes one wave's WM x WN accumulator block to C, staged through the
// wave's private LDS region `ep` in passes of ER rows so that every global
// access is a full 16-byte row segment.  Rows at or beyond `mend` are not
// written.  Accumulator layout of sub-tile (i, j), lane l = 16 g + l16:
// TRL = 0 (A the matrix instruction's first operand): rows 16 i + 4 g + r,
// column 16 j + l16; TRL = 1 (B first): row 16 i + l16, columns
// 16 j + 4 g + r.
template <int TM, int TN, int OUT_F32, int ER, int NTS = 0, bool TRL = false>
__device__ __forceinline__ void store_tile(const float (&acc)[TM][TN][4], uint8_t* ep, const GemmArgs& p,
                                           int64_t row0, int64_t mend, int col0, int lane) {
  constexpr int WM = 16 * TM, WN = 16 * TN;
  constexpr int ES = OUT_F32 ? 4 : 2;
  constexpr int P = WN * ES + 16;       // padded LDS row pitch
  constexpr int CPR = WN * ES / 16;     // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;         // rows per store instruction
  constexpr int PASSES = WM / ER;
  static_assert(64 % CPR == 0 && ER % RPI == 0 && ER % 16 == 0 && WM % ER == 0, "epilogue store shape");
  const int g = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int pass = 0; pass < PASSES; ++pass) {
    if (pass) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the previous pass's LDS reads are done
      __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int i = pass * (ER / 16); i < (pass + 1) * (ER / 16); ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr (TRL) {
          const int rl = 16 * i + l16 - pass * ER, cl = 16 * j + 4 * g;
          if (OUT_F32) {
            *reinterpret_cast<float4*>(ep + rl * P + 4 * cl) =
                make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
          } else {
            const uint32_t lo = f32_to_bf16_rne(acc[i][j][0]) | (f32_to_bf16_rne(acc[i][j][1]) << 16);
            const uint32_t hi = f32_to_bf16_rne(acc[i][j][2]) | (f32_to_bf16_rne(acc[i][j][3]) << 16);
            *reinterpret_cast<uint2*>(ep + rl * P + 2 * cl) = make_uint2(lo, hi);
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int rl = 16 * i + 4 * g + r - pass * ER, cl = 16 * j + l16;
            if (OUT_F32)
              *reinterpret_cast<float*>(ep + rl * P + 4 * cl) = acc[i][j][r];
            else
              *reinterpret_cast<uint16_t*>(ep + rl * P + 2 * cl) = (uint16_t)f32_to_bf16_rne(acc[i][j][r]);
          }
        }
      }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
    __builtin_amdgcn_wave_barrier();
    // (row addresses by pointer increments: a 64-bit multiply per store was
    // most of the epilogue's address arithmetic)
    uint8_t* dst = reinterpret_cast<uint8_t*>(p.C) +
                   ((row0 + pass * ER + lane / CPR) * p.ldc + col0) * ES + 16 * (lane % CPR);
    const int64_t it_step = (int64_t)RPI * p.ldc * ES;
#pragma unroll
    for (int it = 0; it < ER / RPI; ++it, dst += it_step) {
      const int rl = it * RPI + lane / CPR, ch = lane % CPR;
      const int64_t row = row0 + pass * ER + rl;
      if (row >= mend) continue;
      const uint4 v = *reinterpret_cast<const uint4*>(ep + rl * P + 16 * ch);
      if (OUT_F32 && p.accumulate) {
        const float4 o = *reinterpret_cast<const float4*>(dst);
        float4 f = *reinterpret_cast<const float4*>(&v);
        f.x += o.x; f.y += o.y; f.z += o.z; f.w += o.w;
        *reinterpret_cast<float4*>(dst) = f;
      } else {
        st_stream16<NTS>(dst, v.x, v.y, v.z, v.w);
      }
    }
  }
}

// The epilogue with the output's own quantization fused in (BF16 output,
// accumulators in the TRL = 1 layout of store_tile: lane 16 g + l16 holds row
// 16 i + l16, columns 16 j + 4 g + r): every wave's strip is 128 columns wide
// and starts on a multiple of 128, so each of its rows holds exactly one 1x128
// group of the output, spread over the four lanes l16, l16 + 16, l16 + 32,
// l16 + 48.  Each value is first rounded to BF16 (RNE); the group's max-abs,
// scale and codes are then taken from those BF16 values with the quantizers'
// own arithmetic (group_scale, pack4_e4m3_grp), so the codes and scales equal
// what quant_act_1x128 computes from the stored BF16 output.  The BF16 values
// leave through store_tile (skipped when p.C is NULL); the scaled values are
// staged through the wave's LDS region in passes of 16 rows so that every
// code store is a full 16-byte row segment.  The accumulators are only read.
template <int TM, int TN, int ER>
__device__ __forceinline__ void store_tile_q(const float (&acc)[TM][TN][4], uint8_t* ep, const GemmArgs& p,
                                             int64_t row0, int64_t mend, int col0, int lane) {
  static_assert(TN == 8, "a wave's strip is one 128-column group wide");
  constexpr int P = 128 * 4 + 16;  // padded LDS row pitch of the scaled values
  const int g = lane >> 4, l16 = lane & 15;
  auto rounded = [](float v) { return bf16_to_f32(f32_to_bf16_rne(v)); };
  if (p.C != nullptr) {
    store_tile<TM, TN, 0, ER, 0, true>(acc, ep, p, row0, mend, col0, lane);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the staging area is read out
    __builtin_amdgcn_wave_barrier();
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {  // one 16-row sub-tile per pass
    if (i) {
      __builtin_amdgcn_s_waitcnt(0xC07F);
      __builtin_amdgcn_wave_barrier();
    }
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) m = max(m, abs_bits(rounded(acc[i][j][r])));
    m = max(m, (uint32_t)__shfl_xor((int)m, 16));  // the row's other three lanes
    m = max(m, (uint32_t)__shfl_xor((int)m, 32));
    float sc, inv;
    group_scale(__uint_as_float(m), sc, inv);
    const int64_t row = row0 + 16 * i + l16;
    if (g == 0 && row < mend) p.so[row * p.ld_so + (col0 >> 7)] = sc;
#pragma unroll
    for (int j = 0; j < TN; ++j)
      *reinterpret_cast<float4*>(ep + l16 * P + 4 * (16 * j + 4 * g)) =
          make_float4(rounded(acc[i][j][0]) * inv, rounded(acc[i][j][1]) * inv, rounded(acc[i][j][2]) * inv,
                      rounded(acc[i][j][3]) * inv);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_wave_barrier();
    // lane (rl = lane / 8, ch = lane % 8): 16 consecutive values of row rl
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int rl = it * 8 + (lane >> 3), ch = lane & 7;
      const int64_t orow = row0 + 16 * i + rl;
      const float4* src = reinterpret_cast<const float4*>(ep + rl * P + 64 * ch);
      const float4 v0 = src[0], v1 = src[1], v2 = src[2], v3 = src[3];
      if (orow >= mend) continue;
      const uint32_t w0 = pack4_e4m3_grp(v0.x, v0.y, v0.z, v0.w), w1 = pack4_e4m3_grp(v1.x, v1.y, v1.z, v1.w);
      const uint32_t w2 = pack4_e4m3_grp(v2.x, v2.y, v2.z, v2.w), w3 = pack4_e4m3_grp(v3.x, v3.y, v3.z, v3.w);
      st_stream16<0>(p.qo + orow * p.ld_qo + col0 + 16 * ch, w0, w1, w2, w3);
    }
  }
}

}  // namespace fp8q
