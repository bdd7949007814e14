// Block-scaled FP8 GEMM with FP32 promotion every 128-long K chunk (gfx950).
//
// What is computed ("DeepSeek FP8 Training", Fprop pipeline and the weight-
// and input-gradient lists; innerforce.co.kr excerpt of the DeepSeek-V3 report,
// paragraph after Figure 7 (a): dequantization folded into increased-precision
// accumulation; "unified E4M3 format" page, "Enhanced Numerical Stability":
// partial results promoted to FP32 registers at intervals):
//
//     C[m, n] = sum_kb  P_kb[m, n] * sA(m, kb) * sB(n, kb)
//
// where P_kb is the FP8 x FP8 product over the 128 K of chunk kb, computed by
// one v_mfma_f32_16x16x128_f8f6f4 per 16x16 sub-tile (so one MFMA is exactly
// one promotion interval), and the scale-and-add runs as FP32 FMAs on the
// vector ALU into accumulators kept in architectural VGPRs.
//
// Tiling (MI355X-first: 256 CUs, 64-wide waves, 160 KB LDS per CU):
//   * workgroup tile 256 x 128, 512 threads = 8 waves in a 4 x 2 grid, each
//     wave 64 x 64 (4 x 4 MFMA sub-tiles, 64 FP32 accumulators per lane);
//     two waves per SIMD so one wave's promotion FMAs issue under the other's
//     MFMAs;
//   * B (the operand every wave of a column shares) is staged through a
//     double-buffered LDS tile with a 144-byte row pitch (conflict-free 16-byte
//     reads across 16 rows); A goes from global memory straight into the MFMA
//     register layout, one chunk ahead;
//   * the chunk's A-row scales (and per-column B scales for Wgrad) are staged
//     in LDS beside the tile;
//   * the epilogue stages the tile through LDS so every global store is a full
//     16-byte row segment;
//   * tiles are renumbered so that the workgroups of one XCD (dispatch is
//     round-robin over the 8 XCDs) form a compact 2-D block of the output and
//     share A rows and B columns in that XCD's L2.
//
// Exact-accumulation variant (EXACT = true): gfx950's FP8 MFMA aligns the 8
// products of each group of 8 consecutive K to the largest one and truncates
// the others 13 bits below its exponent (measured), the analogue of the
// limited accumulation the pages report for H800 tensor cores.  The EXACT
// variant converts the codes exactly to BF16 (every E4M3 value is a BF16
// value) and runs four v_mfma_f32_16x16x32_bf16 per chunk, whose products are
// exact and whose sums are FP32; B is converted once per workgroup while it is
// staged in LDS, A once per wave per chunk.  Same promotion, same epilogue.
//
// MFMA operand layout used (the same permutation of the 128 K positions for A
// and B, which leaves every dot product unchanged): lane l supplies row l%16
// of the 16-row slice, bytes [16g, 16g+16) and [64+16g, 64+16g+16) of the
// chunk, g = l/16.  Result: lane l holds C[4g + r][l%16], r = 0..3.

#include "device_common.h"
#include "launch.h"

namespace fp8q {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int BM = 256, BN = 128, BK = 128;
constexpr int NWAVES = 8, NTHREADS = 512;
constexpr int WM = 64, WN = 64;      // wave tile
constexpr int BPITCH = 144;          // LDS row pitch of the B tile (bytes)
constexpr int GROUP_M = 4;           // m-tiles per band in the tile order

constexpr int BPITCH_X = BK * 2 + 16;  // row pitch of the BF16 B tile (exact variant)

constexpr int kEpiPitchBF16 = WN * 2 + 16;              // 144
constexpr int kEpiPitchF32 = WN * 4 + 16;               // 272

template <int OUT_F32, bool EXACT>
struct Lds {
  static constexpr int stage_b = BN * (EXACT ? BPITCH_X : BPITCH);
  static constexpr int b = 2 * stage_b;
  static constexpr int sa = 2 * BM * 4;
  static constexpr int sb = 2 * BN * 4;
  static constexpr int main = b + sa + sb;
  static constexpr int epi = NWAVES * WM * (OUT_F32 ? kEpiPitchF32 : kEpiPitchBF16);
  static constexpr int total = epi > main ? epi : main;
};

// 8 E4M3 codes (two dwords) -> 8 BF16 values, exactly (scale 1.0).
__device__ __forceinline__ v8bf fp8x8_to_bf16(uint32_t d0, uint32_t d1) {
  const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)d0, 1.0f, false);
  const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)d0, 1.0f, true);
  const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)d1, 1.0f, false);
  const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)d1, 1.0f, true);
  v8bf r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

__device__ __forceinline__ v8i make_frag(uint4 lo, uint4 hi) {
  v8i f;
  f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
  f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
  return f;
}

template <int SB_MODE, int OUT_F32, bool GROUPED, bool EXACT>
__global__ __launch_bounds__(NTHREADS) void k_gemm(GemmArgs p) {
  typedef Lds<OUT_F32, EXACT> L;
  __shared__ __attribute__((aligned(16))) uint8_t lds[L::total];
  uint8_t* ldsB = lds;
  float* ldsSa = reinterpret_cast<float*>(lds + L::b);
  float* ldsSb = reinterpret_cast<float*>(lds + L::b + L::sa);
  constexpr int kPitchB = EXACT ? BPITCH_X : BPITCH;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int l16 = lane & 15, g = lane >> 4;

  // ---- which output tile: XCD-aware renumbering of the workgroup id
  const int G = gridDim.x, bid = blockIdx.x;
  const int xcd = bid & 7, q8 = G >> 3, r8 = G & 7;
  const int t = xcd * q8 + min(xcd, r8) + (bid >> 3);
  const int tiles_n = (int)(p.N / BN);

  const uint8_t* B = p.B;
  const float* sb = p.sb;
  int64_t m0, mend;
  int n0;
  if (!GROUPED) {
    const int tiles_m = (int)((p.M + BM - 1) / BM);
    const int band = GROUP_M * tiles_n;
    const int b = t / band, first_m = b * GROUP_M;
    const int gm = min(tiles_m - first_m, GROUP_M);
    const int in_band = t - b * band;
    const int tm = first_m + in_band % gm;
    const int tn = in_band / gm;
    m0 = (int64_t)tm * BM;
    n0 = tn * BN;
    mend = p.M;
  } else {
    // walk the experts' tile counts; tiles never straddle experts
    int64_t base = 0;
    int e = 0;
    int64_t lo = 0, hi = 0, mt = 0;
    for (; e < (int)p.E; ++e) {
      lo = p.offsets[e];
      hi = p.offsets[e + 1];
      mt = (hi - lo + BM - 1) / BM;
      const int64_t cnt = mt * tiles_n;
      if (t < base + cnt) break;
      base += cnt;
    }
    if (e >= (int)p.E) return;  // more workgroups than tiles: nothing to do
    const int64_t local = t - base;
    const int64_t tm = local % mt, tn = local / mt;
    m0 = lo + tm * BM;
    n0 = (int)tn * BN;
    mend = hi;
    B += (int64_t)e * p.b_estride;
    sb += (int64_t)e * p.sb_estride;
  }

  const int nk = (int)(p.K / BK);

  // ---- per-lane A row pointers (rows beyond the tile's end are clamped to the
  // last valid row: they are loaded but never stored)
  const uint8_t* pa[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int64_t row = m0 + wm * WM + 16 * i + l16;
    row = row < mend ? row : mend - 1;
    pa[i] = p.A + row * p.lda + 16 * g;
  }
  // ---- B loader: thread -> (row, 16-byte column chunk), two rows 64 apart
  const int bl_row = tid >> 3, bl_c = tid & 7;
  const uint8_t* pb0 = B + (int64_t)(n0 + bl_row) * p.ldb + 16 * bl_c;
  const uint8_t* pb1 = pb0 + 64 * p.ldb;
  const int lds_b0 = bl_row * kPitchB + (EXACT ? 32 : 16) * bl_c;
  const int lds_b1 = lds_b0 + 64 * kPitchB;
  // ---- scale loaders
  const float* psa = nullptr;
  if (tid < BM) {
    int64_t row = m0 + tid;
    row = row < mend ? row : mend - 1;
    psa = p.sa + row * p.ld_sa;
  }
  const float* psb_row = nullptr;
  if (SB_MODE == kSbRow && tid >= BM && tid < BM + BN) psb_row = sb + (int64_t)(n0 + tid - BM) * p.sb_rs;
  const float* psb_blk = sb + (int64_t)(n0 / 128) * p.sb_rs;  // block mode: + kb * sb_cs

  float acc[4][4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.f;

  v8i a0[4], a1[4];
  uint4 bst0, bst1;
  float sav = 0.f, sbv = 0.f, sbk_next = 0.f;

  auto load_a = [&](v8i (&a)[4], int kb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint8_t* q = pa[i] + (int64_t)kb * BK;
      uint4 lo = *reinterpret_cast<const uint4*>(q);
      uint4 hi = *reinterpret_cast<const uint4*>(q + 64);
      a[i] = make_frag(lo, hi);
    }
  };
  auto load_stage = [&](int kb) {
    bst0 = *reinterpret_cast<const uint4*>(pb0 + (int64_t)kb * BK);
    bst1 = *reinterpret_cast<const uint4*>(pb1 + (int64_t)kb * BK);
    if (psa) sav = psa[kb];
    if (SB_MODE == kSbRow && psb_row) sbv = psb_row[kb];
    if (SB_MODE == kSbBlock) sbk_next = psb_blk[(int64_t)kb * p.sb_cs];
  };
  auto store_stage = [&](int stage) {
    if (EXACT) {
      const v8bf c0 = fp8x8_to_bf16(bst0.x, bst0.y), c1 = fp8x8_to_bf16(bst0.z, bst0.w);
      const v8bf c2 = fp8x8_to_bf16(bst1.x, bst1.y), c3 = fp8x8_to_bf16(bst1.z, bst1.w);
      *reinterpret_cast<v8bf*>(ldsB + stage * L::stage_b + lds_b0) = c0;
      *reinterpret_cast<v8bf*>(ldsB + stage * L::stage_b + lds_b0 + 16) = c1;
      *reinterpret_cast<v8bf*>(ldsB + stage * L::stage_b + lds_b1) = c2;
      *reinterpret_cast<v8bf*>(ldsB + stage * L::stage_b + lds_b1 + 16) = c3;
    } else {
      *reinterpret_cast<uint4*>(ldsB + stage * L::stage_b + lds_b0) = bst0;
      *reinterpret_cast<uint4*>(ldsB + stage * L::stage_b + lds_b1) = bst1;
    }
    if (psa) ldsSa[stage * BM + tid] = sav;
    if (SB_MODE == kSbRow && psb_row) ldsSb[stage * BN + tid - BM] = sbv;
  };

  auto compute = [&](const v8i (&a)[4], int stage, float sbk) {
    const uint8_t* bs = ldsB + stage * L::stage_b;
    float sc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 s4 = *reinterpret_cast<const float4*>(ldsSa + stage * BM + wm * WM + 16 * i + 4 * g);
      if (SB_MODE == kSbBlock) {
        sc[i][0] = s4.x * sbk; sc[i][1] = s4.y * sbk; sc[i][2] = s4.z * sbk; sc[i][3] = s4.w * sbk;
      } else {
        sc[i][0] = s4.x; sc[i][1] = s4.y; sc[i][2] = s4.z; sc[i][3] = s4.w;
      }
    }
    // exact variant: the wave's A fragments as BF16, four quarters of 8 K each
    v8bf ax[4][4];
    if (EXACT) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) ax[i][qq] = fp8x8_to_bf16((uint32_t)a[i][2 * qq], (uint32_t)a[i][2 * qq + 1]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int brow = wn * WN + 16 * j + l16;
      v8i b;
      v8bf bx[4];
      if (EXACT) {
        // quarter qq of lane group g covers K [16g + 8qq, +8) for qq < 2 and
        // [64 + 16g + 8(qq-2), +8) for qq >= 2, matching the A fragment order
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const int k0 = (qq < 2 ? 0 : 64) + 16 * g + 8 * (qq & 1);
          bx[qq] = *reinterpret_cast<const v8bf*>(bs + brow * BPITCH_X + 2 * k0);
        }
      } else {
        const uint4 lo = *reinterpret_cast<const uint4*>(bs + brow * BPITCH + 16 * g);
        const uint4 hi = *reinterpret_cast<const uint4*>(bs + brow * BPITCH + 64 + 16 * g);
        b = make_frag(lo, hi);
      }
      float sbj = 1.f;
      if (SB_MODE == kSbRow) sbj = ldsSb[stage * BN + brow];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v4f pp = {0.f, 0.f, 0.f, 0.f};
        if (EXACT) {
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) pp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ax[i][qq], bx[qq], pp, 0, 0, 0);
        } else {
          pp = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[i], b, pp, 0, 0, 0, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float s = SB_MODE == kSbRow ? sc[i][r] * sbj : sc[i][r];
          acc[i][j][r] = __builtin_fmaf(pp[r], s, acc[i][j][r]);
        }
      }
    }
  };

  // ---- prologue
  load_stage(0);
  load_a(a0, 0);
  store_stage(0);
  float sbk_cur = sbk_next;
  __syncthreads();

  // ---- main loop, unrolled by two so the A register sets alternate
  for (int kb = 0; kb < nk; kb += 2) {
    {
      const bool more = kb + 1 < nk;
      if (more) {
        load_stage(kb + 1);
        load_a(a1, kb + 1);
      }
      compute(a0, 0, sbk_cur);
      if (more) store_stage(1);
      sbk_cur = sbk_next;
      __syncthreads();
      if (!more) break;
    }
    {
      const bool more = kb + 2 < nk;
      if (more) {
        load_stage(kb + 2);
        load_a(a0, kb + 2);
      }
      compute(a1, 1, sbk_cur);
      if (more) store_stage(0);
      sbk_cur = sbk_next;
      __syncthreads();
    }
  }

  // ---- epilogue: stage this wave's 64x64 tile in LDS, then 16-byte row stores
  if (!OUT_F32) {
    uint8_t* ep = lds + w * (WM * kEpiPitchBF16);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rl = 16 * i + 4 * g + r, cl = 16 * j + l16;
          *reinterpret_cast<uint16_t*>(ep + rl * kEpiPitchBF16 + 2 * cl) = (uint16_t)f32_to_bf16_rne(acc[i][j][r]);
        }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes done
    __builtin_amdgcn_wave_barrier();
    uint16_t* C = reinterpret_cast<uint16_t*>(p.C);
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int rl = it * 8 + (lane >> 3), ch = lane & 7;
      const int64_t row = m0 + wm * WM + rl;
      const uint4 v = *reinterpret_cast<const uint4*>(ep + rl * kEpiPitchBF16 + 16 * ch);
      if (row < mend) *reinterpret_cast<uint4*>(C + row * p.ldc + n0 + wn * WN + 8 * ch) = v;
    }
  } else {
    uint8_t* ep = lds + w * (WM * kEpiPitchF32);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rl = 16 * i + 4 * g + r, cl = 16 * j + l16;
          *reinterpret_cast<float*>(ep + rl * kEpiPitchF32 + 4 * cl) = acc[i][j][r];
        }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    float* C = reinterpret_cast<float*>(p.C);
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int rl = it * 4 + (lane >> 4), ch = lane & 15;
      const int64_t row = m0 + wm * WM + rl;
      float4 v = *reinterpret_cast<const float4*>(ep + rl * kEpiPitchF32 + 16 * ch);
      if (row < mend) {
        float4* dst = reinterpret_cast<float4*>(C + row * p.ldc + n0 + wn * WN + 4 * ch);
        if (p.accumulate) {
          const float4 o = *dst;
          v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
        }
        *dst = v;
      }
    }
  }
}

template <int SB_MODE, int OUT_F32, bool GROUPED, bool EXACT>
static hipError_t launch_one(const GemmArgs& a, hipStream_t st) {
  int64_t tiles;
  const int64_t tiles_n = a.N / BN;
  if (!GROUPED)
    tiles = ((a.M + BM - 1) / BM) * tiles_n;
  else
    tiles = ((a.M + BM - 1) / BM + a.E) * tiles_n;  // upper bound: one partial tile per expert
  if (tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL((k_gemm<SB_MODE, OUT_F32, GROUPED, EXACT>), dim3((uint32_t)tiles), dim3(NTHREADS), 0, st, a);
  return hipGetLastError();
}

template <bool EXACT>
static hipError_t launch_mode(const GemmArgs& a, hipStream_t st) {
  const bool grouped = a.offsets != nullptr;
  if (a.sb_mode == kSbRow) {
    // per-column B scales: the weight-gradient product, FP32 output
    return launch_one<kSbRow, 1, false, EXACT>(a, st);
  }
  if (grouped)
    return a.out_f32 ? launch_one<kSbBlock, 1, true, EXACT>(a, st) : launch_one<kSbBlock, 0, true, EXACT>(a, st);
  return a.out_f32 ? launch_one<kSbBlock, 1, false, EXACT>(a, st) : launch_one<kSbBlock, 0, false, EXACT>(a, st);
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st) {
  return a.exact ? launch_mode<true>(a, st) : launch_mode<false>(a, st);
}

}  // namespace fp8q
