// Exact-accumulation variant of the block-scaled FP8 GEMM (gfx950): the
// `_exact` entry points.
//
// What is computed is the same as the FP8 kernel's ("DeepSeek FP8 Training",
// Fprop pipeline and the weight- and input-gradient lists; innerforce.co.kr
// excerpt of the DeepSeek-V3 report, paragraph after Figure 7 (a):
// dequantization folded into increased-precision accumulation; "unified E4M3
// format" page, "Enhanced Numerical Stability": partial results promoted to
// FP32 registers at intervals):
//
//     C[m, n] = sum_kb  P_kb[m, n] * sA(m, kb) * sB(n, kb)
//
// gfx950's FP8 matrix instruction aligns the 8 products of each group of 8
// consecutive K to the largest one and truncates the others 13 bits below
// its exponent (measured), the analogue of the limited accumulation the pages
// report for H800 tensor cores.  This kernel converts the codes exactly to
// BF16 (every E4M3 value is a BF16 value) and forms P_kb with four
// v_mfma_f32_16x16x32_bf16 per 16x16 sub-tile, whose products are exact and
// whose sums are FP32; the promotion is the FP8 kernel's (one FMA per element
// and chunk into FP32 accumulators).
//
// Tiling: workgroup tile 256 x 128, four waves of 64 x 128 (4 x 8 sub-tiles).
// B, shared by the waves, is converted to BF16 once per workgroup while it is
// staged in a double-buffered LDS tile (272-byte row pitch: conflict-free
// 16-byte reads across 16 rows); A, private to a wave, goes from global memory
// into registers one chunk ahead and is converted per wave.  The chunk's
// A-row scales (and per-column B scales for Wgrad) are staged in LDS beside
// the tile; the epilogue stages the tile through LDS so every global store is
// a full 16-byte row segment; tiles are renumbered so that the workgroups of
// one XCD form a compact block of the output.
//
// Operand layout (the same permutation of the 128 K positions for A and B,
// which leaves every dot product unchanged): lane l supplies row l%16 of the
// 16-row slice, bytes [16g, 16g+16) and [64+16g, 64+16g+16) of the chunk,
// g = l/16, as four quarters of 8 K.  Result: lane l holds C[4g + r][l%16].

#include "device_common.h"
#include "launch.h"

namespace fp8q {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int BK = 128;          // one chunk = one promotion interval
constexpr int kMaxChunks = 1024; // contraction length limit: 1024 chunks of 128
constexpr int BPITCH_X = 272;    // LDS row pitch of the BF16 B tile
[[maybe_unused]] constexpr int GROUP_M = 4;  // m-tiles per band in the tile order

// Tile configuration: WAVES_M x WAVES_N waves, each TM x TN MFMA sub-tiles of 16 x 16.
template <int WAVES_M_, int WAVES_N_, int TM_, int TN_>
struct Cfg {
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, TM = TM_, TN = TN_;
  static constexpr int NWAVES = WAVES_M * WAVES_N, NT = 64 * NWAVES;
  static constexpr int WM = 16 * TM, WN = 16 * TN;
  static constexpr int BM = WAVES_M * WM, BN = WAVES_N * WN;
  static_assert(NT >= BM, "one A-scale load per thread");
  static_assert(NT >= BN, "one B-scale load per thread");
  static_assert((BN * 8) % NT == 0, "B tile loads split evenly");
  static_assert(BN <= 128 && 128 % BN == 0, "a tile's columns share one 128-block");
};

typedef Cfg<4, 1, 4, 8> DefaultCfg;   // 256 x 128, 4 waves of 64 x 128

// LDS of one workgroup: two stages, each with its own arrays (BF16 B tile,
// A scales, B scales); the epilogue has its own staging area (FP32 tiles go
// out in two passes of half the rows).
template <class C, int OUT_F32>
struct Lds {
  static constexpr int stage_b = C::BN * BPITCH_X;  // BF16 rows with a padded pitch
  static constexpr int stages = 2;                  // pipeline depth (chunks in flight + 1)
  static constexpr int epi_pitch = C::WN * (OUT_F32 ? 4 : 2) + 16;
  static constexpr int epi_passes = OUT_F32 ? 2 : 1;
  static constexpr int epi_rows = C::WM / epi_passes;
  static constexpr int epi = C::NWAVES * epi_rows * epi_pitch;
  // scale arrays: every wave's 64 lanes write one slot each (spare slots park
  // the values of lanes without a row/column of their own)
  static constexpr int sa_len = (C::BM > C::NWAVES * 64 ? C::BM : C::NWAVES * 64) + 4;
  static constexpr int sb_len = (C::BN > C::NWAVES * 64 ? C::BN : C::NWAVES * 64) + 4;
  static constexpr int total = stages * (stage_b + 4 * sa_len + 4 * sb_len) + epi;
  static_assert(total <= 160 * 1024, "LDS budget of one CU");
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

template <class C, int SB_MODE, int OUT_F32, bool GROUPED>
__global__ __launch_bounds__(C::NT) void k_gemm(GemmArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  constexpr int BM = C::BM, BN = C::BN, WM = C::WM, WN = C::WN, TM = C::TM, TN = C::TN, NT = C::NT;
  constexpr int UB = BN * 8 / NT;  // 16-byte B units per thread per chunk
  typedef Lds<C, OUT_F32> L;
  constexpr int NS = L::stages, D = NS - 1;  // stages, prefetch distance in chunks
  constexpr int S2 = NS > 2 ? 1 : 0;           // third stage present
  __shared__ __attribute__((aligned(16))) uint8_t ldsB0[L::stage_b];
  __shared__ __attribute__((aligned(16))) uint8_t ldsB1[L::stage_b];
  __shared__ __attribute__((aligned(16))) uint8_t ldsB2[S2 ? L::stage_b : 16];
  __shared__ __attribute__((aligned(16))) float ldsSa0[L::sa_len];  // [BM..]: parking slots
  __shared__ __attribute__((aligned(16))) float ldsSa1[L::sa_len];
  __shared__ __attribute__((aligned(16))) float ldsSa2[S2 ? L::sa_len : 4];
  __shared__ __attribute__((aligned(16))) float ldsSb0[L::sb_len];
  __shared__ __attribute__((aligned(16))) float ldsSb1[L::sb_len];
  __shared__ __attribute__((aligned(16))) float ldsSb2[S2 ? L::sb_len : 4];
  __shared__ __attribute__((aligned(16))) uint8_t ldsE[L::epi];
  __shared__ float ldsSbk[kMaxChunks];  // block mode: the tile's B scale of every chunk
  auto stB = [&](int stage) { return stage == 0 ? ldsB0 : stage == 1 ? ldsB1 : ldsB2; };
  auto stSa = [&](int stage) { return stage == 0 ? ldsSa0 : stage == 1 ? ldsSa1 : ldsSa2; };
  auto stSb = [&](int stage) { return stage == 0 ? ldsSb0 : stage == 1 ? ldsSb1 : ldsSb2; };
  constexpr int kPitchB = BPITCH_X;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, provably uniform
  const int wm = w / C::WAVES_N, wn = w % C::WAVES_N;
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
  const uint8_t* pa[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    int64_t row = m0 + wm * WM + 16 * i + l16;
    row = row < mend ? row : mend - 1;
    pa[i] = p.A + row * p.lda + 16 * g;
  }
  // ---- B loader: unit u = tid + NT*q -> (row u/8, chunk u%8), through
  // registers, converted to BF16 on the way into LDS
  const uint8_t* pb[UB];
  int lds_b[UB];
#pragma unroll
  for (int q = 0; q < UB; ++q) {
    const int u = tid + NT * q, row = u >> 3, c = u & 7;
    pb[q] = B + (int64_t)(n0 + row) * p.ldb + 16 * c;
    lds_b[q] = row * kPitchB + 32 * c;
  }
  // ---- scale loaders.  Every thread issues the same loads (threads without a
  // scale of their own read a clamped, valid address and park the value in a
  // spare LDS slot), so the main loop has no divergent branches.
  int64_t sa_row = m0 + (tid & (BM - 1));
  sa_row = sa_row < mend ? sa_row : mend - 1;
  const float* psa = p.sa + sa_row * p.ld_sa;
  const int lds_sa_slot = tid < BM ? tid : BM;  // BM: parking slot (never read)
  const float* psb_row = sb + (int64_t)(n0 + (tid & (BN - 1))) * p.sb_rs;
  const int lds_sb_slot = tid < BN ? tid : BN;
  const float* psb_blk = sb + (int64_t)(n0 / 128) * p.sb_rs;  // block mode: + kb * sb_cs

  float acc[TM][TN][4];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.f;

  v8i abuf[NS][TM];     // A fragments of the chunks in flight, one set per stage
  uint4 bst[UB];        // B staging registers
  float sav = 0.f, sbv = 0.f;

  auto load_a = [&](v8i (&a)[TM], int kb) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const uint8_t* q = pa[i] + (int64_t)kb * BK;
      const uint4 lo = *reinterpret_cast<const uint4*>(q);
      const uint4 hi = *reinterpret_cast<const uint4*>(q + 64);
      a[i] = make_frag(lo, hi);
    }
  };
  // load chunk kb into registers (store_stage converts and writes them)
  auto load_stage = [&](int kb, int stage) {
    (void)stage;
#pragma unroll
    for (int q = 0; q < UB; ++q) bst[q] = *reinterpret_cast<const uint4*>(pb[q] + (int64_t)kb * BK);
    sav = psa[kb];
    if (SB_MODE == kSbRow) sbv = psb_row[kb];
  };
  auto store_stage = [&](int stage) {
    uint8_t* dst = stB(stage);
#pragma unroll
    for (int q = 0; q < UB; ++q) {
      *reinterpret_cast<v8bf*>(dst + lds_b[q]) = fp8x8_to_bf16(bst[q].x, bst[q].y);
      *reinterpret_cast<v8bf*>(dst + lds_b[q] + 16) = fp8x8_to_bf16(bst[q].z, bst[q].w);
    }
    stSa(stage)[lds_sa_slot] = sav;  // parked values land in the spare slot
    if (SB_MODE == kSbRow) stSb(stage)[lds_sb_slot] = sbv;
  };

  auto compute = [&](const v8i (&a)[TM], int stage, int c) {
    const float sbk = SB_MODE == kSbBlock ? ldsSbk[c] : 1.f;
    const uint8_t* bs = stB(stage);
    float sc[TM][4];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const float4 s4 = *reinterpret_cast<const float4*>(stSa(stage) + wm * WM + 16 * i + 4 * g);
      if (SB_MODE == kSbBlock) {
        sc[i][0] = s4.x * sbk; sc[i][1] = s4.y * sbk; sc[i][2] = s4.z * sbk; sc[i][3] = s4.w * sbk;
      } else {
        sc[i][0] = s4.x; sc[i][1] = s4.y; sc[i][2] = s4.z; sc[i][3] = s4.w;
      }
    }
    // the wave's A fragments as BF16, four quarters of 8 K each
    v8bf ax[TM][4];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) ax[i][qq] = fp8x8_to_bf16((uint32_t)a[i][2 * qq], (uint32_t)a[i][2 * qq + 1]);
    // Software pipeline over the TN column sub-tiles: the TM MFMAs of column
    // j+1 are issued before the promotion FMAs of column j, so the matrix core
    // works while the vector ALU scales and accumulates the previous partials.
    auto mfma_col = [&](int j, v4f (&pp)[TM]) {
      const int brow = wn * WN + 16 * j + l16;
      // quarter qq of lane group g covers K [16g + 8qq, +8) for qq < 2 and
      // [64 + 16g + 8(qq-2), +8) for qq >= 2, matching the A fragment order
      v8bf bx[4];
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int k0 = (qq < 2 ? 0 : 64) + 16 * g + 8 * (qq & 1);
        bx[qq] = *reinterpret_cast<const v8bf*>(bs + brow * BPITCH_X + 2 * k0);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        pp[i] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) pp[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ax[i][qq], bx[qq], pp[i], 0, 0, 0);
      }
    };
    auto promote_col = [&](int j, const v4f (&pp)[TM]) {
      float sbj = 1.f;
      if (SB_MODE == kSbRow) sbj = stSb(stage)[wn * WN + 16 * j + l16];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float s = SB_MODE == kSbRow ? sc[i][r] * sbj : sc[i][r];
          acc[i][j][r] = __builtin_fmaf(pp[i][r], s, acc[i][j][r]);
        }
    };
    v4f pa0[TM], pa1[TM];
    mfma_col(0, pa0);
#pragma unroll
    for (int j = 1; j < TN; ++j) {
      if (j & 1) {
        mfma_col(j, pa1);
        promote_col(j - 1, pa0);
      } else {
        mfma_col(j, pa0);
        promote_col(j - 1, pa1);
      }
    }
    if (TN & 1) promote_col(TN - 1, pa0); else promote_col(TN - 1, pa1);
  };

  // ---- pipeline.  Chunk c lives in stage c % NS.  Iteration c loads chunk
  // c + D into registers, computes chunk c, writes chunk c+1 (loaded the
  // iteration before) into its stage and synchronises the workgroup.  The
  // barrier is a bare s_barrier with compiler memory fences: __syncthreads()
  // would also wait for every outstanding global load, i.e. drain the
  // prefetch.  Past the last chunk the index is clamped (the last chunk is
  // re-read into a stage nobody reads again), so every iteration is the same.
  auto block_sync = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS stores are done
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  auto issue = [&](int c, int stage) {
    load_stage(c, stage);
    load_a(abuf[stage], c);
  };

  // prologue: the tile's block-mode B scales of all chunks go to LDS once;
  // chunks 0 .. D-1 in flight, chunk 0 published
  if (SB_MODE == kSbBlock)
    for (int q = tid; q < nk; q += NT) ldsSbk[q] = psb_blk[(int64_t)q * p.sb_cs];
#pragma unroll
  for (int c = 0; c < D; ++c) issue(min(c, nk - 1), c);
  store_stage(0);
  block_sync();

  // The empty asm memory barriers stop the IR optimizers from moving loads of
  // the next chunks down to their uses, and sched_barrier(0) stops the
  // machine scheduler from pulling those uses up; either would expose the full
  // memory latency every chunk.
  auto step = [&](int c, int u) {  // u = c % NS, a compile-time constant at every call
    issue(min(c + D, nk - 1), (u + D) % NS);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    compute(abuf[u], u, c);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    store_stage((u + 1) % NS);
    block_sync();
  };
  int kb = 0;
  for (; kb + NS <= nk; kb += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) step(kb + u, u);
  }
#pragma unroll
  for (int u = 0; u < NS - 1; ++u)
    if (kb + u < nk) step(kb + u, u);

  // ---- epilogue: stage this wave's tile in LDS (in passes of epi_rows rows),
  // then write full 16-byte row segments
  constexpr int ES = OUT_F32 ? 4 : 2;
  constexpr int P = L::epi_pitch;
  constexpr int ER = L::epi_rows;
  constexpr int CPR = WN * ES / 16;     // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;         // rows per store instruction
  static_assert(64 % CPR == 0 && ER % RPI == 0 && ER % 16 == 0, "epilogue store shape");
  uint8_t* ep = ldsE + w * (ER * P);
#pragma unroll
  for (int pass = 0; pass < L::epi_passes; ++pass) {
    if (pass) {
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): previous pass's LDS reads done
      __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int i = pass * (TM / L::epi_passes); i < (pass + 1) * (TM / L::epi_passes); ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rl = 16 * i + 4 * g + r - pass * ER, cl = 16 * j + l16;
          if (OUT_F32)
            *reinterpret_cast<float*>(ep + rl * P + 4 * cl) = acc[i][j][r];
          else
            *reinterpret_cast<uint16_t*>(ep + rl * P + 2 * cl) = (uint16_t)f32_to_bf16_rne(acc[i][j][r]);
        }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int it = 0; it < ER / RPI; ++it) {
      const int rl = it * RPI + lane / CPR, ch = lane % CPR;
      const int64_t row = m0 + wm * WM + pass * ER + rl;
      if (row >= mend) continue;
      const uint4 v = *reinterpret_cast<const uint4*>(ep + rl * P + 16 * ch);
      uint8_t* dst = reinterpret_cast<uint8_t*>(p.C) + (row * p.ldc + n0 + wn * WN) * ES + 16 * ch;
      if (OUT_F32 && p.accumulate) {
        const float4 o = *reinterpret_cast<const float4*>(dst);
        float4 f = *reinterpret_cast<const float4*>(&v);
        f.x += o.x; f.y += o.y; f.z += o.z; f.w += o.w;
        *reinterpret_cast<float4*>(dst) = f;
      } else {
        *reinterpret_cast<uint4*>(dst) = v;
      }
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

template <class C, int SB_MODE, int OUT_F32, bool GROUPED>
static hipError_t launch_one(const GemmArgs& a, hipStream_t st) {
  int64_t tiles;
  const int64_t tiles_n = a.N / C::BN;
  if (!GROUPED)
    tiles = ((a.M + C::BM - 1) / C::BM) * tiles_n;
  else
    tiles = ((a.M + C::BM - 1) / C::BM + a.E) * tiles_n;  // upper bound: one partial tile per expert
  if (tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL((k_gemm<C, SB_MODE, OUT_F32, GROUPED>), dim3((uint32_t)tiles), dim3(C::NT), 0, st, a);
  return hipGetLastError();
}

static hipError_t launch_exact(const GemmArgs& a, hipStream_t st) {
  typedef DefaultCfg C;
  const bool grouped = a.offsets != nullptr;
  if (a.sb_mode == kSbRow) {
    // per-column B scales: the weight-gradient product, FP32 output
    return launch_one<C, kSbRow, 1, false>(a, st);
  }
  if (grouped)
    return a.out_f32 ? launch_one<C, kSbBlock, 1, true>(a, st) : launch_one<C, kSbBlock, 0, true>(a, st);
  return a.out_f32 ? launch_one<C, kSbBlock, 1, false>(a, st) : launch_one<C, kSbBlock, 0, false>(a, st);
}

// The FP8 entry points run the FP8 matrix-instruction kernel (gemm_fp8.hip);
// the _exact ones this kernel.
hipError_t launch_gemm(const GemmArgs& a, hipStream_t st) {
  return a.exact ? launch_exact(a, st) : launch_gemm_fp8(a, st);
}

}  // namespace fp8q
