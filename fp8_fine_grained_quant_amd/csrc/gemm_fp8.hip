// FP8 GEMM with FP32 promotion after every 128-long K chunk, gfx950.
//
// What is computed ("DeepSeek FP8 Training", the Fprop pipeline and the
// weight- and input-gradient lists; the innerforce.co.kr excerpt of the
// DeepSeek-V3 report, the paragraph after Figure 7 (a): dequantization folded
// into the increased-precision accumulation; the "unified E4M3 format" page,
// "Enhanced Numerical Stability": partial results promoted to FP32 registers
// at a fixed interval of 128 elements):
//
//     C[m, n] = sum_kb  P_kb[m, n] * sA(m, kb) * sB(n, kb)
//
// P_kb is the FP8 x FP8 product over the 128 K of chunk kb, one
// v_mfma_f32_16x16x128_f8f6f4 per 16x16 sub-tile, so one MFMA is exactly one
// promotion interval; the scale-and-add runs as FP32 FMAs on the vector ALU
// into accumulators held in architectural VGPRs.
//
// Design (MI355X: 256 CUs, one 4-SIMD CU per workgroup, 160 KB LDS):
//   * workgroup tile 256 x 128, four waves (one per SIMD), each wave a
//     64 x 128 strip of 4 x 8 sub-tiles (128 FP32 accumulators per lane);
//   * every operand byte reaches LDS by direct buffer loads (global -> LDS,
//     no registers): A tile 32 KB, B tile 16 KB and the chunk's scales per
//     stage, three stages, 16-byte chunks XOR-swizzled by (row & 7) so the
//     fragment reads of 16 rows hit distinct banks;
//   * each stage is one LDS object, so the compiler can tell the stage being
//     read from the one being filled and never waits for the latter;
//   * one chunk = 32 matrix "slots"; slot t issues one MFMA and the promotion
//     of slot t-3, whose result is then complete, so the matrix core and the
//     vector ALU work side by side; the skew runs across chunk boundaries
//     (the last three promotions of a chunk are issued under the first MFMAs
//     of the next), and the next chunk's fragments are read under the last
//     column's MFMAs;
//   * two barriers per chunk: after the first column (every wave is done with
//     the previous chunk, whose stage is then refilled with chunk c+2), and
//     before the last column (chunk c+1 has landed), giving each chunk's
//     loads about one chunk time to arrive;
//   * buffer loads range-check the A rows: rows past the tile's last valid
//     row read nothing and are never stored;
//   * the epilogue stages each wave's strip through LDS so every global store
//     is a full 16-byte row segment.
//
// MFMA operand layout (the same permutation of the 128 K positions for A and
// B, which leaves every dot product unchanged): lane l supplies row l%16 of
// the 16-row slice, bytes [16g, 16g+16) and [64+16g, 64+16g+16) of the chunk,
// g = l/16.  Block-scaled B (Fprop, Dgrad): B is the first operand, so lane l
// holds C[l%16][4g + r], r = 0..3 (one output row per lane: its promotion
// needs one row scale per sub-tile, read from LDS, where the other order
// needed four per sub-tile, broadcast across the lanes with DPP).  Row-scaled
// B (Wgrad): A first, lane l holds C[4g + r][l%16] (one column per lane, its
// column scale per lane).
//
// Exact mode (the _exact entry points, template flag EX of the 256 x 128
// kernel).  gfx950's FP8 matrix instruction aligns the 8 products of each
// group of 8 consecutive K to the largest one and truncates the others 13
// bits below its exponent (measured), the analogue of the limited
// accumulation the innerforce.co.kr excerpt reports for H800 tensor cores
// (paragraph after Figure 7 (a)).  Exact mode keeps the same data movement,
// slot schedule and promotion, but converts each lane's 32 code bytes exactly
// to BF16 (every E4M3 value is a BF16 value) and forms the chunk's partial
// with four v_mfma_f32_16x16x32_bf16 over quarters of 8 K per lane, whose
// products are exact and whose sums are FP32.  A fragments are converted once
// per chunk, B fragments once per column.

#include "device_common.h"
#include "gemm_tile.h"
#include "launch.h"

namespace fp8q {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_ptr;

constexpr int kBM = 256, kBN = 128, kBK = 128;
constexpr int kNT = 256;                          // four waves
constexpr int kTM = 4, kTN = 8;                   // sub-tiles per wave: 64 x 128
constexpr int kIA = kBM * kBK / (16 * kNT);       // 16-byte A loads per lane per chunk
constexpr int kIB = kBN * kBK / (16 * kNT);       // 16-byte B loads per lane per chunk
constexpr int kMaxChunks = 1024;
constexpr int kSkew = 3;                          // promotion trails its MFMA by 3 slots
static_assert(kTM == 4 && kSkew == kTM - 1, "the slot schedule below assumes 4 row sub-tiles");

// SC4: the row scales travel in blocks of 4 chunks (16 bytes per row, one
// load per 4 chunks into a 2-block ring) instead of 4 bytes per row per
// chunk in every stage.  A row's scales of consecutive chunks sit in one
// cache line, so this cuts the scale loads' line requests fourfold; it needs
// 16-byte aligned scale rows.
template <int SB_MODE, bool SC4>
struct Stage {
  static constexpr int a = 0;                     // [256 rows][128 B], swizzled
  static constexpr int b = kBM * kBK;             // [128 rows][128 B], swizzled
  static constexpr int sa = b + kBN * kBK;        // 256 row scales (not SC4)
  static constexpr int sb = sa + (SC4 ? 0 : 4 * kNT);  // row mode: 128 column scales (+128 spare)
  static constexpr int bytes = sb + (SB_MODE == kSbRow ? 4 * kNT : 0);
  static constexpr int sbk_len = SB_MODE == kSbBlock ? kMaxChunks : 4;
  static constexpr int ring = SC4 ? 2 * 256 * 4 : 4;      // floats of the SC4 row-scale ring
  static constexpr int dummy = SC4 ? 1024 : 16;           // bytes: target of count-keeping loads
  static_assert(3 * bytes + 4 * sbk_len + 4 * ring + dummy <= 160 * 1024, "LDS of one CU");
  static_assert(4 * 12288 <= bytes, "epilogue staging fits in one stage");
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // raw buffer: stride 0, range `bytes`, default data format for gfx9
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ v8i make_frag(uint4 lo, uint4 hi) {
  v8i f;
  f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
  f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
  return f;
}

// Exact mode: a lane's 32 code bytes of a fragment -> four groups of 8 BF16
// values (bytes [8q, 8q+8) -> out[q]).  Every E4M3 value is a BF16 value, so
// the conversion (scale 1.0) is exact.
__device__ __forceinline__ void to_bf16_quarters(const v8i& f, v8bf (&out)[4]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const v2bf c0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(f[2 * q], 1.0f, false);
    const v2bf c1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(f[2 * q], 1.0f, true);
    const v2bf c2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(f[2 * q + 1], 1.0f, false);
    const v2bf c3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(f[2 * q + 1], 1.0f, true);
    out[q] = v8bf{c0[0], c0[1], c1[0], c1[1], c2[0], c2[1], c3[0], c3[1]};
  }
}

template <int V>
struct IC {
  static constexpr int value = V;
};

// The four row scales of sub-tile I held by lanes 4I .. 4I+3 of each row.
template <int I>
__device__ __forceinline__ void row_scales(float v, float k, float (&out)[4]) {
  out[0] = row_bcast<4 * I + 0>(v) * k;
  out[1] = row_bcast<4 * I + 1>(v) * k;
  out[2] = row_bcast<4 * I + 2>(v) * k;
  out[3] = row_bcast<4 * I + 3>(v) * k;
}

}  // namespace

template <int SB_MODE, int OUT_F32, bool GROUPED, bool KG, bool SC4, bool EX, bool QO, int INTV>
__global__ __launch_bounds__(kNT) void k_gemm_fp8(GemmArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  typedef Stage<SB_MODE, SC4> S;
  constexpr bool ROW = SB_MODE == kSbRow;
  // Block-scaled B: B is the matrix instruction's first operand, so lane
  // 16 g + l16 holds output row 16 i + l16 (columns 16 j + 4 g + r) of each
  // sub-tile and needs one row scale per sub-tile.  Row mode keeps A first
  // (rows 16 i + 4 g + r, column 16 j + l16), its column scales per lane.
  constexpr bool TR = !ROW;
  __shared__ __attribute__((aligned(16))) uint8_t st0[S::bytes];
  __shared__ __attribute__((aligned(16))) uint8_t st1[S::bytes];
  __shared__ __attribute__((aligned(16))) uint8_t st2[S::bytes];
  __shared__ __attribute__((aligned(16))) float sbk_all[S::sbk_len];  // block mode: B scale per chunk
  __shared__ __attribute__((aligned(16))) float scA[S::ring];          // SC4: row scales, 2 blocks of 4 chunks
  __shared__ __attribute__((aligned(16))) uint8_t dmy[S::dummy];

  TileCoord tc;
  if (!tile_coord<kBM, kBN, GROUPED>(p, tc)) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  // chunks of the contraction this tile runs over: all of K, or (grouped
  // contraction) the expert's padded chunks starting at chunk cb
  int nk = (int)(p.K / kBK), cb = 0;
  if (KG) {
    const int lo = p.offsets[tc.e], hi = p.offsets[tc.e + 1];
    nk = (hi - lo + kBK - 1) / kBK;
    cb = lo / kBK + tc.e;
  }
  GemmArgs po = p;  // the output this tile writes (grouped contraction: the expert's own)
  if (KG) po.C = reinterpret_cast<float*>(p.C) + (int64_t)tc.e * p.c_estride;
  const uint8_t* Bp = p.B + (GROUPED ? (int64_t)tc.e * p.b_estride : 0);
  const float* sbp = p.sb + (GROUPED ? (int64_t)tc.e * p.sb_estride : 0);
  const int rows = (int)min(tc.mend - tc.m0, (int64_t)kBM);  // valid rows of the tile, >= 1

  // ---- direct-load sources.  Buffer ranges: A covers exactly the tile's valid
  // rows (a row past them is out of range: nothing is read), B the tile's 128
  // columns, the scale vectors their rows.
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A + tc.m0 * p.lda, (uint32_t)(rows * p.lda));
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(Bp + (int64_t)tc.n0 * p.ldb, (uint32_t)(kBN * p.ldb));
  const __amdgpu_buffer_rsrc_t rSa = make_rsrc(p.sa + tc.m0 * p.ld_sa, (uint32_t)(rows * p.ld_sa * 4));
  const __amdgpu_buffer_rsrc_t rSb = make_rsrc(sbp + (int64_t)tc.n0 * p.sb_rs, (uint32_t)(kBN * p.sb_rs * 4));
  // Wave w's q-th 16-byte load of a tile writes LDS bytes [(w*I + q)*1024, +1024):
  // rows (w*I + q)*8 + lane/8, physical chunk lane%8, which holds the logical
  // chunk (lane%8) ^ (row%8); row%8 == lane/8.
  const int r8 = lane >> 3, lc = (lane & 7) ^ r8;
  const uint32_t voffA = (uint32_t)((w * kIA * 8 + r8) * p.lda + 16 * lc);
  const uint32_t voffB = (uint32_t)((w * kIB * 8 + r8) * p.ldb + 16 * lc);
  const uint32_t stepA = (uint32_t)(8 * p.lda), stepB = (uint32_t)(8 * p.ldb);
  // scales: lane (w, l) fetches row 64w + l (clamped to a valid row) and, in
  // row mode, column 64w + l for w < 2 (waves 2, 3 load nothing into spare slots)
  const uint32_t voffSa = (uint32_t)(min(w * 64 + lane, rows - 1) * p.ld_sa * 4);
  const uint32_t voffSb = (uint32_t)(((w * 64 + lane) & (kBN - 1)) * p.sb_rs * 4);

  // direct loads one wave issues per chunk; vmcnt counts them in issue order
  constexpr int kDma = kIA + kIB + 1 + (ROW ? 1 : 0);
  // the d-th direct load of chunk kb into stage st
  auto issue_one = [&](int kb, uint8_t* st, int d) {
    kb += cb;
    const uint32_t ka = (uint32_t)kb * kBK;
    if (d < kIA) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_ptr)(st + S::a + (w * kIA + d) * 1024), 16,
                                               voffA + d * stepA, ka, 0, 0);
    } else if (d < kIA + kIB) {
      const int q = d - kIA;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_ptr)(st + S::b + (w * kIB + q) * 1024), 16,
                                               voffB + q * stepB, ka, 0, 0);
    } else if (d == kIA + kIB) {
      if (SC4) {
        // the row scales of the aligned block of 4 chunks that starts at
        // chunk kb (or holds the tile's first chunk), else an out-of-range
        // load (no memory access) that keeps the count per chunk
        const bool real = (kb & 3) == 0 || kb == cb;
        uint8_t* dst = real ? reinterpret_cast<uint8_t*>(scA) + ((kb >> 2) & 1) * 4096 + w * 1024 : dmy;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rSa, (lds_ptr)dst, 16, real ? voffSa : kNoAccess,
                                                 real ? (uint32_t)(kb & ~3) * 4 : 0u, 0, 0);
      } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rSa, (lds_ptr)(st + S::sa + w * 256), 4, voffSa, (uint32_t)kb * 4,
                                                 0, 0);
      }
    } else {
      // waves 2, 3 keep the load count with an out-of-range load (no memory
      // access) into the spare slots
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rSb, (lds_ptr)(st + S::sb + w * 256), 4, w < 2 ? voffSb : kNoAccess,
                                               w < 2 ? (uint32_t)kb * 4 : 0u, 0, 0);
    }
  };
  auto issue = [&](int kb, uint8_t* st) {
#pragma unroll
    for (int d = 0; d < kDma; ++d) issue_one(kb, st, d);
  };
  // Inside a chunk the loads of chunk c+2 are spread over the slots between
  // the two barriers (a burst of them fills the memory pipeline's queue and
  // stalls the issuing wave, MFMAs included): load d goes out in slot
  // kFirstDmaSlot + (d * kDmaSlots) / kDma.
  constexpr int kFirstDmaSlot = kTM, kDmaSlots = kTM * (kTN - 2);
  static_assert(kDma <= kDmaSlots, "one direct load per slot at most");
  static_assert(kDma < 64, "vmcnt range");
  constexpr int kWaitPrev = 0x0F70 | (kDma & 15) | ((kDma >> 4) << 14);  // vmcnt(kDma) only

  // ---- LDS fragment reads
  const int sw = l16 & 7;
  const int offLo = l16 * kBK + 16 * (g ^ sw);
  const int offHi = l16 * kBK + 16 * ((4 + g) ^ sw);
  auto rdA = [&](const uint8_t* st, int i) -> v8i {
    const uint8_t* base = st + S::a + (w * 64 + 16 * i) * kBK;
    return make_frag(*reinterpret_cast<const uint4*>(base + offLo), *reinterpret_cast<const uint4*>(base + offHi));
  };
  auto rdB = [&](const uint8_t* st, int j) -> v8i {
    const uint8_t* base = st + S::b + 16 * j * kBK;
    return make_frag(*reinterpret_cast<const uint4*>(base + offLo), *reinterpret_cast<const uint4*>(base + offHi));
  };
  // Row scales.  TR: lane (l16, g) needs rows 16 i + l16 of its wave's strip,
  // one 4-byte read each.  Row mode: lane (l16, g) reads the scale of row
  // 16*(l16/4) + 4g + l16%4, the (i, r) = (l16/4, l16%4) entry of its lane
  // group's 16 values, and row_scales hands every lane of the group entry
  // (i, r) (DPP row_newbcast).
  // (TR: each of the four reads takes its offset through an empty asm, so the
  // compiler cannot fuse them into one two-address LDS read: the fused form
  // loses the operands' LDS objects, and the wait the compiler then puts in
  // front of it for the pending direct loads drained the load pipeline every
  // chunk, measured 60 -> 65 us on the 4096 x 2048 x 7168 Fprop.)
  auto rdSa1 = [&](const uint8_t* st, int kb, int row) -> float {  // kb: the tile's chunk index
    kb += cb;
    if (TR) {
      int off = SC4 ? ((kb >> 2) & 1) * 1024 + row * 4 + (kb & 3) : row;
      asm volatile("" : "+v"(off));
      return SC4 ? scA[off] : reinterpret_cast<const float*>(st + S::sa)[off];
    }
    if (SC4) return scA[((kb >> 2) & 1) * 1024 + row * 4 + (kb & 3)];
    return *reinterpret_cast<const float*>(st + S::sa + 4 * row);
  };
  auto rdSa = [&](const uint8_t* st, int kb, float (&v)[kTM]) {
    if (TR) {
#pragma unroll
      for (int i = 0; i < kTM; ++i) v[i] = rdSa1(st, kb, w * 64 + 16 * i + l16);
    } else {
      v[0] = rdSa1(st, kb, w * 64 + 16 * (l16 >> 2) + 4 * g + (l16 & 3));
    }
  };

  auto rdSb = [&](const uint8_t* st, int j) -> float {
    return *reinterpret_cast<const float*>(st + S::sb + 4 * (16 * j + l16));
  };

  float acc[kTM][kTN][4];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.f;
  if (KG && nk == 0) {
    // an expert without tokens: its gradient is zero
    if (!p.accumulate)
      store_tile<kTM, kTN, OUT_F32, OUT_F32 ? 16 : 32, 0, TR>(acc, st0 + w * 12288, po, tc.m0 + w * 64, tc.mend, tc.n0,
                                                              lane);
    return;
  }

  // state carried from chunk to chunk
  v8i a[kTM];           // A fragments of the current chunk
  v8i bring[3];         // B fragments, ring over the global column index 8c + j
  v4f pp[kTM];          // MFMA partials, ring indexed by slot % 4
  float sc[kTM][4];     // row scales (times the block's B scale) in use; TR: [i][0] only
  float sa_nx[kTM] = {};  // the next chunk's row scales, as read (TR: one per sub-tile; else [0])
  float sbk_nx = 1.f;   // the next chunk's block B scale
  float sbc_prev = 0.f; // row mode: scale of the previous chunk's last column
  float sbc_first = 0.f;  // row mode: scale of the current chunk's column 0

  // Promotion interval study (INTV != 1): within an interval of INTV chunks
  // (INTV == 0: the whole contraction) each sub-tile's partial is chained
  // through the matrix instruction's accumulator operand, and only the
  // interval's sum is promoted, with the scales of its last chunk (the
  // caller makes the scales constant over each interval).  INTV == 1 is the
  // method: a fresh partial per chunk, promoted at once.
  v4f pch[kTM][kTN];
  if (INTV != 1) {
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j) pch[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  bool promote_now = true;  // INTV != 1: the chunk being promoted ends its interval
  auto promote = [&](int i, int j, float sbc) {
    if (INTV != 1 && !promote_now) return;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float s = TR ? sc[i][0] : ROW ? sc[i][r] * sbc : sc[i][r];
      const float part = INTV == 1 ? pp[i][r] : pch[i][j][r];
      acc[i][j][r] = __builtin_fmaf(part, s, acc[i][j][r]);
    }
  };
  auto load_sc = [&](int i) {
    const float k = ROW ? 1.f : sbk_nx;
    if (TR) {
      sc[i][0] = sa_nx[i] * k;
      return;
    }
    switch (i) {
      case 0: row_scales<0>(sa_nx[0], k, sc[0]); break;
      case 1: row_scales<1>(sa_nx[0], k, sc[1]); break;
      case 2: row_scales<2>(sa_nx[0], k, sc[2]); break;
      default: row_scales<3>(sa_nx[0], k, sc[3]); break;
    }
  };
  // the chunk partial of A fragment x and B fragment y (TR: B first)
  auto mfma = [&](const v8i& x, const v8i& y) -> v4f {
    if (TR) return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(y, x, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
  };
  // exact mode: the chunk's partial as four BF16 instructions over quarters
  // of 8 K per lane (exact products, FP32 sums); lane group g covers the same
  // K positions of A and B in each, so together they cover the chunk once
  v8bf abf[kTM][4];  // A fragments of the current chunk in BF16 (exact mode)
  auto mfma_ex = [&](const v8bf (&xa)[4], const v8bf (&ya)[4]) -> v4f {
    const v8bf(&x)[4] = TR ? ya : xa;
    const v8bf(&y)[4] = TR ? xa : ya;
    v4f c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x[0], y[0], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x[1], y[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x[2], y[2], c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(x[3], y[3], c, 0, 0, 0);
  };
  auto fence = [] { asm volatile("" ::: "memory"); };

  // ---- prologue: block B scales of every chunk to LDS, chunks 0 and 1 in
  // flight, chunk 0 published, its fragments and scales in registers.  The
  // block scales go by direct loads too (4 bytes per lane, entries past the
  // last chunk out of range), issued first so that their latency overlaps the
  // chunks' instead of preceding it (a load into registers and an LDS write
  // made the prologue wait for them before the first chunk's loads).
  if (!ROW) {
    const float* psb = sbp + (int64_t)(tc.n0 / 128) * p.sb_rs;
    const __amdgpu_buffer_rsrc_t rK = make_rsrc(psb, (uint32_t)(((int64_t)(nk - 1) * p.sb_cs + 1) * 4));
    for (int r = 0; r * kNT < nk; ++r)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rK, (lds_ptr)(sbk_all + r * kNT + w * 64), 4,
                                               (uint32_t)((r * kNT + w * 64 + lane) * p.sb_cs * 4), 0, 0, 0);
  }
  fence();
  issue(0, st0);
  issue(min(1, nk - 1), st1);
  __builtin_amdgcn_s_waitcnt(kWaitPrev);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the block scales are written
  __builtin_amdgcn_s_barrier();
  fence();
#pragma unroll
  for (int i = 0; i < kTM; ++i) {
    a[i] = rdA(st0, i);
    if (i == 0) rdSa(st0, 0, sa_nx);
    pp[i] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  bring[0] = rdB(st0, 0);
  bring[1] = rdB(st0, 1);
  if (ROW) sbc_first = rdSb(st0, 0);
  else sbk_nx = sbk_all[0];
#pragma unroll
  for (int i = 0; i < kTM; ++i) load_sc(i);

  // ---- one chunk.  Stage u holds chunk c; stage (u+1)%3 receives or holds
  // chunk c+1; stage (u+2)%3 held chunk c-1 and is refilled with chunk c+2.
  auto step = [&](int c, auto U) {
    constexpr int u = decltype(U)::value;
    uint8_t* const cur = u == 0 ? st0 : u == 1 ? st1 : st2;
    uint8_t* const nxt = u == 0 ? st1 : u == 1 ? st2 : st0;
    uint8_t* const fut = u == 0 ? st2 : u == 1 ? st0 : st1;

    float sbc[kTN + 1];  // row mode: column scales of this chunk, [kTN] = next chunk's column 0
    sbc[0] = sbc_first;
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
      // the B fragment (and column scale) of the next column: this chunk's
      // column j+1, or the next chunk's column 0 (published by the barrier
      // before the last column)
      // B two columns ahead: this chunk's columns 2..7 at columns 0..5; the
      // next chunk's columns 0 and 1 at column 7, after the barrier that
      // publishes it (column 6 reads none)
      const v8i bcur = bring[(2 * u + j) % 3];
      v8bf bbf[4];
      if (EX) to_bf16_quarters(bcur, bbf);
      if (j + 2 < kTN) {
        bring[(2 * u + j + 2) % 3] = rdB(cur, j + 2);
      } else if (j == kTN - 1) {
        bring[(2 * u + kTN) % 3] = rdB(nxt, 0);
        bring[(2 * u + kTN + 1) % 3] = rdB(nxt, 1);
      }
      if (j + 1 < kTN) {
        if (ROW) sbc[j + 1] = rdSb(cur, j + 1);
      } else {
        if (ROW) sbc[kTN] = rdSb(nxt, 0);
      }
      fence();
#pragma unroll
      for (int i = 0; i < kTM; ++i) {
        const int t = kTM * j + i;
        if (EX) {
          if (j == 0) to_bf16_quarters(a[i], abf[i]);
          pp[i] = mfma_ex(abf[i], bbf);
        } else if (INTV == 1) {
          pp[i] = mfma(a[i], bcur);
        } else {
          const bool first = INTV == 0 ? c == 0 : c % INTV == 0;
          const v4f zero = {0.f, 0.f, 0.f, 0.f};
          pch[i][j] = TR ? __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bcur, a[i], first ? zero : pch[i][j], 0, 0,
                                                                            0, 0, 0, 0)
                         : __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[i], bcur, first ? zero : pch[i][j], 0, 0,
                                                                            0, 0, 0, 0);
        }
        if (t >= kSkew) {
          const int tp = t - kSkew;
          if (INTV != 1) promote_now = INTV == 0 ? c == nk - 1 : ((c + 1) % INTV == 0 || c == nk - 1);
          promote(tp % kTM, tp / kTM, sbc[tp / kTM]);
        } else {
          // the previous chunk's last column, rows t+1; then this chunk's
          // scales for those rows (row 0's were set at the previous chunk end)
          if (INTV != 1) promote_now = INTV != 0 && c > 0 && c % INTV == 0;
          promote(t + 1, kTN - 1, sbc_prev);
          load_sc(t + 1);
        }
        if (t >= kFirstDmaSlot && t < kFirstDmaSlot + kDmaSlots) {
#pragma unroll
          for (int d = 0; d < kDma; ++d)
            if (kFirstDmaSlot + (d * kDmaSlots) / kDma == t) issue_one(min(c + 2, nk - 1), fut, d);
        }
        if (j == kTN - 1) {
          // a[i] is no longer needed for this chunk: fetch the next chunk's
          a[i] = rdA(nxt, i);
          if (i == 0) {
            rdSa(nxt, min(c + 1, nk - 1), sa_nx);
            if (!ROW) sbk_nx = sbk_all[min(c + 1, nk - 1)];
          }
        }
        // exact Wgrad: slots in pairs, so the two sub-tiles' chains of four
        // dependent BF16 MFMAs can interleave (measured 144 -> 138.5 us; the
        // block-scaled exact products measured 1 us slower that way)
        if (!(EX && ROW) || (i & 1)) __builtin_amdgcn_sched_barrier(0);
      }
      if (j == 0) {
        // every wave has finished reading chunk c-1: its stage may be refilled
        // with chunk c+2 (past the end, the last chunk again, so every chunk
        // issues the same loads and the wait counts stay exact)
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        fence();
      }
      if (j == kTN - 2) {
        // chunk c+1 has landed: only the loads of chunk c+2 may be in flight
        __builtin_amdgcn_s_waitcnt(kWaitPrev);
        __builtin_amdgcn_s_barrier();
        fence();
      }
    }
    // slot 31 promoted row 0 of the last column: row 0 takes the next
    // chunk's scales now, rows 1-3 after their last promotion
    load_sc(0);
    sbc_prev = sbc[kTN - 1];
    sbc_first = sbc[kTN];
  };

  int c = 0;
  for (; c + 3 <= nk; c += 3) {
    step(c, IC<0>());
    step(c + 1, IC<1>());
    step(c + 2, IC<2>());
  }
  if (c < nk) step(c, IC<0>());
  if (c + 1 < nk) step(c + 1, IC<1>());
  // the last chunk's last column, rows 1-3 (load_sc(0) above only touched row 0)
  promote_now = true;
#pragma unroll
  for (int i = 1; i < kTM; ++i) promote(i, kTN - 1, sbc_prev);

  // ---- epilogue: no direct load may still target LDS, and every wave is done
  // reading; each wave then stages its strip in its own 12 KB of stage 0
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __builtin_amdgcn_s_barrier();
  fence();
  if constexpr (QO) {
    static_assert(!OUT_F32 && !KG && TR, "fused output quantization: BF16 Fprop/Dgrad only");
    store_tile_q<kTM, kTN, 32>(acc, st0 + w * 12288, po, tc.m0 + w * 64, tc.mend, tc.n0, lane);
  } else {
    store_tile<kTM, kTN, OUT_F32, OUT_F32 ? 16 : 32, 0, TR>(acc, st0 + w * 12288, po, tc.m0 + w * 64, tc.mend, tc.n0,
                                                            lane);
  }
#endif  // __HIP_DEVICE_COMPILE__
}

// ---------------------------------------------------------------------------
// Wide tile: 256 x 256 outputs per workgroup, eight waves (two per SIMD).
//
// Each wave runs exactly the 64 x 128 strip of k_gemm_fp8 above (the same
// MFMAs, promotion order and epilogue), wave w at rows 64 (w % 4) and columns
// 128 (w / 4) of the tile, so the output is bit-identical; only the data
// movement differs:
//   * a chunk's global -> LDS bytes (A 32 KB + B 32 KB) now feed twice the
//     MFMAs (a third fewer bytes per FLOP), and two waves per SIMD issue LDS
//     fragment reads (measured: one wave per SIMD gets ~40 B/ns of them);
//   * two chunks of A and two of B fit in LDS (4 x 32 KB), each in its own
//     LDS object.  A chunk's A fragments move to registers at the end of the
//     previous chunk, so A region c%2 is free from the first barrier of chunk
//     c on and receives chunk c+2 there (about 1.7 chunk times to land); B
//     region c%2 is read until the chunk's seventh column and receives chunk
//     c+2 in the last column (about one chunk time to land).  With A and B in
//     one 64 KB stage per chunk instead, the loads had under one chunk time
//     and the kernel ran 25% slower than the 256 x 128 one.
// Block-scaled B and 16-byte row-scale blocks only (Fprop, Dgrad and their
// grouped forms); used when the tile count fills the chip (see
// launch_gemm_fp8).  Measured on MI355X: 16384 x 2048 x 7168 284 -> 206 us,
// 4096 x 7168 x 2048 81 -> 69 us, the 32-expert grouped Fprop 409 -> 296 us.
constexpr int kWBN = 256, kWNT = 512;
constexpr int kWIA = kBM * kBK / (16 * kWNT);  // 16-byte A loads per lane per chunk (4)
constexpr int kWIB = kWBN * kBK / (16 * kWNT);  // 16-byte B loads per lane per chunk (4)
constexpr int kWDmaA = kWIA + 1;               // A loads and the row-scale load
constexpr int kWFirstSlot = kTM, kWDmaSlots = 20;
static_assert(kWIB == kTM, "one B load per slot of the last column");
static_assert(kWDmaA <= kWDmaSlots && kWFirstSlot + kWDmaSlots <= kTM * (kTN - 1), "A loads between the barriers");
static_assert(4 * kBM * kBK + 4 * 2 * kMaxChunks + 4 * 2 * 256 * 4 + 1024 <= 160 * 1024, "LDS of one CU");

template <int OUT_F32, bool GROUPED, bool QO>
__global__ __launch_bounds__(kWNT) void k_gemm_fp8_wide(GemmArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ __attribute__((aligned(16))) uint8_t sa0[kBM * kBK];
  __shared__ __attribute__((aligned(16))) uint8_t sa1[kBM * kBK];
  __shared__ __attribute__((aligned(16))) uint8_t sb0[kWBN * kBK];
  __shared__ __attribute__((aligned(16))) uint8_t sb1[kWBN * kBK];
  __shared__ __attribute__((aligned(16))) float sbk_all[2 * kMaxChunks];  // B block scales: [half][chunk]
  __shared__ __attribute__((aligned(16))) float scA[2 * 256 * 4];         // row scales, 2 blocks of 4 chunks
  __shared__ __attribute__((aligned(16))) uint8_t dmy[1024];              // target of count-keeping loads

  TileCoord tc;
  if (!tile_coord<kBM, kWBN, GROUPED>(p, tc)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = w & 3, wc = w >> 2;  // the wave's 64-row strip and 128-column half
  const int l16 = lane & 15, g = lane >> 4;
  const int nk = (int)(p.K / kBK);
  const uint8_t* Bp = p.B + (GROUPED ? (int64_t)tc.e * p.b_estride : 0);
  const float* sbp = p.sb + (GROUPED ? (int64_t)tc.e * p.sb_estride : 0);
  const int rows = (int)min(tc.mend - tc.m0, (int64_t)kBM);  // valid rows of the tile, >= 1

  // direct-load sources, range-checked as in k_gemm_fp8
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A + tc.m0 * p.lda, (uint32_t)(rows * p.lda));
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(Bp + (int64_t)tc.n0 * p.ldb, (uint32_t)(kWBN * p.ldb));
  const __amdgpu_buffer_rsrc_t rSa = make_rsrc(p.sa + tc.m0 * p.ld_sa, (uint32_t)(rows * p.ld_sa * 4));
  const int r8 = lane >> 3, lc = (lane & 7) ^ r8;
  const uint32_t voffA = (uint32_t)((w * kWIA * 8 + r8) * p.lda + 16 * lc);
  const uint32_t voffB = (uint32_t)((w * kWIB * 8 + r8) * p.ldb + 16 * lc);
  const uint32_t stepA = (uint32_t)(8 * p.lda), stepB = (uint32_t)(8 * p.ldb);
  const uint32_t voffSa = (uint32_t)(min(wr * 64 + lane, rows - 1) * p.ld_sa * 4);

  // d-th A-side load of chunk kb into A region `ar` (d == kWIA: waves 0-3 load
  // the row scales of the 4-chunk block that starts at kb; every other wave
  // and chunk issues an out-of-range load, so each chunk issues kWDmaA loads)
  auto issue_a = [&](int kb, uint8_t* ar, int d) {
    if (d < kWIA) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_ptr)(ar + (w * kWIA + d) * 1024), 16, voffA + d * stepA,
                                               (uint32_t)kb * kBK, 0, 0);
    } else {
      const bool real = w < 4 && (kb & 3) == 0;
      uint8_t* dst = real ? reinterpret_cast<uint8_t*>(scA) + ((kb >> 2) & 1) * 4096 + w * 1024 : dmy;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rSa, (lds_ptr)dst, 16, real ? voffSa : kNoAccess, real ? (uint32_t)kb * 4 : 0u,
                                               0, 0);
    }
  };
  auto issue_b = [&](int kb, uint8_t* br, int q) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_ptr)(br + (w * kWIB + q) * 1024), 16, voffB + q * stepB,
                                             (uint32_t)kb * kBK, 0, 0);
  };
  constexpr int kWaitA = 0x0F70 | kWDmaA;  // vmcnt(kWDmaA): all but the latest chunk's A-side loads

  const int sw = l16 & 7;
  const int offLo = l16 * kBK + 16 * (g ^ sw);
  const int offHi = l16 * kBK + 16 * ((4 + g) ^ sw);
  auto rdA = [&](const uint8_t* ar, int i) -> v8i {
    const uint8_t* base = ar + (wr * 64 + 16 * i) * kBK;
    return make_frag(*reinterpret_cast<const uint4*>(base + offLo), *reinterpret_cast<const uint4*>(base + offHi));
  };
  auto rdB = [&](const uint8_t* br, int j) -> v8i {
    const uint8_t* base = br + (wc * 128 + 16 * j) * kBK;
    return make_frag(*reinterpret_cast<const uint4*>(base + offLo), *reinterpret_cast<const uint4*>(base + offHi));
  };
  // B is the matrix instruction's first operand (as in k_gemm_fp8's block
  // mode): lane 16 g + l16 holds row 16 i + l16 of each sub-tile
  // (the offsets pass an empty asm so that the four reads stay four: see rdSa1
  // in k_gemm_fp8)
  auto rdSa = [&](int kb, float (&v)[kTM]) {
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      int off = ((kb >> 2) & 1) * 1024 + (wr * 64 + 16 * i + l16) * 4 + (kb & 3);
      asm volatile("" : "+v"(off));
      v[i] = scA[off];
    }
  };

  float acc[kTM][kTN][4];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.f;

  v8i a[kTM];          // A fragments of the current chunk
  v8i bring[2];        // B fragments: this column's and the next one's
  v4f pp[kTM];         // MFMA partials, ring indexed by slot % 4
  float sc[kTM];       // row scales times the block's B scale
  float sa_nx[kTM] = {};
  float sbk_nx = 1.f;
  auto promote = [&](int i, int j) {
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(pp[i][r], sc[i], acc[i][j][r]);
  };
  auto load_sc = [&](int i) { sc[i] = sa_nx[i] * sbk_nx; };
  auto mfma = [&](const v8i& x, const v8i& y) -> v4f {  // B first
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(y, x, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
  };
  auto fence = [] { asm volatile("" ::: "memory"); };

  // ---- prologue: both halves' block B scales of every chunk to LDS (direct
  // loads as in k_gemm_fp8: waves 0-3 the first half, 4-7 the second); A(0),
  // B(0), A(1), B(1) in flight in that order; chunk 0 published
  {
    const float* psb = sbp + (int64_t)(tc.n0 / 128 + wc) * p.sb_rs;
    const __amdgpu_buffer_rsrc_t rK = make_rsrc(psb, (uint32_t)(((int64_t)(nk - 1) * p.sb_cs + 1) * 4));
    for (int r = 0; r * 256 < nk; ++r)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rK, (lds_ptr)(sbk_all + wc * kMaxChunks + r * 256 + wr * 64), 4,
                                               (uint32_t)((r * 256 + wr * 64 + lane) * p.sb_cs * 4), 0, 0, 0);
  }
  fence();
#pragma unroll
  for (int d = 0; d < kWDmaA; ++d) issue_a(0, sa0, d);
#pragma unroll
  for (int q = 0; q < kWIB; ++q) issue_b(0, sb0, q);
#pragma unroll
  for (int d = 0; d < kWDmaA; ++d) issue_a(min(1, nk - 1), sa1, d);
#pragma unroll
  for (int q = 0; q < kWIB; ++q) issue_b(min(1, nk - 1), sb1, q);
  __builtin_amdgcn_s_waitcnt(0x0F70 | (kWDmaA + kWIB));  // A(0), B(0) landed
  __builtin_amdgcn_s_waitcnt(0xC07F);                  // lgkmcnt(0): the block scales are written
  __builtin_amdgcn_s_barrier();
  fence();
#pragma unroll
  for (int i = 0; i < kTM; ++i) {
    a[i] = rdA(sa0, i);
    if (i == 0) rdSa(0, sa_nx);
    pp[i] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  bring[0] = rdB(sb0, 0);
  sbk_nx = sbk_all[wc * kMaxChunks];
#pragma unroll
  for (int i = 0; i < kTM; ++i) load_sc(i);

  // ---- one chunk (regions u = c % 2 hold chunk c; 1-u hold or receive c+1)
  auto step = [&](int c, auto U) {
    constexpr int u = decltype(U)::value;
    uint8_t* const acur = u == 0 ? sa0 : sa1;
    uint8_t* const anxt = u == 0 ? sa1 : sa0;
    uint8_t* const bcur = u == 0 ? sb0 : sb1;
    uint8_t* const bnxt = u == 0 ? sb1 : sb0;
    const int c2 = min(c + 2, nk - 1);  // past the end, the last chunk again (same counts)
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
      const v8i bj = bring[j & 1];
      if (j + 1 < kTN) bring[(j + 1) & 1] = rdB(bcur, j + 1);
      else bring[0] = rdB(bnxt, 0);
      fence();
#pragma unroll
      for (int i = 0; i < kTM; ++i) {
        const int t = kTM * j + i;
        pp[i] = mfma(a[i], bj);
        if (t >= kSkew) {
          const int tp = t - kSkew;
          promote(tp % kTM, tp / kTM);
        } else {
          promote(t + 1, kTN - 1);
          load_sc(t + 1);
        }
        if (t >= kWFirstSlot && t < kWFirstSlot + kWDmaSlots) {
#pragma unroll
          for (int d = 0; d < kWDmaA; ++d)
            if (kWFirstSlot + (d * kWDmaSlots) / kWDmaA == t) issue_a(c2, acur, d);
        }
        if (j == kTN - 1) {
          issue_b(c2, bcur, i);
          a[i] = rdA(anxt, i);
          if (i == 0) {
            rdSa(min(c + 1, nk - 1), sa_nx);
            sbk_nx = sbk_all[wc * kMaxChunks + min(c + 1, nk - 1)];
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (j == 0) {
        // every wave holds A(c) in registers: A region u may take A(c+2)
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();
        fence();
      }
      if (j == kTN - 2) {
        // every wave has read B(c)'s last column (B region u may take B(c+2)),
        // and A(c+1), B(c+1) have landed
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_waitcnt(kWaitA);
        __builtin_amdgcn_s_barrier();
        fence();
      }
    }
    load_sc(0);
  };

  int c = 0;
  for (; c + 2 <= nk; c += 2) {
    step(c, IC<0>());
    step(c + 1, IC<1>());
  }
  if (c < nk) step(c, IC<0>());
#pragma unroll
  for (int i = 1; i < kTM; ++i) promote(i, kTN - 1);

  // ---- epilogue: two waves' 12 KB staging areas in each 32 KB region
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __builtin_amdgcn_s_barrier();
  fence();
  uint8_t* const ep = (w >> 1) == 0 ? sa0 : (w >> 1) == 1 ? sa1 : (w >> 1) == 2 ? sb0 : sb1;
  if constexpr (QO) {
    static_assert(!OUT_F32 && !GROUPED, "fused output quantization: BF16 Fprop/Dgrad only");
    store_tile_q<kTM, kTN, 32>(acc, ep + (w & 1) * 12288, p, tc.m0 + wr * 64, tc.mend, tc.n0 + wc * 128, lane);
  } else {
    store_tile<kTM, kTN, OUT_F32, OUT_F32 ? 16 : 32, 0, true>(acc, ep + (w & 1) * 12288, p, tc.m0 + wr * 64, tc.mend,
                                                              tc.n0 + wc * 128, lane);
  }
#endif  // __HIP_DEVICE_COMPILE__
}

// Wide tile for the weight gradients (one B scale per output column per
// chunk, FP32 output, optionally C +=): the same schedule as k_gemm_fp8_wide.
// Each chunk's 256 row scales ride with its A loads and its 256 column
// scales with its B loads, 4 bytes per lane, into 2 KB beside each region
// (waves 4-7 write a spare copy so every wave issues the same loads).  KG:
// the grouped contraction (per-expert token chunks, per-expert output), as
// in k_gemm_fp8.
constexpr int kWRowPad = 2048;

template <bool KG>
__global__ __launch_bounds__(kWNT) void k_gemm_fp8_wide_row(GemmArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int RA = kBM * kBK, RB = kWBN * kBK;  // scale areas start after the codes
  __shared__ __attribute__((aligned(16))) uint8_t sa0[RA + kWRowPad];
  __shared__ __attribute__((aligned(16))) uint8_t sa1[RA + kWRowPad];
  __shared__ __attribute__((aligned(16))) uint8_t sb0[RB + kWRowPad];
  __shared__ __attribute__((aligned(16))) uint8_t sb1[RB + kWRowPad];

  TileCoord tc;
  if (!tile_coord<kBM, kWBN, KG>(p, tc)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = w & 3, wc = w >> 2;
  const int l16 = lane & 15, g = lane >> 4;
  int nk = (int)(p.K / kBK), cb = 0;
  if (KG) {
    const int lo = p.offsets[tc.e], hi = p.offsets[tc.e + 1];
    nk = (hi - lo + kBK - 1) / kBK;
    cb = lo / kBK + tc.e;
  }
  GemmArgs po = p;
  if (KG) po.C = reinterpret_cast<float*>(p.C) + (int64_t)tc.e * p.c_estride;
  const int rows = (int)min(tc.mend - tc.m0, (int64_t)kBM);

  float acc[kTM][kTN][4];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.f;
  uint8_t* const ep = (w >> 1) == 0 ? sa0 : (w >> 1) == 1 ? sa1 : (w >> 1) == 2 ? sb0 : sb1;
  if (KG && nk == 0) {
    // an expert without tokens: its gradient is zero
    if (!p.accumulate)
      store_tile<kTM, kTN, 1, 16, 1>(acc, ep + (w & 1) * 12288, po, tc.m0 + wr * 64, tc.mend, tc.n0 + wc * 128, lane);
    return;
  }

  const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A + tc.m0 * p.lda, (uint32_t)(rows * p.lda));
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(p.B + (int64_t)tc.n0 * p.ldb, (uint32_t)(kWBN * p.ldb));
  const __amdgpu_buffer_rsrc_t rSa = make_rsrc(p.sa + tc.m0 * p.ld_sa, (uint32_t)(rows * p.ld_sa * 4));
  const __amdgpu_buffer_rsrc_t rSb = make_rsrc(p.sb + (int64_t)tc.n0 * p.sb_rs, (uint32_t)(kWBN * p.sb_rs * 4));
  const int r8 = lane >> 3, lc = (lane & 7) ^ r8;
  const uint32_t voffA = (uint32_t)((w * kWIA * 8 + r8) * p.lda + 16 * lc);
  const uint32_t voffB = (uint32_t)((w * kWIB * 8 + r8) * p.ldb + 16 * lc);
  const uint32_t stepA = (uint32_t)(8 * p.lda), stepB = (uint32_t)(8 * p.ldb);
  // lane (w, l), w < 4: row scale of row 64 w + l (clamped to a valid row),
  // column scale of column 64 w + l (waves 4-7 load nothing)
  const uint32_t voffSa = (uint32_t)(min(wr * 64 + lane, rows - 1) * p.ld_sa * 4);
  const uint32_t voffSb = (uint32_t)(((w * 64 + lane) & (kWBN - 1)) * p.sb_rs * 4);

  auto issue_a = [&](int kb, uint8_t* ar, int d) {
    kb += cb;
    if (d < kWIA)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_ptr)(ar + (w * kWIA + d) * 1024), 16, voffA + d * stepA,
                                               (uint32_t)kb * kBK, 0, 0);
    else
      // waves 4-7 keep the load count with an out-of-range load (no memory
      // access) into the second KB, which nothing reads
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rSa, (lds_ptr)(ar + RA + w * 256), 4, w < 4 ? voffSa : kNoAccess,
                                               w < 4 ? (uint32_t)kb * 4 : 0u, 0, 0);
  };
  auto issue_b = [&](int kb, uint8_t* br, int q) {
    kb += cb;
    if (q < kWIB)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_ptr)(br + (w * kWIB + q) * 1024), 16, voffB + q * stepB,
                                               (uint32_t)kb * kBK, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rSb, (lds_ptr)(br + RB + w * 256), 4, w < 4 ? voffSb : kNoAccess,
                                               w < 4 ? (uint32_t)kb * 4 : 0u, 0, 0);
  };
  constexpr int kDmaB = kWIB + 1;
  constexpr int kWaitA = 0x0F70 | kWDmaA;

  const int sw = l16 & 7;
  const int offLo = l16 * kBK + 16 * (g ^ sw);
  const int offHi = l16 * kBK + 16 * ((4 + g) ^ sw);
  auto rdA = [&](const uint8_t* ar, int i) -> v8i {
    const uint8_t* base = ar + (wr * 64 + 16 * i) * kBK;
    return make_frag(*reinterpret_cast<const uint4*>(base + offLo), *reinterpret_cast<const uint4*>(base + offHi));
  };
  auto rdB = [&](const uint8_t* br, int j) -> v8i {
    const uint8_t* base = br + (wc * 128 + 16 * j) * kBK;
    return make_frag(*reinterpret_cast<const uint4*>(base + offLo), *reinterpret_cast<const uint4*>(base + offHi));
  };
  // row scale: lane (l16, g) holds row 16 (l16 / 4) + 4 g + l16 % 4 of its
  // wave's strip (row_scales broadcasts); column scale of column 16 j + l16
  const int rowSa = wr * 64 + 16 * (l16 >> 2) + 4 * g + (l16 & 3);
  auto rdSa = [&](const uint8_t* ar) -> float { return *reinterpret_cast<const float*>(ar + RA + 4 * rowSa); };
  auto rdSb = [&](const uint8_t* br, int j) -> float {
    return *reinterpret_cast<const float*>(br + RB + 4 * (wc * 128 + 16 * j + l16));
  };

  v8i a[kTM];
  v8i bring[2];
  v4f pp[kTM];
  float sc[kTM][4];       // row scales in use
  float sa_nx = 0.f;      // the next chunk's row scale, as read
  float sbc_prev = 0.f;   // column scale of the previous chunk's last column
  float sbc_first = 0.f;  // column scale of this chunk's column 0
  auto promote = [&](int i, int j, float sbc) {
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(pp[i][r], sc[i][r] * sbc, acc[i][j][r]);
  };
  auto load_sc = [&](int i) {
    switch (i) {
      case 0: row_scales<0>(sa_nx, 1.f, sc[0]); break;
      case 1: row_scales<1>(sa_nx, 1.f, sc[1]); break;
      case 2: row_scales<2>(sa_nx, 1.f, sc[2]); break;
      default: row_scales<3>(sa_nx, 1.f, sc[3]); break;
    }
  };
  auto mfma = [&](const v8i& x, const v8i& y) -> v4f {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
  };
  auto fence = [] { asm volatile("" ::: "memory"); };

  // ---- prologue: A(0), B(0), A(1), B(1) in flight in that order; chunk 0 published
#pragma unroll
  for (int d = 0; d < kWDmaA; ++d) issue_a(0, sa0, d);
#pragma unroll
  for (int q = 0; q < kDmaB; ++q) issue_b(0, sb0, q);
#pragma unroll
  for (int d = 0; d < kWDmaA; ++d) issue_a(min(1, nk - 1), sa1, d);
#pragma unroll
  for (int q = 0; q < kDmaB; ++q) issue_b(min(1, nk - 1), sb1, q);
  __builtin_amdgcn_s_waitcnt(0x0F70 | (kWDmaA + kDmaB));
  __builtin_amdgcn_s_barrier();
  fence();
#pragma unroll
  for (int i = 0; i < kTM; ++i) {
    a[i] = rdA(sa0, i);
    pp[i] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  sa_nx = rdSa(sa0);
  bring[0] = rdB(sb0, 0);
  sbc_first = rdSb(sb0, 0);
#pragma unroll
  for (int i = 0; i < kTM; ++i) load_sc(i);

  auto step = [&](int c, auto U) {
    constexpr int u = decltype(U)::value;
    uint8_t* const acur = u == 0 ? sa0 : sa1;
    uint8_t* const anxt = u == 0 ? sa1 : sa0;
    uint8_t* const bcur = u == 0 ? sb0 : sb1;
    uint8_t* const bnxt = u == 0 ? sb1 : sb0;
    const int c2 = min(c + 2, nk - 1);
    float sbc[kTN + 1];  // this chunk's column scales, [kTN] = the next chunk's column 0
    sbc[0] = sbc_first;
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
      const v8i bj = bring[j & 1];
      if (j + 1 < kTN) {
        bring[(j + 1) & 1] = rdB(bcur, j + 1);
        sbc[j + 1] = rdSb(bcur, j + 1);
      } else {
        bring[0] = rdB(bnxt, 0);
        sbc[kTN] = rdSb(bnxt, 0);
      }
      fence();
#pragma unroll
      for (int i = 0; i < kTM; ++i) {
        const int t = kTM * j + i;
        pp[i] = mfma(a[i], bj);
        if (t >= kSkew) {
          const int tp = t - kSkew;
          promote(tp % kTM, tp / kTM, sbc[tp / kTM]);
        } else {
          promote(t + 1, kTN - 1, sbc_prev);
          load_sc(t + 1);
        }
        if (t >= kWFirstSlot && t < kWFirstSlot + kWDmaSlots) {
#pragma unroll
          for (int d = 0; d < kWDmaA; ++d)
            if (kWFirstSlot + (d * kWDmaSlots) / kWDmaA == t) issue_a(c2, acur, d);
        }
        if (j == kTN - 1) {
          issue_b(c2, bcur, i);
          if (i == kTM - 1) issue_b(c2, bcur, kWIB);  // the column scales
          a[i] = rdA(anxt, i);
          if (i == 0) sa_nx = rdSa(anxt);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (j == 0) {
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();
        fence();
      }
      if (j == kTN - 2) {
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_waitcnt(kWaitA);
        __builtin_amdgcn_s_barrier();
        fence();
      }
    }
    load_sc(0);
    sbc_prev = sbc[kTN - 1];
    sbc_first = sbc[kTN];
  };

  int c = 0;
  for (; c + 2 <= nk; c += 2) {
    step(c, IC<0>());
    step(c + 1, IC<1>());
  }
  if (c < nk) step(c, IC<0>());
#pragma unroll
  for (int i = 1; i < kTM; ++i) promote(i, kTN - 1, sbc_prev);

  __builtin_amdgcn_s_waitcnt(0x0F70);
  __builtin_amdgcn_s_barrier();
  fence();
  store_tile<kTM, kTN, 1, 16, 1>(acc, ep + (w & 1) * 12288, po, tc.m0 + wr * 64, tc.mend, tc.n0 + wc * 128, lane);
#endif  // __HIP_DEVICE_COMPILE__
}

namespace {

template <int SB_MODE, int OUT_F32, bool GROUPED, bool KG = false, bool SC4 = false, bool EX = false,
          bool QO = false, int INTV = 1>
hipError_t launch_one(const GemmArgs& a, hipStream_t st) {
  const int64_t tiles_n = a.N / kBN, tiles_m = (a.M + kBM - 1) / kBM;
  const int64_t tiles = KG ? a.E * 8 * ((tiles_m * tiles_n + 7) / 8)  // every expert: 8 XCD shares
                        : GROUPED ? (tiles_m + a.E) * tiles_n             // upper bound: a partial tile per expert
                                  : tiles_m * tiles_n;
  if (tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL((k_gemm_fp8<SB_MODE, OUT_F32, GROUPED, KG, SC4, EX, QO, INTV>), dim3((uint32_t)tiles), dim3(kNT),
                     0, st, a);
  return hipGetLastError();
}

}  // namespace

// Tile choice for block-scaled products.  A 256 x 256 tile takes about 1.3x
// the time of a 256 x 128 one (measured) for twice the work, so it wins
// whenever it makes more than one tile per two compute units: below that the
// 256 x 128 grid also finishes in one round and keeps every unit busy.
// Grouped launches estimate the tile count from the total rows.
// fp8q_set_gemm_tile forces either tile (both give bit-identical results),
// for tests and measurement.
static bool use_wide_tile(const GemmArgs& a) {
  if (a.N % kWBN != 0) return false;
  const int forced = gemm_tile_setting();
  if (forced != 0) return forced == 2;
  const int64_t tiles = ((a.M + kBM - 1) / kBM) * (a.N / kWBN);
  return 2 * tiles > device_cu_count();
}

// The exact-accumulation entry points: the 256 x 128 kernel in exact mode.
static hipError_t launch_exact(const GemmArgs& a, hipStream_t st) {
  const bool sc4 = a.ld_sa % 4 == 0 && (reinterpret_cast<uintptr_t>(a.sa) & 15) == 0;
  const bool g = a.offsets != nullptr;
  if (a.qo != nullptr)  // fused output quantization (BF16 Fprop / Dgrad)
    return sc4 ? launch_one<kSbBlock, 0, false, false, true, true, true>(a, st)
               : launch_one<kSbBlock, 0, false, false, false, true, true>(a, st);
  if (a.sb_mode == kSbRow) return launch_one<kSbRow, 1, false, false, false, true>(a, st);
  if (sc4) {
    if (g) return a.out_f32 ? launch_one<kSbBlock, 1, true, false, true, true>(a, st)
                            : launch_one<kSbBlock, 0, true, false, true, true>(a, st);
    return a.out_f32 ? launch_one<kSbBlock, 1, false, false, true, true>(a, st)
                     : launch_one<kSbBlock, 0, false, false, true, true>(a, st);
  }
  if (g) return a.out_f32 ? launch_one<kSbBlock, 1, true, false, false, true>(a, st)
                          : launch_one<kSbBlock, 0, true, false, false, true>(a, st);
  return a.out_f32 ? launch_one<kSbBlock, 1, false, false, false, true>(a, st)
                   : launch_one<kSbBlock, 0, false, false, false, true>(a, st);
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st) {
  return a.exact ? launch_exact(a, st) : launch_gemm_fp8(a, st);
}

// The promotion-interval study: Fprop-form products (block B scales, FP32
// output, 16-byte row-scale blocks) with the partials chained through the
// matrix instruction over `chunks` chunks (0: the whole contraction).
hipError_t launch_gemm_interval(const GemmArgs& a, int chunks, hipStream_t st) {
  switch (chunks) {
    case 1: return launch_one<kSbBlock, 1, false, false, true, false, false, 1>(a, st);
    case 2: return launch_one<kSbBlock, 1, false, false, true, false, false, 2>(a, st);
    case 4: return launch_one<kSbBlock, 1, false, false, true, false, false, 4>(a, st);
    case 8: return launch_one<kSbBlock, 1, false, false, true, false, false, 8>(a, st);
    case 0: return launch_one<kSbBlock, 1, false, false, true, false, false, 0>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_fp8(const GemmArgs& a, hipStream_t st) {
  const bool sc4 = a.ld_sa % 4 == 0 && (reinterpret_cast<uintptr_t>(a.sa) & 15) == 0;
  if (a.sb_mode == kSbRow) {  // weight gradients: FP32 out (row scales 128 B per row: no gain from blocks)
    if (use_wide_tile(a)) {
      const int64_t tn = a.N / kWBN, tm = (a.M + kBM - 1) / kBM;
      if (a.k_grouped)
        hipLaunchKernelGGL((k_gemm_fp8_wide_row<true>), dim3((uint32_t)(a.E * 8 * ((tm * tn + 7) / 8))),
                           dim3(kWNT), 0, st, a);
      else
        hipLaunchKernelGGL((k_gemm_fp8_wide_row<false>), dim3((uint32_t)(tm * tn)), dim3(kWNT), 0, st, a);
      return hipGetLastError();
    }
    if (a.k_grouped) return launch_one<kSbRow, 1, true, true>(a, st);
    return launch_one<kSbRow, 1, false>(a, st);
  }
  if (a.qo != nullptr) {  // fused output quantization (BF16 Fprop / Dgrad)
    if (sc4 && use_wide_tile(a)) {
      hipLaunchKernelGGL((k_gemm_fp8_wide<0, false, true>), dim3((uint32_t)(((a.M + kBM - 1) / kBM) * (a.N / kWBN))),
                         dim3(kWNT), 0, st, a);
      return hipGetLastError();
    }
    return sc4 ? launch_one<kSbBlock, 0, false, false, true, false, true>(a, st)
               : launch_one<kSbBlock, 0, false, false, false, false, true>(a, st);
  }
  // the 256 x 256 tile when it leaves no more than half of the chip idle
  if (sc4 && !(a.out_f32 && a.offsets != nullptr) && use_wide_tile(a)) {  // no FP32-output grouped instantiation
    const int64_t tn = a.N / kWBN, tm = (a.M + kBM - 1) / kBM;
    const int64_t tiles = a.offsets != nullptr ? (tm + a.E) * tn : tm * tn;  // grouped: upper bound
    if (a.offsets != nullptr)
      hipLaunchKernelGGL((k_gemm_fp8_wide<0, true, false>), dim3((uint32_t)tiles), dim3(kWNT), 0, st, a);
    else if (a.out_f32)
      hipLaunchKernelGGL((k_gemm_fp8_wide<1, false, false>), dim3((uint32_t)tiles), dim3(kWNT), 0, st, a);
    else
      hipLaunchKernelGGL((k_gemm_fp8_wide<0, false, false>), dim3((uint32_t)tiles), dim3(kWNT), 0, st, a);
    return hipGetLastError();
  }
  // row scales in 16-byte blocks of 4 chunks when every scale row is 16-byte aligned
  if (a.offsets != nullptr) {
    if (sc4) return a.out_f32 ? launch_one<kSbBlock, 1, true, false, true>(a, st)
                              : launch_one<kSbBlock, 0, true, false, true>(a, st);
    return a.out_f32 ? launch_one<kSbBlock, 1, true>(a, st) : launch_one<kSbBlock, 0, true>(a, st);
  }
  if (sc4) return a.out_f32 ? launch_one<kSbBlock, 1, false, false, true>(a, st)
                            : launch_one<kSbBlock, 0, false, false, true>(a, st);
  return a.out_f32 ? launch_one<kSbBlock, 1, false>(a, st) : launch_one<kSbBlock, 0, false>(a, st);
}

}  // namespace fp8q
