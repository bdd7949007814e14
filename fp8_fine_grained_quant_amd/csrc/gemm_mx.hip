// MXFP8 GEMM on gfx950's block-scaled matrix instruction.
//
// The microscaling variant of the FP8 GEMM: both operands carry E4M3 codes
// with one E8M0 power-of-two scale per 32 consecutive K (OCP Microscaling
// v1.0, MXFP8; the pages name such hardware-supported small-group scaling as
// the counterpart of the method's FP32 group scales, innerforce.co.kr excerpt
// of the DeepSeek-V3 report, paragraph on Figure 7 (a)):
//
//     C[m, n] = sum_k  dec(qa[m, k]) * 2^(ea[m, k/32] - 127) * dec(qb[n, k]) * 2^(eb[n, k/32] - 127)
//
// v_mfma_scale_f32_16x16x128_f8f6f4 applies the scales itself: per row of
// each operand, each of the four 32-K blocks of the instruction takes one
// scale byte from one lane, so every product is scaled before the
// instruction sums it, and the FP32 accumulator is chained through the
// instruction's C operand.  There is no per-chunk promotion on the
// vector ALU: the matrix core does all the arithmetic.
//
// Pipeline (the layout of the method's FP8 kernel, minus its promotion):
// 256 x 128 workgroup tile, four waves of 64 x 128 (4 x 8 sub-tiles),
// operands brought to LDS by direct buffer loads in three stages with 16-byte
// chunks XOR-swizzled by row, two barriers per 128-K chunk, the next chunk's
// loads spread over the slots between them.
//
// Operand layout: lane l supplies row l%16 of the 16-row slice and bytes
// [16g, 16g + 16) and [64 + 16g, 64 + 16g + 16) of the chunk, g = l/16 (the
// FP8 kernel's layout).  Under this layout the instruction scales chunk bytes
// [32b, 32b + 32), the 32-block 4*kb + b, by the scale byte that lane group b
// passes for that row (so a lane group's scale covers data held by two lane
// groups); the parity tests against the oracle establish it.  Lane (l, g)
// therefore passes byte g of the row's 4-byte scale word of the chunk,
// shifted down to bits [7:0] (operand select 0).

#include "device_common.h"
#include "gemm_tile.h"
#include "launch.h"

namespace fp8q {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr;

constexpr int kBM = 256, kBN = 128, kBK = 128;
constexpr int kNT = 256;
constexpr int kTM = 4, kTN = 8;
constexpr int kIA = kBM * kBK / (16 * kNT);       // 16-byte A loads per lane per chunk
constexpr int kIB = kBN * kBK / (16 * kNT);       // 16-byte B loads per lane per chunk

// SC4: the A scale words travel in blocks of 4 chunks (16 bytes per row, one
// load per 4 chunks into a 2-block ring); it needs 16-byte aligned scale rows.
template <bool SC4>
struct MxStage {
  static constexpr int a = 0;                     // [256 rows][128 B], swizzled
  static constexpr int b = kBM * kBK;             // [128 rows][128 B], swizzled
  static constexpr int sa = b + kBN * kBK;        // 256 A scale words (not SC4)
  static constexpr int sb = sa + (SC4 ? 0 : 4 * kNT);  // 128 B scale words as [l16][j] (+128 spare)
  static constexpr int bytes = sb + 4 * kNT;
  static constexpr int ring = SC4 ? 2 * 256 * 4 : 4;   // words of the SC4 ring
  static constexpr int dummy = SC4 ? 1024 : 16;
  static_assert(3 * bytes + 4 * ring + dummy <= 160 * 1024, "LDS of one CU");
  static_assert(4 * 12288 <= bytes, "epilogue staging fits in one stage");
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ v8i make_frag(uint4 lo, uint4 hi) {
  v8i f;
  f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
  f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
  return f;
}

template <int V>
struct IC {
  static constexpr int value = V;
};

}  // namespace

// GROUPED: rows grouped by expert (g.offsets, g.E), tiles never straddle
// experts, and expert e's B codes and scales start g.b_estride and
// sb_estride bytes after expert e-1's.
template <int OUT_F32, bool SC4, bool GROUPED>
__global__ __launch_bounds__(kNT) void k_gemm_mx(MxArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef MxStage<SC4> S;
  __shared__ __attribute__((aligned(16))) uint8_t st0[S::bytes];
  __shared__ __attribute__((aligned(16))) uint8_t st1[S::bytes];
  __shared__ __attribute__((aligned(16))) uint8_t st2[S::bytes];
  __shared__ __attribute__((aligned(16))) uint32_t scA[S::ring];
  __shared__ __attribute__((aligned(16))) uint8_t dmy[S::dummy];

  const GemmArgs& q = p.g;
  TileCoord tc;
  if (!tile_coord<kBM, kBN, GROUPED>(q, tc)) return;
  const uint8_t* Bp = q.B + (GROUPED ? (int64_t)tc.e * q.b_estride : 0);
  const uint8_t* sbp = p.sb + (GROUPED ? (int64_t)tc.e * p.sb_estride : 0);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int nk = (int)(q.K / kBK);
  const int rows = (int)min(tc.mend - tc.m0, (int64_t)kBM);

  // Buffer ranges: A and its scales cover the tile's valid rows only (a row
  // past them reads nothing), B and its scales the tile's 128 rows.
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(q.A + tc.m0 * q.lda, (uint32_t)(rows * q.lda));
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(Bp + (int64_t)tc.n0 * q.ldb, (uint32_t)(kBN * q.ldb));
  const __amdgpu_buffer_rsrc_t rSa = make_rsrc(p.sa + tc.m0 * p.ld_sa, (uint32_t)(rows * p.ld_sa));
  const __amdgpu_buffer_rsrc_t rSb = make_rsrc(sbp + (int64_t)tc.n0 * p.ld_sb, (uint32_t)(kBN * p.ld_sb));
  // Wave w's d-th 16-byte load of a tile fills LDS bytes [(w*I + d)*1024, +1024):
  // rows (w*I + d)*8 + lane/8, physical piece lane%8 = logical piece (lane%8) ^ (row%8).
  const int r8 = lane >> 3, lc = (lane & 7) ^ r8;
  const uint32_t voffA = (uint32_t)((w * kIA * 8 + r8) * q.lda + 16 * lc);
  const uint32_t voffB = (uint32_t)((w * kIB * 8 + r8) * q.ldb + 16 * lc);
  const uint32_t stepA = (uint32_t)(8 * q.lda), stepB = (uint32_t)(8 * q.ldb);
  // A scales: lane (w, l) fetches row 64w + l (clamped to a valid row).
  // B scales: lane L = 64w + l (mod 128) fetches tile row 16*(L%8) + L/8 into
  // word L, so the words land as [l16][j] and a lane reads its 8 columns'
  // words with two 16-byte LDS reads (waves 2, 3 load nothing into spare words).
  const uint32_t voffSa = (uint32_t)(min(w * 64 + lane, rows - 1) * p.ld_sa);
  const int Lb = (w * 64 + lane) & (kBN - 1);
  const uint32_t voffSb = (uint32_t)((16 * (Lb & 7) + (Lb >> 3)) * p.ld_sb);

  constexpr int kDma = kIA + kIB + 2;
  auto issue_one = [&](int kb, uint8_t* st, int d) {
    const uint32_t ka = (uint32_t)kb * kBK;
    if (d < kIA) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_ptr)(st + S::a + (w * kIA + d) * 1024), 16,
                                               voffA + d * stepA, ka, 0, 0);
    } else if (d < kIA + kIB) {
      const int qq = d - kIA;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_ptr)(st + S::b + (w * kIB + qq) * 1024), 16,
                                               voffB + qq * stepB, ka, 0, 0);
    } else if (d == kIA + kIB) {
      if (SC4) {
        // the block of 4 chunks that starts at chunk kb, else an out-of-range
        // load (no memory access) that keeps the per-chunk load count
        const bool real = (kb & 3) == 0;
        uint8_t* dst = real ? reinterpret_cast<uint8_t*>(scA) + ((kb >> 2) & 1) * 4096 + w * 1024 : dmy;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rSa, (lds_ptr)dst, 16, real ? voffSa : kNoAccess,
                                                 real ? (uint32_t)kb * 4 : 0u, 0, 0);
      } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rSa, (lds_ptr)(st + S::sa + w * 256), 4, voffSa, (uint32_t)kb * 4,
                                                 0, 0);
      }
    } else {
      // waves 2, 3: an out-of-range load (no memory access) into the spare
      // words, which keeps every wave's load count per chunk
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rSb, (lds_ptr)(st + S::sb + w * 256), 4, w < 2 ? voffSb : kNoAccess,
                                               w < 2 ? (uint32_t)kb * 4 : 0u, 0,
                                               0);
    }
  };
  auto issue = [&](int kb, uint8_t* st) {
#pragma unroll
    for (int d = 0; d < kDma; ++d) issue_one(kb, st, d);
  };
  constexpr int kFirstDmaSlot = kTM, kDmaSlots = kTM * (kTN - 2);
  static_assert(kDma <= kDmaSlots, "one direct load per slot at most");
  constexpr int kWaitPrev = 0x0F70 | (kDma & 15) | ((kDma >> 4) << 14);  // vmcnt(kDma) only

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
  const uint32_t sh = 8 * g;
  // A scale of sub-tile i's row l16 for chunk kb, lane group g's byte in bits [7:0]
  auto rdSa = [&](const uint8_t* st, int kb, int i) -> int {
    const int row = w * 64 + 16 * i + l16;
    if (SC4) return (int)(scA[((kb >> 2) & 1) * 1024 + row * 4 + (kb & 3)] >> sh);
    return (int)(*reinterpret_cast<const uint32_t*>(st + S::sa + 4 * row) >> sh);
  };
  // B scales of the lane's 8 columns 16j + l16, j = 0..7
  auto rdSb = [&](const uint8_t* st, int (&out)[kTN]) {
    const uint4 lo = *reinterpret_cast<const uint4*>(st + S::sb + 32 * l16);
    const uint4 hi = *reinterpret_cast<const uint4*>(st + S::sb + 32 * l16 + 16);
    out[0] = (int)(lo.x >> sh); out[1] = (int)(lo.y >> sh); out[2] = (int)(lo.z >> sh); out[3] = (int)(lo.w >> sh);
    out[4] = (int)(hi.x >> sh); out[5] = (int)(hi.y >> sh); out[6] = (int)(hi.z >> sh); out[7] = (int)(hi.w >> sh);
  };

  v4f acc[kTM][kTN];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  v8i a[kTM];       // A fragments of the current chunk
  v8i bring[3];     // B fragments, ring over the global column index 8c + j
  int sa[kTM];      // A scale bytes of the current chunk
  int sb[kTN];      // B scale bytes of the current chunk
  auto fence = [] { asm volatile("" ::: "memory"); };

  // ---- prologue: chunks 0 and 1 in flight, chunk 0 published, its fragments
  // and scales in registers
  issue(0, st0);
  issue(min(1, nk - 1), st1);
  __builtin_amdgcn_s_waitcnt(kWaitPrev);
  __builtin_amdgcn_s_barrier();
  fence();
#pragma unroll
  for (int i = 0; i < kTM; ++i) {
    a[i] = rdA(st0, i);
    sa[i] = rdSa(st0, 0, i);
  }
  bring[0] = rdB(st0, 0);
  bring[1] = rdB(st0, 1);
  rdSb(st0, sb);

  // ---- one chunk.  Stage u holds chunk c; stage (u+1)%3 receives or holds
  // chunk c+1; stage (u+2)%3 held chunk c-1 and is refilled with chunk c+2.
  auto step = [&](int c, auto U) {
    constexpr int u = decltype(U)::value;
    uint8_t* const cur = u == 0 ? st0 : u == 1 ? st1 : st2;
    uint8_t* const nxt = u == 0 ? st1 : u == 1 ? st2 : st0;
    uint8_t* const fut = u == 0 ? st2 : u == 1 ? st0 : st1;
    int sb_nx[kTN];
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
      // B two columns ahead: this chunk's columns 2..7 at columns 0..5, the
      // next chunk's columns 0 and 1 at column 7 (after the barrier that
      // publishes it), with the next chunk's B scales
      const v8i bcur = bring[(2 * u + j) % 3];
      if (j + 2 < kTN) {
        bring[(2 * u + j + 2) % 3] = rdB(cur, j + 2);
      } else if (j == kTN - 1) {
        bring[(2 * u + kTN) % 3] = rdB(nxt, 0);
        bring[(2 * u + kTN + 1) % 3] = rdB(nxt, 1);
        rdSb(nxt, sb_nx);
      }
      fence();
#pragma unroll
      for (int i = 0; i < kTM; ++i) {
        const int t = kTM * j + i;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[i], bcur, acc[i][j], 0, 0, 0, sa[i], 0, sb[j]);
        if (t >= kFirstDmaSlot && t < kFirstDmaSlot + kDmaSlots) {
#pragma unroll
          for (int d = 0; d < kDma; ++d)
            if (kFirstDmaSlot + (d * kDmaSlots) / kDma == t) issue_one(min(c + 2, nk - 1), fut, d);
        }
        if (j == kTN - 1) {
          // a[i] and sa[i] are no longer needed for this chunk: fetch the next chunk's
          a[i] = rdA(nxt, i);
          sa[i] = rdSa(nxt, min(c + 1, nk - 1), i);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (j == 0) {
        // every wave has finished reading chunk c-1: its stage may be
        // refilled with chunk c+2 (past the end, the last chunk again, so
        // every chunk issues the same loads and the wait counts stay exact)
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
#pragma unroll
    for (int j = 0; j < kTN; ++j) sb[j] = sb_nx[j];
  };

  int c = 0;
  for (; c + 3 <= nk; c += 3) {
    step(c, IC<0>());
    step(c + 1, IC<1>());
    step(c + 2, IC<2>());
  }
  if (c < nk) step(c, IC<0>());
  if (c + 1 < nk) step(c + 1, IC<1>());

  // ---- epilogue: no direct load may still target LDS, and every wave is
  // done reading; each wave stages its strip in its own 12 KB of stage 0
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __builtin_amdgcn_s_barrier();
  fence();
  float out[kTM][kTN][4];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) out[i][j][r] = acc[i][j][r];
  store_tile<kTM, kTN, OUT_F32, OUT_F32 ? 16 : 32>(out, st0 + w * 12288, q, tc.m0 + w * 64, tc.mend, tc.n0, lane);
#endif  // __HIP_DEVICE_COMPILE__
}

// ---------------------------------------------------------------------------
// Wide tile: 256 x 256 outputs, eight waves (two per SIMD), each the 64 x 128
// strip above, so results are bit-identical to k_gemm_mx.  A and B live in
// separate LDS regions, two chunks each: A region c%2 takes A(c+2) as soon as
// every wave holds A(c) in registers (first barrier of chunk c), B region c%2
// takes B(c+2) in the last column, after every wave has read B(c) -- the same
// schedule as the FP8 kernel's wide tile.  The chunk's B scale words ride
// with its B loads ([half][l16][j] words beside the B region); the A scale
// words travel in the 4-chunk ring (16-byte aligned scale rows only).
constexpr int kWBN = 256, kWNT = 512;
constexpr int kWIA = kBM * kBK / (16 * kWNT);  // 4
constexpr int kWIB = kWBN * kBK / (16 * kWNT);  // 4
constexpr int kWDmaA = kWIA + 1, kWDmaB = kWIB + 1;
constexpr int kWFirstSlot = kTM, kWDmaSlots = 20;
constexpr int kWScB = 2048;  // bytes beside each B region: 256 scale words (+ a spare copy)
static_assert(kWIB == kTM && kWDmaA <= kWDmaSlots && kWFirstSlot + kWDmaSlots <= kTM * (kTN - 1), "schedule");

template <int OUT_F32>
__global__ __launch_bounds__(kWNT) void k_gemm_mx_wide(MxArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int RA = kBM * kBK, RB = kWBN * kBK;
  __shared__ __attribute__((aligned(16))) uint8_t sa0[RA];
  __shared__ __attribute__((aligned(16))) uint8_t sa1[RA];
  __shared__ __attribute__((aligned(16))) uint8_t sb0[RB + kWScB];
  __shared__ __attribute__((aligned(16))) uint8_t sb1[RB + kWScB];
  __shared__ __attribute__((aligned(16))) uint32_t scA[2 * 256 * 4];
  __shared__ __attribute__((aligned(16))) uint8_t dmy[1024];

  const GemmArgs& q = p.g;
  TileCoord tc;
  tile_coord<kBM, kWBN, false>(q, tc);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = w & 3, wc = w >> 2;
  const int l16 = lane & 15, g = lane >> 4;
  const int nk = (int)(q.K / kBK);
  const int rows = (int)min(tc.mend - tc.m0, (int64_t)kBM);

  const __amdgpu_buffer_rsrc_t rA = make_rsrc(q.A + tc.m0 * q.lda, (uint32_t)(rows * q.lda));
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(q.B + (int64_t)tc.n0 * q.ldb, (uint32_t)(kWBN * q.ldb));
  const __amdgpu_buffer_rsrc_t rSa = make_rsrc(p.sa + tc.m0 * p.ld_sa, (uint32_t)(rows * p.ld_sa));
  const __amdgpu_buffer_rsrc_t rSb = make_rsrc(p.sb + (int64_t)tc.n0 * p.ld_sb, (uint32_t)(kWBN * p.ld_sb));
  const int r8 = lane >> 3, lc = (lane & 7) ^ r8;
  const uint32_t voffA = (uint32_t)((w * kWIA * 8 + r8) * q.lda + 16 * lc);
  const uint32_t voffB = (uint32_t)((w * kWIB * 8 + r8) * q.ldb + 16 * lc);
  const uint32_t stepA = (uint32_t)(8 * q.lda), stepB = (uint32_t)(8 * q.ldb);
  // A scales: lane (w, l), w < 4, fetches row 64w + l (clamped to a valid
  // row).  B scales: lane L = 64w + l (L < 256, w < 4) fetches the word of
  // column 128 (L / 128) + 16 ((L % 128) % 8) + (L % 128) / 8 into word L, so
  // each half's words land as [l16][j]; waves 4-7 load nothing into a spare copy.
  const uint32_t voffSa = (uint32_t)(min(wr * 64 + lane, rows - 1) * p.ld_sa);
  const int Lb = (w * 64 + lane) & (kWBN - 1), Lh = Lb & 127;
  const uint32_t voffSb = (uint32_t)((128 * (Lb >> 7) + 16 * (Lh & 7) + (Lh >> 3)) * p.ld_sb);

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
  auto issue_b = [&](int kb, uint8_t* br, int qq) {
    if (qq < kWIB)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_ptr)(br + (w * kWIB + qq) * 1024), 16, voffB + qq * stepB,
                                               (uint32_t)kb * kBK, 0, 0);
    else
      // waves 4-7: an out-of-range load (no memory access) into the spare
      // copy, which keeps every wave's load count per chunk
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rSb, (lds_ptr)(br + RB + w * 256), 4, w < 4 ? voffSb : kNoAccess,
                                               w < 4 ? (uint32_t)kb * 4 : 0u, 0, 0);
  };
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
  const uint32_t sh = 8 * g;
  auto rdSa = [&](int kb, int i) -> int {
    const int row = wr * 64 + 16 * i + l16;
    return (int)(scA[((kb >> 2) & 1) * 1024 + row * 4 + (kb & 3)] >> sh);
  };
  auto rdSb = [&](const uint8_t* br, int (&out)[kTN]) {
    const uint8_t* base = br + RB + 512 * wc + 32 * l16;
    const uint4 lo = *reinterpret_cast<const uint4*>(base);
    const uint4 hi = *reinterpret_cast<const uint4*>(base + 16);
    out[0] = (int)(lo.x >> sh); out[1] = (int)(lo.y >> sh); out[2] = (int)(lo.z >> sh); out[3] = (int)(lo.w >> sh);
    out[4] = (int)(hi.x >> sh); out[5] = (int)(hi.y >> sh); out[6] = (int)(hi.z >> sh); out[7] = (int)(hi.w >> sh);
  };

  v4f acc[kTM][kTN];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  v8i a[kTM];
  v8i bring[2];
  int sa[kTM], sb[kTN];
  auto fence = [] { asm volatile("" ::: "memory"); };

#pragma unroll
  for (int d = 0; d < kWDmaA; ++d) issue_a(0, sa0, d);
#pragma unroll
  for (int qq = 0; qq < kWDmaB; ++qq) issue_b(0, sb0, qq);
#pragma unroll
  for (int d = 0; d < kWDmaA; ++d) issue_a(min(1, nk - 1), sa1, d);
#pragma unroll
  for (int qq = 0; qq < kWDmaB; ++qq) issue_b(min(1, nk - 1), sb1, qq);
  __builtin_amdgcn_s_waitcnt(0x0F70 | (kWDmaA + kWDmaB));  // A(0), B(0) landed
  __builtin_amdgcn_s_barrier();
  fence();
#pragma unroll
  for (int i = 0; i < kTM; ++i) {
    a[i] = rdA(sa0, i);
    sa[i] = rdSa(0, i);
  }
  bring[0] = rdB(sb0, 0);
  rdSb(sb0, sb);

  auto step = [&](int c, auto U) {
    constexpr int u = decltype(U)::value;
    uint8_t* const acur = u == 0 ? sa0 : sa1;
    uint8_t* const anxt = u == 0 ? sa1 : sa0;
    uint8_t* const bcur = u == 0 ? sb0 : sb1;
    uint8_t* const bnxt = u == 0 ? sb1 : sb0;
    const int c2 = min(c + 2, nk - 1);
    int sb_nx[kTN];
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
      const v8i bj = bring[j & 1];
      if (j + 1 < kTN) {
        bring[(j + 1) & 1] = rdB(bcur, j + 1);
      } else {
        bring[0] = rdB(bnxt, 0);
        rdSb(bnxt, sb_nx);
      }
      fence();
#pragma unroll
      for (int i = 0; i < kTM; ++i) {
        const int t = kTM * j + i;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[i], bj, acc[i][j], 0, 0, 0, sa[i], 0, sb[j]);
        if (t >= kWFirstSlot && t < kWFirstSlot + kWDmaSlots) {
#pragma unroll
          for (int d = 0; d < kWDmaA; ++d)
            if (kWFirstSlot + (d * kWDmaSlots) / kWDmaA == t) issue_a(c2, acur, d);
        }
        if (j == kTN - 1) {
          issue_b(c2, bcur, i);
          if (i == kTM - 1) issue_b(c2, bcur, kWIB);  // the B scale words
          a[i] = rdA(anxt, i);
          sa[i] = rdSa(min(c + 1, nk - 1), i);
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
        // every wave has read B(c) and its scale words; A(c+1), B(c+1) landed
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_waitcnt(kWaitA);
        __builtin_amdgcn_s_barrier();
        fence();
      }
    }
#pragma unroll
    for (int j = 0; j < kTN; ++j) sb[j] = sb_nx[j];
  };

  int c = 0;
  for (; c + 2 <= nk; c += 2) {
    step(c, IC<0>());
    step(c + 1, IC<1>());
  }
  if (c < nk) step(c, IC<0>());

  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __builtin_amdgcn_s_barrier();
  fence();
  float out[kTM][kTN][4];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) out[i][j][r] = acc[i][j][r];
  uint8_t* const ep = (w >> 1) == 0 ? sa0 : (w >> 1) == 1 ? sa1 : (w >> 1) == 2 ? sb0 : sb1;
  store_tile<kTM, kTN, OUT_F32, OUT_F32 ? 16 : 32>(out, ep + (w & 1) * 12288, q, tc.m0 + wr * 64, tc.mend,
                                                 tc.n0 + wc * 128, lane);
#endif  // __HIP_DEVICE_COMPILE__
}

namespace {

template <int OUT_F32, bool SC4, bool GROUPED = false>
hipError_t launch_mx(const MxArgs& a, hipStream_t st) {
  const int64_t tiles_m = (a.g.M + kBM - 1) / kBM, tiles_n = a.g.N / kBN;
  // grouped: an upper bound (a partial m-tile per expert); the kernel counts the real tiles
  const int64_t tiles = GROUPED ? (tiles_m + a.g.E) * tiles_n : tiles_m * tiles_n;
  if (tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL((k_gemm_mx<OUT_F32, SC4, GROUPED>), dim3((uint32_t)tiles), dim3(kNT), 0, st, a);
  return hipGetLastError();
}

}  // namespace

// The 256 x 256 tile when its grid has more tiles than half the compute
// units (the rule and the fp8q_set_gemm_tile setting of the FP8 GEMM).
static bool use_wide_mx(const MxArgs& a) {
  if (a.g.N % kWBN != 0) return false;
  const int forced = gemm_tile_setting();
  if (forced != 0) return forced == 2;
  return 2 * ((a.g.M + kBM - 1) / kBM) * (a.g.N / kWBN) > device_cu_count();
}

hipError_t launch_gemm_mx(const MxArgs& a, hipStream_t st) {
  const bool sc4 = a.ld_sa % 16 == 0 && (reinterpret_cast<uintptr_t>(a.sa) & 15) == 0;
  if (a.g.offsets != nullptr) {  // grouped rows: the 256 x 128 tile
    if (sc4) return a.g.out_f32 ? launch_mx<1, true, true>(a, st) : launch_mx<0, true, true>(a, st);
    return a.g.out_f32 ? launch_mx<1, false, true>(a, st) : launch_mx<0, false, true>(a, st);
  }
  if (sc4 && use_wide_mx(a)) {
    const int64_t tiles = ((a.g.M + kBM - 1) / kBM) * (a.g.N / kWBN);
    if (tiles <= 0) return hipSuccess;
    if (a.g.out_f32)
      hipLaunchKernelGGL((k_gemm_mx_wide<1>), dim3((uint32_t)tiles), dim3(kWNT), 0, st, a);
    else
      hipLaunchKernelGGL((k_gemm_mx_wide<0>), dim3((uint32_t)tiles), dim3(kWNT), 0, st, a);
    return hipGetLastError();
  }
  if (sc4) return a.g.out_f32 ? launch_mx<1, true>(a, st) : launch_mx<0, true>(a, st);
  return a.g.out_f32 ? launch_mx<1, false>(a, st) : launch_mx<0, false>(a, st);
}

}  // namespace fp8q
