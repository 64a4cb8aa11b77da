// kvq_decode_fast.hip -- matrix-core (MFMA) split-context decode over the
// packed cache for uniform 2/4/8-bit keys and values.
//
// One wavefront per split; a 32-token block is two 16-token tiles.
//   scores  S[r][t] = sum_c A[r][c] B[c][t] with v_mfma_f32_16x16x32_f16.  B
//           holds the codes as normal fp16 values base + code / inv_unit
//           (every product exact); with one key scale per channel per block
//           (KVTuner obs. 2 / KVQuant (i)) A = q * s as an exact fp16 hi + lo
//           pair, and the offset and the zero points enter through one more
//           MFMA against the block's (z, s) columns.  For InnerQ inner-dimension
//           groups (per-token scales) A = q and the group sums are scaled
//           afterwards; an 8-bit group of a mixed 4/8-bit layer enters the
//           same 4-bit operand with its low nibble in the next four mantissa
//           bits (1 + c/256 instead of 1 + c/16) and takes its own scale.
//   values  O[r][c] += sum_t (p[r][t] * s[t][g]) code[t][c]: per-token value
//           scales (KIVI layout) fold into P as an exact hi + lo pair; the zero
//           points and the code offset are one more MFMA against the block's
//           (z, s) columns.
//   online softmax in the log2 domain; P is rounded to fp16 once and the
//   denominator sums the same rounded weights.
// Only the first G rows of the 16-row tiles carry queries (the GQA group of a
// kv head); the keys and values of a block are read once for all of them.
// Block records stream HBM -> LDS with global_load_lds_dwordx4 into a ring of
// NBUF slots; a slot takes its next block as soon as the current one has read
// its record out, so NBUF - 1 to NBUF blocks are in flight behind the one
// being computed.  Sink / window
// tokens (fp16) are read straight into registers by splits of their own,
// after the body splits.  Each split writes an
// (o, max, sum) partial; decode_merge_kernel combines them by log-sum-exp and
// undoes the value rotation.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_mfma.h"

namespace kvq {
namespace {

// ---- code words -> eight fp16 code values, K-order = element order.
// 2-bit codes become 1 + c/4 and 4-bit codes 1 + c/16 (code bits placed at
// the top of the fp16 mantissa under the exponent of 1.0: a shift and one
// v_and_or_b32 per output word); 8-bit codes become 1024 + c (one byte
// permute per output word against a register of 0x64 exponent bytes).
// Normal fp16 operands keep every MFMA product exact; the constant offset
// (base * sum of A) is removed afterwards.
template <int B> struct CodeEnc;
template <> struct CodeEnc<2> { static constexpr float base = 1.f, inv_unit = 4.f; };
template <> struct CodeEnc<4> { static constexpr float base = 1.f, inv_unit = 16.f; };
template <> struct CodeEnc<8> { static constexpr float base = 1024.f, inv_unit = 1.f; };

// Loop-invariant unpack constants, held in registers (the VOP3 forms take
// no literal operands) and made opaque once, so that the and-or pairs are
// selected as single v_and_or_b32 and the constants are not rematerialised.
struct Unpack {
  uint32_t m4, m2, e8, m4lo, m4a, m4b;  // VGPRs
  uint32_t one2, e64, e4;               // SGPRs: fp16 1.0, 64.0, 4.0 in both halves
};
__device__ __forceinline__ uint32_t andor(uint32_t x, uint32_t m, uint32_t o) { return (x & m) | o; }
__device__ __forceinline__ half8 ex4(const Unpack& k, uint32_t x) {
  return h8(andor(x << 6, k.m4, k.one2), andor(x << 2, k.m4, k.one2), andor(x >> 2, k.m4, k.one2),
            andor(x >> 6, k.m4, k.one2));
}
// 4-bit fields x with low nibbles y below them (8-bit codes c = 16 x + y of
// mixed-width key groups): 1 + x/16 + y/256 = 1 + c/256; y = 0 gives ex4.
__device__ __forceinline__ half8 ex4lo(const Unpack& k, uint32_t x, uint32_t y) {
  return h8(andor(y << 2, k.m4lo, andor(x << 6, k.m4, k.one2)), andor(y >> 2, k.m4lo, andor(x << 2, k.m4, k.one2)),
            andor(y >> 6, k.m4lo, andor(x >> 2, k.m4, k.one2)), andor(y >> 10, k.m4lo, andor(x >> 6, k.m4, k.one2)));
}
// Inner-group 4-bit operands, two of four words without a shift: each field
// takes the exponent under which its code weighs c/16 -- bits 0-3 of a half
// read as 64 + c/16, bits 4-7 as 4 + c/16 -- so the constant part depends on
// the position (64 for elements 0-1 of an eight-element K chunk, 4 for 2-7)
// and the group-sum MFMA starts from minus the matching weighted sum of q.
__device__ __forceinline__ half8 ex4w(const Unpack& k, uint32_t x) {
  return h8(andor(x, k.m4a, k.e64), andor(x, k.m4b, k.e4), andor(x >> 4, k.m4b, k.e4), andor(x >> 8, k.m4b, k.e4));
}
template <int E>
__device__ __forceinline__ half8 ex2(const Unpack& k, uint32_t x) {
  if constexpr (E == 0)
    return h8(andor(x << 8, k.m2, k.one2), andor(x << 6, k.m2, k.one2), andor(x << 4, k.m2, k.one2),
              andor(x << 2, k.m2, k.one2));
  else
    return h8(andor(x, k.m2, k.one2), andor(x >> 2, k.m2, k.one2), andor(x >> 4, k.m2, k.one2),
              andor(x >> 6, k.m2, k.one2));
}
// bytes b0, b1 (sh = 0) or b2, b3 (sh = 16) of x as fp16 1024 + b
__device__ __forceinline__ uint32_t u8pair(const Unpack& k, uint32_t x, int sh) {
  return __builtin_amdgcn_perm(k.e8, x, sh == 0 ? 0x04010400u : 0x04030402u);
}
__device__ __forceinline__ half8 ex8(const Unpack& k, uint32_t x, uint32_t y) {
  return h8(u8pair(k, x, 0), u8pair(k, x, 16), u8pair(k, y, 0), u8pair(k, y, 16));
}

// B operand of K-step j from a lane's key chunk (32 channels, KB bits each)
template <int KB>
__device__ __forceinline__ half8 kstep(const Unpack& k, const uint32_t* w, int j) {
  if constexpr (KB == 4) return ex4(k, w[j]);
  if constexpr (KB == 2) return (j & 1) ? ex2<1>(k, w[j >> 1]) : ex2<0>(k, w[j >> 1]);
  if constexpr (KB == 8) return ex8(k, w[2 * j], w[2 * j + 1]);
}
// B operand of value N-tile nt from a lane's value chunk
template <int VB>
__device__ __forceinline__ half8 vtile(const Unpack& k, const uint32_t* w, int nt) {
  if constexpr (VB == 4) return ex4(k, w[nt]);
  if constexpr (VB == 2) return (nt & 1) ? ex2<1>(k, w[nt >> 1]) : ex2<0>(k, w[nt >> 1]);
  if constexpr (VB == 8) return ex8(k, w[2 * nt], w[2 * nt + 1]);
}

// channel of K-step j, element kk for lane group g4
template <bool INNER>
__device__ __forceinline__ int kchan(int g4, int j, int kk) {
  if constexpr (INNER) return (j < 2 ? 16 * g4 + 8 * j : 64 + 16 * g4 + 8 * (j - 2)) + kk;
  return 32 * g4 + 8 * j + kk;
}


// Compile-time record layout of a block (D = 128, value groups of 32, no
// sparse outliers; MIX: inner groups of 64 with one 8-bit group per token);
// the launcher checks it against the layer's layout.
template <int KB, int VB, bool INNER, bool MIX = false>
struct Rec {
  static constexpr int kc = 32 * 16 * KB;
  static constexpr int km = INNER ? 32 * 2 * 4 : 2 * D * 2;
  static constexpr int vc = 32 * 16 * VB;
  static constexpr int vm = 2 * 4 * 32 * 2;
  static constexpr int kx = MIX ? 32 * 32 : 0;  // low nibbles: 32 tokens x 64 channels
  static constexpr int ks = MIX ? 32 : 0;       // group masks
  static constexpr int off_km = kc;
  static constexpr int off_vc = off_km + km;
  static constexpr int off_vm = off_vc + vc;
  static constexpr int off_kx = off_vm + vm;
  static constexpr int off_ks = off_kx + kx;
  static constexpr int bytes = off_ks + ks;
  static constexpr int loads = (bytes + 1023) / 1024;  // 1 KiB per wave-wide load
};

// Ring depth and residency.  Every instance is sized for three wavefronts
// per SIMD (twelve per CU): the ring takes as many slots (2..4) as a twelfth
// of the CU's LDS allows (deeper rings keep more blocks in flight behind the
// VALU / MFMA work of the block being computed).  Residency must come out as
// a multiple of four wavefronts per CU, or the SIMDs get unequal shares of
// the split plan's equal splits: an instance whose LDS would admit 9..11
// workgroups per CU pads its first ring slot (static LDS) to admit eight.
constexpr int kLdsPerCu = 160 * 1024;
constexpr int kLdsShare3 = kLdsPerCu / 12;       // three wavefronts per SIMD
constexpr int kLdsShare2 = kLdsPerCu / 9 + 512;  // at most eight per CU
template <int KB, int VB, int G, bool INNER, bool MIX>
constexpr int ring_slots() {
  constexpr int budget = kLdsShare3 - 512 - 16 * 32 * 2 - 512;
  constexpr int n = budget / (Rec<KB, VB, INNER, MIX>::loads * 1024);
  return n < 2 ? 2 : (n > 4 ? 4 : n);
}
template <int KB, int VB, bool INNER, bool MIX, int NBUF>
constexpr int ring_pad() {
  constexpr int slot = Rec<KB, VB, INNER, MIX>::loads * 1024;
  constexpr int used = NBUF * slot + 16 * 32 * 2 + (NBUF < 3 ? 16 : 0) + (NBUF < 4 ? 16 : 0);
  return (used > kLdsShare3 && used < kLdsShare2) ? kLdsShare2 - used : 0;
}
// Wavefronts per SIMD the register allocation is held to: three for the
// GQA instances whose registers fit 168 with at most a spill outside the
// block loop and for the 2-bit rotated-value instances with per-channel keys
// (whose appended-token rotation would otherwise set their register count),
// else what they need.
template <int KB, int VB, int G, bool INNER, bool MIX, bool PLO = false>
constexpr int waves_per_simd() {
  return ((G >= 4 && (VB == 2 || (VB == 4 && !INNER && KB != 8))) || (PLO && !INNER && VB == 2)) ? 3 : 1;
}
template <int KB, int VB, int G, bool INNER, bool MIX, int NBUF, bool PLO>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(waves_per_simd<KB, VB, G, INNER, MIX, PLO>())))
decode_mfma_kernel(LayerDesc L, DecodeJob J) {
  using R = Rec<KB, VB, INNER, MIX>;
  static_assert(!MIX || (INNER && KB == 4), "mixed groups: 4-bit inner keys");
  // one LDS object per ring slot: the compiler then tells the slots apart and
  // keeps the partial vmcnt waits instead of draining every in-flight load
  static_assert(NBUF >= 2 && NBUF <= 4, "ring of 2 to 4 slots");
  __shared__ __attribute__((aligned(16))) uint8_t ring0[R::loads * 1024 + ring_pad<KB, VB, INNER, MIX, NBUF>()];
  __shared__ __attribute__((aligned(16))) uint8_t ring1[R::loads * 1024];
  __shared__ __attribute__((aligned(16))) uint8_t ring2[NBUF >= 3 ? R::loads * 1024 : 16];
  __shared__ __attribute__((aligned(16))) uint8_t ring3[NBUF >= 4 ? R::loads * 1024 : 16];
  lds_u8* const slot0 = (lds_u8*)ring0;
  lds_u8* const slot1 = (lds_u8*)ring1;
  lds_u8* const slot2 = (lds_u8*)ring2;
  lds_u8* const slot3 = (lds_u8*)ring3;
  auto slot_at = [&](int k) __attribute__((always_inline)) {
    return k == 0 ? slot0 : (k == 1 ? slot1 : (k == 2 ? slot2 : slot3));
  };
  __shared__ __attribute__((aligned(16))) _Float16 ptile[16][32];
  // PLO: the weights' residuals fp16(p - fp16(p)), so that P enters the
  // value products as a hi + lo pair too (rows G..2G-1 of the value tiles)
  __shared__ __attribute__((aligned(16))) _Float16 plo[PLO ? 16 : 1][32];
  const int l = threadIdx.x;
  const int n16 = l & 15, g4 = l >> 4;
  const int nsplit = J.nsplit;
  const int sp = blockIdx.x;
  const int u = blockIdx.y;
  const int b = u / L.Hkv, h = u % L.Hkv;
  const TokenState st = J.st;
  constexpr int RI = G < 4 ? G : 4;           // output rows per lane (registers)
  const bool rows_here = 4 * g4 < G;           // lane holds real query rows
  constexpr int ngv = D / 32;                  // value groups of 32 channels
  // Query groups of 8 (or 4) rows fill only lanes 0-31 (or 0-15) of a score
  // tile's accumulators.  The two 16-token tiles of a block are folded into
  // one register set with a permlane swap: tile 1's live lanes move into
  // tile 0's empty half (row of 16), so the per-token score factors and the
  // softmax run once per lane for the whole block instead of once per tile.
  // Folded, lane (n16, g4) holds rows frow..frow+3 of token ftok.
  constexpr int kFold = G == 8 ? 32 : (G == 4 ? 16 : 0);
  const int ftile = kFold == 32 ? g4 >> 1 : g4 & 1;
  const int ftok = n16 + 16 * ftile;
  const int frow = kFold == 32 ? 4 * (g4 & 1) : 8 * (g4 >> 1);
  // Groups of 8, 4 or 1 query rows: the value products use the next G rows
  // of the 16-row MFMA too -- rows 0..G-1 take the hi parts of p * s, rows
  // G..2G-1 the lo parts of the same query rows -- so each value tile needs
  // one MFMA instead of two; the split's epilogue adds rows G..2G-1 onto
  // rows 0..G-1 (lanes 32-63 onto 0-31, 16-31 onto 0-15, or row 1 onto row
  // 0 in the same lanes).  A single query row with per-channel keys packs
  // the key products q * s the same way (row 1 of the score tiles, added
  // to row 0 before the softmax).
  constexpr bool kPackLo = G == 8 || G == 4 || G == 1;
  // per-channel keys pack the key products the same way: rows G..2G-1 of
  // the score tiles take the lo parts of q * s (one MFMA per K-step and tile
  // instead of two, half the accumulation chain); they are added onto rows
  // 0..G-1 in the same lane (G = 1) or by the permlane swap that folds the
  // two tiles (G = 4, 8)
  constexpr bool kPackK = !INNER && (G == 1 || G == 4 || G == 8);
  static_assert(!PLO || kPackLo, "the weights' lo parts ride in the packed lo rows");
  auto fold = [&](float a, float b) __attribute__((always_inline)) {
    return kFold == 32 ? swap32(a, b).x : swap16(a, b).x;
  };
  Unpack unp{0x03C003C0u, 0x03000300u, 0x64646464u, 0x003C003Cu, 0x000F000Fu, 0x00F000F0u,
             0x3C003C00u, 0x54005400u, 0x44004400u};
  constexpr bool kWeighted = INNER && !MIX;  // inner 4-bit keys read through ex4w
  pin(unp.m4);
  pin(unp.m2);
  pin(unp.e8);
  if constexpr (MIX) pin(unp.m4lo);
  if constexpr (kWeighted) {
    pin(unp.m4a);
    pin(unp.m4b);
    asm volatile("" : "+s"(unp.e64));
    asm volatile("" : "+s"(unp.e4));
  }
  asm volatile("" : "+s"(unp.one2));

  // LDS byte offsets of this lane's key chunks (K-steps of tile 0; tile 1
  // rows are 16 further).  Key rows stay in their record order: an XOR
  // swizzle of their 16-byte chunks spreads a K-step's 16 rows over more
  // banks, but its address registers made the 168-register instances spill
  // inside the block loop, and it measured slower.
  const uint32_t koff0 = KB == 8 ? n16 * 128 + 32 * g4 : n16 * 16 * KB + 4 * KB * g4;
  const uint32_t koff1 = KB == 8 ? koff0 + 16 : koff0;

  // ---- query operand (natural channel order per K-step)
  half8 qa[4];
  {
    const bool live = n16 < (kPackK ? 2 * G : G);  // packed keys: rows G..2G-1 hold rows 0..G-1 again
    const uint16_t* qp = J.q + (static_cast<int64_t>(b) * L.Hq + h * G + (n16 & (G - 1))) * D;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4 v = ld16(qp + kchan<INNER>(g4, j, 0));
      qa[j] = live ? h8(v) : h8(0u, 0u, 0u, 0u);
    }
  }
  float qsum[2][RI];  // inner groups: per-row sums of q over each 64-channel group
  f32x4 qinit[2];     // inner 4-bit keys: minus the position-weighted sums (group-sum start)

  const float kscale = kLog2e / sqrtf(static_cast<float>(D));
  // row ceilings, starting from a finite value below every score so that
  // masked -inf scores weigh 2^-inf = 0
  constexpr float kNoScore = -3.0e38f;
  float m_run[RI];
#pragma unroll
  for (int i = 0; i < RI; ++i) m_run[i] = kNoScore;
  f32x4 oacc[8];
  // zacc: per query row, columns 0-3 sum_t p_t z_tg, 4-7 sum_t p_t s_tg
  // (value groups g) and column 8 sum_t p_t, the softmax denominator: P is
  // used as fp16 in every product and the denominator sums the same rounded
  // weights, through the same matrix-core product (a column of ones)
  f32x4 zacc = {0.f, 0.f, 0.f, 0.f};
  constexpr uint32_t kOnes = 0x3C003C00u;
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) oacc[nt] = {0.f, 0.f, 0.f, 0.f};

  // Online softmax of one 32-token block in the two-tile layout (lane holds
  // rows 4 g4 + i of tokens n16 and 16 + n16); P (fp16) lands in ptile and
  // the accumulators are rescaled when a row's reference moves.  The row
  // reference m_run is a ceiling rather than the running maximum (see the
  // folded variant below for the reasons and the weight lift).
  constexpr float kPad = 2.f;
  constexpr float kLift = VB == 8 ? 6.f : (VB == 4 ? 2.f : 0.f);
  // Each softmax returns the block's P operands: pa (rows 0..2G-1 hold the
  // fp16 weights of rows 0..G-1, twice) and pz (rows 0..G-1 the same weights;
  // with PLO rows G..2G-1 their residuals, else pa again).
  struct POps {
    half8 pa, pz;
  };
  // LDS byte offsets of the weight tiles (element (r, t) at 2 (32 r + t))
  const uint32_t pt_base = lds_off((lds_u8*)ptile);
  const uint32_t plo_base = lds_off((lds_u8*)plo);
  // lanes of rows G..2G-1 read the residual tile, the others the weights
  const uint32_t pz_addr = (PLO && n16 >= G && n16 < 2 * G ? plo_base : pt_base) + 2 * (32 * (n16 & (G - 1)) + 8 * g4);
  auto p_operands = [&]() __attribute__((always_inline)) -> POps {
    if constexpr (kPackLo) {  // rows G..2G-1 read rows 0..G-1 again
      const bool live = n16 < 2 * G;
      const half8 pr = h8(dsr16_now(pt_base + 2 * (32 * (n16 & (G - 1)) + 8 * g4)));
      const half8 pa = live ? pr : h8(0u, 0u, 0u, 0u);
      if constexpr (PLO) {
        const half8 zr = h8(dsr16_now(pz_addr));
        return POps{pa, live ? zr : h8(0u, 0u, 0u, 0u)};
      }
      return POps{pa, pa};
    }
    const half8 pr = h8(dsr16_now(pt_base + 2 * (32 * n16 + 8 * g4)));
    const half8 pa = n16 < G ? pr : h8(0u, 0u, 0u, 0u);
    return POps{pa, pa};
  };
  auto softmax_tile = [&](f32x4 (&sacc)[2], int count) __attribute__((always_inline)) -> POps {
    if (count < kBlockTokens) {  // wave-uniform: only a partial last block
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        if (16 * nt + n16 >= count)
#pragma unroll
          for (int i = 0; i < 4; ++i) sacc[nt][i] = -INFINITY;
    }
    bool over = false;
#pragma unroll
    for (int i = 0; i < RI; ++i) over |= fmaxf(sacc[0][i], sacc[1][i]) > m_run[i];
    if (__builtin_amdgcn_ballot_w64(over)) {
      float alpha[RI];
#pragma unroll
      for (int i = 0; i < RI; ++i) {
        const float bm = row16_max(fmaxf(sacc[0][i], sacc[1][i]));
        const float mn = bm > m_run[i] ? bm + kPad : m_run[i];
        alpha[i] = fexp2(m_run[i] - mn);  // 1 where the ceiling stays, 0 from the start value
        m_run[i] = mn;
      }
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int i = 0; i < RI; ++i) oacc[nt][i] *= alpha[i];
      if constexpr (kPackLo && G == 1) {
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) oacc[nt][1] *= alpha[0];  // row 1: lo parts of row 0
        if constexpr (PLO) zacc[1] *= alpha[0];
      }
#pragma unroll
      for (int i = 0; i < RI; ++i) zacc[i] *= alpha[i];
    }
#pragma unroll
    for (int i = 0; i < RI; ++i) {
      // every lane writes its rows; rows past the query group are never read
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const float p = fexp2(sacc[nt][i] - (m_run[i] - kLift));
        const _Float16 ph = static_cast<_Float16>(p);
        const uint32_t e = 2 * (32 * (4 * g4 + i) + 16 * nt + n16);
        dsw_h(pt_base + e, ph);
        if constexpr (PLO) dsw_h(plo_base + e, static_cast<_Float16>(p - static_cast<float>(ph)));
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    return p_operands();
  };

  // the same on a folded block (kFold): s[i] is the score of row frow + i
  // and token ftok.  The row reference m_run is a ceiling rather than the
  // running maximum: weights are 2^(s - m_run) <= 1 as long as no score
  // passes it, and only a block with such a score (the first one, and
  // rarely later) pays for the row maxima (a 16-lane row reduction joined
  // with the partner lane that holds the other tile's tokens) and the
  // rescale.  The new ceiling sits kPad above the block's maximum, so that
  // slowly rising maxima do not trigger it block after block.  The weights
  // are lifted by 2^kLift (the partial's maximum is lowered to match): with
  // the small value scales of 4- and 8-bit groups, p * s would otherwise fall
  // into the fp16 subnormals for tokens a few binades below the ceiling, and
  // the hi + lo pair would lose its precision.  The lift keeps p * s within
  // fp16 for any fp16 value range (s <= 131008 / (2^VB - 1)).
  auto softmax_fold = [&](f32x4 s, int count) __attribute__((always_inline)) -> POps {
    if (count < kBlockTokens) {  // wave-uniform: only a partial last block
      if (ftok >= count)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[i] = -INFINITY;
    }
    bool over = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) over |= s[i] > m_run[i];
    if (__builtin_amdgcn_ballot_w64(over)) {
      float alpha[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float bm = row16_max(s[i]);
        const float2 pr = kFold == 32 ? swap32(bm, bm) : swap16(bm, bm);
        const float mx = fmaxf(pr.x, pr.y);
        const float mn = mx > m_run[i] ? mx + kPad : m_run[i];
        alpha[i] = fexp2(m_run[i] - mn);  // 1 where the ceiling stays, 0 from the start value
        m_run[i] = mn;
      }
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[nt][i] *= alpha[i];
#pragma unroll
      for (int i = 0; i < 4; ++i) zacc[i] *= alpha[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // rows past the query group (fold by 16: rows 8-11) are never read
      const float p = fexp2(s[i] - (m_run[i] - kLift));
      const _Float16 ph = static_cast<_Float16>(p);
      const uint32_t e = 2 * (32 * (frow + i) + ftok);
      dsw_h(pt_base + e, ph);
      if constexpr (PLO) dsw_h(plo_base + e, static_cast<_Float16>(p - static_cast<float>(ph)));
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    return p_operands();
  };

  // one quantized block whose record sits in LDS at rec; refill() runs once
  // the block's last read of its record has completed (the slot is free)
  auto body_block = [&](const lds_u8* rec, int count, auto refill) __attribute__((always_inline)) {
    // inner-key instances (and the 4-bit GQA one, measured faster with it)
    // take the slot's base afresh for every block: hoisted out of the loop,
    // each slot's lane addresses held registers of their own, and the
    // spilled ones were reloaded inside the loop, whose wait on the reload
    // drained the ring
    uint32_t r0 = lds_off(rec);
    if constexpr (INNER || (KB == 4 && VB == 4 && G >= 4)) asm volatile("" : "+s"(r0));
    f32x4 sacc[2];
    f32x4 sf;  // folded block scores (kFold)
    // ---------------- keys: one batch of LDS reads
    uint32_t kw[2][KB];
    u32x4 kmeta[8];
    u32x2 imeta[2];
    u32x2 xlo[2];     // mixed groups: low nibbles of the token's 8-bit group
    uint32_t selw[2]; // mixed groups: group masks of tokens 16 nt + (n16 & 12) ..
    {
      if constexpr (INNER) {
        const uint32_t a = r0 + n16 * 64 + 8 * g4;
        const u32x2 x0 = dsr8<0>(a), x1 = dsr8<32>(a), y0 = dsr8<1024>(a), y1 = dsr8<1024 + 32>(a);
        // (s, z) pairs of token 16 nt + n16, or of the lane's one token ftok
        // when the block is folded
        const uint32_t am = r0 + R::off_km + 8 * (kFold ? ftok : n16);
        imeta[0] = dsr8<0>(am);
        if constexpr (!kFold) imeta[1] = dsr8<128>(am);
        if constexpr (MIX) {
          const uint32_t ax = r0 + R::off_kx + n16 * 32 + 8 * g4;
          const uint32_t as = r0 + R::off_ks + (n16 & 12);
          xlo[0] = dsr8<0>(ax);
          xlo[1] = dsr8<512>(ax);
          selw[0] = dsr4<0>(as);
          selw[1] = dsr4<16>(as);
        }
        kw[0][0] = x0[0]; kw[0][1] = x0[1]; kw[0][2] = x1[0]; kw[0][3] = x1[1];
        kw[1][0] = y0[0]; kw[1][1] = y0[1]; kw[1][2] = y1[0]; kw[1][3] = y1[1];
      } else {
        constexpr int RB = 16 * KB;  // key row bytes
        const uint32_t a = r0 + koff0;
        if constexpr (KB == 4) {
          const u32x4 x = dsr16<0>(a), y = dsr16<16 * RB>(a);
#pragma unroll
          for (int e = 0; e < 4; ++e) { kw[0][e] = x[e]; kw[1][e] = y[e]; }
        } else if constexpr (KB == 2) {
          const u32x2 x = dsr8<0>(a), y = dsr8<16 * RB>(a);
#pragma unroll
          for (int e = 0; e < 2; ++e) { kw[0][e] = x[e]; kw[1][e] = y[e]; }
        } else {
          const uint32_t a1 = r0 + koff1;
          const u32x4 x0 = dsr16<0>(a), x1 = dsr16<0>(a1), y0 = dsr16<16 * RB>(a), y1 = dsr16<16 * RB>(a1);
#pragma unroll
          for (int e = 0; e < 4; ++e) { kw[0][e] = x0[e]; kw[0][4 + e] = x1[e]; kw[1][e] = y0[e]; kw[1][4 + e] = y1[e]; }
        }
        // C-term operand (z for columns 0-7, s for 8-15) and the scale chunk
        const uint32_t ac = r0 + R::off_km + (n16 < 8 ? 2 * D : 0) + 64 * g4;
        const uint32_t as = r0 + R::off_km + 64 * g4;
        kmeta[0] = dsr16<0>(ac); kmeta[1] = dsr16<16>(ac); kmeta[2] = dsr16<32>(ac); kmeta[3] = dsr16<48>(ac);
        kmeta[4] = dsr16<0>(as); kmeta[5] = dsr16<16>(as); kmeta[6] = dsr16<32>(as); kmeta[7] = dsr16<48>(as);
      }
      lds_wait();
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int e = 0; e < KB; ++e) pin(kw[nt][e]);
      if constexpr (INNER) {
        pin(imeta[0]);
        if constexpr (!kFold) pin(imeta[1]);
        if constexpr (MIX) {
          pin(xlo[0]);
          pin(xlo[1]);
          pin(selw[0]);
          pin(selw[1]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) pin(kmeta[e]);
      }
    }
    if constexpr (!INNER) {
      // A = q * s per channel as a pair hi + lo of fp16 exact to ~2^-22
      // (lo = fma(q, s, -hi) rounds only the residual).  One MFMA chain
      // against the block's parameters broadcast over the tile's columns
      // gives, per query row, C_z = sum_c q_c z_c (columns 0-7) and
      // C_s = sum_c q_c s_c (columns 8-15); the score of token t is
      //   (sum_c A_c B_ct - base * C_s) * inv_unit + C_z.
      constexpr float base = CodeEnc<KB>::base, iu = CodeEnc<KB>::inv_unit;
      f32x4 cacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) cacc = mfma(qa[j], h8(kmeta[j]), cacc);
      // rows past the lane's query rows start from 0 (with packed keys, rows
      // G..2G-1 accumulate the lo parts only)
      f32x4 init = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < RI; ++i) {
        const float other = dppf<kRowRor8>(cacc[i]);
        const float cz = n16 < 8 ? cacc[i] : other;
        const float cs = n16 < 8 ? other : cacc[i];
        init[i] = (kPackK && 4 * g4 + i >= G) ? 0.f : fmaf(cz, 1.f / iu, -base * cs);
      }
      sacc[0] = init;
      sacc[1] = init;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const half8 s8 = h8(kmeta[4 + j]);
        if constexpr (kPackK) {
          half8 w = qa[j] * s8;
          if (n16 >= G) lo_in_place(w, qa[j], s8);  // rows G..2G-1: the lo parts
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) sacc[nt] = mfma(w, kstep<KB>(unp, kw[nt], j), sacc[nt]);
        } else {
          const half8 qh = qa[j] * s8;
          const half8 ql = __builtin_elementwise_fma(qa[j], s8, -qh);
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            const half8 bk = kstep<KB>(unp, kw[nt], j);
            sacc[nt] = mfma(qh, bk, sacc[nt]);
            sacc[nt] = mfma(ql, bk, sacc[nt]);
          }
        }
      }
      if constexpr (kPackK && G == 1) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) sacc[nt][0] += sacc[nt][1];
      }
      if constexpr (kFold && kPackK) {
        // the swap that folds tile 1's live lanes into tile 0's empty ones
        // also brings each tile's lo rows next to its hi rows
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float2 r = kFold == 32 ? swap32(sacc[0][i], sacc[1][i]) : swap16(sacc[0][i], sacc[1][i]);
          sf[i] = (r.x + r.y) * (iu * kscale);
        }
      } else if constexpr (kFold) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sf[i] = fold(sacc[0][i], sacc[1][i]) * (iu * kscale);
      } else {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) sacc[nt][i] *= iu * kscale;
      }
    } else {
      // per-token groups of 64 channels: group sums sum_c q_c B_ct, offset
      // removed with the group sums of q, then scaled per token
      // (mixed layers: the token's 8-bit group, marked in its mask, reads
      // 1 + c/256 operands, so its sums take 256 s and the symmetric offset 128)
      constexpr float base = CodeEnc<KB>::base, iu = CodeEnc<KB>::inv_unit;
      // score of group g: sg (code sum) + zg qsum_g, times kscale, with the
      // per-token factors formed once per lane; mixed layers remove the
      // offset here: sg (p_g - qsum_g) + zg qsum_g = sg p_g + (zg - sg) qsum_g
      auto factors = [&](u32x2 mm, uint32_t sel, float (&sk)[2], float (&zk)[2]) __attribute__((always_inline)) {
        if constexpr (!MIX) {
          // a symmetric group stores its zero point as +0 and its flag as the
          // scale's sign: zg = z - 2^(KB-1) |s| = z + 2^(KB-1) min(s, 0) for
          // both kinds (products by powers of two are exact, so the factors
          // equal sv iu kscale and zg kscale as written out below)
#pragma unroll
          for (int gg = 0; gg < 2; ++gg) {
            const float sv = h2f(static_cast<uint16_t>(mm[gg] & 0xffff));
            const float zv = h2f(static_cast<uint16_t>(mm[gg] >> 16));
            sk[gg] = fabsf(sv) * (iu * kscale);
            zk[gg] = fmaf(fminf(sv, 0.f), static_cast<float>(1 << (KB - 1)) * kscale, zv * kscale);
          }
          return;
        }
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
          const uint16_t s16 = static_cast<uint16_t>(mm[gg] & 0xffff);
          const uint16_t z16 = static_cast<uint16_t>(mm[gg] >> 16);
          const float sv = h2f(s16 & 0x7fff);
          const bool sym = (s16 & 0x8000) != 0;
          const bool wide = MIX && ((sel >> gg) & 1u) != 0;
          const float sg = sv * (wide ? 256.f : iu);
          const float zg = sym ? -(wide ? 128.f : static_cast<float>(1 << (KB - 1))) * sv : h2f(z16);
          sk[gg] = sg * kscale;
          zk[gg] = (MIX ? fmaf(-base, sg, zg) : zg) * kscale;
        }
      };
      f32x4 pg[2][2];  // folded blocks: group sums [tile][group] before the fold
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        uint32_t sel = 0, lo[4] = {0u, 0u, 0u, 0u};
        if constexpr (MIX) {
          sel = (selw[nt] >> (8 * (n16 & 3))) & 3u;
          lo[0] = (sel & 1u) ? xlo[nt][0] : 0u;
          lo[1] = (sel & 1u) ? xlo[nt][1] : 0u;
          lo[2] = (sel & 2u) ? xlo[nt][0] : 0u;
          lo[3] = (sel & 2u) ? xlo[nt][1] : 0u;
        }
        auto bk = [&](int j) __attribute__((always_inline)) {
          if constexpr (MIX) return ex4lo(unp, kw[nt][j], lo[j]);
          else return ex4w(unp, kw[nt][j]);
        };
        // group sums of q_c B_ct; 4-bit groups start from minus the weighted
        // sums of q, so they come out as sum_c q_c c_ct / 16 directly
        f32x4 p0 = MIX ? f32x4{0.f, 0.f, 0.f, 0.f} : qinit[0];
        f32x4 p1 = MIX ? f32x4{0.f, 0.f, 0.f, 0.f} : qinit[1];
        p0 = mfma(qa[0], bk(0), p0);
        p0 = mfma(qa[1], bk(1), p0);
        p1 = mfma(qa[2], bk(2), p1);
        p1 = mfma(qa[3], bk(3), p1);
        if constexpr (kFold) {
          pg[nt][0] = p0;
          pg[nt][1] = p1;
        } else {
          float sk[2], zk[2];
          factors(imeta[nt], sel, sk, zk);  // (s0, z0), (s1, z1) of token 16 nt + n16
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sacc[nt][i] = i < RI ? fmaf(sk[0], p0[i], fmaf(sk[1], p1[i], fmaf(zk[0], qsum[0][i], zk[1] * qsum[1][i])))
                                 : 0.f;
        }
      }
      if constexpr (kFold) {
        // the group sums of both tiles in one register set, then the factors
        // of the lane's one token
        uint32_t sel = 0;
        if constexpr (MIX) sel = ((ftile ? selw[1] : selw[0]) >> (8 * (n16 & 3))) & 3u;
        float sk[2], zk[2];
        factors(imeta[0], sel, sk, zk);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float g0 = fold(pg[0][0][i], pg[1][0][i]);
          const float g1 = fold(pg[0][1][i], pg[1][1][i]);
          sf[i] = fmaf(sk[0], g0, fmaf(sk[1], g1, fmaf(zk[0], qsum[0][i], zk[1] * qsum[1][i])));
        }
      }
    }
    // ---------------- values: one batch of LDS reads (issued before the softmax)
    uint32_t vw[2 * VB];
    u32x4 vmeta[5];
    {
      const uint32_t av = r0 + R::off_vc + l * (8 * VB);
      u32x4 c[(2 * VB) / 4];
      c[0] = dsr16<0>(av);
      if constexpr (VB >= 4) c[1] = dsr16<16>(av);
      if constexpr (VB == 8) { c[2] = dsr16<32>(av); c[3] = dsr16<48>(av); }
      const uint32_t az = r0 + R::off_vm + (n16 < 4 ? 2 * ngv * kBlockTokens : 0) + 2 * ((n16 & 3) * kBlockTokens + 8 * g4);
      const uint32_t asv = r0 + R::off_vm + 16 * g4;
      vmeta[4] = dsr16<0>(az);
      vmeta[0] = dsr16<0>(asv); vmeta[1] = dsr16<64>(asv); vmeta[2] = dsr16<128>(asv); vmeta[3] = dsr16<192>(asv);
      lds_wait();
#pragma unroll
      for (int q4 = 0; q4 < (2 * VB) / 4; ++q4) {
        pin(c[q4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) vw[4 * q4 + e] = c[q4][e];
      }
#pragma unroll
      for (int e = 0; e < 5; ++e) pin(vmeta[e]);
    }
    refill();
    const POps P = kFold ? softmax_fold(sf, count) : softmax_tile(sacc, count);
    const half8 pa = P.pa;
    // one MFMA of P against the block's value parameters: column g < 4 holds
    // z_g (zero points), column 4 + g holds s_g (removes the code offset),
    // column 8 ones (the denominator); with PLO rows G..2G-1 add the
    // residuals' share
    zacc = mfma(P.pz, n16 < 2 * ngv ? h8(vmeta[4]) : (n16 == 8 ? h8(kOnes, kOnes, kOnes, kOnes) : h8(0u, 0u, 0u, 0u)),
                zacc);
    // weights w = p * s per (token, value group) as an exact hi + lo pair
#pragma unroll
    for (int g = 0; g < ngv; ++g) {
      const half8 s8 = h8(vmeta[g]);
      if constexpr (kPackLo) {
        // lanes of rows G.. replace their hi part by the lo part (exec-masked),
        // plus the weight residual's product with PLO
        half8 w = pa * s8;
        if (n16 >= G) {
          if constexpr (PLO) lo_plus_in_place(w, pa, s8, P.pz);
          else lo_in_place(w, pa, s8);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int nt = 2 * g + t;
          oacc[nt] = mfma(w, vtile<VB>(unp, vw, nt), oacc[nt]);
        }
      } else {
        const half8 wh = pa * s8;
        const half8 wl = __builtin_elementwise_fma(pa, s8, -wh);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int nt = 2 * g + t;
          const half8 bv = vtile<VB>(unp, vw, nt);
          oacc[nt] = mfma(wh, bv, oacc[nt]);
          oacc[nt] = mfma(wl, bv, oacc[nt]);
        }
      }
    }
  };

  constexpr float vbase = CodeEnc<VB>::base, viu = CodeEnc<VB>::inv_unit;
  const int nblk_body = (st.nb + kBlockTokens - 1) / kBlockTokens;
  const int c_begin = sp * J.blocks_per_split;
  const int c_end = sp < J.nsplit_body ? min(nblk_body, c_begin + J.blocks_per_split) : c_begin;
  const int nmy = c_end - c_begin;
  const uint8_t* ubase = L.body + static_cast<int64_t>(u) * L.nblk_cap * L.rec_bytes;
  auto issue = [&](int i, lds_u8* dst) __attribute__((always_inline)) {
    const uint8_t* src = ubase + static_cast<int64_t>(c_begin + i) * L.rec_bytes;
#pragma unroll
    for (int k = 0; k < R::loads; ++k) {
      const int off = k * 1024 + l * 16;
      if (off < R::bytes) ring_load(src + off, dst + k * 1024);
    }
  };
#pragma unroll
  for (int k = 0; k < NBUF; ++k)
    if (k < nmy) issue(k, slot_at(k));

  // ---------------- sink / window tokens: fp16 operands as stored, one
  // 32-slot chunk at a time (slots without a live token are masked).  They
  // are accumulated at 1/inv_unit scale so that the body's final code-unit
  // rescale (a power of two, exact) restores them.
  {
    const int slots = L.sinks_cap + L.win_cap;
    uint16_t* const kf = L.fp16 + static_cast<int64_t>(u) * 2 * slots * D;
    uint16_t* const vf = kf + static_cast<int64_t>(slots) * D;
    const int wchunks = L.win_cap / kBlockTokens;
    const int wstart = st.nb % L.win_cap;  // ring index of the oldest window token
    for (int c = sp - J.fp16_split0; c >= 0 && c < J.fp16_chunks; c += J.fp16_nsplit) {
      const bool sinkc = c < J.sink_chunks;
      const int slot0 = sinkc ? kBlockTokens * c
                              : L.sinks_cap + kBlockTokens * ((J.win_chunk0 + c - J.sink_chunks) % wchunks);
      u32x4 kv[2][4], vv[8];
      // an appended token carried by this launch is read from its source
      // (its slot is written below, and read by no other split)
      const int xs = J.new_slot - slot0;  // in [0, 32) for the chunk holding it
      const uint16_t* const nk = J.new_k + static_cast<int64_t>(u) * D;
      // rotated values (PLO instances serve exactly those layers; the host
      // fuses the append for per-channel keys only): the token's channels 2l
      // and 2l + 1 as the window keeps them, c H v, taken before the chunk's
      // operands are in registers
      constexpr bool kRotNew = PLO && !INNER;
      uint32_t vrot = 0;
      if constexpr (kRotNew) {
        if (xs >= 0 && xs < kBlockTokens)  // wave-uniform
          vrot = hadamard_pair_rows(*reinterpret_cast<const uint32_t*>(J.new_v + static_cast<int64_t>(u) * D + 2 * l),
                                    L.had_scale, l);
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          kv[nt][j] = ld16((16 * nt + n16 == xs ? nk : kf + (slot0 + 16 * nt + n16) * D) + kchan<INNER>(g4, j, 0));
      // lane: slots slot0 + 8*g4 .. +7 of channel 16*nt + n16 (16 contiguous bytes)
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) vv[nt] = ld16(vf + (static_cast<int64_t>(slot0 / 8 + g4) * D + 16 * nt + n16) * 8);
      if (xs >= 0 && xs < kBlockTokens) {  // wave-uniform
        const uint16_t* const nv = J.new_v + static_cast<int64_t>(u) * D;
        const int e = xs - 8 * g4;  // element of the lane's eight slots
        uint32_t vw;
        if constexpr (kRotNew) {
          vw = vrot;
          // channel 16 nt + n16 sits in lane 8 nt + n16 / 2 (every lane takes part)
          uint32_t pw[8];
#pragma unroll
          for (int nt = 0; nt < 8; ++nt)
            pw[nt] = static_cast<uint32_t>(
                __builtin_amdgcn_ds_bpermute((8 * nt + (n16 >> 1)) << 2, static_cast<int>(vw)));
          if (e >= 0 && e < 8) {
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) {
              const uint32_t x = (n16 & 1) ? pw[nt] >> 16 : pw[nt] & 0xffffu;
#pragma unroll
              for (int w = 0; w < 4; ++w) {
                if (e == 2 * w) vv[nt][w] = (vv[nt][w] & 0xffff0000u) | x;
                if (e == 2 * w + 1) vv[nt][w] = (vv[nt][w] & 0x0000ffffu) | (x << 16);
              }
            }
          }
        } else {
          vw = *reinterpret_cast<const uint32_t*>(nv + 2 * l);
          if (e >= 0 && e < 8) {
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) {
              const uint32_t x = nv[16 * nt + n16];
#pragma unroll
              for (int w = 0; w < 4; ++w) {
                if (e == 2 * w) vv[nt][w] = (vv[nt][w] & 0xffff0000u) | x;
                if (e == 2 * w + 1) vv[nt][w] = (vv[nt][w] & 0x0000ffffu) | (x << 16);
              }
            }
          }
        }
        // store the token: lane l takes channels 2l and 2l + 1
        const int x = slot0 + xs;
        const uint32_t kw = *reinterpret_cast<const uint32_t*>(nk + 2 * l);
        *reinterpret_cast<uint32_t*>(kf + static_cast<int64_t>(x) * D + 2 * l) = kw;
        vf[vslot(x, 2 * l)] = static_cast<uint16_t>(vw);
        vf[vslot(x, 2 * l + 1)] = static_cast<uint16_t>(vw >> 16);
      }
      f32x4 sacc[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int x = slot0 + 16 * nt + n16;
        bool live;
        if (sinkc) {
          live = x < st.s_eff;
        } else {
          int d = x - L.sinks_cap - wstart;
          if (d < 0) d += L.win_cap;
          live = d < st.r;
        }
        sacc[nt] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) sacc[nt] = mfma(qa[j], h8(kv[nt][j]), sacc[nt]);
#pragma unroll
        for (int i = 0; i < 4; ++i) sacc[nt][i] = live ? sacc[nt][i] * kscale : -INFINITY;
      }
      f32x4 sf;
      if constexpr (kFold)
#pragma unroll
        for (int i = 0; i < 4; ++i) sf[i] = fold(sacc[0][i], sacc[1][i]);
      const POps P = kFold ? softmax_fold(sf, kBlockTokens) : softmax_tile(sacc, kBlockTokens);
      // fp16 values take no lo part of a product: rows G..2G-1 carry the
      // weights' residuals with PLO, nothing otherwise
      half8 pa = P.pa;
      if constexpr (PLO) pa = P.pz;
      else if constexpr (kPackLo) pa = n16 < G ? pa : h8(0u, 0u, 0u, 0u);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) oacc[nt] = mfma(pa, h8(vv[nt]), oacc[nt]);
      zacc = mfma(pa, n16 == 8 ? h8(kOnes, kOnes, kOnes, kOnes) : h8(0u, 0u, 0u, 0u), zacc);
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[nt][i] *= 1.0f / viu;
  }

  if constexpr (INNER) {
    // body keys normalized per channel at prefill (InnerQ, method 4): the
    // query takes the inverse powers of two, q'_c = q_c 2^-shift_c (exact
    // unless q'_c falls below the fp16 normal range)
    if (L.kshift) {
      const int8_t* shp = L.kshift + static_cast<int64_t>(u) * D;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x2 w = ld8(shp + kchan<INNER>(g4, j, 0));
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const int sh = static_cast<int8_t>((w[kk >> 2] >> (8 * (kk & 3))) & 0xffu);
          qa[j][kk] = static_cast<_Float16>(ldexpf(static_cast<float>(qa[j][kk]), -sh));
        }
      }
    }
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
      float s = 0.f, sw = 0.f;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const float v = static_cast<float>(qa[2 * gg + jj][kk]);
          s += v;
          sw = fmaf(v, kk < 2 ? 64.f : 4.f, sw);  // constant parts of the ex4w operands
        }
      s += xshflf<16>(s);
      s += __int_as_float(__builtin_amdgcn_ds_bpermute((l ^ 32) << 2, __float_as_int(s)));
      sw += xshflf<16>(sw);
      sw += __int_as_float(__builtin_amdgcn_ds_bpermute((l ^ 32) << 2, __float_as_int(sw)));
      qinit[gg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < RI; ++i) {
        qsum[gg][i] = lane_bcast(s, kFold ? frow + i : 20 * g4 + i);  // lane n16 = row holds its sum
        qinit[gg][i] = -lane_bcast(sw, 20 * g4 + i);
      }
    }
  }

  // ---------------- quantized body blocks through the LDS ring
  {
    // block i sits in slot i % NBUF.  Steady state: a step waits until only
    // the (NBUF - 1) newer blocks are in flight, and as soon as the block has
    // read its record out of LDS (half-way through its work, before the
    // softmax and the value products) the slot takes block i + NBUF, so
    // NBUF - 1 to NBUF blocks stay in flight behind the compute.  The waits
    // are the same on every path.  The tail drains.
    // Wavefronts sharing a SIMD are picked oldest first, so without help the
    // last one dispatched finishes long after the others.  Each wavefront
    // lowers its priority as it gets through its blocks: one that is ahead
    // yields to those behind and the SIMD's wavefronts finish together.
    int prio_q = 0;
    auto age = [&](int i) __attribute__((always_inline)) {
      const int q = (4 * i) / nmy;
      if (q != prio_q) {
        prio_q = q;
        if (q == 1) __builtin_amdgcn_s_setprio(2);
        else if (q == 2) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
      }
    };
    __builtin_amdgcn_s_setprio(3);
    auto step = [&](int i, lds_u8* cur) __attribute__((always_inline)) {
      age(i);
      wait_vm<(NBUF - 1) * R::loads>();
      const int ch = c_begin + i;
      body_block(cur, min(kBlockTokens, st.nb - ch * kBlockTokens),
                 [&]() __attribute__((always_inline)) { issue(i + NBUF, cur); });
    };
    int i = 0;
    // every step of an iteration refills its slot: blocks up to i + 2 NBUF - 1
    for (; i + 2 * NBUF - 1 < nmy; i += NBUF) {
      if constexpr (NBUF == 4) {
        step(i, slot0);
        step(i + 1, slot1);
        step(i + 2, slot2);
        step(i + 3, slot3);
      } else if constexpr (NBUF == 3) {
        step(i, slot0);
        step(i + 1, slot1);
        step(i + 2, slot2);
      } else {
        step(i, slot0);
        step(i + 1, slot1);
      }
    }
    for (; i < nmy; ++i) {
      age(i);
      // remaining blocks (every one up to i + NBUF - 1 is issued): wait for
      // block i only, the blocks issued after it stay in flight
      const int newer = min(NBUF - 1, nmy - 1 - i);
      if (NBUF >= 4 && newer >= 3)
        wait_vm<(NBUF >= 4 ? 3 : 0) * R::loads>();
      else if (NBUF >= 3 && newer >= 2)
        wait_vm<(NBUF >= 3 ? 2 : 0) * R::loads>();
      else if (newer >= 1)
        wait_vm<R::loads>();
      else
        wait_vm<0>();
      const int s_cur = i % NBUF;
      const int ch = c_begin + i;
      body_block(slot_at(s_cur), min(kBlockTokens, st.nb - ch * kBlockTokens), [&]() __attribute__((always_inline)) {
        if (i + NBUF < nmy) issue(i + NBUF, slot_at(s_cur));
      });
    }
  }

  __builtin_amdgcn_s_setprio(0);
  // ---------------- partial of this split: o = (O_raw - base * W_g) * inv_unit + Z_g,
  // merged by decode_merge_kernel (launched next on the same stream)
  if constexpr (kPackLo) {
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (G == 8) oacc[nt][i] += swap32(oacc[nt][i], oacc[nt][i]).y;
        else if constexpr (G == 4) oacc[nt][i] += swap16(oacc[nt][i], oacc[nt][i]).y;
        else if (i == 0) oacc[nt][0] += oacc[nt][1];
      }
  }
  if constexpr (PLO) {  // the residuals' sums (rows G..2G-1) onto rows 0..G-1
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (G == 8) zacc[i] += swap32(zacc[i], zacc[i]).y;
      else if constexpr (G == 4) zacc[i] += swap16(zacc[i], zacc[i]).y;
      else if (i == 0) zacc[0] += zacc[1];
    }
  }
  float* opart = J.partials + (static_cast<int64_t>(u) * nsplit + sp) * G * D;
  float* mlpart = J.partials + J.ml_off + (static_cast<int64_t>(u) * nsplit + sp) * G * 2;
#pragma unroll
  for (int i = 0; i < RI; ++i) {
    const float lsum = lane_bcast(zacc[i], (l & 48) | 8);
    const int row = 4 * g4 + i;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const float z = lane_bcast(zacc[i], (l & 48) | (nt >> 1));
      const float w = lane_bcast(zacc[i], (l & 48) | (4 + (nt >> 1)));
      const float o = fmaf(fmaf(-vbase, w, oacc[nt][i]), viu, z);
      if (rows_here && row < G) opart[row * D + 16 * nt + n16] = o;
    }
    if (rows_here && row < G && n16 == 0) {
      // the weights' reference is the ceiling minus the lift; a split that
      // saw no live token reports -inf
      mlpart[row * 2] = m_run[i] == kNoScore ? -INFINITY : m_run[i] - kLift;
      mlpart[row * 2 + 1] = lsum;
    }
  }
}

// groups of 32 threads in a merge workgroup (16: the 96 split partials of a 32K-token MHA
// unit are all requested in one batch per group)
constexpr int kMergeGroups = 16;

// Log-sum-exp merge of the split partials of one unit (all its query rows).
// NG groups of 32 threads; thread (group, q) owns channels 4q..4q+3.
// With G rows, NG/G groups share a row (G <= NG) and take its splits in turn;
// each group pulls every (max, sum) pair of its row from LDS, so the row
// maximum needs no extra pass, and requests its partial vectors eight at a
// time.  The groups of a row meet in LDS; values stored Hadamard-rotated are
// rotated back there (c * H * o, H Sylvester).
template <int NG>
__global__ void __launch_bounds__(32 * NG) decode_merge_kernel(LayerDesc L, DecodeJob J) {
  // the split plan keeps nsplit (body and fp16 splits) <= kMaxBodySplits = 256
  constexpr int kMaxSplits = 256;
  static_assert(kMaxBodySplits <= kMaxSplits && kMaxFp16Splits <= kMaxSplits, "split bound");
  constexpr int kMaxRows = kMaxGroupRows;
  __shared__ float ms[kMaxSplits * kMaxRows], ls[kMaxSplits * kMaxRows];
  __shared__ float red[NG][D];
  const int tid = threadIdx.x, grp = tid >> 5, cq = tid & 31;
  const int u = blockIdx.x;
  const int G = L.G, nsplit = J.nsplit;
  const int b = u / L.Hkv, h = u % L.Hkv;
  const float* obase = J.partials + static_cast<int64_t>(u) * nsplit * G * D;
  const float* mlbase = J.partials + J.ml_off + static_cast<int64_t>(u) * nsplit * G * 2;
  for (int i = tid; i < nsplit * G; i += 32 * NG) {
    ms[i] = mlbase[2 * i];
    ls[i] = mlbase[2 * i + 1];
  }
  __syncthreads();
  const int lpr = G >= NG ? 1 : NG / G;    // groups per row
  const int so = grp % lpr;                // this group's first split
  for (int r = grp / lpr; r < G; r += NG / lpr) {
    // row maximum and sum over all splits (32 lanes, then the group)
    float M = -INFINITY;
    for (int i = cq; i < nsplit; i += 32) M = fmaxf(M, ms[i * G + r]);
    M = fmaxf(M, xshflf<1>(M));
    M = fmaxf(M, xshflf<2>(M));
    M = fmaxf(M, xshflf<4>(M));
    M = fmaxf(M, xshflf<8>(M));
    M = fmaxf(M, xshflf<16>(M));
    float Ls = 0.f;
    bool bad = false;
    for (int i = cq; i < nsplit; i += 32) {
      const float mi = ms[i * G + r];
      bad |= bad_partial(mi, ls[i * G + r]);
      Ls = fmaf(ls[i * G + r], mi == -INFINITY ? 0.f : exp2f(mi - M), Ls);
    }
    {
      const uint64_t m = __ballot(bad);
      bad = ((tid & 32) ? static_cast<uint32_t>(m >> 32) : static_cast<uint32_t>(m)) != 0u;
    }
    Ls += xshflf<1>(Ls);
    Ls += xshflf<2>(Ls);
    Ls += xshflf<4>(Ls);
    Ls += xshflf<8>(Ls);
    Ls += xshflf<16>(Ls);
    // weighted sum of this group's splits so, so + lpr, ...
    constexpr int kBatch = 8;
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    for (int i0 = so; i0 < nsplit; i0 += kBatch * lpr) {
      f32x4 v[kBatch];
      float wt[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const int i = i0 + k * lpr;
        v[k] = i < nsplit ? *reinterpret_cast<const f32x4*>(obase + (static_cast<int64_t>(i) * G + r) * D + 4 * cq)
                          : f32x4{0.f, 0.f, 0.f, 0.f};
        const float mi = i < nsplit ? ms[i * G + r] : -INFINITY;
        wt[k] = mi == -INFINITY ? 0.f : exp2f(mi - M);
      }
#pragma unroll
      for (int k = 0; k < kBatch; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = fmaf(v[k][e], wt[k], a[e]);
    }
    if (lpr > 1) {
#pragma unroll
      for (int e = 0; e < 4; ++e) red[grp][4 * cq + e] = a[e];
    }
    __syncthreads();
    if (so == 0) {
      if (lpr > 1) {
        for (int k = 1; k < lpr; ++k)
#pragma unroll
          for (int e = 0; e < 4; ++e) a[e] += red[grp + k][4 * cq + e];
      }
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = a[e] / Ls;
      if (L.v_had) {
        // channels 4q + e: butterflies over e in-lane, over q across the group
        float t0 = y[0] + y[1], t1 = y[0] - y[1], t2 = y[2] + y[3], t3 = y[2] - y[3];
        y[0] = t0 + t2;
        y[1] = t1 + t3;
        y[2] = t0 - t2;
        y[3] = t1 - t3;
        const int lane = tid & 63;
#pragma unroll
        for (int hb = 1; hb < 32; hb <<= 1) {
          const bool hi = (cq & hb) != 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float o = __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ hb) << 2, __float_as_int(y[e])));
            y[e] = hi ? o - y[e] : y[e] + o;
          }
        }
        const float c = static_cast<float>(L.had_scale);
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] *= c;
      }
      if (bad) {
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = __uint_as_float(0x7fc00000u);
      }
      float* op = J.out + (static_cast<int64_t>(b) * L.Hq + h * G + r) * D + 4 * cq;
      *reinterpret_cast<f32x4*>(op) = f32x4{y[0], y[1], y[2], y[3]};
      const bool nf = nonfinite_bits(y[0]) || nonfinite_bits(y[1]) || nonfinite_bits(y[2]) ||
                      nonfinite_bits(y[3]);
      const uint64_t m = __ballot(nf);
      const uint32_t mine = (tid & 32) ? static_cast<uint32_t>(m >> 32) : static_cast<uint32_t>(m);
      if (cq == 0 && mine != 0u) atomicAdd(J.nonfinite, 1u);
    }
    __syncthreads();
  }
}

template <int KB, int VB, int G, bool INNER, bool MIX, bool PLO>
hipError_t launch_t(const LayerDesc& L, const DecodeJob& j, hipStream_t s, int* waves) {
  using R = Rec<KB, VB, INNER, MIX>;
  if (L.off_km != R::off_km || L.off_vc != R::off_vc || L.off_vm != R::off_vm) return hipSuccess;
  if (MIX && (L.off_kx != R::off_kx || L.off_ks != R::off_ks)) return hipSuccess;
  constexpr int NB = ring_slots<KB, VB, G, INNER, MIX>();
  auto kern = decode_mfma_kernel<KB, VB, G, INNER, MIX, NB, PLO>;
  // one full round of resident wavefronts, from the runtime's occupancy of
  // this instance (registers and LDS as compiled) and the device's CU count
  static std::atomic<int> resident[kMaxDevices];
  if (resident_waves(kern, resident, waves) != hipSuccess) return hipErrorInvalidValue;
  if (!j.q) return hipSuccess;  // query only
  hipLaunchKernelGGL(kern, dim3(j.nsplit, L.units), dim3(64), 0, s, L, j);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  return launch_decode_merge(L, j, s);
}

// Hadamard-rotated 2-bit values (the Hadamard 2-bit page's scheme) carry the
// attention weights as a hi + lo pair (PLO): their near-uniform attention
// over rotated values is where fp16-rounded weights cost the most accuracy.
template <int G, bool INNER, bool MIX>
hipError_t by_bits(const LayerDesc& L, const DecodeJob& j, hipStream_t s, int* waves) {
  const int k = L.kb, v = L.vb;
  const bool plo = L.v_had != 0;
#define KVQ_CASE(KB, VB)                                                                   \
  if (k == KB && v == VB) {                                                                \
    if constexpr (VB == 2)                                                                 \
      if (plo) return launch_t<KB, VB, G, INNER, MIX, true>(L, j, s, waves);               \
    return launch_t<KB, VB, G, INNER, MIX, false>(L, j, s, waves);                         \
  }
  if constexpr (MIX) {
    KVQ_CASE(4, 2) KVQ_CASE(4, 4)
  } else if constexpr (INNER) {
    KVQ_CASE(4, 2) KVQ_CASE(4, 4)
  } else {
    KVQ_CASE(2, 2) KVQ_CASE(2, 4) KVQ_CASE(2, 8)
    KVQ_CASE(4, 2) KVQ_CASE(4, 4) KVQ_CASE(4, 8)
    KVQ_CASE(8, 2) KVQ_CASE(8, 4) KVQ_CASE(8, 8)
  }
#undef KVQ_CASE
  return hipSuccess;
}

hipError_t dispatch(const LayerDesc& L, const DecodeJob& j, hipStream_t s, int* waves) {
  *waves = 0;
  if (L.nuq || L.outk || L.pre_rope || (L.k_hybrid && !L.k_inner)) return hipSuccess;
  if (L.k_inner && L.k_group != 64) return hipSuccess;
  if (L.k_hi && (L.k_hi != 1 || L.kb != 4)) return hipSuccess;  // one 8-bit group of two
  if (L.v_group != 32) return hipSuccess;
  auto pick = [&](auto g) {
    constexpr int GG = decltype(g)::value;
    if (L.k_hi) return by_bits<GG, true, true>(L, j, s, waves);
    return L.k_inner ? by_bits<GG, true, false>(L, j, s, waves) : by_bits<GG, false, false>(L, j, s, waves);
  };
  switch (L.G) {
    case 1: return pick(std::integral_constant<int, 1>{});
    case 4: return pick(std::integral_constant<int, 4>{});
    case 8: return pick(std::integral_constant<int, 8>{});
    default: return hipSuccess;
  }
}

}  // namespace

namespace {

// Log-sum-exp merge for units with few splits (batched GQA layers): one
// wavefront per (unit, query row).  Every split's (max, sum) and the lane's
// two channels 2 lane, 2 lane + 1 of every split's partial are requested at
// once (split indices past nsplit reread split 0 and are not used), so the
// merge takes one round trip to memory; the Hadamard rotation is undone
// in-lane (channel bit 0) and across lanes (bits 1-6).
template <int MAXS>
__global__ void __launch_bounds__(256) decode_merge_rows_kernel(LayerDesc L, DecodeJob J) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x) * 4 + (static_cast<int>(threadIdx.x) >> 6));
  const int G = L.G, nsplit = J.nsplit;
  if (w >= L.units * G) return;
  const int u = w / G, r = w - u * G;
  const float* ob = J.partials + (static_cast<int64_t>(u) * nsplit * G + r) * D + 2 * lane;
  const float* mb = J.partials + J.ml_off + (static_cast<int64_t>(u) * nsplit * G + r) * 2;
  float2 ml[MAXS], oi[MAXS];
#pragma unroll
  for (int i = 0; i < MAXS; ++i) {
    const int ii = i < nsplit ? i : 0;
    ml[i] = *reinterpret_cast<const float2*>(mb + static_cast<int64_t>(ii) * G * 2);
    oi[i] = *reinterpret_cast<const float2*>(ob + static_cast<int64_t>(ii) * G * D);
  }
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < MAXS; ++i)
    if (i < nsplit) M = fmaxf(M, ml[i].x);
  float Ls = 0.f, a0 = 0.f, a1 = 0.f;
  bool bad = false;
#pragma unroll
  for (int i = 0; i < MAXS; ++i) {
    if (i < nsplit) bad |= bad_partial(ml[i].x, ml[i].y);
    const float wt = (i >= nsplit || ml[i].x == -INFINITY) ? 0.f : exp2f(ml[i].x - M);
    Ls = fmaf(ml[i].y, wt, Ls);
    a0 = fmaf(oi[i].x, wt, a0);
    a1 = fmaf(oi[i].y, wt, a1);
  }
  float y0 = a0 / Ls, y1 = a1 / Ls;
  if (bad) y0 = y1 = __uint_as_float(0x7fc00000u);
  if (L.v_had) {
    // o <- c H o, H Sylvester: butterflies over channel bit 0 in-lane, then
    // over bits 1-6 with the lane whose index differs in bit 0-5
    const float t = y0;
    y0 = t + y1;
    y1 = t - y1;
#pragma unroll
    for (int hb = 1; hb < 64; hb <<= 1) {
      const bool hi = (lane & hb) != 0;
      const float o0 = __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ hb) << 2, __float_as_int(y0)));
      const float o1 = __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ hb) << 2, __float_as_int(y1)));
      y0 = hi ? o0 - y0 : y0 + o0;
      y1 = hi ? o1 - y1 : y1 + o1;
    }
    const float c = static_cast<float>(L.had_scale);
    y0 *= c;
    y1 *= c;
  }
  const int b = u / L.Hkv, h = u - b * L.Hkv;
  float* op = J.out + (static_cast<int64_t>(b) * L.Hq + h * G + r) * D + 2 * lane;
  *reinterpret_cast<float2*>(op) = make_float2(y0, y1);
  if (__ballot(nonfinite_bits(y0) || nonfinite_bits(y1)) != 0u && lane == 0) atomicAdd(J.nonfinite, 1u);
}

}  // namespace

hipError_t launch_decode_merge(const LayerDesc& L, const DecodeJob& j, hipStream_t s) {
  // every group of the workgroup runs the same number of row passes
  if (L.G < 1 || L.G > kMaxGroupRows || (L.G & (L.G - 1)) != 0) return hipErrorInvalidValue;
  if (j.nsplit < 1 || j.nsplit > kMaxBodySplits) return hipErrorInvalidValue;  // LDS tables hold 256
  // up to eight splits per unit: one wavefront per (unit, row) with every
  // split requested at once (512 units x 6 splits of a batch-64 GQA layer:
  // 3 us faster than a workgroup per unit; with 24 splits, 1.3 us slower, and
  // a 32-split variant is 5 us slower per call on the 512-unit layers)
  if (j.nsplit <= 8) {
    hipLaunchKernelGGL(decode_merge_rows_kernel<8>, dim3((L.units * L.G + 3) / 4), dim3(256), 0, s, L, j);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(decode_merge_kernel<kMergeGroups>, dim3(L.units), dim3(32 * kMergeGroups), 0, s, L, j);
  return hipGetLastError();
}

int decode_fast_waves(const LayerDesc& L) {
  DecodeJob none{};
  int waves = 0;
  (void)dispatch(L, none, nullptr, &waves);
  return waves;
}

hipError_t launch_decode_fast(const LayerDesc& L, const DecodeJob& j, hipStream_t s, bool* used) {
  int waves = 0;
  const hipError_t e = dispatch(L, j, s, &waves);
  *used = waves > 0;
  return e;
}

}  // namespace kvq
