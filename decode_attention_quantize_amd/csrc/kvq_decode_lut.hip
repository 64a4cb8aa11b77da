// kvq_decode_lut.hip -- split-context decode for MHA layers whose keys and
// values are 3-bit codes with per-layer level tables (KVQuant (iii) codebooks,
// or the uniform grid 0..7), per-vector sparse fp16 outliers (KVQuant (iv))
// and keys cached before RoPE (KVQuant (ii)).
//
// One wavefront per split, one query row per kv head.  A 32-token block:
//   keys    lane l owns RoPE pair (l, l + 64) for all 32 tokens; a token's
//           two codes form one 6-bit field that indexes a 64-entry LDS table
//           of level pairs.  Keys are dequantized in fp32 (L * s + z) and
//           dotted with the query rotated back to the token's position,
//           q . R(p) k = (R(-p) q) . k: the lane steps its pair of the
//           rotated query one position per token (fp32 rotation by theta_l,
//           tokens 0..15 and 16..31 as two chains), and both chains are
//           recomputed exactly (fp64 angle reduction) at each split start.
//   scores  the 64 lanes' partial dots of 32 tokens are summed by a
//           transpose-reduce (permlane swaps across halves and rows, then DPP
//           inside rows) that leaves token l/2 in lanes l; the outlier
//           corrections (x_out - k_dense) * (R(-p) q)[col] are computed in
//           those same lanes.
//   values  O += sum_t (p_t s_tg) L[code] on v_mfma_f32_16x16x32_f16, with the
//           level pairs from a second LDS table as the B operand, the
//           zero points through one more MFMA, and the value outliers
//           (x_out - v_dense) * p_t accumulated per channel in LDS.
// Splits write (o, max, sum) partials for decode_merge_kernel.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_mfma.h"

namespace kvq {
namespace {

// Ring copies issued from inline assembly.  Through the builtin, the compiler
// knows of the copy into LDS and, unable to tell the ring apart from the
// kernel's tables, waits for every copy in flight (the next block's too)
// before its first LDS access of each block.  Issued here, the copies are
// awaited only by ring_wait, at the top of the block that reads them; a
// slot is refilled one block after its last read, whose results the block
// has consumed by then.  M0 holds the LDS base (one nop between its write
// and the copy); each lane's 16 bytes land at M0 + 16 * lane.
__device__ __forceinline__ void ring_load_opaque(const uint8_t* src, uint32_t lds_dst) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" : : "v"(src), "s"(lds_dst)
               : "memory", "m0");
}
// wait until at most N ring copies are in flight; also a compiler barrier
// for the LDS reads that follow
template <int N>
__device__ __forceinline__ void ring_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Record of a block with 3-bit keys and values, value groups of 32 and K
// outliers per token vector (the host layout rules, fixed at compile time).
template <int OUTK>
struct Rec3 {
  static constexpr int off_km = 1536;
  static constexpr int off_vc = off_km + 512;
  static constexpr int off_vm = off_vc + 1536;
  static constexpr int off_ko = off_vm + 512;
  static constexpr int off_vo = off_ko + (32 * OUTK * 4 + 15) / 16 * 16;
  static constexpr int bytes = off_vo + (32 * OUTK * 4 + 15) / 16 * 16;
  static constexpr int loads = (bytes + 1023) / 1024;
};

constexpr double kTwoPi = 6.283185307179586476925286766559;
constexpr double kInvTwoPi = 0.15915494309189533576888376337251;

// cos/sin of an angle given in revolutions (|x| <= 256): the hardware
// v_cos_f32 / v_sin_f32 (absolute error about 1e-6)
__device__ __forceinline__ void cs_rev(float x, float& c, float& s) {
  c = __builtin_amdgcn_cosf(x);
  s = __builtin_amdgcn_sinf(x);
}
// cos/sin of p * theta: the angle is reduced modulo 2 pi in binary64 (error
// ~1e-11 rad for the positions here), then evaluated as above
__device__ __forceinline__ void rot_cs(double p, double theta, float& c, float& s) {
  const double a = p * theta;
  const double r = fma(-rint(a * kInvTwoPi), kTwoPi, a);
  cs_rev(static_cast<float>(r * kInvTwoPi), c, s);
}

// cos/sin of a (radians) to fp32 rounding: reduction modulo 2 pi in binary64,
// Taylor series of degree 12 at a/8 (|a/8| <= pi/8, truncation < 1e-14),
// then three angle doublings.  For the per-lane rotation constants that are
// applied many times in a row.
__device__ __forceinline__ void cs_accurate(double a, float& c, float& s) {
  const double r = fma(-rint(a * kInvTwoPi), kTwoPi, a) * 0.125;
  const double x2 = r * r;
  double sn = r * (1.0 + x2 * (-1.0 / 6 + x2 * (1.0 / 120 + x2 * (-1.0 / 5040 + x2 * (1.0 / 362880 + x2 * (-1.0 / 39916800))))));
  double cs = 1.0 + x2 * (-0.5 + x2 * (1.0 / 24 + x2 * (-1.0 / 720 + x2 * (1.0 / 40320 + x2 * (-1.0 / 3628800 + x2 * (1.0 / 479001600))))));
  for (int k = 0; k < 3; ++k) {
    const double s2 = 2.0 * sn * cs;
    cs = 1.0 - 2.0 * sn * sn;
    sn = s2;
  }
  c = static_cast<float>(cs);
  s = static_cast<float>(sn);
}

// Two 3-bit codes of a lane's chunk (six words) as one 6-bit field at bit
// offset `bit` of the 192-bit stream: the entry it selects in a table of
// 32-bit level pairs.
__device__ __forceinline__ uint32_t pair_at(const uint32_t (&w)[6], int bit, const uint32_t* table) {
  const int q = bit >> 5, r = bit & 31;
  const uint32_t f = r <= 26 ? __builtin_amdgcn_ubfe(w[q], r, 6) : (__builtin_amdgcn_alignbit(w[q + 1], w[q], r) & 63u);
  return table[f];
}

// 3-bit code of (token slot j, channel c) in an LDS copy of a record section
// (the lane-chunk maps of the key and value layouts).
__device__ __forceinline__ int chunk3_lds(const lds_u8* codes, int lane, int e) {
  typedef __attribute__((address_space(3))) const uint32_t lds_u32;
  const lds_u32* w = reinterpret_cast<lds_u32*>(codes) + 6 * lane;
  const int bit = 3 * e;
  const uint32_t lo = w[bit >> 5];
  const uint32_t hi = (bit >> 5) < 5 ? w[(bit >> 5) + 1] : 0u;
  return static_cast<int>(__builtin_amdgcn_alignbit(hi, lo, bit & 31) & 7u);
}
__device__ __forceinline__ int k3_lds(const lds_u8* codes, int j, int c) {
  return chunk3_lds(codes, c & 63, 2 * j + (c >> 6));
}
__device__ __forceinline__ int v3_lds(const lds_u8* codes, int j, int c) {
  return chunk3_lds(codes, 16 * (j >> 3) + (c & 15), 8 * (c >> 4) + (j & 7));
}

template <int OUTK, bool ROPE, int NBUF>
__global__ void __launch_bounds__(64) decode_lut_kernel(LayerDesc L, DecodeJob J) {
  using R = Rec3<OUTK>;
  static_assert(NBUF >= 2 && NBUF <= 3, "ring of 2 or 3 slots");
  static_assert(OUTK >= 0 && OUTK <= 2, "one outlier entry per lane");
  // a slot holds exactly one record: lanes past the record's end issue no copy
  __shared__ __attribute__((aligned(16))) uint8_t ring0[R::bytes];
  __shared__ __attribute__((aligned(16))) uint8_t ring1[R::bytes];
  __shared__ __attribute__((aligned(16))) uint8_t ring2[NBUF >= 3 ? R::bytes : 16];
  __shared__ uint32_t lutk[64], lutv[64];
  __shared__ __attribute__((aligned(16))) _Float16 ptile[32];  // P of the query row
  __shared__ float ocorr[D], qs[D];
  __shared__ float2 tb[64];
  __shared__ float thf[64];
  __shared__ double thd[64];
  lds_u8* const slot0 = (lds_u8*)ring0;
  lds_u8* const slot1 = (lds_u8*)ring1;
  lds_u8* const slot2 = (lds_u8*)ring2;
  auto slot_at = [&](int k) __attribute__((always_inline)) {
    return k == 0 ? slot0 : (k == 1 ? slot1 : slot2);
  };

  const int l = threadIdx.x;
  const int n16 = l & 15, g4 = l >> 4;
  const int nsplit = J.nsplit;
  const int sp = blockIdx.x;
  const int u = blockIdx.y;
  const int b = u / L.Hkv, h = u % L.Hkv;
  const TokenState st = J.st;
  const float kscale = kLog2e / sqrtf(static_cast<float>(D));

  // ---- level-pair tables, query, per-channel value corrections
  {
    // entry c0 + 8 c1 = (L[c0], L[c1]); levels picked with constant indices.
    // Without codebooks the levels are the uniform grid 0..7 (fp16 bits).
    constexpr uint16_t kGrid[8] = {0x0000, 0x3C00, 0x4000, 0x4200, 0x4400, 0x4500, 0x4600, 0x4700};
    uint32_t k0 = 0, k1 = 0, v0 = 0, v1 = 0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t lk = L.nuq ? L.lev_k[c] : kGrid[c], lv = L.nuq ? L.lev_v[c] : kGrid[c];
      if ((l & 7) == c) { k0 = lk; v0 = lv; }
      if ((l >> 3) == c) { k1 = lk; v1 = lv; }
    }
    lutk[l] = k0 | (k1 << 16);
    lutv[l] = v0 | (v1 << 16);
  }
  const uint16_t* qp = J.q + (static_cast<int64_t>(b) * L.Hq + h) * D;
  const float q_lo = h2f(qp[l]), q_hi = h2f(qp[64 + l]);  // pair l: channels l, l + 64
  qs[l] = q_lo;
  qs[64 + l] = q_hi;
  ocorr[l] = 0.f;
  ocorr[64 + l] = 0.f;
  const double theta_l = pow(static_cast<double>(L.rope_base), -2.0 * l / D);
  thf[l] = static_cast<float>(theta_l);
  thd[l] = theta_l;
  // rotation of pair l by one and by 16 positions
  float c1 = 1.f, s1 = 0.f, c16 = 1.f, s16 = 0.f;
  if constexpr (ROPE) {
    cs_accurate(theta_l, c1, s1);
    cs_accurate(16.0 * theta_l, c16, s16);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // this lane's pairs p = 0..15: channels 16g + p and 64 + 16g + p
  // (query halves qs, binary64 frequencies thd: read from LDS where needed)
  const float* qa = qs + 16 * g4;
  const float* qb = qs + 64 + 16 * g4;
  const double* th = thd + 16 * g4;

  // row ceiling (no score seen so far exceeds it), starting from a finite
  // value below every score so that masked -inf scores weigh 2^-inf = 0
  constexpr float kNoScore = -3.0e38f;
  float m_run = kNoScore, l_run = 0.f;
  f32x4 oacc[8];
  f32x4 zacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) oacc[nt] = {0.f, 0.f, 0.f, 0.f};

  // online softmax of the 32 scores (lanes 2t and 2t + 1 hold token t);
  // P (fp16) of the query row lands in ptile, l_run keeps this lane's share
  // of the row sum (even lanes).  The weights are 2^(s - m_run) <= 1 under
  // the row ceiling; only a block with a score above it (the first, rarely
  // a later one) reduces the block maximum, moves the ceiling 2 binades above
  // it and rescales the accumulators.
  auto softmax_tile = [&](float sv) __attribute__((always_inline)) -> half8 {
    if (__builtin_amdgcn_ballot_w64(sv > m_run)) {
      const float mn = wave_max(sv) + 2.f;
      const float alpha = fexp2(m_run - mn);  // 0 from the start value
      m_run = mn;
      l_run *= alpha;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        oacc[nt][0] *= alpha;
        oacc[nt][1] *= alpha;  // row 1: the lo parts of the value products
      }
      zacc[0] *= alpha;
      ocorr[l] *= alpha;
      ocorr[64 + l] *= alpha;
    }
    const _Float16 pt = static_cast<_Float16>(fexp2(sv - m_run));
    l_run += (l & 1) ? 0.f : static_cast<float>(pt);
    if (!(l & 1)) ptile[l >> 1] = pt;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // row 1 reads row 0 again: it carries the lo parts of the value products
    return n16 < 2 ? *reinterpret_cast<const half8*>(&ptile[8 * g4]) : h8(0u, 0u, 0u, 0u);
  };
  // sum over the four lanes that hold one token's partial dots
  auto lanes4_sum = [&](float v) __attribute__((always_inline)) {
    v += xshflf<16>(v);
    v += __int_as_float(__builtin_amdgcn_ds_bpermute((l ^ 32) << 2, __float_as_int(v)));
    return v;
  };

  // ---- this lane's pair of the rotated query, W = R(-pos) q, at the
  // block's tokens 0 (w1) and 16 (w2); each chain steps one position per token
  float w1a = q_lo, w1b = q_hi, w2a = q_lo, w2b = q_hi;
  float tc = 1.f, ts = 0.f, trc = 1.f, trs = 0.f;  // (cos, sin)(theta_l * block start), step
  auto rot_by = [](float& a, float& b, float c, float s) __attribute__((always_inline)) {
    const float a0 = a, b0 = b;
    a = fmaf(c, a0, s * b0);
    b = fmaf(c, b0, -(s * a0));
  };
  auto init_w = [&](int pos_first) __attribute__((always_inline)) {
    if constexpr (ROPE) {
      float c, s;
      rot_cs(static_cast<double>(pos_first), theta_l, c, s);
      w1a = fmaf(q_lo, c, q_hi * s);
      w1b = fmaf(q_hi, c, -(q_lo * s));
      rot_cs(static_cast<double>(pos_first + 16), theta_l, c, s);
      w2a = fmaf(q_lo, c, q_hi * s);
      w2b = fmaf(q_hi, c, -(q_lo * s));
    }
  };

  // ================= sink / window tokens (fp16), one 32-slot chunk at a time
  {
    const int slots = L.sinks_cap + L.win_cap;
    const uint16_t* kf = L.fp16 + static_cast<int64_t>(u) * 2 * slots * D;
    const uint16_t* vf = kf + static_cast<int64_t>(slots) * D;
    const int wchunks = L.win_cap / kBlockTokens;
    const int wstart = st.nb % L.win_cap;
    for (int c = sp - J.fp16_split0; c >= 0 && c < J.fp16_chunks; c += J.fp16_nsplit) {
      const bool sinkc = c < J.sink_chunks;
      const int s0 = sinkc ? kBlockTokens * c
                           : L.sinks_cap + kBlockTokens * ((J.win_chunk0 + c - J.sink_chunks) % wchunks);
      float sc[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int x = s0 + 16 * nt + n16;
        bool live;
        int pos;
        if (sinkc) {
          live = x < st.s_eff;
          pos = x;
        } else {
          int d = x - L.sinks_cap - wstart;
          if (d < 0) d += L.win_cap;
          live = d < st.r;
          pos = st.s_eff + st.nb + d;
        }
        const uint16_t* kr = kf + static_cast<int64_t>(x) * D;
        const u32x4 ka0 = ld16(kr + 16 * g4), ka1 = ld16(kr + 16 * g4 + 8);
        const u32x4 kb0 = ld16(kr + 64 + 16 * g4), kb1 = ld16(kr + 64 + 16 * g4 + 8);
        const half8 ha0 = h8(ka0), ha1 = h8(ka1), hb0 = h8(kb0), hb1 = h8(kb1);
        float acc = 0.f;
#pragma unroll
        for (int p = 0; p < 16; ++p) {
          float c1 = 1.f, s1 = 0.f;
          if constexpr (ROPE) rot_cs(static_cast<double>(pos), th[p], c1, s1);
          const float wa1 = fmaf(qa[p], c1, qb[p] * s1), wb1 = fmaf(qb[p], c1, -(qa[p] * s1));
          const float ka = static_cast<float>(p < 8 ? ha0[p] : ha1[p - 8]);
          const float kb = static_cast<float>(p < 8 ? hb0[p] : hb1[p - 8]);
          acc = fmaf(ka, wa1, fmaf(kb, wb1, acc));
        }
        acc = lanes4_sum(acc);
        sc[nt] = live ? acc * kscale : -INFINITY;
      }
      u32x4 vv[8];
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) vv[nt] = ld16(vf + (static_cast<int64_t>(s0 / 8 + g4) * D + 16 * nt + n16) * 8);
      // token l/2 of the chunk: tile (l/2)/16, lane (l/2)%16 of row 0
      const float sa0 = lane_bcast(sc[0], (l >> 1) & 15), sa1 = lane_bcast(sc[1], (l >> 1) & 15);
      const half8 pa = softmax_tile(l < 32 ? sa0 : sa1);
      const half8 p0 = n16 == 0 ? pa : h8(0u, 0u, 0u, 0u);  // fp16 values: no lo row
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) oacc[nt] = mfma(p0, h8(vv[nt]), oacc[nt]);
    }
  }

  // ================= quantized body blocks through the LDS ring
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
      if (off < R::bytes) ring_load_opaque(src + off, lds_off(dst) + k * 1024);
    }
  };
#pragma unroll
  for (int k = 0; k < NBUF - 1; ++k)
    if (k < nmy) issue(k, slot_at(k));

  if (nmy > 0) {
    const int pos0 = st.s_eff + kBlockTokens * c_begin;
    init_w(pos0);
    if constexpr (ROPE) {
      if constexpr (OUTK > 0) {
        rot_cs(static_cast<double>(pos0), theta_l, tc, ts);
        rot_cs(32.0, theta_l, trc, trs);
      }
    }
  }

  // one block whose record sits in LDS at rec
  auto body_block = [&](const lds_u8* rec, int count) __attribute__((always_inline)) {
    const uint32_t r0 = lds_off(rec);
    const lds_u8* rb = rec;
    typedef __attribute__((address_space(3))) const uint32_t lds_u32;
    typedef __attribute__((address_space(3))) const uint16_t lds_u16;
    uint32_t kw[6];  // this lane's 64 key codes: token t's pair in bits 6t..6t+5
    {
      const uint32_t ak = r0 + 24 * l;
      u32x2 k0 = dsr8<0>(ak), k1 = dsr8<8>(ak), k2 = dsr8<16>(ak);
      lds_wait();
      pin(k0);
      pin(k1);
      pin(k2);
      kw[0] = k0[0]; kw[1] = k0[1]; kw[2] = k1[0]; kw[3] = k1[1]; kw[4] = k2[0]; kw[5] = k2[1];
    }
    const lds_u16* km = reinterpret_cast<lds_u16*>(rb + R::off_km);
    const float sa = h2f(km[l]), sb = h2f(km[64 + l]), za = h2f(km[D + l]), zb = h2f(km[D + 64 + l]);

    // ---- key outliers: lanes 2t, 2t + 1 compute (x_out - k_dense) * W_t[col]
    // for the entries of token t (one each, or the same one for a single entry)
    float kcorr = 0.f;
    if constexpr (OUTK > 0) {
      const int t = l >> 1;
      if (t < count) {
        const uint32_t ent = *reinterpret_cast<lds_u32*>(rb + R::off_ko + 4 * (t * OUTK + (OUTK == 2 ? (l & 1) : 0)));
        const int col = static_cast<int>(ent & 0x7Fu);  // columns are < 128
        const float val = h2f(static_cast<uint16_t>(ent >> 16));
        const int code = k3_lds(rb, t, col);
        const float kd = fmaf(h2f(static_cast<uint16_t>(lutk[9 * code])), h2f(km[col]), h2f(km[D + col]));
        const int i = col & 63;
        float w;
        if constexpr (ROPE) {
          const float2 base = tb[i];
          float st_, ct_;
          cs_rev(static_cast<float>(t) * thf[i] * static_cast<float>(kInvTwoPi), ct_, st_);
          const float c = base.x * ct_ - base.y * st_;
          const float sn = base.y * ct_ + base.x * st_;
          w = col < 64 ? fmaf(qs[i], c, qs[64 + i] * sn) : fmaf(qs[64 + i], c, -(qs[i] * sn));
        } else {
          w = qs[col];
        }
        kcorr = (val - kd) * w;
      }
      if constexpr (OUTK == 2) kcorr += dppf<kQuadXor1>(kcorr);
    }

    // ---- keys: dequantize this lane's pair for tokens k and 16 + k, dot with
    // the rotated query, and fold the two tokens across the lane halves
    uint32_t lk[32];  // level pairs of the 32 tokens
#pragma unroll
    for (int t = 0; t < 32; ++t) lk[t] = pair_at(kw, 6 * t, lutk);
    float e1[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const half2v lp1 = __builtin_bit_cast(half2v, lk[k]);
      const half2v lp2 = __builtin_bit_cast(half2v, lk[16 + k]);
      const float d1 = fmaf(fmaf(static_cast<float>(lp1[0]), sa, za), w1a, fmaf(static_cast<float>(lp1[1]), sb, zb) * w1b);
      const float d2 = fmaf(fmaf(static_cast<float>(lp2[0]), sa, za), w2a, fmaf(static_cast<float>(lp2[1]), sb, zb) * w2b);
      const float2 x = swap32(d1, d2);
      e1[k] = x.x + x.y;  // token k + 16 (l / 32), lanes l and l ^ 32
      if constexpr (ROPE) {
        if (k < 15) rot_by(w1a, w1b, c1, s1);
        rot_by(w2a, w2b, c1, s1);
      }
    }
    if constexpr (ROPE) {  // chain 1 restarts 32 positions on, chain 2 16 after it
      w1a = w2a;
      w1b = w2b;
      rot_by(w2a, w2b, c16, s16);
    }
    // remaining folds: rows (xor 16), then xor 8, xor 7, xor 2 inside rows;
    // the lane keeps the token whose index bit matches its own lane bit
    float e2[8], e3[4], e4[2];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float2 x = swap16(e1[k], e1[k + 8]);
      e2[k] = x.x + x.y;
    }
    const bool b3 = (l & 8) != 0, b2 = (l & 4) != 0, b1 = (l & 2) != 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) e3[k] = (b3 ? e2[k + 4] : e2[k]) + dppf<kRowRor8>(b3 ? e2[k] : e2[k + 4]);
#pragma unroll
    for (int k = 0; k < 2; ++k) e4[k] = (b2 ? e3[k + 2] : e3[k]) + dppf<kRowHalfMirror>(b2 ? e3[k] : e3[k + 2]);
    float dot = (b1 ? e4[1] : e4[0]) + dppf<kQuadXor2>(b1 ? e4[0] : e4[1]);
    dot += dppf<kQuadXor1>(dot);  // token l / 2, whole sum
    const float sc = (l >> 1) < count ? (dot + kcorr) * kscale : -INFINITY;

    // ---- values: level pairs through lutv as the MFMA B operand
    uint32_t vw[6];
    u32x4 vmeta[5];
    {
      const uint32_t av = r0 + R::off_vc + 24 * l;
      u32x2 v0 = dsr8<0>(av), v1 = dsr8<8>(av), v2 = dsr8<16>(av);
      const uint32_t az = r0 + R::off_vm + (n16 < 4 ? 2 * 4 * kBlockTokens : 0) + 2 * ((n16 & 3) * kBlockTokens + 8 * g4);
      const uint32_t asv = r0 + R::off_vm + 16 * g4;
      vmeta[4] = dsr16<0>(az);
      vmeta[0] = dsr16<0>(asv);
      vmeta[1] = dsr16<64>(asv);
      vmeta[2] = dsr16<128>(asv);
      vmeta[3] = dsr16<192>(asv);
      lds_wait();
      pin(v0);
      pin(v1);
      pin(v2);
#pragma unroll
      for (int e = 0; e < 5; ++e) pin(vmeta[e]);
      vw[0] = v0[0]; vw[1] = v0[1]; vw[2] = v1[0]; vw[3] = v1[1]; vw[4] = v2[0]; vw[5] = v2[1];
    }
    uint32_t vl[32];  // level pairs of the B operands
#pragma unroll
    for (int x = 0; x < 32; ++x) vl[x] = pair_at(vw, 6 * x, lutv);
    const half8 pa = softmax_tile(sc);
    zacc = mfma(pa, n16 < 8 ? h8(vmeta[4]) : h8(0u, 0u, 0u, 0u), zacc);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      // row 0: hi parts of p * s, row 1: lo parts (added at the end), one MFMA per tile
      half8 w = pa * h8(vmeta[g]);
      if (n16 >= 1) lo_in_place(w, pa, h8(vmeta[g]));
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const int nt = 2 * g + t2;
        const half8 bv = h8(vl[4 * nt], vl[4 * nt + 1], vl[4 * nt + 2], vl[4 * nt + 3]);
        oacc[nt] = mfma(w, bv, oacc[nt]);
      }
    }

    // ---- value outliers: (x_out - v_dense) * p_t into ocorr[col]
    if constexpr (OUTK > 0) {
      const int t = OUTK == 2 ? (l >> 1) : l;
      if (t < count && (OUTK == 2 || l < 32)) {
        const uint32_t ent = *reinterpret_cast<lds_u32*>(rb + R::off_vo + 4 * (t * OUTK + (OUTK == 2 ? (l & 1) : 0)));
        const int col = static_cast<int>(ent & 0x7Fu);  // columns are < 128
        const float val = h2f(static_cast<uint16_t>(ent >> 16));
        const int code = v3_lds(rb + R::off_vc, t, col);
        const lds_u16* vm = reinterpret_cast<lds_u16*>(rb + R::off_vm);
        const int g = col >> 5;
        const float vd = fmaf(h2f(static_cast<uint16_t>(lutv[9 * code])), h2f(vm[g * kBlockTokens + t]),
                              h2f(vm[4 * kBlockTokens + g * kBlockTokens + t]));
        atomicAdd(&ocorr[col], (val - vd) * static_cast<float>(ptile[t]));
      }
    }

    // ---- advance the rotated queries (and the outlier angle table) by 32 positions
    if constexpr (ROPE) {
      if constexpr (OUTK > 0) {
        const float c = tc, s = ts;
        tc = fmaf(c, trc, -(s * trs));
        ts = fmaf(s, trc, c * trs);
        tb[l] = make_float2(tc, ts);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  if constexpr (ROPE && OUTK > 0) {
    tb[l] = make_float2(tc, ts);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  {
    // Wavefronts sharing a SIMD are picked oldest first; each one lowers its
    // priority as it gets through its blocks so that they finish together.
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
    auto step = [&](int i, lds_u8* cur, lds_u8* ahead) __attribute__((always_inline)) {
      age(i);
      issue(i + NBUF - 1, ahead);
      ring_wait<(NBUF - 1) * R::loads>();
      const int ch = c_begin + i;
      body_block(cur, min(kBlockTokens, st.nb - ch * kBlockTokens));
    };
    int i = 0;
    for (; i + 2 * NBUF - 2 < nmy; i += NBUF) {
      if constexpr (NBUF == 3) {
        step(i, slot0, slot2);
        step(i + 1, slot1, slot0);
        step(i + 2, slot2, slot1);
      } else {
        step(i, slot0, slot1);
        step(i + 1, slot1, slot0);
      }
    }
    for (; i < nmy; ++i) {
      age(i);
      const int ahead = i + NBUF - 1;
      if (ahead < nmy) issue(ahead, slot_at(ahead % NBUF));
      const int newer = min(NBUF - 1, nmy - 1 - i);
      if (NBUF >= 3 && newer >= 2)
        ring_wait<(NBUF >= 3 ? 2 : 0) * R::loads>();
      else if (newer >= 1)
        ring_wait<R::loads>();
      else
        ring_wait<0>();
      const int ch = c_begin + i;
      body_block(slot_at(i % NBUF), min(kBlockTokens, st.nb - ch * kBlockTokens));
    }
  }

  __builtin_amdgcn_s_setprio(0);
  // ---- partial of this split (row 0): o = O_raw + Z + value-outlier corrections
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float* opart = J.partials + (static_cast<int64_t>(u) * nsplit + sp) * D;
  float* mlpart = J.partials + J.ml_off + (static_cast<int64_t>(u) * nsplit + sp) * 2;
  const float lsum = wave_sum(l_run);
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    const float z = lane_bcast(zacc[0], (l & 48) | (nt >> 1));
    const float o = (oacc[nt][0] + oacc[nt][1]) + z + ocorr[16 * nt + n16];
    if (g4 == 0) opart[16 * nt + n16] = o;
  }
  if (l == 0) {
    mlpart[0] = m_run == kNoScore ? -INFINITY : m_run;  // no live token seen: -inf
    mlpart[1] = lsum;
  }
}

template <int OUTK, bool ROPE>
hipError_t launch_lut(const LayerDesc& L, const DecodeJob& j, hipStream_t s, int* waves) {
  using R = Rec3<OUTK>;
  if (L.off_km != R::off_km || L.off_vc != R::off_vc || L.off_vm != R::off_vm ||
      (OUTK > 0 && (L.off_ko != R::off_ko || L.off_vo != R::off_vo)))
    return hipSuccess;
  // two ring slots: with them LDS admits three wavefronts per SIMD, as the
  // register budget does
  constexpr int NB = 2;
  static std::atomic<int> resident[kMaxDevices];
  if (resident_waves(decode_lut_kernel<OUTK, ROPE, NB>, resident, waves) != hipSuccess)
    return hipErrorInvalidValue;
  if (!j.q) return hipSuccess;  // query only
  hipLaunchKernelGGL((decode_lut_kernel<OUTK, ROPE, NB>), dim3(j.nsplit, L.units), dim3(64), 0, s, L, j);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  return launch_decode_merge(L, j, s);
}

hipError_t dispatch_lut(const LayerDesc& L, const DecodeJob& j, hipStream_t s, int* waves) {
  *waves = 0;
  if (L.G != 1 || L.kb != 3 || L.vb != 3 || L.k_inner || L.k_hybrid || L.v_had || L.v_group != 32)
    return hipSuccess;
  const bool rope = L.pre_rope != 0;
  switch (L.outk) {
    case 0: return rope ? launch_lut<0, true>(L, j, s, waves) : launch_lut<0, false>(L, j, s, waves);
    case 1: return rope ? launch_lut<1, true>(L, j, s, waves) : launch_lut<1, false>(L, j, s, waves);
    case 2: return rope ? launch_lut<2, true>(L, j, s, waves) : launch_lut<2, false>(L, j, s, waves);
    default: return hipSuccess;
  }
}

}  // namespace

int decode_lut_waves(const LayerDesc& L) {
  DecodeJob none{};
  int waves = 0;
  dispatch_lut(L, none, nullptr, &waves);
  return waves;
}

hipError_t launch_decode_lut(const LayerDesc& L, const DecodeJob& j, hipStream_t s, bool* used) {
  int waves = 0;
  const hipError_t e = dispatch_lut(L, j, s, &waves);
  *used = waves > 0;
  return e;
}

}  // namespace kvq
