// kvq_decode_fast.hip -- matrix-core (MFMA) split-context decode over the
// packed cache for uniform 2/4/8-bit keys and values.
//
// One wavefront per split.  A 32-token block is two 16-token tiles:
//   scores  S[r][t] = sum_c A[r][c] B[c][t] with v_mfma_f32_16x16x32_f16, where
//           B holds the codes as fp16 subnormals (bit pattern = code, value
//           code * 2^-24: exact in the MFMA, no offset to undo) and
//           A = fp16(q * s) when keys have one scale per channel per block
//           (KVTuner obs. 2 / KVQuant (i)); the zero points enter as the
//           per-row constant sum_c q_c z_c.  For InnerQ inner-dimension groups
//           (per-token scales) A = q and the group sums are scaled afterwards.
//   values  O[r][c] += sum_t (p[r][t] * s[t][g]) code[t][c]: per-token value
//           scales (RateQuant sec. 3, KIVI layout) fold into P; the zero points
//           sum_t p z are one more MFMA against the block's z column.
//   online softmax in the log2 domain; splits merged by log-sum-exp in the
//   last wavefront of each unit; Hadamard-rotated values unrotated there.
// Only the first G rows of the 16-row MFMA tiles carry queries (the GQA group
// of a kv head); keys of one block are read once for all of them.
#include <hip/hip_runtime.h>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int D = kHeadDim;
constexpr int PW = D + 2;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaves = 4;

struct WaveSmem {
  _Float16 p[16][32];
  float row[16];
};

__device__ __forceinline__ f32x4 mfma(half8 a, half8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ half8 h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const u32x4 v = {a, b, c, d};
  return __builtin_bit_cast(half8, v);
}
__device__ __forceinline__ half8 h8(u32x4 v) { return __builtin_bit_cast(half8, v); }
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }

// ---- code words -> eight fp16 code values, K-order = element order.
// 2-bit codes become 1 + c/4 and 4-bit codes 1 + c/16 (code bits placed at
// the top of the fp16 mantissa under the exponent of 1.0: one and-or per word);
// 8-bit codes become the integer c.  Normal fp16 operands keep every MFMA
// product exact; the constant offset (base * sum of A) is removed afterwards.
template <int B> struct CodeEnc;
template <> struct CodeEnc<2> { static constexpr float base = 1.f, inv_unit = 4.f; };
template <> struct CodeEnc<4> { static constexpr float base = 1.f, inv_unit = 16.f; };
template <> struct CodeEnc<8> { static constexpr float base = 0.f, inv_unit = 1.f; };

__device__ __forceinline__ uint32_t andor(uint32_t x, uint32_t m, uint32_t o) { return (x & m) | o; }
__device__ __forceinline__ half8 ex4(uint32_t x) {
  constexpr uint32_t M = 0x03C003C0u, O = 0x3C003C00u;
  return h8(andor(x << 6, M, O), andor(x << 2, M, O), andor(x >> 2, M, O), andor(x >> 6, M, O));
}
template <int E>
__device__ __forceinline__ half8 ex2(uint32_t x) {
  constexpr uint32_t M = 0x03000300u, O = 0x3C003C00u;
  if constexpr (E == 0)
    return h8(andor(x << 8, M, O), andor(x << 6, M, O), andor(x << 4, M, O), andor(x << 2, M, O));
  else
    return h8(andor(x, M, O), andor(x >> 2, M, O), andor(x >> 4, M, O), andor(x >> 6, M, O));
}
__device__ __forceinline__ uint32_t u8pair(uint32_t x, int sh) {
  const float a = static_cast<float>((x >> sh) & 0xffu);
  const float b = static_cast<float>((x >> (sh + 8)) & 0xffu);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}
__device__ __forceinline__ half8 ex8(uint32_t x, uint32_t y) {
  return h8(u8pair(x, 0), u8pair(x, 16), u8pair(y, 0), u8pair(y, 16));
}

// B operand of K-step j from a lane's key chunk (32 channels, KB bits each)
template <int KB>
__device__ __forceinline__ half8 kstep(const uint32_t* w, int j) {
  if constexpr (KB == 4) return ex4(w[j]);
  if constexpr (KB == 2) return (j & 1) ? ex2<1>(w[j >> 1]) : ex2<0>(w[j >> 1]);
  if constexpr (KB == 8) return ex8(w[2 * j], w[2 * j + 1]);
}
// B operand of value N-tile nt from a lane's value chunk
template <int VB>
__device__ __forceinline__ half8 vtile(const uint32_t* w, int nt) {
  if constexpr (VB == 4) return ex4(w[nt]);
  if constexpr (VB == 2) return (nt & 1) ? ex2<1>(w[nt >> 1]) : ex2<0>(w[nt >> 1]);
  if constexpr (VB == 8) return ex8(w[2 * nt], w[2 * nt + 1]);
}

template <int W>
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, xshflf<1>(v));
  v = fmaxf(v, xshflf<2>(v));
  v = fmaxf(v, xshflf<4>(v));
  v = fmaxf(v, xshflf<8>(v));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += xshflf<1>(v);
  v += xshflf<2>(v);
  v += xshflf<4>(v);
  v += xshflf<8>(v);
  return v;
}
__device__ __forceinline__ float lane_bcast(float v, int src) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(v)));
}

// channel of K-step j, element kk for lane group g4
template <bool INNER>
__device__ __forceinline__ int kchan(int g4, int j, int kk) {
  if constexpr (INNER) return (j < 2 ? 16 * g4 + 8 * j : 64 + 16 * g4 + 8 * (j - 2)) + kk;
  return 32 * g4 + 8 * j + kk;
}

template <int KB, int VB, int G, bool INNER>
__global__ void __launch_bounds__(64 * kWaves) decode_mfma_kernel(LayerDesc L, DecodeJob J) {
  __shared__ WaveSmem smem[kWaves];
  const int wave = threadIdx.x >> 6;
  const int l = threadIdx.x & 63;
  const int n16 = l & 15, g4 = l >> 4;
  WaveSmem& sm = smem[wave];
  const int nsplit = J.nsplit_body + J.fp16_split;
  const int sp = blockIdx.x * kWaves + wave;
  if (sp >= nsplit) return;
  const int u = blockIdx.y;
  const int b = u / L.Hkv, h = u % L.Hkv;
  const TokenState st = J.st;
  constexpr int RI = G < 4 ? G : 4;           // output rows per lane (registers)
  const bool rows_here = 4 * g4 < G;           // lane holds real query rows
  constexpr int ngv = D / 32;  // value groups of 32 channels

  // ---- query operand (natural channel order per K-step)
  half8 qa[4];
  {
    const bool live = n16 < G;
    const uint16_t* qp = J.q + (static_cast<int64_t>(b) * L.Hq + h * G + (live ? n16 : 0)) * D;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4 v = ld16(qp + kchan<INNER>(g4, j, 0));
      qa[j] = live ? h8(v) : h8(0u, 0u, 0u, 0u);
    }
  }
  // inner groups: per-row sums of q over each 64-channel group
  float qsum[2][RI];
  if constexpr (INNER) {
    float part[2];
    // full-row sums: lanes n16, n16+16, n16+32, n16+48 hold the four quarters
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
      float s = 0.f;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) s += static_cast<float>(qa[2 * gg + jj][kk]);
      s += xshflf<16>(s);
      s += __int_as_float(__builtin_amdgcn_ds_bpermute((l ^ 32) << 2, __float_as_int(s)));
      part[gg] = s;
#pragma unroll
      for (int i = 0; i < RI; ++i) qsum[gg][i] = lane_bcast(part[gg], 20 * g4 + i);
    }
  }

  const float kscale = kLog2e / sqrtf(static_cast<float>(D));
  float m_run[RI], l_run[RI];
#pragma unroll
  for (int i = 0; i < RI; ++i) {
    m_run[i] = -INFINITY;
    l_run[i] = 0.f;
  }
  f32x4 oacc[8];
  f32x4 zacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) oacc[nt] = {0.f, 0.f, 0.f, 0.f};

  const bool fp16_part = J.fp16_split && sp == J.nsplit_body;
  const int nblk_body = (st.nb + kBlockTokens - 1) / kBlockTokens;
  int c_begin, c_end;
  if (fp16_part) {
    c_begin = 0;
    c_end = (st.s_eff + st.r + kBlockTokens - 1) / kBlockTokens;
  } else {
    c_begin = sp * J.blocks_per_split;
    c_end = min(nblk_body, c_begin + J.blocks_per_split);
  }
  const int slots = L.sinks_cap + L.win_cap;
  const uint16_t* kf = L.fp16 + static_cast<int64_t>(u) * 2 * slots * D;
  const uint16_t* vf = kf + static_cast<int64_t>(slots) * D;

  for (int ch = c_begin; ch < c_end; ++ch) {
    f32x4 sacc[2];
    int count;
    half8 pa;
    if (!fp16_part) {
      const uint8_t* rec = L.body + (static_cast<int64_t>(u) * L.nblk_cap + ch) * L.rec_bytes;
      count = min(kBlockTokens, st.nb - ch * kBlockTokens);
      // ---------------- keys
      uint32_t kw[2][KB];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const uint8_t* row = rec + L.off_kc + (16 * nt + n16) * (16 * KB);
        if constexpr (INNER) {
          const u32x2 a = ld8(row + 8 * g4);
          const u32x2 c2 = ld8(row + 32 + 8 * g4);
          kw[nt][0] = a[0]; kw[nt][1] = a[1]; kw[nt][2] = c2[0]; kw[nt][3] = c2[1];
        } else if constexpr (KB == 4) {
          const u32x4 a = ld16(row + 16 * g4);
          kw[nt][0] = a[0]; kw[nt][1] = a[1]; kw[nt][2] = a[2]; kw[nt][3] = a[3];
        } else if constexpr (KB == 2) {
          const u32x2 a = ld8(row + 8 * g4);
          kw[nt][0] = a[0]; kw[nt][1] = a[1];
        } else {
          const u32x4 a = ld16(row + 32 * g4);
          const u32x4 c2 = ld16(row + 32 * g4 + 16);
          kw[nt][0] = a[0]; kw[nt][1] = a[1]; kw[nt][2] = a[2]; kw[nt][3] = a[3];
          kw[nt][4] = c2[0]; kw[nt][5] = c2[1]; kw[nt][6] = c2[2]; kw[nt][7] = c2[3];
        }
      }
      if constexpr (!INNER) {
        // A = q * s per channel as a pair hi + lo of fp16 exact to ~2^-22
        // (lo = fma(q, s, -hi) rounds only the residual).  One MFMA chain
        // against the block's parameters broadcast over the tile's columns
        // gives, per query row, C_z = sum_c q_c z_c (columns 0-7) and
        // C_s = sum_c q_c s_c (columns 8-15); the score of token t is
        //   (sum_c A_c B_ct - base * C_s) * inv_unit + C_z.
        const uint16_t* km = reinterpret_cast<const uint16_t*>(rec + L.off_km);
        half8 qh[4], ql[4];
        f32x4 cacc = {0.f, 0.f, 0.f, 0.f};
        const uint16_t* zs = km + (n16 < 8 ? D : 0) + 32 * g4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const half8 s8 = h8(ld16(km + 32 * g4 + 8 * j));
          qh[j] = qa[j] * s8;
          ql[j] = __builtin_elementwise_fma(qa[j], s8, -qh[j]);
          cacc = mfma(qa[j], h8(ld16(zs + 8 * j)), cacc);
        }
        constexpr float base = CodeEnc<KB>::base, iu = CodeEnc<KB>::inv_unit;
        f32x4 init;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float other = xshflf<8>(cacc[i]);
          const float cz = n16 < 8 ? cacc[i] : other;
          const float cs = n16 < 8 ? other : cacc[i];
          init[i] = fmaf(cz, 1.f / iu, -base * cs);
        }
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          sacc[nt] = init;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const half8 bk = kstep<KB>(kw[nt], j);
            sacc[nt] = mfma(qh[j], bk, sacc[nt]);
            sacc[nt] = mfma(ql[j], bk, sacc[nt]);
          }
        }
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) sacc[nt][i] *= iu * kscale;
      } else {
        // per-token groups of 64 channels: group sums sum_c q_c B_ct, offset
        // removed with the group sums of q, then scaled per token
        constexpr float base = CodeEnc<KB>::base, iu = CodeEnc<KB>::inv_unit;
        const uint16_t* km = reinterpret_cast<const uint16_t*>(rec + L.off_km);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          f32x4 p0 = {0.f, 0.f, 0.f, 0.f}, p1 = {0.f, 0.f, 0.f, 0.f};
          p0 = mfma(qa[0], kstep<KB>(kw[nt], 0), p0);
          p0 = mfma(qa[1], kstep<KB>(kw[nt], 1), p0);
          p1 = mfma(qa[2], kstep<KB>(kw[nt], 2), p1);
          p1 = mfma(qa[3], kstep<KB>(kw[nt], 3), p1);
          const int tok = 16 * nt + n16;
          const u32x2 mm = ld8(km + tok * 4);  // (s0, z0), (s1, z1)
          float sg[2], zg[2];
#pragma unroll
          for (int gg = 0; gg < 2; ++gg) {
            const uint16_t s16 = static_cast<uint16_t>(mm[gg] & 0xffff);
            const uint16_t z16 = static_cast<uint16_t>(mm[gg] >> 16);
            const float sv = h2f(s16 & 0x7fff);
            const bool sym = (s16 & 0x8000) != 0;
            sg[gg] = sv * iu;
            zg[gg] = sym ? -static_cast<float>(1 << (KB - 1)) * sv : h2f(z16);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float sc = 0.f;
            if (i < RI) {
              sc = fmaf(sg[0], fmaf(-base, qsum[0][i], p0[i]), zg[0] * qsum[0][i]);
              sc = fmaf(sg[1], fmaf(-base, qsum[1][i], p1[i]), fmaf(zg[1], qsum[1][i], sc));
            }
            sacc[nt][i] = sc * kscale;
          }
        }
      }
    } else {
      // ---------------- fp16 sinks / window tokens: B = keys as stored
      count = min(kBlockTokens, st.s_eff + st.r - ch * kBlockTokens);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int vi = ch * kBlockTokens + 16 * nt + n16;
        int slot = 0;
        if (vi < count + ch * kBlockTokens) {
          const int pos = vi < st.s_eff ? vi : st.s_eff + st.nb + (vi - st.s_eff);
          slot = vi < st.s_eff ? vi : L.sinks_cap + (pos - st.s_eff) % L.win_cap;
        }
        sacc[nt] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          sacc[nt] = mfma(qa[j], h8(ld16(kf + slot * D + kchan<INNER>(g4, j, 0))), sacc[nt]);
#pragma unroll
        for (int i = 0; i < 4; ++i) sacc[nt][i] *= kscale;
      }
    }

    // ---------------- online softmax over the block (rows 4*g4 + i)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
      if (16 * nt + n16 >= count)
#pragma unroll
        for (int i = 0; i < 4; ++i) sacc[nt][i] = -INFINITY;
    float alpha[RI];
#pragma unroll
    for (int i = 0; i < RI; ++i) {
      const float bm = row16_max<16>(fmaxf(sacc[0][i], sacc[1][i]));
      const float mn = fmaxf(m_run[i], bm);
      alpha[i] = exp2f(m_run[i] - mn);
      // P is used as fp16 in every product below; the denominator sums the
      // same rounded weights so numerator and denominator stay consistent
      const _Float16 p0 = static_cast<_Float16>(exp2f(sacc[0][i] - mn));
      const _Float16 p1 = static_cast<_Float16>(exp2f(sacc[1][i] - mn));
      l_run[i] = fmaf(l_run[i], alpha[i], static_cast<float>(p0) + static_cast<float>(p1));
      m_run[i] = mn;
      if (rows_here) {
        sm.p[4 * g4 + i][n16] = p0;
        sm.p[4 * g4 + i][16 + n16] = p1;
      }
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int i = 0; i < RI; ++i) oacc[nt][i] *= alpha[i];
#pragma unroll
    for (int i = 0; i < RI; ++i) zacc[i] *= alpha[i];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    pa = n16 < G ? *reinterpret_cast<const half8*>(&sm.p[n16][8 * g4]) : h8(0u, 0u, 0u, 0u);

    // ---------------- values
    if (!fp16_part) {
      const uint8_t* rec = L.body + (static_cast<int64_t>(u) * L.nblk_cap + ch) * L.rec_bytes;
      const uint16_t* vm = reinterpret_cast<const uint16_t*>(rec + L.off_vm);
      uint32_t vw[2 * VB];
      const uint8_t* chunk = rec + L.off_vc + l * (8 * VB);
#pragma unroll
      for (int q4 = 0; q4 < (2 * VB) / 4; ++q4) {
        const u32x4 a = ld16(chunk + 16 * q4);
        vw[4 * q4] = a[0]; vw[4 * q4 + 1] = a[1]; vw[4 * q4 + 2] = a[2]; vw[4 * q4 + 3] = a[3];
      }
      // one MFMA of P against the block's value parameters: column g < 4 holds
      // z_g (zero points), column 4 + g holds s_g (removes the code offset)
      {
        const int col = n16 & 3;
        const uint16_t* src = vm + (n16 < 4 ? ngv * kBlockTokens : 0) + col * kBlockTokens + 8 * g4;
        const half8 bz = h8(ld16(src));
        zacc = mfma(pa, n16 < 2 * ngv ? bz : h8(0u, 0u, 0u, 0u), zacc);
      }
      // weights w = p * s per (token, value group) as an exact hi + lo pair
      half8 wh[ngv], wl[ngv];
#pragma unroll
      for (int g = 0; g < ngv; ++g) {
        const half8 s8 = h8(ld16(vm + g * kBlockTokens + 8 * g4));
        wh[g] = pa * s8;
        wl[g] = __builtin_elementwise_fma(pa, s8, -wh[g]);
      }
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const half8 bv = vtile<VB>(vw, nt);
        oacc[nt] = mfma(wh[nt >> 1], bv, oacc[nt]);
        oacc[nt] = mfma(wl[nt >> 1], bv, oacc[nt]);
      }
    } else {
      // fp16 values: B[t][c] = v[t][c], gathered per lane (8 tokens of one channel)
      const int vi0 = ch * kBlockTokens + 8 * g4;
      int slot[8];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int vi = vi0 + kk;
        const int pos = vi < st.s_eff ? vi : st.s_eff + st.nb + (vi - st.s_eff);
        slot[kk] = (vi - ch * kBlockTokens) >= count ? 0
                   : (vi < st.s_eff ? vi : L.sinks_cap + (pos - st.s_eff) % L.win_cap);
      }
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const int c = 16 * nt + n16;
        uint32_t w[4];
#pragma unroll
        for (int kk = 0; kk < 8; kk += 2)
          w[kk / 2] = static_cast<uint32_t>(vf[slot[kk] * D + c]) |
                      (static_cast<uint32_t>(vf[slot[kk + 1] * D + c]) << 16);
        oacc[nt] = mfma(pa, h8(w[0], w[1], w[2], w[3]), oacc[nt]);
      }
    }
  }

  // ---------------- partial of this split
  //   o = (O_raw - base * W_g) * inv_unit + Z_g  (body splits; fp16 split: O_raw)
  constexpr float vbase = CodeEnc<VB>::base, viu = CodeEnc<VB>::inv_unit;
  float* part = J.partials + (static_cast<int64_t>(u) * nsplit + sp) * G * PW;
#pragma unroll
  for (int i = 0; i < RI; ++i) {
    const float lsum = row16_sum(l_run[i]);
    const int row = 4 * g4 + i;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const float z = lane_bcast(zacc[i], (l & 48) | (nt >> 1));
      const float w = lane_bcast(zacc[i], (l & 48) | (4 + (nt >> 1)));
      const float o = fp16_part ? oacc[nt][i] : fmaf(fmaf(-vbase, w, oacc[nt][i]), viu, z);
      if (rows_here && row < G) part[row * PW + 16 * nt + n16] = o;
    }
    if (rows_here && row < G && n16 == 0) {
      part[row * PW + D] = m_run[i];
      part[row * PW + D + 1] = lsum;
    }
  }
  __threadfence();
  uint32_t prev = 0;
  if (l == 0)
    prev = __hip_atomic_fetch_add(J.counters + u, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
  prev = __builtin_amdgcn_readfirstlane(prev);
  if (prev != static_cast<uint32_t>(nsplit - 1)) return;
  __threadfence();

  // ---------------- log-sum-exp merge (this wavefront is the last of the unit)
  const float* base = J.partials + static_cast<int64_t>(u) * nsplit * G * PW;
  for (int r = 0; r < G; ++r) {
    float M = -INFINITY;
    for (int i = 0; i < nsplit; ++i) M = fmaxf(M, base[(i * G + r) * PW + D]);
    float Ls = 0.f, a0 = 0.f, a1 = 0.f;
    for (int i = 0; i < nsplit; ++i) {
      const float* pr = base + (i * G + r) * PW;
      const float mi = pr[D];
      if (mi == -INFINITY) continue;
      const float w = exp2f(mi - M);
      Ls = fmaf(pr[D + 1], w, Ls);
      a0 = fmaf(pr[2 * l], w, a0);
      a1 = fmaf(pr[2 * l + 1], w, a1);
    }
    float y0 = a0 / Ls, y1 = a1 / Ls;
    if (L.v_had) {
      // c * H * o with H the Sylvester matrix; lane l holds channels 2l, 2l+1
      float t0 = y0 + y1, t1 = y0 - y1;
      y0 = t0;
      y1 = t1;
#pragma unroll
      for (int hb = 1; hb < 64; hb <<= 1) {
        const float o0 = __int_as_float(__builtin_amdgcn_ds_bpermute((l ^ hb) << 2, __float_as_int(y0)));
        const float o1 = __int_as_float(__builtin_amdgcn_ds_bpermute((l ^ hb) << 2, __float_as_int(y1)));
        const bool hi = (l & hb) != 0;
        y0 = hi ? o0 - y0 : y0 + o0;
        y1 = hi ? o1 - y1 : y1 + o1;
      }
      const float c = static_cast<float>(L.had_scale);
      y0 *= c;
      y1 *= c;
    }
    float* op = J.out + (static_cast<int64_t>(b) * L.Hq + h * G + r) * D;
    op[2 * l] = y0;
    op[2 * l + 1] = y1;
  }
  if (l == 0) J.counters[u] = 0;
}

template <int KB, int VB, int G, bool INNER>
hipError_t launch_t(const LayerDesc& L, const DecodeJob& j, hipStream_t s) {
  const int nsplit = j.nsplit_body + j.fp16_split;
  hipLaunchKernelGGL((decode_mfma_kernel<KB, VB, G, INNER>), dim3((nsplit + kWaves - 1) / kWaves, L.units),
                     dim3(64 * kWaves), 0, s, L, j);
  return hipGetLastError();
}

template <int G, bool INNER>
hipError_t by_bits(const LayerDesc& L, const DecodeJob& j, hipStream_t s, bool* used) {
  *used = true;
  const int k = L.kb, v = L.vb;
#define KVQ_CASE(KB, VB) \
  if (k == KB && v == VB) return launch_t<KB, VB, G, INNER>(L, j, s);
  if constexpr (INNER) {
    KVQ_CASE(4, 2) KVQ_CASE(4, 4)
  } else {
    KVQ_CASE(2, 2) KVQ_CASE(2, 4) KVQ_CASE(2, 8)
    KVQ_CASE(4, 2) KVQ_CASE(4, 4) KVQ_CASE(4, 8)
    KVQ_CASE(8, 2) KVQ_CASE(8, 4) KVQ_CASE(8, 8)
  }
#undef KVQ_CASE
  *used = false;
  return hipSuccess;
}

}  // namespace

hipError_t launch_decode_fast(const LayerDesc& L, const DecodeJob& j, hipStream_t s, bool* used) {
  *used = false;
  if (L.nuq || L.outk || L.pre_rope || (L.k_hybrid && !L.k_inner)) return hipSuccess;
  if (L.k_inner && L.k_group != 64) return hipSuccess;
  if (L.v_group != 32) return hipSuccess;
  switch (L.G) {
    case 1: return L.k_inner ? by_bits<1, true>(L, j, s, used) : by_bits<1, false>(L, j, s, used);
    case 4: return L.k_inner ? by_bits<4, true>(L, j, s, used) : by_bits<4, false>(L, j, s, used);
    case 8: return L.k_inner ? by_bits<8, true>(L, j, s, used) : by_bits<8, false>(L, j, s, used);
    default: return hipSuccess;
  }
}

}  // namespace kvq
