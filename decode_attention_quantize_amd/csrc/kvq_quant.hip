// kvq_quant.hip -- quantize/pack kernels (prefill blocks, window flushes,
// per-token appends) and the fp16 sink/window copy.
//
// Arithmetic per group (no contraction, IEEE division, round-half-even):
//   asymmetric (KVTuner review obs. 2; RateQuant sec. 3; InnerQ method 2):
//     s = fp16(fp32(max-min)/Q), z = min, code = clamp(rne(fp32(x-z)/s), 0, Q)
//   symmetric (InnerQ method 2): s = fp16(fp32(max|x|)/(2^(b-1)-1)),
//     code = clamp(rne(x/s), -Qs, Qs) + 2^(b-1), sign bit of s set
//   hybrid choice: symmetric iff den*|sum x| <= num*g*(max-min), on exact
//     int64 sums of fp16 values in units of 2^-24
//   codebook (KVQuant iii): s = fp16(max-min), z = min, code = number of level
//     midpoints strictly below fp32(x-z)/s
//   sparse outliers (KVQuant iv): top-k |x| of each token row, lower column
//     first on ties, excluded from the group statistics
//   Hadamard values (aitrends.kr page): v' = fp16(fl64(H v) * 1/sqrt(D)) with
//     exact binary64 butterflies
//   mixed 4/8-bit inner key groups (InnerQ, limitations and future work): per
//     token, the k_hi groups with the largest 4-bit step (fp16 scale
//     magnitude, the lower group first on ties) keep an 8-bit quantization
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"

#pragma clang fp contract(off)

namespace kvq {
namespace {

constexpr int D = kHeadDim;

// 48 KiB: the fp64 Hadamard rows are dead before codes and masks are written.
struct QuantSmem {
  uint16_t k[kBlockTokens][D];
  uint16_t v[kBlockTokens][D];
  union {
    double had[kBlockTokens][D];
    struct {
      uint8_t ck[kBlockTokens][D];
      uint8_t cv[kBlockTokens][D];
      uint8_t exk[kBlockTokens][D];
      uint8_t exv[kBlockTokens][D];
      // mixed 4/8-bit key groups: 8-bit codes, then their low nibbles; the
      // (s4, z4, s8, z8) of every (token, group); the per-token group masks
      uint8_t lok[kBlockTokens][D];
      uint16_t gm[kBlockTokens][D / 16][4];
      uint8_t sel[kBlockTokens];
    };
  };
};

__device__ __forceinline__ void asym_params(float mn, float mx, bool any, int Q, uint16_t& s,
                                            uint16_t& z) {
  if (!any) {
    s = 0;
    z = 0;
    return;
  }
  const float range = __fsub_rn(mx, mn);
  s = f2h(__fdiv_rn(range, static_cast<float>(Q)));
  if (mx > mn && s == 0) s = 1;
  z = f2h(mn);
}

__device__ __forceinline__ int asym_code(float x, float mn, uint16_t s, int Q) {
  if (s == 0) return 0;
  const float t = __fdiv_rn(__fsub_rn(x, mn), h2f(s));
  const float r = fminf(fmaxf(rintf(t), 0.f), static_cast<float>(Q));
  return static_cast<int>(r);
}

__device__ __forceinline__ uint16_t sym_scale(float a, int bits) {
  const int Qs = (1 << (bits - 1)) - 1;
  uint16_t s = f2h(__fdiv_rn(a, static_cast<float>(Qs)));
  if (a > 0.f && s == 0) s = 1;
  return s;
}

__device__ __forceinline__ int sym_code(float x, uint16_t s, int bits) {
  if (s == 0) return 0;
  const int Qs = (1 << (bits - 1)) - 1;
  const float r = fminf(fmaxf(rintf(__fdiv_rn(x, h2f(s))), static_cast<float>(-Qs)),
                        static_cast<float>(Qs));
  return static_cast<int>(r) + (1 << (bits - 1));
}

__device__ __forceinline__ void nuq_params(float mn, float mx, bool any, uint16_t& s, uint16_t& z) {
  if (!any) {
    s = 0;
    z = 0;
    return;
  }
  s = f2h(__fsub_rn(mx, mn));
  if (s == 0x7c00) s = 0x7bff;
  if (mx > mn && s == 0) s = 1;
  z = f2h(mn);
}

__device__ __forceinline__ int nuq_code(float x, float mn, uint16_t s, const uint16_t* lev) {
  if (s == 0) return 0;
  const float u = __fdiv_rn(__fsub_rn(x, mn), h2f(s));
  int c = 0;
#pragma unroll
  for (int j = 0; j < 7; ++j) {
    const float mid = __fmul_rn(__fadd_rn(h2f(lev[j]), h2f(lev[j + 1])), 0.5f);
    c += u > mid ? 1 : 0;
  }
  return c;
}

// Exact fp64 fast Walsh-Hadamard transform of `rows` rows held in had[][],
// then v' = fp16(fl64(S * c)).  All 128 threads cooperate.
__device__ void hadamard_rows(QuantSmem& sm, uint16_t (*vrows)[D], int rows, double c) {
  const int t = threadIdx.x;
  for (int j = 0; j < rows; ++j) sm.had[j][t] = static_cast<double>(h2f(vrows[j][t]));
  __syncthreads();
  for (int h = 1; h < D; h <<= 1) {
    // rows*D/2 butterflies, 128 threads
    for (int i = t; i < rows * (D / 2); i += blockDim.x) {
      const int j = i / (D / 2);
      const int p = i % (D / 2);
      const int lo = ((p / h) * 2 * h) + (p % h);
      const double a = sm.had[j][lo];
      const double b = sm.had[j][lo + h];
      sm.had[j][lo] = a + b;
      sm.had[j][lo + h] = a - b;
    }
    __syncthreads();
  }
  for (int j = 0; j < rows; ++j) vrows[j][t] = d2h(sm.had[j][t] * c);
  __syncthreads();
}

// top-k columns of each row by |x|, lower column first on equal magnitude.
__device__ void mark_outliers(const uint16_t (*rows)[D], uint8_t (*ex)[D], int nrows, int k,
                              uint8_t* out_base, int slot0) {
  const int t = threadIdx.x;
  for (int j = 0; j < nrows; ++j) ex[j][t] = 0;
  __syncthreads();
  if (t < nrows) {
    int chosen[kMaxOutliers];
    for (int i = 0; i < k; ++i) {
      int best = -1;
      uint16_t bm = 0;
      for (int c = 0; c < D; ++c) {
        if (ex[t][c]) continue;
        const uint16_t m = rows[t][c] & 0x7fff;
        if (best < 0 || m > bm) {
          best = c;
          bm = m;
        }
      }
      ex[t][best] = 1;
      chosen[i] = best;
    }
    // ascending column order
    for (int a = 1; a < k; ++a)
      for (int b = a; b > 0 && chosen[b] < chosen[b - 1]; --b) {
        const int tmp = chosen[b];
        chosen[b] = chosen[b - 1];
        chosen[b - 1] = tmp;
      }
    uint32_t* rec = reinterpret_cast<uint32_t*>(out_base) + (slot0 + t) * k;
    for (int i = 0; i < k; ++i)
      rec[i] = static_cast<uint32_t>(chosen[i]) | (static_cast<uint32_t>(rows[t][chosen[i]]) << 16);
  }
  __syncthreads();
}

// Quantize one token's per-token group (v_group or inner key group) with the
// lanes of the group cooperating through xor shuffles.
template <int W>
__device__ __forceinline__ void token_group(uint16_t xh, bool excluded, int bits, bool nuq,
                                            const uint16_t* lev, bool hybrid, int rnum, int rden,
                                            bool tern, int& code, uint16_t& s, uint16_t& z) {
  const float x = h2f(xh);
  if (tern) {
    // ternary levels {-s, 0, s}, s = max |x| over the non-outlier members (an
    // fp16 value); 2-bit code clamp(rne(x / s), -1, 1) + 1 with z = -s
    const float a = group_max<W>(excluded ? 0.f : fabsf(x));
    s = f2h(a);
    z = static_cast<uint16_t>(s ^ 0x8000u);
    code = s == 0 ? 1 : static_cast<int>(fminf(fmaxf(rintf(x / h2f(s)), -1.f), 1.f)) + 1;
    return;
  }
  float mn = excluded ? __int_as_float(0x7f800000) : x;
  float mx = excluded ? __int_as_float(0xff800000) : x;
  group_minmax<W>(mn, mx);
  const bool any = mn <= mx;
  bool sym = false;
  if (hybrid) {
    const int64_t fx = h2fixed(xh);
    const int64_t sum = group_sum64<W>(fx);
    int64_t fmn = fx, fmx = fx;
    // exact integer extremes
    {
      float a = x, b = x;
      group_minmax<W>(a, b);
      fmn = h2fixed(f2h(a));
      fmx = h2fixed(f2h(b));
    }
    const int64_t lhs = static_cast<int64_t>(rden) * (sum < 0 ? -sum : sum);
    const int64_t rhs = static_cast<int64_t>(rnum) * W * (fmx - fmn);
    sym = lhs <= rhs;
  }
  if (sym) {
    const float a = group_max<W>(fabsf(x));
    const uint16_t sv = sym_scale(a, bits);
    code = sym_code(x, sv, bits);
    s = sv | 0x8000;
    z = 0;
  } else if (nuq) {
    nuq_params(mn, mx, any, s, z);
    code = nuq_code(x, mn, s, lev);
  } else {
    asym_params(mn, mx, any, (1 << bits) - 1, s, z);
    code = asym_code(x, mn, s, (1 << bits) - 1);
  }
}

template <int W>
__device__ void quant_token_groups(const uint16_t (*rows)[D], const uint8_t (*ex)[D],
                                   uint8_t (*codes)[D], int nrows, int bits, bool nuq,
                                   const uint16_t* lev, bool hybrid, int rnum, int rden, bool tern,
                                   uint8_t* meta_base, int meta_kind, int slot0) {
  // meta_kind 0: inner keys [32][D/W] (s,z) pairs; 1: values s[D/W][32], z[D/W][32]
  const int t = threadIdx.x;
  const int g = t / W;
  const int ng = D / W;
  uint16_t* m16 = reinterpret_cast<uint16_t*>(meta_base);
  for (int j = 0; j < nrows; ++j) {
    int code;
    uint16_t s, z;
    token_group<W>(rows[j][t], ex ? ex[j][t] != 0 : false, bits, nuq, lev, hybrid, rnum, rden, tern,
                   code, s, z);
    codes[j][t] = static_cast<uint8_t>(code);
    if ((t % W) == 0) {
      const int slot = slot0 + j;
      if (meta_kind == 0) {
        m16[(slot * ng + g) * 2 + 0] = s;
        m16[(slot * ng + g) * 2 + 1] = z;
      } else {
        m16[g * kBlockTokens + slot] = s;
        m16[ng * kBlockTokens + g * kBlockTokens + slot] = z;
      }
    }
  }
}

__device__ void quant_groups_any(int w, const uint16_t (*rows)[D], const uint8_t (*ex)[D],
                                 uint8_t (*codes)[D], int nrows, int bits, bool nuq,
                                 const uint16_t* lev, bool hybrid, int rnum, int rden, bool tern,
                                 uint8_t* meta, int kind, int slot0) {
  switch (w) {
    case 16:
      quant_token_groups<16>(rows, ex, codes, nrows, bits, nuq, lev, hybrid, rnum, rden, tern, meta,
                             kind, slot0);
      break;
    case 32:
      quant_token_groups<32>(rows, ex, codes, nrows, bits, nuq, lev, hybrid, rnum, rden, tern, meta,
                             kind, slot0);
      break;
    default:
      quant_token_groups<64>(rows, ex, codes, nrows, bits, nuq, lev, hybrid, rnum, rden, tern, meta,
                             kind, slot0);
      break;
  }
}

// Mixed 4/8-bit inner key groups.  Every group of a row is quantized at 4 and
// at 8 bits; the k_hi groups whose 4-bit step ranks highest (ties: lower
// group first) keep the 8-bit result: its high nibble goes to the 4-bit code
// plane (ck), its low nibble to lok, its parameters to k_meta, and the
// token's group mask to k_sel.
template <int W>
__device__ void quant_mixed_groups(QuantSmem& sm, int nrows, const LayerDesc& L, uint8_t* rec, int slot0) {
  constexpr int ng = D / W;
  const int t = threadIdx.x, g = t / W;
  const bool hyb = L.k_hybrid != 0;
  for (int j = 0; j < nrows; ++j) {
    int c4, c8;
    uint16_t s4, z4, s8, z8;
    token_group<W>(sm.k[j][t], false, 4, false, nullptr, hyb, L.ratio_num, L.ratio_den, false, c4, s4, z4);
    token_group<W>(sm.k[j][t], false, 8, false, nullptr, hyb, L.ratio_num, L.ratio_den, false, c8, s8, z8);
    sm.ck[j][t] = static_cast<uint8_t>(c4);
    sm.lok[j][t] = static_cast<uint8_t>(c8);
    if (t % W == 0) {
      sm.gm[j][g][0] = s4;
      sm.gm[j][g][1] = z4;
      sm.gm[j][g][2] = s8;
      sm.gm[j][g][3] = z8;
    }
  }
  __syncthreads();
  uint16_t* m16 = reinterpret_cast<uint16_t*>(rec + L.off_km);
  for (int j = 0; j < nrows; ++j) {
    uint32_t sel = 0;
    for (int a = 0; a < ng; ++a) {
      const uint16_t sa = sm.gm[j][a][0] & 0x7fff;
      int rank = 0;
      for (int b = 0; b < ng; ++b) {
        const uint16_t sb = sm.gm[j][b][0] & 0x7fff;
        rank += (sb > sa || (sb == sa && b < a)) ? 1 : 0;
      }
      if (rank < L.k_hi) sel |= 1u << a;
    }
    const bool hi = ((sel >> g) & 1u) != 0;
    const int c8 = sm.lok[j][t];
    if (hi) sm.ck[j][t] = static_cast<uint8_t>(c8 >> 4);
    sm.lok[j][t] = hi ? static_cast<uint8_t>(c8 & 15) : 0;
    if (t % W == 0) {
      m16[((slot0 + j) * ng + g) * 2 + 0] = sm.gm[j][g][hi ? 2 : 0];
      m16[((slot0 + j) * ng + g) * 2 + 1] = sm.gm[j][g][hi ? 3 : 1];
    }
    if (t == 0) {
      sm.sel[j] = static_cast<uint8_t>(sel);
      rec[L.off_ks + slot0 + j] = static_cast<uint8_t>(sel);
    }
  }
}

// Low nibbles of each row's 8-bit key groups into k_ext: slot i of a token is
// its i-th 8-bit group in ascending order, k_group/8 pair-split words.
__device__ void pack_mixed_ext(const QuantSmem& sm, int nrows, const LayerDesc& L, uint8_t* rec, int slot0) {
  const int wps = L.k_group / 8;
  const int per_row = L.k_hi * wps;
  uint32_t* dst = reinterpret_cast<uint32_t*>(rec + L.off_kx);
  for (int i = threadIdx.x; i < nrows * per_row; i += blockDim.x) {
    const int j = i / per_row, r = i % per_row, k = r / wps, w = r % wps;
    uint32_t sel = sm.sel[j];
    for (int d = 0; d < k; ++d) sel &= sel - 1u;  // drop the k lowest groups
    const int g = __ffs(static_cast<int>(sel)) - 1;
    uint32_t word = 0;
    for (int e = 0; e < 8; ++e)
      word |= static_cast<uint32_t>(sm.lok[j][g * L.k_group + 8 * w + e]) << pair_split_pos(4, e);
    dst[((slot0 + j) * L.k_hi + k) * wps + w] = word;
  }
}

// Pack token-major 2/4/8-bit key rows for slots [slot0, slot0+nrows).
__device__ void pack_rows(const uint8_t (*codes)[D], int nrows, int bits, uint8_t* dst, int row_bytes,
                          int slot0) {
  const int wpr = row_bytes / 4;
  for (int i = threadIdx.x; i < nrows * wpr; i += blockDim.x) {
    const int j = i / wpr;
    const int w = i % wpr;
    uint32_t word = 0;
    if (bits == 8) {
      for (int e = 0; e < 4; ++e) word |= static_cast<uint32_t>(codes[j][4 * w + e]) << (8 * e);
    } else {
      const int n = 32 / bits;
      for (int e = 0; e < n; ++e)
        word |= static_cast<uint32_t>(codes[j][n * w + e]) << pair_split_pos(bits, e);
    }
    reinterpret_cast<uint32_t*>(dst + (slot0 + j) * row_bytes)[w] = word;
  }
}

// 3-bit codes: 64 lane chunks of 6 words, element E at bits 3E..3E+2 of the
// chunk's bit stream (see the decode readers for the element maps).
// Bits of 3-bit element e that fall into 32-bit word w of a stream.
__device__ __forceinline__ uint32_t bits3_in_word(uint32_t code, int e, int w) {
  const int sh = 3 * e - 32 * w;
  if (sh <= -3 || sh >= 32) return 0u;
  return sh >= 0 ? code << sh : code >> -sh;
}

// Pack 3-bit codes into 64 lane chunks of six words; map(lane, e) gives the
// (token slot, channel) of element e.  A fresh block (slot0 == 0) is written
// whole (elements of slots >= nrows get code 0); otherwise only the bits of
// slots [slot0, slot0 + nrows) are replaced.
template <class Map>
__device__ void pack3(const uint8_t (*codes)[D], int nrows, uint8_t* dst, int slot0, Map map) {
  for (int i = threadIdx.x; i < 64 * 6; i += blockDim.x) {
    const int lane = i / 6, w = i % 6;
    uint32_t word = 0, keep = 0xffffffffu;
    for (int e = (32 * w) / 3; e <= (32 * w + 31) / 3 && e < 64; ++e) {
      int j, c;
      map(lane, e, j, c);
      if (j >= slot0 && j < slot0 + nrows) {
        word |= bits3_in_word(codes[j - slot0][c], e, w);
        keep &= ~bits3_in_word(7u, e, w);
      }
    }
    uint32_t* wp = reinterpret_cast<uint32_t*>(dst) + i;
    if (slot0 == 0)
      *wp = word;
    else if (keep != 0xffffffffu)
      *wp = (*wp & keep) | word;
  }
}
// Keys: chunk l holds RoPE pair (l, l + 64); element 2t + e is token t of
// channel l + 64e, so a token's two codes form one 6-bit field.
__device__ void pack_k3(const uint8_t (*codes)[D], int nrows, uint8_t* dst, int slot0) {
  pack3(codes, nrows, dst, slot0, [](int lane, int e, int& j, int& c) {
    j = e >> 1;
    c = lane + 64 * (e & 1);
  });
}
// Values: chunk 16g + n, element 8t + i = token 8g + i of channel 16t + n.
__device__ void pack_v3(const uint8_t (*codes)[D], int nrows, uint8_t* dst, int slot0) {
  pack3(codes, nrows, dst, slot0, [](int lane, int e, int& j, int& c) {
    j = 8 * (lane >> 4) + (e & 7);
    c = 16 * (e >> 3) + (lane & 15);
  });
}

// Pack values into the lane-chunk layout.  A fresh block (slot0 == 0) is
// written whole (slots >= nrows get code 0); otherwise only the bits of slots
// [slot0, slot0+nrows) are replaced.
__device__ void pack_vchunks(const uint8_t (*codes)[D], int nrows, int bits, uint8_t* dst,
                             int slot0) {
  const int words = 64 * 2 * bits;
  const int n = bits == 8 ? 4 : 32 / bits;
  const uint32_t fmask = (1u << bits) - 1;
  for (int i = threadIdx.x; i < words; i += blockDim.x) {
    const int lane = i / (2 * bits);
    const int wi = i % (2 * bits);
    uint32_t word = 0, keep = 0xffffffffu;
    for (int e = 0; e < n; ++e) {
      const int idx = wi * n + e;
      const int j = 8 * (lane >> 4) + (idx & 7);  // token slot
      const int c = 16 * (idx >> 3) + (lane & 15);
      const int pos = bits == 8 ? 8 * e : pair_split_pos(bits, e);
      if (j >= slot0 && j < slot0 + nrows) {
        word |= static_cast<uint32_t>(codes[j - slot0][c]) << pos;
        keep &= ~(fmask << pos);
      }
    }
    uint32_t* wp = reinterpret_cast<uint32_t*>(dst) + i;
    if (slot0 == 0)
      *wp = word;
    else if (keep != 0xffffffffu)
      *wp = (*wp & keep) | word;
  }
}

// A fresh block filled only up to nrows tokens: the per-token sections of the
// slots past them (key code rows, inner key parameters, value parameters,
// sparse outliers, mixed-group low nibbles and masks) are zeroed, so that
// the record holds no bytes the buffer had before.  The decode weighs those
// slots by exactly 0, and 0 times a stale non-finite parameter would not be 0.
// Value codes and 3-bit key chunks are written whole for a fresh block.
__device__ void zero_record_tail(const LayerDesc& L, uint8_t* rec, int nrows) {
  const int t = threadIdx.x, nt = blockDim.x;
  const int rest = kBlockTokens - nrows;
  if (L.kb != 3) {
    uint32_t* w = reinterpret_cast<uint32_t*>(rec + L.off_kc + nrows * L.k_row_bytes);
    for (int i = t; i < rest * L.k_row_bytes / 4; i += nt) w[i] = 0u;
  }
  if (L.k_inner) {
    const int ng = D / L.k_group;  // one (s, z) pair per group and token
    uint32_t* w = reinterpret_cast<uint32_t*>(rec + L.off_km) + nrows * ng;
    for (int i = t; i < rest * ng; i += nt) w[i] = 0u;
  }
  {
    const int rows = 2 * (D / L.v_group);  // s[g][32] then z[g][32]
    uint16_t* m = reinterpret_cast<uint16_t*>(rec + L.off_vm);
    for (int i = t; i < rows * rest; i += nt) m[(i / rest) * kBlockTokens + nrows + i % rest] = 0;
  }
  if (L.outk) {
    uint32_t* ko = reinterpret_cast<uint32_t*>(rec + L.off_ko) + nrows * L.outk;
    uint32_t* vo = reinterpret_cast<uint32_t*>(rec + L.off_vo) + nrows * L.outk;
    for (int i = t; i < rest * L.outk; i += nt) {
      ko[i] = 0u;
      vo[i] = 0u;
    }
  }
  if (L.k_hi) {
    const int wpt = L.k_hi * (L.k_group / 8);  // low-nibble words per token
    uint32_t* x = reinterpret_cast<uint32_t*>(rec + L.off_kx) + nrows * wpt;
    for (int i = t; i < rest * wpt; i += nt) x[i] = 0u;
    for (int i = t; i < rest; i += nt) rec[L.off_ks + nrows + i] = 0;
  }
}

__global__ void __launch_bounds__(128) quantize_kernel(LayerDesc L, QuantJob J) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  QuantSmem& sm = *reinterpret_cast<QuantSmem*>(smem_raw);
  const int t = threadIdx.x;
  const int u = blockIdx.y;
  const int bi = blockIdx.x;
  const int blk = J.blk0 + bi;
  const int nrows = (bi == J.nblocks - 1) ? J.last_cnt : J.cnt;
  const int slot0 = J.tok0;
  uint8_t* rec = L.body + (static_cast<int64_t>(u) * L.nblk_cap + blk) * L.rec_bytes;

  const int tt0 = J.src_t0 + kBlockTokens * bi;
  const int64_t base = u * J.src_unit_stride + static_cast<int64_t>(tt0) * D;
  const uint16_t* vsrc = J.v_src + u * J.src_unit_stride;
  if (slot0 == 0 && nrows < kBlockTokens) zero_record_tail(L, rec, nrows);
  for (int j = 0; j < kBlockTokens; ++j) {
    sm.k[j][t] = j < nrows ? J.k_src[base + j * D + t] : 0;
    const int64_t vo = J.v_interleaved ? vslot(tt0 + j, t) : static_cast<int64_t>(tt0 + j) * D + t;
    sm.v[j][t] = j < nrows ? vsrc[vo] : 0;
  }
  if (L.kshift) {
    // normalized keys fp16(K * 2^shift), saturating (InnerQ, method 4)
    const int sh = L.kshift[static_cast<int64_t>(u) * D + t];
    for (int j = 0; j < nrows; ++j)
      sm.k[j][t] = f2h(fminf(fmaxf(ldexpf(h2f(sm.k[j][t]), sh), -65504.f), 65504.f));
  }
  __syncthreads();
  if (J.rotate_v) hadamard_rows(sm, sm.v, nrows, L.had_scale);

  const bool out = L.outk > 0;
  if (out) {
    mark_outliers(sm.k, sm.exk, nrows, L.outk, rec + L.off_ko, slot0);
    mark_outliers(sm.v, sm.exv, nrows, L.outk, rec + L.off_vo, slot0);
  }

  // ---- keys
  if (!L.k_inner) {
    // one group per channel over the block's tokens: thread t owns channel t
    bool any = false;
    float mn = 0.f, mx = 0.f;
    for (int j = 0; j < nrows; ++j) {
      if (out && sm.exk[j][t]) continue;
      const float x = h2f(sm.k[j][t]);
      if (!any) {
        mn = mx = x;
        any = true;
      } else {
        mn = fminf(mn, x);
        mx = fmaxf(mx, x);
      }
    }
    uint16_t s, z;
    bool sym = false;
    if (L.k_hybrid) {
      int64_t sum = 0, fmn = 0, fmx = 0;
      for (int j = 0; j < nrows; ++j) {
        const int64_t f = h2fixed(sm.k[j][t]);
        sum += f;
        if (j == 0 || f < fmn) fmn = f;
        if (j == 0 || f > fmx) fmx = f;
      }
      sym = static_cast<int64_t>(L.ratio_den) * (sum < 0 ? -sum : sum) <=
            static_cast<int64_t>(L.ratio_num) * nrows * (fmx - fmn);
    }
    if (sym) {
      float a = 0.f;
      for (int j = 0; j < nrows; ++j) a = fmaxf(a, fabsf(h2f(sm.k[j][t])));
      const uint16_t sv = sym_scale(a, L.kb);
      for (int j = 0; j < nrows; ++j) sm.ck[j][t] = static_cast<uint8_t>(sym_code(h2f(sm.k[j][t]), sv, L.kb));
      s = sv | 0x8000;
      z = 0;
    } else if (L.nuq) {
      nuq_params(mn, mx, any, s, z);
      for (int j = 0; j < nrows; ++j)
        sm.ck[j][t] = static_cast<uint8_t>(nuq_code(h2f(sm.k[j][t]), mn, s, L.lev_k));
    } else {
      asym_params(mn, mx, any, (1 << L.kb) - 1, s, z);
      for (int j = 0; j < nrows; ++j)
        sm.ck[j][t] = static_cast<uint8_t>(asym_code(h2f(sm.k[j][t]), mn, s, (1 << L.kb) - 1));
    }
    for (int j = nrows; j < kBlockTokens; ++j) sm.ck[j][t] = 0;
    uint16_t* km = reinterpret_cast<uint16_t*>(rec + L.off_km);
    km[t] = s;
    km[D + t] = z;
  } else if (L.k_hi) {
    if (L.k_group == 16)
      quant_mixed_groups<16>(sm, nrows, L, rec, slot0);
    else if (L.k_group == 32)
      quant_mixed_groups<32>(sm, nrows, L, rec, slot0);
    else
      quant_mixed_groups<64>(sm, nrows, L, rec, slot0);
  } else {
    quant_groups_any(L.k_group, sm.k, out ? sm.exk : nullptr, sm.ck, nrows, L.kb, L.nuq != 0,
                     L.lev_k, L.k_hybrid != 0, L.ratio_num, L.ratio_den, false, rec + L.off_km, 0,
                     slot0);
  }
  // ---- values: per-token groups
  quant_groups_any(L.v_group, sm.v, out ? sm.exv : nullptr, sm.cv, nrows, L.vb, L.nuq != 0,
                   L.lev_v, false, 1, 1, L.v_tern != 0, rec + L.off_vm, 1, slot0);
  __syncthreads();

  if (L.kb == 3)
    pack_k3(sm.ck, nrows, rec + L.off_kc, slot0);
  else
    pack_rows(sm.ck, nrows, L.kb, rec + L.off_kc, L.k_row_bytes, slot0);
  if (L.k_hi) pack_mixed_ext(sm, nrows, L, rec, slot0);
  if (L.vb == 3)
    pack_v3(sm.cv, nrows, rec + L.off_vc, slot0);
  else
    pack_vchunks(sm.cv, nrows, L.vb, rec + L.off_vc, slot0);
}

// ===================================================================== fresh blocks
// prefill_kernel quantizes whole fresh blocks (slot 0 onward: prefill and
// window flushes) with the same arithmetic as quantize_kernel but organised
// for bandwidth: every thread issues its 16-byte loads of the block at once;
// each per-token group (values, inner key groups) is one thread's task with
// its statistics in registers (no per-row chains of cross-lane reductions);
// value codes are staged in the lane-chunk order of the record, so each
// packed word is one wide LDS read.  Mixed 4/8-bit key groups and appends
// into a partly filled block stay on quantize_kernel.

// binary64 -> binary16, round to nearest even, through binary32: x is first
// rounded to odd in binary32 (round to nearest, then, if inexact, toward
// zero with the last bit set), which keeps the information needed for the
// second rounding because binary32 carries 13 more fraction bits than
// binary16 (Boldo & Melquiond, "Emulation of FMA and correctly rounded sums:
// proved algorithms using rounding to odd", IEEE TC 2008).  Equal to d2h.
__device__ __forceinline__ uint16_t d2h_odd(double x) {
  const float r = static_cast<float>(x);
  const double back = static_cast<double>(r);
  uint32_t rb = __float_as_uint(r);
  if (back != x) {
    if (fabs(back) > fabs(x)) rb -= 1u;  // one binary32 step toward zero
    rb |= 1u;
  }
  return f2h(__uint_as_float(rb));
}

// Shared memory of prefill_kernel (dynamic size, offsets in bytes):
//   k16, v16 [32][D] fp16 | ck [32][D] key codes | cv value codes: [32][D]
//   (3-bit) or lane-chunk order [64 chunks][64 elements] | exk, exv [32][D]
//   outlier masks (layers with outliers).
constexpr int kPfK = 0, kPfV = 8192, kPfCk = 16384, kPfCv = 20480, kPfExk = 24576, kPfExv = 28672;
__host__ __device__ constexpr int prefill_smem(bool outk) { return outk ? 32768 : 24576; }

// Element of lane chunk l = 16 (j / 8) + (c % 16) that holds code (token j,
// channel c) of the value layout: e = 8 (c / 16) + j % 8.
__device__ __forceinline__ int vchunk_off(int j, int c) {
  return (16 * (j >> 3) + (c & 15)) * 64 + 8 * (c >> 4) + (j & 7);
}

// rne(fl32(a / b)) -- the correctly rounded quotient rounded to an integer --
// from a reciprocal estimate: t = a * rcp(b) lies within 1.5 * 2^-23 |a / b|
// of the exact quotient (v_rcp_f32 is accurate to 1 ulp), i.e. within 2^-13
// for the |a / b| <= 512 of every code formula here, while fl32(a / b) lies
// within 2^-15 of it.  Unless t is within 2^-10 of a rounding boundary
// k + 1/2, both therefore round to the same integer; near one, the quotient
// is recomputed with the correctly rounded division.
__device__ __forceinline__ float rint_quot(float a, float b) {
  const float t = a * __builtin_amdgcn_rcpf(b);
  const float r = rintf(t);
  if (fabsf(fabsf(t - r) - 0.5f) < 0x1p-10f) return rintf(__fdiv_rn(a, b));
  return r;
}
__device__ __forceinline__ int asym_code_fast(float x, float mn, uint16_t s, int Q) {
  if (s == 0) return 0;
  return static_cast<int>(fminf(fmaxf(rint_quot(__fsub_rn(x, mn), h2f(s)), 0.f), static_cast<float>(Q)));
}
__device__ __forceinline__ int sym_code_fast(float x, uint16_t s, int bits) {
  if (s == 0) return 0;
  const int Qs = (1 << (bits - 1)) - 1;
  const float r = fminf(fmaxf(rint_quot(x, h2f(s)), static_cast<float>(-Qs)), static_cast<float>(Qs));
  return static_cast<int>(r) + (1 << (bits - 1));
}
// Codebook codes: u = fl32((x - mn) / s) in [0, 1] against the seven level
// midpoints; the reciprocal estimate of u (within 2^-21 of it) decides unless
// it lies within 2^-18 of a midpoint.
__device__ __forceinline__ int nuq_code_fast(float x, float mn, uint16_t s, const float (&mid)[7]) {
  if (s == 0) return 0;
  const float d = __fsub_rn(x, mn), sv = h2f(s);
  float u = d * __builtin_amdgcn_rcpf(sv);
  bool near = false;
#pragma unroll
  for (int j = 0; j < 7; ++j) near |= fabsf(u - mid[j]) < 0x1p-18f;
  if (near) u = __fdiv_rn(d, sv);
  int c = 0;
#pragma unroll
  for (int j = 0; j < 7; ++j) c += u > mid[j] ? 1 : 0;
  return c;
}
__device__ __forceinline__ void nuq_mids(const uint16_t* lev, float (&mid)[7]) {
#pragma unroll
  for (int j = 0; j < 7; ++j) mid[j] = __fmul_rn(__fadd_rn(h2f(lev[j]), h2f(lev[j + 1])), 0.5f);
}

// One per-token group (W channels of one row) with its values in registers:
// the arithmetic of token_group, written per element instead of per lane.
// SPLIT lanes (adjacent, 1 or 2) share a group: each holds N = W / SPLIT of
// its channels and the statistics are joined across the pair.
template <int N, int SPLIT>
__device__ __forceinline__ void group_in_regs(const uint16_t (&xh)[N], uint64_t exm, int bits, bool nuq,
                                              const uint16_t* lev, bool hybrid, int rnum, int rden, bool tern,
                                              uint8_t (&code)[N], uint16_t& s, uint16_t& z) {
  constexpr int W = N * SPLIT;  // group size
  auto join_max = [](float v) __attribute__((always_inline)) { return SPLIT == 2 ? fmaxf(v, xshflf<1>(v)) : v; };
  auto join_min = [](float v) __attribute__((always_inline)) { return SPLIT == 2 ? fminf(v, xshflf<1>(v)) : v; };
  if (tern) {
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < N; ++i) a = fmaxf(a, ((exm >> i) & 1u) ? 0.f : fabsf(h2f(xh[i])));
    a = join_max(a);
    s = f2h(a);
    z = static_cast<uint16_t>(s ^ 0x8000u);
    const float sv = h2f(s);
#pragma unroll
    for (int i = 0; i < N; ++i)
      code[i] = static_cast<uint8_t>(s == 0 ? 1 : static_cast<int>(fminf(fmaxf(rint_quot(h2f(xh[i]), sv), -1.f), 1.f)) + 1);
    return;
  }
  float mn = __int_as_float(0x7f800000), mx = __int_as_float(0xff800000);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if ((exm >> i) & 1u) continue;
    const float x = h2f(xh[i]);
    mn = fminf(mn, x);
    mx = fmaxf(mx, x);
  }
  mn = join_min(mn);
  mx = join_max(mx);
  const bool any = mn <= mx;
  bool sym = false;
  if (hybrid) {
    // exact sum and extremes over every member, in units of 2^-24
    int64_t sum = 0;
    float amn = h2f(xh[0]), amx = amn;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      sum += h2fixed(xh[i]);
      const float x = h2f(xh[i]);
      amn = fminf(amn, x);
      amx = fmaxf(amx, x);
    }
    if constexpr (SPLIT == 2) sum += xshfl64<1>(sum);
    amn = join_min(amn);
    amx = join_max(amx);
    const int64_t lhs = static_cast<int64_t>(rden) * (sum < 0 ? -sum : sum);
    const int64_t rhs = static_cast<int64_t>(rnum) * W * (h2fixed(f2h(amx)) - h2fixed(f2h(amn)));
    sym = lhs <= rhs;
  }
  if (sym) {
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < N; ++i) a = fmaxf(a, fabsf(h2f(xh[i])));
    a = join_max(a);
    const uint16_t sv = sym_scale(a, bits);
#pragma unroll
    for (int i = 0; i < N; ++i) code[i] = static_cast<uint8_t>(sym_code_fast(h2f(xh[i]), sv, bits));
    s = sv | 0x8000;
    z = 0;
  } else if (nuq) {
    nuq_params(mn, mx, any, s, z);
    float mid[7];
    nuq_mids(lev, mid);
#pragma unroll
    for (int i = 0; i < N; ++i) code[i] = static_cast<uint8_t>(nuq_code_fast(h2f(xh[i]), mn, s, mid));
  } else {
    const int Q = (1 << bits) - 1;
    asym_params(mn, mx, any, Q, s, z);
#pragma unroll
    for (int i = 0; i < N; ++i) code[i] = static_cast<uint8_t>(asym_code_fast(h2f(xh[i]), mn, s, Q));
  }
}

// All per-token group tasks of one tensor of the block: task = (row j,
// group g, part h), N = W / SPLIT channels of the group; the SPLIT tasks of
// a group are adjacent lanes.  Codes go to LDS (keys and 3-bit values
// row-major, 2/4/8-bit values in lane-chunk order), parameters straight to
// the record.  Every lane of the block runs the same number of loop trips
// (the pair exchanges need both lanes of a pair active).
template <int W>
__device__ void group_tasks(const uint8_t* sm, int src_off, int ex_off, bool has_ex, int code_off, bool chunk_order,
                            int nrows, int bits, bool nuq, const uint16_t* lev, bool hybrid, int rnum, int rden,
                            bool tern, uint16_t* meta, int meta_kind) {
  constexpr int SPLIT = W == 64 ? 2 : 1;
  constexpr int N = W / SPLIT;
  constexpr int ng = D / W;
  const uint16_t* x16 = reinterpret_cast<const uint16_t*>(sm + src_off);
  uint8_t* codes = const_cast<uint8_t*>(sm) + code_off;
  const int ntask = nrows * ng * SPLIT;
  for (int t0 = 0; t0 < ntask; t0 += blockDim.x) {
    const int task = t0 + static_cast<int>(threadIdx.x);
    const bool live = task < ntask;  // a pair's two lanes are live together (ntask is a multiple of SPLIT)
    const int gt = live ? task / SPLIT : 0, part = task % SPLIT;
    const int j = gt / ng, g = gt % ng;
    const int c0 = g * W + part * N;  // first channel of this lane's part
    uint16_t xh[N];
    const uint4* xs = reinterpret_cast<const uint4*>(x16 + j * D + c0);
#pragma unroll
    for (int q = 0; q < N / 8; ++q) {
      const uint4 v = xs[q];
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xh[8 * q + 2 * e] = static_cast<uint16_t>(w4[e] & 0xffffu);
        xh[8 * q + 2 * e + 1] = static_cast<uint16_t>(w4[e] >> 16);
      }
    }
    uint64_t exm = 0;
    if (has_ex) {
      const uint8_t* ex = sm + ex_off + j * D + c0;
#pragma unroll
      for (int i = 0; i < N; ++i) exm |= static_cast<uint64_t>(ex[i] != 0) << i;
    }
    uint8_t code[N];
    uint16_t s, z;
    group_in_regs<N, SPLIT>(xh, exm, bits, nuq, lev, hybrid, rnum, rden, tern, code, s, z);
    if (!live) continue;
    if (chunk_order) {
#pragma unroll
      for (int i = 0; i < N; ++i) codes[vchunk_off(j, c0 + i)] = code[i];
    } else {
      uint32_t* dst = reinterpret_cast<uint32_t*>(codes + j * D + c0);
#pragma unroll
      for (int q = 0; q < N / 4; ++q)
        dst[q] = code[4 * q] | (code[4 * q + 1] << 8) | (code[4 * q + 2] << 16) | (static_cast<uint32_t>(code[4 * q + 3]) << 24);
    }
    if (part != 0) continue;
    if (meta_kind == 0) {  // inner keys: [32][ng] (s, z)
      reinterpret_cast<uint32_t*>(meta)[j * ng + g] = s | (static_cast<uint32_t>(z) << 16);
    } else {  // values: s[ng][32] then z[ng][32]
      meta[g * kBlockTokens + j] = s;
      meta[ng * kBlockTokens + g * kBlockTokens + j] = z;
    }
  }
}

// top-k columns of each token row by |x| (fp16 magnitudes, the lower column
// on equal magnitude), one thread per (tensor, row), a single pass keeping
// the k largest keys (magnitude << 7 | 127 - column); columns ascending in
// the record; the mask bytes mark them for the group statistics.
__device__ void outliers_tasks(uint8_t* sm, int nrows, int k, uint8_t* kout, uint8_t* vout) {
  for (int task = threadIdx.x; task < 2 * nrows; task += blockDim.x) {
    const int tsr = task / nrows, j = task % nrows;
    const uint16_t* row = reinterpret_cast<const uint16_t*>(sm + (tsr ? kPfV : kPfK)) + j * D;
    uint32_t top[kMaxOutliers];
#pragma unroll
    for (int i = 0; i < kMaxOutliers; ++i) top[i] = 0u;
    for (int c = 0; c < D; ++c) {
      uint32_t key = (static_cast<uint32_t>(row[c] & 0x7fffu) << 7) | static_cast<uint32_t>(127 - c);
      // keep top[0..k) sorted descending: bubble the new key in
#pragma unroll
      for (int i = 0; i < kMaxOutliers; ++i) {
        if (i < k && key > top[i]) {
          const uint32_t t = top[i];
          top[i] = key;
          key = t;
        }
      }
    }
    int col[kMaxOutliers];
#pragma unroll
    for (int i = 0; i < kMaxOutliers; ++i) col[i] = 127 - static_cast<int>(top[i] & 127u);
    for (int a = 1; a < k; ++a)
      for (int b = a; b > 0 && col[b] < col[b - 1]; --b) {
        const int t = col[b];
        col[b] = col[b - 1];
        col[b - 1] = t;
      }
    uint8_t* ex = sm + (tsr ? kPfExv : kPfExk) + j * D;
    uint32_t* rec = reinterpret_cast<uint32_t*>(tsr ? vout : kout) + j * k;
    for (int i = 0; i < k; ++i) {
      ex[col[i]] = 1;
      rec[i] = static_cast<uint32_t>(col[i]) | (static_cast<uint32_t>(row[col[i]]) << 16);
    }
  }
}

// Token-major key code rows (2/4/8 bits) from the row-major code tile: one
// thread per output word, reading its codes as one 4-, 8- or 16-byte word.
__device__ void pack_rows_fast(const uint8_t* ck, int nrows, int bits, uint8_t* dst, int row_bytes) {
  const int wpr = row_bytes / 4;
  for (int i = threadIdx.x; i < nrows * wpr; i += blockDim.x) {
    const int j = i / wpr, w = i % wpr;
    const uint8_t* src = ck + j * D;
    uint32_t word = 0;
    if (bits == 8) {
      word = reinterpret_cast<const uint32_t*>(src)[w];
    } else if (bits == 4) {
      const uint2 b = reinterpret_cast<const uint2*>(src)[w];  // elements 8w..8w+7
      const uint32_t bb[2] = {b.x, b.y};
#pragma unroll
      for (int e = 0; e < 8; ++e) word |= ((bb[e >> 2] >> (8 * (e & 3))) & 15u) << pair_split_pos(4, e);
    } else {
      const uint4 b = reinterpret_cast<const uint4*>(src)[w];  // elements 16w..16w+15
      const uint32_t bb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int e = 0; e < 16; ++e) word |= ((bb[e >> 2] >> (8 * (e & 3))) & 3u) << pair_split_pos(2, e);
    }
    reinterpret_cast<uint32_t*>(dst + j * row_bytes)[w] = word;
  }
}

// Value lane chunks (2/4/8 bits) from the chunk-order code tile: word wi of
// chunk l holds its elements n wi .. n wi + n - 1 (n = 32 / bits), pair-split.
__device__ void pack_vchunks_fast(const uint8_t* cvc, int bits, uint8_t* dst) {
  const int wpc = 2 * bits;  // words per chunk
  for (int i = threadIdx.x; i < 64 * wpc; i += blockDim.x) {
    const int l = i / wpc, w = i % wpc;
    const uint8_t* src = cvc + l * 64;
    uint32_t word = 0;
    if (bits == 8) {
      word = reinterpret_cast<const uint32_t*>(src)[w];
    } else if (bits == 4) {
      const uint2 b = reinterpret_cast<const uint2*>(src)[w];
      const uint32_t bb[2] = {b.x, b.y};
#pragma unroll
      for (int e = 0; e < 8; ++e) word |= ((bb[e >> 2] >> (8 * (e & 3))) & 15u) << pair_split_pos(4, e);
    } else {
      const uint4 b = reinterpret_cast<const uint4*>(src)[w];
      const uint32_t bb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int e = 0; e < 16; ++e) word |= ((bb[e >> 2] >> (8 * (e & 3))) & 3u) << pair_split_pos(2, e);
    }
    reinterpret_cast<uint32_t*>(dst)[i] = word;
  }
}

// Exact fp64 Walsh-Hadamard transform of the value rows in place (fp16 in,
// fp16(fl64(S * c)) out): sixteen lanes per row, eight channels per lane
// (channel 8 cc + i), eight rows per pass.  Butterflies over channel bits
// 0-2 stay in the lane, over bits 3-6 they pair lanes cc and cc ^ m through
// two 32-bit swizzles per binary64 value.  Partial sums of fp16 inputs are
// exact in binary64, so the order of the stages does not matter.  Rows past
// the block's tokens hold zeros and stay zero.
__device__ void hadamard_rows_fast(uint8_t* sm, double c) {
  uint16_t* v16 = reinterpret_cast<uint16_t*>(sm + kPfV);
  const int t = threadIdx.x, cc = t & 15;
  for (int r0 = 0; r0 < kBlockTokens; r0 += 8) {
    const int j = r0 + (t >> 4);
    uint4* row = reinterpret_cast<uint4*>(v16 + j * D) + cc;
    const uint4 w = *row;
    const uint32_t w4[4] = {w.x, w.y, w.z, w.w};
    double x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = static_cast<double>(h2f(static_cast<uint16_t>(w4[e] & 0xffffu)));
      x[2 * e + 1] = static_cast<double>(h2f(static_cast<uint16_t>(w4[e] >> 16)));
    }
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (!(i & h)) {
          const double a = x[i], b = x[i + h];
          x[i] = a + b;
          x[i + h] = a - b;
        }
    auto xor_lanes = [&](auto mc) __attribute__((always_inline)) {
      constexpr int M = decltype(mc)::value;
      const bool hi = (cc & M) != 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t bits = __double_as_longlong(x[i]);
        const double o = __longlong_as_double(xshfl64<M>(bits));
        x[i] = hi ? o - x[i] : x[i] + o;
      }
    };
    xor_lanes(std::integral_constant<int, 1>{});
    xor_lanes(std::integral_constant<int, 2>{});
    xor_lanes(std::integral_constant<int, 4>{});
    xor_lanes(std::integral_constant<int, 8>{});
    uint32_t o4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o4[e] = static_cast<uint32_t>(d2h_odd(x[2 * e] * c)) | (static_cast<uint32_t>(d2h_odd(x[2 * e + 1] * c)) << 16);
    *row = make_uint4(o4[0], o4[1], o4[2], o4[3]);
  }
  __syncthreads();
}

__global__ void __launch_bounds__(128) prefill_kernel(LayerDesc L, QuantJob J) {
  extern __shared__ __align__(16) uint8_t sm[];
  const int t = threadIdx.x;
  const int u = blockIdx.y;
  const int bi = blockIdx.x;
  const int blk = J.blk0 + bi;
  const int nrows = (bi == J.nblocks - 1) ? J.last_cnt : J.cnt;
  uint8_t* rec = L.body + (static_cast<int64_t>(u) * L.nblk_cap + blk) * L.rec_bytes;
  uint16_t* k16 = reinterpret_cast<uint16_t*>(sm + kPfK);
  uint16_t* v16 = reinterpret_cast<uint16_t*>(sm + kPfV);
  const bool outk = L.outk > 0;
  const bool chunk_v = L.vb != 3;

  // ---- loads: 32 rows x 16 chunks of 16 bytes per tensor; thread t takes
  // chunk t % 16 of rows t / 16 + 8 i, every load issued before the first use
  const int tt0 = J.src_t0 + kBlockTokens * bi;
  {
    const uint16_t* ksrc = J.k_src + u * J.src_unit_stride + static_cast<int64_t>(tt0) * D;
    uint4 kv[4], vv[4];
    const int cc = t & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = (t >> 4) + 8 * i;
      kv[i] = j < nrows ? reinterpret_cast<const uint4*>(ksrc + j * D)[cc] : make_uint4(0u, 0u, 0u, 0u);
    }
    if (!J.v_interleaved) {
      const uint16_t* vsrc = J.v_src + u * J.src_unit_stride + static_cast<int64_t>(tt0) * D;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = (t >> 4) + 8 * i;
        vv[i] = j < nrows ? reinterpret_cast<const uint4*>(vsrc + j * D)[cc] : make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = (t >> 4) + 8 * i;
      reinterpret_cast<uint4*>(k16 + j * D)[cc] = kv[i];
      if (!J.v_interleaved) reinterpret_cast<uint4*>(v16 + j * D)[cc] = vv[i];
    }
    if (J.v_interleaved) {  // a window flush: values in the fp16 ring's 8-slot interleaved layout
      const uint16_t* vsrc = J.v_src + u * J.src_unit_stride;
      for (int j = 0; j < kBlockTokens; ++j) v16[j * D + t] = j < nrows ? vsrc[vslot(tt0 + j, t)] : 0;
    }
  }
  if (nrows < kBlockTokens) zero_record_tail(L, rec, nrows);
  __syncthreads();
  if (L.kshift) {
    // normalized keys fp16(K * 2^shift), saturating (InnerQ, method 4)
    const int sh = L.kshift[static_cast<int64_t>(u) * D + t];
    for (int j = 0; j < nrows; ++j)
      k16[j * D + t] = f2h(fminf(fmaxf(ldexpf(h2f(k16[j * D + t]), sh), -65504.f), 65504.f));
    __syncthreads();
  }
  if (J.rotate_v) hadamard_rows_fast(sm, L.had_scale);

  // ---- code tiles start at zero (rows past nrows pack as code 0)
  {
    uint4* z = reinterpret_cast<uint4*>(sm + kPfCk);
    const int n16 = (outk ? 16384 : 8192) / 16;
    for (int i = t; i < n16; i += blockDim.x) z[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();
  if (outk) {
    outliers_tasks(sm, nrows, L.outk, rec + L.off_ko, rec + L.off_vo);
    __syncthreads();
  }

  // ---- keys
  if (!L.k_inner) {
    // one group per channel over the block's tokens: thread t owns channel t
    const uint8_t* exk = sm + kPfExk;
    uint8_t* ck = sm + kPfCk;
    bool any = false;
    float mn = 0.f, mx = 0.f;
    for (int j = 0; j < nrows; ++j) {
      if (outk && exk[j * D + t]) continue;
      const float x = h2f(k16[j * D + t]);
      if (!any) {
        mn = mx = x;
        any = true;
      } else {
        mn = fminf(mn, x);
        mx = fmaxf(mx, x);
      }
    }
    uint16_t s, z;
    bool sym = false;
    if (L.k_hybrid) {
      int64_t sum = 0, fmn = 0, fmx = 0;
      for (int j = 0; j < nrows; ++j) {
        const int64_t f = h2fixed(k16[j * D + t]);
        sum += f;
        if (j == 0 || f < fmn) fmn = f;
        if (j == 0 || f > fmx) fmx = f;
      }
      sym = static_cast<int64_t>(L.ratio_den) * (sum < 0 ? -sum : sum) <=
            static_cast<int64_t>(L.ratio_num) * nrows * (fmx - fmn);
    }
    if (sym) {
      float a = 0.f;
      for (int j = 0; j < nrows; ++j) a = fmaxf(a, fabsf(h2f(k16[j * D + t])));
      const uint16_t sv = sym_scale(a, L.kb);
      for (int j = 0; j < nrows; ++j) ck[j * D + t] = static_cast<uint8_t>(sym_code_fast(h2f(k16[j * D + t]), sv, L.kb));
      s = sv | 0x8000;
      z = 0;
    } else if (L.nuq) {
      nuq_params(mn, mx, any, s, z);
      float mid[7];
      nuq_mids(L.lev_k, mid);
      for (int j = 0; j < nrows; ++j) ck[j * D + t] = static_cast<uint8_t>(nuq_code_fast(h2f(k16[j * D + t]), mn, s, mid));
    } else {
      const int Q = (1 << L.kb) - 1;
      asym_params(mn, mx, any, Q, s, z);
      for (int j = 0; j < nrows; ++j) ck[j * D + t] = static_cast<uint8_t>(asym_code_fast(h2f(k16[j * D + t]), mn, s, Q));
    }
    uint16_t* km = reinterpret_cast<uint16_t*>(rec + L.off_km);
    km[t] = s;
    km[D + t] = z;
  } else {
    uint16_t* km = reinterpret_cast<uint16_t*>(rec + L.off_km);
    const bool hy = L.k_hybrid != 0;
    if (L.k_group == 16)
      group_tasks<16>(sm, kPfK, kPfExk, outk, kPfCk, false, nrows, L.kb, L.nuq != 0, L.lev_k, hy, L.ratio_num, L.ratio_den, false, km, 0);
    else if (L.k_group == 32)
      group_tasks<32>(sm, kPfK, kPfExk, outk, kPfCk, false, nrows, L.kb, L.nuq != 0, L.lev_k, hy, L.ratio_num, L.ratio_den, false, km, 0);
    else
      group_tasks<64>(sm, kPfK, kPfExk, outk, kPfCk, false, nrows, L.kb, L.nuq != 0, L.lev_k, hy, L.ratio_num, L.ratio_den, false, km, 0);
  }
  // ---- values: per-token groups
  {
    uint16_t* vm = reinterpret_cast<uint16_t*>(rec + L.off_vm);
    const bool tern = L.v_tern != 0;
    if (L.v_group == 16)
      group_tasks<16>(sm, kPfV, kPfExv, outk, kPfCv, chunk_v, nrows, L.vb, L.nuq != 0, L.lev_v, false, 1, 1, tern, vm, 1);
    else if (L.v_group == 32)
      group_tasks<32>(sm, kPfV, kPfExv, outk, kPfCv, chunk_v, nrows, L.vb, L.nuq != 0, L.lev_v, false, 1, 1, tern, vm, 1);
    else
      group_tasks<64>(sm, kPfV, kPfExv, outk, kPfCv, chunk_v, nrows, L.vb, L.nuq != 0, L.lev_v, false, 1, 1, tern, vm, 1);
  }
  __syncthreads();

  // ---- pack
  const uint8_t(*ckr)[D] = reinterpret_cast<const uint8_t(*)[D]>(sm + kPfCk);
  if (L.kb == 3)
    pack_k3(ckr, nrows, rec + L.off_kc, 0);
  else
    pack_rows_fast(sm + kPfCk, nrows, L.kb, rec + L.off_kc, L.k_row_bytes);
  if (chunk_v)
    pack_vchunks_fast(sm + kPfCv, L.vb, rec + L.off_vc);
  else
    pack_v3(reinterpret_cast<const uint8_t(*)[D]>(sm + kPfCv), nrows, rec + L.off_vc, 0);
}

// ===================================================================== KIVI-layout prefill
// prefill_kivi_kernel quantizes the whole prompt blocks of layers with
// per-channel asymmetric keys and per-token asymmetric (or 2-bit ternary)
// values in groups of 32 channels (2/4/8-bit codes; no outliers, rotation or
// key normalization), with the arithmetic of prefill_kernel.  The two wavefronts of a workgroup split a
// block by tensor, each lane holding whole groups: wavefront 0 the keys (lane
// l: channels 2l and 2l + 1 of the 32 tokens), wavefront 1 the values (lane l:
// channels 64 (l % 2) .. + 63 of token l / 2, two groups).  Each loads its
// tensor straight into registers in that layout, one block ahead: each
// workgroup walks a grid stride of blocks and a wavefront's next 8 KiB of
// reads are in flight while it codes the current block.  The codes meet in LDS (key rows, value lane
// chunks) and both wavefronts pack the record.

// Packed binary16 minimum / maximum of two element pairs, written as asm so
// that no canonicalizing operation precedes each use (for the fp16 elements
// here the result is the plain minimum / maximum that fminf / fmaxf give).
__device__ __forceinline__ uint32_t pk_min_h(uint32_t a, uint32_t b) {
  uint32_t d;
  asm("v_pk_min_f16 %0, %1, %2" : "=v"(d) : "v"(a), "v"(b));
  return d;
}
__device__ __forceinline__ uint32_t pk_max_h(uint32_t a, uint32_t b) {
  uint32_t d;
  asm("v_pk_max_f16 %0, %1, %2" : "=v"(d) : "v"(a), "v"(b));
  return d;
}

// Asymmetric codes clamp(rne(fl32(a / s)), 0, Q) of a group sharing the scale
// s (a = fl32(x - base), base = the group minimum), as asym_code defines them,
// from a reciprocal estimate without a branch per element.  With rc =
// rcp(s) (v_rcp_f32, accurate to 1 ulp) and nb = fl32(-base * rc), the
// element's estimate is t = fl32(x * rc + nb), one fused multiply-add that
// reads the binary16 element directly.  Where the quotient is not clamped
// (|a / s| <= Q + 1), t lies within (Q + 1) 2.5 * 2^-23 + |base * rc| 2^-24 of
// fl32(a / s) (the reciprocal's error, the roundings of nb, of t, of a and of
// the quotient), so the two round to the same integer unless t lies within
// E = (Q + 1) 2^-21 + |base * rc| 2^-23 of a half-integer.  Clamping t to
// [lo, Q] first gives the clamped code directly: a t beyond Q (below lo)
// means a quotient above Q - 0.5 (below lo + 0.5).  quot_fast keeps the
// running maximum of |t - rne(t)|; a lane whose maximum passes the group's
// bound 0.5 - E (probability about 2^-19 (Q + 1) per element when base / s
// is of the order of Q) recomputes its codes with the correctly rounded
// division (quot_exact) where quot_near says so.  For 8-bit codes most
// wavefronts see such an element somewhere, so that pass re-tests each
// element and divides only the flagged ones.  rc = 0 (s = 0) codes every
// element 0 and flags nothing.  The same for symmetric codes (base 0,
// quotient clamped to [-Q, Q]) with lo = -Q; asymmetric ones use lo = 0.
struct QuotGroup {
  float rc, nb, lo, Q, bound;
};
__device__ __forceinline__ QuotGroup quot_group(float base, float rc, float lo, float Q) {
  const float e = (Q + 1.f) * 0x1p-21f + fabsf(base * rc) * 0x1p-23f;
  return QuotGroup{rc, -(base * rc), lo, Q, 0.5f - e};
}
__device__ __forceinline__ float quot_t(float x, const QuotGroup& g) {
  return __builtin_amdgcn_fmed3f(fmaf(x, g.rc, g.nb), g.lo, g.Q);
}
// x: the element (a binary16 value widened to fp32)
__device__ __forceinline__ int quot_fast(float x, const QuotGroup& g, float& worst) {
  const float t = quot_t(x, g);
  const float r = rintf(t);
  worst = fmaxf(worst, fabsf(t - r));
  return static_cast<int>(r);
}
__device__ __forceinline__ bool quot_near(float x, const QuotGroup& g) {
  const float t = quot_t(x, g);
  return fabsf(t - rintf(t)) > g.bound;
}
__device__ __forceinline__ int quot_exact(float a, uint16_t s, float lo, float Q) {
  if (s == 0) return 0;
  return static_cast<int>(fminf(fmaxf(rintf(__fdiv_rn(a, h2f(s))), lo), Q));
}
__device__ __forceinline__ int quot_exact(float a, uint16_t s, float Q) { return quot_exact(a, s, 0.f, Q); }
// A copy the compiler cannot prove equal to its input: the rare exact
// recomputation reads its operands through it, so that the fast pass does
// not keep every element's intermediate live across the check.
__device__ __forceinline__ uint32_t opaque_u32(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Parameters of an asymmetric group from its packed binary16 extremes
// (element e of the pairs lo2 / hi2), and the reciprocal of its scale.
__device__ __forceinline__ void asym_pair_params(uint32_t lo2, uint32_t hi2, int e, int Q, float& mn, uint16_t& s,
                                                 uint16_t& z, float& rc) {
  mn = h2f(static_cast<uint16_t>(lo2 >> (16 * e)));
  asym_params(mn, h2f(static_cast<uint16_t>(hi2 >> (16 * e))), true, Q, s, z);
  rc = s == 0 ? 0.f : __builtin_amdgcn_rcpf(h2f(s));
}

// Keys of one lane: channels 2l, 2l + 1 (halves of x[j]) of tokens j = 0..31.
__device__ __forceinline__ void kivi_key_lane(const uint32_t (&x)[kBlockTokens], int bits, int l, uint8_t* ck,
                                              uint16_t* km) {
  uint32_t lo2 = x[0], hi2 = x[0];
#pragma unroll
  for (int j = 1; j < kBlockTokens; ++j) {
    lo2 = pk_min_h(lo2, x[j]);
    hi2 = pk_max_h(hi2, x[j]);
  }
  const int Qi = (1 << bits) - 1;
  const float Q = static_cast<float>(Qi);
  float mn0, mn1, rc0, rc1;
  uint16_t s0, z0, s1, z1;
  asym_pair_params(lo2, hi2, 0, Qi, mn0, s0, z0, rc0);
  asym_pair_params(lo2, hi2, 1, Qi, mn1, s1, z1, rc1);
  uint8_t* dst = ck + 2 * l;
  const QuotGroup g0 = quot_group(mn0, rc0, 0.f, Q), g1 = quot_group(mn1, rc1, 0.f, Q);
  float worst = 0.f;
#pragma unroll
  for (int j = 0; j < kBlockTokens; ++j) {
    const int c0 = quot_fast(h2f(static_cast<uint16_t>(x[j])), g0, worst);
    const int c1 = quot_fast(h2f(static_cast<uint16_t>(x[j] >> 16)), g1, worst);
    *reinterpret_cast<uint16_t*>(dst + j * D) = static_cast<uint16_t>(c0 | (c1 << 8));
  }
  if (worst > fminf(g0.bound, g1.bound)) {
#pragma unroll
    for (int j = 0; j < kBlockTokens; ++j) {
      const uint32_t w = opaque_u32(x[j]);
      const float x0 = h2f(static_cast<uint16_t>(w)), x1 = h2f(static_cast<uint16_t>(w >> 16));
      if (quot_near(x0, g0)) dst[j * D] = static_cast<uint8_t>(quot_exact(__fsub_rn(x0, mn0), s0, Q));
      if (quot_near(x1, g1)) dst[j * D + 1] = static_cast<uint8_t>(quot_exact(__fsub_rn(x1, mn1), s1, Q));
    }
  }
  reinterpret_cast<uint32_t*>(km)[l] = s0 | (static_cast<uint32_t>(s1) << 16);
  reinterpret_cast<uint32_t*>(km + D)[l] = z0 | (static_cast<uint32_t>(z1) << 16);
}

// Values of one lane: token j = l / 2, groups g = 2 (l % 2) + gi of 32
// channels (element i of group gi is half i % 2 of x[16 gi + i / 2]).
// Ternary groups (2-bit codes): s = max |x|, z = -s, and the code of
// clamp(rne(x / s), -1, 1) + 1, which is 1 unless 2 |x| > s exactly (x / s
// of two binary16 values other than +-1/2 lies at least 2^-12 relative from
// +-1/2, beyond any rounding of the quotient; +-1/2 itself rounds to 0).
__device__ __forceinline__ void kivi_value_lane(const uint32_t (&x)[kBlockTokens], int bits, bool tern, int l,
                                                uint8_t* cvc, uint16_t* vm) {
  const int j = l >> 1;
  const int Qi = (1 << bits) - 1;
  const float Q = static_cast<float>(Qi);
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    const int g = 2 * (l & 1) + gi;
    if (tern) {
      uint32_t a2 = x[16 * gi] & 0x7fff7fffu;
#pragma unroll
      for (int q = 1; q < 16; ++q) a2 = pk_max_h(a2, x[16 * gi + q] & 0x7fff7fffu);
      a2 = pk_max_h(a2, a2 >> 16);
      const uint16_t s = static_cast<uint16_t>(a2);
      const float half = 0.5f * h2f(s);  // exact
      uint8_t* dst = cvc + vchunk_off(j, 32 * g);
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const float xe = h2f(static_cast<uint16_t>(x[16 * gi + (i >> 1)] >> (16 * (i & 1))));
        dst[vchunk_off(0, i)] = static_cast<uint8_t>(fabsf(xe) > half ? (xe < 0.f ? 0 : 2) : 1);
      }
      vm[g * kBlockTokens + j] = s;
      vm[4 * kBlockTokens + g * kBlockTokens + j] = static_cast<uint16_t>(s ^ 0x8000u);
      continue;
    }
    uint32_t lo2 = x[16 * gi], hi2 = x[16 * gi];
#pragma unroll
    for (int q = 1; q < 16; ++q) {
      lo2 = pk_min_h(lo2, x[16 * gi + q]);
      hi2 = pk_max_h(hi2, x[16 * gi + q]);
    }
    // fold the two halves into the low one
    lo2 = pk_min_h(lo2, lo2 >> 16);
    hi2 = pk_max_h(hi2, hi2 >> 16);
    float mn, rc;
    uint16_t s, z;
    asym_pair_params(lo2, hi2, 0, Qi, mn, s, z, rc);
    uint8_t* dst = cvc + vchunk_off(j, 32 * g);
    const QuotGroup qg = quot_group(mn, rc, 0.f, Q);
    float worst = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i)
      dst[vchunk_off(0, i)] =
          static_cast<uint8_t>(quot_fast(h2f(static_cast<uint16_t>(x[16 * gi + (i >> 1)] >> (16 * (i & 1)))), qg, worst));
    if (worst > qg.bound) {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const uint32_t w = opaque_u32(x[16 * gi + (i >> 1)]);
        const float xe = h2f(static_cast<uint16_t>(w >> (16 * (i & 1))));
        if (quot_near(xe, qg)) dst[vchunk_off(0, i)] = static_cast<uint8_t>(quot_exact(__fsub_rn(xe, mn), s, Q));
      }
    }
    vm[g * kBlockTokens + j] = s;
    vm[4 * kBlockTokens + g * kBlockTokens + j] = z;
  }
}

__global__ void __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(3)))
prefill_kivi_kernel(LayerDesc L, QuantJob J) {
  __shared__ __align__(16) uint8_t ck[kBlockTokens * D];
  __shared__ __align__(16) uint8_t cvc[64 * 64];
  const int l = threadIdx.x & 63;
  const bool keys = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) == 0;
  const uint32_t total = static_cast<uint32_t>(J.nblocks) * static_cast<uint32_t>(L.units);  // below 2^31 (checked at launch)
  auto load = [&](uint32_t w, uint32_t (&x)[kBlockTokens]) __attribute__((always_inline)) {
    const uint32_t nbk = static_cast<uint32_t>(J.nblocks);
    const int u = static_cast<int>(w / nbk), bi = static_cast<int>(w % nbk);
    const int64_t row0 = u * J.src_unit_stride + static_cast<int64_t>(J.src_t0 + kBlockTokens * bi) * D;
    if (keys) {
      const uint16_t* src = J.k_src + row0 + 2 * l;
#pragma unroll
      for (int j = 0; j < kBlockTokens; ++j) x[j] = *reinterpret_cast<const uint32_t*>(src + j * D);
    } else {
      const uint4* src = reinterpret_cast<const uint4*>(J.v_src + row0 + (l >> 1) * D + 64 * (l & 1));
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint4 v = src[q];
        x[4 * q] = v.x;
        x[4 * q + 1] = v.y;
        x[4 * q + 2] = v.z;
        x[4 * q + 3] = v.w;
      }
    }
  };
  auto block = [&](uint32_t w, const uint32_t (&x)[kBlockTokens]) __attribute__((always_inline)) {
    const uint32_t nbk = static_cast<uint32_t>(J.nblocks);
    const int u = static_cast<int>(w / nbk), bi = static_cast<int>(w % nbk);
    uint8_t* rec = L.body + (static_cast<int64_t>(u) * L.nblk_cap + J.blk0 + bi) * L.rec_bytes;
    if (keys)
      kivi_key_lane(x, L.kb, l, ck, reinterpret_cast<uint16_t*>(rec + L.off_km));
    else
      kivi_value_lane(x, L.vb, L.v_tern != 0, l, cvc, reinterpret_cast<uint16_t*>(rec + L.off_vm));
    __syncthreads();
    pack_rows_fast(ck, kBlockTokens, L.kb, rec + L.off_kc, L.k_row_bytes);
    pack_vchunks_fast(cvc, L.vb, rec + L.off_vc);
    __syncthreads();  // the code tiles are free for the next block
  };
  uint32_t xa[kBlockTokens], xb[kBlockTokens];
  const uint32_t step = gridDim.x;
  uint32_t w = blockIdx.x;
  if (w < total) load(w, xa);
  for (; w < total; w += 2 * step) {
    if (w + step < total) load(w + step, xb);
    block(w, xa);
    if (w + step >= total) break;
    if (w + 2 * step < total) load(w + 2 * step, xa);
    block(w + step, xb);
  }
}

// ===================================================================== inner-group prefill
// prefill_inner_kernel quantizes the whole prompt blocks of layers with keys
// in inner groups of 64 channels (each group symmetric or asymmetric by the
// hybrid test, or always asymmetric) and per-token asymmetric values in
// groups of 32, optionally Hadamard-rotated (2/4/8-bit; 4-bit keys may mix
// in 8-bit groups, keys may be normalized per channel; no outliers), with the
// arithmetic of prefill_kernel and quant_mixed_groups.  Its
// three wavefronts hold whole groups in registers: wavefront 0 the keys (lane
// l: group l % 2 of token l / 2), wavefronts 1 and 2 the values of tokens
// 16 (w - 1) .. + 15 (lane l: channels 32 (l % 4) .. + 31 of one token, so that
// after the rotation a lane holds one value group).  The rotation is the
// exact binary64 butterfly network of hadamard_rows_fast: five stages inside a
// lane, two across the lane quad through DPP moves.  Loads run one block
// ahead along a grid stride of blocks, as in prefill_kivi_kernel.  The
// CHAN instance takes per-channel asymmetric keys with rotated values
// instead: its key wavefront is prefill_kivi_kernel's (lane l: channels 2l,
// 2l + 1 of the 32 tokens).

// 64-bit lane exchange inside a quad (DPP quad_perm: xor 1 or xor 2).
template <int M>
__device__ __forceinline__ double quad_xor(double v) {
  constexpr int ctrl = M == 1 ? 0xB1 : 0x4E;  // [1,0,3,2] / [2,3,0,1]
  const int64_t b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_mov_dpp(static_cast<int>(b & 0xffffffff), ctrl, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_mov_dpp(static_cast<int>(b >> 32), ctrl, 0xf, 0xf, false);
  return __longlong_as_double((static_cast<int64_t>(hi) << 32) | static_cast<uint32_t>(lo));
}

// acc + (half H of w), the binary16 operand widened inside one fused
// multiply-add (one rounding)
template <int H>
__device__ __forceinline__ float add_half(float acc, uint32_t w) {
  if constexpr (H == 0)
    asm("v_fma_mix_f32 %0, %1, 1.0, %0 op_sel_hi:[1,0,0]" : "+v"(acc) : "v"(w));
  else
    asm("v_fma_mix_f32 %0, %1, 1.0, %0 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "+v"(acc) : "v"(w));
  return acc;
}

// Exact binary64 sum of fp16 elements as an int64 count of 2^-24 units (the
// sum of up to 64 values below 2^16 in those units stays below 2^46, exact in
// binary64 and in int64).
__device__ __forceinline__ int64_t units_of(double sum) {
  const double u = sum * 0x1p24;                    // exact integer, |u| < 2^46
  const double hi = floor(u * 0x1p-32);             // exact
  const double lo = u - hi * 0x1p32;                // exact, in [0, 2^32)
  return (static_cast<int64_t>(static_cast<int32_t>(hi)) << 32) + static_cast<int64_t>(static_cast<uint32_t>(lo));
}

// Keys of one lane: group g = l % 2 (channels 64 g ..) of token j = l / 2,
// element i = half i % 2 of x[i / 2].
// Eight 4-bit codes, the low nibbles of the bytes of a (elements 0..3) and b
// (4..7), in the pair-split order of the key extension words.
__device__ __forceinline__ uint32_t nibbles_pair_split(uint32_t a, uint32_t b) {
  uint32_t w = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    w |= ((a >> (8 * e)) & 15u) << pair_split_pos(4, e);
    w |= ((b >> (8 * e)) & 15u) << pair_split_pos(4, 4 + e);
  }
  return w;
}

// Keys of one lane: group g = l % 2 (channels 64 g ..) of token j = l / 2,
// element i = half i % 2 of x[i / 2].  With mixed 4/8-bit groups (k_hi > 0)
// the token's k_hi groups whose 4-bit step ranks highest (ties: the lower
// group) take 8-bit codes: the high nibbles stay in the 4-bit code tile, the
// low nibbles go to the group's k_ext slot and the token's group mask to
// k_sel.
__device__ __forceinline__ void inner_key_lane(uint32_t (&x)[32], const uint32_t (&sw)[16], const LayerDesc& L, int l,
                                               uint8_t* ck, uint32_t* kmeta, uint32_t* kext, uint8_t* ksel) {
  const int j = l >> 1, g = l & 1;
  if (L.kshift) {
    // normalized keys fp16(K * 2^shift), saturating (InnerQ, method 4), in
    // place; sw holds the group's 64 channel shifts (int8)
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const int s0 = static_cast<int8_t>((sw[k >> 1] >> (16 * (k & 1))) & 0xffu);
      const int s1 = static_cast<int8_t>((sw[k >> 1] >> (16 * (k & 1) + 8)) & 0xffu);
      const float a = fminf(fmaxf(ldexpf(h2f(static_cast<uint16_t>(x[k])), s0), -65504.f), 65504.f);
      const float b = fminf(fmaxf(ldexpf(h2f(static_cast<uint16_t>(x[k] >> 16)), s1), -65504.f), 65504.f);
      x[k] = static_cast<uint32_t>(f2h(a)) | (static_cast<uint32_t>(f2h(b)) << 16);
    }
  }
  uint32_t lo2 = x[0], hi2 = x[0];
#pragma unroll
  for (int q = 1; q < 32; ++q) {
    lo2 = pk_min_h(lo2, x[q]);
    hi2 = pk_max_h(hi2, x[q]);
  }
  lo2 = pk_min_h(lo2, lo2 >> 16);
  hi2 = pk_max_h(hi2, hi2 >> 16);
  const uint16_t hmn = static_cast<uint16_t>(lo2), hmx = static_cast<uint16_t>(hi2);
  const float mn = h2f(hmn), mx = h2f(hmx);
  const int bits = L.kb;
  bool sym = false;
  if (L.k_hybrid) {
    // symmetric iff den |sum x| <= num W (max - min), exactly.  First an
    // fp32 estimate of the sum (four chains of 16; each add widens its
    // binary16 operand exactly): every element passes through at most 17
    // roundings, so |est - sum| <= 17.1 * 2^-24 * sum |x| <= 2^-13 A with
    // A = max(|min|, |max|) >= |x|.  Only a group whose test lies within
    // that margin sums again exactly (binary64, units of 2^-24).
    float p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      p[(2 * i) & 3] = add_half<0>(p[(2 * i) & 3], x[i]);
      p[(2 * i + 1) & 3] = add_half<1>(p[(2 * i + 1) & 3], x[i]);
    }
    const double den = static_cast<double>(L.ratio_den);
    const double est = fabs(static_cast<double>((p[0] + p[1]) + (p[2] + p[3])));
    const double margin = static_cast<double>(fmaxf(fabsf(mn), fabsf(mx))) * 0x1p-13;
    const double rhs = static_cast<double>(L.ratio_num) * 64.0 * (static_cast<double>(mx) - static_cast<double>(mn));
    if (den * (est + margin) <= rhs) {
      sym = true;
    } else if (den * (est - margin) > rhs) {
      sym = false;
    } else {
      double sum = 0.0;
#pragma unroll
      for (int i = 0; i < 64; ++i)
        sum += static_cast<double>(h2f(static_cast<uint16_t>(opaque_u32(x[i >> 1]) >> (16 * (i & 1)))));
      int64_t su = units_of(sum);
      su = su < 0 ? -su : su;
      sym = static_cast<int64_t>(L.ratio_den) * su <= static_cast<int64_t>(L.ratio_num) * 64 * (h2fixed(hmx) - h2fixed(hmn));
    }
  }
  uint16_t s, z;
  float lo, Q, rc, base;
  int off;
  auto params = [&](int nbits) __attribute__((always_inline)) {
    if (sym) {
      const uint16_t sv = sym_scale(fmaxf(fabsf(mn), fabsf(mx)), nbits);
      s = sv | 0x8000;
      z = 0;
      Q = static_cast<float>((1 << (nbits - 1)) - 1);
      lo = -Q;
      off = sv == 0 ? 0 : 1 << (nbits - 1);
      rc = sv == 0 ? 0.f : __builtin_amdgcn_rcpf(h2f(sv));
      base = 0.f;
    } else {
      const int Qi = (1 << nbits) - 1;
      asym_params(mn, mx, true, Qi, s, z);
      Q = static_cast<float>(Qi);
      lo = 0.f;
      off = 0;
      rc = s == 0 ? 0.f : __builtin_amdgcn_rcpf(h2f(s));
      base = mn;
    }
  };
  bool wide = false;  // an 8-bit group of a mixed layer
  if (L.k_hi) {
    params(4);
    // rank of the 4-bit steps within the token (the other group is lane l ^ 1)
    const uint32_t sa = s & 0x7fffu;
    const uint32_t sb = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(sa), 0xB1, 0xf, 0xf, false));
    const bool first = sa > sb || (sa == sb && g == 0);
    wide = L.k_hi >= 2 || first;
    const bool other = L.k_hi >= 2 || !first;
    if (g == 0) ksel[j] = static_cast<uint8_t>((wide ? 1u : 0u) | (other ? 2u : 0u));
  }
  params(wide ? 8 : bits);
  const uint16_t sdiv = static_cast<uint16_t>(s & 0x7fff);
  uint32_t* dst = reinterpret_cast<uint32_t*>(ck + j * D + 64 * g);
  const QuotGroup qg = quot_group(base, rc, lo, Q);
  float worst = 0.f;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * q + e;
      w |= static_cast<uint32_t>(quot_fast(h2f(static_cast<uint16_t>(x[i >> 1] >> (16 * (i & 1)))), qg, worst) + off)
           << (8 * e);
    }
    dst[q] = w;
  }
  if (worst > qg.bound) {
    uint8_t* db = reinterpret_cast<uint8_t*>(dst);
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const uint32_t w = opaque_u32(x[i >> 1]);
      const float xe = h2f(static_cast<uint16_t>(w >> (16 * (i & 1))));
      if (quot_near(xe, qg)) db[i] = static_cast<uint8_t>(quot_exact(__fsub_rn(xe, base), sdiv, lo, Q) + off);
    }
  }
  if (wide) {
    // 8-bit codes: high nibbles back to the tile, low nibbles to k_ext slot
    // k (the group's place among the token's 8-bit groups)
    uint32_t* ext = kext + (j * L.k_hi + (L.k_hi >= 2 ? g : 0)) * 8;
#pragma unroll
    for (int q = 0; q < 16; q += 2) {
      const uint32_t a = dst[q], b = dst[q + 1];
      ext[q >> 1] = nibbles_pair_split(a, b);
      dst[q] = (a >> 4) & 0x0f0f0f0fu;
      dst[q + 1] = (b >> 4) & 0x0f0f0f0fu;
    }
  }
  kmeta[j * 2 + g] = s | (static_cast<uint32_t>(z) << 16);
}

// Values of one lane: channels 32 q .. 32 q + 31 (q = l % 4) of token j,
// element i = half i % 2 of x[i / 2]; rotated first when `rotate` (the lane
// quad holds the token's 128 channels), then coded as value group q.
template <class Next>
__device__ __forceinline__ void inner_value_lane(uint32_t (&x)[16], const LayerDesc& L, bool rotate, int l, int j,
                                                 uint8_t* cvc, uint16_t* vm, Next next) {
  const int q = l & 3;
  uint32_t v[16];
  if (rotate) {
    double y[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) y[i] = static_cast<double>(h2f(static_cast<uint16_t>(x[i >> 1] >> (16 * (i & 1)))));
    next(x);  // x is consumed: the next block's loads go in flight now
#pragma unroll
    for (int h = 1; h < 32; h <<= 1)
#pragma unroll
      for (int i = 0; i < 32; ++i)
        if (!(i & h)) {
          const double a = y[i], b = y[i + h];
          y[i] = a + b;
          y[i + h] = a - b;
        }
    // channel bits 5 and 6 across the quad: x <- x + o (bit clear), o - x (set)
    const double sg1 = (q & 1) ? -1.0 : 1.0, sg2 = (q & 2) ? -1.0 : 1.0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      y[i] = fma(y[i], sg1, quad_xor<1>(y[i]));
      if ((i & 3) == 3) __builtin_amdgcn_sched_barrier(0);  // a few partners in flight at a time
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      y[i] = fma(y[i], sg2, quad_xor<2>(y[i]));
      if ((i & 3) == 3) __builtin_amdgcn_sched_barrier(0);
    }
    const double c = L.had_scale;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      v[i] = static_cast<uint32_t>(d2h_odd(y[2 * i] * c)) | (static_cast<uint32_t>(d2h_odd(y[2 * i + 1] * c)) << 16);
      if ((i & 1) == 1) __builtin_amdgcn_sched_barrier(0);  // retire the doubles as they are rounded
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = x[i];
    next(x);
  }
  uint32_t lo2 = v[0], hi2 = v[0];
#pragma unroll
  for (int k = 1; k < 16; ++k) {
    lo2 = pk_min_h(lo2, v[k]);
    hi2 = pk_max_h(hi2, v[k]);
  }
  lo2 = pk_min_h(lo2, lo2 >> 16);
  hi2 = pk_max_h(hi2, hi2 >> 16);
  const int Qi = (1 << L.vb) - 1;
  const float Q = static_cast<float>(Qi);
  float mn, rc;
  uint16_t s, z;
  asym_pair_params(lo2, hi2, 0, Qi, mn, s, z, rc);
  uint8_t* dst = cvc + vchunk_off(j, 32 * q);
  const QuotGroup qg = quot_group(mn, rc, 0.f, Q);
  float worst = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i)
    dst[vchunk_off(0, i)] = static_cast<uint8_t>(quot_fast(h2f(static_cast<uint16_t>(v[i >> 1] >> (16 * (i & 1)))), qg, worst));
  if (worst > qg.bound) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t w = opaque_u32(v[i >> 1]);
      const float xe = h2f(static_cast<uint16_t>(w >> (16 * (i & 1))));
      if (quot_near(xe, qg)) dst[vchunk_off(0, i)] = static_cast<uint8_t>(quot_exact(__fsub_rn(xe, mn), s, Q));
    }
  }
  vm[q * kBlockTokens + j] = s;
  vm[4 * kBlockTokens + q * kBlockTokens + j] = z;
}

// One wavefront's walk over the grid's blocks: ROLE 0 keys (32 words of a
// lane's key group), ROLE 1 values (16 words of a lane's value quarter); its
// own double buffer, so the two roles' registers do not add up.  Every
// wavefront of the workgroup walks the same blocks and meets the same two
// barriers per block.
template <bool CHAN, int ROLE>
__device__ __forceinline__ void inner_walk(const LayerDesc& L, const QuantJob& J, int l, int vj, uint8_t* ck,
                                           uint8_t* cvc) {
  constexpr int NW = ROLE == 0 ? 32 : 16;
  const uint32_t total = static_cast<uint32_t>(J.nblocks) * static_cast<uint32_t>(L.units);  // below 2^31 (checked at launch)
  const uint32_t nbk = static_cast<uint32_t>(J.nblocks);
  // a block's words of this lane (and, for normalized keys, the group's 64
  // channel shifts of the block's unit)
  auto load = [&](uint32_t w, uint32_t (&x)[NW], uint32_t (&sh)[16]) __attribute__((always_inline)) {
    const int u = static_cast<int>(w / nbk), bi = static_cast<int>(w % nbk);
    const int64_t row0 = u * J.src_unit_stride + static_cast<int64_t>(J.src_t0 + kBlockTokens * bi) * D;
    if constexpr (ROLE == 0 && CHAN) {
      // per-channel keys: channels 2l, 2l + 1 of each token
      const uint16_t* src = J.k_src + row0 + 2 * l;
#pragma unroll
      for (int j = 0; j < kBlockTokens; ++j) x[j] = *reinterpret_cast<const uint32_t*>(src + j * D);
    } else {
      const uint4* src = ROLE == 0 ? reinterpret_cast<const uint4*>(J.k_src + row0 + (l >> 1) * D + 64 * (l & 1))
                                   : reinterpret_cast<const uint4*>(J.v_src + row0 + vj * D + 32 * (l & 3));
#pragma unroll
      for (int k = 0; k < NW / 4; ++k) {
        const uint4 v = src[k];
        x[4 * k] = v.x;
        x[4 * k + 1] = v.y;
        x[4 * k + 2] = v.z;
        x[4 * k + 3] = v.w;
      }
    }
    if (ROLE == 0 && !CHAN && L.kshift) {
      const uint4* sp = reinterpret_cast<const uint4*>(L.kshift + static_cast<int64_t>(u) * D + 64 * (l & 1));
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint4 v = sp[k];
        sh[4 * k] = v.x;
        sh[4 * k + 1] = v.y;
        sh[4 * k + 2] = v.z;
        sh[4 * k + 3] = v.w;
      }
    }
  };
  auto pack = [&](uint8_t* rec) __attribute__((always_inline)) {
    __syncthreads();
    pack_rows_fast(ck, kBlockTokens, L.kb, rec + L.off_kc, L.k_row_bytes);
    pack_vchunks_fast(cvc, L.vb, rec + L.off_vc);
    __syncthreads();  // the code tiles are free for the next block
  };
  auto record = [&](uint32_t w) __attribute__((always_inline)) {
    const int u = static_cast<int>(w / nbk), bi = static_cast<int>(w % nbk);
    return L.body + (static_cast<int64_t>(u) * L.nblk_cap + J.blk0 + bi) * L.rec_bytes;
  };
  const uint32_t step = gridDim.x;
  uint32_t w = blockIdx.x;
  if constexpr (ROLE == 0) {
    auto keys = [&](uint32_t (&x)[NW], const uint32_t (&sh)[16], uint8_t* rec) __attribute__((always_inline)) {
      if constexpr (CHAN)
        kivi_key_lane(x, L.kb, l, ck, reinterpret_cast<uint16_t*>(rec + L.off_km));
      else
        inner_key_lane(x, sh, L, l, ck, reinterpret_cast<uint32_t*>(rec + L.off_km),
                       reinterpret_cast<uint32_t*>(rec + L.off_kx), rec + L.off_ks);
    };
    // keys: two buffers (the group's words are read until its codes are out)
    uint32_t xa[NW], xb[NW], sa[16], sb[16];
    if (w < total) load(w, xa, sa);
    for (; w < total; w += 2 * step) {
      if (w + step < total) load(w + step, xb, sb);
      uint8_t* rec = record(w);
      keys(xa, sa, rec);
      pack(rec);
      if (w + step >= total) break;
      if (w + 2 * step < total) load(w + 2 * step, xa, sa);
      rec = record(w + step);
      keys(xb, sb, rec);
      pack(rec);
    }
  } else {
    // values: one buffer, refilled as soon as the lane has converted it
    uint32_t x[NW], unused[16];
    if (w < total) load(w, x, unused);
    for (; w < total; w += step) {
      const uint32_t wn = w + step;
      uint8_t* rec = record(w);
      inner_value_lane(x, L, J.rotate_v != 0, l, vj, cvc, reinterpret_cast<uint16_t*>(rec + L.off_vm),
                       [&](uint32_t (&buf)[NW]) __attribute__((always_inline)) {
                         if (wn < total) load(wn, buf, unused);
                       });
      pack(rec);
    }
  }
}

template <bool CHAN>
__global__ void __launch_bounds__(192) __attribute__((amdgpu_waves_per_eu(3)))
prefill_inner_kernel(LayerDesc L, QuantJob J) {
  __shared__ __align__(16) uint8_t ck[kBlockTokens * D];
  __shared__ __align__(16) uint8_t cvc[64 * 64];
  const int l = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // 0 keys, 1 and 2 values
  if (wv == 0)
    inner_walk<CHAN, 0>(L, J, l, 0, ck, cvc);
  else
    inner_walk<CHAN, 1>(L, J, l, 16 * (wv - 1) + (l >> 2), ck, cvc);
}

// ===================================================================== codebook prefill
// prefill_codebook_kernel quantizes the whole prompt blocks of layers with
// 3-bit codebook keys (per channel) and values (per token, groups of 32) and
// two sparse fp16 outliers per token row of each tensor (no rotation or key
// normalization), with the arithmetic of prefill_kernel.  Four wavefronts:
// 0 and 1 hold key channels l and l + 64 of tokens 16 w .. + 15 (lane l:
// the channel pair of its own 3-bit record chunk), 2 and 3 hold key and
// value rows of tokens 16 (w - 2) .. + 15 (lane l: quarter l % 4 of token
// l / 4, so a lane holds one value group).  Per block: the row wavefronts
// find each row's two outliers (a top-2 of sortable keys in the lane, then
// across the lane quad), write the outlier entries, publish the key rows'
// outlier masks in LDS and code the values; the key wavefronts read the
// masks, exchange the two halves of each channel's extremes through LDS and
// write their record chunks straight from registers.  Codebook codes use a
// three-level search of the sorted level midpoints; the estimate of u =
// (x - min) / s decides unless it lies within 2^-18 of one of the midpoints
// the search compared (the two neighbours of u are among them), as in
// nuq_code_fast.

// code = #{j : u > mid_j} by binary search; `gap` = min distance from u to
// the midpoints compared (its bracketing midpoints are among them).
__device__ __forceinline__ int nuq_search(float u, const float (&m)[7], float& gap) {
  // flat selects (a nested conditional can end up as branches)
  const bool b2 = u > m[3];
  const float ma = b2 ? m[5] : m[1];
  const float mhi = b2 ? m[6] : m[2];
  const float mlo = b2 ? m[4] : m[0];
  const bool b1 = u > ma;
  const float mb = b1 ? mhi : mlo;
  const bool b0 = u > mb;
  gap = fminf(fminf(fabsf(u - m[3]), fabsf(u - ma)), fabsf(u - mb));
  return (b2 ? 4 : 0) + (b1 ? 2 : 0) + (b0 ? 1 : 0);
}
// Codebook code of element x with group minimum mn and scale s, from the
// estimate u = fl32(x * rc + nb) (rc = rcp(s), 0 when s == 0: code 0; nb =
// fl32(-mn * rc)), tracking the smallest gap seen.  Near the midpoints
// (|u| <= 1 + 2^-18) u lies within 2^-21 + |mn * rc| 2^-24 of the quotient
// fl32(fl32(x - mn) / s) (the reciprocal and the four roundings), so a gap
// of at least nuq_thr = 2^-18 + |mn * rc| 2^-22 leaves the code unchanged;
// a lane whose smallest gap is below it redoes those elements with
// nuq_exact and the correctly rounded quotient.
__device__ __forceinline__ float nuq_thr(float mn, float rc) { return 0x1p-18f + fabsf(mn * rc) * 0x1p-22f; }
__device__ __forceinline__ int nuq_fast(float x, float rc, float nb, const float (&m)[7], float& worst_gap) {
  float gap;
  const int c = nuq_search(fmaf(x, rc, nb), m, gap);
  worst_gap = fminf(worst_gap, gap);
  return c;
}
__device__ __forceinline__ bool nuq_near(float x, float rc, float nb, const float (&m)[7], float thr) {
  float gap;
  nuq_search(fmaf(x, rc, nb), m, gap);
  return gap < thr;
}
__device__ __forceinline__ int nuq_exact(float d, uint16_t s, const float (&m)[7]) {
  if (s == 0) return 0;
  float gap;
  return nuq_search(__fdiv_rn(d, h2f(s)), m, gap);
}

// Cell tables for the codebook search.  The estimate is taken on the grid
// t' = u * 256 + o (o = k / 64 chosen per layer so that every midpoint sits at
// least kCellMargin from a cell edge, at most one per cell, all below cell
// 254).  Entry c of a table is the shifted midpoint fl32(m * 256 + o) inside
// cell c (1e30 when the cell holds none) with its three lowest mantissa bits
// replaced by the number of midpoints below the cell; the code of t' in cell
// c is that count plus (t' > entry).  The entry moves by at most 2^-13
// (rounding and the count bits); t' lies within 2^-13.6 + |mn * rc| 2^-15 of
// 256 fl32(fl32(x - mn) / s) + o (the reciprocal, the roundings of nb, of the
// offset, of t' and of the quotient), so a distance |t' - entry| of at least
// cell_thr = 2^-11 + |mn * rc| 2^-14 leaves the code unchanged: the cell's
// other neighbours are at least kCellMargin >= cell_thr away.  A lane that
// sees a smaller distance (or a group whose cell_thr passes the margin)
// recodes its elements by the midpoint search and the exact quotient.
constexpr float kCellMargin = 1.f / 32;
__device__ __forceinline__ float cell_thr(float mn, float rc) { return 0x1p-11f + fabsf(mn * rc) * 0x1p-14f; }
__device__ __forceinline__ uint32_t cvt_u32_sat(float x) {
  uint32_t r;
  asm("v_cvt_u32_f32 %0, %1" : "=v"(r) : "v"(x));  // negative and NaN give 0
  return r;
}
__device__ __forceinline__ int cell_code(float x, float rc256, float nbo, const float* table, float& worst) {
  const float tp = fmaf(x, rc256, nbo);
  const float e = table[min(cvt_u32_sat(tp), 255u)];
  const float d = tp - e;
  worst = fminf(worst, fabsf(d));
  return static_cast<int>(__float_as_uint(e) & 7u) + (d > 0.f ? 1 : 0);
}
// Grid offset o for midpoints m (lanes test o = l / 64; the lowest that works
// wins), or -1 when none does; then thread i of the workgroup fills entry i.
__device__ __forceinline__ float cell_offset(const float (&m)[7], int l) {
  const float o = static_cast<float>(l) * (1.f / 64);
  bool ok = true;
  int prev = -1;
#pragma unroll
  for (int j = 0; j < 7; ++j) {
    const float pj = fmaf(m[j], 256.f, o);
    const float fl = floorf(pj);
    ok = ok && pj >= 0.f && pj < 254.f && pj - fl >= kCellMargin && fl + 1.f - pj >= kCellMargin &&
         static_cast<int>(fl) > prev;
    prev = static_cast<int>(fl);
  }
  const uint64_t b = __ballot(ok);
  return b == 0 ? -1.f : static_cast<float>(__builtin_ctzll(b)) * (1.f / 64);
}
__device__ __forceinline__ float cell_entry(const float (&m)[7], float o, int c) {
  uint32_t below = 0;
  float e = 1e30f;
#pragma unroll
  for (int j = 0; j < 7; ++j) {
    const float pj = fmaf(m[j], 256.f, o);
    below += pj < static_cast<float>(c) ? 1u : 0u;
    if (floorf(pj) == static_cast<float>(c)) e = pj;
  }
  return __uint_as_float((__float_as_uint(e) & ~7u) | below);
}

// Sortable outlier key of an element: its magnitude (bits 16..30), then the
// lower column (127 - c in bits 8..15), then the high byte of the binary16
// (bits 0..7, the sign at bit 7, so the raw value can be rebuilt).  In the
// lane the column byte holds 31 - i for element i of the lane's 32 columns;
// one byte permute and one mask build the key from the element's half of
// its word (H = 0 low half, 1 high half).
template <int H>
__device__ __forceinline__ uint32_t outlier_key_local(uint32_t w, int i) {
  constexpr uint32_t sel = H == 0 ? 0x05040005u : 0x07060007u;  // [hi byte, lo byte, column, hi byte]
  return __builtin_amdgcn_perm(w, static_cast<uint32_t>(31 - i), sel) & 0x7fffffffu;
}
__device__ __forceinline__ int outlier_col(uint32_t key) { return 127 - static_cast<int>((key >> 8) & 127u); }
__device__ __forceinline__ uint32_t outlier_bits(uint32_t key) { return ((key >> 16) & 0x7fffu) | ((key & 0x80u) << 8); }

// Top two keys of a row held by a lane quad (lane q: columns 32 q .. + 31,
// element i = half i % 2 of x[i / 2]); every lane of the quad gets them.
__device__ __forceinline__ void row_top2(const uint32_t (&x)[16], int q, uint32_t& t0, uint32_t& t1) {
  t0 = 0u;
  t1 = 0u;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t k = (i & 1) ? outlier_key_local<1>(x[i >> 1], i) : outlier_key_local<0>(x[i >> 1], i);
    uint32_t m;  // second largest of {t0, t1, k} (t0 >= t1)
    asm("v_med3_u32 %0, %1, %2, %3" : "=v"(m) : "v"(t0), "v"(t1), "v"(k));
    t1 = m;
    t0 = max(t0, k);
  }
  // lane-local columns to row columns (127 - c = 32 (3 - q) + 31 - i)
  t0 += static_cast<uint32_t>(3 - q) << 13;
  t1 += static_cast<uint32_t>(3 - q) << 13;
  auto join = [&](uint32_t o0, uint32_t o1) __attribute__((always_inline)) {
    t1 = max(min(t0, o0), max(t1, o1));
    t0 = max(t0, o0);
  };
  // across the quad: xor 1, then xor 2 (DPP quad_perm [1,0,3,2], [2,3,0,1])
  join(static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(t0), 0xB1, 0xf, 0xf, false)),
       static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(t1), 0xB1, 0xf, 0xf, false)));
  join(static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(t0), 0x4E, 0xf, 0xf, false)),
       static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(t1), 0x4E, 0xf, 0xf, false)));
}

// The outlier entries of one row ({column, fp16}, columns ascending) and the
// row's mask word for columns 32 q .. + 31.
__device__ __forceinline__ uint32_t row_outliers(uint32_t t0, uint32_t t1, int q, uint32_t* entries) {
  const int c0 = outlier_col(t0), c1 = outlier_col(t1);
  const uint32_t e0 = static_cast<uint32_t>(c0) | (outlier_bits(t0) << 16);
  const uint32_t e1 = static_cast<uint32_t>(c1) | (outlier_bits(t1) << 16);
  if (q == 0) {
    entries[0] = c0 < c1 ? e0 : e1;
    entries[1] = c0 < c1 ? e1 : e0;
  }
  uint32_t m = 0u;
  if ((c0 >> 5) == q) m |= 1u << (c0 & 31);
  if ((c1 >> 5) == q) m |= 1u << (c1 & 31);
  return m;
}

// Halves of w whose element is excluded (mask bits lo / hi set) replaced by
// the binary16 bit pattern `fill` (both halves).
__device__ __forceinline__ uint32_t mask_halves(uint32_t w, uint32_t ex, int lo_bit, uint32_t ex_hi, int hi_bit,
                                                uint32_t fill) {
  const uint32_t ml = static_cast<uint32_t>(__builtin_amdgcn_sbfe(static_cast<int>(ex), lo_bit, 1));
  const uint32_t mh = static_cast<uint32_t>(__builtin_amdgcn_sbfe(static_cast<int>(ex_hi), hi_bit, 1));
  const uint32_t m = __builtin_amdgcn_perm(mh, ml, 0x07060100u);  // low half from ml, high half from mh
  return (fill & m) | (w & ~m);
}
constexpr uint32_t kInf2 = 0x7c007c00u, kNegInf2 = 0xfc00fc00u;

// Extremes of the members (elements whose mask bit is clear) of 32 halves,
// on the binary16 pairs (excluded elements read as +inf for the minimum and
// -inf for the maximum).
__device__ __forceinline__ bool masked_extremes(const uint32_t (&x)[16], uint32_t ex, float& mn, float& mx) {
  uint32_t lo2 = kInf2, hi2 = kNegInf2;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    lo2 = pk_min_h(lo2, mask_halves(x[k], ex, 2 * k, ex, 2 * k + 1, kInf2));
    hi2 = pk_max_h(hi2, mask_halves(x[k], ex, 2 * k, ex, 2 * k + 1, kNegInf2));
  }
  lo2 = pk_min_h(lo2, lo2 >> 16);
  hi2 = pk_max_h(hi2, hi2 >> 16);
  mn = h2f(static_cast<uint16_t>(lo2));
  mx = h2f(static_cast<uint16_t>(hi2));
  return mn <= mx;
}

template <int ROLE>  // 0 keys, 1 rows
__device__ __forceinline__ void codebook_walk(const LayerDesc& L, const QuantJob& J, int wv, int l, uint32_t* kmask,
                                              float* kext, uint8_t* cv, const float* cells, float off) {
  constexpr int NW = ROLE == 0 ? 16 : 32;
  const uint32_t total = static_cast<uint32_t>(J.nblocks) * static_cast<uint32_t>(L.units);  // below 2^31 (checked at launch)
  const uint32_t nbk = static_cast<uint32_t>(J.nblocks);
  const int half = ROLE == 0 ? wv : wv - 2;  // tokens 16 half .. + 15
  const int q = l & 3, rj = 16 * half + (l >> 2);
  float mk[7], mv[7];  // level midpoints (read by value: no pointer into the kernel arguments)
#pragma unroll
  for (int j = 0; j < 7; ++j) {
    mk[j] = __fmul_rn(__fadd_rn(h2f(L.lev_k[j]), h2f(L.lev_k[j + 1])), 0.5f);
    mv[j] = __fmul_rn(__fadd_rn(h2f(L.lev_v[j]), h2f(L.lev_v[j + 1])), 0.5f);
  }
  auto load = [&](uint32_t w, uint32_t (&x)[NW]) __attribute__((always_inline)) {
    const int u = static_cast<int>(w / nbk), bi = static_cast<int>(w % nbk);
    const int64_t row0 = u * J.src_unit_stride + static_cast<int64_t>(J.src_t0 + kBlockTokens * bi) * D;
    if constexpr (ROLE == 0) {
      const uint16_t* src = J.k_src + row0 + static_cast<int64_t>(16 * half) * D + l;
#pragma unroll
      for (int t = 0; t < 16; ++t)
        x[t] = static_cast<uint32_t>(src[t * D]) | (static_cast<uint32_t>(src[t * D + 64]) << 16);
    } else {
      const uint4* ks = reinterpret_cast<const uint4*>(J.k_src + row0 + rj * D + 32 * q);
      const uint4* vs = reinterpret_cast<const uint4*>(J.v_src + row0 + rj * D + 32 * q);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint4 a = ks[k], b = vs[k];
        x[4 * k] = a.x;
        x[4 * k + 1] = a.y;
        x[4 * k + 2] = a.z;
        x[4 * k + 3] = a.w;
        x[16 + 4 * k] = b.x;
        x[16 + 4 * k + 1] = b.y;
        x[16 + 4 * k + 2] = b.z;
        x[16 + 4 * k + 3] = b.w;
      }
    }
  };
  auto block = [&](uint32_t w, const uint32_t (&x)[NW]) __attribute__((always_inline)) {
    const int u = static_cast<int>(w / nbk), bi = static_cast<int>(w % nbk);
    uint8_t* rec = L.body + (static_cast<int64_t>(u) * L.nblk_cap + J.blk0 + bi) * L.rec_bytes;
    if constexpr (ROLE == 1) {
      // ---- outliers of the key and value rows; value codes
      uint32_t kx[16], vx[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        kx[i] = x[i];
        vx[i] = x[16 + i];
      }
      uint32_t t0, t1;
      row_top2(kx, q, t0, t1);
      kmask[rj * 4 + q] = row_outliers(t0, t1, q, reinterpret_cast<uint32_t*>(rec + L.off_ko) + rj * 2);
      row_top2(vx, q, t0, t1);
      const uint32_t vex = row_outliers(t0, t1, q, reinterpret_cast<uint32_t*>(rec + L.off_vo) + rj * 2);
      float mn, mx;
      const bool any = masked_extremes(vx, vex, mn, mx);
      uint16_t s, z;
      nuq_params(mn, mx, any, s, z);
      const float rc = s == 0 ? 0.f : __builtin_amdgcn_rcpf(h2f(s));
      const float nb = -(mn * rc), thr = nuq_thr(mn, rc);
      uint32_t* dst = reinterpret_cast<uint32_t*>(cv + rj * D + 32 * q);
      if (off >= 0.f) {
        // cell tables (cells + 256: the value table)
        const float rc256 = rc * 256.f, nbo = -(mn * rc256) + off, cthr = cell_thr(mn, rc);
        float worst = cthr > kCellMargin ? -1.f : 1e30f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          uint32_t wd = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * k + e;
            const float xe = h2f(static_cast<uint16_t>(opaque_u32(vx[i >> 1]) >> (16 * (i & 1))));
            wd |= static_cast<uint32_t>(cell_code(xe, rc256, nbo, cells + 256, worst)) << (8 * e);
          }
          dst[k] = wd;
          __builtin_amdgcn_sched_barrier(0);  // keep the code words' live ranges short
        }
        if (worst < cthr) {
          uint8_t* db = reinterpret_cast<uint8_t*>(dst);
#pragma unroll
          for (int i = 0; i < 32; ++i) {
            const float xe = h2f(static_cast<uint16_t>(opaque_u32(vx[i >> 1]) >> (16 * (i & 1))));
            float gap;
            const int c = nuq_search(fmaf(xe, rc, nb), mv, gap);
            db[i] = static_cast<uint8_t>(gap < thr ? nuq_exact(__fsub_rn(xe, mn), s, mv) : c);
          }
        }
      } else {
        float worst = 1.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          uint32_t wd = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * k + e;
            // converted again rather than kept from the extremes pass (registers)
            const float xe = h2f(static_cast<uint16_t>(opaque_u32(vx[i >> 1]) >> (16 * (i & 1))));
            wd |= static_cast<uint32_t>(nuq_fast(xe, rc, nb, mv, worst)) << (8 * e);
          }
          dst[k] = wd;
          __builtin_amdgcn_sched_barrier(0);  // keep the code words' live ranges short
        }
        if (worst < thr) {
          uint8_t* db = reinterpret_cast<uint8_t*>(dst);
#pragma unroll
          for (int i = 0; i < 32; ++i) {
            const float xe = h2f(static_cast<uint16_t>(opaque_u32(vx[i >> 1]) >> (16 * (i & 1))));
            if (nuq_near(xe, rc, nb, mv, thr)) db[i] = static_cast<uint8_t>(nuq_exact(__fsub_rn(xe, mn), s, mv));
          }
        }
      }
      uint16_t* vm = reinterpret_cast<uint16_t*>(rec + L.off_vm);
      vm[q * kBlockTokens + rj] = s;
      vm[4 * kBlockTokens + q * kBlockTokens + rj] = z;
    }
    __syncthreads();  // key outlier masks and value codes complete
    if constexpr (ROLE == 0) {
      // ---- value chunks (the key wavefronts wait less than the row ones):
      // lane l packs elements 32 half .. + 31 of chunk l, i.e. its words
      // 3 half .. 3 half + 2 (element e of chunk l is code (token 8 (l / 16) +
      // e % 8, channel 16 (e / 8) + l % 16))
      {
        uint32_t wd[3] = {0u, 0u, 0u};
#pragma unroll
        for (int ep = 0; ep < 32; ++ep) {
          const int e = 32 * half + ep;
          const uint32_t code = cv[(8 * (l >> 4) + (e & 7)) * D + 16 * (e >> 3) + (l & 15)];
          const int b = 3 * ep, wi = b >> 5, sh = b & 31;
          wd[wi] |= code << sh;
          if (sh > 29) wd[wi + 1] |= code >> (32 - sh);
        }
        uint32_t* chunk = reinterpret_cast<uint32_t*>(rec + L.off_vc) + 6 * l + 3 * half;
#pragma unroll
        for (int k = 0; k < 3; ++k) chunk[k] = wd[k];
      }

      // ---- key channels l (half 0) and l + 64 (half 1) of the wavefront's 16 tokens
      uint32_t ex0 = 0, ex1 = 0;  // bit t: token 16 half + t is an outlier of the channel
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const uint32_t* m = kmask + (16 * half + t) * 4;
        ex0 |= ((m[l >> 5] >> (l & 31)) & 1u) << t;
        ex1 |= ((m[2 + (l >> 5)] >> (l & 31)) & 1u) << t;
      }
      // channel l in the low halves, l + 64 in the high ones
      uint32_t lo2 = kInf2, hi2 = kNegInf2;
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        lo2 = pk_min_h(lo2, mask_halves(x[t], ex0, t, ex1, t, kInf2));
        hi2 = pk_max_h(hi2, mask_halves(x[t], ex0, t, ex1, t, kNegInf2));
      }
      const float e4[4] = {h2f(static_cast<uint16_t>(lo2)), h2f(static_cast<uint16_t>(hi2)),
                           h2f(static_cast<uint16_t>(lo2 >> 16)), h2f(static_cast<uint16_t>(hi2 >> 16))};
#pragma unroll
      for (int k = 0; k < 4; ++k) kext[(half * 4 + k) * 64 + l] = e4[k];
    }
    __syncthreads();  // both halves' extremes; masks and value codes read
    if constexpr (ROLE == 0) {
      float mn[2], rc[2];
      uint16_t sz[2][2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        mn[e] = fminf(kext[(0 * 4 + 2 * e) * 64 + l], kext[(1 * 4 + 2 * e) * 64 + l]);
        const float mx = fmaxf(kext[(0 * 4 + 2 * e + 1) * 64 + l], kext[(1 * 4 + 2 * e + 1) * 64 + l]);
        nuq_params(mn[e], mx, mn[e] <= mx, sz[e][0], sz[e][1]);
        rc[e] = sz[e][0] == 0 ? 0.f : __builtin_amdgcn_rcpf(h2f(sz[e][0]));
      }
      // 6-bit fields (c1 << 3 | c0) of tokens t at bit 6 t of the chunk's
      // 96-bit half 3 half .. 3 half + 2 (words)
      uint32_t f[16];
      const float nb0 = -(mn[0] * rc[0]), nb1 = -(mn[1] * rc[1]);
      const float thr0 = nuq_thr(mn[0], rc[0]), thr1 = nuq_thr(mn[1], rc[1]);
      if (off >= 0.f) {
        const float r0 = rc[0] * 256.f, r1 = rc[1] * 256.f;
        const float o0 = -(mn[0] * r0) + off, o1 = -(mn[1] * r1) + off;
        const float cthr = fmaxf(cell_thr(mn[0], rc[0]), cell_thr(mn[1], rc[1]));
        float worst = cthr > kCellMargin ? -1.f : 1e30f;
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const float x0 = h2f(static_cast<uint16_t>(x[t])), x1 = h2f(static_cast<uint16_t>(x[t] >> 16));
          f[t] = static_cast<uint32_t>(cell_code(x0, r0, o0, cells, worst)) |
                 (static_cast<uint32_t>(cell_code(x1, r1, o1, cells, worst)) << 3);
          if ((t & 3) == 3) __builtin_amdgcn_sched_barrier(0);  // keep the live ranges short
        }
        if (worst < cthr) {
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            const uint32_t xw = opaque_u32(x[t]);
            const float x0 = h2f(static_cast<uint16_t>(xw)), x1 = h2f(static_cast<uint16_t>(xw >> 16));
            float g0, g1;
            int c0 = nuq_search(fmaf(x0, rc[0], nb0), mk, g0);
            int c1 = nuq_search(fmaf(x1, rc[1], nb1), mk, g1);
            if (g0 < thr0) c0 = nuq_exact(__fsub_rn(x0, mn[0]), sz[0][0], mk);
            if (g1 < thr1) c1 = nuq_exact(__fsub_rn(x1, mn[1]), sz[1][0], mk);
            f[t] = static_cast<uint32_t>(c0) | (static_cast<uint32_t>(c1) << 3);
          }
        }
      } else {
        float worst = 1.f;
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const float x0 = h2f(static_cast<uint16_t>(x[t])), x1 = h2f(static_cast<uint16_t>(x[t] >> 16));
          f[t] = static_cast<uint32_t>(nuq_fast(x0, rc[0], nb0, mk, worst)) |
                 (static_cast<uint32_t>(nuq_fast(x1, rc[1], nb1, mk, worst)) << 3);
          if ((t & 3) == 3) __builtin_amdgcn_sched_barrier(0);  // keep the searches' live ranges short
        }
        if (worst < fmaxf(thr0, thr1)) {
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            const uint32_t xw = opaque_u32(x[t]);
            const float x0 = h2f(static_cast<uint16_t>(xw)), x1 = h2f(static_cast<uint16_t>(xw >> 16));
            if (nuq_near(x0, rc[0], nb0, mk, thr0))
              f[t] = (f[t] & ~7u) | static_cast<uint32_t>(nuq_exact(__fsub_rn(x0, mn[0]), sz[0][0], mk));
            if (nuq_near(x1, rc[1], nb1, mk, thr1))
              f[t] = (f[t] & 7u) | (static_cast<uint32_t>(nuq_exact(__fsub_rn(x1, mn[1]), sz[1][0], mk)) << 3);
          }
        }
      }
      uint32_t wd[3] = {0u, 0u, 0u};
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int b = 6 * t, wi = b >> 5, sh = b & 31;
        wd[wi] |= f[t] << sh;
        if (sh > 26) wd[wi + 1] |= f[t] >> (32 - sh);
      }
      uint32_t* chunk = reinterpret_cast<uint32_t*>(rec + L.off_kc) + 6 * l + 3 * half;
#pragma unroll
      for (int k = 0; k < 3; ++k) chunk[k] = wd[k];
      if (half == 0) {
        uint16_t* km = reinterpret_cast<uint16_t*>(rec + L.off_km);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          km[l + 64 * e] = sz[e][0];
          km[D + l + 64 * e] = sz[e][1];
        }
      }
    }
  };
  uint32_t xa[NW], xb[NW];
  const uint32_t step = gridDim.x;
  uint32_t w = blockIdx.x;
  if (w < total) load(w, xa);
  for (; w < total; w += 2 * step) {
    if (w + step < total) load(w + step, xb);
    block(w, xa);
    if (w + step >= total) break;
    if (w + 2 * step < total) load(w + 2 * step, xa);
    block(w + step, xb);
  }
}

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
prefill_codebook_kernel(LayerDesc L, QuantJob J) {
  __shared__ __align__(16) uint32_t kmask[kBlockTokens * 4];   // key-row outlier bits per token
  __shared__ __align__(16) float kext[2 * 4 * 64];             // [token half][min0, max0, min1, max1][lane]
  __shared__ __align__(16) uint8_t cv[kBlockTokens * D];       // value codes, row-major
  __shared__ float cells[2 * 256];                             // key and value cell tables
  __shared__ float offs[2];
  const int l = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  {
    float mk[7], mv[7];
#pragma unroll
    for (int j = 0; j < 7; ++j) {
      mk[j] = __fmul_rn(__fadd_rn(h2f(L.lev_k[j]), h2f(L.lev_k[j + 1])), 0.5f);
      mv[j] = __fmul_rn(__fadd_rn(h2f(L.lev_v[j]), h2f(L.lev_v[j + 1])), 0.5f);
    }
    if (wv == 0) {
      const float ok = cell_offset(mk, l), ov = cell_offset(mv, l);
      if (l == 0) {
        offs[0] = ok < 0.f || ov < 0.f ? -1.f : ok;
        offs[1] = ov;
      }
    }
    __syncthreads();
    const float ok = offs[0], ov = offs[1];
    if (ok >= 0.f) {
      cells[threadIdx.x] = cell_entry(mk, ok, threadIdx.x);
      cells[256 + threadIdx.x] = cell_entry(mv, ov, threadIdx.x);
    }
    __syncthreads();
  }
  // one offset per table: the key walk reads offs[0], the row walk offs[1]
  // (both are -1 when either table cannot be built)
  const float off = offs[0] < 0.f ? -1.f : offs[wv < 2 ? 0 : 1];
  if (wv < 2)
    codebook_walk<0>(L, J, wv, l, kmask, kext, cv, cells, off);
  else
    codebook_walk<1>(L, J, wv, l, kmask, kext, cv, cells, off);
}

__global__ void __launch_bounds__(128) copy_fp16_kernel(LayerDesc L, CopyJob J) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  QuantSmem& sm = *reinterpret_cast<QuantSmem*>(smem_raw);
  const int t = threadIdx.x;
  const int u = blockIdx.y;
  const int j0 = blockIdx.x * kBlockTokens;
  const int rows = min(kBlockTokens, J.count - j0);
  const int64_t base = u * J.src_unit_stride + static_cast<int64_t>(J.src_t0 + j0) * D;
  for (int j = 0; j < rows; ++j) {
    sm.k[j][t] = J.k_src[base + j * D + t];
    sm.v[j][t] = J.v_src[base + j * D + t];
  }
  __syncthreads();
  if (J.rotate_v) hadamard_rows(sm, sm.v, rows, L.had_scale);
  const int slots = L.sinks_cap + L.win_cap;
  uint16_t* kdst = L.fp16 + static_cast<int64_t>(u) * 2 * slots * D;
  uint16_t* vdst = kdst + static_cast<int64_t>(slots) * D;
  for (int j = 0; j < rows; ++j) {
    const int p = J.pos0 + j0 + j;
    const int slot = p < J.s_eff ? p : L.sinks_cap + (p - J.s_eff) % L.win_cap;
    kdst[slot * D + t] = sm.k[j][t];
    vdst[vslot(slot, t)] = sm.v[j][t];
  }
}

// InnerQ, method 4 (one-time per-channel key normalization from the
// prefill): per unit, shift_c = min(E - e_c, 14) with e_c the binary exponent
// of max_t |K[t][c]| (a = m 2^e, 1/2 <= m < 1) and E = max_c e_c; an all-zero
// channel gets 0.  Magnitudes are compared as fp16 bit patterns (exact), the
// exponent is read from the maximum's bits.  Block: 16 groups of 16 lanes, a
// group reads whole token rows as 16-byte vectors.
__global__ void __launch_bounds__(256) knorm_shift_kernel(const uint16_t* k, int32_t T, int8_t* out) {
  __shared__ uint16_t part[16][D];
  __shared__ int e_max;
  const int tid = threadIdx.x, rg = tid >> 4, cl = tid & 15;
  const int u = blockIdx.x;
  const uint4* src = reinterpret_cast<const uint4*>(k + static_cast<int64_t>(u) * T * D) + cl;
  uint32_t m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  auto take = [&](const uint4 v) __attribute__((always_inline)) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m[2 * i] = max(m[2 * i], w[i] & 0x7fffu);
      m[2 * i + 1] = max(m[2 * i + 1], (w[i] >> 16) & 0x7fffu);
    }
  };
  // eight rows per group in flight at a time
  constexpr int kRows = 8;
  int t = rg;
  for (; t + 16 * (kRows - 1) < T; t += 16 * kRows) {
    uint4 v[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) v[r] = src[static_cast<int64_t>(t + 16 * r) * (D / 8)];
#pragma unroll
    for (int r = 0; r < kRows; ++r) take(v[r]);
  }
  for (; t < T; t += 16) take(src[static_cast<int64_t>(t) * (D / 8)]);
#pragma unroll
  for (int i = 0; i < 8; ++i) part[rg][8 * cl + i] = static_cast<uint16_t>(m[i]);
  if (tid == 0) e_max = -1000;
  __syncthreads();
  int e = 0;
  bool zero = true;
  if (tid < D) {
    uint32_t a = 0;
    for (int r = 0; r < 16; ++r) a = max(a, static_cast<uint32_t>(part[r][tid]));
    zero = a == 0;
    if (!zero) {
      // normal: (1 + f) 2^(E5 - 15) = 0.5 (1 + f) 2^(E5 - 14); subnormal: a 2^-24
      e = a >= 0x400u ? static_cast<int>(a >> 10) - 14 : (32 - __clz(static_cast<int>(a))) - 24;
      atomicMax(&e_max, e);
    }
  }
  __syncthreads();
  if (tid < D) out[static_cast<int64_t>(u) * D + tid] = static_cast<int8_t>(zero ? 0 : min(e_max - e, 14));
}

__global__ void __launch_bounds__(256) zero_kernel(uint4* p, int64_t n16) {
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n16; i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

hipError_t launch_zero_fp16(const LayerDesc& L, hipStream_t s) {
  const int64_t bytes = static_cast<int64_t>(L.units) * 2 * (L.sinks_cap + L.win_cap) * D * 2;
  const int64_t n16 = bytes / 16;  // slots are a multiple of 32, so bytes is a multiple of 16
  const int grid = static_cast<int>(std::min<int64_t>((n16 + 255) / 256, 4096));
  hipLaunchKernelGGL(zero_kernel, dim3(grid), dim3(256), 0, s, reinterpret_cast<uint4*>(L.fp16), n16);
  return hipGetLastError();
}

hipError_t launch_knorm_shifts(const LayerDesc& L, const uint16_t* k, int32_t T, hipStream_t s) {
  if (!L.kshift) return hipSuccess;
  hipLaunchKernelGGL(knorm_shift_kernel, dim3(L.units), dim3(256), 0, s, k, T, L.kshift);
  return hipGetLastError();
}

// Grid of a block-walking prefill kernel: `rounds` times the workgroups
// resident at once, capped at one per block.  A grid of exactly one resident
// round leaves the kernel's length to the most loaded compute unit, and
// where the hardware places a workgroup depends on what ran before (the
// same launch measured up to 1.4x slower after one other short kernel);
// more, shorter workgroups let the dispatcher even the load out, at the cost
// of one unhidden block load per workgroup.
template <class Kernel>
hipError_t walk_grid(Kernel kern, int block, std::atomic<int>* cache, int rounds, int64_t blocks, int* grid) {
  int resident = 0;
  const hipError_t e = resident_blocks(kern, block, 0, cache, &resident);
  if (e != hipSuccess) return e;
  *grid = static_cast<int>(std::min<int64_t>(blocks, static_cast<int64_t>(resident) * rounds));
  return hipSuccess;
}

hipError_t launch_quantize(const LayerDesc& L, const QuantJob& job, hipStream_t s) {
  if (job.nblocks <= 0) return hipSuccess;
  // whole fresh blocks of the common schemes take the register kernels
  // (16-byte loads: the sources must be 16-byte aligned; row strides are
  // whole 256-byte rows); the other schemes take prefill_kernel, appends
  // into a partly filled block quantize_kernel
  const bool aligned = ((reinterpret_cast<uintptr_t>(job.k_src) | reinterpret_cast<uintptr_t>(job.v_src)) & 15) == 0;
  const bool kivi_layout = job.tok0 == 0 && !job.v_interleaved && job.cnt == kBlockTokens &&
                           job.last_cnt == kBlockTokens && aligned && L.k_hi == 0 && !L.k_inner && !L.k_hybrid &&
                           !L.nuq && L.outk == 0 && L.kshift == nullptr && L.v_group == 32 && L.kb != 3 && L.vb != 3;
  const bool kivi = kivi_layout && !job.rotate_v && (!L.v_tern || L.vb == 2);
  const bool kivi_rotated = kivi_layout && job.rotate_v && !L.v_tern &&
                            static_cast<int64_t>(job.nblocks) * L.units < (int64_t(1) << 31);
  const bool inner = job.tok0 == 0 && !job.v_interleaved && job.cnt == kBlockTokens &&
                     job.last_cnt == kBlockTokens && aligned && (L.k_hi == 0 || (L.kb == 4 && L.k_hi <= 2)) &&
                     L.k_inner && L.k_group == 64 &&
                     !L.nuq && !L.v_tern && L.outk == 0 && L.v_group == 32 && L.kb != 3 &&
                     L.vb != 3 && static_cast<int64_t>(job.nblocks) * L.units < (int64_t(1) << 31);
  const bool codebook = job.tok0 == 0 && !job.v_interleaved && !job.rotate_v && job.cnt == kBlockTokens &&
                        job.last_cnt == kBlockTokens && aligned && L.k_hi == 0 && !L.k_inner && !L.k_hybrid &&
                        L.nuq && !L.v_tern && L.outk == 2 && L.kshift == nullptr && L.v_group == 32 && L.kb == 3 &&
                        L.vb == 3 && static_cast<int64_t>(job.nblocks) * L.units < (int64_t(1) << 31);
  if (codebook) {
    static std::atomic<int> resident[kMaxDevices];
    int grid = 0;
    const hipError_t e =
        walk_grid(prefill_codebook_kernel, 256, resident, 8, static_cast<int64_t>(job.nblocks) * L.units, &grid);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(prefill_codebook_kernel, dim3(grid), dim3(256), 0, s, L, job);
    return hipGetLastError();
  }
  if (inner) {
    static std::atomic<int> resident[kMaxDevices];
    int grid = 0;
    const hipError_t e =
        walk_grid(prefill_inner_kernel<false>, 192, resident, 32, static_cast<int64_t>(job.nblocks) * L.units, &grid);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(prefill_inner_kernel<false>, dim3(grid), dim3(192), 0, s, L, job);
    return hipGetLastError();
  }
  if (kivi_rotated) {
    static std::atomic<int> resident[kMaxDevices];
    int grid = 0;
    const hipError_t e =
        walk_grid(prefill_inner_kernel<true>, 192, resident, 32, static_cast<int64_t>(job.nblocks) * L.units, &grid);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(prefill_inner_kernel<true>, dim3(grid), dim3(192), 0, s, L, job);
    return hipGetLastError();
  }
  if (kivi && static_cast<int64_t>(job.nblocks) * L.units < (int64_t(1) << 31)) {
    static std::atomic<int> resident[kMaxDevices];
    int grid = 0;
    const hipError_t e =
        walk_grid(prefill_kivi_kernel, 128, resident, 32, static_cast<int64_t>(job.nblocks) * L.units, &grid);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(prefill_kivi_kernel, dim3(grid), dim3(128), 0, s, L, job);
    return hipGetLastError();
  }
  if (job.tok0 == 0 && L.k_hi == 0 && aligned) {
    const size_t smem = prefill_smem(L.outk > 0);
    hipLaunchKernelGGL(prefill_kernel, dim3(job.nblocks, L.units), dim3(128), smem, s, L, job);
    return hipGetLastError();
  }
  const size_t smem = sizeof(QuantSmem);
  hipLaunchKernelGGL(quantize_kernel, dim3(job.nblocks, L.units), dim3(128), smem, s, L, job);
  return hipGetLastError();
}

hipError_t launch_copy_fp16(const LayerDesc& L, const CopyJob& job, hipStream_t s) {
  if (job.count <= 0) return hipSuccess;
  const size_t smem = sizeof(QuantSmem);
  const int grid = (job.count + kBlockTokens - 1) / kBlockTokens;
  hipLaunchKernelGGL(copy_fp16_kernel, dim3(grid, L.units), dim3(128), smem, s, L, job);
  return hipGetLastError();
}

}  // namespace kvq
