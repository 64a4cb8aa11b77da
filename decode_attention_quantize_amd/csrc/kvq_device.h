// kvq_device.h -- device helpers: binary16 rounding, packed-code access,
// cross-lane reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <cstdint>

#include "kvq_internal.h"

namespace kvq {

// ---------------------------------------------------------------- binary16
__device__ __forceinline__ float h2f(uint16_t h) {
  return __half2float(__ushort_as_half(h));
}
// fp32 -> fp16, round to nearest even (v_cvt_f16_f32 in the default mode).
__device__ __forceinline__ uint16_t f2h(float x) {
  return __half_as_ushort(__float2half_rn(x));
}

// fp64 -> fp16, round to nearest even, straight from the binary64 fields
// (no intermediate binary32 rounding).
__device__ __forceinline__ uint16_t d2h(double x) {
  const uint64_t b = static_cast<uint64_t>(__double_as_longlong(x));
  const uint16_t sign = static_cast<uint16_t>((b >> 48) & 0x8000u);
  const int e = static_cast<int>((b >> 52) & 0x7ff);
  const uint64_t frac = b & ((1ull << 52) - 1);
  if (e == 0x7ff) return sign | (frac ? 0x7e00 : 0x7c00);
  if (e == 0) return sign;  // binary64 subnormals are far below half of 2^-24
  const int E = e - 1023;
  if (E > 15) return sign | 0x7c00;
  const uint64_t sig = frac | (1ull << 52);
  // keep 10 fraction bits for normal results; subnormal results keep fewer
  const int shift = E >= -14 ? 42 : 28 - E;
  if (shift >= 64) return sign;
  uint64_t q = sig >> shift;
  const uint64_t rem = sig & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) ++q;
  if (E >= -14) {
    int ex = E + 15;
    if (q == 2048) {
      q = 1024;
      ++ex;
    }
    if (ex >= 31) return sign | 0x7c00;
    return sign | static_cast<uint16_t>((ex << 10) | static_cast<int>(q - 1024));
  }
  return sign | static_cast<uint16_t>(q);  // q == 1024 is the smallest normal
}

// fp16 value as an exact integer multiple of 2^-24.
__device__ __forceinline__ int64_t h2fixed(uint16_t h) {
  const int e = (h >> 10) & 0x1f;
  const int64_t m = h & 0x3ff;
  const int64_t mag = e == 0 ? m : ((1024 + m) << (e - 1));
  return (h & 0x8000) ? -mag : mag;
}

// ---------------------------------------------------------------- cross-lane
// xor-shuffle within a wave: ds_swizzle (bit mode) for masks below 32,
// ds_bpermute across the two 32-lane halves.
template <int M>
__device__ __forceinline__ int xshfl(int v) {
  if constexpr (M < 32) {
    return __builtin_amdgcn_ds_swizzle(v, 0x1f | (M << 10));
  } else {
    const int lane = __lane_id();
    return __builtin_amdgcn_ds_bpermute((lane ^ M) << 2, v);
  }
}
template <int M>
__device__ __forceinline__ float xshflf(float v) {
  return __int_as_float(xshfl<M>(__float_as_int(v)));
}
template <int M>
__device__ __forceinline__ int64_t xshfl64(int64_t v) {
  const int lo = xshfl<M>(static_cast<int>(v & 0xffffffff));
  const int hi = xshfl<M>(static_cast<int>(v >> 32));
  return (static_cast<int64_t>(hi) << 32) | static_cast<uint32_t>(lo);
}

template <int M>
__device__ __forceinline__ double xshfld(double v) {
  return __longlong_as_double(xshfl64<M>(__double_as_longlong(v)));
}

// One 128-channel row rotated by the normalized Hadamard matrix, c H v with
// c = fl64(1 / sqrt(128)), across a wavefront: lane l holds channels 2l and
// 2l + 1 as a binary16 pair.  The butterflies run in binary64, where every
// sum of up to 128 binary16 values is exact; the product with c is the one
// rounding before the binary16 result (round to nearest even).
__device__ __forceinline__ uint32_t hadamard_pair_rows(uint32_t w, double c, int lane) {
  const double a = static_cast<double>(h2f(static_cast<uint16_t>(w)));
  const double b = static_cast<double>(h2f(static_cast<uint16_t>(w >> 16)));
  double y0 = a + b, y1 = a - b;  // channel bit 0, inside the lane
  auto stage = [&](double p0, double p1, bool upper) __attribute__((always_inline)) {
    y0 = upper ? p0 - y0 : y0 + p0;
    y1 = upper ? p1 - y1 : y1 + p1;
  };
  // channel bits 1..6 are lane bits 0..5
  stage(xshfld<1>(y0), xshfld<1>(y1), (lane & 1) != 0);
  stage(xshfld<2>(y0), xshfld<2>(y1), (lane & 2) != 0);
  stage(xshfld<4>(y0), xshfld<4>(y1), (lane & 4) != 0);
  stage(xshfld<8>(y0), xshfld<8>(y1), (lane & 8) != 0);
  stage(xshfld<16>(y0), xshfld<16>(y1), (lane & 16) != 0);
  stage(xshfld<32>(y0), xshfld<32>(y1), (lane & 32) != 0);
  return static_cast<uint32_t>(d2h(y0 * c)) | (static_cast<uint32_t>(d2h(y1 * c)) << 16);
}

// Reductions over aligned groups of W lanes (W a power of two <= 64).
template <int W>
__device__ __forceinline__ void group_minmax(float& mn, float& mx) {
  if constexpr (W > 1) { mn = fminf(mn, xshflf<1>(mn)); mx = fmaxf(mx, xshflf<1>(mx)); }
  if constexpr (W > 2) { mn = fminf(mn, xshflf<2>(mn)); mx = fmaxf(mx, xshflf<2>(mx)); }
  if constexpr (W > 4) { mn = fminf(mn, xshflf<4>(mn)); mx = fmaxf(mx, xshflf<4>(mx)); }
  if constexpr (W > 8) { mn = fminf(mn, xshflf<8>(mn)); mx = fmaxf(mx, xshflf<8>(mx)); }
  if constexpr (W > 16) { mn = fminf(mn, xshflf<16>(mn)); mx = fmaxf(mx, xshflf<16>(mx)); }
  if constexpr (W > 32) { mn = fminf(mn, xshflf<32>(mn)); mx = fmaxf(mx, xshflf<32>(mx)); }
}
template <int W>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (W > 1) v = fmaxf(v, xshflf<1>(v));
  if constexpr (W > 2) v = fmaxf(v, xshflf<2>(v));
  if constexpr (W > 4) v = fmaxf(v, xshflf<4>(v));
  if constexpr (W > 8) v = fmaxf(v, xshflf<8>(v));
  if constexpr (W > 16) v = fmaxf(v, xshflf<16>(v));
  if constexpr (W > 32) v = fmaxf(v, xshflf<32>(v));
  return v;
}
template <int W>
__device__ __forceinline__ int64_t group_sum64(int64_t v) {
  if constexpr (W > 1) v += xshfl64<1>(v);
  if constexpr (W > 2) v += xshfl64<2>(v);
  if constexpr (W > 4) v += xshfl64<4>(v);
  if constexpr (W > 8) v += xshfl64<8>(v);
  if constexpr (W > 16) v += xshfl64<16>(v);
  if constexpr (W > 32) v += xshfl64<32>(v);
  return v;
}

// ---------------------------------------------------------------- packing
// Bit position of element e inside a pair-split word of b-bit fields
// (b = 2 or 4): even elements fill the low half-word, odd ones the high one.
__device__ __forceinline__ int pair_split_pos(int b, int e) {
  return ((e & 1) ? 16 : 0) + b * (e >> 1);
}

// Code of channel c in a token-major row (keys; 3-bit values).
// 3-bit codes live in 64 lane chunks of 24 bytes (one little-endian bit
// stream per chunk, element E at bits 3E..3E+2), so that a lane's operand
// for one matrix step is a contiguous 24-bit field.
//   keys:   chunk 16g + n, element 32*tile + 8*j + i = token n + 16*tile,
//           channel (j < 2 ? 16g + 8j : 64 + 16g + 8(j-2)) + i
//   values: chunk 16g + n, element 8*t + i = token 8g + i, channel 16t + n
__device__ __forceinline__ int chunk3_code(const uint8_t* codes, int lane, int e) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(codes) + 6 * lane;
  const int bit = 3 * e;
  const uint64_t pair = static_cast<uint64_t>(w[bit >> 5]) |
                        (static_cast<uint64_t>((bit >> 5) < 5 ? w[(bit >> 5) + 1] : 0u) << 32);
  return static_cast<int>((pair >> (bit & 31)) & 7u);
}
__device__ __forceinline__ int k3_code(const uint8_t* codes, int j, int c) {
  return chunk3_code(codes, c & 63, 2 * j + (c >> 6));
}
__device__ __forceinline__ int v3_code(const uint8_t* codes, int j, int c) {
  return chunk3_code(codes, 16 * (j >> 3) + (c & 15), 8 * (c >> 4) + (j & 7));
}

// Code of (token slot j, channel c) in a token-major row of 2/4/8-bit codes.
__device__ __forceinline__ int row_code(const uint8_t* row, int bits, int c) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(row);
  if (bits == 8) return row[c];
  const int n = 32 / bits;
  return (w[c / n] >> pair_split_pos(bits, c % n)) & ((1 << bits) - 1);
}

// Location of value (token slot j, channel c) in the lane-chunk layout.
struct VLoc {
  int word;   // 32-bit word index inside the v_codes section
  int shift;  // bit position inside the word
};
__device__ __forceinline__ VLoc v_loc(int bits, int j, int c) {
  const int lane = 16 * (j >> 3) + (c & 15);
  const int idx = 8 * (c >> 4) + (j & 7);  // element index in the chunk
  const int words_per_chunk = 2 * bits;
  if (bits == 8) return VLoc{lane * words_per_chunk + (idx >> 2), 8 * (idx & 3)};
  const int n = 32 / bits;
  return VLoc{lane * words_per_chunk + idx / n, pair_split_pos(bits, idx % n)};
}

__device__ __forceinline__ int v_code(const uint8_t* vc, int bits, int j, int c) {
  if (bits == 3) return v3_code(vc, j, c);
  const VLoc l = v_loc(bits, j, c);
  return (reinterpret_cast<const uint32_t*>(vc)[l.word] >> l.shift) & ((1 << bits) - 1);
}

// Dequantized value of a code with fp16 parameters (s, z); a set sign bit on
// s marks a symmetric group.
__device__ __forceinline__ float dequant(int code, uint16_t s, uint16_t z, int bits,
                                         const uint16_t* levels) {
  if (levels) return fmaf(h2f(levels[code]), h2f(s), h2f(z));
  if (s & 0x8000) return static_cast<float>(code - (1 << (bits - 1))) * h2f(s & 0x7fff);
  return fmaf(static_cast<float>(code), h2f(s), h2f(z));
}

}  // namespace kvq
