// kvq_mfma.h -- device helpers shared by the matrix-core decode kernels:
// MFMA operand types, 16-lane row reductions, LDS-ring reads and waits.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

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
constexpr float kLog2e = 1.4426950408889634f;

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

// 2^x with the hardware approximation (v_exp_f32, about 1 ulp); inputs are
// <= 0 here and results that would be fp32 subnormal only ever weigh tokens
// far below fp16 resolution of the row maximum
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Cross-lane steps inside rows of 16 lanes as DPP moves (VALU latency, no
// LDS round trip): quad permutes for xor 1 / xor 2, row rotations by 4 and 8
// (a rotation by 8 inside a 16-lane row is xor 8).
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E, kRowRor4 = 0x124, kRowRor8 = 0x128;
constexpr int kRowHalfMirror = 0x141;  // lane i <-> i ^ 7 inside each group of 8
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dppf<kQuadXor1>(v));
  v = fmaxf(v, dppf<kQuadXor2>(v));
  v = fmaxf(v, dppf<kRowRor4>(v));
  v = fmaxf(v, dppf<kRowRor8>(v));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dppf<kQuadXor1>(v);
  v += dppf<kQuadXor2>(v);
  v += dppf<kRowRor4>(v);
  v += dppf<kRowRor8>(v);
  return v;
}
// Exchanges between 16-lane rows and 32-lane halves (gfx950 permlane swaps).
// swap32(a, b) = ([a_lo, b_lo], [a_hi, b_hi]) over the halves of 32 lanes;
// swap16(a, b) = ([a0, b0, a2, b2], [a1, b1, a3, b3]) over the rows of 16.
__device__ __forceinline__ float2 swap32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float2 swap16(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  float2 r = swap16(v, v);
  v = fmaxf(r.x, r.y);
  r = swap32(v, v);
  return fmaxf(r.x, r.y);
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  float2 r = swap16(v, v);
  v = r.x + r.y;
  r = swap32(v, v);
  return r.x + r.y;
}
__device__ __forceinline__ float lane_bcast(float v, int src) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(v)));
}

// w <- fma(a, s, -w) per fp16 element, in place: the lo part of a product
// whose hi part w = fp16(a * s) is already in w.  Written out so that the
// caller's lane-dependent branch stays an exec-masked branch (an asm
// statement is not speculated into a select, which would cost one more VALU
// operation per word) and the negation stays an operand modifier; it is not
// volatile, so the scheduler may still move it within the block.
__device__ __forceinline__ void lo_in_place(half8& w, half8 a, half8 s) {
  u32x4 wv = __builtin_bit_cast(u32x4, w);
  const u32x4 av = __builtin_bit_cast(u32x4, a), sv = __builtin_bit_cast(u32x4, s);
#pragma unroll
  for (int e = 0; e < 4; ++e)
    asm("v_pk_fma_f16 %0, %1, %2, %0 neg_lo:[0,0,1] neg_hi:[0,0,1]" : "+v"(wv[e]) : "v"(av[e]), "v"(sv[e]));
  w = __builtin_bit_cast(half8, wv);
}

// w <- fma(z, s, fma(a, s, -w)) per fp16 element, in place: the lo part of
// a * s plus the product of a's residual z (each step rounds once; used by
// the lanes of the lo rows, exec-masked like lo_in_place).
__device__ __forceinline__ void lo_plus_in_place(half8& w, half8 a, half8 s, half8 z) {
  u32x4 wv = __builtin_bit_cast(u32x4, w);
  const u32x4 av = __builtin_bit_cast(u32x4, a), sv = __builtin_bit_cast(u32x4, s),
              zv = __builtin_bit_cast(u32x4, z);
#pragma unroll
  for (int e = 0; e < 4; ++e)
    asm("v_pk_fma_f16 %0, %1, %2, %0 neg_lo:[0,0,1] neg_hi:[0,0,1]\n\t"
        "v_pk_fma_f16 %0, %3, %2, %0"
        : "+v"(wv[e]) : "v"(av[e]), "v"(sv[e]), "v"(zv[e]));
  w = __builtin_bit_cast(half8, wv);
}

// Reads of the LDS ring filled by global_load_lds.  They are issued as
// inline-asm ds_reads: the compiler's wait insertion cannot see through the
// DMA writes precisely (it would drain every in-flight block), so the ring is
// guarded by explicit vmcnt waits, and each batch of reads is completed by
// lds_done(), which pins the loaded registers behind an lgkmcnt(0) wait.
typedef __attribute__((address_space(3))) uint8_t lds_u8;  // LDS byte (no generic-pointer checks)
// Cache policy of the ring's loads: nontemporal (nt).  Every record is read
// once per decode step, so keeping it out of the caches costs nothing, and
// streaming reads with nt reach about 7.0 TB/s on the device against about
// 6.1 TB/s with the default policy.
constexpr int kRingLoadPolicy = 2;
__device__ __forceinline__ void ring_load(const uint8_t* src, lds_u8* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, kRingLoadPolicy);
}
__device__ __forceinline__ uint32_t lds_off(const lds_u8* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}
template <int OFF>
__device__ __forceinline__ u32x4 dsr16(uint32_t a) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(a), "i"(OFF));
  return r;
}
// The weights' tile that a wavefront writes and then reads back goes through
// inline asm as well: a compiler-visible LDS access while ring blocks are in
// flight gets a wait for all of them.  One binary16 store, and a 16-byte load
// that waits for its data in the same statement.
__device__ __forceinline__ void dsw_h(uint32_t a, _Float16 v) {
  const uint32_t b = __builtin_bit_cast(uint16_t, v);
  asm volatile("ds_write_b16 %0, %1" : : "v"(a), "v"(b));
}
__device__ __forceinline__ u32x4 dsr16_now(uint32_t a) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(r) : "v"(a));
  return r;
}
template <int OFF>
__device__ __forceinline__ u32x2 dsr8(uint32_t a) {
  u32x2 r;
  asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(r) : "v"(a), "i"(OFF));
  return r;
}
template <int OFF>
__device__ __forceinline__ uint32_t dsr4(uint32_t a) {
  uint32_t r;
  asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(r) : "v"(a), "i"(OFF));
  return r;
}
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
template <class T>
__device__ __forceinline__ void pin(T& v) { asm volatile("" : "+v"(v)); }

// s_waitcnt vmcnt(N) leaving the other counters free
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

}  // namespace
}  // namespace kvq
