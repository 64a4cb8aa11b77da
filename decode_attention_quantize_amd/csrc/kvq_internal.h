// kvq_internal.h -- descriptors shared by the host entry points and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

namespace kvq {

constexpr int kBlockTokens = 32;  // tokens per body block (= per-channel key group)
constexpr int kHeadDim = 128;
constexpr int kMaxGroupRows = 16;  // query heads per kv head
constexpr int kMaxOutliers = 8;

// Everything a kernel needs to read or write one layer, passed by value.
struct LayerDesc {
  // shapes
  int32_t B, Hq, Hkv, G;  // G = Hq / Hkv
  int32_t units;          // B * Hkv
  // scheme
  int32_t kb, vb;
  int32_t k_inner, k_group, v_group;
  int32_t k_hybrid, ratio_num, ratio_den;
  int32_t nuq, outk, v_had, pre_rope;
  int32_t v_tern;  // values as ternary levels {-s, 0, s} in 2-bit codes (z = -s)
  int32_t k_hi;    // mixed 4/8-bit inner key groups: 8-bit groups per token (0: none)
  float rope_base;
  uint16_t lev_k[8], lev_v[8];
  double had_scale;  // fl64(1/sqrt(D)), computed on the host
  // record layout
  int32_t rec_bytes, k_row_bytes;
  int32_t off_kc, off_km, off_vc, off_vm, off_ko, off_vo;
  int32_t off_kx, off_ks;  // mixed key groups: low code nibbles, per-token group mask
  int32_t nblk_cap;  // blocks per unit
  // fp16 area
  int32_t sinks_cap, win_cap;  // slots per unit, both multiples of 32
  // buffers
  uint8_t* body;     // [units][nblk_cap][rec_bytes]
  uint16_t* fp16;    // per unit: K [slots][D], then V [slots / 8][D][8]
  int8_t* kshift;    // per-channel key normalization shifts [units][D], or null
};

// Element offset of value (slot, channel) inside a unit's fp16 value area:
// eight consecutive slots of one channel are adjacent, which is the operand
// order of a matrix-core product over tokens.
__host__ __device__ inline int64_t vslot(int slot, int c) {
  return static_cast<int64_t>(slot >> 3) * (kHeadDim * 8) + c * 8 + (slot & 7);
}

// Token state of a layer at a decode call.
struct TokenState {
  int32_t n, s_eff, nb, r;
};

// ---------------------------------------------------------------- launchers
// Quantize tokens into body blocks.  For each unit u and each of nblocks
// blocks: block index blk0 + i, slots [tok0, tok0 + cnt) (cnt tokens, all in
// the same block when nblocks == 1, else cnt == 32 for every block but the
// last, which holds last_cnt).  Source token j of block i of unit u is at
// src + u * src_unit_stride + (src_t0 + 32*i + j) * D (fp16 elements); the
// value source is rotated first when rotate_v.
struct QuantJob {
  const uint16_t* k_src;
  const uint16_t* v_src;
  int64_t src_unit_stride;  // elements
  int32_t src_t0;
  int32_t blk0, nblocks, tok0, cnt, last_cnt;
  int32_t rotate_v;
  int32_t v_interleaved;
};
hipError_t launch_quantize(const LayerDesc& L, const QuantJob& job, hipStream_t s);

// Copy fp16 tokens into the sink/window area: for each unit, tokens
// [src_t0, src_t0 + count) of the source go to slots slot_of(t) where sink
// positions p < s_eff use slot p and window positions use
// sinks_cap + ((p - s_eff) mod win_cap); positions are src_pos0 + j.
struct CopyJob {
  const uint16_t* k_src;
  const uint16_t* v_src;
  int64_t src_unit_stride;
  int32_t src_t0, count, pos0, s_eff;
  int32_t rotate_v;
};
hipError_t launch_copy_fp16(const LayerDesc& L, const CopyJob& job, hipStream_t s);

// Zero a layer's fp16 area (every unit), so that slots never written hold
// finite values.
hipError_t launch_zero_fp16(const LayerDesc& L, hipStream_t s);
// Per-channel key normalization shifts of every unit from its T prefill
// tokens (k: fp16 [units][T][D]); T == 0 writes zero shifts.
hipError_t launch_knorm_shifts(const LayerDesc& L, const uint16_t* k, int32_t T, hipStream_t s);

// Decode attention.  grid.x = nsplit wavefront groups per unit.
// partials: LDS-staged path [units][nsplit][G][D + 2] fp32; matrix-core path
// o [units][nsplit][G][D] then (max, sum) [units][nsplit][G][2] at ml_off.
// counters: [units] uint32 (zero on entry, zero on exit).
constexpr int kMaxBodySplits = 256;
constexpr int kMaxFp16Splits = 8;
struct DecodeJob {
  const uint16_t* q;  // [B][Hq][D]
  float* out;         // [B][Hq][D]
  float* partials;
  uint32_t* counters;
  TokenState st;
  int32_t nsplit;
  int32_t nsplit_body;    // the first nsplit_body splits own body blocks
  int32_t blocks_per_split;
  // sink / window tokens.  LDS-staged path: when fp16_split, split
  // nsplit_body walks them in position order.  Matrix-core path: 32-slot
  // chunk c < fp16_chunks goes to split fp16_split0 + c % fp16_nsplit;
  // chunks below sink_chunks are sink slots 32c.., the others window ring
  // chunks win_chunk0, +1, ... (mod win_cap / 32); slots holding no live
  // token are masked.
  int32_t fp16_split;
  int32_t fp16_chunks, sink_chunks, win_chunk0;
  int32_t fp16_split0, fp16_nsplit;
  int64_t ml_off;         // matrix-core path: float offset of the (max, sum) records
  uint32_t* nonfinite;    // count of output rows with a non-finite element (never reset here)
  // Appended token carried by the decode launch (matrix-core path only):
  // new_slot >= 0 is the fp16 slot of position st.n - 1, whose key and value
  // ([units][D] fp16) the chunk holding that slot reads from new_k / new_v
  // and writes into the slot; -1 when the token was stored beforehand.
  const uint16_t* new_k;
  const uint16_t* new_v;
  int32_t new_slot;
};
// Log-sum-exp merge of matrix-core split partials into job.out (one
// (unit, query row) per workgroup); undoes the value rotation when set.
hipError_t launch_decode_merge(const LayerDesc& L, const DecodeJob& job, hipStream_t s);

// Workgroups of `block` threads and `smem` bytes of dynamic LDS resident on
// the current device in one round (runtime occupancy x CU count); for a
// 64-thread kernel, resident wavefronts.  `cache` is the caller's per-kernel
// table, indexed by device; concurrent first calls store the same value.
constexpr int kMaxDevices = 64;
template <class Kernel>
hipError_t resident_blocks(Kernel kern, int block, size_t smem, std::atomic<int>* cache, int* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return hipErrorInvalidDevice;
  if (dev < kMaxDevices) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) {
      *out = v;
      return hipSuccess;
    }
  }
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, block, smem) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return hipErrorInvalidValue;
  const int v = (per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
  if (dev < kMaxDevices) cache[dev].store(v, std::memory_order_relaxed);
  *out = v;
  return hipSuccess;
}
template <class Kernel>
hipError_t resident_waves(Kernel kern, std::atomic<int>* cache, int* out) {
  return resident_blocks(kern, 64, 0, cache, out);
}

// Static decode scratch (kvq_static.hip): a fixed device array per GPU for the
// decode entry point that allocates nothing.  Partials first, then a fixed
// tail of per-unit arrival counters whose last word is the non-finite row
// count.
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
constexpr size_t kStaticCounterBytes = size_t(64) << 10;
constexpr size_t kStaticPartialsBytes = kStaticScratchBytes - kStaticCounterBytes;
constexpr int kStaticMaxUnits = static_cast<int>(kStaticCounterBytes / 4) - 1;
hipError_t static_scratch(void** out);

// Device helpers: tests for non-finite values on the bit pattern.  The bits
// pass through an empty asm statement, so that no floating-point assumption
// (the decode files are compiled without NaN semantics, under which a test
// of a value's bits could be rewritten as a compare that is false for NaN)
// can reach the test.
__device__ __forceinline__ uint32_t opaque_bits(float x) {
  uint32_t b = __float_as_uint(x);
  asm volatile("" : "+v"(b));
  return b;
}
__device__ __forceinline__ bool nonfinite_bits(float x) { return (opaque_bits(x) & 0x7f800000u) == 0x7f800000u; }
__device__ __forceinline__ bool nan_bits(float x) { return (opaque_bits(x) & 0x7fffffffu) > 0x7f800000u; }
// A split partial (max m, sum l) that cannot be trusted: a NaN maximum, or a
// non-finite sum (scores that came out NaN -- a query / key-scale product
// beyond binary16 -- leave the split's maximum at its start value and make
// its sum NaN).  The merge then writes the row as NaN and counts it, instead
// of dropping the split.
__device__ __forceinline__ bool bad_partial(float m, float l) { return nan_bits(m) || nonfinite_bits(l); }

}  // namespace kvq
