// kvq_decode_generic.hip -- split-context decode attention over the packed
// cache for every scheme (per-channel / inner keys, codebooks, sparse
// outliers, pre-RoPE keys, Hadamard-rotated values), with the log-sum-exp
// merge of the splits done by the last workgroup of each unit.
//
// One 128-thread workgroup per (split, unit); thread t owns channel t.  Each
// 32-token chunk is dequantized into LDS (keys rotated by RoPE at their
// absolute positions when stored pre-RoPE), scored against the unit's query
// rows, folded into a running (max, sum, output) per row (online softmax),
// and the values are accumulated by the thread that owns their channel.
#include <hip/hip_runtime.h>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int D = kHeadDim;
constexpr int PW = D + 2;  // partial record: o[D], m, l

template <int G>
struct DecSmem {
  float q[G][D];
  float k[kBlockTokens][D + 1];
  float p[G][kBlockTokens];
  float m[G], l[G], a[G];
  float o[D];
  int last;
};

struct Chunk {
  const uint8_t* rec;    // body block record, or nullptr for fp16 tokens
  int count;             // tokens in the chunk
  int first;             // body: first token index inside the block; fp16: virtual index
};

__device__ __forceinline__ void fp16_slot(const LayerDesc& L, const TokenState& st, int vi,
                                          int& slot, int& pos) {
  if (vi < st.s_eff) {
    slot = vi;
    pos = vi;
  } else {
    pos = st.s_eff + st.nb + (vi - st.s_eff);
    slot = L.sinks_cap + (pos - st.s_eff) % L.win_cap;
  }
}

__device__ __forceinline__ float load_k_body(const LayerDesc& L, const uint8_t* rec, int j, int c) {
  int code = L.kb == 3 ? k3_code(rec + L.off_kc, j, c) : row_code(rec + L.off_kc + j * L.k_row_bytes, L.kb, c);
  int bits = L.kb;
  const uint16_t* km = reinterpret_cast<const uint16_t*>(rec + L.off_km);
  uint16_t s, z;
  if (!L.k_inner) {
    s = km[c];
    z = km[D + c];
  } else {
    const int ng = D / L.k_group;
    const int g = c / L.k_group;
    s = km[(j * ng + g) * 2];
    z = km[(j * ng + g) * 2 + 1];
    if (L.k_hi) {
      // 8-bit group of a mixed layer: high nibble from the code plane, low
      // nibble from the token's slot for this group in k_ext
      const uint32_t sel = rec[L.off_ks + j];
      if ((sel >> g) & 1u) {
        const int slot = __popc(sel & ((1u << g) - 1u));
        const int cc = c % L.k_group;
        const uint32_t* w = reinterpret_cast<const uint32_t*>(rec + L.off_kx) +
                            (j * L.k_hi + slot) * (L.k_group / 8);
        code = (code << 4) | static_cast<int>((w[cc >> 3] >> pair_split_pos(4, cc & 7)) & 15u);
        bits = 8;
      }
    }
  }
  float x = dequant(code, s, z, bits, L.nuq ? L.lev_k : nullptr);
  if (L.outk) {
    const uint32_t* o = reinterpret_cast<const uint32_t*>(rec + L.off_ko) + j * L.outk;
    for (int i = 0; i < L.outk; ++i)
      if (static_cast<int>(o[i] & 0xffff) == c) x = h2f(static_cast<uint16_t>(o[i] >> 16));
  }
  return x;
}

__device__ __forceinline__ float load_v_body(const LayerDesc& L, const uint8_t* rec, int j, int c) {
  const int code = v_code(rec + L.off_vc, L.vb, j, c);
  const uint16_t* vm = reinterpret_cast<const uint16_t*>(rec + L.off_vm);
  const int ng = D / L.v_group;
  const int g = c / L.v_group;
  const uint16_t s = vm[g * kBlockTokens + j];
  const uint16_t z = vm[ng * kBlockTokens + g * kBlockTokens + j];
  float x = dequant(code, s, z, L.vb, L.nuq ? L.lev_v : nullptr);
  if (L.outk) {
    const uint32_t* o = reinterpret_cast<const uint32_t*>(rec + L.off_vo) + j * L.outk;
    for (int i = 0; i < L.outk; ++i)
      if (static_cast<int>(o[i] & 0xffff) == c) x = h2f(static_cast<uint16_t>(o[i] >> 16));
  }
  return x;
}

template <int G>
__global__ void __launch_bounds__(128) decode_generic_kernel(LayerDesc L, DecodeJob J) {
  __shared__ DecSmem<G> sm;
  const int t = threadIdx.x;
  const int u = blockIdx.y;
  const int sp = blockIdx.x;
  const int b = u / L.Hkv, h = u % L.Hkv;
  const int nsplit = J.nsplit;
  const TokenState st = J.st;
  const float scale = 1.0f / sqrtf(static_cast<float>(D));

  for (int r = 0; r < G; ++r)
    sm.q[r][t] = h2f(J.q[(static_cast<int64_t>(b) * L.Hq + h * G + r) * D + t]);
  if (t < G) {
    sm.m[t] = -INFINITY;
    sm.l[t] = 0.f;
  }
  float o[G];
  for (int r = 0; r < G; ++r) o[r] = 0.f;

  const bool fp16_part = J.fp16_split && sp == J.nsplit_body;
  const int nblk_body = st.nb / kBlockTokens + ((st.nb % kBlockTokens) ? 1 : 0);
  int c_begin, c_end;  // chunk range
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
  __syncthreads();

  for (int ch = c_begin; ch < c_end; ++ch) {
    const uint8_t* rec = nullptr;
    int count;
    if (fp16_part) {
      count = min(kBlockTokens, st.s_eff + st.r - ch * kBlockTokens);
    } else {
      rec = L.body + (static_cast<int64_t>(u) * L.nblk_cap + ch) * L.rec_bytes;
      count = min(kBlockTokens, st.nb - ch * kBlockTokens);
    }
    // keys of the chunk (body keys were normalized per channel at prefill:
    // scale back by 2^-shift, exact in fp32)
    const int ksh = (rec && L.kshift) ? L.kshift[static_cast<int64_t>(u) * D + t] : 0;
    for (int j = 0; j < count; ++j) {
      float x;
      if (rec) {
        x = ldexpf(load_k_body(L, rec, j, t), -ksh);
      } else {
        int slot, pos;
        fp16_slot(L, st, ch * kBlockTokens + j, slot, pos);
        x = h2f(kf[slot * D + t]);
      }
      sm.k[j][t] = x;
    }
    __syncthreads();
    if (L.pre_rope && t < D / 2) {
      const double theta = pow(static_cast<double>(L.rope_base), -2.0 * t / D);
      for (int j = 0; j < count; ++j) {
        int pos;
        if (rec) {
          pos = st.s_eff + ch * kBlockTokens + j;
        } else {
          int slot;
          fp16_slot(L, st, ch * kBlockTokens + j, slot, pos);
        }
        double sn, cs;
        sincos(static_cast<double>(pos) * theta, &sn, &cs);
        const float a = sm.k[j][t], bb = sm.k[j][t + D / 2];
        sm.k[j][t] = static_cast<float>(a * cs - bb * sn);
        sm.k[j][t + D / 2] = static_cast<float>(bb * cs + a * sn);
      }
    }
    __syncthreads();
    // scores
    for (int i = t; i < G * kBlockTokens; i += 128) {
      const int r = i / kBlockTokens, j = i % kBlockTokens;
      float s = -INFINITY;
      if (j < count) {
        float acc = 0.f;
        for (int c = 0; c < D; ++c) acc = fmaf(sm.q[r][c], sm.k[j][c], acc);
        s = acc * scale;
      }
      sm.p[r][j] = s;
    }
    __syncthreads();
    if (t < G) {
      float mx = -INFINITY;
      for (int j = 0; j < count; ++j) mx = fmaxf(mx, sm.p[t][j]);
      const float mn = fmaxf(sm.m[t], mx);
      sm.a[t] = expf(sm.m[t] - mn);  // exp(-inf) = 0 on the first chunk
      sm.m[t] = mn;
    }
    __syncthreads();
    for (int i = t; i < G * kBlockTokens; i += 128) {
      const int r = i / kBlockTokens, j = i % kBlockTokens;
      sm.p[r][j] = j < count ? expf(sm.p[r][j] - sm.m[r]) : 0.f;
    }
    __syncthreads();
    if (t < G) {
      float sum = 0.f;
      for (int j = 0; j < count; ++j) sum += sm.p[t][j];
      sm.l[t] = sm.l[t] * sm.a[t] + sum;
    }
    for (int r = 0; r < G; ++r) o[r] *= sm.a[r];
    for (int j = 0; j < count; ++j) {
      float x;
      if (rec) {
        x = load_v_body(L, rec, j, t);
      } else {
        int slot, pos;
        fp16_slot(L, st, ch * kBlockTokens + j, slot, pos);
        x = h2f(vf[vslot(slot, t)]);
      }
      for (int r = 0; r < G; ++r) o[r] = fmaf(sm.p[r][j], x, o[r]);
    }
    __syncthreads();
  }

  // partial of this split
  float* part = J.partials + (static_cast<int64_t>(u) * nsplit + sp) * G * PW;
  for (int r = 0; r < G; ++r) part[r * PW + t] = o[r];
  if (t < G) {
    part[t * PW + D] = sm.m[t];
    part[t * PW + D + 1] = sm.l[t];
  }
  __threadfence();
  __syncthreads();
  if (t == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(J.counters + u, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    sm.last = prev == static_cast<uint32_t>(nsplit - 1);
  }
  __syncthreads();
  if (!sm.last) return;
  __threadfence();

  // log-sum-exp merge of all splits of this unit
  const float* base = J.partials + static_cast<int64_t>(u) * nsplit * G * PW;
  for (int r = 0; r < G; ++r) {
    float M = -INFINITY;
    for (int i = 0; i < nsplit; ++i) M = fmaxf(M, __builtin_nontemporal_load(base + (i * G + r) * PW + D));
    float Ls = 0.f, acc = 0.f;
    bool bad = false;
    for (int i = 0; i < nsplit; ++i) {
      const float* pr = base + (i * G + r) * PW;
      const float mi = __builtin_nontemporal_load(pr + D);
      bad |= bad_partial(mi, __builtin_nontemporal_load(pr + D + 1));
      if (mi == -INFINITY) continue;
      const float w = expf(mi - M);
      Ls = fmaf(__builtin_nontemporal_load(pr + D + 1), w, Ls);
      acc = fmaf(__builtin_nontemporal_load(pr + t), w, acc);
    }
    float y = bad ? __uint_as_float(0x7fc00000u) : acc / Ls;
    if (L.v_had) {
      // o <- c H o (values were stored rotated)
      sm.o[t] = y;
      __syncthreads();
      for (int hh = 1; hh < D; hh <<= 1) {
        const float a = sm.o[t], bb = sm.o[t ^ hh];
        __syncthreads();
        sm.o[t] = (t & hh) ? bb - a : a + bb;
        __syncthreads();
      }
      y = sm.o[t] * static_cast<float>(L.had_scale);
      __syncthreads();
    }
    J.out[(static_cast<int64_t>(b) * L.Hq + h * G + r) * D + t] = y;
    if (__syncthreads_or(nonfinite_bits(y)) && t == 0) atomicAdd(J.nonfinite, 1u);
  }
  if (t == 0) J.counters[u] = 0;
}

template <int G>
hipError_t launch_g(const LayerDesc& L, const DecodeJob& j, hipStream_t s) {
  const int nsplit = j.nsplit;
  hipLaunchKernelGGL(decode_generic_kernel<G>, dim3(nsplit, L.units), dim3(128), 0, s, L, j);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_generic(const LayerDesc& L, const DecodeJob& job, hipStream_t s) {
  switch (L.G) {
    case 1: return launch_g<1>(L, job, s);
    case 2: return launch_g<2>(L, job, s);
    case 4: return launch_g<4>(L, job, s);
    case 8: return launch_g<8>(L, job, s);
    case 16: return launch_g<16>(L, job, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
