// kvq_host.cpp -- the C ABI: validation, buffer sizing, the sink / body /
// window token accounting of each layer, and kernel dispatch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "../../include/kvq.h"
#include "kvq_internal.h"

namespace kvq {
hipError_t launch_decode_generic(const LayerDesc& L, const DecodeJob& job, hipStream_t s);
hipError_t launch_decode_fast(const LayerDesc& L, const DecodeJob& job, hipStream_t s, bool* used);
int decode_fast_waves(const LayerDesc& L);  // resident wavefront target, 0 if the layer is not covered
hipError_t launch_decode_lut(const LayerDesc& L, const DecodeJob& job, hipStream_t s, bool* used);
int decode_lut_waves(const LayerDesc& L);
}  // namespace kvq

using kvq::LayerDesc;

namespace {

constexpr int kD = kvq::kHeadDim;

struct Layer {
  LayerDesc d{};
  bool bound = false;
  bool filled = false;  // prefilled at least once since binding
  int32_t n = 0, s_eff = 0, nb = 0, r = 0;
};

int32_t align_up(int64_t x, int64_t a) { return static_cast<int32_t>((x + a - 1) / a * a); }

bool pow2_in(int v, int lo, int hi) { return v >= lo && v <= hi && (v & (v - 1)) == 0; }

}  // namespace

struct kvq_cache {
  kvq_config cfg{};
  bool force_generic = false;  // KVQ_DECODE_KERNEL=generic: always use the LDS-staged decode
  int32_t G = 1, units = 1, F = 32, sink_cap = 0, win_cap = 0, nblk_cap = 0;
  std::vector<Layer> layers;
};

namespace {

kvq_status fill_layout(const kvq_cache& c, int kb, int vb, const uint16_t* cb, LayerDesc& d) {
  const kvq_config& g = c.cfg;
  d = LayerDesc{};
  d.B = g.batch;
  d.Hq = g.n_q_heads;
  d.Hkv = g.n_kv_heads;
  d.G = c.G;
  d.units = c.units;
  d.kb = kb;
  d.vb = vb;
  d.k_inner = g.k_mode == KVQ_K_INNER;
  d.k_group = g.k_group;
  d.v_group = g.v_group;
  d.k_hybrid = g.k_hybrid != 0;
  d.ratio_num = g.sym_ratio_num;
  d.ratio_den = g.sym_ratio_den;
  d.nuq = g.nuq != 0;
  d.outk = g.outliers_per_vector;
  d.v_had = g.v_mode == KVQ_V_HADAMARD;
  d.v_tern = g.v_mode == KVQ_V_TERNARY;
  d.k_hi = (g.k_mode == KVQ_K_INNER && kb == 4) ? g.k_hi_groups : 0;
  d.pre_rope = g.k_pre_rope != 0;
  d.rope_base = g.rope_base;
  if (cb) {
    std::memcpy(d.lev_k, cb, 16);
    std::memcpy(d.lev_v, cb + 8, 16);
  }
  d.had_scale = 1.0 / std::sqrt(static_cast<double>(kD));
  d.k_row_bytes = kD * kb / 8;
  int64_t off = 0;
  d.off_kc = 0;
  off = align_up(off + static_cast<int64_t>(kvq::kBlockTokens) * d.k_row_bytes, 16);
  d.off_km = static_cast<int32_t>(off);
  off = align_up(off + (d.k_inner ? kvq::kBlockTokens * (kD / d.k_group) * 4 : 2 * kD * 2), 16);
  d.off_vc = static_cast<int32_t>(off);
  off = align_up(off + kvq::kBlockTokens * kD * vb / 8, 16);
  d.off_vm = static_cast<int32_t>(off);
  off = align_up(off + 2 * (kD / d.v_group) * kvq::kBlockTokens * 2, 16);
  d.off_ko = static_cast<int32_t>(off);
  off = align_up(off + kvq::kBlockTokens * d.outk * 4, 16);
  d.off_vo = static_cast<int32_t>(off);
  off = align_up(off + kvq::kBlockTokens * d.outk * 4, 16);
  d.off_kx = static_cast<int32_t>(off);
  off = align_up(off + static_cast<int64_t>(kvq::kBlockTokens) * d.k_hi * (d.k_group / 2), 16);
  d.off_ks = static_cast<int32_t>(off);
  off = align_up(off + (d.k_hi ? kvq::kBlockTokens : 0), 16);
  d.rec_bytes = align_up(off, 128);
  d.nblk_cap = c.nblk_cap;
  d.sinks_cap = c.sink_cap;
  d.win_cap = c.win_cap;
  return KVQ_OK;
}

// bytes of the fp16 sink/window slots of all units (the key normalization
// shifts, when enabled, follow them in the same buffer)
size_t fp16_area_bytes(const kvq_cache& c) {
  return static_cast<size_t>(c.units) * 2 * (c.sink_cap + c.win_cap) * kD * sizeof(uint16_t);
}

int max_splits(const kvq_cache& c) {
  return std::min(kvq::kMaxBodySplits, c.nblk_cap) + kvq::kMaxFp16Splits;
}
size_t partials_bytes(const kvq_cache& c) {
  return static_cast<size_t>(c.units) * max_splits(c) * c.G * (kD + 2) * sizeof(float);
}

// Workspace: split partials (256-byte aligned), one arrival counter per unit
// (LDS-staged path), then the non-finite output row count.
size_t partials_padded(const kvq_cache& c) { return (partials_bytes(c) + 255) / 256 * 256; }
size_t workspace_bytes(const kvq_cache& c) {
  return partials_padded(c) + (static_cast<size_t>(c.units) + 1) * sizeof(uint32_t);
}
uint32_t* nonfinite_counter(const kvq_cache& c, void* ws) {
  return reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + partials_padded(c)) + c.units;
}

// A failed launch can leave some of a call's kernels queued and others not,
// so the layer's device contents no longer match any host state: the layer
// is marked empty and needs a new prefill (its appends and decodes return
// KVQ_ERR_STATE until then).
kvq_status device_error(Layer& L) {
  L.filled = false;
  L.n = L.s_eff = L.nb = L.r = 0;
  return KVQ_ERR_DEVICE;
}

bool valid_layer(const kvq_cache* c, int32_t layer) {
  return c && layer >= 0 && layer < static_cast<int32_t>(c->layers.size());
}

// Split plan.  The matrix-core path runs one wavefront per split and aims at
// one full round of resident wavefronts (fast_waves, from the kernel's ring
// depth and register budget); the 32-slot sink / window chunks get splits of
// their own after the body splits, inside the same round.
// The LDS-staged path walks the sink / window tokens in one extra split.
void plan_splits(const kvq_cache& c, const kvq::TokenState& st, int fast_waves, kvq::DecodeJob& j) {
  const bool fast = fast_waves > 0;
  const int nblk = (st.nb + kvq::kBlockTokens - 1) / kvq::kBlockTokens;
  j.fp16_split = 0;
  j.fp16_chunks = j.sink_chunks = j.win_chunk0 = 0;
  if (fast) {
    j.sink_chunks = (st.s_eff + kvq::kBlockTokens - 1) / kvq::kBlockTokens;
    int wchunks = 0;
    if (st.r > 0) {
      const int start = st.nb % c.win_cap;  // ring index of the oldest window token
      j.win_chunk0 = start / kvq::kBlockTokens;
      // chunks the live ring range touches; a range that wraps back into its
      // first chunk still visits each chunk once (the live mask covers both ends)
      wchunks = std::min((start + st.r - 1) / kvq::kBlockTokens - j.win_chunk0 + 1,
                         c.win_cap / kvq::kBlockTokens);
    }
    j.fp16_chunks = j.sink_chunks + wchunks;
  } else {
    j.fp16_split = st.s_eff + st.r > 0 ? 1 : 0;
  }
  // matrix-core path: the fp16 chunks get splits of their own after the body
  // splits, about two chunks per body split's worth of blocks, so that no
  // split carries both a full body share and fp16 chunks
  j.fp16_split0 = 0;
  j.fp16_nsplit = 1;
  if (nblk <= 0) {
    j.nsplit_body = 0;
    j.blocks_per_split = 1;
    if (fast && j.fp16_chunks > 0) j.fp16_nsplit = std::min(j.fp16_chunks, kvq::kMaxFp16Splits);
  } else {
    const int resident = std::max(1, (fast ? fast_waves : 2048) / std::max(1, c.units));
    int want = std::min({resident, kvq::kMaxBodySplits, std::max(1, nblk / 4)});
    if (fast && j.fp16_chunks > 0) {
      const int bps0 = (nblk + want - 1) / want;
      j.fp16_nsplit = std::min({kvq::kMaxFp16Splits, j.fp16_chunks,
                                std::max(1, (2 * j.fp16_chunks + bps0 - 1) / bps0)});
      // body + fp16 splits within one resident round and the merge's bound
      want = std::max(1, std::min({want, resident - j.fp16_nsplit, kvq::kMaxBodySplits - j.fp16_nsplit}));
    }
    j.blocks_per_split = (nblk + want - 1) / want;
    j.nsplit_body = (nblk + j.blocks_per_split - 1) / j.blocks_per_split;
  }
  if (fast) {
    j.fp16_split0 = j.nsplit_body;
    j.nsplit = j.nsplit_body + (j.fp16_chunks > 0 ? j.fp16_nsplit : 0);
    if (j.nsplit == 0) j.nsplit = 1;
  } else {
    j.nsplit = j.nsplit_body + j.fp16_split;
  }
}

enum class DecodeKind { kMatrixCore, kTables, kStaged };

// Kernel family and split plan of a decode over the layer's current tokens
// (matrix-core kernels first: uniform 2/4/8-bit; then the 3-bit table kernel
// with outliers and pre-RoPE keys for MHA layers; the LDS-staged kernel
// otherwise).  Fills j.st and the split fields.
DecodeKind plan_decode(const kvq_cache& c, const Layer& L, kvq::DecodeJob& j) {
  j.st = kvq::TokenState{L.n, L.s_eff, L.nb, L.r};
  j.new_k = j.new_v = nullptr;
  j.new_slot = -1;
  if (!c.force_generic) {
    int waves = kvq::decode_fast_waves(L.d);
    if (waves > 0) {
      plan_splits(c, j.st, waves, j);
      return DecodeKind::kMatrixCore;
    }
    waves = kvq::decode_lut_waves(L.d);
    if (waves > 0) {
      plan_splits(c, j.st, waves, j);
      return DecodeKind::kTables;
    }
  }
  plan_splits(c, j.st, 0, j);
  return DecodeKind::kStaged;
}

kvq_status launch_decode(const Layer& L, DecodeKind kind, const kvq::DecodeJob& j, hipStream_t s) {
  bool used = false;
  hipError_t e = hipSuccess;
  if (kind == DecodeKind::kMatrixCore)
    e = kvq::launch_decode_fast(L.d, j, s, &used);
  else if (kind == DecodeKind::kTables)
    e = kvq::launch_decode_lut(L.d, j, s, &used);
  else
    e = kvq::launch_decode_generic(L.d, j, s), used = true;
  if (!used) return KVQ_ERR_DEVICE;  // the planned kernel did not take the layer
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_DEVICE;
}

}  // namespace

extern "C" {

const char* kvq_status_str(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_ARG: return "invalid argument";
    case KVQ_ERR_CAPACITY: return "capacity exceeded";
    case KVQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case KVQ_ERR_STATE: return "invalid call order";
    case KVQ_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

kvq_status kvq_create(const kvq_config* cfg, const kvq_bitpair* layer_bits, const uint16_t* codebooks,
                      kvq_cache** out) {
  if (!cfg || !layer_bits || !out) return KVQ_ERR_ARG;
  *out = nullptr;
  const kvq_config& g = *cfg;
  if (g.batch < 1 || g.n_kv_heads < 1 || g.n_q_heads < 1 || g.n_layers < 1 || g.max_tokens < 1 ||
      g.sink_tokens < 0 || g.recent_window < 0 || g.head_dim < 1)
    return KVQ_ERR_ARG;
  if (g.n_q_heads % g.n_kv_heads) return KVQ_ERR_ARG;
  if (g.max_tokens > (1 << 24) || g.sink_tokens > g.max_tokens || g.recent_window > (1 << 20))
    return KVQ_ERR_ARG;
  if (g.k_mode != KVQ_K_PER_CHANNEL && g.k_mode != KVQ_K_INNER) return KVQ_ERR_ARG;
  if (g.v_mode != KVQ_V_PER_TOKEN && g.v_mode != KVQ_V_HADAMARD && g.v_mode != KVQ_V_TERNARY)
    return KVQ_ERR_ARG;
  if (g.outliers_per_vector < 0 || g.outliers_per_vector > kvq::kMaxOutliers) return KVQ_ERR_ARG;
  if (g.k_hybrid && (g.sym_ratio_num < 0 || g.sym_ratio_den <= 0)) return KVQ_ERR_ARG;
  if (g.k_pre_rope && !(g.rope_base > 0.f)) return KVQ_ERR_ARG;
  if (g.nuq && !codebooks) return KVQ_ERR_ARG;
  if (g.k_norm != 0 && g.k_norm != 1) return KVQ_ERR_ARG;
  const int G = g.n_q_heads / g.n_kv_heads;
  if (g.head_dim != kD) return KVQ_ERR_UNSUPPORTED;
  if (!pow2_in(G, 1, kvq::kMaxGroupRows)) return KVQ_ERR_UNSUPPORTED;
  if (g.k_mode == KVQ_K_PER_CHANNEL && g.k_group != kvq::kBlockTokens) return KVQ_ERR_UNSUPPORTED;
  if (g.k_mode == KVQ_K_INNER && !pow2_in(g.k_group, 16, 64)) return KVQ_ERR_UNSUPPORTED;
  if (!pow2_in(g.v_group, 16, 64)) return KVQ_ERR_UNSUPPORTED;
  if (g.nuq && g.k_hybrid) return KVQ_ERR_UNSUPPORTED;
  if (g.k_norm && g.k_mode != KVQ_K_INNER) return KVQ_ERR_UNSUPPORTED;
  if (g.v_mode == KVQ_V_TERNARY && g.nuq) return KVQ_ERR_UNSUPPORTED;
  if (g.k_hi_groups < 0) return KVQ_ERR_ARG;
  if (g.k_hi_groups > 0) {
    if (g.k_mode != KVQ_K_INNER || g.nuq || g.outliers_per_vector) return KVQ_ERR_UNSUPPORTED;
    if (g.k_hi_groups > kD / g.k_group) return KVQ_ERR_ARG;
  }
  for (int l = 0; l < g.n_layers; ++l) {
    const int kb = layer_bits[l].k_bits, vb = layer_bits[l].v_bits;
    if (g.nuq) {
      if (kb != 3 || vb != 3) return KVQ_ERR_UNSUPPORTED;
      for (int t = 0; t < 2; ++t) {
        const uint16_t* lv = codebooks + (l * 2 + t) * 8;
        for (int i = 0; i < 8; ++i)
          if ((lv[i] & 0x7c00) == 0x7c00) return KVQ_ERR_ARG;  // inf / NaN level
      }
    } else {
      auto ok = [](int b) { return b == 2 || b == 3 || b == 4 || b == 8; };
      if (!ok(kb) || !ok(vb)) return KVQ_ERR_UNSUPPORTED;
    }
    if (g.k_hybrid && kb < 2) return KVQ_ERR_UNSUPPORTED;
    if (g.v_mode == KVQ_V_TERNARY && vb != 2) return KVQ_ERR_UNSUPPORTED;
  }
  kvq_cache* c = new (std::nothrow) kvq_cache();
  if (!c) return KVQ_ERR_ARG;
  c->cfg = g;
  if (const char* e = std::getenv("KVQ_DECODE_KERNEL")) c->force_generic = std::strcmp(e, "generic") == 0;
  c->G = G;
  c->units = g.batch * g.n_kv_heads;
  c->F = g.k_mode == KVQ_K_PER_CHANNEL ? kvq::kBlockTokens : 1;
  // fp16 slot counts are multiples of 32: whole 32-slot chunks for the decode
  // and whole 8-slot groups for the interleaved value layout
  c->sink_cap = align_up(g.sink_tokens, kvq::kBlockTokens);
  c->win_cap = align_up(g.recent_window + c->F, kvq::kBlockTokens);
  c->nblk_cap = (g.max_tokens + kvq::kBlockTokens - 1) / kvq::kBlockTokens;
  c->layers.resize(g.n_layers);
  for (int l = 0; l < g.n_layers; ++l)
    fill_layout(*c, layer_bits[l].k_bits, layer_bits[l].v_bits,
                g.nuq ? codebooks + l * 16 : nullptr, c->layers[l].d);
  *out = c;
  return KVQ_OK;
}

kvq_status kvq_destroy(kvq_cache* c) {
  delete c;
  return KVQ_OK;
}

kvq_status kvq_layer_buffer_sizes(const kvq_cache* c, int32_t layer, size_t sizes[KVQ_NBUF]) {
  if (!valid_layer(c, layer) || !sizes) return KVQ_ERR_ARG;
  const LayerDesc& d = c->layers[layer].d;
  sizes[KVQ_BUF_BODY] = static_cast<size_t>(c->units) * c->nblk_cap * d.rec_bytes;
  sizes[KVQ_BUF_FP16] = fp16_area_bytes(*c) + (c->cfg.k_norm ? static_cast<size_t>(c->units) * kD : 0);
  return KVQ_OK;
}

kvq_status kvq_block_layout(const kvq_cache* c, int32_t layer, kvq_block_layout_t* o) {
  if (!valid_layer(c, layer) || !o) return KVQ_ERR_ARG;
  const LayerDesc& d = c->layers[layer].d;
  o->record_bytes = d.rec_bytes;
  o->k_codes = d.off_kc;
  o->k_meta = d.off_km;
  o->v_codes = d.off_vc;
  o->v_meta = d.off_vm;
  o->k_out = d.off_ko;
  o->v_out = d.off_vo;
  o->k_row_bytes = d.k_row_bytes;
  o->sink_cap = c->sink_cap;
  o->window_cap = c->win_cap;
  o->flush_tokens = c->F;
  o->k_ext = d.off_kx;
  o->k_sel = d.off_ks;
  return KVQ_OK;
}

kvq_status kvq_bind_layer(kvq_cache* c, int32_t layer, void* const bufs[KVQ_NBUF]) {
  if (!valid_layer(c, layer) || !bufs) return KVQ_ERR_ARG;
  for (int i = 0; i < KVQ_NBUF; ++i)
    if (!bufs[i] || (reinterpret_cast<uintptr_t>(bufs[i]) & 255)) return KVQ_ERR_ARG;
  Layer& L = c->layers[layer];
  L.d.body = static_cast<uint8_t*>(bufs[KVQ_BUF_BODY]);
  L.d.fp16 = static_cast<uint16_t*>(bufs[KVQ_BUF_FP16]);
  L.d.kshift = c->cfg.k_norm ? static_cast<int8_t*>(bufs[KVQ_BUF_FP16]) + fp16_area_bytes(*c) : nullptr;
  L.bound = true;
  L.filled = false;
  L.n = L.s_eff = L.nb = L.r = 0;
  return KVQ_OK;
}

kvq_status kvq_unbind_layer(kvq_cache* c, int32_t layer) {
  if (!valid_layer(c, layer)) return KVQ_ERR_ARG;
  Layer& L = c->layers[layer];
  L.d.body = nullptr;
  L.d.fp16 = nullptr;
  L.d.kshift = nullptr;
  L.bound = false;
  L.filled = false;
  L.n = L.s_eff = L.nb = L.r = 0;
  return KVQ_OK;
}

kvq_status kvq_workspace_size(const kvq_cache* c, size_t* bytes) {
  if (!c || !bytes) return KVQ_ERR_ARG;
  *bytes = workspace_bytes(*c);
  return KVQ_OK;
}

kvq_status kvq_decode_nonfinite_rows(const kvq_cache* c, void* workspace, void* stream, uint32_t* rows) {
  if (!c || !rows) return KVQ_ERR_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint32_t* dev = nullptr;
  if (workspace) {
    dev = nonfinite_counter(*c, workspace);
  } else {  // the static scratch of the current device (kvq_decode_attn_static)
    void* base = nullptr;
    if (kvq::static_scratch(&base) != hipSuccess) return KVQ_ERR_DEVICE;
    dev = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(base) + kvq::kStaticPartialsBytes) +
          kvq::kStaticMaxUnits;
  }
  uint32_t v = 0;
  if (hipMemcpyAsync(&v, dev, sizeof(v), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return KVQ_ERR_DEVICE;
  if (v != 0 && (hipMemsetAsync(dev, 0, sizeof(uint32_t), s) != hipSuccess ||
                 hipStreamSynchronize(s) != hipSuccess))
    return KVQ_ERR_DEVICE;
  *rows = v;
  return KVQ_OK;
}

kvq_status kvq_average_bits(const kvq_cache* c, double* code_bits, double* stored_bits) {
  if (!c) return KVQ_ERR_ARG;
  double code = 0.0, stored = 0.0;
  for (const Layer& L : c->layers) {
    const LayerDesc& d = L.d;
    const double kbits = d.kb + (d.k_hi ? (8.0 - d.kb) * d.k_hi / (kD / d.k_group) : 0.0);
    code += kbits + d.vb;
    stored += 8.0 * d.rec_bytes / (2.0 * kvq::kBlockTokens * kD);
  }
  const double nl = static_cast<double>(c->layers.size());
  if (code_bits) *code_bits = code / (2.0 * nl);
  if (stored_bits) *stored_bits = stored / nl;
  return KVQ_OK;
}

kvq_status kvq_layer_state(const kvq_cache* c, int32_t layer, int32_t* n, int32_t* sinks,
                           int32_t* body, int32_t* window) {
  if (!valid_layer(c, layer)) return KVQ_ERR_ARG;
  const Layer& L = c->layers[layer];
  if (n) *n = L.n;
  if (sinks) *sinks = L.s_eff;
  if (body) *body = L.nb;
  if (window) *window = L.r;
  return KVQ_OK;
}

kvq_status kvq_quantize_prefill(kvq_cache* c, int32_t layer, const void* k, const void* v, int32_t T,
                                void* /*workspace*/, void* stream) {
  if (!valid_layer(c, layer) || T < 0) return KVQ_ERR_ARG;
  Layer& L = c->layers[layer];
  if (!L.bound) return KVQ_ERR_STATE;
  if (T > 0 && (!k || !v)) return KVQ_ERR_ARG;
  if (T > c->cfg.max_tokens) return KVQ_ERR_CAPACITY;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int S = c->cfg.sink_tokens, W = c->cfg.recent_window, F = c->F;
  const int s_eff = std::min(S, T);
  const int avail = T - s_eff - W;
  const int nb = avail > 0 ? avail / F * F : 0;
  const int r = T - s_eff - nb;
  const auto* ks = static_cast<const uint16_t*>(k);
  const auto* vs = static_cast<const uint16_t*>(v);
  if (L.d.kshift) {
    // shifts from the whole prefill, before any body block is quantized
    // (read as 16-byte vectors)
    if (T > 0 && (reinterpret_cast<uintptr_t>(k) & 15)) return KVQ_ERR_ARG;
    if (kvq::launch_knorm_shifts(L.d, ks, T, s) != hipSuccess) return device_error(L);
  }
  if (nb > 0) {
    kvq::QuantJob j{};
    j.k_src = ks;
    j.v_src = vs;
    j.src_unit_stride = static_cast<int64_t>(T) * kD;
    j.src_t0 = s_eff;
    j.blk0 = 0;
    j.nblocks = (nb + kvq::kBlockTokens - 1) / kvq::kBlockTokens;
    j.tok0 = 0;
    j.cnt = kvq::kBlockTokens;
    j.last_cnt = nb - kvq::kBlockTokens * (j.nblocks - 1);
    j.rotate_v = L.d.v_had;
    if (kvq::launch_quantize(L.d, j, s) != hipSuccess) return device_error(L);
  }
  if (kvq::launch_zero_fp16(L.d, s) != hipSuccess) return device_error(L);
  kvq::CopyJob cj{};
  cj.k_src = ks;
  cj.v_src = vs;
  cj.src_unit_stride = static_cast<int64_t>(T) * kD;
  cj.s_eff = s_eff;
  cj.rotate_v = L.d.v_had;
  if (s_eff > 0) {
    cj.src_t0 = 0;
    cj.count = s_eff;
    cj.pos0 = 0;
    if (kvq::launch_copy_fp16(L.d, cj, s) != hipSuccess) return device_error(L);
  }
  if (r > 0) {
    cj.src_t0 = s_eff + nb;
    cj.count = r;
    cj.pos0 = s_eff + nb;
    if (kvq::launch_copy_fp16(L.d, cj, s) != hipSuccess) return device_error(L);
  }
  L.filled = true;
  L.n = T;
  L.s_eff = s_eff;
  L.nb = nb;
  L.r = r;
  return KVQ_OK;
}

kvq_status kvq_append_token(kvq_cache* c, int32_t layer, const void* k_new, const void* v_new,
                            void* stream) {
  if (!valid_layer(c, layer) || !k_new || !v_new) return KVQ_ERR_ARG;
  Layer& L = c->layers[layer];
  if (!L.bound || !L.filled) return KVQ_ERR_STATE;
  if (L.n + 1 > c->cfg.max_tokens) return KVQ_ERR_CAPACITY;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int S = c->cfg.sink_tokens, W = c->cfg.recent_window, F = c->F;
  const auto* ks = static_cast<const uint16_t*>(k_new);
  const auto* vs = static_cast<const uint16_t*>(v_new);
  if (L.s_eff < S) {
    // a prompt shorter than S: the token is the next sink (the body and the
    // window are still empty, so its position n equals s_eff)
    kvq::CopyJob cj{};
    cj.k_src = ks;
    cj.v_src = vs;
    cj.src_unit_stride = kD;
    cj.src_t0 = 0;
    cj.count = 1;
    cj.pos0 = L.n;
    cj.s_eff = L.s_eff + 1;
    cj.rotate_v = L.d.v_had;
    if (kvq::launch_copy_fp16(L.d, cj, s) != hipSuccess) return device_error(L);
    L.s_eff += 1;
    L.n += 1;
    return KVQ_OK;
  }
  if (F == 1 && W == 0) {
    // every token goes straight into the body
    kvq::QuantJob j{};
    j.k_src = ks;
    j.v_src = vs;
    j.src_unit_stride = kD;
    j.src_t0 = 0;
    j.blk0 = L.nb / kvq::kBlockTokens;
    j.nblocks = 1;
    j.tok0 = L.nb % kvq::kBlockTokens;
    j.cnt = j.last_cnt = 1;
    j.rotate_v = L.d.v_had;
    if (kvq::launch_quantize(L.d, j, s) != hipSuccess) return device_error(L);
    L.nb += 1;
    L.n += 1;
    return KVQ_OK;
  }
  kvq::CopyJob cj{};
  cj.k_src = ks;
  cj.v_src = vs;
  cj.src_unit_stride = kD;
  cj.src_t0 = 0;
  cj.count = 1;
  cj.pos0 = L.n;
  cj.s_eff = L.s_eff;
  cj.rotate_v = L.d.v_had;
  if (kvq::launch_copy_fp16(L.d, cj, s) != hipSuccess) return device_error(L);
  int nb = L.nb, r = L.r + 1;
  if (r == W + F) {
    // flush the oldest F window tokens (contiguous ring slots) into the body
    const int slots = c->sink_cap + c->win_cap;
    kvq::QuantJob j{};
    j.k_src = L.d.fp16 + static_cast<int64_t>(c->sink_cap) * kD;
    j.v_src = j.k_src + static_cast<int64_t>(slots) * kD;  // sink_cap is a multiple of 8
    j.v_interleaved = 1;
    j.src_unit_stride = static_cast<int64_t>(2) * slots * kD;
    j.src_t0 = nb % c->win_cap;
    j.blk0 = nb / kvq::kBlockTokens;
    j.nblocks = 1;
    j.tok0 = nb % kvq::kBlockTokens;
    j.cnt = j.last_cnt = F;
    j.rotate_v = 0;  // ring values are stored rotated already
    if (kvq::launch_quantize(L.d, j, s) != hipSuccess) return device_error(L);
    nb += F;
    r -= F;
  }
  L.nb = nb;
  L.r = r;
  L.n += 1;
  return KVQ_OK;
}

kvq_status kvq_decode_attn(kvq_cache* c, int32_t layer, const void* q, float* out, void* workspace,
                           void* stream) {
  if (!valid_layer(c, layer) || !q || !out || !workspace) return KVQ_ERR_ARG;
  Layer& L = c->layers[layer];
  if (!L.bound || !L.filled || L.n == 0) return KVQ_ERR_STATE;
  kvq::DecodeJob j{};
  const DecodeKind kind = plan_decode(*c, L, j);
  j.q = static_cast<const uint16_t*>(q);
  j.out = out;
  j.partials = static_cast<float*>(workspace);
  j.counters = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(workspace) + partials_padded(*c));
  j.nonfinite = nonfinite_counter(*c, workspace);
  j.ml_off = static_cast<int64_t>(c->units) * max_splits(*c) * c->G * kD;
  return launch_decode(L, kind, j, reinterpret_cast<hipStream_t>(stream));
}

kvq_status kvq_append_decode_attn(kvq_cache* c, int32_t layer, const void* k_new, const void* v_new,
                                  const void* q, float* out, void* workspace, void* stream) {
  if (!valid_layer(c, layer) || !k_new || !v_new || !q || !out || !workspace) return KVQ_ERR_ARG;
  Layer& L = c->layers[layer];
  if (!L.bound || !L.filled) return KVQ_ERR_STATE;
  if (L.n + 1 > c->cfg.max_tokens) return KVQ_ERR_CAPACITY;
  const int S = c->cfg.sink_tokens, W = c->cfg.recent_window, F = c->F;
  // One launch when the token only needs storing (the next sink, or a window
  // slot without a flush) and the layer decodes on the matrix-core kernel:
  // the decode reads the token from k_new / v_new (rotating its values when
  // the layer keeps them rotated; per-channel keys only) and stores it.
  // Otherwise the two calls this one stands for.
  const bool sink = L.s_eff < S;
  const bool plain = !(L.d.v_had && L.d.k_inner) && (sink || (!(F == 1 && W == 0) && L.r + 1 < W + F));
  if (plain && !c->force_generic && kvq::decode_fast_waves(L.d) > 0) {
    const int p = L.n;
    const int slot = sink ? p : c->sink_cap + (p - L.s_eff) % c->win_cap;
    if (sink)
      L.s_eff += 1;
    else
      L.r += 1;
    L.n += 1;
    kvq::DecodeJob j{};
    const DecodeKind kind = plan_decode(*c, L, j);
    j.q = static_cast<const uint16_t*>(q);
    j.out = out;
    j.partials = static_cast<float*>(workspace);
    j.counters = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(workspace) + partials_padded(*c));
    j.nonfinite = nonfinite_counter(*c, workspace);
    j.ml_off = static_cast<int64_t>(c->units) * max_splits(*c) * c->G * kD;
    j.new_k = static_cast<const uint16_t*>(k_new);
    j.new_v = static_cast<const uint16_t*>(v_new);
    j.new_slot = slot;
    const kvq_status e = launch_decode(L, kind, j, reinterpret_cast<hipStream_t>(stream));
    return e == KVQ_OK ? e : device_error(L);
  }
  const kvq_status e = kvq_append_token(c, layer, k_new, v_new, stream);
  if (e != KVQ_OK) return e;
  return kvq_decode_attn(c, layer, q, out, workspace, stream);
}

kvq_status kvq_decode_attn_static(kvq_cache* c, int32_t layer, const void* q, float* out, void* stream) {
  if (!valid_layer(c, layer) || !q || !out) return KVQ_ERR_ARG;
  Layer& L = c->layers[layer];
  if (!L.bound || !L.filled || L.n == 0) return KVQ_ERR_STATE;
  kvq::DecodeJob j{};
  const DecodeKind kind = plan_decode(*c, L, j);
  // partials sized by this call's split plan: o [units][nsplit][G][D] then
  // (max, sum) [units][nsplit][G][2] (the LDS-staged layout [..][D + 2] has
  // the same size); counters in the array's fixed tail
  const size_t need = static_cast<size_t>(c->units) * j.nsplit * c->G * (kD + 2) * sizeof(float);
  if (need > kvq::kStaticPartialsBytes || c->units > kvq::kStaticMaxUnits) return KVQ_ERR_CAPACITY;
  void* base = nullptr;
  if (kvq::static_scratch(&base) != hipSuccess) return KVQ_ERR_DEVICE;
  j.q = static_cast<const uint16_t*>(q);
  j.out = out;
  j.partials = static_cast<float*>(base);
  j.counters = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(base) + kvq::kStaticPartialsBytes);
  j.nonfinite = j.counters + kvq::kStaticMaxUnits;
  j.ml_off = static_cast<int64_t>(c->units) * j.nsplit * c->G * kD;
  return launch_decode(L, kind, j, reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"
