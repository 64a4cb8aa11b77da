// kvq_oracle.cpp -- plain, slow, CPU reference for the packed-KV quantizers,
// the cache state machine and decode attention.
//
// TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke entry point and
// the benchmark's CPU-baseline leg may load this library.  It shares no code
// with the GPU library: no headers, helpers, tables or constants.
//
// Arithmetic rules (the pages fix no precision for these steps, so these are
// readings): quantizer parameters and codes follow an fp32 formula with IEEE
// division and round-half-even, results rounded to fp16 with
// round-to-nearest-even; dequantization, RoPE and attention run in binary64.
// Build: g++ -O2 -std=c++17 -ffp-contract=off (no -ffast-math, no SIMD intrinsics).
//
// Sources (pages as titled):
//  * KVTuner review (velog): per-channel asymmetric keys (observation 2);
//    keys deserve more bits (observation 3); candidate pairs
//    {KV8,K8V4,KV4,K4V2,KV2} (method step 1); average-bits objective
//    f_m(P) = sum(P)/2L (method step 0); static table applied online (step 4).
//  * KVQuant (hotpaper, 2401.18079): per-channel keys, pre-RoPE keys,
//    per-layer non-uniform datatype, per-vector dense-and-sparse outliers at
//    about 1% (abstract; technical approach list).
//  * RateQuant (gist.science): KIVI keys per channel, values per token
//    (section 3, K/V separation).
//  * InnerQ (euno.news, 2602.23200): inner-dimension groups (method 1),
//    per-group symmetric/asymmetric choice from local statistics (method 2),
//    fp16 recent and sink windows (method 4), one-time per-channel key
//    normalization computed at prefill and folded into the query (method 4;
//    key contributions list); 4-bit and 8-bit groups mixed in one layer
//    (limitations and future work).
//  * Hadamard 2-bit values (aitrends.kr): rotate values by a Hadamard matrix,
//    quantize uniformly to 2 bits, undo the rotation after the attention sum
//    (TL;DR; section details; glossary).
//
// Functions whose result no independent pin fixes are marked "parity unpinned".

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

namespace {

// ---------------------------------------------------------------- binary16
// Exact widening of an IEEE binary16 pattern.
double f16_to_f64(uint16_t h) {
  const int sgn = h >> 15;
  const int e = (h >> 10) & 0x1f;
  const int m = h & 0x3ff;
  double v;
  if (e == 0)
    v = std::ldexp(static_cast<double>(m), -24);
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = std::ldexp(static_cast<double>(m + 1024), e - 25);
  return sgn ? -v : v;
}

// Round a binary64 value to binary16, round-to-nearest, ties to even.
// The value is scaled by the binary16 quantum of its binade (a power of two,
// so the scaling is exact), rounded to an integer with nearbyint in the
// default rounding mode, and re-assembled.  Overflow goes to infinity.
uint16_t f64_to_f16(double x) {
  if (std::isnan(x)) return 0x7e00;
  const uint16_t sgn = std::signbit(x) ? 0x8000 : 0;
  const double a = std::fabs(x);
  if (a >= 65520.0) return sgn | 0x7c00;  // 65520 is the tie between 65504 and 2^16
  if (a == 0.0) return sgn;
  int e2;
  std::frexp(a, &e2);        // a in [2^(e2-1), 2^e2)
  int E = e2 - 1;
  if (E < -14) E = -14;      // subnormal binade shares the quantum 2^-24
  const double quantum = std::ldexp(1.0, E - 10);
  double r = std::nearbyint(a / quantum);
  if (r >= 2048.0) {         // rounded up into the next binade
    r = 1024.0;
    E += 1;
  }
  if (r < 1024.0) return sgn | static_cast<uint16_t>(r);  // subnormal (E == -14)
  return sgn | static_cast<uint16_t>(((E + 15) << 10) | (static_cast<int>(r) - 1024));
}

inline float h2f(uint16_t h) { return static_cast<float>(f16_to_f64(h)); }

// ---------------------------------------------------------------- quantizers
// Uniform asymmetric quantizer over one group.  Statistics skip members
// flagged in excl (sparse outliers).  s = fp16(fl32(fl32(max-min)/Q)),
// z = min; code = clamp(rne(fl32(fl32(x-z)/s)), 0, Q); a non-zero range whose
// scale underflows fp16 gets the smallest subnormal; a constant group keeps
// s = 0 and all codes 0.  Groups with no included member get (0, 0), codes 0.
void quant_asym(const uint16_t* x, const uint8_t* excl, int n, int bits, uint8_t* codes,
                uint16_t* s_out, uint16_t* z_out) {
  const int Q = (1 << bits) - 1;
  bool any = false;
  float mn = 0.f, mx = 0.f;
  for (int i = 0; i < n; ++i) {
    if (excl && excl[i]) continue;
    const float v = h2f(x[i]);
    if (!any) {
      mn = mx = v;
      any = true;
    } else {
      if (v < mn) mn = v;
      if (v > mx) mx = v;
    }
  }
  if (!any) {
    *s_out = 0;
    *z_out = 0;
    for (int i = 0; i < n; ++i) codes[i] = 0;
    return;
  }
  const float range = mx - mn;
  const float sf = range / static_cast<float>(Q);
  uint16_t s = f64_to_f16(static_cast<double>(sf));
  if (mx > mn && s == 0) s = 0x0001;
  *s_out = s;
  *z_out = f64_to_f16(static_cast<double>(mn));
  const float sv = h2f(s);
  for (int i = 0; i < n; ++i) {
    if (s == 0) {
      codes[i] = 0;
      continue;
    }
    const float d = h2f(x[i]) - mn;
    const float t = d / sv;
    float r = std::nearbyint(t);
    if (!(r > 0.f)) r = 0.f;
    if (r > static_cast<float>(Q)) r = static_cast<float>(Q);
    codes[i] = static_cast<uint8_t>(r);
  }
}

// Uniform symmetric quantizer: a = max|x|, Qs = 2^(b-1)-1,
// s = fp16(fl32(a/Qs)); code = clamp(rne(fl32(x/s)), -Qs, Qs) + 2^(b-1).
// The stored scale carries its sign bit set as the "symmetric" flag; the
// zero slot holds +0.  An all-zero group stores -0 and codes 0.
void quant_sym(const uint16_t* x, int n, int bits, uint8_t* codes, uint16_t* s_out,
               uint16_t* z_out) {
  const int Qs = (1 << (bits - 1)) - 1;
  const int mid = 1 << (bits - 1);
  float a = 0.f;
  for (int i = 0; i < n; ++i) {
    const float v = std::fabs(h2f(x[i]));
    if (v > a) a = v;
  }
  const float sf = a / static_cast<float>(Qs);
  uint16_t s = f64_to_f16(static_cast<double>(sf));
  if (a > 0.f && s == 0) s = 0x0001;
  *s_out = static_cast<uint16_t>(s | 0x8000);
  *z_out = 0;
  const float sv = h2f(s);
  for (int i = 0; i < n; ++i) {
    if (s == 0) {
      codes[i] = 0;
      continue;
    }
    const float t = h2f(x[i]) / sv;
    float r = std::nearbyint(t);
    if (r < static_cast<float>(-Qs)) r = static_cast<float>(-Qs);
    if (r > static_cast<float>(Qs)) r = static_cast<float>(Qs);
    codes[i] = static_cast<uint8_t>(static_cast<int>(r) + mid);
  }
}

// Ternary values, the Hadamard 2-bit page's first attempt (about 1.58 bits
// per value; section details, last paragraph), kept as a negative control.
// Reading: per-token groups, levels {-s, 0, +s} with s = max |x| over the
// group's non-outlier members (an fp16 value, so exact), code =
// clamp(rne(fl32(x / s)), -1, 1) + 1 stored as a 2-bit code with z = -s, so
// that the plain asymmetric dequantization code * s + z yields the level.
// An all-zero group has s = 0, z = -0 and code 1.
void quant_tern(const uint16_t* x, const uint8_t* excl, int n, uint8_t* codes, uint16_t* s_out,
                uint16_t* z_out) {
  float a = 0.f;
  for (int i = 0; i < n; ++i) {
    if (excl && excl[i]) continue;
    const float v = std::fabs(h2f(x[i]));
    if (v > a) a = v;
  }
  const uint16_t s = f64_to_f16(static_cast<double>(a));
  *s_out = s;
  *z_out = static_cast<uint16_t>(s ^ 0x8000);
  const float sv = h2f(s);
  for (int i = 0; i < n; ++i) {
    if (s == 0) {
      codes[i] = 1;
      continue;
    }
    float r = std::nearbyint(h2f(x[i]) / sv);
    if (r < -1.f) r = -1.f;
    if (r > 1.f) r = 1.f;
    codes[i] = static_cast<uint8_t>(static_cast<int>(r) + 1);
  }
}

// Hybrid choice (InnerQ method 2): symmetric when the group is centred on
// zero.  Reading: |mean| / range <= ratio, evaluated exactly as
// den*|sum| <= num*g*(max-min) on fp16 values taken as integers in units of
// 2^-24 (int64 sums are exact and order independent); ratio = num/den.
bool hybrid_is_sym(const uint16_t* x, int n, int64_t num, int64_t den) {
  int64_t sum = 0, mn = 0, mx = 0;
  for (int i = 0; i < n; ++i) {
    const int64_t v = static_cast<int64_t>(std::ldexp(f16_to_f64(x[i]), 24));
    sum += v;
    if (i == 0 || v < mn) mn = v;
    if (i == 0 || v > mx) mx = v;
  }
  const int64_t lhs = den * (sum < 0 ? -sum : sum);
  const int64_t rhs = num * static_cast<int64_t>(n) * (mx - mn);
  return lhs <= rhs;
}

// Non-uniform quantizer over 8 sorted fp16 levels in [0,1]: the group is
// normalised by (min, range): s = fp16(fl32(max-min)), z = min,
// u = fl32(fl32(x-z)/s), code = #{j : u > fl32(fl32(L_j+L_j+1)*0.5)}
// (nearest level, ties to the lower one); a scale that overflows fp16
// saturates to 65504.  Reading: the pages give only a
// "per-layer sensitivity-weighted non-uniform datatype", not its range or
// normalisation.
void quant_nuq(const uint16_t* x, const uint8_t* excl, int n, const uint16_t* levels,
               uint8_t* codes, uint16_t* s_out, uint16_t* z_out) {
  bool any = false;
  float mn = 0.f, mx = 0.f;
  for (int i = 0; i < n; ++i) {
    if (excl && excl[i]) continue;
    const float v = h2f(x[i]);
    if (!any) {
      mn = mx = v;
      any = true;
    } else {
      if (v < mn) mn = v;
      if (v > mx) mx = v;
    }
  }
  if (!any) {
    *s_out = 0;
    *z_out = 0;
    for (int i = 0; i < n; ++i) codes[i] = 0;
    return;
  }
  const float range = mx - mn;
  uint16_t s = f64_to_f16(static_cast<double>(range));
  if (s == 0x7c00) s = 0x7bff;  // reading: a range beyond fp16 saturates to 65504
  if (mx > mn && s == 0) s = 0x0001;
  *s_out = s;
  *z_out = f64_to_f16(static_cast<double>(mn));
  float mid[7];
  for (int j = 0; j < 7; ++j) {
    const float sum = h2f(levels[j]) + h2f(levels[j + 1]);
    mid[j] = sum * 0.5f;
  }
  const float sv = h2f(s);
  for (int i = 0; i < n; ++i) {
    if (s == 0) {
      codes[i] = 0;
      continue;
    }
    const float d = h2f(x[i]) - mn;
    const float u = d / sv;
    int c = 0;
    for (int j = 0; j < 7; ++j)
      if (u > mid[j]) ++c;
    codes[i] = static_cast<uint8_t>(c);
  }
}

// Top-k by magnitude of one vector (KVQuant per-vector dense-and-sparse):
// descending |x|, lower index first on equal magnitude; returned in
// ascending column order.
void topk_cols(const uint16_t* row, int d, int k, int32_t* cols) {
  std::vector<int32_t> idx(d);
  std::vector<double> mag(d);  // |x| widened once per element
  for (int i = 0; i < d; ++i) {
    idx[i] = i;
    mag[i] = std::fabs(f16_to_f64(row[i]));
  }
  std::stable_sort(idx.begin(), idx.end(), [&](int32_t a, int32_t b) { return mag[a] > mag[b]; });
  std::vector<int32_t> top(idx.begin(), idx.begin() + k);
  std::sort(top.begin(), top.end());
  for (int i = 0; i < k; ++i) cols[i] = top[i];
}

// Sylvester Hadamard entry (+1/-1) of order d (a power of two).
inline int had(int i, int j) { return (__builtin_popcount(static_cast<unsigned>(i & j)) & 1) ? -1 : 1; }

// v' = fp16(fl64(S * c)) with S = H v summed exactly in binary64 (fp16 inputs
// are integers in units of 2^-24 below 2^16, so every partial sum of d <= 512
// terms is exact) and c = fl64(1/sqrt(d)).
void hadamard_fp16(const uint16_t* v, int d, uint16_t* out) {
  const double c = 1.0 / std::sqrt(static_cast<double>(d));
  std::vector<double> x(d);
  for (int j = 0; j < d; ++j) x[j] = f16_to_f64(v[j]);  // exact widening, once per element
  for (int i = 0; i < d; ++i) {
    double s = 0.0;
    for (int j = 0; j < d; ++j) s += had(i, j) * x[j];
    out[i] = f64_to_f16(s * c);
  }
}

// c H v in binary64 (no fp16 step).
void hadamard_f64(const double* v, int d, double* out) {
  const double c = 1.0 / std::sqrt(static_cast<double>(d));
  for (int i = 0; i < d; ++i) {
    double s = 0.0;
    for (int j = 0; j < d; ++j) s += had(i, j) * v[j];
    out[i] = s * c;
  }
}

double dequant(uint8_t code, uint16_t s, uint16_t z, int bits, const uint16_t* levels) {
  if (levels) return f16_to_f64(levels[code]) * f16_to_f64(s) + f16_to_f64(z);
  if (s & 0x8000) {
    const int mid = 1 << (bits - 1);
    return static_cast<double>(static_cast<int>(code) - mid) * f16_to_f64(s & 0x7fff);
  }
  return static_cast<double>(code) * f16_to_f64(s) + f16_to_f64(z);
}

}  // namespace

extern "C" {

// Scheme of one layer.
typedef struct {
  int32_t D;
  int32_t k_mode;      // 0: per-channel groups of k_group tokens; 1: inner groups of k_group channels
  int32_t k_group;
  int32_t v_group;     // per-token groups of v_group channels
  int32_t k_bits, v_bits;
  int32_t k_hybrid;    // inner groups choose sym/asym
  int32_t ratio_num, ratio_den;  // hybrid threshold |mean|/range <= num/den
  int32_t nuq;         // 3-bit codebook quantizer for K and V
  int32_t outliers;    // sparse fp16 entries per token vector
  int32_t v_hadamard;
  int32_t pre_rope;
  double rope_base;
  uint16_t levels_k[8];
  uint16_t levels_v[8];
  int32_t v_ternary;   // values as ternary levels {-s, 0, s} in 2-bit codes
  int32_t k_hi_groups; // inner 4-bit keys: groups per token quantized at 8 bits instead
} oq_scheme;

uint16_t oq_f64_to_f16(double x) { return f64_to_f16(x); }
double oq_f16_to_f64(uint16_t h) { return f16_to_f64(h); }
void oq_f64_to_f16_n(const double* x, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = f64_to_f16(x[i]);
}
void oq_f32_to_f16_n(const float* x, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = f64_to_f16(static_cast<double>(x[i]));
}

void oq_quant_asym(const uint16_t* x, const uint8_t* excl, int32_t n, int32_t bits, uint8_t* codes,
                   uint16_t* meta) {
  quant_asym(x, excl, n, bits, codes, &meta[0], &meta[1]);
}
void oq_quant_sym(const uint16_t* x, int32_t n, int32_t bits, uint8_t* codes, uint16_t* meta) {
  quant_sym(x, n, bits, codes, &meta[0], &meta[1]);
}
int32_t oq_hybrid_is_sym(const uint16_t* x, int32_t n, int32_t num, int32_t den) {
  return hybrid_is_sym(x, n, num, den) ? 1 : 0;
}
void oq_quant_tern(const uint16_t* x, const uint8_t* excl, int32_t n, uint8_t* codes, uint16_t* meta) {
  quant_tern(x, excl, n, codes, &meta[0], &meta[1]);
}
void oq_quant_nuq(const uint16_t* x, const uint8_t* excl, int32_t n, const uint16_t* levels,
                  uint8_t* codes, uint16_t* meta) {
  quant_nuq(x, excl, n, levels, codes, &meta[0], &meta[1]);
}
void oq_topk(const uint16_t* row, int32_t d, int32_t k, int32_t* cols) { topk_cols(row, d, k, cols); }
void oq_hadamard_fp16(const uint16_t* v, int32_t d, uint16_t* out) { hadamard_fp16(v, d, out); }
void oq_hadamard_f64(const double* v, int32_t d, double* out) { hadamard_f64(v, d, out); }
double oq_dequant(uint8_t code, uint16_t s, uint16_t z, int32_t bits, const uint16_t* levels) {
  return dequant(code, s, z, bits, levels);
}

// ---------------------------------------------------------------- cache state
// Reading of InnerQ method 4 ("most recent N tokens and sink tokens in fp16"):
// sinks are positions [0, S_eff), S_eff = min(S, n); the quantized body is a
// whole number of flush blocks F after them; the rest (W <= r < W+F once the
// body exists) is the fp16 window.
void oq_state_prefill(int32_t n, int32_t S, int32_t W, int32_t F, int32_t* s_eff, int32_t* nb,
                      int32_t* r) {
  const int32_t se = n < S ? n : S;
  const int32_t avail = n - se - W;
  const int32_t body = avail > 0 ? (avail / F) * F : 0;
  *s_eff = se;
  *nb = body;
  *r = n - se - body;
}

// One appended token.  The first S positions are the sink tokens, kept in
// fp16 whatever the prompt length: while fewer than S sinks exist (a prompt
// shorter than S), the token becomes the next sink.  Otherwise it enters the
// window; when the window reaches W + F tokens its oldest F are flushed into
// the body.  Returns 1 on a flush.
int32_t oq_state_append(int32_t* n, int32_t* s_eff, int32_t* nb, int32_t* r, int32_t S, int32_t W,
                        int32_t F) {
  *n += 1;
  if (*s_eff < S) {  // only reachable with an empty body and window
    *s_eff += 1;
    return 0;
  }
  *r += 1;
  if (*r == W + F) {
    *nb += F;
    *r -= F;
    return 1;
  }
  return 0;
}

// ---------------------------------------------------------------- key normalization
// InnerQ, method 4: a per-channel key scaling computed once over the prefill
// and folded into the query.  The pages name neither the statistic nor the
// form of the factor; the readings here:
//   a_c     = max over the T prefill tokens of |K[t][c]|
//   e_c     = binary exponent of a_c (a_c = m 2^e_c, 1/2 <= m < 1); a zero
//             channel takes e_c = E (no scaling)
//   E       = max_c e_c
//   shift_c = min(E - e_c, 14)       (an integer >= 0)
// Normalized keys x_c = K_c * 2^shift_c (every channel scaled toward the
// range of the largest one), rounded to fp16 with saturation at +-65504
// (exact unless a later token exceeds its channel's prefill range by 2^shift
// beyond fp16); the query is folded as q'_c = q_c * 2^-shift_c, so that
// q' . x = q . K exactly.  Powers of two keep the fold exact.
void oq_knorm_shifts(const uint16_t* K, int32_t T, int32_t D, int8_t* shift) {
  std::vector<int> e(D, 0);
  std::vector<bool> zero(D, true);
  int E = 0;
  bool anyc = false;
  for (int c = 0; c < D; ++c) {
    double a = 0.0;
    for (int t = 0; t < T; ++t) a = std::max(a, std::fabs(f16_to_f64(K[static_cast<size_t>(t) * D + c])));
    if (a > 0.0) {
      int ex = 0;
      std::frexp(a, &ex);
      e[c] = ex;
      zero[c] = false;
      E = anyc ? std::max(E, ex) : ex;
      anyc = true;
    }
  }
  for (int c = 0; c < D; ++c) shift[c] = static_cast<int8_t>(zero[c] ? 0 : std::min(E - e[c], 14));
}
// x = fp16(K * 2^shift) per channel for n rows (saturating).
void oq_knorm_apply(const uint16_t* K, int32_t n, int32_t D, const int8_t* shift, uint16_t* X) {
  for (int t = 0; t < n; ++t)
    for (int c = 0; c < D; ++c) {
      double x = std::ldexp(f16_to_f64(K[static_cast<size_t>(t) * D + c]), shift[c]);
      x = std::max(-65504.0, std::min(65504.0, x));
      X[static_cast<size_t>(t) * D + c] = f64_to_f16(x);
    }
}

// ---------------------------------------------------------------- encoding
// Encode the quantized body [s_eff, s_eff+nb) of one (batch, kv-head) unit.
// K, V: fp16 [n][D] (V before any rotation).  Outputs (logical, unpacked):
//   vrot    [n][D]              fp16 V after rotation (copy of V without it)
//   kcodes  [nb][D]             u8
//   kmeta   channel: [nb/kg][D][2]  inner: [nb][D/kg][2]   (s, z) fp16 bits
//   vcodes  [nb][D]             u8
//   vmeta   [nb][D/vg][2]
//   kocol/koval, vocol/voval  [nb][outliers]  (int32 column, fp16 value)
//   kwidth  inner keys: [nb][D/kg] code width of each key group (nullable)
// Returns 0, or -1 on an unsupported scheme.
int32_t oq_encode_unit(const oq_scheme* sc, const uint16_t* K, const uint16_t* V, int32_t n,
                       int32_t s_eff, int32_t nb, uint16_t* vrot, uint8_t* kcodes,
                       uint16_t* kmeta, uint8_t* vcodes, uint16_t* vmeta, int32_t* kocol,
                       uint16_t* koval, int32_t* vocol, uint16_t* voval, uint8_t* kwidth) {
  const int D = sc->D;
  const int kg = sc->k_group, vg = sc->v_group, ko = sc->outliers;
  if (D <= 0 || kg <= 0 || vg <= 0 || D % vg) return -1;
  if (sc->k_mode == 0 && nb % kg) return -1;
  if (sc->k_mode == 1 && D % kg) return -1;
  if (sc->nuq && sc->k_hybrid) return -1;
  if (sc->v_ternary && (sc->v_bits != 2 || sc->nuq || sc->v_hadamard)) return -1;
  if (sc->k_hi_groups < 0 || (sc->k_mode == 1 && sc->k_hi_groups > D / kg)) return -1;
  if (sc->k_hi_groups && (sc->k_mode != 1 || sc->k_bits != 4 || sc->nuq || ko)) return -1;
  // values: optional rotation of every token
  for (int t = 0; t < n; ++t) {
    if (sc->v_hadamard)
      hadamard_fp16(V + static_cast<size_t>(t) * D, D, vrot + static_cast<size_t>(t) * D);
    else
      std::memcpy(vrot + static_cast<size_t>(t) * D, V + static_cast<size_t>(t) * D, 2 * D);
  }
  // outlier masks of body rows
  std::vector<uint8_t> kex(static_cast<size_t>(nb) * D, 0), vex(static_cast<size_t>(nb) * D, 0);
  if (ko > 0) {
    std::vector<int32_t> cols(ko);
    for (int i = 0; i < nb; ++i) {
      const size_t row = static_cast<size_t>(s_eff + i) * D;
      topk_cols(K + row, D, ko, cols.data());
      for (int j = 0; j < ko; ++j) {
        kocol[i * ko + j] = cols[j];
        koval[i * ko + j] = K[row + cols[j]];
        kex[static_cast<size_t>(i) * D + cols[j]] = 1;
      }
      topk_cols(vrot + row, D, ko, cols.data());
      for (int j = 0; j < ko; ++j) {
        vocol[i * ko + j] = cols[j];
        voval[i * ko + j] = vrot[row + cols[j]];
        vex[static_cast<size_t>(i) * D + cols[j]] = 1;
      }
    }
  }
  std::vector<uint16_t> grp(std::max(kg, vg));
  std::vector<uint8_t> gex(std::max(kg, vg)), gcode(std::max(kg, vg));
  // keys
  if (sc->k_mode == 0) {
    for (int blk = 0; blk < nb / kg; ++blk)
      for (int c = 0; c < D; ++c) {
        for (int j = 0; j < kg; ++j) {
          const int i = blk * kg + j;
          grp[j] = K[static_cast<size_t>(s_eff + i) * D + c];
          gex[j] = kex[static_cast<size_t>(i) * D + c];
        }
        uint16_t* m = kmeta + (static_cast<size_t>(blk) * D + c) * 2;
        if (sc->nuq)
          quant_nuq(grp.data(), gex.data(), kg, sc->levels_k, gcode.data(), &m[0], &m[1]);
        else if (sc->k_hybrid && hybrid_is_sym(grp.data(), kg, sc->ratio_num, sc->ratio_den))
          quant_sym(grp.data(), kg, sc->k_bits, gcode.data(), &m[0], &m[1]);
        else
          quant_asym(grp.data(), gex.data(), kg, sc->k_bits, gcode.data(), &m[0], &m[1]);
        for (int j = 0; j < kg; ++j) kcodes[static_cast<size_t>(blk * kg + j) * D + c] = gcode[j];
      }
  } else {
    // InnerQ, limitations and future work: a layer may mix 4-bit and 8-bit
    // groups.  Reading: per token, the k_hi_groups groups whose 4-bit
    // quantizer has the largest step (fp16 scale magnitude; on equal steps the
    // lower group first) are quantized again at 8 bits, with the same
    // symmetric / asymmetric choice.
    const int ng = D / kg;
    std::vector<uint16_t> step(ng);
    std::vector<uint8_t> hi(ng);
    for (int i = 0; i < nb; ++i) {
      auto quant_group = [&](int g, int bits) {
        const uint16_t* src = K + static_cast<size_t>(s_eff + i) * D + g * kg;
        const uint8_t* ex = kex.data() + static_cast<size_t>(i) * D + g * kg;
        uint8_t* dst = kcodes + static_cast<size_t>(i) * D + g * kg;
        uint16_t* m = kmeta + (static_cast<size_t>(i) * ng + g) * 2;
        if (sc->nuq)
          quant_nuq(src, ex, kg, sc->levels_k, dst, &m[0], &m[1]);
        else if (sc->k_hybrid && hybrid_is_sym(src, kg, sc->ratio_num, sc->ratio_den))
          quant_sym(src, kg, bits, dst, &m[0], &m[1]);
        else
          quant_asym(src, ex, kg, bits, dst, &m[0], &m[1]);
        return static_cast<uint16_t>(m[0] & 0x7fff);
      };
      for (int g = 0; g < ng; ++g) {
        step[g] = quant_group(g, sc->k_bits);
        hi[g] = 0;
      }
      for (int k = 0; k < sc->k_hi_groups; ++k) {
        int best = -1;
        for (int g = 0; g < ng; ++g)
          if (!hi[g] && (best < 0 || step[g] > step[best])) best = g;
        hi[best] = 1;
      }
      for (int g = 0; g < ng; ++g) {
        if (hi[g]) quant_group(g, 8);
        if (kwidth) kwidth[static_cast<size_t>(i) * ng + g] = static_cast<uint8_t>(hi[g] ? 8 : sc->k_bits);
      }
    }
  }
  // values: per-token groups
  for (int i = 0; i < nb; ++i)
    for (int g = 0; g < D / vg; ++g) {
      const uint16_t* src = vrot + static_cast<size_t>(s_eff + i) * D + g * vg;
      const uint8_t* ex = vex.data() + static_cast<size_t>(i) * D + g * vg;
      uint8_t* dst = vcodes + static_cast<size_t>(i) * D + g * vg;
      uint16_t* m = vmeta + (static_cast<size_t>(i) * (D / vg) + g) * 2;
      if (sc->nuq)
        quant_nuq(src, ex, vg, sc->levels_v, dst, &m[0], &m[1]);
      else if (sc->v_ternary)
        quant_tern(src, ex, vg, dst, &m[0], &m[1]);
      else
        quant_asym(src, ex, vg, sc->v_bits, dst, &m[0], &m[1]);
    }
  return 0;
}

// ---------------------------------------------------------------- dequantization
// Rebuild the attended keys and values of one unit in binary64:
// sinks and window from fp16 (V rotated when the scheme rotates), the body
// from codes and parameters, sparse outliers overwriting their dense value,
// then RoPE on every key at its absolute position when keys are pre-RoPE.
// Khat, Vhat: [n][D]; only rows [t_begin, t_end) are written.
// kshift (nullable): per-channel key normalization shifts; body keys (codes
// and outliers, which live in the normalized domain) are scaled back by
// 2^-shift before RoPE.  kwidth (nullable, inner keys): code width of each
// key group as returned by oq_encode_unit.
int32_t oq_dequant_unit(const oq_scheme* sc, const uint16_t* K, const uint16_t* vrot, int32_t n,
                        int32_t s_eff, int32_t nb, int32_t t_begin, int32_t t_end,
                        const uint8_t* kcodes, const uint16_t* kmeta,
                        const uint8_t* vcodes, const uint16_t* vmeta, const int32_t* kocol,
                        const uint16_t* koval, const int32_t* vocol, const uint16_t* voval,
                        const int8_t* kshift, const uint8_t* kwidth, double* Khat, double* Vhat) {
  const int D = sc->D, kg = sc->k_group, vg = sc->v_group, ko = sc->outliers;
  const uint16_t* lk = sc->nuq ? sc->levels_k : nullptr;
  const uint16_t* lv = sc->nuq ? sc->levels_v : nullptr;
  if (t_begin < 0 || t_end > n || t_begin > t_end) return -1;
  for (int t = t_begin; t < t_end; ++t) {
    double* kh = Khat + static_cast<size_t>(t) * D;
    double* vh = Vhat + static_cast<size_t>(t) * D;
    const int i = t - s_eff;
    if (i >= 0 && i < nb) {
      for (int c = 0; c < D; ++c) {
        const uint16_t* m = sc->k_mode == 0
                                ? kmeta + (static_cast<size_t>(i / kg) * D + c) * 2
                                : kmeta + (static_cast<size_t>(i) * (D / kg) + c / kg) * 2;
        const int kbits = (kwidth && sc->k_mode == 1) ? kwidth[static_cast<size_t>(i) * (D / kg) + c / kg]
                                                      : sc->k_bits;
        kh[c] = dequant(kcodes[static_cast<size_t>(i) * D + c], m[0], m[1], kbits, lk);
        const uint16_t* mv = vmeta + (static_cast<size_t>(i) * (D / vg) + c / vg) * 2;
        vh[c] = dequant(vcodes[static_cast<size_t>(i) * D + c], mv[0], mv[1], sc->v_bits, lv);
      }
      for (int j = 0; j < ko; ++j) {
        kh[kocol[i * ko + j]] = f16_to_f64(koval[i * ko + j]);
        vh[vocol[i * ko + j]] = f16_to_f64(voval[i * ko + j]);
      }
      if (kshift)
        for (int c = 0; c < D; ++c) kh[c] = std::ldexp(kh[c], -kshift[c]);
    } else {
      for (int c = 0; c < D; ++c) {
        kh[c] = f16_to_f64(K[static_cast<size_t>(t) * D + c]);
        vh[c] = f16_to_f64(vrot[static_cast<size_t>(t) * D + c]);
      }
    }
    if (sc->pre_rope) {
      // rotate-half pairing (i, i + D/2), angle t * base^(-2i/D)
      const int h = D / 2;
      for (int p = 0; p < h; ++p) {
        const double theta = std::pow(sc->rope_base, -2.0 * p / D);
        const double phi = static_cast<double>(t) * theta;
        const double cs = std::cos(phi), sn = std::sin(phi);
        const double a = kh[p], b = kh[p + h];
        kh[p] = a * cs - b * sn;
        kh[p + h] = b * cs + a * sn;
      }
    }
  }
  return 0;
}

// ---------------------------------------------------------------- attention
// Scaled dot-product decode attention in binary64 for G query rows:
// s_t = q.k_t / sqrt(D); softmax with max subtraction; o = sum p_t v_t.
// unrotate: o <- c H o (values were stored rotated).
void oq_attention(const double* q, int32_t G, const double* Khat, const double* Vhat, int32_t n,
                  int32_t D, int32_t unrotate, double* out) {
  std::vector<double> sc(n), o(D);
  const double inv = 1.0 / std::sqrt(static_cast<double>(D));
  for (int g = 0; g < G; ++g) {
    const double* qg = q + static_cast<size_t>(g) * D;
    double m = -INFINITY;
    for (int t = 0; t < n; ++t) {
      double s = 0.0;
      for (int c = 0; c < D; ++c) s += qg[c] * Khat[static_cast<size_t>(t) * D + c];
      sc[t] = s * inv;
      if (sc[t] > m) m = sc[t];
    }
    double l = 0.0;
    std::fill(o.begin(), o.end(), 0.0);
    for (int t = 0; t < n; ++t) {
      const double p = std::exp(sc[t] - m);
      l += p;
      for (int c = 0; c < D; ++c) o[c] += p * Vhat[static_cast<size_t>(t) * D + c];
    }
    double* og = out + static_cast<size_t>(g) * D;
    for (int c = 0; c < D; ++c) o[c] /= l;
    if (unrotate)
      hadamard_f64(o.data(), D, og);
    else
      for (int c = 0; c < D; ++c) og[c] = o[c];
  }
}

// Split-context form: tokens cut into nsplit contiguous ranges, each giving a
// partial (max m_i, sum l_i, unnormalised o_i); merged by log-sum-exp:
// m = max m_i, l = sum l_i e^(m_i-m), o = sum o_i e^(m_i-m) / l.
void oq_attention_split(const double* q, int32_t G, const double* Khat, const double* Vhat,
                        int32_t n, int32_t D, int32_t unrotate, int32_t nsplit, double* out) {
  const double inv = 1.0 / std::sqrt(static_cast<double>(D));
  std::vector<double> pm(nsplit), pl(nsplit), po(static_cast<size_t>(nsplit) * D), o(D);
  for (int g = 0; g < G; ++g) {
    const double* qg = q + static_cast<size_t>(g) * D;
    for (int sp = 0; sp < nsplit; ++sp) {
      const int t0 = static_cast<int>(static_cast<int64_t>(n) * sp / nsplit);
      const int t1 = static_cast<int>(static_cast<int64_t>(n) * (sp + 1) / nsplit);
      double m = -INFINITY;
      std::vector<double> s(t1 - t0);
      for (int t = t0; t < t1; ++t) {
        double a = 0.0;
        for (int c = 0; c < D; ++c) a += qg[c] * Khat[static_cast<size_t>(t) * D + c];
        s[t - t0] = a * inv;
        if (s[t - t0] > m) m = s[t - t0];
      }
      double l = 0.0;
      double* os = po.data() + static_cast<size_t>(sp) * D;
      for (int c = 0; c < D; ++c) os[c] = 0.0;
      for (int t = t0; t < t1; ++t) {
        const double p = std::exp(s[t - t0] - m);
        l += p;
        for (int c = 0; c < D; ++c) os[c] += p * Vhat[static_cast<size_t>(t) * D + c];
      }
      pm[sp] = m;
      pl[sp] = l;
    }
    double M = -INFINITY;
    for (int sp = 0; sp < nsplit; ++sp)
      if (pm[sp] > M) M = pm[sp];
    double L = 0.0;
    std::fill(o.begin(), o.end(), 0.0);
    for (int sp = 0; sp < nsplit; ++sp) {
      if (pl[sp] == 0.0) continue;  // empty range
      const double w = std::exp(pm[sp] - M);
      L += pl[sp] * w;
      for (int c = 0; c < D; ++c) o[c] += po[static_cast<size_t>(sp) * D + c] * w;
    }
    double* og = out + static_cast<size_t>(g) * D;
    for (int c = 0; c < D; ++c) o[c] /= L;
    if (unrotate)
      hadamard_f64(o.data(), D, og);
    else
      for (int c = 0; c < D; ++c) og[c] = o[c];
  }
}

}  // extern "C"
