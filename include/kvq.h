/* kvq.h -- packed KV-cache quantization and fused dequantize-attend decode
 * for AMD Instinct MI355X (gfx950).
 *
 * The library keeps an LLM key/value cache as packed 2/3/4/8-bit codes with
 * per-group fp16 parameters, and computes decode attention directly over it.
 * Three calls make the path, in the order the Hadamard 2-bit values page
 * (aitrends.kr, "practical advice") says quantized caches must be exercised:
 * quantize the prompt into the cache, then decode token by token through it.
 *
 *   kvq_quantize_prefill  quantize a prompt's keys/values into one layer's cache
 *   kvq_append_token      add one decoded token (quantizing a flush block when due)
 *   kvq_decode_attn       attention of one query step over the whole cache
 *   kvq_append_decode_attn  the two above for one layer, in one launch where it can
 *
 * Schemes (pages as titled):
 *   keys per channel, asymmetric, groups of 32 tokens  -- KVTuner review,
 *       observation 2; KVQuant abstract item (i)
 *   values per token, asymmetric, groups of v_group channels -- RateQuant,
 *       section 3 (KIVI layout); Hadamard page, KIVI int4 glossary entry
 *   keys in inner-dimension groups of k_group channels with a per-group
 *       symmetric/asymmetric choice -- InnerQ, methodology 1 and 2
 *   pre-RoPE keys with RoPE applied after dequantization -- KVQuant (ii)
 *   3-bit per-layer non-uniform codebooks -- KVQuant (iii)
 *   per-vector sparse fp16 outliers (top-k by magnitude) -- KVQuant (iv)
 *   values rotated by a normalised Hadamard matrix before 2-bit quantization,
 *       rotation undone after the attention sum -- Hadamard page, TL;DR
 *   fp16 sink tokens and recent window -- InnerQ, methodology 4
 *   4-bit and 8-bit key groups mixed inside a layer -- InnerQ, limitations
 *       and future work
 *   per-layer (k_bits, v_bits) pair chosen offline from
 *       {KV8, K8V4, KV4, K4V2, KV2} -- KVTuner review, method steps 1 and 4
 *
 * Ownership.  The library allocates no device memory.  The caller sizes the
 * per-layer buffers with kvq_layer_buffer_sizes(), allocates them (any
 * allocator, 256-byte aligned), binds them with kvq_bind_layer(), and owns
 * them.  The handle holds host metadata only (token counts per layer).
 *
 * Streams.  Every device call is asynchronous on the caller's HIP stream
 * (passed as void*; NULL is the null stream).  Calls on one cache must be
 * stream-ordered; the handle has no internal locking.
 *
 * Errors.  Argument, state and capacity checks run on the host before any
 * launch; a call failing them returns its status and leaves host state and
 * device buffers untouched.  A failed kernel launch returns KVQ_ERR_DEVICE;
 * since a call may already have queued some of its kernels, the layer's
 * device buffers can then hold a partial update, so the layer is marked
 * empty: its appends and decodes return KVQ_ERR_STATE until the next
 * kvq_quantize_prefill.  No C++ exception crosses this interface.
 *
 * Data types: fp16 = IEEE binary16 bit patterns in uint16 storage.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kvq_cache kvq_cache;

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_ARG = 1,          /* null pointer, out-of-range layer, bad size or config field */
  KVQ_ERR_CAPACITY = 2,     /* the call would hold more than max_tokens tokens */
  KVQ_ERR_UNSUPPORTED = 3,  /* valid but not implemented (bit width, head_dim, group) */
  KVQ_ERR_STATE = 4,        /* wrong call order: unbound layer, append/decode before prefill */
  KVQ_ERR_DEVICE = 5        /* a HIP runtime call or kernel launch failed */
} kvq_status;

enum { KVQ_K_PER_CHANNEL = 0, KVQ_K_INNER = 1 };
/* Values: per-token groups; KVQ_V_HADAMARD rotates each value row by the
 * normalized 128x128 Hadamard matrix first (the Hadamard 2-bit page) and the
 * decode undoes it after the attention sum; KVQ_V_TERNARY quantizes to the
 * three levels {-s, 0, +s} with s = max |v| over the group, stored as 2-bit
 * codes with z = -s (that page's failed first attempt at about 1.58 bits,
 * kept as a negative control; needs v_bits == 2, no codebooks). */
enum { KVQ_V_PER_TOKEN = 0, KVQ_V_HADAMARD = 1, KVQ_V_TERNARY = 2 };

/* (k_bits, v_bits) of one layer: 2, 3, 4 or 8 each (3 only with nuq). */
typedef struct {
  uint8_t k_bits, v_bits;
} kvq_bitpair;

typedef struct {
  int32_t batch;          /* B  >= 1 */
  int32_t n_q_heads;      /* Hq, a multiple of n_kv_heads; Hq/Hkv <= 16 */
  int32_t n_kv_heads;     /* Hkv >= 1 */
  int32_t head_dim;       /* D; must be 128 */
  int32_t n_layers;       /* L >= 1 */
  int32_t max_tokens;     /* capacity per (layer, batch, kv head) */
  int32_t sink_tokens;    /* S: first S positions kept fp16 */
  int32_t recent_window;  /* W: most recent W..W+F-1 positions kept fp16 */
  int32_t k_mode;         /* KVQ_K_PER_CHANNEL (k_group must be 32) | KVQ_K_INNER */
  int32_t k_group;        /* tokens per key group (per channel) or channels (inner: 16, 32 or 64) */
  int32_t v_mode;         /* KVQ_V_PER_TOKEN | KVQ_V_HADAMARD | KVQ_V_TERNARY */
  int32_t v_group;        /* channels per value group: 16, 32 or 64 */
  int32_t k_hybrid;       /* inner groups: symmetric iff |mean|/range <= num/den */
  int32_t sym_ratio_num, sym_ratio_den;  /* e.g. 1/10 */
  int32_t k_pre_rope;     /* keys are stored pre-RoPE; RoPE applied at decode */
  float rope_base;        /* e.g. 10000 (rotate-half pairs (i, i+D/2)) */
  int32_t nuq;            /* 1: 3-bit codebook quantizer for keys and values */
  int32_t outliers_per_vector; /* 0, or k sparse fp16 entries per token row (k <= 8) */
  int32_t k_norm;         /* 1: one-time per-channel key normalization (InnerQ, method 4;
                             inner key groups only).  kvq_quantize_prefill takes, per
                             (batch, kv head) and channel c, the binary exponent e_c of
                             max_t |K[t][c]| over the prefill (a = m 2^e, 1/2 <= m < 1),
                             E = max_c e_c and shift_c = min(E - e_c, 14) (0 for an all-zero
                             channel); body keys are quantized as fp16(K * 2^shift_c)
                             (saturating at +-65504) and the decode folds 2^-shift_c into
                             the query for them, so q'.x = q.K.  Sink and window tokens stay
                             as given.  The shifts live in the KVQ_BUF_FP16 buffer after the
                             fp16 slots (units * 128 int8).  With k_norm the prefill
                             keys must be 16-byte aligned (else KVQ_ERR_ARG). */
  int32_t k_hi_groups;    /* m >= 0: mixed 4/8-bit key groups (InnerQ, limitations and future
                             work; inner key groups only, no codebooks, no sparse outliers).
                             In every layer whose k_bits is 4, each quantized token's m inner
                             groups with the largest 4-bit step (the magnitude of the fp16
                             scale its 4-bit quantizer gets; the lower group first on equal
                             steps) are quantized at 8 bits instead, with the same
                             symmetric / asymmetric choice.  m <= head_dim / k_group.  Layers
                             with other key widths ignore it.  0 disables. */
} kvq_config;

/* Per-layer device buffers (caller-owned). */
#define KVQ_NBUF 2
enum {
  KVQ_BUF_BODY = 0,   /* packed blocks: [B*Hkv][ceil(max_tokens/32)][record] */
  KVQ_BUF_FP16 = 1    /* fp16 sinks and window ring, see below */
};

/* fp16 area of one (batch, kv head) unit, units back to back: Scap + Wcap
 * slots (Scap = S and Wcap = W + F, each rounded up to a multiple of 32).
 * Position p < S' sits in slot p; a window position p sits in slot
 * Scap + (p - S') mod Wcap.  Keys: [Scap + Wcap][D] token-major.  Values:
 * [(Scap + Wcap)/8][D][8], i.e. value (slot, c) at ((slot/8)*D + c)*8 +
 * slot%8.  Slots holding no token are zero after a prefill. */

/* Byte layout of one body block record (32 consecutive quantized tokens of one
 * (batch, kv head) unit), as reported by kvq_block_layout().  Every section
 * starts 16-byte aligned.
 *
 *  k_codes  2/4/8 bits: token-major rows of D codes, row_bytes = D*k_bits/8.
 *           2/4 bits: each 32-bit word holds n = 32/bits consecutive channels
 *             e_0..e_(n-1) with e_(2j) at bit bits*j and e_(2j+1) at bit
 *             16 + bits*j ("pair-split" word).
 *           8 bits: one byte per channel.
 *           3 bits: 64 lane chunks of 24 bytes, each a little-endian bit
 *             stream with element E at bits 3E..3E+2.  Chunk l holds the
 *             RoPE pair (l, l + 64): element 2t + e = code(token t, channel
 *             l + 64e), so token t's two codes are the 6-bit field at 6t.
 *  k_meta   per-channel keys: s[D] fp16 then z[D] fp16 (one group per channel
 *           per block).  Inner keys: [32 tokens][D/k_group] pairs (s, z).
 *           A set sign bit on s marks a symmetric group: value = (code-2^(b-1))*|s|;
 *           otherwise value = code*s + z; codebook mode: value = L[code]*s + z.
 *  v_codes  2/4/8 bits: 64 lane chunks of 8*v_bits bytes; chunk l covers
 *           tokens 8*(l/16)..+7 and channels 16*t + l%16 (t = 0..7); its
 *           element sequence is e_(8t+j) = code(token 8*(l/16)+j, channel
 *           16t + l%16), packed in pair-split words (2/4 bits) or bytes (8).
 *           3 bits: 64 lane chunks of 24 bytes (bit stream as for keys);
 *             chunk 16g + n holds element 8t + i = code(token 8g + i,
 *             channel 16t + n).
 *  v_meta   s[D/v_group][32 tokens] fp16 then z[D/v_group][32 tokens] fp16.
 *  k_out,   outliers_per_vector entries per token: {uint16 column, fp16
 *  v_out    value}, columns ascending; the fp16 value replaces the dequantized
 *           element.
 *  k_ext    mixed 4/8-bit key groups only (else empty): [32 tokens][m slots]
 *           [k_group/2 bytes]; slot i of a token holds the low four bits of
 *           the 8-bit codes of its i-th 8-bit group (ascending group order),
 *           channels of the group in pair-split words of 4-bit fields.  The
 *           high four bits sit in k_codes at the group's own channels, so
 *           code = (k_codes field << 4) | k_ext field for an 8-bit group, whose
 *           k_meta pair is its 8-bit (s, z) (symmetric: (code - 128) * |s|).
 *  k_sel    mixed 4/8-bit key groups only: [32 tokens] uint8, bit g set iff
 *           inner group g of the token is an 8-bit group.
 */
typedef struct {
  int32_t record_bytes;
  int32_t k_codes, k_meta, v_codes, v_meta, k_out, v_out;  /* section offsets */
  int32_t k_row_bytes;
  int32_t sink_cap;       /* Scap: sink slots per unit */
  int32_t window_cap;     /* Wcap: window ring slots per unit */
  int32_t flush_tokens;   /* F: 32 for per-channel keys, 1 for inner keys */
  int32_t k_ext, k_sel;   /* mixed 4/8-bit key group sections (offsets; equal when unused) */
} kvq_block_layout_t;

/* Create a cache handle.  layer_bits[n_layers]; codebooks: NULL or
 * [n_layers][2 (K,V)][8] fp16 levels sorted ascending (required when nuq).
 * The inputs are copied.  Errors: KVQ_ERR_ARG, KVQ_ERR_UNSUPPORTED. */
kvq_status kvq_create(const kvq_config* cfg, const kvq_bitpair* layer_bits,
                      const uint16_t* codebooks, kvq_cache** out);

/* Release the handle (not the caller's buffers). NULL is accepted. */
kvq_status kvq_destroy(kvq_cache* cache);

/* Bytes needed for each KVQ_BUF_* buffer of a layer. */
kvq_status kvq_layer_buffer_sizes(const kvq_cache* cache, int32_t layer, size_t sizes[KVQ_NBUF]);

/* Record layout of a layer's body blocks. */
kvq_status kvq_block_layout(const kvq_cache* cache, int32_t layer, kvq_block_layout_t* out);

/* Attach caller-owned device buffers to a layer (re-binding resets the layer). */
kvq_status kvq_bind_layer(kvq_cache* cache, int32_t layer, void* const bufs[KVQ_NBUF]);

/* Detach a layer's buffers (before the caller frees them): the layer becomes
 * unbound and its device calls return KVQ_ERR_STATE until it is bound again.
 * Calls already queued on a stream still use the old buffers, so the caller
 * frees them only after those have completed.  Errors: KVQ_ERR_ARG. */
kvq_status kvq_unbind_layer(kvq_cache* cache, int32_t layer);

/* Bytes of device workspace kvq_decode_attn needs.  The workspace must be
 * zero-filled once before its first use; each decode call leaves its
 * completion counters at zero again.  One workspace serves one stream.  Its
 * last 4 bytes count the output rows that came out non-finite (see
 * kvq_decode_nonfinite_rows). */
kvq_status kvq_workspace_size(const kvq_cache* cache, size_t* bytes);

/* Quantize a prompt of T tokens into a layer, replacing its contents.
 * k, v: device fp16 [B][Hkv][T][D] (keys pre-RoPE when k_pre_rope).
 * Positions [0,S') become fp16 sinks (S' = min(S,T)); then the largest whole
 * number of flush blocks is quantized; the remaining tokens form the fp16
 * window.  workspace is unused (may be NULL).
 * Errors: KVQ_ERR_ARG, KVQ_ERR_STATE (unbound), KVQ_ERR_CAPACITY (T > max_tokens). */
kvq_status kvq_quantize_prefill(kvq_cache* cache, int32_t layer, const void* k, const void* v,
                                int32_t T, void* workspace, void* stream);

/* Append one token per unit.  k_new, v_new: device fp16 [B][Hkv][D].  While
 * the layer holds fewer than S sink tokens (a prompt shorter than S) the
 * token becomes the next fp16 sink, so the first S positions are always
 * sinks.  Otherwise it enters the fp16 window; when the window reaches W+F
 * tokens its oldest F tokens are quantized into the next body block (keys
 * and values together).  With inner keys and W = 0 the token is quantized at
 * once.
 * Errors: KVQ_ERR_ARG, KVQ_ERR_STATE (before prefill), KVQ_ERR_CAPACITY. */
kvq_status kvq_append_token(kvq_cache* cache, int32_t layer, const void* k_new,
                            const void* v_new, void* stream);

/* Decode attention over every token currently in the layer (append first).
 * q: device fp16 [B][Hq][D], already position-encoded; q head h reads kv
 * head h / (Hq/Hkv).  out: device fp32 [B][Hq][D] =
 * softmax(q.K^T / sqrt(D)) V, with keys/values dequantized (outliers merged,
 * RoPE applied to pre-RoPE keys, Hadamard rotation undone).
 * Numerical domain: with per-channel key groups (2/4/8-bit codes) the
 * product of each query element and its channel's key scale, q_c * s_c, is
 * formed in binary16 (as an exact hi + lo pair), so |q_c * s_c| must stay
 * below 65504 for every body block; beyond it the output row is not finite.
 * Every other product on the path is exact or formed in fp32.  Each output
 * row holding a non-finite element is counted in the workspace (read with
 * kvq_decode_nonfinite_rows), so a caller can detect such inputs after the
 * fact without inspecting the output.
 * Errors: KVQ_ERR_ARG, KVQ_ERR_STATE (empty cache / unbound), KVQ_ERR_DEVICE. */
kvq_status kvq_decode_attn(kvq_cache* cache, int32_t layer, const void* q, float* out,
                           void* workspace, void* stream);

/* kvq_append_token followed by kvq_decode_attn on the same stream, with the
 * same arguments, state changes, results and errors (the step a decoding
 * model takes for each layer: the new token enters the cache and the query
 * attends over it; InnerQ, methodology 4, the fp16 window; KVQuant,
 * technical approach, the fused dequantize-attend read).  When the token
 * only needs storing -- the next sink, or a window slot without a flush --
 * and the layer's decode runs on the matrix-core kernel, both happen in the
 * decode's own launch: it reads the token from k_new / v_new, rotates its
 * values when the layer keeps them rotated (Hadamard page; layers with
 * per-channel keys), and stores it into its slot.  Otherwise it makes the
 * two calls.
 * k_new, v_new: device fp16 [B][Hkv][D]; q, out, workspace as for
 * kvq_decode_attn.  A failed launch leaves the layer in KVQ_ERR_STATE until
 * the next prefill, as for the calls it stands for.
 * Errors: KVQ_ERR_ARG, KVQ_ERR_STATE, KVQ_ERR_CAPACITY, KVQ_ERR_DEVICE. */
kvq_status kvq_append_decode_attn(kvq_cache* cache, int32_t layer, const void* k_new, const void* v_new,
                                  const void* q, float* out, void* workspace, void* stream);

/* kvq_decode_attn without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP stream/graph capture, serving loops
 * with a fixed memory footprint, harnesses that forbid hipMalloc.  The call
 * allocates nothing (no hipMalloc, no allocating library routine): the split
 * partials, the per-unit arrival counters and the non-finite row count live
 * in a static device array of the library, KVQ_STATIC_SCRATCH_BYTES (32 MiB)
 * per GPU, held by every GPU the library runs on until the process ends.
 * Arguments, layouts and results are those of kvq_decode_attn; q and out are
 * still the caller's.  The first call on a device looks up and clears that
 * device's array and waits for the device, so make one call before any
 * stream capture.  Every call on a GPU shares that GPU's array: calls that
 * may overlap on one GPU (different streams, or several threads) race and
 * must be serialized by the caller, e.g. issued on one stream.  The non-finite
 * row count of these calls is read with kvq_decode_nonfinite_rows(cache,
 * NULL, ...).
 * Errors: those of kvq_decode_attn, and KVQ_ERR_CAPACITY when the layer's
 * split plan needs more than the array's 32 MiB - 64 KiB of partials
 * (units * splits * (Hq/Hkv) * 520 bytes) or more than 16383 units. */
#define KVQ_STATIC_SCRATCH_BYTES (32u << 20)
kvq_status kvq_decode_attn_static(kvq_cache* cache, int32_t layer, const void* q, float* out,
                                  void* stream);

/* Output rows with a non-finite element written by the decodes that used this
 * workspace since the last call (counted on the device by the merge step);
 * workspace NULL reads the count of kvq_decode_attn_static calls on the
 * current device.  Waits for the stream, reads the count into *rows and
 * resets it; not for use under stream capture.
 * Errors: KVQ_ERR_ARG, KVQ_ERR_DEVICE. */
kvq_status kvq_decode_nonfinite_rows(const kvq_cache* cache, void* workspace, void* stream,
                                     uint32_t* rows);

/* Host-side token accounting of a layer: total tokens n, sink tokens,
 * quantized body tokens and fp16 window tokens (n = sinks + body + window). */
kvq_status kvq_layer_state(const kvq_cache* cache, int32_t layer, int32_t* n, int32_t* sinks,
                           int32_t* body, int32_t* window);

/* Average bits of the cache's quantized tensors.  code_bits is the
 * KVTuner review's memory objective f_m = sum(P) / 2L (method step 0): the
 * mean over the 2L key and value tensors of their code width, where a layer
 * with mixed 4/8-bit key groups counts 4 + 4 m / (head_dim / k_group) for
 * its keys.  stored_bits adds everything a body block stores per element
 * (parameters, outliers, mixed-group sections and the record's alignment
 * padding): 8 * record_bytes / (2 * 32 * head_dim), averaged over layers.
 * Either pointer may be NULL.  Errors: KVQ_ERR_ARG. */
kvq_status kvq_average_bits(const kvq_cache* cache, double* code_bits, double* stored_bits);

/* Read ceiling of the decode's access pattern (measurement helper): streams
 * `bytes` of device memory at `src` the way kvq_decode_attn streams body
 * records -- `splits` wavefronts, each reading a contiguous run of 4 KiB
 * chunks as 1 KiB wave loads into a two-slot LDS ring -- with no arithmetic
 * on the data.  Its duration against `bytes` is the read bandwidth a decode
 * of that shape can reach.  src: 256-byte aligned, bytes a multiple of 4096;
 * sink: device uint32[splits], written only in the (practically never) case
 * that a split's XOR of sampled words equals 0x9e3779b9.  Asynchronous on
 * the stream.  Errors: KVQ_ERR_ARG, KVQ_ERR_DEVICE. */
kvq_status kvq_stream_read(const void* src, size_t bytes, int32_t splits, uint32_t* sink, void* stream);

/* Static text for a status code. */
const char* kvq_status_str(kvq_status s);

/* ---- Offline bit allocation (host only; no device work) --------------------
 * RateQuant technical summary, methodology: each quantized component i (the
 * keys or the values of one layer) follows D_i(b) = alpha_i beta_i^-b; the
 * widths minimise sum_i w_i D_i(b_i) under sum_i b_i = B (w_i: sensitivity).
 * The integer result is what kvq_create's per-layer (k_bits, v_bits) table
 * takes.  All arrays are host memory owned by the caller. */

/* Least-squares fit of ln mse = ln alpha - b ln beta over n >= 2 measured
 * points (bits[i], mse[i] > 0, at least two distinct widths).
 * Errors: KVQ_ERR_ARG. */
kvq_status kvq_fit_rate_distortion(int32_t n, const double* bits, const double* mse,
                                   double* alpha, double* beta);

/* Real-valued optimum (reverse water-filling, methodology step 1): every
 * component's w_i alpha_i ln(beta_i) beta_i^-b_i is equal and sum b_i =
 * total_bits; with one common (alpha, beta) this is b_i = mean + (ln w_i -
 * ln w_geo) / ln beta.  Needs alpha_i > 0, beta_i > 1, w_i > 0.  No range
 * clipping.  Errors: KVQ_ERR_ARG. */
kvq_status kvq_waterfill_bits(int32_t n, const double* alpha, const double* beta,
                              const double* w, double total_bits, double* bits_out);

/* Integer widths from the allowed set (methodology step 3, greedy marginal
 * gain): all components start at the smallest allowed width; while budget is
 * left, the component whose next allowed width gives the largest weighted
 * distortion reduction per bit, and still fits, takes it (ties: lowest
 * index).  sum bits_out <= total_bits.  Errors: KVQ_ERR_ARG (bad model
 * values, empty or out-of-range allowed set, budget below n * min width). */
kvq_status kvq_allocate_bits(int32_t n, const double* alpha, const double* beta,
                             const double* w, const int32_t* allowed, int32_t n_allowed,
                             int32_t total_bits, int32_t* bits_out);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H */
