/*
 * gemma_attn.h -- C ABI of the Gemma-family decoder attention block on MI355X (gfx950).
 *
 * One attention layer of the Gemma family (Gemma, Gemma 2, Gemma 3, Gemma 4):
 * interleaved sliding-window (local) and causal (global) layers, grouped- and
 * multi-query KV heads, RMSNorm QK-norm, dual-base and partial rotary position
 * embedding, keys-as-values global layers, query_pre_attn_scalar scaling and the
 * tanh attention-logit soft cap.
 *
 * Sources: the Gemma model pages ("Gemma", "Gemma 2", "Gemma 3", "Gemma 4") and
 * their API argument tables, and the "google-gemma-4" architecture summary.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Activations and caches are bf16 (raw 16-bit patterns), row-major and
 *    contiguous: q [B,S,Hq,D], k and v [B,S,Hkv,D], caches [B,Smax,Hkv,D].
 *    Norm weights are fp32 [D].  Log-sum-exp outputs are fp32, natural log.
 *  - Every data pointer is a DEVICE pointer owned by the caller; the library
 *    allocates nothing, keeps no state between calls and is re-entrant (the
 *    one exception: the fixed device array that gemma_attn_decode_multi_noalloc
 *    uses in place of a workspace, see there).
 *    Configuration structs and layer structs are HOST pointers, read during the
 *    call only.
 *  - Device pointers must be 16-byte aligned.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *    asynchronously; nothing in the library synchronizes the host.
 *  - Every argument check runs on the host before anything is enqueued; a
 *    call that returns an error has enqueued nothing (except GA_ERR_HIP from a
 *    decode, whose second launch can fail after its first was enqueued).
 *    GA_ERR_HIP carries the status the runtime returned for the library's own
 *    launch; an error left pending by an earlier, unrelated call is neither
 *    reported nor cleared.
 *  - Launch plans follow the current device's CU count, LDS size and XCD
 *    count (queried once per device), so a partitioned MI355X is planned for
 *    what it has.  Workspace sizes are those of the current device.
 */
#ifndef GEMMA_ATTN_H
#define GEMMA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  GA_OK = 0,
  GA_ERR_INVALID_ARG = 1, /* a null pointer, a size out of range, an inconsistent config */
  GA_ERR_UNSUPPORTED = 2, /* valid, but no kernel instantiation (head width, group size) or a shape
                             beyond the launch limits (batch or grid too large) */
  GA_ERR_WORKSPACE = 3,   /* decode workspace missing or smaller than required */
  GA_ERR_HIP = 4,         /* the HIP runtime rejected a launch */
  GA_ERR_SCRATCH_LIMIT = 5 /* gemma_attn_decode_multi_noalloc: the shape needs more workspace than
                              the library's fixed scratch array holds */
};

/*
 * The attention knobs of a Gemma model, named as in the pages' argument tables
 * (GemmaModel, Gemma2Model, Gemma3Model, Gemma4Model).
 */
typedef struct gemma_attn_config {
  int32_t num_heads;              /* query heads Hq */
  int32_t num_kv_heads;           /* KV heads on local layers (Hq % it == 0) */
  int32_t num_global_kv_heads;    /* KV heads on global layers; 0 = num_kv_heads (Gemma 4 table) */
  int32_t head_dim;               /* D on local layers */
  int32_t global_head_dim;        /* D on global layers; 0 = head_dim (Gemma 4 table) */
  int32_t sliding_window;         /* local attention span W; <= 0: every layer is global */
  int32_t sliding_window_pattern; /* N >= 1: layer l is global iff (l+1) % N == 0; <= 0: all local */
  int32_t k_eq_v;                 /* global layers use the processed keys as values (Gemma 4 "K=V") */
  int32_t norm_weight_offset;     /* QK-norm scales by (offset + w): 1 for Gemma 1-3, 0 for Gemma 4 */
  int32_t reserved;               /* must be 0 */
  double rope_theta;              /* rotary base on global layers (all layers when no local base) */
  double rope_local_theta;        /* rotary base on local layers; <= 0: rope_theta (Gemma 3 dual bases) */
  double partial_rotary_factor;   /* fraction of each head rotated, in [0, 1] (Gemma 4: 0.25) */
  double attn_logit_softcapping;  /* tanh cap on scaled logits; <= 0: off (Gemma 2: 50) */
  double query_pre_attn_scalar;   /* logits scale = this^-1/2; <= 0: the layer's D (Gemma 2/3: 256) */
  double norm_eps;                /* QK-norm epsilon inside the root (1e-6) */
  double rope_scaling_factor;     /* > 0: global layers take position p / factor in the rotary
                                     angle (Gemma 3 table, long-context scaling; read as linear);
                                     <= 0: off */
} gemma_attn_config;

/* Values one layer resolves to (see gemma_attn_resolve_layer). */
typedef struct gemma_attn_layer {
  int32_t is_global;    /* 1: full causal layer; 0: sliding-window layer */
  int32_t window;       /* W on local layers, 0 on global layers */
  int32_t num_kv_heads; /* Hkv of this layer */
  int32_t head_dim;     /* D of this layer */
  int32_t group;        /* g = Hq / Hkv; query head h reads KV head h / g */
  int32_t rotary_dim;   /* r = 2*floor(partial_rotary_factor * D / 2): dims [0, r) rotate */
  int32_t k_eq_v;       /* values are the processed keys on this layer */
  int32_t reserved;
  double theta;         /* rotary base of this layer */
  double scale;         /* query_pre_attn_scalar^-1/2 (or D^-1/2) */
  double softcap;       /* cap, or 0 when off */
  double pos_div;       /* rotary positions are divided by this (rope_scaling_factor on
                           global layers, else 1) */
} gemma_attn_layer;

/*
 * Resolve layer `layer_idx` of a model (pure host function, no HIP call).
 * Local/global interleave: "one global layer every N" (Gemma 3 table,
 * sliding_window_pattern; Gemma 2 introduction: every other layer), read as
 * local layers first in each period.  Global layers take the global KV-head
 * count, global head width and keys-as-values flag (Gemma 4 table) and the
 * rope scaling factor; local layers take rope_local_theta (Gemma 3 "Dual RoPE
 * bases").
 * Returns GA_ERR_INVALID_ARG for a null pointer, a negative layer, or a config
 * that fails validation (Hq not a multiple of Hkv, a non-positive D, a factor
 * outside [0, 1], a non-positive theta or eps).
 */
int gemma_attn_resolve_layer(const gemma_attn_config* cfg, int32_t layer_idx, gemma_attn_layer* out);

/*
 * QK-norm + rotary prologue for one layer, in one fused pass over q and k.
 * Per token s of sequence b and per head vector x (width D of the layer):
 *   1. if a norm weight w is given: x <- x / sqrt(mean(x^2) + eps) * (w + offset)
 *      (RMSNorm; Gemma 4 "Plain-weight RMSNorm" uses offset 0);
 *   2. the first r dims rotate in pairs (i, i + r/2) by the angle
 *      (p / pos_div) * theta^(-2i/r) with p = pos0[b] + s (pos_div: the
 *      layer's rope scaling, 1 when off); dims [r, D) pass through
 *      (Gemma 4 "Zero-pad partial rope"; r from partial_rotary_factor).
 * q_in [B,S,Hq,D] -> q_out, k_in [B,S,Hkv,D] -> k_out; bf16.  Outputs may alias
 * their inputs exactly (in place) but must not partially overlap them.
 * k_in may be NULL (then k_out is ignored): queries only, as in decode.
 * q_in may be NULL (then q_out is ignored): keys only, for
 * gemma_attn_prefill_qrope, which rotates the queries itself.  Not both.
 * q_norm_w / k_norm_w: fp32 [D] device arrays, or NULL for no norm on that side.
 * pos0: device int32 [B] first position of each sequence, or NULL for zeros.
 * Values are never normed or rotated.  Accumulation is fp32; the angle is
 * formed in fp64 in revolutions (p * theta^(-2i/r) / (2 pi pos_div)), reduced
 * to its fractional part there, and evaluated by the hardware fp32 cosine and
 * sine; outputs round to nearest even.
 */
int gemma_qk_prologue(const gemma_attn_config* cfg, int32_t layer_idx, int32_t batch, int32_t seq,
                      const void* q_in, const void* k_in, void* q_out, void* k_out,
                      const float* q_norm_w, const float* k_norm_w, const int32_t* pos0,
                      void* stream);

/*
 * Causal self-attention of one layer over a whole prompt (prefill).
 * For query head h at position i, against KV head h / g:
 *   s_ij = (q_i . k_j) * scale;  s_ij <- cap * tanh(s_ij / cap) if cap > 0
 *   (Gemma 2 "Logit softcapping");  allowed iff j <= i and, on local layers,
 *   i - j < W (exactly W keys including i: the reading of "local attention
 *   span");  out_i = softmax_j(s_ij) . v_j;  lse_i = log sum_j exp(s_ij).
 * q [B,S,Hq,D], k [B,S,Hkv,D], v [B,S,Hkv,D] bf16 (outputs of the prologue for
 * q and k).  On keys-as-values layers v is ignored (may be NULL) and k serves
 * as values (Gemma 4 "K=V global MQA").  out [B,S,Hq,D] bf16.
 * lse: fp32 [B,Hq,S] or NULL.  Supported: D in {64, 256, 512},
 * g in {1, 2, 4, 8, 16}; anything else returns GA_ERR_UNSUPPORTED.
 * bf16 MFMA with fp32 accumulation; probabilities are rounded to bf16 before
 * the value product and the row sum uses the same rounded values.
 */
int gemma_attn_prefill(const gemma_attn_config* cfg, int32_t layer_idx, int32_t batch, int32_t seq,
                       const void* q, const void* k, const void* v, void* out, float* lse,
                       void* stream);

/*
 * gemma_attn_prefill with the query rotary done inside the attention kernel:
 * the prologue's step 2 for q (no query norm) without its write and re-read
 * of q.  q_raw [B,S,Hq,D] bf16 holds the queries before rotary; each
 * workgroup turns the columns it loads in registers, in the prologue's pairs
 * (i, i + D/2) by the angle (p / pos_div) * theta^(-2i/D), p = pos0[b] + s,
 * and rounds them to bf16 as the prologue does before the products.  k must
 * already be processed (gemma_qk_prologue with q_in = NULL); v and the rest as
 * for gemma_attn_prefill.  pos0: device int32 [B], or NULL for zeros.
 * The rotation is the prologue's own arithmetic (the same fp64 angles,
 * hardware cosine and sine, and fused multiply-add), so without a query norm
 * the result equals gemma_qk_prologue + gemma_attn_prefill bit for bit.
 * For layers with no query norm and a full-width rotary (r = D), at head width
 * 256 with separate keys and values (the Gemma 2 layers); other layers return
 * GA_ERR_UNSUPPORTED and take gemma_qk_prologue + gemma_attn_prefill.
 */
int gemma_attn_prefill_qrope(const gemma_attn_config* cfg, int32_t layer_idx, int32_t batch, int32_t seq,
                             const void* q_raw, const void* k, const void* v, const int32_t* pos0, void* out,
                             float* lse, void* stream);

/*
 * gemma_attn_prefill over a padded batch.  generate() on the Gemma, Gemma 2
 * and Gemma 4 pages takes attention_mask (batch, seq) with 1 = keep and
 * 0 = padding; read here as contiguous padding at the ends, so sequence b
 * keeps rows [seq_start[b], seq_end[b]) (left padding: start > 0; ragged
 * lengths: end < seq).  Padded rows are neither queries nor keys and are never
 * read (they may hold anything); their output rows are 0 and their lse -inf.
 * The causal and window masks stay positional (i - j).  seq_start / seq_end:
 * device int32 [B], or NULL for 0 / seq; clamped on the device to
 * 0 <= start <= end <= seq.  Other arguments as for gemma_attn_prefill.
 */
int gemma_attn_prefill_ragged(const gemma_attn_config* cfg, int32_t layer_idx, int32_t batch, int32_t seq,
                              const void* q, const void* k, const void* v, void* out, float* lse,
                              const int32_t* seq_start, const int32_t* seq_end, void* stream);

/*
 * Bytes of device workspace gemma_attn_decode needs for (layer, batch, max_ctx)
 * on the current device; 0 when the arguments are invalid or the shape is
 * unsupported (batch > 65535).
 */
size_t gemma_attn_decode_workspace_size(const gemma_attn_config* cfg, int32_t layer_idx, int32_t batch,
                                        int32_t max_ctx);

/*
 * One new token per sequence against a contiguous KV cache (the decode step of
 * the pages' generate()).  q [B,Hq,D] bf16 is the processed query of the token at
 * position ctx_len[b] - 1.  k_cache, v_cache [B,max_ctx,Hkv,D] bf16 hold the
 * processed keys and the values of positions 0..max_ctx-1, the current token
 * included; v_cache is ignored (may be NULL) on keys-as-values layers.
 * ctx_len: device int32 [B]; entries are clamped to [0, max_ctx] on the device.
 * Keys read: rows [max(0, ctx - W), ctx) on local layers, [0, ctx) on global
 * layers; no other cache row is touched.  ctx = 0 gives out = 0, lse = -inf.
 * out [B,Hq,D] bf16; lse fp32 [B,Hq] or NULL.
 * workspace: device buffer of at least gemma_attn_decode_workspace_size() bytes
 * (split-KV partials; contents on entry are ignored).  Supported: D in
 * {64, 256, 512}, g in {1, 2, 4, 8, 16}.
 */
int gemma_attn_decode(const gemma_attn_config* cfg, int32_t layer_idx, int32_t batch, int32_t max_ctx,
                      const void* q, const void* k_cache, const void* v_cache, const int32_t* ctx_len,
                      void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Several new tokens per sequence against the contiguous cache: chunked
 * prefill and the verification of speculative drafts (generate() on the Gemma
 * pages; the atlas summary's MTP drafter, which scores any draft length).
 * Token t of sequence b sits at position i = ctx_len[b] - q_len + t and sees
 * cache rows j <= i, and on local layers j > i - W (the same mask as prefill,
 * against the cache).  q [B,q_len,Hq,D] bf16 holds the processed queries; the
 * caches hold processed keys and values of positions 0..ctx-1, new tokens
 * included (see gemma_qk_prologue_cache); v_cache is ignored on keys-as-values
 * layers.  kv_start: device int32 [B] or NULL: cache rows before kv_start[b]
 * are not read (the left padding of a padded prefill, see
 * gemma_attn_prefill_ragged).  out [B,q_len,Hq,D] bf16; lse fp32
 * [B,Hq,q_len] or NULL.  Rows with no visible key (i < 0, or i < kv_start[b])
 * give out = 0, lse = -inf.  ctx_len entries are clamped to [0, max_ctx] on
 * the device; 1 <= q_len <= max_ctx.  workspace: at least
 * gemma_attn_decode_multi_workspace_size() bytes.  q_len = 1 with kv_start =
 * NULL is exactly gemma_attn_decode.
 */
int gemma_attn_decode_multi(const gemma_attn_config* cfg, int32_t layer_idx, int32_t batch, int32_t q_len,
                            int32_t max_ctx, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* ctx_len, const int32_t* kv_start, void* out, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Workspace bytes of gemma_attn_decode_multi on the current device, which
 * also cover gemma_attn_decode_int8 of the same shape (the larger of the two
 * launch plans' needs); 0 when the arguments are invalid or the shape is
 * unsupported (batch > 65535, KV heads x ceil(g * q_len / 16) > 65535,
 * Hq x q_len >= 2^31). */
size_t gemma_attn_decode_multi_workspace_size(const gemma_attn_config* cfg, int32_t layer_idx, int32_t batch,
                                              int32_t q_len, int32_t max_ctx);

/*
 * gemma_attn_decode_multi without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  It allocates nothing: the split
 * partials live in a fixed 80 MiB device array of the library, one per GPU,
 * held from the library's first use of that GPU until the process ends.  Every
 * call on a GPU uses that GPU's one array, so calls that overlap on one GPU
 * (on different streams, or from different threads) race and must be
 * serialised by the caller; calls on different GPUs are independent.  Each
 * call writes every part of the array it reads before reading it, so nothing
 * needs clearing between calls.  Arguments, results and errors as for
 * gemma_attn_decode_multi, plus GA_ERR_SCRATCH_LIMIT when
 * gemma_attn_decode_multi_workspace_size() of the shape exceeds 80 MiB
 * (e.g. 64 sequences of up to 65536 keys at head width 512 with 16 new tokens);
 * nothing is enqueued then.
 */
int gemma_attn_decode_multi_noalloc(const gemma_attn_config* cfg, int32_t layer_idx, int32_t batch, int32_t q_len,
                                    int32_t max_ctx, const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* ctx_len, const int32_t* kv_start, void* out, float* lse,
                                    void* stream);

/*
 * Prologue of q_len new tokens per sequence that appends them to the cache:
 * the same QK-norm and rotary as gemma_qk_prologue, with token s of sequence
 * b at position p = ctx_len[b] - q_len + s (ctx_len counts the new tokens).
 * q_in [B,q_len,Hq,D] -> q_out (bf16, may alias q_in exactly); k_in
 * [B,q_len,Hkv,D] is normed and rotated into k_cache [B,max_ctx,Hkv,D] at row
 * p; v_in [B,q_len,Hkv,D] is copied unchanged into v_cache at row p (both
 * ignored, may be NULL, on keys-as-values layers).  Rows p outside
 * [0, max_ctx) are skipped; no other cache row is written.
 */
int gemma_qk_prologue_cache(const gemma_attn_config* cfg, int32_t layer_idx, int32_t batch, int32_t q_len,
                            int32_t max_ctx, const void* q_in, const void* k_in, const void* v_in, void* q_out,
                            void* k_cache, void* v_cache, const float* q_norm_w, const float* k_norm_w,
                            const int32_t* ctx_len, void* stream);

/*
 * int8 KV cache (the google-gemma-4 atlas summary, "Training" section: int8
 * KV caching is offered; no format is given).  Reading adopted: symmetric
 * absmax quantization of each (token, KV head) vector x of width D:
 *   s = max|x| / 127 (fp32),  c = round-half-even(x / s) in [-127, 127]
 * (fp32 division; s = 0 and c = 0 for an all-zero vector), dequantized as
 * c * s.  Layouts: codes int8 [B,max_ctx,Hkv,D] (the bf16 cache's layout at
 * one byte per element); scales fp32 [B,Hkv,max_ctx] (the scales of one head
 * are contiguous over positions).  Keys are quantized after QK-norm and
 * rotary and their bf16 rounding, values as given.
 */

/*
 * gemma_attn_decode_multi against an int8 cache.  k_codes/k_scales hold the
 * processed keys, v_codes/v_scales the values (both ignored, may be NULL, on
 * keys-as-values layers, where the key codes serve as values).  Scores use
 * s_j * (q . c_j); the value scale multiplies each probability before its
 * bf16 rounding.  q, out, lse, ctx_len, kv_start, workspace and errors as
 * for gemma_attn_decode_multi, whose workspace size applies unchanged.
 * Pointers 16-byte aligned.
 */
int gemma_attn_decode_int8(const gemma_attn_config* cfg, int32_t layer_idx, int32_t batch, int32_t q_len,
                           int32_t max_ctx, const void* q, const void* k_codes, const float* k_scales,
                           const void* v_codes, const float* v_scales, const int32_t* ctx_len,
                           const int32_t* kv_start, void* out, float* lse, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * gemma_qk_prologue_cache appending to an int8 cache: the processed keys
 * (bf16-rounded) and the raw values of the q_len new tokens are quantized
 * into rows p = ctx_len[b] - q_len + s of the codes and scales (rows outside
 * [0, max_ctx) skipped).  Value arguments are ignored, may be NULL, on
 * keys-as-values layers.
 */
int gemma_qk_prologue_cache_int8(const gemma_attn_config* cfg, int32_t layer_idx, int32_t batch, int32_t q_len,
                                 int32_t max_ctx, const void* q_in, const void* k_in, const void* v_in, void* q_out,
                                 void* k_codes, float* k_scales, void* v_codes, float* v_scales,
                                 const float* q_norm_w, const float* k_norm_w, const int32_t* ctx_len, void* stream);

/*
 * Quantize rows x [B,S,Hkv,D] bf16 (keys already processed, or values) into an
 * int8 cache at rows pos0[b] + s (pos0: device int32 [B], NULL for zeros);
 * rows outside [0, max_ctx) are skipped.  Fills a cache from a prefill's
 * keys and values.  D a power of two in [8, 512].
 */
int gemma_kv_quantize_int8(int32_t batch, int32_t seq, int32_t num_kv_heads, int32_t head_dim, int32_t max_ctx,
                           const void* x, const int32_t* pos0, void* codes, float* scales, void* stream);

/* Static, human-readable text of an error code. */
const char* gemma_attn_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* GEMMA_ATTN_H */
