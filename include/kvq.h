/*
 * kvq.h - quantized paged KV cache for decode attention on MI355X (gfx950).
 *
 * C ABI of libkvq.so. Every argument is a plain pointer or integer: host
 * pointers are marked [host], device (HBM) pointers [dev]. The library never
 * allocates device memory (its one device-resident buffer, the static
 * workspace of kvq_decode_noalloc, is part of its loaded code); every
 * device buffer an argument names belongs to the caller and
 * must stay alive until the work queued on `stream` has finished. `stream`
 * is a hipStream_t passed as void* (NULL = the default stream). All device
 * work is enqueued asynchronously on that stream; no entry point synchronizes
 * the host or allocates, so store/decode may be recorded in a HIP graph.
 *
 * Errors: every entry point returns KVQ_OK (0) or a negative kvq_status.
 * Argument errors are detected on the host BEFORE anything is enqueued, so a
 * failed call has no device side effect. Values that live in device memory
 * (slot ids, sequence lengths, page ids) are not read by the host; kernels
 * skip slots outside the cache and treat page ids outside [0, num_pages) as
 * pages with no tokens, so bad device data gives wrong numbers, never an
 * out-of-bounds access.
 *
 * Sources (the pages this library implements):
 *  [P1] SGLang "Quantized KV Cache" documentation page: the KV formats
 *       (FP8 E4M3/E5M2, FP4 E2M1 with 8-bit block exponents over 16
 *       elements, NVFP4), per-tensor scales defaulting to 1.0, and the
 *       requirement that dequantization be fused into the attention kernel.
 *  [P2] "KV cache quantization mechanism and traps": bytes per token and the
 *       K-channel / V-token outlier structure; scales fixed at prefill are
 *       reused for appended tokens.
 *  [P3] vLLM "Quantized KV Cache" page: per-tensor k/v scales, calibration.
 *  [P4] Analysis of SGLang PR #21954 (NVFP4 KV cache): create_buffers /
 *       quantize_and_store, separate data and block-scale buffers, the
 *       two-level FP32 global + E4M3 per-16-block NVFP4 scaling, E2M1_MAX.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* KV code format ([P1] "Supported formats"; [P4] strategy classes). */
typedef enum kvq_dtype {
  KVQ_FP8_E4M3 = 1, /* OCP E4M3FN, max 448, one fp32 scale per tensor      */
  KVQ_FP8_E5M2 = 2, /* OCP E5M2, max 57344, one fp32 scale per tensor      */
  KVQ_FP4_MX16 = 3, /* E2M1 + one E8M0 (2^(c-127)) scale per 16 elements   */
  KVQ_NVFP4 = 4     /* E2M1 + one E4M3 scale per 16 elements + fp32 global */
} kvq_dtype;

typedef enum kvq_kind {
  KVQ_GQA = 0, /* K and V rows per KV head; G = Hq / Hkv query heads share one */
  KVQ_MLA = 1  /* one latent row per token shared by every query head;
                  K = the whole row (head_dim), V = its first v_dim elements   */
} kvq_kind;

/* How FP8 scales are kept (cache descriptor field scale_mode). */
typedef enum kvq_scale_mode {
  KVQ_SCALE_TENSOR = 0, /* one k_scale and one v_scale ([P1] "Scaling factors")           */
  KVQ_SCALE_HEAD = 1,   /* one per KV head: k/v_scale = [num_kv_heads] ([P3] "Supported
                           schemes", per-attention-head quantization)                    */
  KVQ_SCALE_KIVI = 2    /* K: one scale per (KV head, channel), k_scale = [num_kv_heads]
                           [head_dim]; V: one scale per (token, KV head), computed when
                           the token is stored ([P2] "why K and V distributions differ":
                           per-channel K, per-token V)                                    */
} kvq_scale_mode;

typedef enum kvq_status {
  KVQ_OK = 0,
  KVQ_ERR_ARG = -1,         /* null pointer, negative size, inconsistent shape */
  KVQ_ERR_UNSUPPORTED = -2, /* valid but not implemented (dtype x kind x dims) */
  KVQ_ERR_SIZE = -3,        /* caller buffer (cache memory, workspace) too small */
  KVQ_ERR_HIP = -4,         /* a HIP launch reported an error */
  KVQ_ERR_WORKSPACE = -5    /* kvq_decode_noalloc: the call needs more than the
                               library's static workspace (80 MiB) */
} kvq_status;

/* Shape of one layer's cache. */
typedef struct kvq_cache_desc {
  int32_t dtype;        /* kvq_dtype */
  int32_t kind;         /* kvq_kind */
  int32_t num_kv_heads; /* GQA: 1 <= Hkv <= 4096; MLA: must be 1 */
  int32_t head_dim;     /* GQA: D; MLA: latent + rope dims (Dk) */
  int32_t v_dim;        /* GQA: must equal head_dim; MLA: latent dims (Dv) */
  int32_t page_size;    /* tokens per page, a multiple of 16, at most 65536 */
  int64_t num_pages;    /* physical pages in the pool, >= 1 */
  int32_t scale_mode;   /* kvq_scale_mode; KVQ_SCALE_HEAD and KVQ_SCALE_KIVI are for
                           FP8 GQA only, every other cache uses KVQ_SCALE_TENSOR.
                           HEAD: every k_scale / v_scale argument is an array of
                           num_kv_heads floats. KIVI: k_scale is [num_kv_heads]
                           [head_dim] floats, v_scale is unused (NULL), and the
                           cache holds one fp32 V scale per stored token. */
} kvq_cache_desc;

/* Supported combinations (others return KVQ_ERR_UNSUPPORTED):
 *   GQA x {E4M3, E5M2}: head_dim in {64, 128}, any scale_mode
 *   GQA x FP4_MX16:     head_dim == 128
 *   MLA x NVFP4:        head_dim == 576, v_dim == 512
 *   decode, GQA:        G = Hq / Hkv in [1, 16], max_seq_len <= 2,097,152
 *   decode, MLA:        1 <= Hq <= 128                                       */

/* Byte offsets (from the start of the caller's cache memory) and sizes of the
 * buffers inside one cache. Absent buffers have size 0. Each buffer is
 * [num_pages][num_kv_heads][page block]; the page block is page_size tokens
 * in 16-token tiles. Element (t, d) of a page (t16 = t % 16, tile = t / 16,
 * b = d / 16; offsets inside the block):
 *   GQA FP8, tile = 16*D bytes, offset tile*16*D +
 *     K: 256*(d/16) + 16*t16 + d%16
 *     V: 1024*(d/64) + 16*(16*(t16/4) + d%16) + 4*((d/16)%4) + t16%4
 *   GQA FP4_MX16 (two E2M1 codes per byte, even d in the low nibble),
 *   code tile = 8*D bytes, scale tile = D bytes:
 *     K code:  256*(d/32) + 16*t16 + (d%32)/2
 *     V code:  1024*(d/128) + 16*(16*(t16/4) + (d%128)/8) + 4*(t16%4) + (d%8)/2
 *     K scale: 32*(b/2) + 2*t16 + b%2             (E8M0 code)
 *     V scale: 4*((D/16)*(t16/4) + b) + t16%4     (E8M0 code)
 *   MLA NVFP4 (Dk 576, Dv 512), code tile = 4608 B, scale tile = 576 B,
 *   g4 = t16/4, tt = t16%4:
 *     code,  d < 512:  2*(((d/64*4 + g4)*16 + (d%64)/4)*4 + tt) + (d%4)/2
 *     code,  d >= 512: 4096 + 2*((g4*16 + (d-512)/4)*4 + tt) + (d%4)/2
 *     scale, b < 32:   4*((b/4*4 + g4)*4 + b%4) + tt      (E4M3 code)
 *     scale, b >= 32:  512 + 4*(g4*4 + b-32) + tt
 *   GQA FP8 with scale_mode KIVI adds the V scale buffer, one fp32 per token:
 *     V scale of token t: float t of the (page, kv head) block (4*page_size B)
 * The K layouts put the 16 tokens of a tile at consecutive 16-byte lanes and
 * the V layouts put 4 consecutive tokens of one element (FP8) or of one
 * 4- or 8-element group (MLA, FP4) in one lane load, so each wave of the
 * decode kernels reads a tile with fully coalesced 16-byte loads straight
 * into matrix-core operand order. Every byte holds codes of one token only,
 * so a store never rewrites another token's bits.                          */
typedef struct kvq_layout {
  size_t k_codes_offset, k_codes_bytes;
  size_t v_codes_offset, v_codes_bytes;
  size_t k_scales_offset, k_scales_bytes;
  size_t v_scales_offset, v_scales_bytes;
  size_t scratch_offset, scratch_bytes; /* used by kvq_compute_scale */
  size_t total_bytes;
} kvq_layout;

typedef struct kvq_cache kvq_cache; /* opaque host handle */

/* Human-readable text of a kvq_status. Never NULL. */
const char* kvq_status_string(int status);

/* Storage bytes per cached token of one layer, K+V codes plus per-block
 * scales ([P2] bytes-per-token formula; [P1] "Memory savings": the FP4
 * block-scale overhead, 4 + 8/16 bits per element). [host] out. */
int kvq_bytes_per_token(const kvq_cache_desc* desc, double* bytes_out);

/* create_buffers analogue ([P4]): lay out the data and block-scale buffers of
 * one cache inside ONE caller-owned device allocation.
 *   Query:  dev_mem == NULL -> *bytes_needed = size to allocate, *out untouched.
 *   Bind:   dev_mem != NULL (256-byte aligned), dev_bytes >= bytes_needed ->
 *           *out = new host handle pointing into dev_mem.
 * Nothing is written to dev_mem (initial contents are the caller's). The
 * handle is freed with kvq_free_handle; it does not own dev_mem.
 * Errors: KVQ_ERR_ARG (null desc/out, bad shape), KVQ_ERR_UNSUPPORTED,
 * KVQ_ERR_SIZE (dev_bytes too small). */
int kvq_alloc_pages(const kvq_cache_desc* desc, void* dev_mem, size_t dev_bytes,
                    size_t* bytes_needed, kvq_cache** out);

/* Offsets of the buffers of a bound cache (see kvq_layout). [host] out. */
int kvq_cache_layout(const kvq_cache* cache, kvq_layout* out);

/* Frees the host handle only (never the device memory). NULL is ignored. */
void kvq_free_handle(kvq_cache* cache);

/* Per-tensor scale from the tensor's absolute maximum ([P1] "Scaling
 * factors"; [P3] calibration: a scale estimated once, then kept fixed):
 *   FP8 caches:  *scale_out = amax / 448 (E4M3) or amax / 57344 (E5M2)
 *   NVFP4 cache: *scale_out = amax / (6 * 448)   (the global scale g)
 *   amax == 0 gives 1.0. amax is taken jointly over x0[0..n0) and
 *   x1[0..n1) (x1 may be NULL with n1 == 0); division is IEEE binary32.
 * x0, x1: [dev] BF16. scale_out: [dev] one float. Uses the cache's scratch
 * buffer: concurrent calls on one cache race.
 * With scale_mode HEAD or KIVI, x0 and x1 are [tokens][num_kv_heads][head_dim]
 * (n0, n1 multiples of num_kv_heads*head_dim, both 16-byte aligned) and
 *   HEAD: scale_out[h] = amax over head h / format max, h < num_kv_heads;
 *   KIVI: scale_out[h*head_dim + d] = amax over channel d of head h / format
 *         max (the K channel scales; V needs none).
 * Errors: KVQ_ERR_ARG, KVQ_ERR_UNSUPPORTED (FP4_MX16 has no tensor scale). */
int kvq_compute_scale(const kvq_cache* cache, const void* x0, int64_t n0, const void* x1,
                      int64_t n1, float* scale_out, void* stream);

/* quantize_and_store ([P4]): quantize num_tokens new tokens and write codes
 * and block scales at their slots.
 *   k, v: [dev] BF16, GQA [num_tokens][num_kv_heads][head_dim] each;
 *         MLA: k = latent rows [num_tokens][head_dim], v must be NULL.
 *   slot_mapping: [dev] int64 [num_tokens], slot = page * page_size + offset;
 *         a negative slot or one >= num_pages*page_size skips the token.
 *   k_scale, v_scale: [dev] fp32 scalars. FP8: per-tensor scales, NULL = 1.0
 *         ([P1]: default when no scale is given); code = RNE_sat(x / scale);
 *         with scale_mode HEAD, [num_kv_heads] arrays indexed by KV head;
 *         KIVI: k_scale = the [num_kv_heads][head_dim] channel scales
 *         (required), v_scale unused; each token's V row gets its own scale
 *         fl32(amax / format max) (1.0 for an all-zero row), stored in the
 *         cache's V scale buffer.
 *         NVFP4: k_scale = global scale g (required), v_scale unused.
 *         FP4_MX16: both unused (block exponents are computed here from each
 *         16-element block's amax: e = floor(log2 amax) - 2).
 * Inputs must be finite. Two tokens mapped to one slot race.
 * Errors: KVQ_ERR_ARG, KVQ_ERR_UNSUPPORTED (more than 2^32 - 256 16-element
 * pieces in one call: num_tokens x rows x head_dim / 16, rows = num_kv_heads
 * or 1 for MLA), KVQ_ERR_HIP. num_tokens == 0 is a no-op. */
int kvq_store(const kvq_cache* cache, const void* k, const void* v,
              const int64_t* slot_mapping, int32_t num_tokens, const float* k_scale,
              const float* v_scale, void* stream);

/* Bytes of device workspace kvq_decode needs for this batch shape: 0 when
 * one context split covers every sequence (no partials to merge), and 0 for
 * arguments the decode itself rejects (a null handle, negative sizes, MLA
 * with more than 128 query heads), which the decode call then reports. */
size_t kvq_decode_workspace_bytes(const kvq_cache* cache, int32_t batch, int32_t num_q_heads,
                                  int32_t max_seq_len);

/* Paged decode attention with dequantization fused into the kernel ([P1]
 * performance warning: unfused dequantization is very slow) and an online
 * softmax. For every sequence b and query head h (kv head = h / G):
 *   out[b][h][:] = sum_t softmax_t(sm_scale * q[b][h] . K^[t]) V^[t]
 *   lse[b][h]    = log sum_t exp(sm_scale * q[b][h] . K^[t])
 * over tokens t < seq_lens[b], token t at page page_table[b*stride + t/P],
 * offset t%P. K^, V^ are the dequantized codes times their scales.
 *   q:          [dev] BF16 [batch][num_q_heads][head_dim]
 *   page_table: [dev] int32, row stride page_table_stride (>= ceil(max_seq_len/P))
 *   seq_lens:   [dev] int32 [batch], each in [0, max_seq_len]
 *   max_seq_len [host]: upper bound used to size the launch
 *   k_scale, v_scale: [dev] fp32 (FP8: per-tensor scales, NULL = 1.0, or
 *               [num_kv_heads] arrays with scale_mode HEAD; KIVI: k_scale =
 *               the channel scales (required), V scales from the cache;
 *               NVFP4: k_scale = global scale g, required; MX16: unused)
 *   out:        [dev] fp32 [batch][num_q_heads][v_dim]
 *   lse:        [dev] fp32 [batch][num_q_heads] (natural log) or NULL
 *   workspace:  [dev] >= kvq_decode_workspace_bytes(...), 256-byte aligned
 *               (partial results of the context splits); may be NULL when
 *               kvq_decode_workspace_bytes returns 0. Calls that share one
 *               workspace must not overlap on the device.
 * A sequence of length 0 gets out = 0 and lse = -inf.
 * Errors: KVQ_ERR_ARG, KVQ_ERR_UNSUPPORTED, KVQ_ERR_SIZE, KVQ_ERR_HIP. */
int kvq_decode(const kvq_cache* cache, const void* q, int32_t batch, int32_t num_q_heads,
               const int32_t* page_table, int32_t page_table_stride, const int32_t* seq_lens,
               int32_t max_seq_len, float sm_scale, const float* k_scale, const float* v_scale,
               float* out, float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* kvq_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation, kernels and split plan, with the split partials kept in
 * a workspace the library holds in device memory (a static array of 80 MiB
 * on every GPU the library runs on, kept until the process ends) instead of
 * a caller buffer. The caller still owns every input and output.
 * The first call on a device looks up that device's workspace address (the
 * device of `stream`; the current device for the null stream); no call
 * allocates or frees memory. Calls on one GPU share its workspace: calls that
 * overlap on that GPU (other streams, other threads, concurrent graph
 * replays) race, and must be serialized by the caller. Each call writes every
 * partial it reads, so nothing has to be cleared between calls.
 * Arguments and errors are kvq_decode's without the workspace, plus
 * KVQ_ERR_WORKSPACE when kvq_decode_workspace_bytes for this shape exceeds
 * 80 MiB (83,886,080 bytes), returned before anything is enqueued. */
int kvq_decode_noalloc(const kvq_cache* cache, const void* q, int32_t batch, int32_t num_q_heads,
                       const int32_t* page_table, int32_t page_table_stride, const int32_t* seq_lens,
                       int32_t max_seq_len, float sm_scale, const float* k_scale, const float* v_scale,
                       float* out, float* lse, void* stream);

/* One decode step in one launch: appends the token at position seq_lens[b] - 1
 * of every sequence b, then decodes. Equivalent to kvq_store of those tokens
 * with slot = page_table[b*stride + (L-1)/P] * P + (L-1)%P (L = seq_lens[b];
 * a sequence with L = 0 or an out-of-pool page stores nothing), followed by
 * kvq_decode with the same arguments: the quantization is the store's and
 * the codes written are bit-identical ([P4] quantize_and_store, then decode
 * over the quantized cache). The context split that holds position L-1
 * quantizes and writes that token before it reads the tile that holds it,
 * which saves the separate store launch of a decode step.
 *   k_new, v_new: [dev] BF16, GQA [batch][num_kv_heads][head_dim] each;
 *                 MLA: k_new = latent rows [batch][head_dim], v_new must be NULL.
 * All other arguments, the workspace and the errors are kvq_decode's; a NULL
 * k_new (or, for GQA, v_new) is KVQ_ERR_ARG. */
int kvq_decode_append(const kvq_cache* cache, const void* k_new, const void* v_new, const void* q,
                      int32_t batch, int32_t num_q_heads, const int32_t* page_table,
                      int32_t page_table_stride, const int32_t* seq_lens, int32_t max_seq_len,
                      float sm_scale, const float* k_scale, const float* v_scale, float* out,
                      float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* FP8-domain decode ([P3] overview: with an FP8 KV cache, the Flash
 * Attention 3 backend runs attention itself in FP8, the query quantized to
 * FP8 like K and V; [P3] "Supported schemes": q_scale = [num_q_heads] per
 * attention head or [1] per tensor). kvq_decode with the query first rounded
 * to E4M3 codes, code = RNE_sat(q / q_scale) (binary32 division, saturating
 * at +-448, E4M3 whatever the cache's FP8 format), and the scores
 *   sm_scale * q_scale * k_scale * (E4M3(code) . K codes)
 * taken on FP8 matrix cores from the cached codes as they are; the softmax,
 * the value side and every other argument are kvq_decode's.
 * MLA (NVFP4 latent): NVFP4 values are not FP8 values, so the keys are the
 * E4M3 rows of the dequantize_prev_kv step ([P4] "code analysis") with the
 * output scale 8g: K8 = RNE_E4M3(K^ / 8g), exact division, no saturation
 * (|K^| <= 6 * 448 * g); the scores are
 *   sm_scale * q_scale * 8g * (E4M3(code) . K8)
 * on FP8 matrix cores, and the values stay the exact NVFP4 latent (V^ =
 * K^[:v_dim], fp16 matrix cores), as in kvq_decode.
 *   q_scale: [dev] fp32, one value (GQA scale_mode TENSOR, and MLA) or
 *            [num_q_heads] (GQA scale_mode HEAD), 4-byte aligned; NULL =
 *            1.0. Queries beyond 448 * q_scale saturate.
 *   k_scale: GQA as kvq_decode; MLA the global scale g (required).
 * Caches: GQA E4M3 or E5M2 with scale_mode TENSOR or HEAD, and MLA NVFP4
 * (KVQ_ERR_UNSUPPORTED otherwise: MX16 codes are not FP8, KIVI folds a
 * channel scale into the query). Errors as kvq_decode. */
int kvq_decode_fp8q(const kvq_cache* cache, const void* q, int32_t batch, int32_t num_q_heads,
                    const int32_t* page_table, int32_t page_table_stride, const int32_t* seq_lens,
                    int32_t max_seq_len, float sm_scale, const float* q_scale, const float* k_scale,
                    const float* v_scale, float* out, float* lse, void* workspace,
                    size_t workspace_bytes, void* stream);

/* kvq_decode_append in the FP8 domain: the append of kvq_decode_append, then
 * kvq_decode_fp8q, in one launch. Arguments as those two; a NULL k_new (or
 * v_new) is KVQ_ERR_ARG. */
int kvq_decode_append_fp8q(const kvq_cache* cache, const void* k_new, const void* v_new,
                           const void* q, int32_t batch, int32_t num_q_heads,
                           const int32_t* page_table, int32_t page_table_stride,
                           const int32_t* seq_lens, int32_t max_seq_len, float sm_scale,
                           const float* q_scale, const float* k_scale, const float* v_scale,
                           float* out, float* lse, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Query scales for kvq_decode_fp8q from a calibration batch of queries ([P3]
 * "Scale calibration": estimated once, then kept fixed):
 *   scale_mode TENSOR: q_scale_out[0] = amax(q) / 448
 *   scale_mode HEAD:   q_scale_out[h] = amax over query head h / 448
 * (binary32 division; an all-zero tensor or head gives 1.0).
 *   q: [dev] BF16 [n_tokens][num_q_heads][head_dim], 16-byte aligned.
 * Uses the cache's scratch buffer: concurrent calls on one cache race.
 * MLA caches (scale_mode TENSOR): one value over [n_tokens][num_q_heads][576].
 * Errors: KVQ_ERR_ARG, KVQ_ERR_UNSUPPORTED (caches kvq_decode_fp8q rejects),
 * KVQ_ERR_HIP. n_tokens = 0 gives 1.0. */
int kvq_compute_q_scale(const kvq_cache* cache, const void* q, int64_t n_tokens,
                        int32_t num_q_heads, float* q_scale_out, void* stream);

/* dequantize_prev_kv ([P4] "code analysis"): turn listed pages of an FP4
 * cache into FP8 E4M3 rows, the dq_k / dq_v workspaces an FP8 prefill kernel
 * reads when a new chunk attends to an already quantized prefix (the pages
 * have no FP4 prefill kernel). Every element is dequantized exactly and
 * rounded once to binary32 (MX16: e2m1 * 2^(c-127); NVFP4: e2m1 * e4m3 * g),
 * then code = RNE_sat_E4M3(x^ / s) with the per-tensor output scale s
 * (binary32 division, saturating at +-448).
 *   pages:       [dev] int32 [n_pages] page ids; an id outside
 *                [0, num_pages) yields all-zero rows.
 *   g_scale:     [dev] fp32, NVFP4 global scale g (required); unused for MX16.
 *   k_scale_out, v_scale_out: [dev] fp32 output scales s, NULL = 1.0; each
 *                must be positive and finite. MLA: v_scale_out must be NULL.
 *   dq_k, dq_v:  [dev] E4M3 bytes, 16-byte aligned, written token-major:
 *                GQA [n_pages][num_kv_heads][page_size][head_dim] each;
 *                MLA dq_k = [n_pages][page_size][head_dim] latent rows
 *                (V is their first v_dim elements), dq_v must be NULL.
 * Reads the cache only; n_pages = 0 launches nothing.
 * Errors: KVQ_ERR_ARG, KVQ_ERR_UNSUPPORTED (FP8 caches), KVQ_ERR_HIP. */
int kvq_dequantize_prev_kv(const kvq_cache* cache, const int32_t* pages, int32_t n_pages,
                           const float* g_scale, const float* k_scale_out, const float* v_scale_out,
                           void* dq_k, void* dq_v, void* stream);

/* Extend (chunked prefill) attention over a quantized prefix ([P4] "code
 * analysis": dequantize_prev_kv turns the FP4 prefix into E4M3 workspaces for
 * an FP8 prefill kernel; this is that kernel). For sequence b with chunk rows
 * cu_q[b] .. cu_q[b+1]-1 (C_b tokens) and prefix length L0 = prefix_len[b],
 * chunk token i and query head h (kv head = h / G) attend to
 *   prefix tokens t < L0: K^ = E4M3(dq_k row) * s_k, V^ = E4M3(dq_v row) * s_v,
 *     token t at row t % page_size of workspace page page_off[b] + t / page_size
 *     (the [n_pages][num_kv_heads][page_size][head_dim] layout that
 *     kvq_dequantize_prev_kv writes), and
 *   chunk tokens 0..i (causal): the BF16 rows k_new / v_new,
 * with scores sm_scale * q . K^ and a softmax over all of them:
 *   out[row][h][:] = sum softmax * V^,  lse[row][h] = log sum exp(score).
 *   q:            [dev] BF16 [total_q][num_q_heads][head_dim]
 *   k_new, v_new: [dev] BF16 [total_q][num_kv_heads][head_dim]
 *   cu_q:         [dev] int32 [batch + 1] chunk offsets (clamped to [0, total_q])
 *   prefix_len, page_off: [dev] int32 [batch]; prefix tokens whose page falls
 *                 outside [0, n_pages) are dropped
 *   dq_k, dq_v:   [dev] E4M3 workspaces of n_pages pages (may be NULL when n_pages is 0)
 *   s_k, s_v:     [dev] fp32 workspace scales, NULL = 1.0
 *   max_chunk:    [host] upper bound of every chunk length (sizes the launch)
 *   out:          [dev] fp32 [total_q][num_q_heads][head_dim]; lse [dev] fp32
 *                 [total_q][num_q_heads] (natural log) or NULL
 * Supported: head_dim 128, G = num_q_heads / num_kv_heads in {1, 2, 4, 8, 16}
 * (KVQ_ERR_UNSUPPORTED otherwise). q, k_new, v_new, dq_k, dq_v and out must be
 * 16-byte aligned. Allocates nothing; batch, total_q or max_chunk 0 is a no-op.
 * Errors: KVQ_ERR_ARG, KVQ_ERR_UNSUPPORTED, KVQ_ERR_HIP. */
int kvq_extend_attention(const void* q, const void* k_new, const void* v_new, const int32_t* cu_q,
                         int32_t total_q, const int32_t* prefix_len, const void* dq_k,
                         const void* dq_v, const int32_t* page_off, int32_t n_pages,
                         const float* s_k, const float* s_v, int32_t batch, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                         int32_t max_chunk, float sm_scale, float* out, float* lse, void* stream);

/* Instrumentation (off by default). While enabled, every kernel launched by
 * kvq_store / kvq_decode(_append)(_fp8q) / kvq_compute_scale / kvq_compute_q_scale /
 * kvq_dequantize_prev_kv / kvq_extend_attention is bracketed by two HIP events
 * recorded on the call's stream (nothing else changes; do not enable while
 * capturing a HIP graph). Enabling or disabling clears the records.
 * kvq_profile_read synchronizes the recorded events and returns, for one
 * kernel family ("store", "decode", "merge", "amax", "dequant_prev", "extend"), the summed device
 * time in milliseconds and the number of launches, then forgets them.
 * Errors: KVQ_ERR_ARG (unknown name, null outputs), KVQ_ERR_HIP. */
int kvq_profile_enable(int on);
int kvq_profile_read(const char* kernel, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H */
