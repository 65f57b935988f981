// Internal declarations shared by the libkvq translation units (host handle,
// device conversion helpers, kernel launchers). Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

// ------------------------------------------------------------ host handle --
struct kvq_cache {
  kvq_cache_desc desc;
  kvq_layout layout;
  uint8_t* base;             // caller's device memory
  int64_t code_block_bytes;  // bytes of codes per (page, kv head)
  int64_t scale_block_bytes; // bytes of block scales per (page, kv head)
  int32_t split_target;      // decode workgroups the split planners aim at; 0 = default
};

namespace kvq {

constexpr int kTile = 16;      // tokens per tile inside a page
constexpr int kWaves = 4;      // waves per decode workgroup
constexpr int kAmaxBlocks = 1024;
constexpr int kMlaMaxSplitPages = 1024;  // page ids one MLA split stages in LDS
constexpr int kExtendRows = 256;         // (chunk token, query head) rows per extend workgroup
// device-resident workspace of kvq_decode_noalloc: 80 MiB per GPU (the
// DeepSeek-R1-shape MLA step, batch 64 x 128 heads x 4 splits, needs 64 MiB)
constexpr size_t kStaticWorkspaceBytes = (size_t)80 << 20;

// ------------------------------------------------------- vector typedefs --
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Two FP8 codes (bytes 0,1 or 2,3 of `w`) -> two exact BF16 / FP16 values.
// gfx950's converts decode OCP E4M3FN / E5M2; a scale operand of 1.0 leaves
// the value unscaled (the converts apply only the scale's power of two).
template <int FMT, bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  bf16x2 r = (FMT == KVQ_FP8_E4M3) ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI)
                                   : __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, HI);
  return __builtin_bit_cast(uint32_t, r);
}
template <int FMT, bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_f16x2(uint32_t w) {
  f16x2 r = (FMT == KVQ_FP8_E4M3) ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI)
                                  : __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(w, 1.0f, HI);
  return __builtin_bit_cast(uint32_t, r);
}

// E8M0 code -> the fp32 power of two 2^(c-127). Code 0 (2^-127 is a binary32
// subnormal, which the scaled converts do not take) maps to 2^-126.
__device__ __forceinline__ float e8m0_to_f32(uint32_t c) {
  c = c < 1u ? 1u : c;
  return __uint_as_float(c << 23);
}

// Byte `sel` of `w` (two E2M1 codes, low nibble first) times 2^e -> BF16 x2,
// exact (E2M1 has two significant bits).
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2_scaled(uint32_t w, float pow2) {
  bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, pow2, SEL);
  return __builtin_bit_cast(uint32_t, r);
}
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_f16x2(uint32_t w) {
  f16x2 r = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  f16x2 r = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 r = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, r);
}

// [lo16(a), lo16(b)] and [hi16(a), hi16(b)]
__device__ __forceinline__ uint32_t lo_halves(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t hi_halves(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// Wave-wide (64 lanes) xor shuffle.
__device__ __forceinline__ float shfl_xor_f32(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

}  // namespace kvq

// ------------------------------------------------------------- launchers --
struct GqaDecodeArgs {
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const uint8_t* k_scales;
  const uint8_t* v_scales;
  int64_t code_block_bytes;
  int64_t scale_block_bytes;
  int64_t num_pages;
  const uint16_t* q;
  const int32_t* page_table;
  int64_t page_table_stride;
  const int32_t* seq_lens;
  const float* k_scale;
  const float* v_scale;
  int scale_mode;       // kvq_scale_mode (FP8): HEAD -> k/v_scale [hkv]; KIVI -> k_scale [hkv][D],
                        // V scales per token in v_scales (fp32, scale_block_bytes = 4*P per page-head)
  float sm_scale_log2;  // sm_scale * log2(e)
  int batch, hq, hkv, group, page_size, max_len;
  int tiles_per_split, num_splits;
  float* ws_o;    // [B][Hq][S][D] when num_splits > 1
  float* ws_lse;  // [B][Hq][S]   (log2 domain)
  float* out;     // [B][Hq][D]
  float* lse;     // [B][Hq] or null (natural log)
  // optional append (kvq_decode_append): BF16 K/V rows [B][Hkv][D] of the token
  // at position seq_lens[b] - 1, quantized and written by the split holding it
  const uint16_t* new_k;
  const uint16_t* new_v;
  // FP8-domain attention (kvq_decode_fp8q): Q rounded to E4M3 with these
  // scales (TENSOR mode: [1]; HEAD mode: [hq]; null = 1.0) and QK^T on FP8
  // matrix cores straight from the cached codes
  int q8;
  const float* q_scale;
};

struct MlaDecodeArgs {
  const uint8_t* codes;
  const uint8_t* scales;
  int64_t num_pages;
  const uint16_t* q;
  const int32_t* page_table;
  int64_t page_table_stride;
  const int32_t* seq_lens;
  const float* g_scale;
  float sm_scale_log2;
  int batch, hq, page_size, max_len;
  int tiles_per_split, num_splits;
  float* ws_o;
  float* ws_lse;
  float* out;
  float* lse;
  // optional append (kvq_decode_append): BF16 latent rows [B][576] of the token
  // at position seq_lens[b] - 1, quantized and written before it is read
  const uint16_t* new_k;
  // FP8-domain attention (kvq_decode_fp8q): Q rounded to E4M3 with q_scale
  // ([1]; null = 1.0), keys as E4M3 codes of K^ / (8g), values exact
  int q8;
  const float* q_scale;
};

struct CombineArgs {
  const float* ws_o;
  const float* ws_lse;
  const int32_t* seq_lens;
  float* out;
  float* lse;
  int batch, hq, dv, num_splits, tokens_per_split, max_len;
};

// Extend attention over an E4M3 prefix workspace (kvq_extend_attention).
struct ExtendArgs {
  const uint16_t* q;       // BF16 [total_q][hq][128]
  const uint16_t* k_new;   // BF16 [total_q][hkv][128]
  const uint16_t* v_new;
  const int32_t* cu_q;     // [batch + 1]
  const int32_t* prefix_len;
  const int32_t* page_off;
  const uint8_t* dq_k;     // E4M3 [n_pages][hkv][page_size][128]
  const uint8_t* dq_v;
  const float* s_k;        // workspace scales (null = 1.0)
  const float* s_v;
  float* out;              // fp32 [total_q][hq][128]
  float* lse;              // fp32 [total_q][hq] or null (natural log)
  int total_q, n_pages, batch, hq, hkv, group, page_size, max_chunk;
  int q_tiles, n_work;     // tiles of kExtendRows/group chunk tokens per sequence; batch * hkv * q_tiles
  float sm_scale;
};

// Device address, on the device `stream` belongs to (the current device for
// the null stream), of the library's static decode workspace of
// kStaticWorkspaceBytes; looked up once per device.
hipError_t kvq_static_workspace(hipStream_t stream, void** addr);
hipError_t kvq_launch_extend(const ExtendArgs& a, hipStream_t s);
hipError_t kvq_launch_amax(const uint16_t* x0, int64_t n0, const uint16_t* x1, int64_t n1,
                           unsigned* scratch, float fmt_div, float* scale_out, hipStream_t s);
hipError_t kvq_launch_store(const kvq_cache* c, const uint16_t* k, const uint16_t* v,
                            const int64_t* slots, int32_t n, const float* k_scale,
                            const float* v_scale, hipStream_t s);
hipError_t kvq_launch_decode_gqa(const kvq_cache* c, const GqaDecodeArgs& a, hipStream_t s);
hipError_t kvq_launch_decode_mla(const kvq_cache* c, const MlaDecodeArgs& a, hipStream_t s);
hipError_t kvq_launch_combine(const CombineArgs& a, hipStream_t s);
hipError_t kvq_launch_dequant_prev(const kvq_cache* c, const int32_t* pages, int32_t n_pages, const float* g_scale,
                                   const float* ks_out, const float* vs_out, uint8_t* dq_k, uint8_t* dq_v,
                                   hipStream_t s);
hipError_t kvq_launch_amax_channels(const uint16_t* x0, int64_t rows0, const uint16_t* x1, int64_t rows1, int cols,
                                   unsigned* scratch, float fmt_div, float* scale_out, hipStream_t s);
hipError_t kvq_launch_amax_heads(const uint16_t* x0, int64_t rows0, const uint16_t* x1, int64_t rows1, int hkv,
                                 int dim, unsigned* scratch, float fmt_div, float* scale_out, hipStream_t s);
