// Paged MLA decode attention over an NVFP4 latent cache, gfx950.
//
// DeepSeek-style multi-head latent attention in absorbed form: every query
// head attends to one shared latent row per token (Dk = 576 = 512 + 64
// rope dims); K^ = the whole row, V^ = its first 512 elements. Codes are
// E2M1 with one E4M3 scale per 16 elements and a global fp32 scale g (the
// two-level NVFP4 scaling of the SGLang PR #21954 analysis page); the
// dequantization happens inside this kernel (SGLang "Quantized KV Cache"
// page, performance warning), into LDS, never back to HBM.
//
// This is a dense contraction (the query heads share each latent element),
// so both products run on matrix cores in fp16, where E2M1 x E4M3 is exact:
//   S^T[t][h]  = K^[t][:] . Qs^T[:][h]      v_mfma_f32_32x32x16_f16
//                 Qs = Q * 2^s_h (a per-head power of two, so fp16 holds the
//                 BF16 query exactly; 2^-s_h goes into the score scale)
//   O^T[d][h] += V^T[d][t] . P^T[t][h]      v_mfma_f32_32x32x16_f16, P * 2^7
// and g is factored out of both (applied to the scores and to the output).
//
// Workgroup = 4 waves, one per SIMD, = all (1 to 128) query heads of one
// (sequence, context split); head columns past the head count carry a zero
// query and are not written. One wave per SIMD has 256 VGPRs and 256 AGPRs:
// wave w owns heads 32w..32w+31 outright, with their query in VGPRs (144)
// and their whole O^T (512 x 32 fp32) in the AGPRs, so its scores, softmax
// and PV need nothing from the other waves. A step covers 32 tokens (two
// 16-token tiles); the K^ tile has four LDS buffers, a step dequantized two
// steps before it is used; per step, wave w
//   1. scores its 32 heads against the 32 tokens over the full dot product
//      (36 MFMAs, the K^ operand read from the current buffer three
//      products ahead);
//   2. forms P (fp16) in the register layout of the PV B operand;
//   3. accumulates O^T for all 512 elements of its heads, the A operand
//      (V^T: one element, 8 tokens per lane) read straight from the
//      token-major K^ tile with ds_read_b64_tr_b16, gfx950's transposing LDS
//      read, so the latent is dequantized once per workgroup;
//   4. dequantizes its share of step st + 2 (elements [128w, 128w+128) and
//      a quarter of the rope group) into its buffer and issues the loads of
//      step st + 3;
// and the workgroup meets at a barrier after every second step.
//
// FP8-domain variant (kQ8: kvq_decode_fp8q and kvq_decode_append_fp8q on an
// MLA cache; vLLM "Quantized KV Cache" page, overview: with an FP8 cache the
// attention runs in FP8 and the query is quantized too). The query becomes
// E4M3 codes of Q / q_scale (one scale per tensor), rounded like the FP8
// store. NVFP4 values are not FP8 values, so the keys take the step the
// PR #21954 analysis page gives dequantize_prev_kv: E4M3 codes of K^ / (8g),
// i.e. each e2m1 * e4m3 product divided by 8 and rounded to nearest even
// (every such value lies within +-336, so none saturates):
//   S^T[t][h]  = K8[t][:] . Q8^T[:][h]     v_mfma_scale_f32_32x32x64_f8f6f4, unit scales
// with the score scale sm_scale * q_scale * 8g. The value side stays exact:
// V^ in fp16 and PV as above. The dequantization writes two token-major
// tiles per step, E4M3 keys (576 elements, 592-byte rows) and fp16 values
// (512 elements, 1,024-byte rows whose 16-byte chunks are XOR-swizzled by
// row, so the four rows a transposed read covers fall in different banks).
// Three such buffers fit the LDS: step st + 2 goes into the buffer step
// st - 1 read, and the workgroup meets at a barrier after every step.
#include <type_traits>

#include "store_row.h"

namespace kvq {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kPBias = 7.0f;   // P is stored as p * 2^7 in fp16
constexpr float kSlack = 8.0f;   // log2 headroom of the lazy reference maximum
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kDk = 576, kDv = 512;
constexpr int kWavesMla = 4;
constexpr int kHeadsPerWave = 32;
constexpr int kThreads = 64 * kWavesMla;
constexpr int kStepTiles = 2;                 // 32 tokens per step
constexpr int kStepTokens = kStepTiles * kTile;
constexpr int kKRow = kDk * 2 + 16;           // bytes per token row of the LDS K^ tile (padded)
constexpr int kBuf = kStepTokens * kKRow;     // one K^ buffer
constexpr int kTileCodes = 4608, kTileScales = 576;
// FP8-domain buffers: an E4M3 key tile and an fp16 value tile per step
constexpr int kK8Row = kDk + 16;                      // bytes per token row of the E4M3 key tile (padded)
constexpr int kVRow8 = kDv * 2;                       // bytes per token row of the fp16 value tile
constexpr int kBufK8 = kStepTokens * kK8Row;          // the key tile, first in the buffer
constexpr int kBuf8 = kBufK8 + kStepTokens * kVRow8;  // one FP8-domain buffer

typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(2))) short s16x2;
typedef __attribute__((ext_vector_type(8))) int i32x8;

__device__ __forceinline__ float f16_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); }
__device__ __forceinline__ float f16_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// transposed 4 x 16-bit LDS read (see the lane mapping where it is used)
__device__ __forceinline__ u32x2 lds_read_tr16(const uint8_t* p) {
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(u32x2, r);
}

// raw per-lane bytes of one 32-token step
struct Step {
  uint2 v[kStepTiles][2];      // [tile][j]: tokens 4g..4g+3, elements 4*col..+3 of 64-element group 2w+j
  uint32_t vs[kStepTiles][2];  // their E4M3 block scales, one byte per token
  uint32_t r[kStepTiles];      // rope codes of this thread's item (2 bytes) per tile
  uint32_t rs[kStepTiles];     // its rope scale byte per tile
  int ok;                      // bit s: tile s holds real tokens
  int tA;                      // first tile of the step
};

// buffer descriptor over one tile's bytes: loads past `bytes` return zero
constexpr int kRsrcWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, bytes, kRsrcWord3);
}

// fp16 values of 4 elements x 4 tokens from 8 code bytes and 4 scale bytes
// (one per token): x[tt] = {elements 0,1 | elements 2,3} of token tt
__device__ __forceinline__ void dequant16(const uint2 v, const uint32_t vs, uint2 (&x)[4]) {
  const f16x2 s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(vs, 1.0f, false);
  const f16x2 s23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(vs, 1.0f, true);
  const f16x2 sc[4] = {f16x2{s01[0], s01[0]}, f16x2{s01[1], s01[1]}, f16x2{s23[0], s23[0]}, f16x2{s23[1], s23[1]}};
  const uint32_t lo = v.x, hi = v.y;  // tokens 0,1 | 2,3
  const f16x2 c[8] = {__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(lo, 1.0f, 0), __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(lo, 1.0f, 1),
                      __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(lo, 1.0f, 2), __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(lo, 1.0f, 3),
                      __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(hi, 1.0f, 0), __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(hi, 1.0f, 1),
                      __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(hi, 1.0f, 2), __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(hi, 1.0f, 3)};
#pragma unroll
  for (int tt = 0; tt < 4; ++tt)
    x[tt] = make_uint2(__builtin_bit_cast(uint32_t, c[2 * tt] * sc[tt]), __builtin_bit_cast(uint32_t, c[2 * tt + 1] * sc[tt]));
}

// E4M3 codes of (4 fp16 values) / 8, rounded to nearest even (the scaled
// convert divides by the power of two it is given)
__device__ __forceinline__ uint32_t e4m3_over8(const uint2 x) {
  s16x2 o = {0, 0};
  o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(o, __builtin_bit_cast(f16x2, x.x), 8.0f, false);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(o, __builtin_bit_cast(f16x2, x.y), 8.0f, true);
  return __builtin_bit_cast(uint32_t, o);
}

// 16-byte chunk swizzle of row r of the fp16 value tile (FP8-domain variant):
// chunk c of the row is stored at chunk c ^ vswz(r)
__device__ __forceinline__ int vswz(int r) { return 4 * ((r & 3) ^ ((r >> 1) & 2)); }

// O *= alpha on accumulators that live in AGPRs, one element at a time
// through a VGPR (VALU cannot read AGPRs), so the rare rescale does not pull
// the whole accumulator set into VGPRs. The trailing s_nop covers the VALU
// write -> matrix-core read of the AGPRs by the next product.
__device__ __forceinline__ void scale_acc(f32x16& o, float alpha) {
  float x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = o[i];
  float t;
  asm volatile(
      "v_accvgpr_read_b32 %16, %0\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %0, %16\n\t"
      "v_accvgpr_read_b32 %16, %1\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %1, %16\n\t"
      "v_accvgpr_read_b32 %16, %2\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %2, %16\n\t"
      "v_accvgpr_read_b32 %16, %3\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %3, %16\n\t"
      "v_accvgpr_read_b32 %16, %4\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %4, %16\n\t"
      "v_accvgpr_read_b32 %16, %5\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %5, %16\n\t"
      "v_accvgpr_read_b32 %16, %6\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %6, %16\n\t"
      "v_accvgpr_read_b32 %16, %7\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %7, %16\n\t"
      "v_accvgpr_read_b32 %16, %8\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %8, %16\n\t"
      "v_accvgpr_read_b32 %16, %9\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %9, %16\n\t"
      "v_accvgpr_read_b32 %16, %10\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %10, %16\n\t"
      "v_accvgpr_read_b32 %16, %11\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %11, %16\n\t"
      "v_accvgpr_read_b32 %16, %12\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %12, %16\n\t"
      "v_accvgpr_read_b32 %16, %13\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %13, %16\n\t"
      "v_accvgpr_read_b32 %16, %14\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %14, %16\n\t"
      "v_accvgpr_read_b32 %16, %15\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %15, %16\n\t"
      "s_nop 4"
      : "+a"(x[0]), "+a"(x[1]), "+a"(x[2]), "+a"(x[3]), "+a"(x[4]), "+a"(x[5]), "+a"(x[6]), "+a"(x[7]),
        "+a"(x[8]), "+a"(x[9]), "+a"(x[10]), "+a"(x[11]), "+a"(x[12]), "+a"(x[13]), "+a"(x[14]), "+a"(x[15]),
        "=&v"(t)
      : "v"(alpha));
#pragma unroll
  for (int i = 0; i < 16; ++i) o[i] = x[i];
}

// kWholeSteps: every 32-token step lies inside one page (pages of a multiple
// of 32 tokens; splits are a whole number of steps), so a step needs one page
// lookup and one buffer descriptor; otherwise every tile is looked up.
// kQ8: the FP8-domain variant (E4M3 query and keys in the score products).
template <bool kWholeSteps, bool kQ8>
__global__ void __launch_bounds__(kThreads, 1) decode_mla_kernel(const MlaDecodeArgs a) {
  const int unit = blockIdx.x;
  if (unit >= a.batch * a.num_splits) return;
  const int b = unit / a.num_splits, split = unit - b * a.num_splits;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, col = lane & 15;   // dequant role: token group, element quad
  const int r32 = lane & 31, hh = lane >> 5;  // MFMA role: row / column, k half
  const int h0 = kHeadsPerWave * wave;        // this wave's first head
  // this lane's head column exists (waves past the head count only dequantize)
  const bool head_ok = h0 + r32 < a.hq;

  const int L = min(max(a.seq_lens[b], 0), a.max_len);
  const int ntiles = (L + kTile - 1) / kTile;
  const int t_begin = split * a.tiles_per_split;
  const int t_end = min(t_begin + a.tiles_per_split, ntiles);
  if (t_begin >= t_end) {
    if (ntiles == 0 && split == 0) {
      for (int idx = tid; idx < a.hq * kDv; idx += kThreads) {
        const int64_t hq = (int64_t)b * a.hq + idx / kDv;
        a.out[hq * kDv + idx % kDv] = 0.f;
        if (idx % kDv == 0 && a.lse) a.lse[hq] = kNegInf;
      }
    }
    return;
  }

  constexpr int kNBuf = kQ8 ? 3 : 4;                 // step buffers
  constexpr int kBufBytes = kQ8 ? kBuf8 : kBuf;
  __shared__ __attribute__((aligned(16))) uint8_t sm_k[kNBuf * kBufBytes];
  __shared__ int sm_pg[kMlaMaxSplitPages];

  const int tpp = a.page_size / kTile;
  const int fp = t_begin / tpp;
  const int n_pg = (t_end - 1) / tpp - fp + 1;
  const int32_t* pt = a.page_table + (int64_t)b * a.page_table_stride;
  for (int i = tid; i < n_pg; i += kThreads) sm_pg[i] = pt[fp + i];
  // Append (kvq_decode_append): the split holding position L-1 quantizes the
  // new latent row and writes it into the cache before any of its loads (the
  // barrier after the Q staging orders them).
  if (a.new_k != nullptr && (L - 1) / kTile < t_end && (L - 1) / kTile >= t_begin && tid < kDk / 16) {
    const int pos = L - 1;
    const int page = pt[pos / a.page_size];
    if ((unsigned)page < (unsigned)a.num_pages) {
      const int t = pos % a.page_size;
      uint8_t* cb = const_cast<uint8_t*>(a.codes) + (int64_t)page * a.page_size * (kDk / 2) + (int64_t)(t >> 4) * kTileCodes;
      uint8_t* sb = const_cast<uint8_t*>(a.scales) + (int64_t)page * a.page_size * (kDk / 16) + (int64_t)(t >> 4) * kTileScales;
      put_nvfp4_block(a.new_k + (int64_t)b * kDk, tid, t & 15, a.g_scale[0], cb, sb);
    }
  }

  // ---- Q of this wave's 32 heads, per-head power-of-two scaled ----
  // B operand of k step ks: head h0 + r32, elements 16*ks + 8*hh .. +7
  // (kQ8: E4M3 codes of Q / q_scale, elements 64*ks + 32*hh .. +31)
  f16x8 qf[kQ8 ? 1 : 36];
  i32x8 q8[kQ8 ? 9 : 1];
  float sscale = 0.f;
  if constexpr (kQ8) {
    const float qs = a.q_scale ? a.q_scale[0] : 1.0f;
    sscale = a.sm_scale_log2 * (qs * (8.0f * a.g_scale[0]));
    if (head_ok) {
      const uint16_t* qrow = a.q + ((int64_t)b * a.hq + h0 + r32) * kDk;
#pragma unroll
      for (int ks = 0; ks < 9; ++ks) {
        uint32_t w[8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint4 raw = *reinterpret_cast<const uint4*>(qrow + 64 * ks + 32 * hh + 8 * u);
          // the same binary32 division and saturating RNE as the FP8 store
          w[2 * u] = encode_fp8x4<KVQ_FP8_E4M3>(bf16_bits_to_f32(raw.x & 0xffffu) / qs, bf16_bits_to_f32(raw.x >> 16) / qs,
                                                bf16_bits_to_f32(raw.y & 0xffffu) / qs, bf16_bits_to_f32(raw.y >> 16) / qs);
          w[2 * u + 1] = encode_fp8x4<KVQ_FP8_E4M3>(bf16_bits_to_f32(raw.z & 0xffffu) / qs, bf16_bits_to_f32(raw.z >> 16) / qs,
                                                    bf16_bits_to_f32(raw.w & 0xffffu) / qs, bf16_bits_to_f32(raw.w >> 16) / qs);
        }
        q8[ks] = __builtin_bit_cast(i32x8, w);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 9; ++ks) q8[ks] = i32x8{};
    }
  } else if (head_ok) {
    const uint16_t* qrow = a.q + ((int64_t)b * a.hq + h0 + r32) * kDk;
    uint32_t mx = 0;
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) {
      const uint4 raw = *reinterpret_cast<const uint4*>(qrow + 16 * ks + 8 * hh);
      const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) mx = max(mx, max(w4[j] & 0x7fffu, (w4[j] >> 16) & 0x7fffu));
      qf[ks] = __builtin_bit_cast(f16x8, raw);
    }
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 32, 64));
    // power of two putting the head's largest |q| in [2^14, 2^15)
    const int e = mx ? (int)(mx >> 7) - 127 : 0;
    const int sh = max(-100, min(100, 14 - e));
    const float qmul = __builtin_ldexpf(1.0f, sh);
    sscale = a.sm_scale_log2 * a.g_scale[0] * __builtin_ldexpf(1.0f, -sh);
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) {
      const u32x4 w4 = __builtin_bit_cast(u32x4, qf[ks]);
      u32x4 h;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        h[j] = pack_f16x2(bf16_bits_to_f32(w4[j] & 0xffffu) * qmul, bf16_bits_to_f32(w4[j] >> 16) * qmul);
      qf[ks] = __builtin_bit_cast(f16x8, h);
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) qf[ks] = f16x8{};
  }
  __syncthreads();  // sm_pg; the append's stores before any load

  const int64_t page_codes = (int64_t)a.page_size * (kDk / 2);
  const int64_t page_scales = (int64_t)a.page_size * (kDk / 16);
  // rope item of this thread in every tile: token 4*r_g + r_tt, elements 512 + 4*r_i .. +3
  const int r_item = tid;
  const int r_g = r_item >> 6, r_i = (r_item >> 2) & 15, r_tt = r_item & 3;

  // tile cursor: page slot and tile within the page of the next tile to load
  // (advanced tile by tile, so no division sits in the step loop)
  int cur_tile = t_begin, cur_pg = 0, cur_sub = t_begin - fp * tpp;
  // loads of one step, issued ahead and unconditionally: a tile past the
  // split or on an out-of-pool page reads page 0 instead and is masked, so
  // every wait count stays static
  auto issue = [&](Step& S) {
    S.tA = cur_tile;
    int ok = 0;
    if constexpr (kWholeSteps) {
      const int slot = min(cur_pg, n_pg - 1);
      const int page = __builtin_amdgcn_readfirstlane(sm_pg[slot]);
      const bool pv = (unsigned)page < (unsigned)a.num_pages;
      const int64_t pg = pv ? page : 0;
      const int sub = pv ? cur_sub : 0;
      const auto rc = tile_rsrc(a.codes + pg * page_codes + (int64_t)sub * kTileCodes, kStepTiles * kTileCodes);
      const auto rs = tile_rsrc(a.scales + pg * page_scales + (int64_t)sub * kTileScales, kStepTiles * kTileScales);
#pragma unroll
      for (int s = 0; s < kStepTiles; ++s) {
        ok |= (int)(pv && cur_tile + s < t_end) << s;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int grp = 2 * wave + j;
          S.v[s][j] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rc, 8 * ((grp * 4 + g) * 16 + col), s * kTileCodes, 0));
          S.vs[s][j] = __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * ((grp * 4 + g) * 4 + (col >> 2)), s * kTileScales, 0);
        }
        S.r[s] = __builtin_amdgcn_raw_buffer_load_b16(rc, 4096 + 2 * r_item, s * kTileCodes, 0);
        S.rs[s] = __builtin_amdgcn_raw_buffer_load_b8(rs, 512 + 4 * (r_g * 4 + (r_i >> 2)) + r_tt, s * kTileScales, 0);
      }
      cur_tile += kStepTiles;
      cur_sub += kStepTiles;
      if (cur_sub == tpp) {
        cur_sub = 0;
        ++cur_pg;
      }
    } else {
#pragma unroll
      for (int s = 0; s < kStepTiles; ++s) {
        const int slot = min(cur_pg, n_pg - 1);
        const int page = __builtin_amdgcn_readfirstlane(sm_pg[slot]);
        const bool v = cur_tile < t_end && (unsigned)page < (unsigned)a.num_pages;
        ok |= (int)v << s;
        const int64_t pg = v ? page : 0;
        const int sub = v ? cur_sub : 0;
        const auto rc = tile_rsrc(a.codes + pg * page_codes + (int64_t)sub * kTileCodes, kTileCodes);
        const auto rs = tile_rsrc(a.scales + pg * page_scales + (int64_t)sub * kTileScales, kTileScales);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int grp = 2 * wave + j;
          S.v[s][j] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rc, 8 * ((grp * 4 + g) * 16 + col), 0, 0));
          S.vs[s][j] = __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * ((grp * 4 + g) * 4 + (col >> 2)), 0, 0);
        }
        S.r[s] = __builtin_amdgcn_raw_buffer_load_b16(rc, 4096 + 2 * r_item, 0, 0);
        S.rs[s] = __builtin_amdgcn_raw_buffer_load_b8(rs, 512 + 4 * (r_g * 4 + (r_i >> 2)) + r_tt, 0, 0);
        ++cur_tile;
        if (++cur_sub == tpp) {
          cur_sub = 0;
          ++cur_pg;
        }
      }
    }
    S.ok = ok;
  };

  // dequantize chunk c of the step held in S into K^ buffer `buf`: chunks
  // 0..3 are elements [64(2w + c%2), +64) of tile c/2's 16 tokens, chunks 4
  // and 5 this thread's rope item of tile c-4; tokens that are not real are
  // written as zeros
  auto dequant_chunk = [&](const Step& S, uint8_t* buf, const int c, auto tail_tag) {
    constexpr bool kTail = decltype(tail_tag)::value;
    const int tA = S.tA;
    if (c < 4) {
      const int s = c >> 1, j = c & 1;
      const int nvalid = kTail ? (((S.ok >> s) & 1) ? max(0, min(4, L - (tA + s) * kTile - 4 * g)) : 0) : 4;
      uint2 x[4];
      dequant16(S.v[s][j], S.vs[s][j], x);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        if (kTail && tt >= nvalid) x[tt] = make_uint2(0u, 0u);
        const int row = 16 * s + 4 * g + tt;
        if constexpr (kQ8) {
          const int ch = (8 * (2 * wave + j) + (col >> 1)) ^ vswz(row);
          *reinterpret_cast<uint2*>(buf + kBufK8 + row * kVRow8 + 16 * ch + 8 * (col & 1)) = x[tt];
          *reinterpret_cast<uint32_t*>(buf + row * kK8Row + 64 * (2 * wave + j) + 4 * col) = e4m3_over8(x[tt]);
        } else {
          *reinterpret_cast<uint2*>(buf + row * kKRow + 2 * (64 * (2 * wave + j) + 4 * col)) = x[tt];
        }
      }
    } else {
      const int s = c - 4;
      const f16x2 rsc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(S.rs[s], 1.0f, false);
      const f16x2 rs2 = {rsc[0], rsc[0]};
      uint32_t r0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(S.r[s], 1.0f, 0) * rs2);
      uint32_t r1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(S.r[s], 1.0f, 1) * rs2);
      if (kTail) {
        const int tok = (tA + s) * kTile + 4 * r_g + r_tt;
        if (!((S.ok >> s) & 1) || tok >= L) r0 = r1 = 0u;
      }
      const int row = 16 * s + 4 * r_g + r_tt;
      if constexpr (kQ8)  // the rope elements are keys only
        *reinterpret_cast<uint32_t*>(buf + row * kK8Row + kDv + 4 * r_i) = e4m3_over8(make_uint2(r0, r1));
      else
        *reinterpret_cast<uint2*>(buf + row * kKRow + 2 * (512 + 4 * r_i)) = make_uint2(r0, r1);
    }
  };
  auto is_tail = [&](int tA, int ok) { return (tA + kStepTiles) * kTile > L || ok != (1 << kStepTiles) - 1; };

  f32x16 o[16];  // O^T accumulators: elements 32*db .. +31 x this wave's 32 heads
#pragma unroll
  for (int db = 0; db < 16; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  // head h0 + r32: reference maximum, sums over this lane's P values of the
  // fp16 weights (normalize the output) and of the unrounded weights (LSE)
  float m_run = kNegInf, l_run = 0.f, e_run = 0.f;

  // V^T reads (ds_read_b64_tr_b16): in each 16-lane group, lane i receives
  // element i%4 of the 8-byte reads addressed by lanes i/4 + 4e (e = 0..3);
  // lane 4e + c therefore addresses token row e, elements D + 4c, and lane i
  // gets element D + i of rows 0..3.
  const int tr_e = col >> 2, tr_c = col & 3;
  const int v_off = (4 * hh + tr_e) * kKRow + 2 * (16 * ((lane >> 4) & 1) + 4 * tr_c);
  // kQ8: the same reads from the swizzled value tile. This lane's rows
  // 16m + 4hh + tr_e (+8) all have swizzle 4 * e8, so the chunk 4db + x it
  // reads sits at 4(db ^ e8) + x; v_off8[r] serves the blocks db with db % 4 = r.
  const int e8 = tr_e ^ (2 * hh);
  int v_off8[kQ8 ? 4 : 1] = {};
  if constexpr (kQ8)
#pragma unroll
  for (int r = 0; r < 4; ++r)
    v_off8[r] = kBufK8 + (4 * hh + tr_e) * kVRow8 + 64 * (r ^ e8) + 16 * (2 * ((lane >> 4) & 1) + (tr_c >> 1)) +
                8 * (tr_c & 1);

  // One step of loads is in flight while the previous step is scored and
  // accumulated: the raw registers are refilled right after they have been
  // dequantized into LDS. The loads past the split read in-pool stand-ins
  // that are dequantized as zeros and never read, which keeps every wait
  // static.
  const int nsteps = (t_end - t_begin + kStepTiles - 1) / kStepTiles;
  Step R;
  auto dequant_all = [&](uint8_t* buf) {
    auto all_chunks = [&](auto tail_tag) {
#pragma unroll
      for (int c = 0; c < 6; ++c) dequant_chunk(R, buf, c, tail_tag);
    };
    if (is_tail(R.tA, R.ok))
      all_chunks(std::true_type{});
    else
      all_chunks(std::false_type{});
  };
  // steps 0 and 1 into buffers 0 and 1; step 2's loads in flight
  issue(R);
  int tA_c = R.tA, ok_c = R.ok;
  dequant_all(sm_k);
  issue(R);
  int tA_1 = R.tA, ok_1 = R.ok;
  dequant_all(sm_k + kBufBytes);
  issue(R);
  __syncthreads();
  int bc = 0;  // kQ8: buffer of the current step (st % 3)

  // Step st is read from buffer st % 4 while step st + 2 is dequantized into
  // buffer (st + 2) % 4 (last read by step st - 2, which every wave finished
  // before the last barrier); the workgroup meets after every odd step.
  // kQ8: buffers st % 3 and (st + 2) % 3 (last read by step st - 1), and a
  // barrier after every step.
  for (int st = 0; st < nsteps; ++st) {
    const int bn = kQ8 ? (bc == 0 ? 2 : bc - 1) : ((st + 2) & 3);
    const uint8_t* kb = sm_k + (kQ8 ? bc : (st & 3)) * kBufBytes;
    uint8_t* nb = sm_k + bn * kBufBytes;

    // 1. S^T[token i][head h0 + r32] over all 576 elements from buffer kb,
    //    the K^ operand read three products ahead. Every product (here and
    //    in PV) is fenced from the scheduler: left free, it hoists all 36
    //    operand reads ahead of the chain and the wave runs out of VGPRs.
    f32x16 sc0;
    if constexpr (kQ8) {
      // 9 products of 64 elements: lane (r32, hh) supplies token r32's codes
      // 64*ks + 32*hh .. +31, the same elements as its query operand
#pragma unroll
      for (int i = 0; i < 16; ++i) sc0[i] = 0.f;
      const uint8_t* krow = kb + r32 * kK8Row + 32 * hh;
      auto kread = [&](int ks) {
        const u32x4 lo = *reinterpret_cast<const u32x4*>(krow + 64 * ks);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(krow + 64 * ks + 16);
        return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      };
      constexpr int kDepth = 3;
      i32x8 ka[kDepth];
#pragma unroll
      for (int ks = 0; ks < kDepth - 1; ++ks) ka[ks] = kread(ks);
#pragma unroll
      for (int ks = 0; ks < 9; ++ks) {
        if (ks + kDepth - 1 < 9) ka[(ks + kDepth - 1) % kDepth] = kread(ks + kDepth - 1);
        sc0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka[ks % kDepth], q8[ks], sc0, 0, 0, 0, 127, 0, 127);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) sc0[i] = 0.f;
      const uint8_t* krow = kb + r32 * kKRow + 16 * hh;
      constexpr int kDepth = 4;
      f16x8 ka[kDepth];
#pragma unroll
      for (int ks = 0; ks < kDepth - 1; ++ks) ka[ks] = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(krow + 32 * ks));
#pragma unroll
      for (int ks = 0; ks < 36; ++ks) {
        if (ks + kDepth - 1 < 36)
          ka[(ks + kDepth - 1) % kDepth] =
              __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(krow + 32 * (ks + kDepth - 1)));
        sc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[ks % kDepth], qf[ks], sc0, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // 2. value v of the scores is token 8(v/4) + 4hh + v%4 of the step
    float s[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) s[v] = sc0[v];
    if (__builtin_expect(is_tail(tA_c, ok_c), 0)) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int tl = 8 * (v >> 2) + 4 * hh + (v & 3);
        if (!((ok_c >> (tl >> 4)) & 1) || tA_c * kTile + tl >= L) s[v] = kNegInf;
      }
    }
    float mx = s[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) mx = fmaxf(mx, s[v]);
    mx = fmaxf(mx, shfl_xor_f32(mx, 32)) * sscale;
    // the reference maximum only moves when a score exceeds it by more than
    // 2^kSlack, so the rescale of the accumulators below is rare; P then
    // stays <= 2^(kSlack + kPBias) = 2^15 in fp16. Both lanes of a head see
    // the same maxima and take the same decisions.
    const bool move = mx > m_run + kSlack;
    const float m_new = move ? mx : m_run;
    const float mb2 = (m_new == kNegInf) ? 0.f : m_new - kPBias;
    const float alpha = move ? ((m_run == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new)) : 1.0f;
    // B operand of PV k step m: values 8m .. 8m+7 = tokens 16m + 8(u/4) + 4hh + u%4
    f16x8 pb[2];
    {
      float p[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) p[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[v], sscale, -mb2));
      uint32_t pk[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) pk[i] = pack_f16x2(p[2 * i], p[2 * i + 1]);
      // the normalizer sums the fp16-rounded weights the PV products use, so
      // the output stays an exact weighted average of V whatever the rounding
      float ls = 0.f, es = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ls += f16_lo(pk[i]) + f16_hi(pk[i]);
        es += p[2 * i] + p[2 * i + 1];
      }
      l_run = l_run * alpha + ls;
      e_run = e_run * alpha + es;
      m_run = m_new;
      pb[0] = __builtin_bit_cast(f16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
      pb[1] = __builtin_bit_cast(f16x8, u32x4{pk[4], pk[5], pk[6], pk[7]});
    }
    if (__any(alpha != 1.0f)) {  // the reference maxima rarely move after the first steps
#pragma unroll
      for (int db = 0; db < 16; ++db) scale_acc(o[db], alpha);
    }

    // 3. O^T[d][h] += V^T[d][t] P^T[t][h]: d = 32db + row, heads h0 + r32
    {
      constexpr int kVDepth = 3;  // V^T fragments read ahead of their products
      auto vread = [&](int j) {
        const int m = j >> 4, db = j & 15;
        constexpr int kRow = kQ8 ? kVRow8 : kKRow;
        const uint8_t* vp = kQ8 ? kb + v_off8[db & 3] + (16 * m) * kRow + 256 * (db >> 2)
                                : kb + v_off + (16 * m) * kRow + 64 * db;
        const u32x2 lo = lds_read_tr16(vp);              // tokens +0..3
        const u32x2 hi = lds_read_tr16(vp + 8 * kRow);   // tokens +8..11
        return __builtin_bit_cast(f16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
      };
      f16x8 va[kVDepth];
#pragma unroll
      for (int j = 0; j < kVDepth - 1; ++j) va[j] = vread(j);
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        if (j + kVDepth - 1 < 32) va[(j + kVDepth - 1) % kVDepth] = vread(j + kVDepth - 1);
        o[j & 15] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[j % kVDepth], pb[j >> 4], o[j & 15], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // 4. step st + 2 into buffer nb, then the loads of step st + 3
    const int tA_2 = R.tA, ok_2 = R.ok;
    dequant_all(nb);
    issue(R);
    if (kQ8 || (st & 1)) __syncthreads();  // uniform: every wave runs the same steps
    bc = kQ8 ? (bc == 2 ? 0 : bc + 1) : 0;
    tA_c = tA_1;
    ok_c = ok_1;
    tA_1 = tA_2;
    ok_1 = ok_2;
  }

  // ---- epilogue: normalize and write this split's partial (or the output) ----
  l_run += shfl_xor_f32(l_run, 32);
  e_run += shfl_xor_f32(e_run, 32);
  if (!head_ok) return;
  const bool direct = a.num_splits == 1;
  const float inv = l_run > 0.f ? a.g_scale[0] / l_run : 0.f;
  const int64_t hq = (int64_t)b * a.hq + h0 + r32;
  float* dst = direct ? a.out + hq * kDv : a.ws_o + (hq * a.num_splits + split) * kDv;
  // value v of accumulator db: element 32db + 8(v/4) + 4hh + v%4
#pragma unroll
  for (int db = 0; db < 16; ++db)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v4 = make_float4(o[db][4 * q] * inv, o[db][4 * q + 1] * inv, o[db][4 * q + 2] * inv,
                                    o[db][4 * q + 3] * inv);
      *reinterpret_cast<float4*>(dst + 32 * db + 8 * q + 4 * hh) = v4;
    }
  if (hh == 0) {
    const float lse2 = e_run > 0.f ? m_run + __log2f(e_run) - kPBias : kNegInf;
    if (direct) {
      if (a.lse) a.lse[hq] = lse2 * kLn2;
    } else {
      a.ws_lse[hq * a.num_splits + split] = lse2;
    }
  }
}

}  // namespace
}  // namespace kvq

hipError_t kvq_launch_decode_mla(const kvq_cache* c, const MlaDecodeArgs& a, hipStream_t s) {
  (void)c;
  const int blocks = a.batch * a.num_splits;
  const int tpp = a.page_size / kvq::kTile;
  const bool whole = tpp % kvq::kStepTiles == 0 && a.tiles_per_split % kvq::kStepTiles == 0;
  if (a.q8) {
    if (whole)
      kvq::decode_mla_kernel<true, true><<<blocks, kvq::kThreads, 0, s>>>(a);
    else
      kvq::decode_mla_kernel<false, true><<<blocks, kvq::kThreads, 0, s>>>(a);
  } else if (whole) {
    kvq::decode_mla_kernel<true, false><<<blocks, kvq::kThreads, 0, s>>>(a);
  } else {
    kvq::decode_mla_kernel<false, false><<<blocks, kvq::kThreads, 0, s>>>(a);
  }
  return hipGetLastError();
}
