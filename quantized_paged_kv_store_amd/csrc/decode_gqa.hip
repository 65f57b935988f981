// Paged GQA decode attention over a quantized KV cache, gfx950.
//
// The pages require dequantization to happen inside the attention kernel
// (SGLang "Quantized KV Cache" page, performance warning in the
// introduction); here it happens in registers, between the 16-byte HBM loads
// and the matrix-core operands, and nothing dequantized is ever written back.
//
// Work split: one workgroup (4 waves) per (sequence b, KV head, split of the
// context); each wave takes pairs of 16-token tiles round-robin and keeps its
// own online-softmax state; the 4 waves merge through LDS and write one
// partial (normalized output + log2-sum-exp) per split, merged by
// combine.hip (one split: the output is written directly). Merging inside
// this kernel (last workgroup of a sequence/head, atomic arrival counter)
// was measured slower: the device-scope release fence each workgroup needs
// writes back the L2.
//
// Per tile pair (32 tokens) a wave runs, with G <= 16 query heads as the MFMA
// N dimension (columns >= G hold zeros and are never written):
//   S^T[t][h]   = K^[t][:] . Q^T[:][h]      v_mfma_f32_16x16x32_bf16, 2*D/32 of them
//                 (K^ = code value; FP8 -> BF16 and E2M1*2^e -> BF16 are exact)
//   p = 2^(s*log2e*scale - m + 15)          online softmax in fp32, the 2^15
//                 keeps fp16 P far from its subnormal range
//   O^T[d][h]  += V^T[d][t] . P^T[t][h]     FP8: fp16 MFMA (E4M3/E5M2 exact in fp16)
//                                          FP4: bf16 MFMA, P split hi + lo (E2M1*2^e
//                                          is exact only in bf16)
// The QK accumulator layout (lane = head column, 4 tokens per lane) is
// exactly the PV B-operand layout once the 32 tokens of a pair are ordered
// [tile A: 4g..4g+3, tile B: 4g..4g+3] along K, so scores never leave the lane.
//
// KIVI-style FP8 caches (K scale per channel, V scale per token; the "KV cache
// quantization mechanism and traps" page, K and V distributions) fold the
// scales into the other operand instead of the codes: Q^T[d][h] * ks[d] once
// per workgroup (fp32, split into bf16 hi + lo, two QK MFMAs), and
// P[t][h] * vs[t] per tile (fp32, bf16 hi + lo for the PV MFMAs, V codes
// exact in bf16); the softmax sum keeps the unscaled P.
//
// FP8-domain attention (vLLM "Quantized KV Cache" page, overview: with an
// FP8 cache the attention itself runs in FP8, the query quantized like K and
// V; "Supported schemes": q_scale per tensor or per query head): each
// workgroup rounds its Q rows to E4M3 codes, RNE_sat(q / q_scale), once, and
// S^T = K . Q^T runs on v_mfma_f32_16x16x32_{fp8,bf8}_fp8 with the cached
// codes as the A operand exactly as loaded (no conversion at all); q_scale
// joins k_scale and sm_scale on the scores. The PV side is unchanged.
#include "store_row.h"

namespace kvq {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kPBias = 15.0f;  // p carries a factor 2^15
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kMaxSplitTiles = 1024;  // host keeps tiles_per_split <= this
// s_waitcnt operand: vector memory count 0, the other counters unconstrained
constexpr int kWaitVm0 = 0x0f70;

// raw per-lane bytes of one 16-token tile
template <int FMT, int D>
struct Tile {
  static constexpr int NK = (FMT == KVQ_FP4_MX16) ? 1 : D / 64;  // uint4 loads per lane for K and for V
  uint4 k[NK];
  uint4 v[NK];
  uint32_t ks;  // FP4: K E8M0 codes of blocks (2g, 2g+1) for token lane%16
  uint32_t vs;  // FP4: V E8M0 codes of tokens 4g..4g+3, block (lane%16)/2
  f32x4 vt;     // KIVI: V scales of tokens 4g..4g+3
};

template <int FMT, int D, bool KIVI = false>
__device__ __forceinline__ void load_tile(Tile<FMT, D>& t, const uint8_t* __restrict__ kb,
                                          const uint8_t* __restrict__ vb, const uint8_t* __restrict__ ksb,
                                          const uint8_t* __restrict__ vsb, int lane) {
  // every KV byte is read once per decode: nontemporal loads keep the stream
  // from evicting other lines (measured ~12% faster than plain loads)
#pragma unroll
  for (int i = 0; i < Tile<FMT, D>::NK; ++i) {
    t.k[i] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + 1024 * i + 16 * lane)));
    t.v[i] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vb + 1024 * i + 16 * lane)));
  }
  if (FMT == KVQ_FP4_MX16) {
    t.ks = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(ksb + 2 * lane));
    t.vs = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(vsb + 4 * (8 * (lane >> 4) + ((lane & 15) >> 1))));
  }
  if (KIVI) t.vt = *reinterpret_cast<const f32x4*>(vsb + 16 * (lane >> 4));  // the tile's 16 floats, 4 per group
}

template <int FMT, int D>
__device__ __forceinline__ void zero_tile(Tile<FMT, D>& t) {
#pragma unroll
  for (int i = 0; i < Tile<FMT, D>::NK; ++i) {
    t.k[i] = make_uint4(0, 0, 0, 0);
    t.v[i] = make_uint4(0, 0, 0, 0);
  }
  t.ks = 0x7f7fu;
  t.vs = 0x7f7f7f7fu;
  t.vt = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Zero the V codes (and neutralize scales) of this lane's tokens 4g+tt with
// tt >= nvalid, so that padding bytes (possibly NaN codes) cannot reach the
// PV product. tokens: nvalid in [0, 4].
template <int FMT, int D>
__device__ __forceinline__ void mask_tile_v(Tile<FMT, D>& t, int nvalid) {
  if (FMT == KVQ_FP4_MX16) {
    uint32_t w[4] = {t.v[0].x, t.v[0].y, t.v[0].z, t.v[0].w};
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
      if (tt >= nvalid) w[tt] = 0;
    t.v[0] = make_uint4(w[0], w[1], w[2], w[3]);
    const uint32_t keep = nvalid >= 4 ? 0xffffffffu : ((1u << (8 * nvalid)) - 1u);
    t.vs = (t.vs & keep) | (0x7f7f7f7fu & ~keep);
  } else {
    const uint32_t keep = nvalid >= 4 ? 0xffffffffu : ((1u << (8 * nvalid)) - 1u);
#pragma unroll
    for (int i = 0; i < Tile<FMT, D>::NK; ++i) {
      t.v[i].x &= keep;
      t.v[i].y &= keep;
      t.v[i].z &= keep;
      t.v[i].w &= keep;
    }
    // KIVI: padding slots may hold NaN scale bytes; P * vs must be 0 there
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i >= nvalid) t.vt[i] = 0.f;
  }
}

__device__ __forceinline__ uint32_t u4_get(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// S^T tile (16 tokens x 16 heads), lane holds tokens 4g..4g+3 of head lane%16.
// KIVI: qf holds the high and ql the low bf16 half of Q * ks.
template <int FMT, int D, bool KIVI = false>
__device__ __forceinline__ f32x4 qk_tile(const Tile<FMT, D>& t, const bf16x8* qf, const bf16x8* ql) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (FMT == KVQ_FP4_MX16) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t w = u4_get(t.k[0], c);
      const float sc = e8m0_to_f32((t.ks >> (8 * (c >> 1))) & 0xffu);
      u32x4 a = {fp4x2_to_bf16x2_scaled<0>(w, sc), fp4x2_to_bf16x2_scaled<1>(w, sc),
                 fp4x2_to_bf16x2_scaled<2>(w, sc), fp4x2_to_bf16x2_scaled<3>(w, sc)};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), qf[c], acc, 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      const uint4& kk = t.k[c >> 1];
      const uint32_t w0 = (c & 1) ? kk.z : kk.x;
      const uint32_t w1 = (c & 1) ? kk.w : kk.y;
      u32x4 a = {fp8x2_to_bf16x2<FMT, false>(w0), fp8x2_to_bf16x2<FMT, true>(w0),
                 fp8x2_to_bf16x2<FMT, false>(w1), fp8x2_to_bf16x2<FMT, true>(w1)};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), qf[c], acc, 0, 0, 0);
      if (KIVI) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), ql[c], acc, 0, 0, 0);
    }
  }
  return acc;
}

// FP8-domain S^T tile: the 8 codes a lane holds per 32-element step are the
// A operand as they are; q8[c] holds the E4M3 codes of the same 8 elements
// of head lane%16 (the MFMA sums over k, so any common order of the 8
// elements on both sides gives the same dot product).
template <int FMT, int D>
__device__ __forceinline__ f32x4 qk_tile_q8(const Tile<FMT, D>& t, const long* q8) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    const uint4& kk = t.k[c >> 1];
    const uint32_t w0 = (c & 1) ? kk.z : kk.x;
    const uint32_t w1 = (c & 1) ? kk.w : kk.y;
    const long a = (long)(((uint64_t)w1 << 32) | w0);
    if constexpr (FMT == KVQ_FP8_E4M3)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, q8[c], acc, 0, 0, 0);
    else
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf8_fp8(a, q8[c], acc, 0, 0, 0);
  }
  return acc;
}

// 8 floats -> bf16 hi (RNE) and lo = bf16(x - hi): 16 significant bits
__device__ __forceinline__ void split_bf16x8(const float* p, bf16x8& bh, bf16x8& bl) {
  float r[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const __bf16 h = (__bf16)p[i];
    r[i] = p[i] - (float)h;
  }
  const u32x4 phi = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                     pack_bf16x2(p[6], p[7])};
  const u32x4 plo = {pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]), pack_bf16x2(r[4], r[5]),
                     pack_bf16x2(r[6], r[7])};
  bh = __builtin_bit_cast(bf16x8, phi);
  bl = __builtin_bit_cast(bf16x8, plo);
}

// O^T += V^T P^T over the 32 tokens of a tile pair.
template <int FMT, int D, bool KIVI = false>
__device__ __forceinline__ void pv_pair(const Tile<FMT, D>& ta, const Tile<FMT, D>& tb, const float* p,
                                        f32x4* o) {
  if (KIVI) {
    float pv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pv[i] = p[i] * ta.vt[i];
      pv[4 + i] = p[4 + i] * tb.vt[i];
    }
    bf16x8 bh, bl;
    split_bf16x8(pv, bh, bl);
#pragma unroll
    for (int j = 0; j < D / 16; ++j) {
      const uint32_t wa = u4_get(ta.v[j >> 2], j & 3);
      const uint32_t wb = u4_get(tb.v[j >> 2], j & 3);
      u32x4 a = {fp8x2_to_bf16x2<FMT, false>(wa), fp8x2_to_bf16x2<FMT, true>(wa), fp8x2_to_bf16x2<FMT, false>(wb),
                 fp8x2_to_bf16x2<FMT, true>(wb)};
      const bf16x8 av = __builtin_bit_cast(bf16x8, a);
      o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bh, o[j], 0, 0, 0);
      o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bl, o[j], 0, 0, 0);
    }
  } else if (FMT == KVQ_FP4_MX16) {
    // P in bf16 as hi + lo (16 significant bits)
    u32x4 phi, plo;
    float r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const __bf16 h = (__bf16)p[i];
      r[i] = p[i] - (float)h;
    }
    phi = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
    plo = u32x4{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]), pack_bf16x2(r[4], r[5]), pack_bf16x2(r[6], r[7])};
    const bf16x8 bh = __builtin_bit_cast(bf16x8, phi);
    const bf16x8 bl = __builtin_bit_cast(bf16x8, plo);
    // X[page][tt][k]: token 4g+tt, elements d = 8c+2k (lo) and 8c+2k+1 (hi)
    uint32_t xa[4][4], xb[4][4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const uint32_t wa = u4_get(ta.v[0], tt), wb = u4_get(tb.v[0], tt);
      const float sa = e8m0_to_f32((ta.vs >> (8 * tt)) & 0xffu);
      const float sb = e8m0_to_f32((tb.vs >> (8 * tt)) & 0xffu);
      xa[tt][0] = fp4x2_to_bf16x2_scaled<0>(wa, sa);
      xa[tt][1] = fp4x2_to_bf16x2_scaled<1>(wa, sa);
      xa[tt][2] = fp4x2_to_bf16x2_scaled<2>(wa, sa);
      xa[tt][3] = fp4x2_to_bf16x2_scaled<3>(wa, sa);
      xb[tt][0] = fp4x2_to_bf16x2_scaled<0>(wb, sb);
      xb[tt][1] = fp4x2_to_bf16x2_scaled<1>(wb, sb);
      xb[tt][2] = fp4x2_to_bf16x2_scaled<2>(wb, sb);
      xb[tt][3] = fp4x2_to_bf16x2_scaled<3>(wb, sb);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      u32x4 lo = {lo_halves(xa[0][k], xa[1][k]), lo_halves(xa[2][k], xa[3][k]), lo_halves(xb[0][k], xb[1][k]),
                  lo_halves(xb[2][k], xb[3][k])};
      u32x4 hi = {hi_halves(xa[0][k], xa[1][k]), hi_halves(xa[2][k], xa[3][k]), hi_halves(xb[0][k], xb[1][k]),
                  hi_halves(xb[2][k], xb[3][k])};
      const bf16x8 al = __builtin_bit_cast(bf16x8, lo), ah = __builtin_bit_cast(bf16x8, hi);
      o[2 * k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, o[2 * k], 0, 0, 0);
      o[2 * k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bl, o[2 * k], 0, 0, 0);
      o[2 * k + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, o[2 * k + 1], 0, 0, 0);
      o[2 * k + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, o[2 * k + 1], 0, 0, 0);
    }
  } else {
    u32x4 pp = {pack_f16x2(p[0], p[1]), pack_f16x2(p[2], p[3]), pack_f16x2(p[4], p[5]), pack_f16x2(p[6], p[7])};
    const f16x8 pb = __builtin_bit_cast(f16x8, pp);
#pragma unroll
    for (int j = 0; j < D / 16; ++j) {
      const uint32_t wa = u4_get(ta.v[j >> 2], j & 3);
      const uint32_t wb = u4_get(tb.v[j >> 2], j & 3);
      u32x4 a = {fp8x2_to_f16x2<FMT, false>(wa), fp8x2_to_f16x2<FMT, true>(wa), fp8x2_to_f16x2<FMT, false>(wb),
                 fp8x2_to_f16x2<FMT, true>(wb)};
      o[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), pb, o[j], 0, 0, 0);
    }
  }
}

// element index d of accumulator (tile j, row r) for a lane in group g
template <int FMT>
__device__ __forceinline__ int out_dim(int j, int g, int r) {
  return (FMT == KVQ_FP4_MX16) ? 8 * (4 * g + r) + j : 16 * j + 4 * g + r;
}

template <int FMT, int D, bool KIVI, bool Q8 = false>
__global__ void __launch_bounds__(256, 2) decode_gqa_kernel(const GqaDecodeArgs a) {
  static_assert(!Q8 || (!KIVI && FMT != KVQ_FP4_MX16), "FP8-domain QK needs FP8 codes with tensor/head scales");
  constexpr int NJ = D / 16;                       // output accumulator tiles
  constexpr int NC = (FMT == KVQ_FP4_MX16) ? 4 : D / 32;  // QK MFMAs per tile
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, hc = lane & 15;
  const int t_begin = split * a.tiles_per_split;
  const int tpp = a.page_size / kTile;
  const int64_t tile_code_bytes = (FMT == KVQ_FP4_MX16) ? 8 * D : 16 * D;
  const int64_t tile_scale_bytes = (FMT == KVQ_FP4_MX16) ? D : (KIVI ? 4 * kTile : 0);
  const int64_t head_code = (int64_t)kvh * a.code_block_bytes;
  const int64_t head_scale = (int64_t)kvh * a.scale_block_bytes;
  const int64_t page_code = (int64_t)a.hkv * a.code_block_bytes;
  const int64_t page_scale = (int64_t)a.hkv * a.scale_block_bytes;
  const int32_t* pt = a.page_table + (int64_t)b * a.page_table_stride;

  // Tile pairs in flight per wave: two for FP8 at D = 128 (8 KB per wave in
  // flight), four for the smaller tiles of FP4-MX16 and FP8 at D = 64, which
  // otherwise leave too few bytes in flight to cover HBM latency. Loads are
  // issued unconditionally (a missing or out-of-pool tile reads an in-pool
  // stand-in and is masked afterwards), so the wait before each compute
  // covers exactly the loads issued earlier.
  constexpr int kDepth = (FMT == KVQ_FP4_MX16 || D == 64) ? 4 : 2;
  struct Pair {
    Tile<FMT, D> t[2];
    int ok;  // bit s: tile s holds real tokens
    int tA;
  };
  Pair R[kDepth];
  auto load_pair_tile = [&](Pair& P, int s2, int64_t pg, int64_t sub) {
    load_tile<FMT, D, KIVI>(P.t[s2], a.k_codes + pg * page_code + head_code + sub * tile_code_bytes,
                            a.v_codes + pg * page_code + head_code + sub * tile_code_bytes,
                            a.k_scales + pg * page_scale + head_scale + sub * tile_scale_bytes,
                            a.v_scales + pg * page_scale + head_scale + sub * tile_scale_bytes, lane);
  };
  // Each wave's first tile pair (pair `wave` of the split) is issued before
  // anything else: its page ids depend on the split alone, not on the
  // sequence length, so the loads start one memory round trip earlier.
  // Tiles past the sequence end are masked once the length is known.
  // The uniform values the prologue needs are read first, with the first
  // pair's page ids, as scalar loads that return together.
  const int seq_len = a.seq_lens[b];
  const int si = a.scale_mode == KVQ_SCALE_HEAD ? kvh : 0;  // per-tensor or per-KV-head FP8 scales
  const float kscale = (!KIVI && a.k_scale) ? a.k_scale[si] : 1.0f;
  const float vscale = (!KIVI && a.v_scale) ? a.v_scale[si] : 1.0f;
  int first_pg[2];
  {
    const int tA = t_begin + 2 * __builtin_amdgcn_readfirstlane(wave);
    // the last tile a page-table row covers (rows hold ceil(max_len / P) ids)
    const int t_last = max((a.max_len + kTile - 1) / kTile, 1) - 1;
    R[0].tA = tA;
    int tile[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      tile[s2] = min(tA + s2, t_last);
      first_pg[s2] = pt[tile[s2] / tpp];
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int64_t pg = (unsigned)first_pg[s2] < (unsigned)a.num_pages ? first_pg[s2] : 0;
      load_pair_tile(R[0], s2, pg, tile[s2] - (tile[s2] / tpp) * tpp);
    }
    // keeps the compiler from sinking these loads below the length check
    // (no wait: nothing reads them here)
    __asm__ volatile("" ::: "memory");
  }

  const int L = min(max(seq_len, 0), a.max_len);  // device data is clamped, never trusted
  const int ntiles = (L + kTile - 1) / kTile;
  const int t_end = min(t_begin + a.tiles_per_split, ntiles);
  if (t_begin >= t_end) {
    // an empty sequence has no split to merge: its first split writes 0 / -inf
    if (ntiles == 0 && split == 0) {
      for (int idx = tid; idx < a.group * D; idx += 256) {
        const int64_t hq = (int64_t)b * a.hq + (int64_t)kvh * a.group + idx / D;
        a.out[hq * D + idx % D] = 0.f;
        if (idx % D == 0 && a.lse) a.lse[hq] = kNegInf;
      }
    }
    return;  // nothing in this split; the merge only counts non-empty splits
  }

  const int G = a.group;
  // validity of the first pair's tiles, now that the length is known
  R[0].ok = 0;
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
    R[0].ok |= (int)(R[0].tA + s2 < t_end && (unsigned)first_pg[s2] < (unsigned)a.num_pages) << s2;

  float s_log2 = a.sm_scale_log2 * kscale;

  // Q^T operand fragments for head hc (zero beyond the group); KIVI: Q * ks
  // as bf16 hi (qf) + lo (ql); FP8 domain: E4M3 codes of Q / q_scale (q8)
  bf16x8 qf[Q8 ? 1 : NC], ql[KIVI ? NC : 1];
  long q8[Q8 ? NC : 1];
  {
    const bool hv = hc < G;
    const uint16_t* qrow = a.q + ((int64_t)b * a.hq + (int64_t)kvh * G + (hv ? hc : 0)) * D;
    float qs = 1.0f;
    if constexpr (Q8) {
      if (a.q_scale) qs = a.q_scale[a.scale_mode == KVQ_SCALE_HEAD ? kvh * G + (hv ? hc : 0) : 0];
      s_log2 *= qs;
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int d0 = (FMT == KVQ_FP4_MX16) ? 32 * g + 8 * c : 64 * (c >> 1) + 16 * g + 8 * (c & 1);
      uint4 w = *reinterpret_cast<const uint4*>(qrow + d0);
      if (!hv) w = make_uint4(0, 0, 0, 0);
      if constexpr (Q8) {
        // the same binary32 division and saturating RNE as the FP8 store
        const uint32_t lo = encode_fp8x4<KVQ_FP8_E4M3>(
            bf16_bits_to_f32(w.x & 0xffffu) / qs, bf16_bits_to_f32(w.x >> 16) / qs,
            bf16_bits_to_f32(w.y & 0xffffu) / qs, bf16_bits_to_f32(w.y >> 16) / qs);
        const uint32_t hi = encode_fp8x4<KVQ_FP8_E4M3>(
            bf16_bits_to_f32(w.z & 0xffffu) / qs, bf16_bits_to_f32(w.z >> 16) / qs,
            bf16_bits_to_f32(w.w & 0xffffu) / qs, bf16_bits_to_f32(w.w >> 16) / qs);
        q8[c] = (long)(((uint64_t)hi << 32) | lo);
      } else if constexpr (KIVI) {
        const float* ksr = a.k_scale + (int64_t)kvh * D + d0;
        const f32x4 s0 = *reinterpret_cast<const f32x4*>(ksr), s1 = *reinterpret_cast<const f32x4*>(ksr + 4);
        const uint32_t wq[4] = {w.x, w.y, w.z, w.w};
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[2 * i] = bf16_bits_to_f32(wq[i] & 0xffffu) * (i < 2 ? s0[2 * i] : s1[2 * i - 4]);
          x[2 * i + 1] = bf16_bits_to_f32(wq[i] >> 16) * (i < 2 ? s0[2 * i + 1] : s1[2 * i - 3]);
        }
        split_bf16x8(x, qf[c], ql[c]);
      } else {
        qf[c] = __builtin_bit_cast(bf16x8, w);
      }
    }
  }

  f32x4 o[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  const int npairs = (t_end - t_begin + 1) >> 1;

  // Append (kvq_decode_append): the split holding position L-1 quantizes the
  // new token's K/V rows and writes them into the cache before any of its
  // tile loads; the barrier below orders those stores before this
  // workgroup's reads of the tile (no other workgroup reads it). The token's
  // page id and rows are loaded ahead of the page-id staging, so the two
  // latencies overlap and the appending workgroup starts its tile loads
  // about when the others do.
  // FP8: wave 0's 64 lanes share the token, D / 32 elements of K (lanes
  // 0-31) or V (lanes 32-63) each; FP4 blocks need a whole 16-element chunk
  // per lane (lanes 0 .. D/16 - 1).
  constexpr bool kElems = FMT != KVQ_FP4_MX16;
  constexpr int kEpl = D / 32;
  const int pos = L - 1;
  const bool app_split = a.new_k != nullptr && pos / kTile < t_end && pos / kTile >= t_begin;
  const bool app = app_split && tid < (kElems ? 64 : D / 16);
  // the wave whose first pair (issued at the start) holds the appended tile
  const bool app_first = app_split && (pos / kTile - R[0].tA) >> 1 == 0;
  int app_page = -1;
  RowChunk nr;
  uint2 ne;
  float4 nks;  // KIVI: the K channel scales of this lane's elements
  if (app) {
    app_page = pt[pos / a.page_size];
    const int64_t row = ((int64_t)b * a.hkv + kvh) * D;
    if constexpr (kElems) {
      const uint16_t* src = (tid < 32 ? a.new_k : a.new_v) + row + kEpl * (tid & 31);
      if constexpr (kEpl == 4)
        ne = *reinterpret_cast<const uint2*>(src);
      else
        ne = make_uint2(*reinterpret_cast<const uint32_t*>(src), 0u);
      if constexpr (KIVI) {
        const float* ks = a.k_scale + (int64_t)kvh * D + kEpl * (tid & 31);
        if constexpr (kEpl == 4)
          nks = *reinterpret_cast<const float4*>(ks);
        else
          nks = make_float4(ks[0], ks[1], 1.0f, 1.0f);
      }
    } else {
      nr = load_row_chunk(a.new_k + row, a.new_v + row, tid);
    }
  }
  // page ids of this split, staged once in LDS
  __shared__ int sm_pg[kMaxSplitTiles];
  const int fp = t_begin / tpp;
  const int n_pg = (t_end - 1) / tpp - fp + 1;
  {
    // every thread's loads issued before any is waited on (a split has at
    // most kMaxSplitTiles pages: up to four per thread)
    int pg_in[kMaxSplitTiles / 256];
#pragma unroll
    for (int j = 0; j < kMaxSplitTiles / 256; ++j)
      if (tid + 256 * j < n_pg) pg_in[j] = pt[fp + tid + 256 * j];
#pragma unroll
    for (int j = 0; j < kMaxSplitTiles / 256; ++j)
      if (tid + 256 * j < n_pg) sm_pg[tid + 256 * j] = pg_in[j];
  }
  // every load above has arrived: otherwise a path that skips the append
  // joins with the rows still in flight, and the compiler then waits after
  // the barrier for all memory operations, the append's stores included
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  if (app && (unsigned)app_page < (unsigned)a.num_pages) {
    const int page = app_page;
    const int t = pos % a.page_size;
    uint8_t* kc = const_cast<uint8_t*>(a.k_codes);
    uint8_t* vc = const_cast<uint8_t*>(a.v_codes);
    if constexpr (FMT == KVQ_FP4_MX16) {
      const int64_t cbase = (int64_t)page * page_code + head_code + (int64_t)(t >> 4) * tile_code_bytes;
      const int64_t sbase = (int64_t)page * page_scale + head_scale + (int64_t)(t >> 4) * tile_scale_bytes;
      put_mx16_block(nr, tid, D / 16, t & 15, kc, vc, const_cast<uint8_t*>(a.k_scales),
                     const_cast<uint8_t*>(a.v_scales), cbase, sbase);
    } else if constexpr (KIVI) {
      // K: x / its channel scale; V: one scale for the row, fl32(amax / max)
      // (1.0 for an all-zero row), the maximum taken over lanes 32-63
      constexpr float MX = (FMT == KVQ_FP8_E4M3) ? 448.0f : 57344.0f;
      const int64_t base = (int64_t)page * page_code + head_code + (int64_t)(t >> 4) * tile_code_bytes;
      const bool is_v = tid >= 32;
      float x[4];
      unpack_elems<kEpl>(ne, x);
      float m = fmaxf(fmaxf(__builtin_fabsf(x[0]), __builtin_fabsf(x[1])),
                      fmaxf(__builtin_fabsf(x[2]), __builtin_fabsf(x[3])));
      for (int off = 1; off < 32; off <<= 1) m = fmaxf(m, shfl_xor_f32(m, off));  // within each half
      const float vs = m == 0.f ? 1.0f : m / MX;  // IEEE binary32 division
      uint32_t q;
      if (is_v) {
        const Divisor vd = make_divisor(vs);
        q = encode_fp8x4<FMT>(quotient(x[0], vd), quotient(x[1], vd), quotient(x[2], vd), quotient(x[3], vd));
      } else {
        q = encode_fp8x4<FMT>(x[0] / nks.x, x[1] / nks.y, x[2] / nks.z, x[3] / nks.w);
      }
      place_fp8_elems<kEpl>(q, is_v, kEpl * (tid & 31), t & 15, is_v ? vc : kc, base);
      if (tid == 32)
        reinterpret_cast<float*>(const_cast<uint8_t*>(a.v_scales) + (int64_t)page * page_scale + head_scale)[t] = vs;
    } else {
      const int64_t base = (int64_t)page * page_code + head_code + (int64_t)(t >> 4) * tile_code_bytes;
      const bool is_v = tid >= 32;
      put_fp8_elems<FMT, kEpl>(ne, is_v, kEpl * (tid & 31), t & 15, make_divisor(is_v ? vscale : kscale),
                               is_v ? vc : kc, base);
    }
  }
  __syncthreads();

  auto issue = [&](int pr, Pair& P) {
    const int tA = t_begin + 2 * pr;
    P.tA = tA;
    int ok = 0;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int tile = min(tA + s2, t_end - 1);
      const int page = __builtin_amdgcn_readfirstlane(sm_pg[tile / tpp - fp]);
      const bool v = (tA + s2 < t_end) && (unsigned)page < (unsigned)a.num_pages;
      ok |= (int)v << s2;
      load_pair_tile(P, s2, v ? page : 0, tile - (tile / tpp) * tpp);
    }
    P.ok = ok;
  };

  auto compute = [&](Pair& P) {
    const int tA = P.tA;
    float s[8];
    {
      f32x4 sa, sb;
      if constexpr (Q8) {
        sa = qk_tile_q8<FMT, D>(P.t[0], q8);
        sb = qk_tile_q8<FMT, D>(P.t[1], q8);
      } else {
        sa = qk_tile<FMT, D, KIVI>(P.t[0], qf, ql);
        sb = qk_tile<FMT, D, KIVI>(P.t[1], qf, ql);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[i] = sa[i] * s_log2;
        s[4 + i] = sb[i] * s_log2;
      }
    }
    // tokens past the sequence end, in a missing second tile or in a page
    // outside the pool are masked (scores -inf, V codes zeroed)
    if ((tA + 2) * kTile > L || P.ok != 3) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int tok0 = (tA + half) * kTile + 4 * g;
        const int nvalid = ((P.ok >> half) & 1) ? max(0, min(4, L - tok0)) : 0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i >= nvalid) s[4 * half + i] = kNegInf;
        mask_tile_v<FMT, D>(P.t[half], nvalid);
      }
    }
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, s[i]);
    mx = fmaxf(mx, shfl_xor_f32(mx, 16));
    mx = fmaxf(mx, shfl_xor_f32(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float mb = (m_new == kNegInf) ? 0.f : m_new - kPBias;
    const float alpha = (m_run == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
    float p[8], psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = __builtin_amdgcn_exp2f(s[i] - mb);
      psum += p[i];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int j = 0; j < NJ; ++j) o[j] *= alpha;
    pv_pair<FMT, D, KIVI>(P.t[0], P.t[1], p, o);
  };

  // Every slot of the unrolled body issues and computes unconditionally (so
  // every wait count is static); the wave's pair count is rounded up to whole
  // bodies. Pairs past the split are clamped in-pool stand-ins whose tokens
  // are all masked: they add exactly nothing to the softmax state.
  int pr = __builtin_amdgcn_readfirstlane(wave);
  if (pr < npairs) {
    const int iters = ((npairs - pr + kWaves - 1) / kWaves + kDepth - 1) / kDepth;
    // R[0] holds pair pr, issued at the start (again here if it holds the
    // appended token, whose stores the barrier above has ordered)
    if (app_first) issue(pr, R[0]);
#pragma unroll
    for (int i = 1; i < kDepth - 1; ++i) issue(pr + i * kWaves, R[i]);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int slot = 0; slot < kDepth; ++slot) {
        issue(pr + (kDepth - 1) * kWaves, R[(slot + kDepth - 1) % kDepth]);
        compute(R[slot]);
        pr += kWaves;
      }
    }
  }

  // ---- merge the 4 waves of this workgroup through LDS ----
  l_run += shfl_xor_f32(l_run, 16);
  l_run += shfl_xor_f32(l_run, 32);
  __shared__ float sm_o[kWaves][16][D + 1];
  __shared__ float sm_m[kWaves][16], sm_l[kWaves][16];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) sm_o[wave][hc][out_dim<FMT>(j, g, r)] = o[j][r];
  if (g == 0) {
    sm_m[wave][hc] = m_run;
    sm_l[wave][hc] = l_run;
  }
  __syncthreads();

  const bool direct = a.num_splits == 1;
  for (int idx = tid; idx < G * D; idx += 256) {
    const int h = idx / D, d = idx - h * D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][h]);
    float osum = 0.f, lsum = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = sm_m[w][h];
        if (mw != kNegInf) {
          const float f = __builtin_amdgcn_exp2f(mw - M);
          osum += f * sm_o[w][h][d];
          lsum += f * sm_l[w][h];
        }
      }
    }
    const float ov = lsum > 0.f ? (osum / lsum) * vscale : 0.f;
    const float lse2 = lsum > 0.f ? M + __log2f(lsum) - kPBias : kNegInf;
    const int64_t hq = (int64_t)b * a.hq + (int64_t)kvh * G + h;
    if (direct) {
      a.out[hq * D + d] = ov;
      if (d == 0 && a.lse) a.lse[hq] = lse2 * kLn2;
    } else {
      a.ws_o[(hq * a.num_splits + split) * D + d] = ov;
      if (d == 0) a.ws_lse[hq * a.num_splits + split] = lse2;
    }
  }
}

}  // namespace
}  // namespace kvq

using namespace kvq;

template <int FMT, int D>
void launch_fp8(const GqaDecodeArgs& a, dim3 grid, hipStream_t s) {
  if (a.scale_mode == KVQ_SCALE_KIVI)
    decode_gqa_kernel<FMT, D, true><<<grid, 256, 0, s>>>(a);
  else if (a.q8)
    decode_gqa_kernel<FMT, D, false, true><<<grid, 256, 0, s>>>(a);
  else
    decode_gqa_kernel<FMT, D, false><<<grid, 256, 0, s>>>(a);
}

hipError_t kvq_launch_decode_gqa(const kvq_cache* c, const GqaDecodeArgs& a, hipStream_t s) {
  const dim3 grid(a.num_splits, a.hkv, a.batch);
  const int dt = c->desc.dtype, D = c->desc.head_dim;
  if (dt == KVQ_FP8_E4M3 && D == 128)
    launch_fp8<KVQ_FP8_E4M3, 128>(a, grid, s);
  else if (dt == KVQ_FP8_E4M3 && D == 64)
    launch_fp8<KVQ_FP8_E4M3, 64>(a, grid, s);
  else if (dt == KVQ_FP8_E5M2 && D == 128)
    launch_fp8<KVQ_FP8_E5M2, 128>(a, grid, s);
  else if (dt == KVQ_FP8_E5M2 && D == 64)
    launch_fp8<KVQ_FP8_E5M2, 64>(a, grid, s);
  else if (dt == KVQ_FP4_MX16 && D == 128 && !a.q8)
    decode_gqa_kernel<KVQ_FP4_MX16, 128, false><<<grid, 256, 0, s>>>(a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}
