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
// The 32x32x16 shape sustains close to the matrix-core peak on gfx950 and
// its operand pattern (32 rows x 16 B) reads LDS without bank conflicts.
//
// Workgroup = 8 waves, two per SIMD (one wave's LDS and matrix latencies
// are covered by the other's work), = 64 query heads of one (sequence,
// context split); the two 64-head groups of a split get block ids 8 apart,
// i.e. the same XCD, so the second reads the latent tiles from that L2. A
// step covers 64 tokens (four 16-token tiles); wave w:
//   1. dequantizes elements [64w, 64w+64) and an eighth of the rope group of
//      the 64 tokens into the LDS K^ tile (token-major, fp16);
//   2. scores heads 32(w&1)..+31 against tokens 32(w>>2)..+31 over half of
//      the dot product (elements [288((w>>1)&1), +288)); Q of those heads and
//      elements stays in registers (72 registers). The two waves splitting a
//      dot product add each other's partial scores through LDS; the two
//      token halves exchange their block maxima;
//   3. turns half of its (now complete) scores into P (fp16), written in the
//      exact register layout of the PV B operand, so the PV waves read it
//      back with conflict-free 16 B reads;
//   4. accumulates O^T for elements [64w, 64w+64) and all 64 heads. Its A
//      operand (V^T: one element, 8 tokens per lane) is read straight from
//      the token-major K^ tile with ds_read_b64_tr_b16, gfx950's transposing
//      LDS read, so the latent is dequantized once.
#include <type_traits>

#include "store_row.h"

namespace kvq {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kPBias = 7.0f;   // P is stored as p * 2^7 in fp16
constexpr float kSlack = 8.0f;   // log2 headroom of the lazy reference maximum
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kDk = 576, kDv = 512;
constexpr int kHeadsPerWG = 64;
constexpr int kWavesMla = 8;
constexpr int kThreads = 64 * kWavesMla;
constexpr int kStepTiles = 4;                 // 64 tokens per step
constexpr int kStepTokens = kStepTiles * kTile;
constexpr int kKRow = kDk * 2 + 16;           // bytes per token row of the LDS K^ tile (padded)
constexpr int kTileCodes = 4608, kTileScales = 576;

typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) short s16x4;

__device__ __forceinline__ float f16_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); }
__device__ __forceinline__ float f16_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// transposed 4 x 16-bit LDS read (see the lane mapping where it is used)
__device__ __forceinline__ u32x2 lds_read_tr16(const uint8_t* p) {
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(u32x2, r);
}

// raw per-lane bytes of one 64-token step
struct Step {
  uint2 v[kStepTiles];      // [tile]: tokens 4g..4g+3, elements 4*col..+3 of this wave's group
  uint32_t vs[kStepTiles];  // their E4M3 block scales, one byte per token
  uint32_t r[2];            // rope codes of this lane's item (2 bytes) in two of the tiles
  uint32_t rs[2];           // rope scale byte per such tile
  int ok;                   // bit s: tile s holds real tokens
  int tA;                   // first tile of the step
};

// buffer descriptor over one tile's bytes: loads past `bytes` return zero
constexpr int kRsrcWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, bytes, kRsrcWord3);
}

// fp16 values of elements 4*col .. 4*col+3 of the wave's group, tokens 4g + tt
// (tt = 0..3) of tile s: x[tt] = {elements 0,1 | elements 2,3}
__device__ __forceinline__ void dequant16(const Step& S, int s, uint2 (&x)[4]) {
  const f16x2 s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(S.vs[s], 1.0f, false);
  const f16x2 s23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(S.vs[s], 1.0f, true);
  const f16x2 sc[4] = {f16x2{s01[0], s01[0]}, f16x2{s01[1], s01[1]}, f16x2{s23[0], s23[0]}, f16x2{s23[1], s23[1]}};
  const uint32_t lo = S.v[s].x, hi = S.v[s].y;  // tokens 0,1 | 2,3
  const f16x2 c[8] = {__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(lo, 1.0f, 0), __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(lo, 1.0f, 1),
                      __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(lo, 1.0f, 2), __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(lo, 1.0f, 3),
                      __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(hi, 1.0f, 0), __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(hi, 1.0f, 1),
                      __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(hi, 1.0f, 2), __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(hi, 1.0f, 3)};
#pragma unroll
  for (int tt = 0; tt < 4; ++tt)
    x[tt] = make_uint2(__builtin_bit_cast(uint32_t, c[2 * tt] * sc[tt]), __builtin_bit_cast(uint32_t, c[2 * tt + 1] * sc[tt]));
}

// kWholeSteps: every 64-token step lies inside one page (pages of a multiple
// of 64 tokens, splits of a multiple of 4 tiles), so a step needs one page
// lookup and one buffer descriptor; otherwise every tile is looked up.
template <bool kWholeSteps>
__global__ void __launch_bounds__(kThreads, 1) decode_mla_kernel(const MlaDecodeArgs a) {
  // ---- block -> (sequence, split, head group); both head groups of a split share an XCD ----
  const int n_units = a.batch * a.num_splits;
  const int id = blockIdx.x;
  const int unit = (id >> 4) * 8 + (id & 7);
  const int hg = (id >> 3) & 1;
  if (unit >= n_units || hg * kHeadsPerWG >= a.hq) return;
  const int b = unit / a.num_splits, split = unit - b * a.num_splits;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, col = lane & 15;   // dequant role: token group, element quad
  const int r32 = lane & 31, hh = lane >> 5;  // MFMA role: row / column, k half
  // score role: 32-head block, half of the dot product, 32-token block
  const int hgp = wave & 1, kh = (wave >> 1) & 1, tb = wave >> 2;

  const int L = min(max(a.seq_lens[b], 0), a.max_len);
  const int ntiles = (L + kTile - 1) / kTile;
  const int t_begin = split * a.tiles_per_split;
  const int t_end = min(t_begin + a.tiles_per_split, ntiles);
  const int h0 = hg * kHeadsPerWG;
  if (t_begin >= t_end) {
    if (ntiles == 0 && split == 0) {
      for (int idx = tid; idx < kHeadsPerWG * kDv; idx += kThreads) {
        const int64_t hq = (int64_t)b * a.hq + h0 + idx / kDv;
        a.out[hq * kDv + idx % kDv] = 0.f;
        if (idx % kDv == 0 && a.lse) a.lse[hq] = kNegInf;
      }
    }
    return;
  }

  __shared__ __attribute__((aligned(16))) uint8_t sm_k[kStepTokens * kKRow];
  __shared__ __attribute__((aligned(16))) uint8_t sm_p[4 * 2 * 64 * 16];           // [k step][head block][lane][8 x fp16]
  __shared__ __attribute__((aligned(16))) float sm_s[kWavesMla * 2 * 64 * 4];     // partial scores [wave][quad][lane][4]
  __shared__ float sm_mx[2][2][kHeadsPerWG];                                       // [token half][k half][head]
  __shared__ float sm_alpha[kHeadsPerWG];
  __shared__ float sm_l[4][kHeadsPerWG];
  __shared__ float sm_e[4][kHeadsPerWG];
  __shared__ float sm_m[kHeadsPerWG];
  __shared__ int sm_pg[kMlaMaxSplitPages];

  const int tpp = a.page_size / kTile;
  const int fp = t_begin / tpp;
  const int n_pg = (t_end - 1) / tpp - fp + 1;
  const int32_t* pt = a.page_table + (int64_t)b * a.page_table_stride;
  for (int i = tid; i < n_pg; i += kThreads) sm_pg[i] = pt[fp + i];
  // Append (kvq_decode_append): the split holding position L-1 quantizes the
  // new latent row and writes it into the cache before any of its loads (the
  // barrier after the Q staging orders them). Both head-group workgroups of
  // the split read that tile, so both write the same bytes.
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

  // ---- Q of this wave's 32 heads and half of the elements, per-head power-of-two scaled ----
  // B operand of step ks: head 32*hgp + r32, elements 288*kh + 16*ks + 8*hh .. +7
  f16x8 qf[18];
  float sscale;
  {
    const int head = h0 + 32 * hgp + r32;
    const uint16_t* qrow = a.q + ((int64_t)b * a.hq + head) * kDk;
    uint32_t mx = 0;
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) {
      // the per-head maximum needs the whole row; only this wave's half is kept
      const uint4 raw = *reinterpret_cast<const uint4*>(qrow + 16 * ks + 8 * hh);
      const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) mx = max(mx, max(w4[j] & 0x7fffu, (w4[j] >> 16) & 0x7fffu));
      if (ks / 18 == kh) qf[ks % 18] = __builtin_bit_cast(f16x8, raw);
    }
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 32, 64));
    // power of two putting the head's largest |q| in [2^14, 2^15)
    const int e = mx ? (int)(mx >> 7) - 127 : 0;
    const int sh = max(-100, min(100, 14 - e));
    const float qmul = __builtin_ldexpf(1.0f, sh);
    sscale = a.sm_scale_log2 * a.g_scale[0] * __builtin_ldexpf(1.0f, -sh);
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      const u32x4 w4 = __builtin_bit_cast(u32x4, qf[ks]);
      u32x4 h;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        h[j] = pack_f16x2(bf16_bits_to_f32(w4[j] & 0xffffu) * qmul, bf16_bits_to_f32(w4[j] >> 16) * qmul);
      qf[ks] = __builtin_bit_cast(f16x8, h);
    }
  }
  __syncthreads();  // sm_pg

  const int64_t page_codes = (int64_t)a.page_size * (kDk / 2);
  const int64_t page_scales = (int64_t)a.page_size * (kDk / 16);
  // rope item of this lane in tiles 2tb, 2tb+1: token 4*r_g + r_tt, elements 512 + 4*r_i .. +3
  const int r_item = tid & 255;
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
        S.v[s] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rc, 8 * ((wave * 4 + g) * 16 + col), s * kTileCodes, 0));
        S.vs[s] = __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * ((wave * 4 + g) * 4 + (col >> 2)), s * kTileScales, 0);
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int s = 2 * tb + s2;
        S.r[s2] = __builtin_amdgcn_raw_buffer_load_b16(rc, 4096 + 2 * r_item, s * kTileCodes, 0);
        S.rs[s2] = __builtin_amdgcn_raw_buffer_load_b8(rs, 512 + 4 * (r_g * 4 + (r_i >> 2)) + r_tt, s * kTileScales, 0);
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
        S.v[s] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rc, 8 * ((wave * 4 + g) * 16 + col), 0, 0));
        S.vs[s] = __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * ((wave * 4 + g) * 4 + (col >> 2)), 0, 0);
        if ((s >> 1) == tb) {  // uniform per wave
          S.r[s & 1] = __builtin_amdgcn_raw_buffer_load_b16(rc, 4096 + 2 * r_item, 0, 0);
          S.rs[s & 1] = __builtin_amdgcn_raw_buffer_load_b8(rs, 512 + 4 * (r_g * 4 + (r_i >> 2)) + r_tt, 0, 0);
        }
        ++cur_tile;
        if (++cur_sub == tpp) {
          cur_sub = 0;
          ++cur_pg;
        }
      }
    }
    S.ok = ok;
  };

  f32x16 o[2][2];  // O^T accumulators [32-element block db][32-head block hb]
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][hb][i] = 0.f;
  // head 32*hgp + r32: reference maximum, sums over this wave's P values of
  // the fp16 weights (normalize the output) and of the unrounded weights
  // (for the LSE)
  float m_run = kNegInf, l_run = 0.f, e_run = 0.f;

  // 1. dequantize elements [64w, 64w+64) and an eighth of the rope group into the LDS K^ tile
  auto dequant = [&](const Step& S, auto tail_tag) {
    constexpr bool kTail = decltype(tail_tag)::value;
    const int tA = S.tA;
#pragma unroll
    for (int s = 0; s < kStepTiles; ++s) {
      const int nvalid = kTail ? (((S.ok >> s) & 1) ? max(0, min(4, L - (tA + s) * kTile - 4 * g)) : 0) : 4;
      uint2 x[4];
      dequant16(S, s, x);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        if (kTail && tt >= nvalid) x[tt] = make_uint2(0u, 0u);
        const int row = 16 * s + 4 * g + tt;
        *reinterpret_cast<uint2*>(sm_k + row * kKRow + 2 * (64 * wave + 4 * col)) = x[tt];
      }
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int s = 2 * tb + s2;
      const f16x2 rsc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(S.rs[s2], 1.0f, false);
      const f16x2 rs2 = {rsc[0], rsc[0]};
      uint32_t r0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(S.r[s2], 1.0f, 0) * rs2);
      uint32_t r1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(S.r[s2], 1.0f, 1) * rs2);
      if (kTail) {
        const int tok = (tA + s) * kTile + 4 * r_g + r_tt;
        if (!((S.ok >> s) & 1) || tok >= L) r0 = r1 = 0u;
      }
      const int row = 16 * s + 4 * r_g + r_tt;
      *reinterpret_cast<uint2*>(sm_k + row * kKRow + 2 * (512 + 4 * r_i)) = make_uint2(r0, r1);
    }
  };

  auto attend = [&](const int tA, const int ok) {
    const bool tail = (tA + kStepTiles) * kTile > L || ok != (1 << kStepTiles) - 1;
    __syncthreads();

    // 2. partial scores S^T[token 32tb + i][head 32hgp + r32] over elements [288kh, +288)
    f32x16 sc;
    {
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] = 0.f;
      const uint8_t* krow = sm_k + (32 * tb + r32) * kKRow + 576 * kh + 16 * hh;
      constexpr int kDepth = 4;  // K^ fragments read ahead of their MFMAs
      f16x8 ka[kDepth];
#pragma unroll
      for (int ks = 0; ks < kDepth - 1; ++ks) ka[ks] = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(krow + 32 * ks));
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
        if (ks + kDepth - 1 < 18)
          ka[(ks + kDepth - 1) % kDepth] =
              __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(krow + 32 * (ks + kDepth - 1)));
        sc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[ks % kDepth], qf[ks], sc, 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, kDepth - 1, 0);
#pragma unroll
      for (int i = 0; i < 18 - (kDepth - 1); ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kDepth - 1, 0);
    }
    // Each wave turns values 8kh..8kh+7 of the scores into P (the B operand
    // of PV k step 2tb + kh), so it needs the other half of the dot product
    // for those 8 only: it publishes the 8 partials its partner (kh ^ 1)
    // needs and adds the 8 it gets back. Same sums, in the same order, as
    // exchanging all 16.
    float mine[8];
    {
      float give[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        mine[u] = kh ? sc[8 + u] : sc[u];
        give[u] = kh ? sc[u] : sc[8 + u];
      }
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2)
        *reinterpret_cast<f32x4*>(sm_s + ((wave * 2 + q2) * 64 + lane) * 4) =
            f32x4{give[4 * q2], give[4 * q2 + 1], give[4 * q2 + 2], give[4 * q2 + 3]};
    }
    __syncthreads();
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
      const f32x4 o4 = *reinterpret_cast<const f32x4*>(sm_s + (((wave ^ 2) * 2 + q2) * 64 + lane) * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) mine[4 * q2 + i] += o4[i];
    }
    // value u of mine is token 32tb + 16kh + 8(u/4) + 4hh + u%4 of the step
    if (__builtin_expect(tail, 0)) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int tl = 32 * tb + 16 * kh + 8 * (u >> 2) + 4 * hh + (u & 3);
        if (!((ok >> (tl >> 4)) & 1) || tA * kTile + tl >= L) mine[u] = kNegInf;
      }
    }
    // maximum over this wave's 16 tokens (8 per lane half), then over the
    // four (token half, k half) waves of the head block
    float mx = mine[0];
#pragma unroll
    for (int u = 1; u < 8; ++u) mx = fmaxf(mx, mine[u]);
    mx = fmaxf(mx, shfl_xor_f32(mx, 32)) * sscale;
    const int hl = 32 * hgp + r32;
    if (hh == 0) sm_mx[tb][kh][hl] = mx;
    __syncthreads();
    {
      mx = fmaxf(fmaxf(sm_mx[0][0][hl], sm_mx[0][1][hl]), fmaxf(sm_mx[1][0][hl], sm_mx[1][1][hl]));
      // the reference maximum only moves when a score exceeds it by more
      // than 2^kSlack, so the rescale of the accumulators below is rare; P
      // then stays <= 2^(kSlack + kPBias) = 2^15 in fp16. The four waves of
      // a head block see the same maxima and take the same decisions.
      const bool move = mx > m_run + kSlack;
      const float m_new = move ? mx : m_run;
      const float mb2 = (m_new == kNegInf) ? 0.f : m_new - kPBias;
      const float alpha = move ? ((m_run == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new)) : 1.0f;
      float p[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) p[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(mine[u], sscale, -mb2));
      uint32_t pk[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pk[i] = pack_f16x2(p[2 * i], p[2 * i + 1]);
      // the normalizer sums the fp16-rounded weights the PV products use, so
      // the output stays an exact weighted average of V whatever the rounding
      float ls = 0.f, es = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ls += f16_lo(pk[i]) + f16_hi(pk[i]);
        es += p[2 * i] + p[2 * i + 1];
      }
      l_run = l_run * alpha + ls;
      e_run = e_run * alpha + es;
      m_run = m_new;
      *reinterpret_cast<u32x4*>(sm_p + (((2 * tb + kh) * 2 + hgp) * 64 + lane) * 16) = u32x4{pk[0], pk[1], pk[2], pk[3]};
      if (kh == 0 && tb == 0 && hh == 0) sm_alpha[hl] = alpha;
    }
    __syncthreads();

    // 4. O^T[d][h] += V^T[d][t] P^T[t][h]: d = 64w + 32db + row, heads 32hb + r32
    {
      float al[2];
      bool need = false;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        al[hb] = sm_alpha[32 * hb + r32];
        need |= al[hb] != 1.0f;
      }
      if (__any(need)) {  // the reference maxima rarely move after the first steps
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) o[db][hb] *= al[hb];
      }
    }
    // k step kk = 2tb' + m covers tokens 32tb' + 16m + 8r + 4hh + e (r = 0,1; e = 0..3)
    // for the lanes of k half hh. ds_read_b64_tr_b16: in each 16-lane group,
    // lane i receives element i%4 of the 8-byte reads of lanes i/4 + 4e
    // (e = 0..3); lane 4e + c therefore addresses token row e, elements
    // D + 4c, and lane i gets element D + i of rows 0..3.
    const int tr_e = col >> 2, tr_c = col & 3;
    const uint8_t* vbase = sm_k + (4 * hh + tr_e) * kKRow + 2 * (64 * wave + 16 * ((lane >> 4) & 1) + 4 * tr_c);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      f16x8 pb[2];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
        pb[hb] = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(sm_p + ((kk * 2 + hb) * 64 + lane) * 16));
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const uint8_t* vp = vbase + (16 * kk) * kKRow + 2 * 32 * db;
        const u32x2 lo = lds_read_tr16(vp);               // tokens +0..3
        const u32x2 hi = lds_read_tr16(vp + 8 * kKRow);   // tokens +8..11
        const f16x8 va = __builtin_bit_cast(f16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) o[db][hb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pb[hb], o[db][hb], 0, 0, 0);
      }
    }
    __syncthreads();  // the next step overwrites the K^ tile
  };

  // One step of loads is in flight while the previous step is scored and
  // accumulated: the raw registers are refilled right after they have been
  // dequantized into LDS. The last step's loads run past the split; they read
  // in-pool stand-ins that are never used, which keeps every wait static.
  const int nsteps = (t_end - t_begin + kStepTiles - 1) / kStepTiles;
  {
    Step R;
    issue(R);
    for (int st = 0; st < nsteps; ++st) {
      const int tA = R.tA, ok = R.ok;
      const bool tail = (tA + kStepTiles) * kTile > L || ok != (1 << kStepTiles) - 1;
      if (tail)
        dequant(R, std::true_type{});
      else
        dequant(R, std::false_type{});
      issue(R);
      attend(tA, ok);
    }
  }

  // ---- epilogue: normalize and write this split's partial (or the output) ----
  l_run += shfl_xor_f32(l_run, 32);
  e_run += shfl_xor_f32(e_run, 32);
  if (hh == 0) {
    sm_l[2 * tb + kh][32 * hgp + r32] = l_run;
    sm_e[2 * tb + kh][32 * hgp + r32] = e_run;
    if (kh == 0 && tb == 0) sm_m[32 * hgp + r32] = m_run;
  }
  __syncthreads();
  const float g_scale = a.g_scale[0];
  const bool direct = a.num_splits == 1;
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int hl = 32 * hb + r32;
    const float lsum = (sm_l[0][hl] + sm_l[1][hl]) + (sm_l[2][hl] + sm_l[3][hl]);
    const float inv = lsum > 0.f ? g_scale / lsum : 0.f;
    const int64_t hq = (int64_t)b * a.hq + h0 + hl;
    float* dst = direct ? a.out + hq * kDv : a.ws_o + (hq * a.num_splits + split) * kDv;
    // value v of accumulator (db, hb): element 64w + 32db + 8(v/4) + 4hh + v%4
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float4 v4 = make_float4(o[db][hb][4 * q] * inv, o[db][hb][4 * q + 1] * inv, o[db][hb][4 * q + 2] * inv,
                                o[db][hb][4 * q + 3] * inv);
        *reinterpret_cast<float4*>(dst + 64 * wave + 32 * db + 8 * q + 4 * hh) = v4;
      }
    if (wave == 0 && hh == 0) {
      const float esum = (sm_e[0][hl] + sm_e[1][hl]) + (sm_e[2][hl] + sm_e[3][hl]);
      const float lse2 = esum > 0.f ? sm_m[hl] + __log2f(esum) - kPBias : kNegInf;
      if (direct) {
        if (a.lse) a.lse[hq] = lse2 * kLn2;
      } else {
        a.ws_lse[hq * a.num_splits + split] = lse2;
      }
    }
  }
}

}  // namespace
}  // namespace kvq

hipError_t kvq_launch_decode_mla(const kvq_cache* c, const MlaDecodeArgs& a, hipStream_t s) {
  (void)c;
  const int n_units = a.batch * a.num_splits;
  const int blocks = (n_units + 7) / 8 * 16;
  const int tpp = a.page_size / kvq::kTile;
  if (tpp % kvq::kStepTiles == 0 && a.tiles_per_split % kvq::kStepTiles == 0)
    kvq::decode_mla_kernel<true><<<blocks, kvq::kThreads, 0, s>>>(a);
  else
    kvq::decode_mla_kernel<false><<<blocks, kvq::kThreads, 0, s>>>(a);
  return hipGetLastError();
}
