// Paged MLA decode attention over an NVFP4 latent cache, gfx950.
//
// DeepSeek-style multi-head latent attention in absorbed form: every query
// head attends to one shared latent row per token (Dk = 576 = 512 + 64
// rope dims); K^ = the whole row, V^ = its first 512 elements. Codes are
// E2M1 with one E4M3 scale per 16 elements and a global fp32 scale g (the
// two-level NVFP4 scaling of the SGLang PR #21954 analysis page); the
// dequantization happens inside this kernel (SGLang "Quantized KV Cache"
// page, performance warning), into registers and LDS, never back to HBM.
//
// This is a dense contraction (the query heads share each latent element),
// so both products run on matrix cores in fp16, where E2M1 x E4M3 is exact:
//   S^T[t][h]  = K^[t][:] . Qs^T[:][h]      v_mfma_f32_16x16x32_f16
//                 Qs = Q * 2^s_h (a per-head power of two, so fp16 holds the
//                 BF16 query exactly; 2^-s_h goes into the score scale)
//   O^T[d][h] += V^T[d][t] . P^T[t][h]      v_mfma_f32_16x16x32_f16, P * 2^15
// and g is factored out of both (applied to the scores and to the output).
//
// Workgroup = 8 waves (2 per SIMD) = 64 query heads of one (sequence,
// context split); the two 64-head groups of a split get block ids 8 apart,
// i.e. the same XCD, so the second reads the latent tile from that L2.
// Per 32-token step (two 16-token tiles):
//   1. wave w loads the V elements [64w, 64w+64) of the 32 tokens in
//      PV-operand order (lane = 4 tokens x 4 elements, 8 bytes per tile) and
//      one rope group, dequantizes in registers, keeps its V slice for PV and
//      writes everything token-major into the LDS K^ tile;
//   2. wave w computes S for heads 16(w%4)..+15 and tokens 16(w/4)..+15 from
//      the LDS K^ tile and the LDS copy of Q (18 MFMAs), the two waves of a
//      head block exchange their maxima,
//      and publish P (fp16) and the rescale factors in LDS;
//   3. wave w accumulates O for its 64 V elements and all 64 heads (16 MFMAs).
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kPBias = 15.0f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kDk = 576, kDv = 512;
constexpr int kHeadsPerWG = 64;
constexpr int kThreads = 512;
constexpr int kKRow = kDk * 2 + 16;   // bytes per token row of the LDS K^ tile (padded)
constexpr int kPRow = 32 * 2 + 16;    // bytes per head row of the LDS P tile (padded)
constexpr int kTileCodes = 4608, kTileScales = 576;
constexpr int kMaxSplitPages = 1024;

typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

// raw per-lane bytes of one 16-token tile
struct MTile {
  uint2 v;      // V slice: tokens 4g..4g+3, elements 64w + 4*col .. +3 (2 bytes per token)
  uint32_t vs;  // E4M3 scales of those tokens (their 16-element block), one byte per token
};

__device__ __forceinline__ uint32_t e4m3_to_f16x2_bcast(uint32_t byte) {
  // E4M3 code -> the same fp16 value in both halves (exact)
  f16x2 r = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(byte | (byte << 8), 1.0f, false);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint32_t pk_mul_f16(uint32_t a, uint32_t b) {
  f16x2 r = __builtin_bit_cast(f16x2, a) * __builtin_bit_cast(f16x2, b);
  return __builtin_bit_cast(uint32_t, r);
}

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
  const int g = lane >> 4, col = lane & 15;
  const int hb = wave & 3, tb = wave >> 2;  // QK role: head block, token block

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

  __shared__ __attribute__((aligned(16))) uint8_t sm_k[32 * kKRow];
  __shared__ __attribute__((aligned(16))) uint8_t sm_p[kHeadsPerWG * kPRow];
  __shared__ float sm_mx[2][kHeadsPerWG];
  __shared__ float sm_alpha[kHeadsPerWG];
  __shared__ float sm_l[2][kHeadsPerWG];
  __shared__ float sm_m[kHeadsPerWG];
  __shared__ int sm_pg[kMaxSplitPages];
  __shared__ __attribute__((aligned(16))) uint8_t sm_q[kHeadsPerWG * kKRow];  // Q^T, fp16, per-head scaled

  const int tpp = a.page_size / kTile;
  const int fp = t_begin / tpp;
  const int n_pg = (t_end - 1) / tpp - fp + 1;
  const int32_t* pt = a.page_table + (int64_t)b * a.page_table_stride;
  for (int i = tid; i < n_pg; i += kThreads) sm_pg[i] = pt[fp + i];

  // ---- Q of head block hb, scaled by a per-head power of two, staged in LDS ----
  // (kept in LDS rather than registers: with 64 accumulators per lane the
  // fragments would spill, and spill reloads queue behind the prefetch loads)
  float sscale;
  {
    const int head = h0 + 16 * hb + col;
    const uint16_t* qrow = a.q + ((int64_t)b * a.hq + head) * kDk + 8 * g;
    uint4 raw[18];
    uint32_t mx = 0;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      raw[ks] = *reinterpret_cast<const uint4*>(qrow + 32 * ks);
      const uint32_t w4[4] = {raw[ks].x, raw[ks].y, raw[ks].z, raw[ks].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) mx = max(mx, max(w4[j] & 0x7fffu, (w4[j] >> 16) & 0x7fffu));
    }
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 16, 64));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 32, 64));
    // power of two putting the head's largest |q| in [2^14, 2^15)
    const int e = mx ? (int)(mx >> 7) - 127 : 0;
    const int sh = max(-100, min(100, 14 - e));
    const float qmul = __builtin_ldexpf(1.0f, sh);
    sscale = a.sm_scale_log2 * a.g_scale[0] * __builtin_ldexpf(1.0f, -sh);
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      const uint32_t w4[4] = {raw[ks].x, raw[ks].y, raw[ks].z, raw[ks].w};
      u32x4 h;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        h[j] = pack_f16x2(bf16_bits_to_f32(w4[j] & 0xffffu) * qmul, bf16_bits_to_f32(w4[j] >> 16) * qmul);
      if (tb == 0)
        *reinterpret_cast<u32x4*>(sm_q + (16 * hb + col) * kKRow + 16 * g + 64 * ks) = h;
    }
  }
  __syncthreads();  // sm_pg, sm_q

  const int64_t page_codes = (int64_t)a.page_size * (kDk / 2);
  const int64_t page_scales = (int64_t)a.page_size * (kDk / 16);
  // rope item of this lane: tile s (0/1 of the step), token 4*rg + rtt, elements 512 + 4*ri .. +3
  const int r_item = wave * 64 + lane;
  const int r_tile = r_item >> 8, r_g = (r_item >> 6) & 3, r_i = (r_item >> 2) & 15, r_tt = r_item & 3;

  struct Step {
    MTile t[2];
    uint32_t r;   // rope codes (2 bytes)
    uint32_t rs;  // rope scale byte
    int ok;       // bit s: tile s holds real tokens
    int tA;
  };
  auto tile_base = [&](int tile, bool& v, int64_t& cbase, int64_t& sbase) {
    const int tl = min(tile, t_end - 1);
    const int page = __builtin_amdgcn_readfirstlane(sm_pg[tl / tpp - fp]);
    v = tile < t_end && (unsigned)page < (unsigned)a.num_pages;
    const int64_t pg = v ? page : 0;
    const int sub = tl - (tl / tpp) * tpp;
    cbase = pg * page_codes + (int64_t)sub * kTileCodes;
    sbase = pg * page_scales + (int64_t)sub * kTileScales;
  };
  // loads of one step: issued one step ahead and unconditionally (a missing
  // tile reads an in-pool stand-in and is masked), so waits are exact
  auto issue = [&](int pr, Step& S) {
    const int tA = t_begin + 2 * pr;
    S.tA = tA;
    int ok = 0;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      bool v;
      int64_t cb, sb;
      tile_base(tA + s2, v, cb, sb);
      ok |= (int)v << s2;
      S.t[s2].v = __builtin_bit_cast(uint2, __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(
                                                 a.codes + cb + 8 * ((wave * 4 + g) * 16 + col))));
      S.t[s2].vs = __builtin_nontemporal_load(
          reinterpret_cast<const uint32_t*>(a.scales + sb + 4 * ((wave * 4 + g) * 4 + (col >> 2))));
    }
    {
      bool v;
      int64_t cb, sb;
      tile_base(tA + r_tile, v, cb, sb);
      S.r = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(a.codes + cb + 4096 + 2 * (r_item & 255)));
      S.rs = a.scales[sb + 512 + 4 * (r_g * 4 + (r_i >> 2)) + r_tt];
    }
    S.ok = ok;
  };

  f32x4 o[4][4];  // [V tile j][head block n]
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int n = 0; n < 4; ++n) o[j][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;  // head 16*hb + col, this wave's token block

  auto compute = [&](Step& S) {
    const int tA = S.tA;
    const bool tail = (tA + 2) * kTile > L || S.ok != 3;
    // 1. dequantize the V slice (kept for PV) and the rope group into the LDS K^ tile
    uint32_t x[2][4][2];  // [tile][token tt][pair k]: fp16 pairs, elements 4*col + 2k, +1
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int nvalid = tail ? (((S.ok >> s2) & 1) ? max(0, min(4, L - (tA + s2) * kTile - 4 * g)) : 0) : 4;
      const uint32_t wlo = S.t[s2].v.x, whi = S.t[s2].v.y;  // tokens 0,1 | 2,3
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const uint32_t w = (tt < 2 ? wlo : whi) >> (16 * (tt & 1));
        const uint32_t sc = e4m3_to_f16x2_bcast((S.t[s2].vs >> (8 * tt)) & 0xffu);
        x[s2][tt][0] = pk_mul_f16(fp4x2_to_f16x2<0>(w), sc);
        x[s2][tt][1] = pk_mul_f16(fp4x2_to_f16x2<1>(w), sc);
        if (tt >= nvalid) x[s2][tt][0] = x[s2][tt][1] = 0u;
        const int row = 16 * s2 + 4 * g + tt;
        *reinterpret_cast<uint2*>(sm_k + row * kKRow + 2 * (64 * wave + 4 * col)) = make_uint2(x[s2][tt][0], x[s2][tt][1]);
      }
    }
    {
      const uint32_t sc = e4m3_to_f16x2_bcast(S.rs & 0xffu);
      uint32_t r0 = pk_mul_f16(fp4x2_to_f16x2<0>(S.r), sc), r1 = pk_mul_f16(fp4x2_to_f16x2<1>(S.r), sc);
      const int tok = (tA + r_tile) * kTile + 4 * r_g + r_tt;
      if (tail && (!((S.ok >> r_tile) & 1) || tok >= L)) r0 = r1 = 0u;
      const int row = 16 * r_tile + 4 * r_g + r_tt;
      *reinterpret_cast<uint2*>(sm_k + row * kKRow + 2 * (512 + 4 * r_i)) = make_uint2(r0, r1);
    }
    __syncthreads();

    // 2. scores: heads 16hb + col, tokens 16tb + 4g + i
    float s[4];
    {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const uint8_t* krow = sm_k + (16 * tb + col) * kKRow + 16 * g;
      const uint8_t* qrow2 = sm_q + (16 * hb + col) * kKRow + 16 * g;
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
        const f16x8 ka = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(krow + 64 * ks));
        const f16x8 qb = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(qrow2 + 64 * ks));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qb, acc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = acc[i] * sscale;
    }
    if (tail) {
      const int tok0 = (tA + tb) * kTile + 4 * g;
      const int nvalid = ((S.ok >> tb) & 1) ? max(0, min(4, L - tok0)) : 0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i >= nvalid) s[i] = kNegInf;
    }
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = fmaxf(mx, shfl_xor_f32(mx, 16));
    mx = fmaxf(mx, shfl_xor_f32(mx, 32));
    if (g == 0) sm_mx[tb][16 * hb + col] = mx;
    __syncthreads();
    mx = fmaxf(mx, sm_mx[tb ^ 1][16 * hb + col]);
    const float m_new = fmaxf(m_run, mx);
    const float mb2 = (m_new == kNegInf) ? 0.f : m_new - kPBias;
    const float alpha = (m_run == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(s[i] - mb2);
    l_run = l_run * alpha + (p[0] + p[1]) + (p[2] + p[3]);
    m_run = m_new;
    // P^T row of head 16hb + col: K order [tile A 4g..4g+3, tile B 4g..4g+3]
    *reinterpret_cast<uint2*>(sm_p + (16 * hb + col) * kPRow + 16 * g + 8 * tb) =
        make_uint2(pack_f16x2(p[0], p[1]), pack_f16x2(p[2], p[3]));
    if (g == 0 && tb == 0) sm_alpha[16 * hb + col] = alpha;
    __syncthreads();

    // 3. O^T[d][h] += V^T[d][t] P^T[t][h]: elements 64w + 4*row + j, all 64 heads
    {
      float al[4];
      bool need = false;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        al[n] = sm_alpha[16 * n + col];
        need |= al[n] != 1.0f;
      }
      if (__any(need)) {  // once the running maxima settle, most steps skip this
#pragma unroll
        for (int n = 0; n < 4; ++n)
#pragma unroll
          for (int j = 0; j < 4; ++j) o[j][n] *= al[n];
      }
    }
    f16x8 pb[4];
#pragma unroll
    for (int n = 0; n < 4; ++n)
      pb[n] = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(sm_p + (16 * n + col) * kPRow + 16 * g));
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      u32x4 lo = {lo_halves(x[0][0][k], x[0][1][k]), lo_halves(x[0][2][k], x[0][3][k]),
                  lo_halves(x[1][0][k], x[1][1][k]), lo_halves(x[1][2][k], x[1][3][k])};
      u32x4 hi = {hi_halves(x[0][0][k], x[0][1][k]), hi_halves(x[0][2][k], x[0][3][k]),
                  hi_halves(x[1][0][k], x[1][1][k]), hi_halves(x[1][2][k], x[1][3][k])};
      const f16x8 vlo = __builtin_bit_cast(f16x8, lo), vhi = __builtin_bit_cast(f16x8, hi);
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        o[2 * k][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vlo, pb[n], o[2 * k][n], 0, 0, 0);
        o[2 * k + 1][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vhi, pb[n], o[2 * k + 1][n], 0, 0, 0);
      }
    }
  };

  // Steps are prefetched three ahead through a ring of registers. One
  // workgroup per CU steps through the tiles in lockstep, so a single step
  // in flight (~10 KB) cannot cover HBM latency. The loads of the last few
  // ring slots may run past the split: they read in-pool stand-ins (masked,
  // never computed), which keeps every wait count in the loop static.
  const int nsteps = (t_end - t_begin + 1) >> 1;
  {
    Step R0, R1, R2, R3;
    issue(0, R0);
    issue(1, R1);
    issue(2, R2);
    for (int st = 0;; st += 4) {
      issue(st + 3, R3);
      compute(R0);
      if (st + 1 >= nsteps) break;
      issue(st + 4, R0);
      compute(R1);
      if (st + 2 >= nsteps) break;
      issue(st + 5, R1);
      compute(R2);
      if (st + 3 >= nsteps) break;
      issue(st + 6, R2);
      compute(R3);
      if (st + 4 >= nsteps) break;
    }
  }

  // ---- epilogue: normalize and write this split's partial (or the output) ----
  l_run += shfl_xor_f32(l_run, 16);
  l_run += shfl_xor_f32(l_run, 32);
  if (g == 0) {
    sm_l[tb][16 * hb + col] = l_run;
    if (tb == 0) sm_m[16 * hb + col] = m_run;
  }
  __syncthreads();
  const float g_scale = a.g_scale[0];
  const bool direct = a.num_splits == 1;
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int hl = 16 * n + col;
    const float lsum = sm_l[0][hl] + sm_l[1][hl];
    const float inv = lsum > 0.f ? g_scale / lsum : 0.f;
    const int64_t hq = (int64_t)b * a.hq + h0 + hl;
    float* dst = direct ? a.out + hq * kDv : a.ws_o + (hq * a.num_splits + split) * kDv;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float4 v4 = make_float4(o[0][n][r] * inv, o[1][n][r] * inv, o[2][n][r] * inv, o[3][n][r] * inv);
      *reinterpret_cast<float4*>(dst + 64 * wave + 4 * (4 * g + r)) = v4;
    }
    if (wave == 0 && g == 0) {
      const float lse2 = lsum > 0.f ? sm_m[hl] + __log2f(lsum) - kPBias : kNegInf;
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
  kvq::decode_mla_kernel<<<blocks, kvq::kThreads, 0, s>>>(a);
  return hipGetLastError();
}
