// kvq_dequantize_prev_kv: FP4 cache pages -> FP8 E4M3 rows, gfx950.
//
// The PR #21954 analysis page ("code analysis") describes dequantize_prev_kv:
// the stored FP4 KV and its scales are turned into FP8 E4M3 (the dq_k_buffer /
// dq_v_buffer workspaces of create_buffers) so that an FP8 prefill kernel can
// read the quantized prefix. Per element: x^ is the exact dequantized value
// rounded once to binary32 (MX16: e2m1 * 2^e; NVFP4: e2m1 * e4m3 * g), and
// code = RNE_sat_E4M3(fl32(x^ / s)) with the per-tensor output scale s.
// Output rows are token-major: GQA [n_pages][Hkv][page_size][D] for K and V,
// MLA [n_pages][page_size][576].
//
// No per-element division. The 16 elements of a block share one scale, so a
// block has only 8 distinct magnitudes |m| in {0, .5, 1, 1.5, 2, 3, 4, 6}: the
// block builds a table of their 8 E4M3 codes and looks the codes up four at a
// time with a byte permute, the E2M1 sign bit XORed on top (rounding to
// nearest even is symmetric, so code(-x) = code(x) ^ 0x80, signed zeros
// included). Each nonzero magnitude is c * 2^k with c in {1, 3}, and scaling
// by a power of two commutes with rounding to binary32 whenever the results
// are normal, so every table entry is a power-of-two multiple of a constant:
//   MX16:  fl32(c * 2^(k+e) / s)          = 2^(k+e)    * fl32(c / s)
//   NVFP4: fl32(fl32(c * 2^k * |b| * g) / s) = 2^(k+eb) * fl32(fl32(c * mb * g) / s)
// with |b| = mb * 2^eb (mb one of the 8 E4M3 mantissas 1 + j/8). The kernel
// computes those constants once per workgroup in LDS (2 per scale for MX16,
// 16 for NVFP4) with IEEE divisions. When an entry's true value is not a
// normal binary32 number it is either below 2^-116 (E4M3 code 0 on both
// routes) or above 2^118 (saturated to 448 on both routes), which holds for
// s (and g) in [2^-100, 2^100]; outside that range the kernel builds every
// table entry by direct multiplication and division instead (same result,
// 7 divisions per block).
// Every listed page id outside [0, num_pages) yields all-zero rows.
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr float kLo = 0x1p-100f, kHi = 0x1p100f;

__device__ __forceinline__ bool in_range(float x) { return x >= kLo && x <= kHi; }

struct Lut {
  uint32_t lo, hi;  // E4M3 codes of magnitudes 0..3 and 4..7, one byte each
};

__device__ __forceinline__ float sat(float v) { return fminf(v, 448.0f); }  // v >= 0 (or +inf)

__device__ __forceinline__ Lut make_lut(float v1, float v2, float v3, float v4, float v5, float v6, float v7) {
  uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(0.0f, sat(v1), 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(sat(v2), sat(v3), lo, true);
  uint32_t hi = __builtin_amdgcn_cvt_pk_fp8_f32(sat(v4), sat(v5), 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(sat(v6), sat(v7), hi, true);
  return {lo, hi};
}

// magnitudes .5 1 1.5 2 3 4 6 = c * 2^k: (1,-1) (1,0) (3,-1) (1,1) (3,0) (1,2) (3,1)
__device__ __forceinline__ Lut lut_scaled(float t1, float t3, int e) {
  return make_lut(__builtin_ldexpf(t1, e - 1), __builtin_ldexpf(t1, e), __builtin_ldexpf(t3, e - 1),
                  __builtin_ldexpf(t1, e + 1), __builtin_ldexpf(t3, e), __builtin_ldexpf(t1, e + 2),
                  __builtin_ldexpf(t3, e + 1));
}

// the same tables by direct arithmetic, in the order the definition rounds:
// MX16 x^ = fl32(m * 2^e) (exact below overflow), NVFP4 x^ = fl32((m * |b|) * |g|)
// (m * |b| exact); entry = fl32(x^ / |s|)
__device__ __forceinline__ Lut lut_direct_mx(int e, float s) {
  return make_lut(__builtin_ldexpf(0.5f, e) / s, __builtin_ldexpf(1.0f, e) / s, __builtin_ldexpf(1.5f, e) / s,
                  __builtin_ldexpf(2.0f, e) / s, __builtin_ldexpf(3.0f, e) / s, __builtin_ldexpf(4.0f, e) / s,
                  __builtin_ldexpf(6.0f, e) / s);
}
__device__ __forceinline__ Lut lut_direct_nv(float b, float g, float s) {
  return make_lut(((0.5f * b) * g) / s, ((1.0f * b) * g) / s, ((1.5f * b) * g) / s, ((2.0f * b) * g) / s,
                  ((3.0f * b) * g) / s, ((4.0f * b) * g) / s, ((6.0f * b) * g) / s);
}

// 8 E2M1 codes (element 2j in the low nibble of byte j) -> 8 E4M3 codes
__device__ __forceinline__ uint2 apply_lut(const Lut& L, uint32_t w, uint32_t sgn) {
  const uint32_t ie = w & 0x07070707u, io = (w >> 4) & 0x07070707u;
  const uint32_t ev = __builtin_amdgcn_perm(L.hi, L.lo, ie) ^ ((w << 4) & 0x80808080u) ^ sgn;
  const uint32_t od = __builtin_amdgcn_perm(L.hi, L.lo, io) ^ (w & 0x80808080u) ^ sgn;
  return make_uint2(__builtin_amdgcn_perm(od, ev, 0x05010400u), __builtin_amdgcn_perm(od, ev, 0x07030602u));
}

__device__ __forceinline__ uint4 block_codes(const Lut& L, uint32_t w0, uint32_t w1, uint32_t sgn) {
  const uint2 a = apply_lut(L, w0, sgn), b = apply_lut(L, w1, sgn);
  return make_uint4(a.x, a.y, b.x, b.y);
}

__device__ __forceinline__ uint32_t sign_mask(float x) { return __float_as_uint(x) >> 31 ? 0x80808080u : 0u; }

// ------------------------------------------------------------------ MX16 --
// One workgroup per listed page; a thread takes one (kv head, token, block
// pair p): K blocks 2p, 2p+1 (16 code bytes, 2 adjacent scale bytes) and the
// same two V blocks (four 4-byte groups, 2 scale bytes).
__global__ void __launch_bounds__(256) dequant_prev_mx16_kernel(
    const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc, const uint8_t* __restrict__ ksc,
    const uint8_t* __restrict__ vsc, const int32_t* __restrict__ pages, int64_t num_pages, int hkv, int page_size,
    int64_t code_block, int64_t scale_block, const float* __restrict__ ks_out, const float* __restrict__ vs_out,
    uint8_t* __restrict__ dq_k, uint8_t* __restrict__ dq_v) {
  constexpr int D = 128;
  __shared__ float sh_r[4];  // fl32(1/sk), fl32(3/sk), fl32(1/sv), fl32(3/sv)
  const float sk = ks_out ? ks_out[0] : 1.0f, sv = vs_out ? vs_out[0] : 1.0f;
  const bool fast = in_range(sk) && in_range(sv);
  if (threadIdx.x < 4) {
    const float s = threadIdx.x < 2 ? sk : sv;
    sh_r[threadIdx.x] = ((threadIdx.x & 1) ? 3.0f : 1.0f) / s;
  }
  __syncthreads();
  const float rk1 = sh_r[0], rk3 = sh_r[1], rv1 = sh_r[2], rv3 = sh_r[3];
  const uint32_t ksg = fast ? 0u : sign_mask(sk), vsg = fast ? 0u : sign_mask(sv);
  const float ska = fabsf(sk), sva = fabsf(sv);

  const int i = blockIdx.x;
  const int page = pages[i];
  const int items = hkv * page_size * 4;
  const int64_t row0 = (int64_t)i * hkv * page_size;  // first output row of this page
  for (int it = threadIdx.x; it < items; it += blockDim.x) {
    const int p = it & 3;
    const int t = (it >> 2) % page_size;
    const int h = (it >> 2) / page_size;
    uint4* ok = reinterpret_cast<uint4*>(dq_k + (row0 + (int64_t)h * page_size + t) * D + 32 * p);
    uint4* ov = reinterpret_cast<uint4*>(dq_v + (row0 + (int64_t)h * page_size + t) * D + 32 * p);
    if ((unsigned)page >= (unsigned long long)num_pages) {  // not a page of the pool: zero rows
      ok[0] = ok[1] = ov[0] = ov[1] = make_uint4(0, 0, 0, 0);
      continue;
    }
    const int t16 = t & 15;
    const int64_t cbase = ((int64_t)page * hkv + h) * code_block + (int64_t)(t >> 4) * 8 * D;
    const int64_t sbase = ((int64_t)page * hkv + h) * scale_block + (int64_t)(t >> 4) * D;
    // K: codes of blocks 2p, 2p+1 at 256*p + 16*t16 (+8), scales at 32*p + 2*t16 (+1)
    const uint4 kw = *reinterpret_cast<const uint4*>(kc + cbase + 256 * p + 16 * t16);
    const uint16_t kse = *reinterpret_cast<const uint16_t*>(ksc + sbase + 32 * p + 2 * t16);
    // V: 8-element groups c8 = 4p..4p+3 at 16*(16*(t16/4) + c8) + 4*(t16%4),
    // scale of block b at 4*(8*(t16/4) + b) + t16%4
    const uint8_t* vb = vc + cbase + 256 * (t16 >> 2) + 4 * (t16 & 3) + 64 * p;
    const uint32_t v0 = *reinterpret_cast<const uint32_t*>(vb), v1 = *reinterpret_cast<const uint32_t*>(vb + 16);
    const uint32_t v2 = *reinterpret_cast<const uint32_t*>(vb + 32), v3 = *reinterpret_cast<const uint32_t*>(vb + 48);
    const uint8_t* vsb = vsc + sbase + 32 * (t16 >> 2) + (t16 & 3) + 8 * p;
    const int vse0 = vsb[0], vse1 = vsb[4];
    const int ke0 = (kse & 0xff) - 127, ke1 = (kse >> 8) - 127;
    Lut lk0, lk1, lv0, lv1;
    if (fast) {
      lk0 = lut_scaled(rk1, rk3, ke0);
      lk1 = lut_scaled(rk1, rk3, ke1);
      lv0 = lut_scaled(rv1, rv3, vse0 - 127);
      lv1 = lut_scaled(rv1, rv3, vse1 - 127);
    } else {
      lk0 = lut_direct_mx(ke0, ska);
      lk1 = lut_direct_mx(ke1, ska);
      lv0 = lut_direct_mx(vse0 - 127, sva);
      lv1 = lut_direct_mx(vse1 - 127, sva);
    }
    ok[0] = block_codes(lk0, kw.x, kw.y, ksg);
    ok[1] = block_codes(lk1, kw.z, kw.w, ksg);
    ov[0] = block_codes(lv0, v0, v1, vsg);
    ov[1] = block_codes(lv1, v2, v3, vsg);
  }
}

// ----------------------------------------------------------------- NVFP4 --
// One workgroup per listed page; a thread takes one (tile, 4-token group g4,
// block b) and its 4 tokens tt: 32 contiguous code bytes (halfword 4q + tt
// holds elements 4q..4q+3 of token tt) and 4 contiguous scale bytes.
__global__ void __launch_bounds__(192) dequant_prev_nvfp4_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, const int32_t* __restrict__ pages,
    int64_t num_pages, int page_size, const float* __restrict__ g_scale, const float* __restrict__ ks_out,
    uint8_t* __restrict__ dq_k) {
  constexpr int DK = 576, NB = DK / 16;
  __shared__ float sh_t[16];  // [c = 1, 3][mantissa j]: fl32(fl32(c * (1 + j/8) * g) / s)
  const float g = g_scale[0], s = ks_out ? ks_out[0] : 1.0f;
  const bool fast = in_range(g) && in_range(s);
  if (threadIdx.x < 16) {
    const float c = threadIdx.x < 8 ? 1.0f : 3.0f;
    sh_t[threadIdx.x] = ((c * (1.0f + 0.125f * (threadIdx.x & 7))) * g) / s;
  }
  __syncthreads();
  const uint32_t gs_sign = fast ? 0u : (sign_mask(g) ^ sign_mask(s));
  const float ga = fabsf(g), sa = fabsf(s);

  const int i = blockIdx.x;
  const int page = pages[i];
  const int items = (page_size / 16) * 4 * NB;
  const int64_t row0 = (int64_t)i * page_size;
  for (int it = threadIdx.x; it < items; it += blockDim.x) {
    const int b = it % NB;
    const int g4 = (it / NB) & 3;
    const int tile = it / (4 * NB);
    const int t0 = tile * 16 + 4 * g4;
    uint8_t* orow = dq_k + (row0 + t0) * DK + 16 * b;
    if ((unsigned)page >= (unsigned long long)num_pages) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) *reinterpret_cast<uint4*>(orow + tt * DK) = make_uint4(0, 0, 0, 0);
      continue;
    }
    const uint8_t* cb = codes + (int64_t)page * page_size * (DK / 2) + (int64_t)tile * 4608;
    const uint8_t* sb = scales + (int64_t)page * page_size * NB + (int64_t)tile * 576;
    const int coff = b < 32 ? 128 * ((b >> 2) * 4 + g4) + 32 * (b & 3) : 4096 + 128 * g4 + 32 * (b - 32);
    const int soff = b < 32 ? 16 * ((b >> 2) * 4 + g4) + 4 * (b & 3) : 512 + 16 * g4 + 4 * (b - 32);
    const uint4 ca = *reinterpret_cast<const uint4*>(cb + coff);       // halfwords 4q+tt, q = 0, 1
    const uint4 cc = *reinterpret_cast<const uint4*>(cb + coff + 16);  // q = 2, 3
    const uint32_t sw = *reinterpret_cast<const uint32_t*>(sb + soff);  // E4M3 scale of token tt in byte tt
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      // elements 0..7 = halfwords tt (q0) and 4+tt (q1); 8..15 = q2, q3
      const uint32_t qa0 = (tt < 2 ? ca.x : ca.y), qa1 = (tt < 2 ? ca.z : ca.w);
      const uint32_t qc0 = (tt < 2 ? cc.x : cc.y), qc1 = (tt < 2 ? cc.z : cc.w);
      const uint32_t sel = (tt & 1) ? 0x07060302u : 0x05040100u;  // halfword tt%2 of each source
      const uint32_t w0 = __builtin_amdgcn_perm(qa1, qa0, sel), w1 = __builtin_amdgcn_perm(qc1, qc0, sel);
      const uint32_t sc = (sw >> (8 * tt)) & 0xffu;
      const float bf = __builtin_amdgcn_cvt_pk_f32_fp8(sc, false)[0];  // exact
      const float ba = fabsf(bf);
      Lut L;
      if (fast) {
        const uint32_t bits = __float_as_uint(ba);
        const int j = (bits >> 20) & 7;
        const int eb = (int)(bits >> 23) - 127;
        L = lut_scaled(sh_t[j], sh_t[8 + j], eb);
        if (ba == 0.0f) L = {0u, 0u};
      } else {
        L = lut_direct_nv(ba, ga, sa);
      }
      *reinterpret_cast<uint4*>(orow + tt * DK) = block_codes(L, w0, w1, sign_mask(bf) ^ gs_sign);
    }
  }
}

}  // namespace
}  // namespace kvq

hipError_t kvq_launch_dequant_prev(const kvq_cache* c, const int32_t* pages, int32_t n_pages, const float* g_scale,
                                   const float* ks_out, const float* vs_out, uint8_t* dq_k, uint8_t* dq_v,
                                   hipStream_t s) {
  const kvq_cache_desc& d = c->desc;
  const kvq_layout& L = c->layout;
  uint8_t* base = c->base;
  if (d.dtype == KVQ_FP4_MX16) {
    kvq::dequant_prev_mx16_kernel<<<n_pages, 256, 0, s>>>(
        base + L.k_codes_offset, base + L.v_codes_offset, base + L.k_scales_offset, base + L.v_scales_offset, pages,
        d.num_pages, d.num_kv_heads, d.page_size, c->code_block_bytes, c->scale_block_bytes, ks_out, vs_out, dq_k,
        dq_v);
  } else {
    kvq::dequant_prev_nvfp4_kernel<<<n_pages, 192, 0, s>>>(base + L.k_codes_offset, base + L.k_scales_offset, pages,
                                                          d.num_pages, d.page_size, g_scale, ks_out, dq_k);
  }
  return hipGetLastError();
}
