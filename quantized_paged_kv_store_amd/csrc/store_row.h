// Quantize-and-place routines shared by the store kernels and the decode
// kernels' append path: each call handles one 16-element chunk of one stored
// row and writes its codes (and block scale) into the cache layouts given in
// include/kvq.h.
//
// Quantization rules (the pages: SGLang "Quantized KV Cache" page, sections
// "Supported formats" and "Scaling factors"; PR #21954 analysis page,
// NVFP4KVMethod / BlockFP4KVMethod and quantize_and_store):
//   FP8:   code = RNE(clamp(x / s, -max, max)) with x / s IEEE binary32; s per
//          tensor, per KV head, or KIVI-style (per channel for K, per token
//          for V: s = fl32(row amax / max))
//   MX16:  per 16 elements e = floor(log2 amax) - 2 (clamped to [-127, 127]),
//          element = RNE_sat_E2M1(x * 2^-e), scale byte = e + 127
//   NVFP4: per 16 elements s = amax / fl32(6 g) -> E4M3 (saturating),
//          sd = E4M3(s) * g, element = RNE_sat_E2M1(x / sd) (signed zero if sd == 0)
// The gfx950 converts round to nearest even; the FP8 ones turn out-of-range
// inputs into NaN/Inf, so values are clamped to the format maximum first
// (which equals round-then-saturate). The E2M1 convert saturates by itself.
#pragma once

#include "kvq_internal.h"

namespace kvq {

// ------------------------------------------------------ binary32 quotient --
// x / s for many x and one s, correctly rounded, without a division per
// element. With r = RN(1/s) and q0 = RN(x r), the remainder x - s q0 is exact
// in one FMA and RN(q0 + (x - s q0) r) = RN(x / s) (Markstein's theorem for
// a correctly rounded reciprocal) while nothing underflows or overflows:
// |x| >= 2^-100 and 2^-100 <= |q0| <= 2^100, for s in [2^-60, 2^60]. Past
// those bounds q0 is kept: it has the quotient's sign and lies below 2^-40
// or above 2^99 with it, where every FP8 and E2M1 encoder gives the same
// code (a signed zero or the saturated maximum). Other divisors divide.
struct Divisor {
  float s, r;
  bool fast;
};
__device__ __forceinline__ Divisor make_divisor(float s) {
  Divisor d;
  d.s = s;
  d.fast = s >= 0x1p-60f && s <= 0x1p60f;
  d.r = d.fast ? 1.0f / s : 0.0f;  // IEEE binary32 division
  return d;
}
__device__ __forceinline__ float quotient(float x, const Divisor& d) {
  if (!d.fast) return x / d.s;
  const float q0 = x * d.r;
  const float q1 = __builtin_fmaf(__builtin_fmaf(-d.s, q0, x), d.r, q0);
  const float aq = __builtin_fabsf(q0);
  return (__builtin_fabsf(x) >= 0x1p-100f && aq >= 0x1p-100f && aq <= 0x1p100f) ? q1 : q0;
}

// ------------------------------------------------------------------- FP8 --
template <int FMT>
__device__ __forceinline__ uint32_t encode_fp8x4(float a, float b, float c, float d) {
  constexpr float MX = (FMT == KVQ_FP8_E4M3) ? 448.0f : 57344.0f;
  a = fminf(fmaxf(a, -MX), MX);
  b = fminf(fmaxf(b, -MX), MX);
  c = fminf(fmaxf(c, -MX), MX);
  d = fminf(fmaxf(d, -MX), MX);
  uint32_t w;
  if (FMT == KVQ_FP8_E4M3) {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
  }
  return w;
}

// 16 BF16 (two uint4) / s -> 16 FP8 codes (uint4).
template <int FMT>
__device__ __forceinline__ uint4 quant_fp8_16(const uint4 lo, const uint4 hi, const Divisor& s) {
  const uint32_t in[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  uint32_t out[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w0 = in[2 * i], w1 = in[2 * i + 1];
    out[i] = encode_fp8x4<FMT>(quotient(bf16_bits_to_f32(w0 & 0xffffu), s), quotient(bf16_bits_to_f32(w0 >> 16), s),
                               quotient(bf16_bits_to_f32(w1 & 0xffffu), s), quotient(bf16_bits_to_f32(w1 >> 16), s));
  }
  return make_uint4(out[0], out[1], out[2], out[3]);
}

// The BF16 inputs of chunk c (elements 16c..16c+15) of one (token, kv head)
// K row and V row, as one lane holds them.
struct RowChunk {
  uint4 k0, k1, v0, v1;
};

__device__ __forceinline__ RowChunk load_row_chunk(const uint16_t* krow, const uint16_t* vrow, int c) {
  const uint4* kp = reinterpret_cast<const uint4*>(krow + 16 * c);
  const uint4* vp = reinterpret_cast<const uint4*>(vrow + 16 * c);
  return RowChunk{kp[0], kp[1], vp[0], vp[1]};
}

// Chunk c (elements 16c..16c+15) of one (token, kv head) row pair, from its
// loaded inputs. `base` addresses the row's 16-token tile inside its
// (page, kv head) block.
template <int FMT>
__device__ __forceinline__ void put_fp8_chunk(const RowChunk& r, int c, int t16, const Divisor& ks,
                                              const Divisor& vs, uint8_t* kc, uint8_t* vc, int64_t base) {
  const uint4 kq = quant_fp8_16<FMT>(r.k0, r.k1, ks);
  const uint4 vq = quant_fp8_16<FMT>(r.v0, r.v1, vs);
  // K: the 16 elements of chunk c are 16 contiguous bytes
  *reinterpret_cast<uint4*>(kc + base + 256 * c + 16 * t16) = kq;
  // V: element d = 16c + r at 1024*(d/64) + 16*(16*(t16/4) + r) + 4*(c%4) + t16%4
  uint8_t* vb = vc + base + 1024 * (c >> 2) + 16 * (16 * (t16 >> 2)) + 4 * (c & 3) + (t16 & 3);
  const uint32_t vw[4] = {vq.x, vq.y, vq.z, vq.w};
#pragma unroll
  for (int e = 0; e < 16; ++e) vb[16 * e] = (uint8_t)(vw[e >> 2] >> (8 * (e & 3)));
}

template <int FMT>
__device__ __forceinline__ void put_fp8_chunk(const uint16_t* krow, const uint16_t* vrow, int c, int t16,
                                              const Divisor& ks, const Divisor& vs, uint8_t* kc, uint8_t* vc,
                                              int64_t base) {
  put_fp8_chunk<FMT>(load_row_chunk(krow, vrow, c), c, t16, ks, vs, kc, vc, base);
}

// Element-wise form of put_fp8_chunk: N = 2 or 4 consecutive elements e0..
// (inside one 16-element chunk) of one (token, kv head) K row (is_v false) or
// V row, so that a whole wave shares one token's store, 64 lanes over K and V,
// where put_fp8_chunk takes a chunk of both rows per lane.
// place_fp8_elems writes the N codes held in q's low bytes at the places
// put_fp8_chunk gives them.
template <int N>
__device__ __forceinline__ void place_fp8_elems(const uint32_t q, bool is_v, int e0, int t16, uint8_t* codes,
                                                int64_t base) {
  static_assert(N == 2 || N == 4, "two or four elements per lane");
  if (!is_v) {
    // K: the chunk's 16 codes are 16 contiguous bytes
    uint8_t* kb = codes + base + 256 * (e0 >> 4) + 16 * t16 + (e0 & 15);
    if constexpr (N == 4)
      *reinterpret_cast<uint32_t*>(kb) = q;
    else
      *reinterpret_cast<uint16_t*>(kb) = (uint16_t)q;
  } else {
    // V: element d at 1024*(d/64) + 16*(16*(t16/4) + d%16) + 4*((d/16)%4) + t16%4
    uint8_t* vb = codes + base + 1024 * (e0 >> 6) + 16 * (16 * (t16 >> 2) + (e0 & 15)) + 4 * ((e0 >> 4) & 3) +
                  (t16 & 3);
#pragma unroll
    for (int i = 0; i < N; ++i) vb[16 * i] = (uint8_t)(q >> (8 * i));
  }
}

// The N elements' values from their BF16 bits (element e0 + i in halfword i
// of w), as floats (zero past N).
template <int N>
__device__ __forceinline__ void unpack_elems(const uint2 w, float (&x)[4]) {
  x[0] = bf16_bits_to_f32(w.x & 0xffffu);
  x[1] = bf16_bits_to_f32(w.x >> 16);
  x[2] = N == 4 ? bf16_bits_to_f32(w.y & 0xffffu) : 0.0f;
  x[3] = N == 4 ? bf16_bits_to_f32(w.y >> 16) : 0.0f;
}

// Codes RNE_sat(x / s) of the N elements, placed.
template <int FMT, int N>
__device__ __forceinline__ void put_fp8_elems(const uint2 w, bool is_v, int e0, int t16, const Divisor& s,
                                              uint8_t* codes, int64_t base) {
  float x[4];
  unpack_elems<N>(w, x);
  place_fp8_elems<N>(encode_fp8x4<FMT>(quotient(x[0], s), quotient(x[1], s), quotient(x[2], s), quotient(x[3], s)),
                     is_v, e0, t16, codes, base);
}

// Store of four tokens that fill one 4-token group of a tile (t16 = 4g..4g+3),
// whose V codes share lane words: the caller for group member i writes
// elements 16c + 4i .. +3 of all four V rows, one 4-byte word per element.
// vrow0 is the first member's V row; the rows are `stride` elements apart.
template <int FMT>
__device__ __forceinline__ void put_fp8_v_group(const uint16_t* vrow0, int64_t stride, int c, int g, int i,
                                                const Divisor& vs, uint8_t* vc, int64_t base) {
  float x[4][4];  // [token][element]
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const uint2 w = *reinterpret_cast<const uint2*>(vrow0 + tt * stride + 16 * c + 4 * i);
    x[tt][0] = bf16_bits_to_f32(w.x & 0xffffu);
    x[tt][1] = bf16_bits_to_f32(w.x >> 16);
    x[tt][2] = bf16_bits_to_f32(w.y & 0xffffu);
    x[tt][3] = bf16_bits_to_f32(w.y >> 16);
  }
  uint8_t* vb = vc + base + 1024 * (c >> 2) + 16 * (16 * g + 4 * i) + 4 * (c & 3);
#pragma unroll
  for (int k = 0; k < 4; ++k)
    *reinterpret_cast<uint32_t*>(vb + 16 * k) = encode_fp8x4<FMT>(
        quotient(x[0][k], vs), quotient(x[1][k], vs), quotient(x[2][k], vs), quotient(x[3][k], vs));
}

// ------------------------------------------------ FP8, KIVI-style scaling --
// K: one scale per (kv head, channel); V: one scale per (token, kv head),
// fl32(row amax / format max) (1.0 for an all-zero row), computed here.
// The "KV cache quantization mechanism and traps" page, K and V distributions.

// 16 BF16 / 16 per-element scales -> 16 FP8 codes.
template <int FMT>
__device__ __forceinline__ uint4 quant_fp8_16_vec(const uint4 lo, const uint4 hi, const float* s) {
  const uint32_t in[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  uint32_t out[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w0 = in[2 * i], w1 = in[2 * i + 1];
    out[i] = encode_fp8x4<FMT>(bf16_bits_to_f32(w0 & 0xffffu) / s[4 * i], bf16_bits_to_f32(w0 >> 16) / s[4 * i + 1],
                               bf16_bits_to_f32(w1 & 0xffffu) / s[4 * i + 2],
                               bf16_bits_to_f32(w1 >> 16) / s[4 * i + 3]);
  }
  return make_uint4(out[0], out[1], out[2], out[3]);
}

// Largest BF16 magnitude bits (finite values order like bits & 0x7fff).
__device__ __forceinline__ uint32_t amax16_bits(const uint4 lo, const uint4 hi) {
  const uint32_t in[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = max(m, max(in[i] & 0x7fffu, (in[i] >> 16) & 0x7fffu));
  return m;
}

// The 16 channel scales of chunk c (ks = the head's D channel scales).
__device__ __forceinline__ void load_chan_scales(const float* ks, int c, float (&kss)[16]) {
  const float4* kq4 = reinterpret_cast<const float4*>(ks + 16 * c);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 q = kq4[i];
    kss[4 * i] = q.x;
    kss[4 * i + 1] = q.y;
    kss[4 * i + 2] = q.z;
    kss[4 * i + 3] = q.w;
  }
}

// Chunk c of one (token, kv head) row pair, from its loaded inputs and channel
// scales, called by the `chunks` = D/16 consecutive lanes of a row together
// (lane c holds chunk c; the lanes form an aligned group of the wave, all
// active). Returns the row's V scale (every lane gets it).
template <int FMT>
__device__ __forceinline__ float put_fp8_chunk_kivi(const RowChunk& r, const float (&kss)[16], int c, int chunks,
                                                    int t16, uint8_t* kc, uint8_t* vc, int64_t base) {
  constexpr float MX = (FMT == KVQ_FP8_E4M3) ? 448.0f : 57344.0f;
  uint32_t m = amax16_bits(r.v0, r.v1);
  for (int off = 1; off < chunks; off <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  const float amax = bf16_bits_to_f32(m);
  const float vs = amax == 0.f ? 1.0f : amax / MX;  // IEEE binary32 division
  const Divisor vd = make_divisor(vs);
  const uint4 kq = quant_fp8_16_vec<FMT>(r.k0, r.k1, kss);
  const uint4 vq = quant_fp8_16<FMT>(r.v0, r.v1, vd);
  *reinterpret_cast<uint4*>(kc + base + 256 * c + 16 * t16) = kq;
  uint8_t* vb = vc + base + 1024 * (c >> 2) + 16 * (16 * (t16 >> 2)) + 4 * (c & 3) + (t16 & 3);
  const uint32_t vw[4] = {vq.x, vq.y, vq.z, vq.w};
#pragma unroll
  for (int e = 0; e < 16; ++e) vb[16 * e] = (uint8_t)(vw[e >> 2] >> (8 * (e & 3)));
  return vs;
}

template <int FMT>
__device__ __forceinline__ float put_fp8_chunk_kivi(const uint16_t* krow, const uint16_t* vrow, int c, int chunks,
                                                    int t16, const float* ks, uint8_t* kc, uint8_t* vc,
                                                    int64_t base) {
  float kss[16];
  load_chan_scales(ks, c, kss);
  return put_fp8_chunk_kivi<FMT>(load_row_chunk(krow, vrow, c), kss, c, chunks, t16, kc, vc, base);
}

// ------------------------------------------------------------- FP4 (E2M1) --
// Eight floats -> one dword of E2M1 codes (element 2i in the low nibble of byte i).
__device__ __forceinline__ uint32_t encode_e2m1x8(const float* f) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[0], f[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[2], f[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[4], f[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[6], f[7], 1.0f, 3);
  return w;
}

__device__ __forceinline__ void unpack_bf16x16(const uint4 lo, const uint4 hi, float* x, uint32_t& amax_bits) {
  const uint32_t in[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[2 * i] = bf16_bits_to_f32(in[i] & 0xffffu);
    x[2 * i + 1] = bf16_bits_to_f32(in[i] >> 16);
    m = max(m, in[i] & 0x7fffu);
    m = max(m, (in[i] >> 16) & 0x7fffu);
  }
  amax_bits = m;
}

// OCP shared exponent of a block whose largest magnitude has BF16 bits m:
// floor(log2 amax) - 2, clamped to [-127, 127]; -127 for an all-zero block.
__device__ __forceinline__ int mx_exponent(uint32_t m) {
  if (m == 0) return -127;
  const int ef = (int)(m >> 7);
  const int fl = ef > 0 ? ef - 127 : (31 - __clz((int)m)) - 133;  // subnormal: m * 2^-133
  const int e = fl - 2;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

__device__ __forceinline__ void quant_mx16(const uint4 lo, const uint4 hi, uint32_t& c0, uint32_t& c1,
                                           uint8_t& sc) {
  float x[16];
  uint32_t m;
  unpack_bf16x16(lo, hi, x, m);
  const int e = mx_exponent(m);
  const float mul = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e, a normal float
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] *= mul;                       // exact
  c0 = encode_e2m1x8(x);
  c1 = encode_e2m1x8(x + 8);
  sc = (uint8_t)(e + 127);
}

// Block b (elements 16b..16b+15) of one (token, kv head) row pair, from its
// loaded inputs; cbase / sbase address the row's 16-token tile of codes /
// scales.
__device__ __forceinline__ void put_mx16_block(const RowChunk& r, int b, int nb, int t16, uint8_t* kc, uint8_t* vc,
                                               uint8_t* ksc, uint8_t* vsc, int64_t cbase, int64_t sbase) {
  uint32_t k0, k1, v0, v1;
  uint8_t kse, vse;
  quant_mx16(r.k0, r.k1, k0, k1, kse);
  quant_mx16(r.v0, r.v1, v0, v1, vse);
  const int d0 = 16 * b;
  // K codes: byte 256*(d/32) + 16*t16 + (d%32)/2 -> 8 contiguous bytes
  *reinterpret_cast<uint2*>(kc + cbase + 256 * (d0 >> 5) + 16 * t16 + ((d0 & 31) >> 1)) = make_uint2(k0, k1);
  // V codes: byte 1024*(d/128) + 16*(16*(t16/4) + (d%128)/8) + 4*(t16%4) + (d%8)/2
  uint8_t* vb = vc + cbase + 1024 * (d0 >> 7) + 16 * (16 * (t16 >> 2)) + 4 * (t16 & 3);
  const int c8 = (d0 & 127) >> 3;
  *reinterpret_cast<uint32_t*>(vb + 16 * c8) = v0;
  *reinterpret_cast<uint32_t*>(vb + 16 * (c8 + 1)) = v1;
  // scales
  ksc[sbase + 32 * (b >> 1) + 2 * t16 + (b & 1)] = kse;
  vsc[sbase + 4 * (nb * (t16 >> 2) + b) + (t16 & 3)] = vse;
}

__device__ __forceinline__ void put_mx16_block(const uint16_t* krow, const uint16_t* vrow, int b, int nb, int t16,
                                               uint8_t* kc, uint8_t* vc, uint8_t* ksc, uint8_t* vsc, int64_t cbase,
                                               int64_t sbase) {
  put_mx16_block(load_row_chunk(krow, vrow, b), b, nb, t16, kc, vc, ksc, vsc, cbase, sbase);
}

// Block b of one MLA latent row (576 elements, 36 blocks); cb / sb address the
// row's 16-token tile of codes (4,608 B) / scales (576 B).
__device__ __forceinline__ void put_nvfp4_block(const uint16_t* row, int b, int t16, float g, uint8_t* cb,
                                                uint8_t* sb) {
  const uint4* kp = reinterpret_cast<const uint4*>(row + 16 * b);
  float x[16];
  uint32_t m;
  unpack_bf16x16(kp[0], kp[1], x, m);
  const float d6 = 6.0f * g;
  float s = bf16_bits_to_f32(m) / d6;         // >= 0
  s = fminf(s, 448.0f);
  const uint32_t sc = __builtin_amdgcn_cvt_pk_fp8_f32(s, 0.0f, 0, false) & 0xffu;
  const float sd = __builtin_amdgcn_cvt_pk_f32_fp8(sc, false)[0] * g;
  if (sd == 0.0f) {
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = __builtin_copysignf(0.0f, x[i]);
  } else {
    const Divisor dd = make_divisor(sd);
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = fminf(fmaxf(quotient(x[i], dd), -6.0f), 6.0f);
  }
  const uint32_t c0 = encode_e2m1x8(x), c1 = encode_e2m1x8(x + 8);
  // MLA tile layout: the 4-element groups of one token and token quad sit in
  // halfwords laid out for the decode kernel's loads (see include/kvq.h)
  const int g4 = t16 >> 2, tt = t16 & 3;
  int oc[4], os;
  if (b < 32) {
    const int w8 = b >> 2;
#pragma unroll
    for (int q = 0; q < 4; ++q) oc[q] = 2 * (((w8 * 4 + g4) * 16 + 4 * (b & 3) + q) * 4 + tt);
    os = 4 * ((w8 * 4 + g4) * 4 + (b & 3)) + tt;
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) oc[q] = 4096 + 2 * ((g4 * 16 + 4 * (b - 32) + q) * 4 + tt);
    os = 512 + 4 * (g4 * 4 + b - 32) + tt;
  }
  *reinterpret_cast<uint16_t*>(cb + oc[0]) = (uint16_t)(c0 & 0xffffu);
  *reinterpret_cast<uint16_t*>(cb + oc[1]) = (uint16_t)(c0 >> 16);
  *reinterpret_cast<uint16_t*>(cb + oc[2]) = (uint16_t)(c1 & 0xffffu);
  *reinterpret_cast<uint16_t*>(cb + oc[3]) = (uint16_t)(c1 >> 16);
  sb[os] = (uint8_t)sc;
}

}  // namespace kvq
