// kvq_store / kvq_compute_scale kernels for gfx950.
//
// Quantization rules (the pages: SGLang "Quantized KV Cache" page, sections
// "Supported formats" and "Scaling factors"; PR #21954 analysis page,
// NVFP4KVMethod / BlockFP4KVMethod and quantize_and_store):
//   FP8:   code = RNE(clamp(x / s, -max, max)) with x / s IEEE binary32
//   MX16:  per 16 elements e = floor(log2 amax) - 2 (clamped to [-127, 127]),
//          element = RNE_sat_E2M1(x * 2^-e), scale byte = e + 127
//   NVFP4: per 16 elements s = amax / fl32(6 g) -> E4M3 (saturating),
//          sd = E4M3(s) * g, element = RNE_sat_E2M1(x / sd) (signed zero if sd == 0)
// The gfx950 converts round to nearest even; the FP8 ones turn out-of-range
// inputs into NaN/Inf, so values are clamped to the format maximum first
// (which equals round-then-saturate). The E2M1 convert saturates by itself.
#include "kvq_internal.h"

namespace kvq {
namespace {

// ------------------------------------------------------------------ amax --
// Magnitude of a finite BF16 value orders like the integer (bits & 0x7fff).
template <bool VEC>
__global__ void __launch_bounds__(256) amax_partial_kernel(const uint16_t* __restrict__ x0, int64_t n0,
                                                           const uint16_t* __restrict__ x1, int64_t n1,
                                                           unsigned* __restrict__ partial) {
  unsigned m = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (int which = 0; which < 2; ++which) {
    const uint16_t* x = which ? x1 : x0;
    const int64_t n = which ? n1 : n0;
    if (x == nullptr || n <= 0) continue;
    int64_t done = 0;
    if (VEC) {
      const int64_t nv = n / 8;
      const uint4* xv = reinterpret_cast<const uint4*>(x);
      for (int64_t i = tid; i < nv; i += stride) {
        uint4 w = xv[i];
        uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          m = max(m, a[j] & 0x7fffu);
          m = max(m, (a[j] >> 16) & 0x7fffu);
        }
      }
      done = nv * 8;
    }
    for (int64_t i = done + tid; i < n; i += stride) m = max(m, (unsigned)(x[i] & 0x7fffu));
  }
  for (int off = 32; off > 0; off >>= 1) m = max(m, (unsigned)__shfl_xor((int)m, off, 64));
  __shared__ unsigned red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = max(max(red[0], red[1]), max(red[2], red[3]));
}

__global__ void __launch_bounds__(256) amax_final_kernel(const unsigned* __restrict__ partial, int n,
                                                         float fmt_div, float* __restrict__ out) {
  unsigned m = 0;
  for (int i = threadIdx.x; i < n; i += blockDim.x) m = max(m, partial[i]);
  for (int off = 32; off > 0; off >>= 1) m = max(m, (unsigned)__shfl_xor((int)m, off, 64));
  __shared__ unsigned red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = max(max(red[0], red[1]), max(red[2], red[3]));
    const float amax = bf16_bits_to_f32(m);
    out[0] = (amax == 0.f) ? 1.0f : amax / fmt_div;  // IEEE binary32 division
  }
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
__device__ __forceinline__ uint4 quant_fp8_16(const uint4 lo, const uint4 hi, float s) {
  const uint32_t in[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  uint32_t out[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w0 = in[2 * i], w1 = in[2 * i + 1];
    out[i] = encode_fp8x4<FMT>(bf16_bits_to_f32(w0 & 0xffffu) / s, bf16_bits_to_f32(w0 >> 16) / s,
                               bf16_bits_to_f32(w1 & 0xffffu) / s, bf16_bits_to_f32(w1 >> 16) / s);
  }
  return make_uint4(out[0], out[1], out[2], out[3]);
}

// one thread per (token, kv head, 16-element chunk)
template <int FMT>
__global__ void __launch_bounds__(256) store_fp8_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const int64_t* __restrict__ slots,
    int32_t n_tok, int hkv, int dim, int page_size, int64_t capacity, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, uint8_t* __restrict__ kc, uint8_t* __restrict__ vc,
    int64_t block_bytes) {
  const int chunks = dim / 16;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)n_tok * hkv * chunks) return;
  const int c = (int)(gid % chunks);
  const int64_t th = gid / chunks;
  const int h = (int)(th % hkv);
  const int64_t tok = th / hkv;
  const int64_t slot = slots[tok];
  if (slot < 0 || slot >= capacity) return;
  const int64_t page = slot / page_size;
  const int t = (int)(slot % page_size);
  const int t16 = t & 15;
  const float ks = k_scale ? k_scale[0] : 1.0f;
  const float vs = v_scale ? v_scale[0] : 1.0f;
  const int64_t row = (tok * hkv + h) * dim + c * 16;
  const uint4* kp = reinterpret_cast<const uint4*>(k + row);
  const uint4* vp = reinterpret_cast<const uint4*>(v + row);
  const uint4 kq = quant_fp8_16<FMT>(kp[0], kp[1], ks);
  const uint4 vq = quant_fp8_16<FMT>(vp[0], vp[1], vs);
  const int64_t base = (page * hkv + h) * block_bytes + (int64_t)(t >> 4) * 16 * dim;
  // K: the 16 elements of chunk c are 16 contiguous bytes
  *reinterpret_cast<uint4*>(kc + base + 256 * c + 16 * t16) = kq;
  // V: element d = 16c + r at 1024*(d/64) + 16*(16*(t16/4) + r) + 4*(c%4) + t16%4
  uint8_t* vb = vc + base + 1024 * (c >> 2) + 16 * (16 * (t16 >> 2)) + 4 * (c & 3) + (t16 & 3);
  const uint32_t vw[4] = {vq.x, vq.y, vq.z, vq.w};
#pragma unroll
  for (int r = 0; r < 16; ++r) vb[16 * r] = (uint8_t)(vw[r >> 2] >> (8 * (r & 3)));
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

// one thread per (token, kv head, 16-element block)
__global__ void __launch_bounds__(256) store_mx16_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const int64_t* __restrict__ slots,
    int32_t n_tok, int hkv, int dim, int page_size, int64_t capacity, uint8_t* __restrict__ kc,
    uint8_t* __restrict__ vc, uint8_t* __restrict__ ksc, uint8_t* __restrict__ vsc, int64_t code_block,
    int64_t scale_block) {
  const int nb = dim / 16;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)n_tok * hkv * nb) return;
  const int b = (int)(gid % nb);
  const int64_t th = gid / nb;
  const int h = (int)(th % hkv);
  const int64_t tok = th / hkv;
  const int64_t slot = slots[tok];
  if (slot < 0 || slot >= capacity) return;
  const int64_t page = slot / page_size;
  const int t = (int)(slot % page_size);
  const int t16 = t & 15;
  const int64_t row = (tok * hkv + h) * dim + b * 16;
  const uint4* kp = reinterpret_cast<const uint4*>(k + row);
  const uint4* vp = reinterpret_cast<const uint4*>(v + row);
  uint32_t k0, k1, v0, v1;
  uint8_t kse, vse;
  quant_mx16(kp[0], kp[1], k0, k1, kse);
  quant_mx16(vp[0], vp[1], v0, v1, vse);
  const int64_t cbase = (page * hkv + h) * code_block + (int64_t)(t >> 4) * 8 * dim;
  const int64_t sbase = (page * hkv + h) * scale_block + (int64_t)(t >> 4) * dim;
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

// ----------------------------------------------------------------- NVFP4 --
// one thread per (token, 16-element block) of the MLA latent row
__global__ void __launch_bounds__(256) store_nvfp4_kernel(
    const uint16_t* __restrict__ k, const int64_t* __restrict__ slots, int32_t n_tok, int dim,
    int page_size, int64_t capacity, const float* __restrict__ g_scale, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales) {
  const int nb = dim / 16;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)n_tok * nb) return;
  const int b = (int)(gid % nb);
  const int64_t tok = gid / nb;
  const int64_t slot = slots[tok];
  if (slot < 0 || slot >= capacity) return;
  const uint4* kp = reinterpret_cast<const uint4*>(k + tok * dim + b * 16);
  float x[16];
  uint32_t m;
  unpack_bf16x16(kp[0], kp[1], x, m);
  const float g = g_scale[0];
  const float d6 = 6.0f * g;
  float s = bf16_bits_to_f32(m) / d6;         // >= 0
  s = fminf(s, 448.0f);
  const uint32_t sc = __builtin_amdgcn_cvt_pk_fp8_f32(s, 0.0f, 0, false) & 0xffu;
  const float sd = __builtin_amdgcn_cvt_pk_f32_fp8(sc, false)[0] * g;
  if (sd == 0.0f) {
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = __builtin_copysignf(0.0f, x[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = fminf(fmaxf(x[i] / sd, -6.0f), 6.0f);
  }
  const uint32_t c0 = encode_e2m1x8(x), c1 = encode_e2m1x8(x + 8);
  // MLA tile layout (16 tokens, 4608 code + 576 scale bytes): the 8-element
  // groups of one token and lane group sit in dwords laid out for the decode
  // kernel's loads (see include/kvq.h)
  const int page = (int)(slot / page_size);
  const int t = (int)(slot % page_size);
  const int t16 = t & 15, g4 = t16 >> 2, tt = t16 & 3;
  uint8_t* cb = codes + (int64_t)page * page_size * (dim / 2) + (int64_t)(t >> 4) * 16 * (dim / 2);
  uint8_t* sb = scales + (int64_t)page * page_size * nb + (int64_t)(t >> 4) * 16 * nb;
  // 16 elements = four 4-element groups, 2 code bytes each
  int64_t oc[4], os;
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

}  // namespace
}  // namespace kvq

using namespace kvq;

hipError_t kvq_launch_amax(const uint16_t* x0, int64_t n0, const uint16_t* x1, int64_t n1, unsigned* scratch,
                           float fmt_div, float* scale_out, hipStream_t s) {
  const int64_t n = n0 + n1;
  int blocks = (int)((n + 256 * 32 - 1) / (256 * 32));
  blocks = blocks < 1 ? 1 : (blocks > kAmaxBlocks ? kAmaxBlocks : blocks);
  const bool vec = ((reinterpret_cast<uintptr_t>(x0) & 15) == 0) && ((reinterpret_cast<uintptr_t>(x1) & 15) == 0);
  if (vec)
    amax_partial_kernel<true><<<blocks, 256, 0, s>>>(x0, n0, x1, n1, scratch);
  else
    amax_partial_kernel<false><<<blocks, 256, 0, s>>>(x0, n0, x1, n1, scratch);
  amax_final_kernel<<<1, 256, 0, s>>>(scratch, blocks, fmt_div, scale_out);
  return hipGetLastError();
}

hipError_t kvq_launch_store(const kvq_cache* c, const uint16_t* k, const uint16_t* v, const int64_t* slots,
                            int32_t n, const float* k_scale, const float* v_scale, hipStream_t s) {
  const kvq_cache_desc& d = c->desc;
  const int64_t capacity = d.num_pages * (int64_t)d.page_size;
  uint8_t* base = c->base;
  const kvq_layout& L = c->layout;
  if (d.dtype == KVQ_FP8_E4M3 || d.dtype == KVQ_FP8_E5M2) {
    const int64_t threads = (int64_t)n * d.num_kv_heads * (d.head_dim / 16);
    const int grid = (int)((threads + 255) / 256);
    if (d.dtype == KVQ_FP8_E4M3)
      store_fp8_kernel<KVQ_FP8_E4M3><<<grid, 256, 0, s>>>(k, v, slots, n, d.num_kv_heads, d.head_dim, d.page_size,
                                                         capacity, k_scale, v_scale, base + L.k_codes_offset,
                                                         base + L.v_codes_offset, c->code_block_bytes);
    else
      store_fp8_kernel<KVQ_FP8_E5M2><<<grid, 256, 0, s>>>(k, v, slots, n, d.num_kv_heads, d.head_dim, d.page_size,
                                                         capacity, k_scale, v_scale, base + L.k_codes_offset,
                                                         base + L.v_codes_offset, c->code_block_bytes);
  } else if (d.dtype == KVQ_FP4_MX16) {
    const int64_t threads = (int64_t)n * d.num_kv_heads * (d.head_dim / 16);
    const int grid = (int)((threads + 255) / 256);
    store_mx16_kernel<<<grid, 256, 0, s>>>(k, v, slots, n, d.num_kv_heads, d.head_dim, d.page_size, capacity,
                                           base + L.k_codes_offset, base + L.v_codes_offset,
                                           base + L.k_scales_offset, base + L.v_scales_offset, c->code_block_bytes,
                                           c->scale_block_bytes);
  } else {
    const int64_t threads = (int64_t)n * (d.head_dim / 16);
    const int grid = (int)((threads + 255) / 256);
    store_nvfp4_kernel<<<grid, 256, 0, s>>>(k, slots, n, d.head_dim, d.page_size, capacity, k_scale,
                                            base + L.k_codes_offset, base + L.k_scales_offset);
  }
  return hipGetLastError();
}
