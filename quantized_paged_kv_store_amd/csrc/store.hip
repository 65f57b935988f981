// kvq_store / kvq_compute_scale kernels for gfx950. The per-chunk quantize-
// and-place routines (and the quantization rules) are in store_row.h.
#include "store_row.h"

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

// Per-KV-head amax of x[rows][hkv][dim] BF16 (16-byte aligned rows): block
// (bx, h) reduces head h over 8-element groups bx, bx + gridDim.x, ...
__global__ void __launch_bounds__(256) amax_head_partial_kernel(const uint16_t* __restrict__ x0, int64_t rows0,
                                                                const uint16_t* __restrict__ x1, int64_t rows1,
                                                                int hkv, int dim, unsigned* __restrict__ partial) {
  const int h = blockIdx.y;
  const int gpr = dim / 8;
  unsigned m = 0;
  for (int which = 0; which < 2; ++which) {
    const uint16_t* x = which ? x1 : x0;
    const int64_t rows = which ? rows1 : rows0;
    if (x == nullptr || rows <= 0) continue;
    const int64_t n = rows * gpr;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
      const int64_t r = i / gpr;
      const int q = (int)(i - r * gpr);
      const uint4 w = *reinterpret_cast<const uint4*>(x + (r * hkv + h) * dim + 8 * q);
      const uint32_t a4[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        m = max(m, a4[j] & 0x7fffu);
        m = max(m, (a4[j] >> 16) & 0x7fffu);
      }
    }
  }
  for (int off = 32; off > 0; off >>= 1) m = max(m, (unsigned)__shfl_xor((int)m, off, 64));
  __shared__ unsigned red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) partial[h * gridDim.x + blockIdx.x] = max(max(red[0], red[1]), max(red[2], red[3]));
}

// out[h] = amax_h / fmt_div (1.0 for an all-zero head), one block per head
__global__ void __launch_bounds__(256) amax_head_final_kernel(const unsigned* __restrict__ partial, int n,
                                                              float fmt_div, float* __restrict__ out) {
  const int h = blockIdx.x;
  unsigned m = 0;
  for (int i = threadIdx.x; i < n; i += blockDim.x) m = max(m, partial[h * n + i]);
  for (int off = 32; off > 0; off >>= 1) m = max(m, (unsigned)__shfl_xor((int)m, off, 64));
  __shared__ unsigned red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = max(max(red[0], red[1]), max(red[2], red[3]));
    const float amax = bf16_bits_to_f32(m);
    out[h] = (amax == 0.f) ? 1.0f : amax / fmt_div;  // IEEE binary32 division
  }
}

// Per-(kv head, channel) amax of x[rows][ng * 8] BF16 for KIVI-style K
// scales: each thread keeps the running max of its 8 columns over a stride of
// rows, then one atomic max per column into acc (zeroed first by
// zero_u32_kernel; a fill kernel rather than a memset keeps the calibration
// capturable in a graph).
__global__ void __launch_bounds__(256) zero_u32_kernel(unsigned* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

__global__ void __launch_bounds__(256) amax_chan_partial_kernel(const uint16_t* __restrict__ x0, int64_t rows0,
                                                                const uint16_t* __restrict__ x1, int64_t rows1,
                                                                int ng, unsigned* __restrict__ acc) {
  const int q = blockIdx.y * blockDim.x + threadIdx.x;
  if (q >= ng) return;
  unsigned m[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
  for (int which = 0; which < 2; ++which) {
    const uint16_t* x = which ? x1 : x0;
    const int64_t rows = which ? rows1 : rows0;
    if (x == nullptr || rows <= 0) continue;
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
      const uint4 w = *reinterpret_cast<const uint4*>(x + (r * ng + q) * 8);
      const uint32_t a4[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        m[2 * j] = max(m[2 * j], a4[j] & 0x7fffu);
        m[2 * j + 1] = max(m[2 * j + 1], (a4[j] >> 16) & 0x7fffu);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (m[j]) atomicMax(acc + 8 * q + j, m[j]);
}

// out[i] = amax_i / fmt_div (1.0 for an all-zero column)
__global__ void __launch_bounds__(256) amax_chan_final_kernel(const unsigned* __restrict__ acc, int n, float fmt_div,
                                                              float* __restrict__ out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float amax = bf16_bits_to_f32(acc[i]);
  out[i] = (amax == 0.f) ? 1.0f : amax / fmt_div;  // IEEE binary32 division
}

// Page and position of a cache slot (slot / page_size, slot % page_size):
// a shift and a mask when the page size is a power of two (a kernel argument,
// so the branch is uniform), else a 64-bit division. slot >= 0.
__device__ __forceinline__ void slot_place(int64_t slot, int page_size, int64_t& page, int& t) {
  if ((page_size & (page_size - 1)) == 0) {
    page = slot >> __builtin_ctz(page_size);
    t = (int)(slot & (page_size - 1));
  } else {
    page = slot / page_size;
    t = (int)(slot - page * page_size);
  }
}

// The store kernels launch one thread per (token, [kv head,] 16-element piece)
// and the C ABI keeps such a launch below 2^32 threads, so the thread's split
// into token, head and piece runs in 32-bit arithmetic.

// one thread per (token, kv head, 16-element chunk); the D/16 chunks of a row
// are consecutive lanes (the KIVI V row amax is reduced across them). A V
// lane word holds one element of four consecutive tokens (t16 = 4g..4g+3):
// when the four tokens of this token's group are the four consecutive list
// entries around it (a prefill or chunk), their threads write whole words,
// each thread four elements of all four tokens; otherwise every token writes
// its own bytes, so the rest of a word is never touched.
template <int FMT>
__global__ void __launch_bounds__(256) store_fp8_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const int64_t* __restrict__ slots,
    int32_t n_tok, int hkv, int dim, int page_size, int64_t capacity, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, int mode, uint8_t* __restrict__ kc, uint8_t* __restrict__ vc,
    int64_t block_bytes, uint8_t* __restrict__ vts, int64_t vts_block) {
  const int chunks = dim / 16;
  const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (uint32_t)n_tok * (uint32_t)hkv * (uint32_t)chunks) return;
  const int c = (int)(gid % (uint32_t)chunks);
  const uint32_t th = gid / (uint32_t)chunks;
  const int h = (int)(th % (uint32_t)hkv);
  const int64_t tok = th / (uint32_t)hkv;
  const int64_t slot = slots[tok];
  if (slot < 0 || slot >= capacity) return;
  int64_t page;
  int t;
  slot_place(slot, page_size, page, t);
  const int t16 = t & 15;
  const int64_t row = (tok * hkv + h) * dim;
  const int64_t base = (page * hkv + h) * block_bytes + (int64_t)(t >> 4) * 16 * dim;
  if (mode == KVQ_SCALE_KIVI) {
    const float vs = put_fp8_chunk_kivi<FMT>(k + row, v + row, c, chunks, t16, k_scale + (int64_t)h * dim, kc, vc,
                                             base);
    if (c == 0) reinterpret_cast<float*>(vts + (page * hkv + h) * vts_block)[t] = vs;
    return;
  }
  const int si = mode == KVQ_SCALE_HEAD ? h : 0;
  const Divisor ks = make_divisor(k_scale ? k_scale[si] : 1.0f);
  const Divisor vs = make_divisor(v_scale ? v_scale[si] : 1.0f);
  const int i = t16 & 3;
  const int64_t j0 = tok - i;  // list position of the group's first token, if the group is whole
  bool whole = j0 >= 0 && j0 + 3 < n_tok;
  if (whole) {
#pragma unroll
    for (int u = 0; u < 4; ++u) whole = whole && slots[j0 + u] == slot - i + u;
  }
  if (!whole) {
    put_fp8_chunk<FMT>(k + row, v + row, c, t16, ks, vs, kc, vc, base);
    return;
  }
  const uint4* kp = reinterpret_cast<const uint4*>(k + row + 16 * c);
  *reinterpret_cast<uint4*>(kc + base + 256 * c + 16 * t16) = quant_fp8_16<FMT>(kp[0], kp[1], ks);
  put_fp8_v_group<FMT>(v + (j0 * hkv + h) * dim, (int64_t)hkv * dim, c, t16 >> 2, i, vs, vc, base);
}

// one thread per (token, kv head, 16-element block)
__global__ void __launch_bounds__(256) store_mx16_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const int64_t* __restrict__ slots,
    int32_t n_tok, int hkv, int dim, int page_size, int64_t capacity, uint8_t* __restrict__ kc,
    uint8_t* __restrict__ vc, uint8_t* __restrict__ ksc, uint8_t* __restrict__ vsc, int64_t code_block,
    int64_t scale_block) {
  const int nb = dim / 16;
  const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (uint32_t)n_tok * (uint32_t)hkv * (uint32_t)nb) return;
  const int b = (int)(gid % (uint32_t)nb);
  const uint32_t th = gid / (uint32_t)nb;
  const int h = (int)(th % (uint32_t)hkv);
  const int64_t tok = th / (uint32_t)hkv;
  const int64_t slot = slots[tok];
  if (slot < 0 || slot >= capacity) return;
  int64_t page;
  int t;
  slot_place(slot, page_size, page, t);
  const int t16 = t & 15;
  const int64_t row = (tok * hkv + h) * dim;
  const int64_t cbase = (page * hkv + h) * code_block + (int64_t)(t >> 4) * 8 * dim;
  const int64_t sbase = (page * hkv + h) * scale_block + (int64_t)(t >> 4) * dim;
  put_mx16_block(k + row, v + row, b, nb, t16, kc, vc, ksc, vsc, cbase, sbase);
}

// ----------------------------------------------------------------- NVFP4 --
// one thread per (token, 16-element block) of the MLA latent row
__global__ void __launch_bounds__(256) store_nvfp4_kernel(
    const uint16_t* __restrict__ k, const int64_t* __restrict__ slots, int32_t n_tok, int dim,
    int page_size, int64_t capacity, const float* __restrict__ g_scale, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales) {
  const int nb = dim / 16;
  const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (uint32_t)n_tok * (uint32_t)nb) return;
  const int b = (int)(gid % (uint32_t)nb);
  const int64_t tok = gid / (uint32_t)nb;
  const int64_t slot = slots[tok];
  if (slot < 0 || slot >= capacity) return;
  int64_t page;
  int t;
  slot_place(slot, page_size, page, t);
  uint8_t* cb = codes + page * page_size * (dim / 2) + (int64_t)(t >> 4) * 16 * (dim / 2);
  uint8_t* sb = scales + page * page_size * nb + (int64_t)(t >> 4) * 16 * nb;
  put_nvfp4_block(k + tok * dim, b, t & 15, g_scale[0], cb, sb);
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

hipError_t kvq_launch_amax_heads(const uint16_t* x0, int64_t rows0, const uint16_t* x1, int64_t rows1, int hkv,
                                 int dim, unsigned* scratch, float fmt_div, float* scale_out, hipStream_t s) {
  // at most kAmaxBlocks partials in the scratch buffer, split over the heads
  const int64_t items = (rows0 + rows1) * (dim / 8);
  int per_head = (int)((items + 256 * 16 - 1) / (256 * 16));
  const int cap = kAmaxBlocks / hkv;
  per_head = per_head < 1 ? 1 : (per_head > cap ? cap : per_head);
  if (cap < 1) return hipErrorInvalidValue;
  amax_head_partial_kernel<<<dim3(per_head, hkv), 256, 0, s>>>(x0, rows0, x1, rows1, hkv, dim, scratch);
  amax_head_final_kernel<<<hkv, 256, 0, s>>>(scratch, per_head, fmt_div, scale_out);
  return hipGetLastError();
}

hipError_t kvq_launch_amax_channels(const uint16_t* x0, int64_t rows0, const uint16_t* x1, int64_t rows1, int cols,
                                   unsigned* scratch, float fmt_div, float* scale_out, hipStream_t s) {
  const int ng = cols / 8;
  const int64_t rows = rows0 + rows1;
  int gx = (int)((rows + 63) / 64);
  gx = gx < 1 ? 1 : (gx > 256 ? 256 : gx);
  zero_u32_kernel<<<(cols + 255) / 256, 256, 0, s>>>(scratch, cols);
  amax_chan_partial_kernel<<<dim3(gx, (ng + 255) / 256), 256, 0, s>>>(x0, rows0, x1, rows1, ng, scratch);
  amax_chan_final_kernel<<<(cols + 255) / 256, 256, 0, s>>>(scratch, cols, fmt_div, scale_out);
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
                                                         capacity, k_scale, v_scale, d.scale_mode,
                                                         base + L.k_codes_offset, base + L.v_codes_offset,
                                                         c->code_block_bytes, base + L.v_scales_offset,
                                                         c->scale_block_bytes);
    else
      store_fp8_kernel<KVQ_FP8_E5M2><<<grid, 256, 0, s>>>(k, v, slots, n, d.num_kv_heads, d.head_dim, d.page_size,
                                                         capacity, k_scale, v_scale, d.scale_mode,
                                                         base + L.k_codes_offset, base + L.v_codes_offset,
                                                         c->code_block_bytes, base + L.v_scales_offset,
                                                         c->scale_block_bytes);
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
