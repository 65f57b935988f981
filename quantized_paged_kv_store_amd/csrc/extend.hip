// Extend (chunked prefill) attention over a quantized prefix, gfx950.
//
// The PR #21954 analysis page ("code analysis") has dequantize_prev_kv turn
// the FP4 prefix of a sequence into FP8 E4M3 workspaces because only FP8
// prefill kernels exist; this is that prefill kernel. The C new tokens of a
// sequence attend to its L0 prefix tokens through the E4M3 rows (value =
// code * s_k or s_v, the workspace's per-tensor scales) and to their own BF16
// K/V causally; the G query heads of a KV head share its K/V (GQA).
//
// Work split: one workgroup (8 waves, two per SIMD) per (sequence, KV head,
// tile of 256 / G chunk tokens): 256 query rows (token, head), 32 per wave.
// Two waves per SIMD let one wave's softmax run under the other's matrix
// products; that needs <= 256 registers per wave, which holds because the
// operands are read from LDS just in time through short rings instead of
// being hoisted, and the next block's staging is spread over 512 threads.
// Block ids are remapped so that all tiles of one (sequence, KV head) run on
// one XCD (the 8 XCDs take block ids round robin): they stream the same
// prefix, which then stays in that XCD's L2.
//
// Per 64-key block, staged in LDS (K and V row-major, K as bf16, V as fp16
// codes for the prefix and bf16 values for the chunk; four buffers, a block
// converted and stored two blocks before it is used, one workgroup barrier
// per two blocks):
//   S^T[key][row]  = K[key][:] . Q^T[:][row]   v_mfma_f32_32x32x16_bf16
//                    (E4M3 codes and BF16 values are exact in bf16; s_k and
//                    sm_scale multiply the scores)
//   online softmax per query row: the row is one lane column, so the block
//   maximum takes one cross-lane step (the two halves of the wave)
//   O^T[d][row]   += V^T[d][key] . P^T[key][row]
//                    prefix: v_mfma_f32_32x32x16_f16 (E4M3 exact in fp16, P
//                    carries 2^15); s_v multiplies O once after the prefix
//                    chunk: bf16 MFMAs with P split hi + lo (BF16 values are
//                    not all representable in fp16)
// P^T goes from the score registers straight into the B operand: within each
// 16-key step, lane half h holds keys {4h..4h+3, 8+4h..8+4h+3}; the V^T
// operand reads the same keys with transposing LDS reads (ds_read_b64_tr_b16).
// The softmax reference maximum moves only when a score exceeds it by more
// than 2^8 (P = 2^(s - ref + 7) <= 2^15 stays in fp16 range), so the
// accumulator rescale is rare.
#include <type_traits>

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int XD = 128;             // head dim
constexpr int XKB = 64;             // keys per block
constexpr int XROWS = kExtendRows;  // query rows per workgroup
constexpr int XWAVES = 8;           // waves per workgroup (two per SIMD)
constexpr int XRB = XROWS / (32 * XWAVES);  // 32-row blocks per wave (each K / V^T fragment feeds all of them)
constexpr int XTHREADS = 64 * XWAVES;
constexpr int XPI = XKB * 8 / XTHREADS;   // 16-byte prefix chunks (K and V each) per thread and block
constexpr int XCI = XKB * 16 / XTHREADS;  // 16-byte chunk chunks (K and V each) per thread and block
static_assert(XRB >= 1 && XPI >= 1 && XCI >= 1, "workgroup shape");
constexpr int XK_STRIDE = XD + 8;   // 16-bit elements per LDS K row: 272 B, rows 4 banks apart
constexpr int XV_STRIDE = XD + 32;  // per LDS V row: 320 B, rows 16 banks apart (transposed reads)
constexpr float kXNegInf = -__builtin_huge_valf();
constexpr float kXPBias = 7.0f;     // P = 2^(s - ref + 7)
constexpr float kXLazy = 8.0f;      // the reference moves when a score exceeds it by this
constexpr float kXLog2e = 1.4426950408889634f;
constexpr float kXLn2 = 0.6931471805599453f;

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

__device__ __forceinline__ void split_bf16(const float* p, bf16x8& hi, bf16x8& lo) {
  float r[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = p[i] - (float)(__bf16)p[i];
  const u32x4 h = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
  const u32x4 l = {pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]), pack_bf16x2(r[4], r[5]), pack_bf16x2(r[6], r[7])};
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}

// transposed 4 x 16-bit LDS read: in each 16-lane group, lane i receives
// element i%4 of the 8-byte reads of lanes i/4 + 4e (e = 0..3)
__device__ __forceinline__ u32x2 lds_tr16(const uint16_t* p) {
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(u32x2, r);
}

// POW2: the workspace page size is a power of two (page and offset of a key
// by shift and mask instead of a division)
template <bool POW2>
__global__ void __launch_bounds__(XTHREADS, 1) extend_attn_kernel(const ExtendArgs a) {
  const int nwg = gridDim.x;  // a multiple of 8
  const int work = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
  if (work >= a.n_work) return;
  const int qt = work % a.q_tiles;
  const int kvh = (work / a.q_tiles) % a.hkv;
  const int b = work / (a.q_tiles * a.hkv);
  const int G = a.group, TT = XROWS / G, P = a.page_size;

  // device data is clamped, never trusted
  const int q0 = min(max(a.cu_q[b], 0), a.total_q);
  const int q1 = min(max(a.cu_q[b + 1], q0), a.total_q);
  const int C = min(q1 - q0, a.max_chunk);
  const int t0 = qt * TT;
  if (t0 >= C) return;
  const int po = a.page_off[b];
  int L0 = max(a.prefix_len[b], 0);
  L0 = (po < 0 || po >= a.n_pages) ? 0 : (int)min((int64_t)L0, (int64_t)(a.n_pages - po) * P);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 31, hh = lane >> 5;
  // this lane's query rows: 32 XRB wave + 32 rb + j for its XRB row blocks
  int tok[XRB], head[XRB];
  bool rv[XRB];
#pragma unroll
  for (int rb = 0; rb < XRB; ++rb) {
    const int row = 32 * XRB * wave + 32 * rb + j;
    tok[rb] = t0 + row / G;
    head[rb] = kvh * G + row % G;
    rv[rb] = tok[rb] < C;
  }

  // Q^T operands: lane (row, half hh) holds d = 16 ks + 8 hh .. + 7 (zero for
  // rows past the chunk: their scores are 0 and their outputs not written)
  bf16x8 qf[XRB][XD / 16];
#pragma unroll
  for (int rb = 0; rb < XRB; ++rb) {
    const uint16_t* qp = a.q + ((int64_t)(q0 + (rv[rb] ? tok[rb] : 0)) * a.hq + head[rb]) * XD + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < XD / 16; ++ks) {
      uint4 w = rv[rb] ? *reinterpret_cast<const uint4*>(qp + 16 * ks) : make_uint4(0, 0, 0, 0);
      qf[rb][ks] = __builtin_bit_cast(bf16x8, w);
    }
  }

  const int nb0 = (L0 + XKB - 1) / XKB;
  const int tl = min(t0 + TT, C) - 1;  // last chunk token of this tile
  const int nb = nb0 + tl / XKB + 1;

  // four block buffers: block kb lives in buffer kb % 4, staged two blocks
  // ahead, and the workgroup meets at a barrier after every odd block
  __shared__ __attribute__((aligned(16))) uint16_t sk[4][XKB * XK_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t sv[4][XKB * XV_STRIDE];

  // global -> registers: a prefix block is 2 + 2 E4M3 chunks of 16 bytes
  // (16 elements) per thread, a chunk block 4 + 4 BF16 chunks (8 elements);
  // keys past the prefix or the chunk read zeros (only blocks that reach
  // past the end check keys). Every register is written on both paths.
  // Thread tid loads keys tid/8 + 32 i (prefix) or tid/16 + 16 i (chunk).
  const int pkey = tid >> 3, pcol = 16 * (tid & 7);
  const int ckey = tid >> 4, ccol = 8 * (tid & 15);
  const int pshift = __builtin_ctz(P);  // used when P is a power of two
  const int64_t crow = (int64_t)a.hkv * XD;  // elements between consecutive chunk tokens
  uint4 rk[XCI], rvv[XCI];
  auto load_block = [&](int kb) {
    if (kb < nb0) {
      const bool full = (kb + 1) * XKB <= L0;
#pragma unroll
      for (int i = 0; i < XPI; ++i) {
        const int t = kb * XKB + pkey + (XTHREADS / 8) * i;
        const int pg = POW2 ? (t >> pshift) : t / P;
        const int off = t - pg * P;
        const int64_t r = ((int64_t)(po + pg) * a.hkv + kvh) * P + off;
        const uint4* kp = reinterpret_cast<const uint4*>(a.dq_k + r * XD + pcol);
        const uint4* vp = reinterpret_cast<const uint4*>(a.dq_v + r * XD + pcol);
        if (full) {
          rk[i] = *kp;
          rvv[i] = *vp;
        } else {
          rk[i] = t < L0 ? *kp : make_uint4(0, 0, 0, 0);
          rvv[i] = t < L0 ? *vp : make_uint4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int i = XPI; i < XCI; ++i) rk[i] = rvv[i] = make_uint4(0, 0, 0, 0);
    } else {
      const int tb = (kb - nb0) * XKB;
      const bool full = tb + XKB <= C;
      const int64_t e0 = (int64_t)(q0 + tb + ckey) * crow + (int64_t)kvh * XD + ccol;
#pragma unroll
      for (int i = 0; i < XCI; ++i) {
        const int t = tb + ckey + (XTHREADS / 16) * i;
        const uint4* kp = reinterpret_cast<const uint4*>(a.k_new + e0 + (XTHREADS / 16) * i * crow);
        const uint4* vp = reinterpret_cast<const uint4*>(a.v_new + e0 + (XTHREADS / 16) * i * crow);
        if (full) {
          rk[i] = *kp;
          rvv[i] = *vp;
        } else {
          rk[i] = t < C ? *kp : make_uint4(0, 0, 0, 0);
          rvv[i] = t < C ? *vp : make_uint4(0, 0, 0, 0);
        }
      }
    }
  };
  // registers -> LDS buffer: K rows as bf16; V rows as fp16 codes (prefix) or
  // bf16 values (chunk)
  auto store_block = [&](int kb, uint16_t* kd, uint16_t* vd) {
    if (kb < nb0) {
#pragma unroll
      for (int i = 0; i < XPI; ++i) {
        const int c = tid + XTHREADS * i, key = c >> 3, dc = c & 7;
        const uint4 k = rk[i], v = rvv[i];
        const uint4 k0 = {fp8x2_to_bf16x2<KVQ_FP8_E4M3, false>(k.x), fp8x2_to_bf16x2<KVQ_FP8_E4M3, true>(k.x),
                          fp8x2_to_bf16x2<KVQ_FP8_E4M3, false>(k.y), fp8x2_to_bf16x2<KVQ_FP8_E4M3, true>(k.y)};
        const uint4 k1 = {fp8x2_to_bf16x2<KVQ_FP8_E4M3, false>(k.z), fp8x2_to_bf16x2<KVQ_FP8_E4M3, true>(k.z),
                          fp8x2_to_bf16x2<KVQ_FP8_E4M3, false>(k.w), fp8x2_to_bf16x2<KVQ_FP8_E4M3, true>(k.w)};
        const uint4 v0 = {fp8x2_to_f16x2<KVQ_FP8_E4M3, false>(v.x), fp8x2_to_f16x2<KVQ_FP8_E4M3, true>(v.x),
                          fp8x2_to_f16x2<KVQ_FP8_E4M3, false>(v.y), fp8x2_to_f16x2<KVQ_FP8_E4M3, true>(v.y)};
        const uint4 v1 = {fp8x2_to_f16x2<KVQ_FP8_E4M3, false>(v.z), fp8x2_to_f16x2<KVQ_FP8_E4M3, true>(v.z),
                          fp8x2_to_f16x2<KVQ_FP8_E4M3, false>(v.w), fp8x2_to_f16x2<KVQ_FP8_E4M3, true>(v.w)};
        *reinterpret_cast<uint4*>(kd + key * XK_STRIDE + 16 * dc) = k0;
        *reinterpret_cast<uint4*>(kd + key * XK_STRIDE + 16 * dc + 8) = k1;
        *reinterpret_cast<uint4*>(vd + key * XV_STRIDE + 16 * dc) = v0;
        *reinterpret_cast<uint4*>(vd + key * XV_STRIDE + 16 * dc + 8) = v1;
      }
    } else {
#pragma unroll
      for (int i = 0; i < XCI; ++i) {
        const int c = tid + XTHREADS * i, key = c >> 4, dc = c & 15;
        *reinterpret_cast<uint4*>(kd + key * XK_STRIDE + 8 * dc) = rk[i];
        *reinterpret_cast<uint4*>(vd + key * XV_STRIDE + 8 * dc) = rvv[i];
      }
    }
  };

  const float sm2 = a.sm_scale * kXLog2e;
  const float skv = a.s_k ? a.s_k[0] : 1.0f;
  const float svv = a.s_v ? a.s_v[0] : 1.0f;
  f32x16 o[XRB][XD / 32];  // O^T per row block: elements 32 dt .. +31 x 32 rows
#pragma unroll
  for (int rb = 0; rb < XRB; ++rb)
#pragma unroll
    for (int dt = 0; dt < XD / 32; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[rb][dt][v] = 0.f;
  float m_ref[XRB], l_run[XRB];
#pragma unroll
  for (int rb = 0; rb < XRB; ++rb) {
    m_ref[rb] = kXNegInf;
    l_run[rb] = 0.f;
  }
  // transposed-read lane address: lane 4e + c of each 16-lane group reads key
  // row 4 hh + e, elements 16 ((lane >> 4) & 1) + 4 c (+ 32 dt)
  const int v_lane = (4 * hh + ((lane & 15) >> 2)) * XV_STRIDE + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  // One 64-key block. PRE: prefix (fp16 PV on E4M3 codes) or chunk (bf16 hi +
  // lo PV); MASK: the block reaches past the prefix end, the chunk end or the
  // tile's diagonal. The four variants are separate code, so the accumulators
  // never cross a branch.
  // block kb + 2 into its buffer (last read by block kb - 2, which every
  // wave finished before the last barrier; read again after the next
  // barrier), then the loads of block kb + 3. A wave may do this before or
  // after block kb's math; the second half of the waves stages first, so the
  // two waves sharing a SIMD run their matrix and vector phases against each
  // other instead of in step.
  const bool stage_first = __builtin_amdgcn_readfirstlane(wave) >= XWAVES / 2;
  auto stage_next = [&](int kb) {
    if (kb + 2 < nb) {
      store_block(kb + 2, sk[(kb + 2) & 3], sv[(kb + 2) & 3]);
      if (kb + 3 < nb) load_block(kb + 3);
    }
  };
  auto block = [&](auto pre_tag, auto mask_tag, int kb) {
    constexpr bool PRE = decltype(pre_tag)::value;
    constexpr bool MASK = decltype(mask_tag)::value;
    if (stage_first) stage_next(kb);
    const uint16_t* kd = sk[kb & 3];
    const uint16_t* vd = sv[kb & 3];
    // scores for the 64 keys, every row block: tile kt holds keys
    // 32 kt + 8 (v/4) + 4 hh + v%4. Each K fragment (read three products
    // ahead) serves all row blocks; every product is fenced from the
    // scheduler, which would otherwise hoist all operand reads and spill.
    f32x16 acc[XRB][2];
#pragma unroll
    for (int rb = 0; rb < XRB; ++rb)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[rb][kt][v] = 0.f;
    {
      constexpr int kDepth = 3;
      auto kread = [&](int i) {  // i = 2 ks + kt
        return *reinterpret_cast<const bf16x8*>(kd + (32 * (i & 1) + j) * XK_STRIDE + 16 * (i >> 1) + 8 * hh);
      };
      bf16x8 ka[kDepth];
#pragma unroll
      for (int i = 0; i < kDepth - 1; ++i) ka[i] = kread(i);
#pragma unroll
      for (int i = 0; i < 2 * (XD / 16); ++i) {
        if (i + kDepth - 1 < 2 * (XD / 16)) ka[(i + kDepth - 1) % kDepth] = kread(i + kDepth - 1);
        const int kt = i & 1, ks = i >> 1;
#pragma unroll
        for (int rb = 0; rb < XRB; ++rb)
          acc[rb][kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[i % kDepth], qf[rb][ks], acc[rb][kt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    const float scl = PRE ? sm2 * skv : sm2;  // > 0: the maximum commutes with it
    // P of every row block in the B-operand layout of the four 16-key PV
    // steps (fp16 for the prefix, bf16 hi + lo for the chunk)
    u32x4 ph[XRB][4], pl[XRB][4];
    bool move_any = false;
    float alpha[XRB];
#pragma unroll
    for (int rb = 0; rb < XRB; ++rb) {
      float s[2][16];
      float mx = kXNegInf;
      if constexpr (MASK) {
        const int lim = PRE ? L0 - kb * XKB : tok[rb] - (kb - nb0) * XKB + 1;  // keys below lim are visible
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = 32 * kt + 8 * (v >> 2) + 4 * hh + (v & 3);
            s[kt][v] = key < lim ? acc[rb][kt][v] : kXNegInf;
            mx = fmaxf(mx, s[kt][v]);
          }
      } else {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            s[kt][v] = acc[rb][kt][v];
            mx = fmaxf(mx, s[kt][v]);
          }
      }
      mx = fmaxf(mx, shfl_xor_f32(mx, 32)) * scl;
      // lazy reference: move (and rescale) only when a score exceeds it by 2^8
      const bool move = mx > m_ref[rb] + kXLazy;
      const float m_new = move ? mx : m_ref[rb];
      alpha[rb] = move ? ((m_ref[rb] == kXNegInf) ? 0.f : __builtin_amdgcn_exp2f(m_ref[rb] - m_new)) : 1.0f;
      move_any |= move;
      m_ref[rb] = m_new;
      const float mb = (m_new == kXNegInf) ? 0.f : m_new - kXPBias;
      float psum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          s[kt][v] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][v], scl, -mb));
          psum += s[kt][v];
        }
      l_run[rb] = l_run[rb] * alpha[rb] + psum;
#pragma unroll
      for (int stp = 0; stp < 4; ++stp) {
        const float* pv = &s[stp >> 1][8 * (stp & 1)];
        if constexpr (PRE) {
          ph[rb][stp] = u32x4{pack_f16x2(pv[0], pv[1]), pack_f16x2(pv[2], pv[3]), pack_f16x2(pv[4], pv[5]),
                              pack_f16x2(pv[6], pv[7])};
        } else {
          bf16x8 h, l;
          split_bf16(pv, h, l);
          ph[rb][stp] = __builtin_bit_cast(u32x4, h);
          pl[rb][stp] = __builtin_bit_cast(u32x4, l);
        }
      }
    }
    if (__builtin_amdgcn_ballot_w64(move_any) != 0ull) {  // rare after the first blocks
#pragma unroll
      for (int rb = 0; rb < XRB; ++rb)
#pragma unroll
        for (int dt = 0; dt < XD / 32; ++dt) o[rb][dt] *= alpha[rb];
    }
    // O^T += V^T P^T, 16 keys per step; each V^T fragment (read two products
    // ahead) serves all row blocks
    {
      constexpr int kVDepth = 3;
      auto vread = [&](int i) {  // i = 4 stp + dt
        const uint16_t* vb = vd + v_lane + (32 * ((i >> 2) >> 1) + 16 * ((i >> 2) & 1)) * XV_STRIDE + 32 * (i & 3);
        const u32x2 lo = lds_tr16(vb), hi = lds_tr16(vb + 8 * XV_STRIDE);
        return u32x4{lo[0], lo[1], hi[0], hi[1]};
      };
      u32x4 va[kVDepth];
#pragma unroll
      for (int i = 0; i < kVDepth - 1; ++i) va[i] = vread(i);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i + kVDepth - 1 < 16) va[(i + kVDepth - 1) % kVDepth] = vread(i + kVDepth - 1);
        const int stp = i >> 2, dt = i & 3;
#pragma unroll
        for (int rb = 0; rb < XRB; ++rb) {
          if constexpr (PRE) {
            o[rb][dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, va[i % kVDepth]),
                                                               __builtin_bit_cast(f16x8, ph[rb][stp]), o[rb][dt], 0, 0, 0);
          } else {
            const bf16x8 ab = __builtin_bit_cast(bf16x8, va[i % kVDepth]);
            o[rb][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, __builtin_bit_cast(bf16x8, ph[rb][stp]), o[rb][dt], 0, 0, 0);
            o[rb][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, __builtin_bit_cast(bf16x8, pl[rb][stp]), o[rb][dt], 0, 0, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (!stage_first) stage_next(kb);
    if (kb & 1) __syncthreads();  // uniform: every wave runs the same blocks
  };

  load_block(0);
  store_block(0, sk[0], sv[0]);
  if (nb > 1) {
    load_block(1);
    store_block(1, sk[1], sv[1]);
    if (nb > 2) load_block(2);
  }
  __syncthreads();
  using T = std::true_type;
  using F = std::false_type;
  // prefix: whole blocks, then the last one if it is partial
  const int nfull0 = L0 / XKB;
  for (int kb = 0; kb < nfull0; ++kb) block(T{}, F{}, kb);
  if (nb0 > nfull0) block(T{}, T{}, nb0 - 1);
  if (nb0 > 0) {  // the prefix values carry the workspace V scale
#pragma unroll
    for (int rb = 0; rb < XRB; ++rb)
#pragma unroll
      for (int dt = 0; dt < XD / 32; ++dt) o[rb][dt] *= svv;
  }
  // chunk: blocks whose keys all precede the tile's first token and lie in
  // the chunk need no mask, the rest (the diagonal) do
  int nfree = t0 / XKB;                      // keys [0, 64 * nfree) <= t0
  nfree = min(nfree, C / XKB);
  for (int kb = nb0; kb < nb0 + nfree; ++kb) block(F{}, F{}, kb);
  for (int kb = nb0 + nfree; kb < nb; ++kb) block(F{}, T{}, kb);

#pragma unroll
  for (int rb = 0; rb < XRB; ++rb) {
    const float lr = l_run[rb] + shfl_xor_f32(l_run[rb], 32);
    if (rv[rb]) {
      const float inv = lr > 0.f ? 1.0f / lr : 0.f;
      float* op = a.out + ((int64_t)(q0 + tok[rb]) * a.hq + head[rb]) * XD;
#pragma unroll
      for (int dt = 0; dt < XD / 32; ++dt)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const float4 val = make_float4(o[rb][dt][4 * a4] * inv, o[rb][dt][4 * a4 + 1] * inv,
                                         o[rb][dt][4 * a4 + 2] * inv, o[rb][dt][4 * a4 + 3] * inv);
          *reinterpret_cast<float4*>(op + 32 * dt + 8 * a4 + 4 * hh) = val;
        }
      if (a.lse && hh == 0)
        a.lse[(int64_t)(q0 + tok[rb]) * a.hq + head[rb]] =
            lr > 0.f ? (m_ref[rb] + __log2f(lr) - kXPBias) * kXLn2 : kXNegInf;
    }
  }
}

}  // namespace
}  // namespace kvq

hipError_t kvq_launch_extend(const ExtendArgs& a, hipStream_t s) {
  const int64_t nwg = (a.n_work + 7) / 8 * 8;
  if ((a.page_size & (a.page_size - 1)) == 0)
    kvq::extend_attn_kernel<true><<<(unsigned)nwg, kvq::XTHREADS, 0, s>>>(a);
  else
    kvq::extend_attn_kernel<false><<<(unsigned)nwg, kvq::XTHREADS, 0, s>>>(a);
  return hipGetLastError();
}
