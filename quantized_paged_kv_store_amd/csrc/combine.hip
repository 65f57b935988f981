// Merge of the per-split partial results of a decode launch.
//
// Split s of sequence b, query head h holds a normalized output o_s and
// lse_s = log2 sum_{t in s} 2^(score_t) (scores in the log2 domain). The full
// result is the log-sum-exp merge
//   LSE = log2 sum_s 2^lse_s,  out = sum_s 2^(lse_s - LSE) o_s,
// reported with the natural-log LSE (LSE * ln 2). Splits past the sequence
// end were never written and are not read.
//
// One workgroup per (sequence, query head): the split weights are computed
// once into LDS, then every thread streams its output elements over the
// splits with independent, coalesced loads.
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kMaxSplits = 128;

__global__ void __launch_bounds__(128) combine_kernel(const CombineArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  int L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > a.max_len ? a.max_len : L);
  int n = (L + a.tokens_per_split - 1) / a.tokens_per_split;
  n = n > a.num_splits ? a.num_splits : n;
  const int64_t hq = (int64_t)b * a.hq + h;
  __shared__ float sw[kMaxSplits];
  __shared__ float s_lse;
  const float* lse_s = a.ws_lse + hq * a.num_splits;
  if (tid < 64) {
    // wave 0: max and sum over at most 128 splits, two per lane
    const float x0 = tid < n ? lse_s[tid] : kNegInf;
    const float x1 = tid + 64 < n ? lse_s[tid + 64] : kNegInf;
    float M = fmaxf(x0, x1);
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    const float e0 = M == kNegInf ? 0.f : __builtin_amdgcn_exp2f(x0 - M);
    const float e1 = M == kNegInf ? 0.f : __builtin_amdgcn_exp2f(x1 - M);
    float W = e0 + e1;
    for (int off = 32; off > 0; off >>= 1) W += __shfl_xor(W, off, 64);
    const float inv = W > 0.f ? 1.0f / W : 0.f;
    sw[tid] = e0 * inv;
    sw[tid + 64] = e1 * inv;
    if (tid == 0) s_lse = W > 0.f ? (M + __log2f(W)) * 0.6931471805599453f : kNegInf;
  }
  __syncthreads();
  const float* o_s = a.ws_o + hq * a.num_splits * (int64_t)a.dv;
  for (int d = tid; d < a.dv; d += blockDim.x) {
    float acc0 = 0.f, acc1 = 0.f;
    int s = 0;
    for (; s + 1 < n; s += 2) {
      acc0 += sw[s] * o_s[(int64_t)s * a.dv + d];
      acc1 += sw[s + 1] * o_s[(int64_t)(s + 1) * a.dv + d];
    }
    if (s < n) acc0 += sw[s] * o_s[(int64_t)s * a.dv + d];
    a.out[hq * a.dv + d] = acc0 + acc1;
  }
  if (tid == 0 && a.lse) a.lse[hq] = s_lse;
}

}  // namespace
}  // namespace kvq

hipError_t kvq_launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.num_splits > kvq::kMaxSplits) return hipErrorInvalidValue;
  const dim3 grid(a.hq, a.batch);
  kvq::combine_kernel<<<grid, 128, 0, s>>>(a);
  return hipGetLastError();
}
