// Merge of the per-split partial results of a decode launch.
//
// Each split s of sequence b, query head h holds a normalized output o_s and
// lse_s = log2 sum_{t in s} 2^(score_t) (scores in the log2 domain). The full
// result is the usual log-sum-exp merge:
//   LSE = log2 sum_s 2^lse_s,  out = sum_s 2^(lse_s - LSE) o_s,
// reported with the natural-log LSE (LSE * ln 2). Splits past the sequence
// end were never written and are not read.
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();

__global__ void __launch_bounds__(256) combine_kernel(const CombineArgs a) {
  const int h = blockIdx.x, b = blockIdx.y;
  int L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > a.max_len ? a.max_len : L);
  int n = (L + a.tokens_per_split - 1) / a.tokens_per_split;
  n = n > a.num_splits ? a.num_splits : n;
  const int64_t hq = (int64_t)b * a.hq + h;
  const float* lse_s = a.ws_lse + hq * a.num_splits;
  float M = kNegInf;
  for (int s = 0; s < n; ++s) M = fmaxf(M, lse_s[s]);
  float W = 0.f;
  if (M != kNegInf)
    for (int s = 0; s < n; ++s) W += __builtin_amdgcn_exp2f(lse_s[s] - M);
  const float inv = W > 0.f ? 1.0f / W : 0.f;
  const float* o_s = a.ws_o + hq * a.num_splits * (int64_t)a.dv;
  for (int d = threadIdx.x; d < a.dv; d += blockDim.x) {
    float acc = 0.f;
    if (W > 0.f)
      for (int s = 0; s < n; ++s) acc += __builtin_amdgcn_exp2f(lse_s[s] - M) * o_s[(int64_t)s * a.dv + d];
    a.out[hq * a.dv + d] = acc * inv;
  }
  if (threadIdx.x == 0 && a.lse) a.lse[hq] = W > 0.f ? (M + __log2f(W)) * 0.6931471805599453f : kNegInf;
}

}  // namespace
}  // namespace kvq

hipError_t kvq_launch_combine(const CombineArgs& a, hipStream_t s) {
  const dim3 grid(a.hq, a.batch);
  const int threads = a.dv >= 256 ? 256 : 128;
  kvq::combine_kernel<<<grid, threads, 0, s>>>(a);
  return hipGetLastError();
}
