// Merge of the per-split partial results of a decode launch.
//
// Split s of sequence b, query head h holds a normalized output o_s and
// lse_s = log2 sum_{t in s} 2^(score_t) (scores in the log2 domain). The full
// result is the log-sum-exp merge
//   LSE = log2 sum_s 2^lse_s,  out = sum_s 2^(lse_s - LSE) o_s,
// reported with the natural-log LSE (LSE * ln 2). Splits past the sequence
// end were never written and are not read.
//
// The merge reads ~1 MB and is bound by memory latency, not bandwidth, so a
// lane owns one output element of one (sequence, query head) and merges
// without any exchange: it loads up to 8 splits' LSEs (the same addresses
// in every lane: one broadcast load each) and its 8 output elements at once,
// folds them into a running (max, sum, weighted sum), and repeats for more
// splits. One HBM round trip for the usual <= 8 splits; no LDS, no barrier.
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kMaxSplits = 128;
constexpr int kBatch = 8;  // splits loaded per round

__global__ void __launch_bounds__(64) combine_kernel(const CombineArgs a) {
  const int chunks = (a.dv + 63) >> 6;
  const int h = blockIdx.x / chunks, d = ((blockIdx.x - h * chunks) << 6) + threadIdx.x;
  const int b = blockIdx.y;
  int L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > a.max_len ? a.max_len : L);
  int n = (L + a.tokens_per_split - 1) / a.tokens_per_split;
  n = n > a.num_splits ? a.num_splits : n;
  const int64_t hq = (int64_t)b * a.hq + h;
  const float* lse_s = a.ws_lse + hq * a.num_splits;
  const float* o_s = a.ws_o + hq * a.num_splits * (int64_t)a.dv + (d < a.dv ? d : 0);
  float M = kNegInf, W = 0.f, acc = 0.f;
  for (int s0 = 0; s0 < n; s0 += kBatch) {
    float x[kBatch], o[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const bool ok = s0 + j < n;
      x[j] = ok ? lse_s[s0 + j] : kNegInf;
      o[j] = ok ? o_s[(int64_t)(s0 + j) * a.dv] : 0.f;
    }
    float Mn = M;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) Mn = fmaxf(Mn, x[j]);
    if (Mn == kNegInf) continue;
    const float r = __builtin_amdgcn_exp2f(M - Mn);  // 0 while M is -inf
    W *= r;
    acc *= r;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const float e = __builtin_amdgcn_exp2f(x[j] - Mn);
      W += e;
      acc = fmaf(e, o[j], acc);
    }
    M = Mn;
  }
  if (d < a.dv) a.out[hq * a.dv + d] = W > 0.f ? acc / W : 0.f;
  if (a.lse && d == 0) a.lse[hq] = W > 0.f ? (M + __log2f(W)) * 0.6931471805599453f : kNegInf;
}

}  // namespace
}  // namespace kvq

hipError_t kvq_launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.num_splits > kvq::kMaxSplits) return hipErrorInvalidValue;
  const dim3 grid(a.hq * ((a.dv + 63) / 64), a.batch);
  kvq::combine_kernel<<<grid, 64, 0, s>>>(a);
  return hipGetLastError();
}
