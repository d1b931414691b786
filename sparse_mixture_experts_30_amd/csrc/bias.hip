// Load-balancing update of the gate's selection bias.  The per-expert bias
// only takes part in choosing experts and is a buffer steered by the experts'
// observed load, not by a gradient (page "从 1024 块 GPU 到 558 万美元：拆解
// DeepSeek-V3 的算法-系统协同设计", section 2.2); the page prints no rule.  The
// rule taken here: each expert's bias moves one fixed step gamma toward the
// mean load sum(counts) / E -- up when the expert is below it, down when
// above, unchanged (bit for bit) at it -- as one fp32 add.  The comparison
// with the mean is exact integer arithmetic, counts[e] * E against
// sum(counts), so the direction never depends on rounding.
#include "moe_internal.hpp"

namespace moe {

namespace {

constexpr int BT = 512;   // one workgroup covers every expert (E <= 512)

__global__ void __launch_bounds__(BT)
bias_update_kernel(const int32_t* __restrict__ counts, float* __restrict__ bias, int E,
                   float gamma) {
  __shared__ long long psum[BT / 64];
  __shared__ int pneg[BT / 64];
  const int e = threadIdx.x;
  const int32_t n = e < E ? counts[e] : 0;
  long long v = n;
  int neg = n < 0;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    v += __shfl_xor(v, o);
    neg |= __shfl_xor(neg, o);
  }
  if ((e & 63) == 0) {
    psum[e >> 6] = v;
    pneg[e >> 6] = neg;
  }
  __syncthreads();
  long long total = 0;
  int any_neg = 0;
#pragma unroll
  for (int w = 0; w < BT / 64; ++w) {
    total += psum[w];
    any_neg |= pneg[w];
  }
  // A negative count is not a load: the bias is left as it is.
  if (e >= E || any_neg) return;
  const long long scaled = (long long)n * E;
  if (scaled < total) bias[e] = bias[e] + gamma;
  else if (scaled > total) bias[e] = bias[e] - gamma;
}

}  // namespace

hipError_t launch_bias_update(const int32_t* counts, float* bias, int E, float gamma,
                              hipStream_t s) {
  if (E < 1 || E > BT) return hipErrorInvalidValue;
  MOE_TIMED_LAUNCH(s, "bias_update_kernel",
                   bias_update_kernel<<<1, BT, 0, s>>>(counts, bias, E, gamma));
  return hipGetLastError();
}

}  // namespace moe
