// Combine: every token collects its expert outputs back (page "从 1024 块 GPU 到 558 万美元：
// 拆解 DeepSeek-V3 的算法-系统协同设计", section 2.3: after the local experts the
// results return to their tokens) and sums them with the gate weights, plus
// the always-active shared expert (same page, section 2.2):
//   out[t] = y_shared[t] + sum_k w[t,k] * y[pos[t*K + k]]
// fp32 accumulation in k order; one rounding to the output type.  One
// workgroup per token, 16-byte coalesced loads of whole rows (an HBM-bound
// gather-add).  A position outside [0, T*K) (only a caller-made pos can hold
// one) contributes nothing.
#include "moe_internal.hpp"
#include "combine_device.hpp"

namespace moe {

namespace {

constexpr int CT = 256;

__global__ void __launch_bounds__(CT)
combine_bf16_kernel(const uint16_t* __restrict__ y, const uint16_t* __restrict__ ys,
                    const int32_t* __restrict__ pos, const float* __restrict__ w,
                    uint16_t* __restrict__ out, int H, int K, int64_t N) {
  __shared__ int32_t sp[64];
  __shared__ float sw[64];
  combine_row_bf16<CT>(y, ys, pos, w, out, blockIdx.x, H, K, N, sp, sw);
}

__global__ void __launch_bounds__(CT)
combine_f32_kernel(const float* __restrict__ y, const float* __restrict__ ys,
                   const int32_t* __restrict__ pos, const float* __restrict__ w,
                   float* __restrict__ out, int H, int K, int64_t N) {
  const int64_t t = blockIdx.x;
  for (int c = threadIdx.x; c < H; c += CT) {
    float acc = ys ? ys[t * H + c] : 0.0f;
    for (int k = 0; k < K; ++k) {
      const int32_t p = pos[t * K + k];
      if (p >= 0 && p < N) acc = fmaf(w[t * K + k], y[(int64_t)p * H + c], acc);
    }
    out[t * H + c] = acc;
  }
}

}  // namespace

hipError_t launch_combine(const void* y, const void* ys, const int32_t* pos, const float* w,
                          void* out, int64_t T, int H, int K, bool bf16, hipStream_t s) {
  if (bf16)
    MOE_TIMED_LAUNCH(s, "combine_bf16_kernel",
      hipLaunchKernelGGL(combine_bf16_kernel, dim3((unsigned)T), dim3(CT), 0, s,
                         (const uint16_t*)y, (const uint16_t*)ys, pos, w, (uint16_t*)out, H, K,
                         T * K));
  else
    MOE_TIMED_LAUNCH(s, "combine_f32_kernel",
      hipLaunchKernelGGL(combine_f32_kernel, dim3((unsigned)T), dim3(CT), 0, s, (const float*)y,
                         (const float*)ys, pos, w, (float*)out, H, K, T * K));
  return hipGetLastError();
}

}  // namespace moe
