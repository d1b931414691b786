// Combine: every token collects its expert outputs back (page "从 1024 块 GPU 到 558 万美元：
// 拆解 DeepSeek-V3 的算法-系统协同设计", section 2.3: after the local experts the
// results return to their tokens) and sums them with the gate weights, plus
// the always-active shared expert (same page, section 2.2):
//   out[t] = y_shared[t] + sum_k w[t,k] * y[pos[t*K + k]]
// fp32 accumulation in k order; one rounding to the output type.  One
// workgroup per token, 16-byte coalesced loads of whole rows (an HBM-bound
// gather-add).
#include "moe_internal.hpp"

namespace moe {

namespace {

constexpr int CT = 256;

__global__ void __launch_bounds__(CT)
combine_bf16_kernel(const uint16_t* __restrict__ y, const uint16_t* __restrict__ ys,
                    const int32_t* __restrict__ pos, const float* __restrict__ w,
                    uint16_t* __restrict__ out, int H, int K) {
  const int64_t t = blockIdx.x;
  __shared__ int32_t sp[64];
  __shared__ float sw[64];
  if (threadIdx.x < K) {
    sp[threadIdx.x] = pos[t * K + threadIdx.x];
    sw[threadIdx.x] = w[t * K + threadIdx.x];
  }
  __syncthreads();
  for (int c = threadIdx.x * 8; c < H; c += CT * 8) {
    float acc[8];
    if (ys) {
      const uint4 v = *reinterpret_cast<const uint4*>(ys + t * H + c);
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] = bf16_bits_to_f32(u[j] & 0xFFFFu);
        acc[2 * j + 1] = bf16_bits_to_f32(u[j] >> 16);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
    }
    // The rows of up to kBatch experts are loaded together, then added in
    // k order (one memory round trip per batch instead of one per expert).
    constexpr int kBatch = 8;
    for (int k0 = 0; k0 < K; k0 += kBatch) {
      uint4 v[kBatch];
#pragma unroll
      for (int b = 0; b < kBatch; ++b)
        if (k0 + b < K) v[b] = *reinterpret_cast<const uint4*>(y + (int64_t)sp[k0 + b] * H + c);
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        if (k0 + b >= K) break;
        const uint32_t u[4] = {v[b].x, v[b].y, v[b].z, v[b].w};
        const float wk = sw[k0 + b];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[2 * j] = fmaf(wk, bf16_bits_to_f32(u[j] & 0xFFFFu), acc[2 * j]);
          acc[2 * j + 1] = fmaf(wk, bf16_bits_to_f32(u[j] >> 16), acc[2 * j + 1]);
        }
      }
    }
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<uint4*>(out + t * H + c) = o;
  }
}

__global__ void __launch_bounds__(CT)
combine_f32_kernel(const float* __restrict__ y, const float* __restrict__ ys,
                   const int32_t* __restrict__ pos, const float* __restrict__ w,
                   float* __restrict__ out, int H, int K) {
  const int64_t t = blockIdx.x;
  for (int c = threadIdx.x; c < H; c += CT) {
    float acc = ys ? ys[t * H + c] : 0.0f;
    for (int k = 0; k < K; ++k)
      acc = fmaf(w[t * K + k], y[(int64_t)pos[t * K + k] * H + c], acc);
    out[t * H + c] = acc;
  }
}

}  // namespace

hipError_t launch_combine(const void* y, const void* ys, const int32_t* pos, const float* w,
                          void* out, int64_t T, int H, int K, bool bf16, hipStream_t s) {
  if (bf16)
    MOE_TIMED_LAUNCH(s, "combine_bf16_kernel",
      hipLaunchKernelGGL(combine_bf16_kernel, dim3((unsigned)T), dim3(CT), 0, s,
                         (const uint16_t*)y, (const uint16_t*)ys, pos, w, (uint16_t*)out, H, K));
  else
    MOE_TIMED_LAUNCH(s, "combine_f32_kernel",
      hipLaunchKernelGGL(combine_f32_kernel, dim3((unsigned)T), dim3(CT), 0, s, (const float*)y,
                         (const float*)ys, pos, w, (float*)out, H, K));
  return hipGetLastError();
}

}  // namespace moe
