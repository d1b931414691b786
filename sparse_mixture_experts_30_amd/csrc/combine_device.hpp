// One token's combine (gfx950 device code), shared by the combine kernel and
// the one-launch decode layer: every token collects its expert outputs back
// (page "从 1024 块 GPU 到 558 万美元：拆解 DeepSeek-V3 的算法-系统协同设计", section
// 2.3: after the local experts the results return to their tokens) and sums
// them with the gate weights, plus the always-active shared expert (same
// page, section 2.2):
//   out[t] = y_shared[t] + sum_k w[t,k] * y[pos[t*K + k]]
// fp32 accumulation in k order, one rounding to bf16; 16-byte coalesced loads
// of whole rows.  A position outside [0, N) (only a caller-made pos can hold
// one) contributes nothing.
#pragma once

#include "moe_internal.hpp"

namespace moe {

// All NTH threads of the workgroup call this (it passes one barrier); sp and
// sw are LDS arrays of at least K entries.
template <int NTH>
__device__ __forceinline__ void combine_row_bf16(const uint16_t* __restrict__ y,
                                                 const uint16_t* __restrict__ ys,
                                                 const int32_t* __restrict__ pos,
                                                 const float* __restrict__ w,
                                                 uint16_t* __restrict__ out, int64_t t, int H,
                                                 int K, int64_t N, int32_t* sp, float* sw) {
  if (threadIdx.x < K) {
    const int32_t p = pos[t * K + threadIdx.x];
    sp[threadIdx.x] = (p >= 0 && p < N) ? p : -1;
    sw[threadIdx.x] = w[t * K + threadIdx.x];
  }
  __syncthreads();
  for (int c = threadIdx.x * 8; c < H; c += NTH * 8) {
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
      for (int b = 0; b < kBatch; ++b) {
        v[b] = make_uint4(0u, 0u, 0u, 0u);
        if (k0 + b < K && sp[k0 + b] >= 0)
          v[b] = *reinterpret_cast<const uint4*>(y + (int64_t)sp[k0 + b] * H + c);
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        if (k0 + b >= K) break;
        if (sp[k0 + b] < 0) continue;
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

}  // namespace moe
