// Exact three-way bf16 split of fp32 gate weights (gfx950 device code),
// shared by the batch gate GEMM and the decode gate.
//
// w = hi + mid + lo with hi = w truncated to bf16, mid = (w - hi) truncated,
// lo = w - hi - mid (at most 8 significant bits left), every difference
// exact in fp32.  With x in bf16, each product x * part is exact in fp32,
// so bf16 MFMAs over the three parts accumulated in fp32 give x w^T as an
// fp32 computation would (the gate's fp32 arithmetic: page "从 1024 块 GPU 到
// 558 万美元：拆解 DeepSeek-V3 的算法-系统协同设计", section 2.2).
#pragma once

#include "moe_internal.hpp"

namespace moe {

// Split 8 fp32 weights into hi/mid/lo bf16x8 operands (exact decomposition).
__device__ __forceinline__ void split3(u32x4 p, u32x4 q, u32x4& h, u32x4& m, u32x4& l) {
  const uint32_t v[8] = {p.x, p.y, p.z, p.w, q.x, q.y, q.z, q.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t hb[2], mb[2], lb[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t b = v[2 * j + u];
      const float r1 = __uint_as_float(b) - __uint_as_float(b & 0xFFFF0000u);  // exact
      const uint32_t b1 = __float_as_uint(r1);
      const float r2 = r1 - __uint_as_float(b1 & 0xFFFF0000u);  // exact, <= 8 bits
      hb[u] = b >> 16;
      mb[u] = b1 >> 16;
      lb[u] = __float_as_uint(r2) >> 16;
    }
    h[j] = hb[0] | (hb[1] << 16);
    m[j] = mb[0] | (mb[1] << 16);
    l[j] = lb[0] | (lb[1] << 16);
  }
}

}  // namespace moe
