// The decode gate's work item (gfx950 device code), shared by the decode
// routing kernels and the one-launch decode layer.
//
// The gate of the layer (page "从 1024 块 GPU 到 558 万美元：拆解 DeepSeek-V3 的算法-系统协同设计",
// section 2.2): logits = x W^T in fp32 arithmetic.  For a batch of at most
// 32 tokens (one 32-row MFMA block) the fp32 gate weight is read straight
// from its copy and split in registers into its exact bf16 parts
// (gate_split.hpp); the three bf16 MFMA products accumulate in fp32.
#pragma once

#include "moe_internal.hpp"
#include "gate_split.hpp"

namespace moe {

constexpr int DG_MAXK = 896;                 // k range per gate item (bounds its registers)
constexpr int DM_STEPS = DG_MAXK / 4 / 16;   // 16-wide k steps per wave, at most

// One gate item: experts 32 eb .. 32 eb + 31 over the ks-th k range of
// kchunk elements, by four waves (wave = 0..3 of the item) that split the
// range in 16-wide k steps.  Per step a lane loads its 8 k of one token row
// (A operand: token lane % 32) and of one fp32 gate row (B operand: expert
// 32 eb + lane % 32), splits the weights into their exact bf16 parts and
// accumulates the three products in fp32; every load of the wave is issued
// before its first MFMA.  The waves' sums are added in wave order through
// `red` (LDS, [3][16][64]) and wave 0 writes part[ks][t][e].  Rows past T and
// experts past E re-read a valid row and are not stored; k past the range is
// zero.  Every wave of the workgroup passes one barrier here; valid = false
// (an item past the last) loads and stores nothing.
__device__ __forceinline__ void gate_mfma_item(const uint16_t* __restrict__ x,
                                               const float* __restrict__ wg,
                                               float* __restrict__ part, int T, int H, int E,
                                               int kchunk, int eb, int ks, int wave, bool valid,
                                               float (*red)[16][kWave]) {
  const int lane = threadIdx.x & 63;
  const int lr = lane & 31, lh = lane >> 5;
  const int k0 = ks * kchunk;
  const int kn = min(H, k0 + kchunk) - k0;      // a multiple of 8
  const int nst = (kn + 15) / 16;
  const int per = (nst + 3) / 4;                // <= DM_STEPS (kchunk <= DG_MAXK)
  const int s0 = wave * per, s1 = valid ? min(nst, s0 + per) : s0;
  const int t = min(lr, T - 1);
  const int e = min(eb * 32 + lr, E - 1);
  const uint16_t* xr = x + (int64_t)t * H + k0 + 8 * lh;
  const float* wr = wg + (int64_t)e * H + k0 + 8 * lh;

  u32x4 xa[DM_STEPS], wa[DM_STEPS], wb[DM_STEPS];
#pragma unroll
  for (int j = 0; j < DM_STEPS; ++j) {
    const int st = s0 + j;
    if (st < s1 && st * 16 + 8 * lh < kn) {
      xa[j] = *reinterpret_cast<const u32x4*>(xr + st * 16);
      wa[j] = *reinterpret_cast<const u32x4*>(wr + st * 16);
      wb[j] = *reinterpret_cast<const u32x4*>(wr + st * 16 + 4);
    } else {
      xa[j] = wa[j] = wb[j] = (u32x4){0u, 0u, 0u, 0u};
    }
  }
  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int j = 0; j < DM_STEPS; ++j) {
    if (s0 + j < s1) {   // uniform over the wave
      u32x4 h, m, l;
      split3(wa[j], wb[j], h, m, l);
      const bf16x8 a = as_bf16x8(xa[j]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_bf16x8(h), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_bf16x8(m), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_bf16x8(l), acc, 0, 0, 0);
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) red[wave - 1][i][lane] = acc[i];
  }
  __syncthreads();
  // C layout: lane holds expert column lr and token rows 8 (i / 4) + 4 lh + i % 4.
  const int ec = eb * 32 + lr;
  if (wave == 0 && valid && ec < E) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int tr = 8 * (i >> 2) + 4 * lh + (i & 3);
      const float v = ((acc[i] + red[0][i][lane]) + red[1][i][lane]) + red[2][i][lane];
      if (tr < T) part[((int64_t)ks * T + tr) * E + ec] = v;
    }
  }
}

}  // namespace moe
