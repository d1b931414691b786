// Per-token expert selection by one wavefront (page "从 1024 块 GPU 到 558 万美元：
// 拆解 DeepSeek-V3 的算法-系统协同设计", section 2.2, MoEGate): sigmoid scores,
// the selection-only bias, the group score as the sum of a group's two
// largest choice scores, the topk_group best groups, the top_k best experts
// inside them (0.0 for experts outside), and the weights from the unbiased
// scores, normalised over the chosen experts when top_k > 1, times
// routed_scaling_factor.
#pragma once

#include "moe_internal.hpp"

namespace moe {

constexpr int SEL_MAXV = 8;   // E <= 512 = 64 lanes x 8
constexpr int SEL_SB = 4;     // k splits whose loads are issued together
constexpr int SEL_DEEP = 16;  // from this many k splits a token's sum is cut in parts
constexpr int SEL_PARTS = 4;  // ... of contiguous splits, summed by SEL_PARTS waves

// First split of part `q` of SEL_PARTS when a token's ksplit partial sums
// are cut into contiguous parts (q = SEL_PARTS gives ksplit).
__device__ __forceinline__ int sel_part_begin(int ksplit, int q) {
  return (int)((int64_t)ksplit * q / SEL_PARTS);
}

// Lane l's logits of token t (experts e = l + 64 v): the k-split partial
// sums of splits [s_begin, s_end) of part ([ksplit][T][E], split stride
// T * E) added in split order.  The loads of SEL_SB splits (for all of the
// lane's experts) are issued together and then added in order, so a deep
// split costs few memory round trips.
__device__ __forceinline__ void sum_splits(const float* __restrict__ part, int64_t stride,
                                           int64_t t, int E, int lane, int s_begin, int s_end,
                                           float (&lgs)[SEL_MAXV]) {
  const int V = (E + 63) / 64;
#pragma unroll
  for (int v = 0; v < SEL_MAXV; ++v) {
    const int e = lane + 64 * v;
    lgs[v] = (v < V && e < E) ? part[(int64_t)s_begin * stride + t * E + e] : 0.0f;
  }
  for (int s0 = s_begin + 1; s0 < s_end; s0 += SEL_SB) {
    float pv[SEL_SB][SEL_MAXV];
#pragma unroll
    for (int j = 0; j < SEL_SB; ++j)
#pragma unroll
      for (int v = 0; v < SEL_MAXV; ++v) {
        const int e = lane + 64 * v;
        pv[j][v] = (s0 + j < s_end && v < V && e < E)
                       ? part[(int64_t)(s0 + j) * stride + t * E + e] : 0.0f;
      }
#pragma unroll
    for (int j = 0; j < SEL_SB; ++j)
#pragma unroll
      for (int v = 0; v < SEL_MAXV; ++v)
        if (s0 + j < s_end) lgs[v] += pv[j][v];
  }
}

// Wave-level argmax of (v, i): larger v wins, equal v -> lower i.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    float ov = __shfl_xor(v, off, 64);
    int oi = __shfl_xor(i, off, 64);
    if (ov > v || (ov == v && oi < i)) {
      v = ov;
      i = oi;
    }
  }
}

// Lane l holds the logits of experts e = l + 64 v (v < ceil(E / 64)).  s_c
// and s_s are this wavefront's LDS rows of at least E floats.  Writes the
// logits row (if logits_row is not null), the K chosen ids and weights; the
// ids also go to idx_lds when it is not null.
__device__ __forceinline__ void select_token(const float (&lgs)[SEL_MAXV], int lane,
                                             const float* __restrict__ bias, float* s_c,
                                             float* s_s, int E, int G, int TG, int K, float rho,
                                             float* logits_row, int32_t* idx_row, float* w_row,
                                             int32_t* idx_lds) {
  const int Eg = E / G;
  const int V = (E + 63) / 64;
  float c[SEL_MAXV], s32[SEL_MAXV];
#pragma unroll
  for (int v = 0; v < SEL_MAXV; ++v) {
    const int e = lane + 64 * v;
    c[v] = -INFINITY;
    s32[v] = 0.0f;
    if (v < V && e < E) {
      const float lg = lgs[v];
      if (logits_row) logits_row[e] = lg;
      const double sd = 1.0 / (1.0 + exp(-(double)lg));
      s32[v] = (float)sd;
      c[v] = s32[v] + bias[e];
      // A NaN choice (NaN in x or the bias) competes as -inf, so every
      // comparison below is a total order and every pick is a valid id.
      if (c[v] != c[v]) c[v] = -INFINITY;
      s_c[e] = c[v];
      s_s[e] = s32[v];
    }
  }
  __syncwarp();

  // Group score: sum of the two largest choice scores of group `lane`.
  float g = -INFINITY;
  if (lane < G) {
    float m1 = -INFINITY, m2 = -INFINITY;
    for (int j = 0; j < Eg; ++j) {
      const float v = s_c[lane * Eg + j];
      if (v > m1) {
        m2 = m1;
        m1 = v;
      } else if (v > m2) {
        m2 = v;
      }
    }
    g = m1 + m2;
    if (g != g) g = -INFINITY;   // -inf + inf
  }
  // Keep the TG best groups.
  uint64_t keep = 0;
  for (int r = 0; r < TG; ++r) {
    float v = g;
    int i = (lane < G && !((keep >> lane) & 1ull)) ? lane : 0x7fffffff;
    if (i == 0x7fffffff) v = -INFINITY;
    wave_argmax(v, i);
    keep |= 1ull << i;
  }
  // Masked choice scores: 0.0 outside the kept groups.
#pragma unroll
  for (int v = 0; v < SEL_MAXV; ++v) {
    const int e = lane + 64 * v;
    if (v < V && e < E && !((keep >> (e / Eg)) & 1ull)) c[v] = 0.0f;
  }
  // Top K, descending, ties to the lower expert id.  A lane offers its best
  // untaken expert even at -inf, so K <= E valid ids always exist.
  float my_s = 0.0f;
  int my_e = 0;
  uint32_t taken = 0;
  for (int k = 0; k < K; ++k) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int v = 0; v < SEL_MAXV; ++v) {
      const int e = lane + 64 * v;
      if (v < V && e < E && !((taken >> v) & 1u) && (c[v] > bv || bi == 0x7fffffff)) {
        bv = c[v];
        bi = e;
      }
    }
    wave_argmax(bv, bi);
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == k) {
      my_e = bi;
      my_s = s_s[bi];
    }
  }
  // Weights: unbiased scores, normalised over the K slots (K > 1), times rho.
  float sum = 0.0f;
  for (int k = 0; k < K; ++k) sum += __shfl(my_s, k, 64);
  if (lane < K) {
    const float wv = (K > 1) ? my_s / (sum + 1e-20f) : my_s;
    idx_row[lane] = my_e;
    w_row[lane] = wv * rho;
    if (idx_lds) idx_lds[lane] = my_e;
  }
}

}  // namespace moe
