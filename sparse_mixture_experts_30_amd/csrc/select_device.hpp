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

// ---------------------------------------------------------------- selection by teams of lanes
//
// The same selection as select_token, spread over a team of SEL_TEAM
// consecutive lanes of one wave per token: thread q of the team holds
// experts [q E/8, (q+1) E/8) in registers.  The group scores (sum of a
// group's two largest choices) are formed per thread (G >= 8: G / 8 whole
// groups per thread) or merged with lane shuffles (G < 8: a group over
// 8 / G threads) and exchanged through LDS; every pick of the top K is the
// team's butterfly maximum (larger choice wins, equal choices go to the
// lower id).  Every score, group score and weight is computed with
// select_token's arithmetic, so both give the same routing from the same
// fp32 logits.
constexpr int SEL_TEAM = 8;          // lanes per token
constexpr int SEL_TQ = 32;           // experts per lane (E <= 256)
constexpr int SEL_TG = 32;           // groups (LDS row of a token's group scores)
constexpr int SEL_TK = 2 * SEL_TEAM; // picks (each lane keeps two)

inline bool select_team_ok(int E, int G, int TG, int K) {
  if (E % 32 || E > SEL_TEAM * SEL_TQ || G < 1 || G > SEL_TG || E % G) return false;
  const int EQ = E / SEL_TEAM, Eg = E / G;
  const bool whole = Eg <= EQ && EQ % Eg == 0;    // a thread holds whole groups
  const bool span = Eg > EQ && Eg % EQ == 0;      // a group spans 2, 4 or 8 threads
  return (whole || span) && TG >= 1 && TG <= G && K >= 1 && K <= SEL_TK;
}

// lg: this lane's logits (experts q E/8 + j, j < E/8); s_grow: the token's
// LDS row of SEL_TG floats (shared by the team).  Contains a workgroup
// barrier: every thread of the workgroup calls it.  Writes the ids and
// weights only when `valid`.
__device__ __forceinline__ void select_team(const float (&lg)[SEL_TQ], int q, bool valid,
                                            const float* __restrict__ bias, float* s_grow, int E,
                                            int G, int TG, int K, float rho, int32_t* idx_row,
                                            float* w_row) {
  const int EQ = E / SEL_TEAM, e0 = q * EQ, Eg = E / G;
  float sc[SEL_TQ], c[SEL_TQ];
#pragma unroll
  for (int j = 0; j < SEL_TQ; j += 4) {
    if (j < EQ) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double sd = 1.0 / (1.0 + exp(-(double)lg[j + i]));
        sc[j + i] = (float)sd;
        float ci = sc[j + i] + bias[e0 + j + i];
        if (ci != ci) ci = -INFINITY;    // a NaN choice competes as -inf
        c[j + i] = ci;
      }
    }
  }

  // Group scores into the token's LDS row.
  {
    float m1 = -INFINITY, m2 = -INFINITY;
    int cnt = 0, gi = e0 / Eg;
#pragma unroll
    for (int j = 0; j < SEL_TQ; ++j) {
      if (j < EQ) {
        const float v = c[j];
        if (v > m1) {
          m2 = m1;
          m1 = v;
        } else if (v > m2) {
          m2 = v;
        }
        if (++cnt == Eg) {
          float g = m1 + m2;
          if (g != g) g = -INFINITY;   // -inf + inf
          s_grow[gi] = g;
          ++gi;
          cnt = 0;
          m1 = m2 = -INFINITY;
        }
      }
    }
    if (Eg > EQ) {
      const int span = Eg / EQ;   // threads per group: 2, 4 or 8
      for (int off = 1; off < span; off <<= 1) {
        const float o1 = __shfl_xor(m1, off, 64), o2 = __shfl_xor(m2, off, 64);
        const float hi = fmaxf(m1, o1), lo = fminf(m1, o1);
        m2 = fmaxf(lo, fmaxf(m2, o2));
        m1 = hi;
      }
      if (q % span == 0) {
        float g = m1 + m2;
        if (g != g) g = -INFINITY;
        s_grow[gi] = g;
      }
    }
  }
  __syncthreads();

  // The TG best groups (ties to the lower index); the same mask in every
  // thread of the team.
  float gs[SEL_TG];
#pragma unroll
  for (int j = 0; j < SEL_TG; ++j) gs[j] = j < G ? s_grow[j] : -INFINITY;
  uint32_t keep = 0;
  for (int r = 0; r < TG; ++r) {
    float bv = -INFINITY;
    int bi = -1;
#pragma unroll
    for (int j = 0; j < SEL_TG; ++j)
      if (j < G && !((keep >> j) & 1u) && (bi < 0 || gs[j] > bv)) {
        bv = gs[j];
        bi = j;
      }
    keep |= 1u << bi;
  }
  // Experts outside the kept groups compete with choice 0.0.
#pragma unroll
  for (int j = 0; j < SEL_TQ; ++j)
    if (j < EQ && !((keep >> ((e0 + j) / Eg)) & 1u)) c[j] = 0.0f;

  // Top K by team maxima; lane q keeps picks q and q + SEL_TEAM.  A lane
  // offers its best untaken expert even at -inf, so K <= E valid ids exist.
  uint32_t taken = 0;
  float sum = 0.0f, ps0 = 0.0f, ps1 = 0.0f;
  int pe0 = 0, pe1 = 0;
  for (int k = 0; k < K; ++k) {
    float bv = -INFINITY, bs = 0.0f;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < SEL_TQ; ++j)
      if (j < EQ && !((taken >> j) & 1u) && (bi == 0x7fffffff || c[j] > bv)) {
        bv = c[j];
        bi = e0 + j;
        bs = sc[j];
      }
#pragma unroll
    for (int off = 1; off < SEL_TEAM; off <<= 1) {
      const float ov = __shfl_xor(bv, off, 64), os = __shfl_xor(bs, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
        bs = os;
      }
    }
    if (bi >= e0 && bi < e0 + EQ) taken |= 1u << (bi - e0);
    sum += bs;   // the unbiased scores of the picks, in pick order
    if (k == q) {
      pe0 = bi;
      ps0 = bs;
    } else if (k == q + SEL_TEAM) {
      pe1 = bi;
      ps1 = bs;
    }
  }
  // Weights: normalised over the K picks (K > 1), times rho.
  if (valid) {
    if (q < K) {
      idx_row[q] = pe0;
      w_row[q] = ((K > 1) ? ps0 / (sum + 1e-20f) : ps0) * rho;
    }
    if (q + SEL_TEAM < K) {
      idx_row[q + SEL_TEAM] = pe1;
      w_row[q + SEL_TEAM] = (ps1 / (sum + 1e-20f)) * rho;
    }
  }
}

}  // namespace moe
