// Stable permutation of a short id list by one workgroup (page "从 1024 块 GPU
// 到 558 万美元：拆解 DeepSeek-V3 的算法-系统协同设计", section 2.3: per-expert counts
// from the one-hot of the chosen ids, then the flat ids sorted so that each
// expert's entries are contiguous).  counts[e] = #{f : idx[f] == e};
// offsets = exclusive scan; perm lists the flat indices f grouped by
// expert, ascending f inside an expert; pos = inverse of perm.  Shared by
// the small-batch permutation kernel and the fused decode routing kernel.
#pragma once

#include "moe_internal.hpp"

namespace moe {

constexpr int PMAXE = 512;   // experts handled (ids >= PMAXE are invalid)

// LDS the routine needs, for a workgroup of NTH threads (NTH >= PMAXE).
template <int NTH>
struct PermuteLds {
  int32_t h[PMAXE + 1];        // h[E] counts ids outside [0, E)
  int32_t s[NTH];
  int32_t running[PMAXE];
  int32_t wcnt[NTH / 64][PMAXE];
  int32_t wsum[NTH / 64];
};

// Inclusive sum of v over the NTH threads of the workgroup (every thread
// calls it): a shuffle scan inside each wavefront, then the totals of the
// wavefronts before this one.  wsum holds NTH / 64 values.
template <int NTH>
__device__ __forceinline__ int32_t block_inclusive_scan(int32_t v, int32_t* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t u = __shfl_up(v, off, 64);
    if (lane >= off) v += u;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  int32_t pre = 0;
  for (int w = 0; w < wave; ++w) pre += wsum[w];
  __syncthreads();   // wsum is free again
  return v + pre;
}

// All NTH threads call this.  idx may be in global memory or LDS.  On
// return (after a barrier) L.h[e] holds counts and L.s[e] the inclusive scan
// of counts, for e < E.  *err (if not null) is 1 when an id was outside
// [0, E), else 0.
template <int NTH>
__device__ void block_permute(PermuteLds<NTH>& L, const int32_t* idx, int N, int E,
                              int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                              int32_t* __restrict__ perm, int32_t* __restrict__ pos,
                              int32_t* __restrict__ err) {
  constexpr int W = NTH / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e <= E; e += NTH) L.h[e] = 0;
  for (int e = tid; e < PMAXE; e += NTH)
#pragma unroll
    for (int w = 0; w < W; ++w) L.wcnt[w][e] = 0;
  __syncthreads();
  for (int f = tid; f < N; f += NTH) {
    const int e = idx[f];
    atomicAdd(&L.h[(e >= 0 && e < E) ? e : E], 1);
  }
  __syncthreads();
  const int32_t mine = (tid < E) ? L.h[tid] : 0;
  if (tid < E) counts[tid] = mine;
  if (tid == 0 && err) *err = L.h[E] ? 1 : 0;
  const int32_t incl = block_inclusive_scan<NTH>(mine, L.wsum);
  L.s[tid] = incl;
  const int32_t excl = incl - mine;
  if (tid < E) {
    offsets[tid] = excl;
    L.running[tid] = excl;
  }
  if (tid == E - 1) offsets[E] = incl;
  __syncthreads();
  // Stable scatter, NTH elements at a time in index order: the rank of an
  // element among the equal ids before it (wave ballots on the id bits,
  // then a prefix over the waves), added to the expert's running base.
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int sub = 0; sub < N; sub += NTH) {
    const int f = sub + tid;
    int e = (f < N) ? idx[f] : -1;
    const bool valid = (e >= 0 && e < E);
    if (!valid) e = -1;
    // Lanes holding the same id: match on the 10 low bits (-1 -> 0x3FF, never
    // a valid id since E <= 512).
    uint64_t peers = ~0ull;
#pragma unroll
    for (int bit = 0; bit < 10; ++bit) {
      const bool b = (e >> bit) & 1;
      const uint64_t m = __ballot(b);
      peers &= b ? m : ~m;
    }
    const int rank = __popcll(peers & lt);
    const bool leader = (peers & lt) == 0;
    const int cnt = __popcll(peers);
    if (valid && leader) L.wcnt[wave][e] = cnt;
    __syncthreads();
    if (valid) {
      int p = L.running[e] + rank;
      for (int w = 0; w < wave; ++w) p += L.wcnt[w][e];
      perm[p] = f;
      pos[f] = p;
    }
    __syncthreads();
    if (valid && leader) {
      atomicAdd(&L.running[e], cnt);
      L.wcnt[wave][e] = 0;
    }
    __syncthreads();
  }
}

}  // namespace moe
