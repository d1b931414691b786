// Token permutation by expert (page "从 1024 块 GPU 到 558 万美元：拆解 DeepSeek-V3 的算法-系统协同设计",
// section 2.3: per-expert counts from the one-hot of the chosen ids, then the
// flattened ids sorted so each expert's tokens are contiguous).
//
// counts[e] = #{f : idx[f] == e}; offsets = exclusive scan; perm lists flat
// indices f = t*K + k grouped by expert, ascending f inside an expert (a
// stable sort); pos = inverse of perm.
//
// Three launches (one for a single chunk), no global atomics, deterministic:
//   1. per-block histograms in LDS over chunks of the flat index range;
//   2. one block: per-expert totals, exclusive scan over experts, and the
//      base position of every (block, expert) pair;
//   3. per block, chunks of 256 in order: the rank of each element among the
//      equal ids before it (wave ballots on the id bits, then a prefix over the
//      waves), added to the running base.
#include "moe_internal.hpp"
#include "permute_device.hpp"

namespace moe {

namespace {

constexpr int PCHUNK = 2048;   // flat indices per block
constexpr int PTHREADS = 256;

__global__ void __launch_bounds__(PTHREADS)
hist_kernel(const int32_t* __restrict__ idx, int64_t N, int E, int32_t* __restrict__ hist) {
  __shared__ int32_t h[PMAXE + 1];   // h[E] counts ids outside [0, E)
  for (int e = threadIdx.x; e <= E; e += PTHREADS) h[e] = 0;
  __syncthreads();
  const int64_t f0 = (int64_t)blockIdx.x * PCHUNK;
  for (int j = threadIdx.x; j < PCHUNK; j += PTHREADS) {
    int64_t f = f0 + j;
    if (f < N) {
      int e = idx[f];
      atomicAdd(&h[(e >= 0 && e < E) ? e : E], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e <= E; e += PTHREADS) hist[(int64_t)blockIdx.x * (E + 1) + e] = h[e];
}

// One block of PMAXE threads.  hist[b][e] (row stride E + 1) becomes the base
// position of block b's elements of expert e; *err is set to 1 if any id was
// outside [0, E), else 0 (each call rewrites it).
__global__ void __launch_bounds__(PMAXE)
scan_kernel(int32_t* __restrict__ hist, int nblk, int E, int32_t* __restrict__ counts,
            int32_t* __restrict__ offsets, int32_t* __restrict__ err) {
  constexpr int B = 16;   // histogram rows read per batch (independent loads)
  __shared__ int32_t s[PMAXE];
  const int e = threadIdx.x;
  const int64_t ld = E + 1;
  // Per-expert total over the blocks (thread E also totals the invalid ids).
  int32_t total = 0;
  if (e <= E) {
    for (int b0 = 0; b0 < nblk; b0 += B) {
      int32_t v[B];
#pragma unroll
      for (int j = 0; j < B; ++j) v[j] = (b0 + j < nblk) ? hist[(b0 + j) * ld + e] : 0;
#pragma unroll
      for (int j = 0; j < B; ++j) total += v[j];
    }
  }
  if (e == E) *err = total ? 1 : 0;
  const int32_t mine = (e < E) ? total : 0;
  if (e < E) counts[e] = mine;
  s[e] = mine;
  __syncthreads();
  // Hillis-Steele inclusive scan over experts.
  for (int off = 1; off < PMAXE; off <<= 1) {
    int32_t v = (e >= off) ? s[e - off] : 0;
    __syncthreads();
    s[e] += v;
    __syncthreads();
  }
  const int32_t excl = s[e] - mine;
  if (e < E) {
    offsets[e] = excl;
    // hist[b][e] becomes the first position of block b's elements of e.
    int32_t run = excl;
    for (int b0 = 0; b0 < nblk; b0 += B) {
      int32_t v[B];
#pragma unroll
      for (int j = 0; j < B; ++j) v[j] = (b0 + j < nblk) ? hist[(b0 + j) * ld + e] : 0;
#pragma unroll
      for (int j = 0; j < B; ++j) {
        if (b0 + j < nblk) hist[(b0 + j) * ld + e] = run;
        run += v[j];
      }
    }
  }
  if (e == E - 1) offsets[E] = s[e];
}

__global__ void __launch_bounds__(PTHREADS)
scatter_kernel(const int32_t* __restrict__ idx, int64_t N, int E,
               const int32_t* __restrict__ base, int32_t* __restrict__ perm,
               int32_t* __restrict__ pos) {
  __shared__ int32_t running[PMAXE];
  __shared__ int32_t wcnt[PTHREADS / 64][PMAXE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += PTHREADS) {
    running[e] = base[(int64_t)blockIdx.x * (E + 1) + e];
#pragma unroll
    for (int w = 0; w < PTHREADS / 64; ++w) wcnt[w][e] = 0;
  }
  __syncthreads();
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t f0 = (int64_t)blockIdx.x * PCHUNK;
  for (int sub = 0; sub < PCHUNK; sub += PTHREADS) {
    const int64_t f = f0 + sub + tid;
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
    if (valid && leader) wcnt[wave][e] = cnt;
    __syncthreads();
    if (valid) {
      int p = running[e] + rank;
      for (int w = 0; w < wave; ++w) p += wcnt[w][e];
      perm[p] = (int32_t)f;
      pos[f] = p;
    }
    __syncthreads();
    if (valid && leader) {
      atomicAdd(&running[e], cnt);
      wcnt[wave][e] = 0;
    }
    __syncthreads();
  }
}

// All three steps in one block of PMAXE threads, for N <= PCHUNK (decode
// batches), where the launches of the three-kernel path would dominate.
__global__ void __launch_bounds__(PMAXE)
permute_small_kernel(const int32_t* __restrict__ idx, int N, int E, int32_t* __restrict__ counts,
                     int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                     int32_t* __restrict__ pos, int32_t* __restrict__ err) {
  __shared__ PermuteLds<PMAXE> L;
  block_permute<PMAXE>(L, idx, N, E, counts, offsets, perm, pos, err);
}

}  // namespace

int permute_nblk(int64_t N) { return (int)((N + PCHUNK - 1) / PCHUNK); }

hipError_t launch_permute(const int32_t* idx, int64_t N, int E, int32_t* hist, int32_t* counts,
                          int32_t* offsets, int32_t* perm, int32_t* pos, int32_t* err,
                          hipStream_t s) {
  const int nblk = permute_nblk(N);
  if (nblk == 1) {
    MOE_TIMED_LAUNCH(s, "permute_small_kernel",
      hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(PMAXE), 0, s, idx, (int)N, E, counts,
                         offsets, perm, pos, err));
    return hipGetLastError();
  }
  MOE_TIMED_LAUNCH(s, "hist_kernel",
    hipLaunchKernelGGL(hist_kernel, dim3(nblk), dim3(PTHREADS), 0, s, idx, N, E, hist));
  MOE_TIMED_LAUNCH(s, "scan_kernel",
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(PMAXE), 0, s, hist, nblk, E, counts, offsets, err));
  MOE_TIMED_LAUNCH(s, "scatter_kernel",
    hipLaunchKernelGGL(scatter_kernel, dim3(nblk), dim3(PTHREADS), 0, s, idx, N, E,
                       (const int32_t*)hist, perm, pos));
  return hipGetLastError();
}

}  // namespace moe
