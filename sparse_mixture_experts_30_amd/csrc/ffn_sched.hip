// Device-side tile schedule for the grouped expert GEMMs.
//
// Group g < E is routed expert g with rows [offsets[g], offsets[g+1]) of the
// expert-sorted order; group E is the shared expert with all T tokens.  Each
// group is cut into M-tiles of at most BM rows: full tiles and a remainder,
// or (balanced) ceil(n / BM) tiles whose sizes differ by at most one row, so
// that the M-tiles that share a weight tile run at the same pace and its
// second reader finds it in L2.  Entry i of the list (8 int32):
//   [0] group, [1] first row, [2] rows in the tile, [3] first entry of the
//   group (L_g), [4] M-tiles of the group (mt_g).
// tiles[0] holds the number of entries; entries start at tiles + 8.  The
// host never reads the list: the GEMM grids are sized for the largest
// possible count and surplus workgroups exit.
#include "moe_internal.hpp"

#include <algorithm>

namespace moe {

namespace {

__global__ void __launch_bounds__(1024)
build_tiles_kernel(const int32_t* __restrict__ offsets, int E, int64_t T, int has_routed,
                   int has_shared, int BM, int balanced, int32_t* __restrict__ tiles) {
  __shared__ int32_t s[1024];
  const int g = threadIdx.x;
  int32_t n = 0, r0 = 0;
  if (g < E) {
    if (has_routed) {
      r0 = offsets[g];
      n = offsets[g + 1] - r0;
    }
  } else if (g == E && has_shared) {
    n = (int32_t)T;
  }
  const int32_t mt = (n + BM - 1) / BM;
  s[g] = mt;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    int32_t v = (g >= off) ? s[g - off] : 0;
    __syncthreads();
    s[g] += v;
    __syncthreads();
  }
  const int32_t L = s[g] - mt;
  for (int32_t m = 0; m < mt; ++m) {
    int32_t* ent = tiles + 8 + 8 * (int64_t)(L + m);
    // balanced: rows [m n / mt, (m + 1) n / mt), each between floor(n / mt)
    // >= 1 and ceil(n / mt) <= BM rows
    const int32_t a = balanced ? (int32_t)((int64_t)m * n / mt) : m * BM;
    const int32_t b = balanced ? (int32_t)((int64_t)(m + 1) * n / mt) : min(n, (m + 1) * BM);
    ent[0] = g;
    ent[1] = r0 + a;
    ent[2] = b - a;
    ent[3] = L;
    ent[4] = mt;
  }
  if (g == 1023) tiles[0] = s[g];
}

}  // namespace

int64_t ffn_max_mtiles(int64_t N, int64_t T, int E, int BM) {
  return (N + BM - 1) / BM + E + (T + BM - 1) / BM;
}

hipError_t launch_build_tiles(const int32_t* offsets, int E, int64_t T, bool has_routed,
                              bool has_shared, int BM, int32_t* tiles, hipStream_t s,
                              bool balanced) {
  MOE_TIMED_LAUNCH(s, "build_tiles_kernel",
    hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(1024), 0, s, offsets, E, T,
                       has_routed ? 1 : 0, has_shared ? 1 : 0, BM, balanced ? 1 : 0, tiles));
  return hipGetLastError();
}

int64_t ffn_grid_mtiles(const FfnDims& d, int BM) {
  // At most min(E, N) routed groups have rows, each with at most one
  // partial tile.
  const bool routed = d.groups & kGroupRouted, shared = (d.groups & kGroupShared) && d.Is > 0;
  return (routed ? (d.N + BM - 1) / BM + std::min<int64_t>(d.E, d.N) : 0) +
         (shared ? (d.T + BM - 1) / BM : 0);
}

hipError_t ffn_build_tiles(const FfnDims& d, const int32_t* offsets, int BM, int32_t* tiles,
                           hipStream_t s, bool balanced) {
  if (d.tiles_ready && d.T <= BM) return hipSuccess;
  return launch_build_tiles(offsets, d.E, d.T, d.groups & kGroupRouted,
                            (d.groups & kGroupShared) && d.Is > 0, BM, tiles, s, balanced);
}
}  // namespace moe
