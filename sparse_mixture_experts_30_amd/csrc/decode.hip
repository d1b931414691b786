// Routing for decode batches (T <= kDecodeMaxT tokens): the gate, the
// selection, the permutation and the expert tile list in three launches.
//
// The method is the one of the batch path (page "从 1024 块 GPU 到 558 万美元：
// 拆解 DeepSeek-V3 的算法-系统协同设计", sections 2.2 and 2.3): logits = x W^T in
// fp32, sigmoid scores with the selection-only bias, group-limited top-k,
// weights from the unbiased scores; then per-expert counts and a stable sort
// of the flat ids by expert.  What changes is the schedule, for a batch too
// small to fill the GPU with any one step:
//
//   1. the gate, over k ranges of at most 896 elements.  bf16 activations
//      (gate_decode_mfma_kernel): a workgroup takes 32 experts and one k
//      range; each wave issues all of its loads at once (one memory round
//      trip), splits the fp32 gate weights in registers into their exact
//      bf16 parts and accumulates the three bf16 MFMA products in fp32.
//      fp32 activations (gate_decode_kernel): a workgroup takes 8 experts,
//      copies the range of all T token rows and of its 8 gate rows into LDS
//      with every load issued at once, then forms the fp32 dot products on
//      the vector ALUs (eight accumulators per thread added in a fixed tree).
//      Either way the gate weight is read once, straight from its fp32 copy;
//      no split copy of it is made.
//   2. the batch path's selection kernel, over the few k-range partials.
//   3. route_decode_kernel: one workgroup permutes the T*K flat ids and
//      writes the tile list of the expert GEMMs (one tile per non-empty
//      group, since no group has more rows than T).
//
// The batch path needs five launches for the same steps (weight split, gate
// GEMM with a deep k split, selection, permutation, tile list).
#include "moe_internal.hpp"
#include "decode_device.hpp"
#include "permute_device.hpp"

#include <algorithm>

namespace moe {

namespace {

constexpr int DG_EXPERTS = 8;     // experts per gate workgroup
constexpr int DG_THREADS = 256;   // 8 experts x 32 token slots
constexpr int DR_THREADS = 1024;  // routing workgroup
static_assert(kDecodeMaxT <= 32, "one thread per token slot in the gate workgroup");
static_assert(kDecodeMaxT <= kMinTileRows, "a decode group fits one tile of every GEMM");

__device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
  const u32x4 q = *reinterpret_cast<const u32x4*>(p);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = __uint_as_float(w[j] << 16);
    v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const u32x4 a = *reinterpret_cast<const u32x4*>(p);
  const u32x4 b = *reinterpret_cast<const u32x4*>(p + 4);
  v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
  v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
  v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
  v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
}


// part[ks][t][e] = sum over k in [ks * kchunk, min(H, (ks + 1) * kchunk)) of
// x[t][k] * wg[e][k] (fp32 activations).  Thread (el, t): el = tid / 32
// picks the expert of the workgroup's eight, t = tid % 32 the token.  kchunk
// and H are multiples of 8.
// LDS: the token rows (row stride kchunk / XV + 1 chunks of 16 bytes, so
// that the 32 rows read at one k fall in different banks), then the 8 gate
// rows.
template <typename XT>
__global__ void __launch_bounds__(DG_THREADS)
gate_decode_kernel(const XT* __restrict__ x, const float* __restrict__ wg,
                   float* __restrict__ part, int T, int H, int E, int kchunk) {
  extern __shared__ u32x4 lds[];
  constexpr int XV = 16 / sizeof(XT);   // elements of x per 16 bytes
  const int tid = threadIdx.x;
  const int e0 = blockIdx.x * DG_EXPERTS, ks = blockIdx.y;
  const int k0 = ks * kchunk, kn = min(H, k0 + kchunk) - k0;
  const int xstride = kchunk / XV + 1;  // 16-byte chunks per LDS token row
  const int xc = kn / XV, wc = kn / 4;  // 16-byte chunks of one row in this range
  u32x4* sx = lds;
  u32x4* sw = lds + T * xstride;        // [8][kchunk / 4]

  // Every load of the range is issued before the first LDS store.
  constexpr int XL = (kDecodeMaxT * (DG_MAXK / XV) + DG_THREADS - 1) / DG_THREADS;
  constexpr int WL = (DG_EXPERTS * (DG_MAXK / 4) + DG_THREADS - 1) / DG_THREADS;
  u32x4 rx[XL], rw[WL];
#pragma unroll
  for (int j = 0; j < XL; ++j) {
    const int c = tid + j * DG_THREADS;
    if (c < T * xc) {
      const int r = c / xc, q = c - r * xc;
      rx[j] = *reinterpret_cast<const u32x4*>(x + (int64_t)r * H + k0 + q * XV);
    }
  }
#pragma unroll
  for (int j = 0; j < WL; ++j) {
    const int c = tid + j * DG_THREADS;
    if (c < DG_EXPERTS * wc) {
      const int r = c / wc, q = c - r * wc;
      const int e = min(e0 + r, E - 1);   // rows past E re-read a valid row (results dropped)
      rw[j] = *reinterpret_cast<const u32x4*>(wg + (int64_t)e * H + k0 + q * 4);
    }
  }
#pragma unroll
  for (int j = 0; j < XL; ++j) {
    const int c = tid + j * DG_THREADS;
    if (c < T * xc) {
      const int r = c / xc, q = c - r * xc;
      sx[r * xstride + q] = rx[j];
    }
  }
#pragma unroll
  for (int j = 0; j < WL; ++j) {
    const int c = tid + j * DG_THREADS;
    if (c < DG_EXPERTS * wc) {
      const int r = c / wc, q = c - r * wc;
      sw[r * (kchunk / 4) + q] = rw[j];
    }
  }
  __syncthreads();

  const int t = tid & 31, el = tid >> 5, e = e0 + el;
  if (t >= T || e >= E) return;   // after the only barrier
  const XT* xr = reinterpret_cast<const XT*>(sx + t * xstride);
  const float* wr = reinterpret_cast<const float*>(sw + el * (kchunk / 4));
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int k = 0; k < kn; k += 8) {
    float xv[8], wv[8];
    load8(xr + k, xv);
    load8(wr + k, wv);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = fmaf(xv[j], wv[j], acc[j]);
  }
  const float sum = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
  part[((int64_t)ks * T + t) * E + e] = sum;
}

// bf16 activations: the same partial sums on bf16 MFMA (gate_mfma_item,
// decode_device.hpp).  Workgroup (eb, ks) takes experts 32 eb .. 32 eb + 31
// and the ks-th k range.
__global__ void __launch_bounds__(DG_THREADS)
gate_decode_mfma_kernel(const uint16_t* __restrict__ x, const float* __restrict__ wg,
                        float* __restrict__ part, int T, int H, int E, int kchunk) {
  __shared__ float red[3][16][kWave];   // accumulators of waves 1..3
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  gate_mfma_item(x, wg, part, T, H, E, kchunk, blockIdx.x, blockIdx.y, wave, true, red);
}

// One workgroup: the permutation of the T*K chosen ids, and (when tiles is
// not null) the tile list with the routed groups (has_routed) and the shared
// group E (has_shared).
__global__ void __launch_bounds__(DR_THREADS)
route_decode_kernel(const int32_t* __restrict__ idx, int T, int E, int K,
                    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                    int32_t* __restrict__ perm, int32_t* __restrict__ pos,
                    int32_t* __restrict__ err, int32_t* __restrict__ tiles, int has_routed,
                    int has_shared) {
  __shared__ PermuteLds<DR_THREADS> L;
  const int tid = threadIdx.x;
  block_permute<DR_THREADS>(L, idx, T * K, E, counts, offsets, perm, pos, err);
  if (!tiles) return;   // uniform

  // Tile list (format of build_tiles_kernel): one tile per non-empty group.
  const int g = tid;
  int32_t n = 0, r0 = 0;
  if (g < E && has_routed) {
    n = L.h[g];
    r0 = L.s[g] - n;
  } else if (g == E && has_shared) {
    n = T;
  }
  const int32_t mt = n > 0 ? 1 : 0;
  const int32_t end = block_inclusive_scan<DR_THREADS>(mt, L.wsum);
  if (mt) {
    int32_t* ent = tiles + 8 + 8 * (int64_t)(end - 1);
    ent[0] = g;
    ent[1] = r0;
    ent[2] = n;
    ent[3] = end - 1;
    ent[4] = 1;
  }
  if (g == DR_THREADS - 1) tiles[0] = end;
}

size_t gate_decode_lds(int T, int kchunk, int xbytes) {
  return (size_t)T * (kchunk * xbytes / 16 + 1) * 16 + (size_t)DG_EXPERTS * kchunk * 4;
}

hipError_t set_gate_decode_attrs() {
  static hipError_t once = []() {
    const int f32 = (int)gate_decode_lds(kDecodeMaxT, DG_MAXK, 4);
    return hipFuncSetAttribute((const void*)gate_decode_kernel<float>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, f32);
  }();
  return once;
}

}  // namespace

bool decode_route_ok(int64_t T, int H, int E, int K) {
  return T >= 1 && T <= kDecodeMaxT && E <= PMAXE && E + 1 <= DR_THREADS && K <= 64 &&
         H % 8 == 0 && H <= 64 * DG_MAXK;
}

int decode_ksplit(int H, int E) {
  // ~256 workgroups, k ranges of at least 64 and at most DG_MAXK elements
  const int eb = (E + DG_EXPERTS - 1) / DG_EXPERTS;
  int ks = std::max(1, std::min(32, 256 / eb));
  ks = std::min(ks, std::max(1, H / 64));
  ks = std::max(ks, (H + DG_MAXK - 1) / DG_MAXK);
  const int kchunk = ((H + ks - 1) / ks + 7) / 8 * 8;
  return (H + kchunk - 1) / kchunk;
}

hipError_t launch_decode_route(const void* x, bool x_bf16, const float* gate_w,
                               const float* bias, float* partials, float* logits_out,
                               int32_t* idx, float* w, int64_t T, int H, int E, int G, int TG,
                               int K, float rho, int32_t* counts, int32_t* offsets,
                               int32_t* perm, int32_t* pos, int32_t* err, int32_t* tiles,
                               bool has_routed, bool has_shared, hipStream_t s) {
  hipError_t e = set_gate_decode_attrs();
  if (e != hipSuccess) return e;
  const int ks = decode_ksplit(H, E);
  const int kchunk = ((H + ks - 1) / ks + 7) / 8 * 8;
  if (kchunk > DG_MAXK) return hipErrorInvalidValue;   // bounds both gate kernels
  if (x_bf16)
    MOE_TIMED_LAUNCH(s, "gate_decode_mfma_kernel",
      hipLaunchKernelGGL(gate_decode_mfma_kernel, dim3((E + 31) / 32, ks), dim3(DG_THREADS), 0,
                         s, (const uint16_t*)x, gate_w, partials, (int)T, H, E, kchunk));
  else
    MOE_TIMED_LAUNCH(s, "gate_decode_kernel",
      hipLaunchKernelGGL(gate_decode_kernel<float>, dim3((E + DG_EXPERTS - 1) / DG_EXPERTS, ks),
                         dim3(DG_THREADS), gate_decode_lds((int)T, kchunk, 4), s,
                         (const float*)x, gate_w, partials, (int)T, H, E, kchunk));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = launch_select(partials, ks, bias, logits_out, idx, w, T, E, G, TG, K, rho, s)) !=
      hipSuccess)
    return e;
  MOE_TIMED_LAUNCH(s, "route_decode_kernel",
    hipLaunchKernelGGL(route_decode_kernel, dim3(1), dim3(DR_THREADS), 0, s, idx, (int)T, E, K,
                       counts, offsets, perm, pos, err, tiles, has_routed ? 1 : 0,
                       has_shared ? 1 : 0));
  return hipGetLastError();
}

}  // namespace moe
