// Grouped expert GEMMs on bf16 MFMA with weights in the packed streaming
// layout (gfx950), fp32 accumulation.
//
// Same layer math as the row-major kernel (SwiGLU experts, the shared expert
// as group E; mqxn.cn/news/19449, section 3.1; "从 1024 块 GPU 到 558 万美元：
// 拆解 DeepSeek-V3 的算法-系统协同设计", section 2.2).  The weights, read exactly
// once per call, dominate the traffic.  In the packed layout every
// (matrix, output tile, 64-k step) is one contiguous 32 KiB block holding the
// MFMA operand fragments in consumption order:
//   block = [wave 4][col block 2][k slice 4][lane 64] x 16 bytes
//   lane l of (wave w, col block cb, slice kk) holds weight row
//     GEMM1: cb = 0 gate row n0 + 32w + l%32, cb = 1 up row I + n0 + 32w + l%32
//     GEMM2: row n0 + 64w + 32cb + l%32
//   at k = 64 step + 32 (l / 32) + 8 kk .. +8 (rows past the matrix: zeros).
// Each wave loads its fragments with fully coalesced 1 KiB loads straight
// into registers, a step ahead, with no LDS traffic; the activation rows
// (shared by the 4 waves) use the double-buffered LDS tile of the row-major
// kernel, with the same k assignment (lane half lh holds k in
// [32 lh, 32 lh + 32)).
#include "moe_internal.hpp"
#include "packed_few.hpp"

#include <algorithm>

namespace moe {

namespace {

constexpr int BM = 256;    // max rows per tile
constexpr int BK = kPackedBK;  // k per step
constexpr int NT = 256;    // threads
// Pipeline depth D in steps: the weights of steps t .. t+D-1 and the
// activation rows of steps t+1 .. t+D sit in registers (or are in flight)
// while step t computes, so loads get D-1 steps to arrive.  On gfx950 one
// step of lead already covers the load latency for every tile height (a
// deeper pipeline only costs registers), so D = 2 throughout.
constexpr int depth_for(int) { return 2; }
constexpr int FRAG = kPackedFrag; // 16-byte fragments per packed block (32 KiB)
constexpr size_t kLdsP = (size_t)2 * BM * 8 * sizeof(u32x4);   // 64 KiB

// ---------------------------------------------------------------- packing

// dst fragment c of a packed matrix with `nt` output tiles and `steps` k
// steps per expert; src row-major [experts][rows_total][kd].
template <bool kGateUp>
__global__ void __launch_bounds__(256)
pack_kernel(const uint16_t* __restrict__ src, u32x4* __restrict__ dst, int64_t nfrag, int n,
            int kd, int rows_total, int nt, int steps) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= nfrag) return;
  const int l = (int)(c & 63), kk = (int)((c >> 6) & 3), cb = (int)((c >> 8) & 1),
            w = (int)((c >> 9) & 3);
  const int64_t rest = c >> 11;
  const int ks = (int)(rest % steps);
  const int64_t rest2 = rest / steps;
  const int tile = (int)(rest2 % nt);
  const int64_t e = rest2 / nt;
  int row;
  bool ok;
  if (kGateUp) {
    const int col = tile * 128 + 32 * w + (l & 31);
    ok = col < n;
    row = cb ? n + col : col;
  } else {
    row = tile * 256 + 64 * w + 32 * cb + (l & 31);
    ok = row < n;
  }
  const int k = ks * BK + 32 * (l >> 5) + 8 * kk;
  u32x4 v = {0, 0, 0, 0};
  if (ok) v = *reinterpret_cast<const u32x4*>(src + (e * rows_total + row) * (int64_t)kd + k);
  dst[c] = v;
}

// ---------------------------------------------------------------- GEMM

__device__ __forceinline__ int swz(int r, int c) { return r * 8 + (c ^ ((r ^ (r >> 3)) & 7)); }

// The work of one tile with NRB 32-row blocks (compile time, so the MFMA
// loop has no branches and the fragment reads of a k slice can all be in
// flight together).  NCB is the number of 32-column weight blocks per wave:
//   NCB = 2: the tile is one packed tile (256 weight rows); wave w takes its
//            own quarter (packed wave slot w).
//   NCB = 4: the tile is two adjacent packed tiles (512 weight rows); wave w
//            takes slots 2 (w % 2) and 2 (w % 2) + 1 of packed tile
//            2 ntile + w / 2, two contiguous 8 KiB pieces per step.  Each
//            activation fragment read from LDS then feeds four MFMAs
//            instead of two, halving the LDS read traffic per MFMA.
template <bool kGateUp, int NRB, int D, bool kStream, int kBM, int NCB = 2>
__device__ __forceinline__ void packed_tile(const PackedArgs& p, u32x4* sA, int g, int row0,
                                            int nrows, int ntile) {
  static_assert(NCB == 2 || NCB == 4, "column blocks per wave");
  constexpr int NB = 4 * NCB;   // weight fragments per wave per step
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lh = lane >> 5;
  const bool sh = (g == p.E);
  const int ncol = sh ? p.ncol_s : p.ncol_r;
  const int nt = sh ? p.nt_s : p.nt_r;
  // packed tile of this wave and its first wave slot in that tile
  int wtile = NCB == 2 ? ntile : 2 * ntile + (wave >> 1);
  const bool wvalid = wtile < nt;   // the second half of a ragged wide tile
  wtile = min(wtile, nt - 1);
  const int slot0 = NCB == 2 ? wave : 2 * (wave & 1);
  const int n0 = wtile * (kGateUp ? 128 : 256);
  const int kdim = sh ? p.kdim_s : p.kdim_r;
  const int nsteps = kdim / BK;
  const int last = nsteps - 1;
  const uint16_t* A = sh ? p.a_s : p.a_r;
  const int64_t lda = sh ? p.lda_s : p.lda_r;
  const u32x4* bw = (sh ? p.b_s : p.b_r + (int64_t)g * p.nt_r * nsteps * FRAG) +
                    (int64_t)wtile * nsteps * FRAG + slot0 * 512 + lane;

  // Activation rows staged by this thread: r = tid/8 + 32 j (j < NRB),
  // chunk tid % 8 (rows past the tile's end re-read the first row).
  const int ch = tid & 7;
  const int first = (!sh && kGateUp) ? p.perm[row0] / p.K : row0;
  int arow[NRB];
#pragma unroll
  for (int j = 0; j < NRB; ++j) {
    const int r = (tid >> 3) + 32 * j;
    int a = first;
    if (r < nrows) a = (!sh && kGateUp) ? p.perm[row0 + r] / p.K : row0 + r;
    arow[j] = a;
  }
  const uint16_t* abase = A + ch * 8;
  u32x4 ra[D][NRB];   // register stages of activation rows
  auto aload = [&](u32x4 (&st)[NRB], int j, int step) {
    st[j] = *reinterpret_cast<const u32x4*>(abase + (int64_t)arow[j] * lda +
                                            min(step, last) * BK);
  };
  auto astore = [&](const u32x4 (&st)[NRB], int j, int buf) {
    sA[buf * kBM * 8 + swz((tid >> 3) + 32 * j, ch)] = st[j];
  };
  u32x4 rb[D][NB];    // weight fragments [slot][c * 4 + kk], c = column block
  // Issued in the order the step refills them (slice by slice), so that the
  // wait counts the compiler merges at the loop head match on both paths.
  auto bload = [&](u32x4 (&dst)[NB], int step) {
    const u32x4* src = bw + (int64_t)min(step, last) * FRAG;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int c = 0; c < NCB; ++c) {
        const int i = c * 4 + kk;
        dst[i] = kStream ? __builtin_nontemporal_load(src + i * 64) : src[i * 64];
        __builtin_amdgcn_sched_barrier(0);   // keep the issue order
      }
  };

  f32x16 acc[NRB][NCB];
#pragma unroll
  for (int r = 0; r < NRB; ++r)
#pragma unroll
    for (int c = 0; c < NCB; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[r][c][i] = 0.0f;

  // One step on LDS buffer `buf` with weight slot `b`.  The instruction
  // order is fixed by hand (scheduling barriers): each pair of MFMAs of row
  // block r is followed by the LDS read of row block r's fragment for the
  // next k slice and by at most one memory operation, so loads, LDS traffic
  // and matrix work stay interleaved instead of queueing up in bursts.
  // Memory operations of slice kk: the activation chunks j = kk, kk + 4 of
  // the next step move from registers `st` to LDS buffer `nbuf` and `st` is
  // refilled with step `ld`; after the slice's last MFMA its two weight
  // fragments, no longer needed, are refilled with step `bld`.
  auto step_body = [&](int buf, u32x4 (&b)[NB], u32x4 (&st)[NRB], int nbuf, int ld, int bld) {
    const u32x4* as = sA + buf * kBM * 8;
    const u32x4* bsrc = bw + (int64_t)min(bld, last) * FRAG;
    bf16x8 a[2][NRB];
#pragma unroll
    for (int r = 0; r < NRB; ++r) a[0][r] = as_bf16x8(as[swz(r * 32 + lr, 4 * lh)]);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8 bf[NCB];
#pragma unroll
      for (int c = 0; c < NCB; ++c) bf[c] = as_bf16x8(b[c * 4 + kk]);
      // activation chunk operations of this slice, in order
      constexpr int kOps = 2 * ((NRB + 3) / 4);
      int nop = 0;
#pragma unroll
      for (int r = 0; r < NRB; ++r) {
        acc[r][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk & 1][r], bf[0], acc[r][0], 0, 0, 0);
        if (kk < 3) a[(kk + 1) & 1][r] = as_bf16x8(as[swz(r * 32 + lr, 4 * lh + kk + 1)]);
#pragma unroll
        for (int c = 1; c < NCB; ++c)
          acc[r][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk & 1][r], bf[c], acc[r][c], 0, 0, 0);
        // one activation operation per group (all of them by the last group)
        const int upto = (r == NRB - 1) ? kOps : r + 1;
#pragma unroll
        for (; nop < upto && nop < kOps; ++nop) {
          const int j = kk + 4 * (nop >> 1);
          if (j < NRB) {
            if ((nop & 1) == 0) astore(st, j, nbuf);
            else aload(st, j, ld);
          }
        }
        if (r == NRB - 1) {
#pragma unroll
          for (int c = 0; c < NCB; ++c)
            b[c * 4 + kk] = kStream ? __builtin_nontemporal_load(bsrc + (c * 4 + kk) * 64)
                                    : bsrc[(c * 4 + kk) * 64];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Prologue: activations of step 0 into LDS buffer 0, of steps 1..D into
  // ra[1 % D] .. ra[D % D], weights of steps 0..D-1 into rb.  The loads are
  // issued in the order the loop issues them (activations of step j + 1, then
  // weights of step j), so that at the loop head every register has as many
  // younger loads on entry as on the back edge: the compiler's wait counts,
  // merged over both paths, then wait only for the step about to be used.
  auto aload_all = [&](u32x4 (&st)[NRB], int step) {
#pragma unroll
    for (int j = 0; j < NRB; ++j) {
      aload(st, j, step);
      __builtin_amdgcn_sched_barrier(0);   // keep the issue order
    }
  };
  aload_all(ra[0], 0);
#pragma unroll
  for (int j = 0; j < D; ++j) {
    if ((j + 1) % D == 0) {
#pragma unroll
      for (int i = 0; i < NRB; ++i) astore(ra[0], i, 0);
    }
    aload_all(ra[(j + 1) % D], j + 1);
    bload(rb[j], j);
  }
  __syncthreads();

  // Step t: LDS buffer t % 2 holds its activations, rb[t % D] its weights,
  // ra[(t + 1) % D] those of step t + 1 (moved to the other LDS buffer during
  // the step and refilled with step t + 1 + D).  Unrolled by U = lcm(D, 2)
  // so every index is static.
  constexpr int U = (D % 2) ? 2 * D : D;
  auto step = [&](int t, int u) {
    step_body(u & 1, rb[u % D], ra[(u + 1) % D], (u + 1) & 1, t + 1 + D, t + D);
    __syncthreads();
  };
  int s = 0;
  for (; s + U <= nsteps; s += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) step(s + u, u);
  }
  // Tail of fewer than U steps (k dimensions that are not a multiple of
  // U * 64); the guard is uniform across the workgroup.
#pragma unroll
  for (int u = 0; u < U - 1; ++u)
    if (s + u < nsteps) step(s + u, u);

  // Epilogue: lane holds column lane%32, rows 8*(i/4) + 4*(lane/32) + i%4.
  // Column block c of the wave is (packed slot slot0 + c / 2, block c % 2).
  if (!wvalid) return;
  uint16_t* C = sh ? p.c_s : p.c_r;
  const int64_t ldc = sh ? p.ldc_s : p.ldc_r;
#pragma unroll
  for (int r = 0; r < NRB; ++r) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = r * 32 + 8 * (i >> 2) + 4 * lh + (i & 3);
      if (row >= nrows) continue;
      uint16_t* crow = C + (int64_t)(row0 + row) * ldc;
      if (kGateUp) {
#pragma unroll
        for (int j = 0; j < NCB / 2; ++j) {
          const int col = n0 + (slot0 + j) * 32 + lr;
          if (col < ncol) {
            const float gv = acc[r][2 * j][i], uv = acc[r][2 * j + 1][i];
            crow[col] = (uint16_t)f32_to_bf16_bits(gv / (1.0f + __expf(-gv)) * uv);
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < NCB; ++c) {
          const int col = n0 + (slot0 + (c >> 1)) * 64 + (c & 1) * 32 + lr;
          if (col < ncol) crow[col] = (uint16_t)f32_to_bf16_bits(acc[r][c][i]);
        }
      }
    }
  }
}

template <bool kGateUp>
__global__ void __launch_bounds__(NT, 1) grouped_gemm_bf16_packed(PackedArgs p) {
  extern __shared__ u32x4 smem[];
  const int64_t work = (int64_t)p.tiles[0] * p.ntn;
  const int64_t w = xcd_chunked(blockIdx.x, work);
  if (w < 0) return;
  int ntile;
  const int32_t* ent = decode_work(p.tiles, w, p.ntn, ntile);
  const int g = ent[0], row0 = ent[1], nrows = ent[2];
  if (ntile >= ((g == p.E) ? p.nt_s : p.nt_r)) return;
  // A weight tile read by one M-tile only streams past the caches
  // (non-temporal loads); one shared by several M-tiles of a group (their
  // workgroups run side by side on one XCD) is kept in L2 for the others.
  const bool stream = ent[4] == 1;
  switch (((nrows + 31) >> 5) * 2 + (stream ? 1 : 0)) {
#define MOE_TILE_CASE(n)                                                                      \
    case 2 * n:                                                                               \
      packed_tile<kGateUp, n, depth_for(n), false, BM>(p, smem, g, row0, nrows, ntile);       \
      break;                                                                                  \
    case 2 * n + 1:                                                                           \
      packed_tile<kGateUp, n, depth_for(n), true, BM>(p, smem, g, row0, nrows, ntile);        \
      break;
    MOE_TILE_CASE(1)
    MOE_TILE_CASE(2)
    MOE_TILE_CASE(3)
    MOE_TILE_CASE(4)
    MOE_TILE_CASE(5)
    MOE_TILE_CASE(6)
    MOE_TILE_CASE(7)
#undef MOE_TILE_CASE
    default:
      if (stream) packed_tile<kGateUp, 8, depth_for(8), true, BM>(p, smem, g, row0, nrows, ntile);
      else packed_tile<kGateUp, 8, depth_for(8), false, BM>(p, smem, g, row0, nrows, ntile);
      break;
  }
}

// Two workgroups per CU: tiles of at most BM2 = 128 rows, a single register
// stage for weights and activations (each weight fragment is refilled for
// the next step right after its last use), so that a wave fits in 256
// registers and two waves share each SIMD, one computing while the other
// waits.  Used for the down projection, whose k dimension (the FFN width) is
// short: with 8 waves per CU the pipeline start of one tile overlaps the
// steady state of the other.
constexpr int BM2 = kMinTileRows;
constexpr size_t kLdsP2 = (size_t)2 * BM2 * 8 * sizeof(u32x4);   // 32 KiB

template <bool kGateUp>
__global__ void __launch_bounds__(NT, 2) grouped_gemm_bf16_packed_x2(PackedArgs p) {
  extern __shared__ u32x4 smem[];
  const int64_t work = (int64_t)p.tiles[0] * p.ntn;
  const int64_t w = xcd_chunked(blockIdx.x, work);
  if (w < 0) return;
  int ntile;
  const int32_t* ent = decode_work(p.tiles, w, p.ntn, ntile);
  const int g = ent[0], row0 = ent[1], nrows = ent[2];
  if (ntile >= ((g == p.E) ? p.nt_s : p.nt_r)) return;
  const bool stream = ent[4] == 1;
  switch (((nrows + 31) >> 5) * 2 + (stream ? 1 : 0)) {
#define MOE_TILE_CASE(n)                                                            \
    case 2 * n: packed_tile<kGateUp, n, 1, false, BM2>(p, smem, g, row0, nrows, ntile); \
      break;                                                                        \
    case 2 * n + 1: packed_tile<kGateUp, n, 1, true, BM2>(p, smem, g, row0, nrows, ntile); \
      break;
    MOE_TILE_CASE(1)
    MOE_TILE_CASE(2)
    MOE_TILE_CASE(3)
    MOE_TILE_CASE(4)
#undef MOE_TILE_CASE
    default:
      break;
  }
}

// Wide tiles for the gate/up projection of large batches (from 256 routed
// rows per expert on average, where the matrix work dominates): 128 rows x
// 512 weight rows, one workgroup per CU, each wave 128 rows x 128 weight rows
// (four column blocks, so every activation fragment read from LDS feeds four
// MFMAs).  The down projection keeps the two-workgroup kernel, which is
// faster there.
constexpr int kWideMinRows = 256;
constexpr int BMW = kMinTileRows;
constexpr size_t kLdsW = (size_t)2 * BMW * 8 * sizeof(u32x4);   // 32 KiB

template <bool kGateUp>
__global__ void __launch_bounds__(NT, 1) grouped_gemm_bf16_packed_wide(PackedArgs p) {
  extern __shared__ u32x4 smem[];
  const int64_t work = (int64_t)p.tiles[0] * p.ntn;
  const int64_t w = xcd_chunked(blockIdx.x, work);
  if (w < 0) return;
  int ntile;
  const int32_t* ent = decode_work(p.tiles, w, p.ntn, ntile);
  const int g = ent[0], row0 = ent[1], nrows = ent[2];
  if (2 * ntile >= ((g == p.E) ? p.nt_s : p.nt_r)) return;
  const bool stream = ent[4] == 1;
  switch (((nrows + 31) >> 5) * 2 + (stream ? 1 : 0)) {
#define MOE_TILE_CASE(n)                                                                     \
    case 2 * n:                                                                              \
      packed_tile<kGateUp, n, 2, false, BMW, 4>(p, smem, g, row0, nrows, ntile);             \
      break;                                                                                 \
    case 2 * n + 1:                                                                          \
      packed_tile<kGateUp, n, 2, true, BMW, 4>(p, smem, g, row0, nrows, ntile);              \
      break;
    MOE_TILE_CASE(1)
    MOE_TILE_CASE(2)
    MOE_TILE_CASE(3)
    MOE_TILE_CASE(4)
#undef MOE_TILE_CASE
    default:
      break;
  }
}

// Wave slots of the GPU at four waves per SIMD (256 CUs x 4 SIMDs x 4).
constexpr int64_t kFewDenseSlots = 4096;

// Few-row variant (decode batches): one wave per workgroup, each running one
// wave slot of one tile (few_tile); see packed_few.hpp.
// WPE = 2: two waves per SIMD with three steps in flight for single-block
// tiles.  WPE = 4 (the down projection of a batch whose waves all fit in
// one round at four per SIMD): two steps in flight, so that every wave is
// resident at once instead of a few running in a second round.
template <bool kGateUp, int NRB, int WPE = 2>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(WPE)))
grouped_gemm_bf16_packed_few(PackedArgs p) {
  constexpr int D = (NRB == 1 && WPE == 2) ? 3 : 2;   // steps of weights + activations in flight
  const int64_t work = (int64_t)p.tiles[0] * p.ntn * kFewSlots;
  const int64_t per = (work + kNumXcd - 1) / kNumXcd;
  const int64_t q = blockIdx.x / kNumXcd;
  const int64_t wi = (int64_t)(blockIdx.x % kNumXcd) * per + q;
  if (q >= per || wi >= work) return;
  const int64_t w = wi / kFewSlots;
  const int wave = (int)(wi % kFewSlots);
  int ntile;
  const int32_t* ent = decode_work(p.tiles, w, p.ntn, ntile);
  const int g = ent[0], row0 = ent[1], nrows = ent[2];
  if (ntile >= (g == p.E ? p.nt_s : p.nt_r)) return;
  few_tile<kGateUp, NRB, D>(p, g, row0, nrows, ntile, wave);
}

hipError_t set_attrs_packed() {
  static hipError_t once = []() {
    hipError_t e = hipFuncSetAttribute((const void*)grouped_gemm_bf16_packed<true>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsP);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)grouped_gemm_bf16_packed_x2<false>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsP2);
    return e;
  }();
  return once;
}

}  // namespace

// Packed sizes in bytes.  GEMM1 matrices (w13, ws13): n = I or Is output
// columns in tiles of 128, kd = H; GEMM2 matrices (w2, ws2): n = H output
// rows in tiles of 256, kd = I or Is.
size_t packed_bytes(bool gate_up, int64_t experts, int n, int kd) {
  const int64_t nt = gate_up ? (n + 127) / 128 : (n + 255) / 256;
  return (size_t)(experts * nt * (kd / BK) * FRAG) * sizeof(u32x4);
}

hipError_t launch_pack(bool gate_up, const uint16_t* src, void* dst, int64_t experts, int n,
                       int kd, hipStream_t s) {
  const int nt = gate_up ? (n + 127) / 128 : (n + 255) / 256;
  const int steps = kd / BK;
  const int64_t nfrag = experts * nt * steps * FRAG;
  const unsigned blocks = (unsigned)((nfrag + 255) / 256);
  if (gate_up)
    MOE_TIMED_LAUNCH(s, "pack_kernel<true>",
      hipLaunchKernelGGL(pack_kernel<true>, dim3(blocks), dim3(256), 0, s, src, (u32x4*)dst, nfrag,
                         n, kd, 2 * n, nt, steps));
  else
    MOE_TIMED_LAUNCH(s, "pack_kernel<false>",
      hipLaunchKernelGGL(pack_kernel<false>, dim3(blocks), dim3(256), 0, s, src, (u32x4*)dst,
                         nfrag, n, kd, n, nt, steps));
  return hipGetLastError();
}

hipError_t launch_ffn_bf16_packed(const FfnDims& d, const uint16_t* x, const int32_t* perm,
                                  const int32_t* offsets, const void* w13p, const void* w2p,
                                  const void* ws13p, const void* ws2p, uint16_t* h,
                                  int32_t* tiles, uint16_t* y, uint16_t* ys, hipStream_t s) {
  hipError_t e = set_attrs_packed();
  if (e != hipSuccess) return e;
  // Small batches take the few-row kernels, which compute 32 * few rows per
  // tile; their tile list is cut at that height, so a group with more rows
  // than T (a caller's routing that names one expert twice for a token) is
  // still covered whole.
  const int few = d.T <= 32 ? 1 : d.T <= 64 ? 2 : 0;
  const bool wide = !few && d.N >= (int64_t)kWideMinRows * d.E;
  const int bm1 = few ? 32 * few : wide ? BMW : BM;
  e = ffn_build_tiles(d, offsets, bm1, tiles, s, true);
  if (e != hipSuccess) return e;
  const int64_t mt = ffn_grid_mtiles(d, bm1);
  uint16_t* hs = h + d.N * d.I;
  auto grid = [](int64_t max_work) {
    return (unsigned)(((max_work + kNumXcd - 1) / kNumXcd) * kNumXcd);
  };

  PackedArgs a1{};
  a1.tiles = tiles;
  a1.nt_r = (d.I + 127) / 128;
  a1.nt_s = (d.Is + 127) / 128;
  a1.ntn = std::max(a1.nt_r, a1.nt_s);
  a1.E = d.E;
  a1.K = d.K;
  a1.a_r = a1.a_s = x;
  a1.lda_r = a1.lda_s = d.H;
  a1.perm = perm;
  a1.kdim_r = a1.kdim_s = d.H;
  a1.b_r = (const u32x4*)w13p;
  a1.b_s = (const u32x4*)ws13p;
  a1.ncol_r = d.I;
  a1.ncol_s = d.Is;
  a1.c_r = h;
  a1.c_s = hs;
  a1.ldc_r = d.I;
  a1.ldc_s = d.Is;
  if (wide) {
    PackedArgs w1 = a1;
    w1.ntn = (a1.ntn + 1) / 2;
    MOE_TIMED_LAUNCH(s, "grouped_gemm_bf16_packed_wide<true>",
      hipLaunchKernelGGL(grouped_gemm_bf16_packed_wide<true>, dim3(xcd_grid(mt * w1.ntn)), dim3(NT),
                         kLdsW, s, w1));
  } else if (few == 1)
    MOE_TIMED_LAUNCH(s, "grouped_gemm_bf16_packed_few<true, 1>",
      hipLaunchKernelGGL((grouped_gemm_bf16_packed_few<true, 1>),
                         dim3(grid(mt * a1.ntn * kFewSlots)), dim3(64), 0, s, a1));
  else if (few == 2)
    MOE_TIMED_LAUNCH(s, "grouped_gemm_bf16_packed_few<true, 2>",
      hipLaunchKernelGGL((grouped_gemm_bf16_packed_few<true, 2>),
                         dim3(grid(mt * a1.ntn * kFewSlots)), dim3(64), 0, s, a1));
  else
    MOE_TIMED_LAUNCH(s, "grouped_gemm_bf16_packed<true>",
      hipLaunchKernelGGL(grouped_gemm_bf16_packed<true>, dim3(xcd_grid(mt * a1.ntn)), dim3(NT), kLdsP, s,
                         a1));
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  PackedArgs a2{};
  a2.tiles = tiles;
  a2.nt_r = a2.nt_s = (d.H + 255) / 256;
  a2.ntn = a2.nt_r;
  a2.E = d.E;
  a2.K = d.K;
  a2.a_r = h;
  a2.a_s = hs;
  a2.lda_r = d.I;
  a2.lda_s = d.Is;
  a2.perm = nullptr;
  a2.kdim_r = d.I;
  a2.kdim_s = d.Is;
  a2.b_r = (const u32x4*)w2p;
  a2.b_s = (const u32x4*)ws2p;
  a2.ncol_r = a2.ncol_s = d.H;
  a2.c_r = y;
  a2.c_s = ys;
  a2.ldc_r = a2.ldc_s = d.H;
  if (few == 1 && mt * a2.ntn * kFewSlots <= kFewDenseSlots)
    MOE_TIMED_LAUNCH(s, "grouped_gemm_bf16_packed_few<false, 1, 4>",
      hipLaunchKernelGGL((grouped_gemm_bf16_packed_few<false, 1, 4>),
                         dim3(grid(mt * a2.ntn * kFewSlots)), dim3(64), 0, s, a2));
  else if (few == 1)
    MOE_TIMED_LAUNCH(s, "grouped_gemm_bf16_packed_few<false, 1>",
      hipLaunchKernelGGL((grouped_gemm_bf16_packed_few<false, 1>),
                         dim3(grid(mt * a2.ntn * kFewSlots)), dim3(64), 0, s, a2));
  else if (few == 2)
    MOE_TIMED_LAUNCH(s, "grouped_gemm_bf16_packed_few<false, 2>",
      hipLaunchKernelGGL((grouped_gemm_bf16_packed_few<false, 2>),
                         dim3(grid(mt * a2.ntn * kFewSlots)), dim3(64), 0, s, a2));
  else {
    // The down projection uses 128-row tiles, two workgroups per CU (with
    // wide tiles the list is already at 128 rows).
    if (!wide) e = ffn_build_tiles(d, offsets, BM2, tiles, s, true);
    if (e != hipSuccess) return e;
    const int64_t mt2 = ffn_grid_mtiles(d, BM2);
    MOE_TIMED_LAUNCH(s, "grouped_gemm_bf16_packed_x2<false>",
      hipLaunchKernelGGL(grouped_gemm_bf16_packed_x2<false>, dim3(xcd_grid(mt2 * a2.ntn)), dim3(NT),
                         kLdsP2, s, a2));
  }
  return hipGetLastError();
}

}  // namespace moe
