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
// into registers, PF steps ahead, with no LDS traffic; the activation rows
// (shared by the 4 waves) use the double-buffered LDS tile of the row-major
// kernel, with the same k assignment (lane half lh holds k in
// [32 lh, 32 lh + 32)).
#include "moe_internal.hpp"

#include <algorithm>

namespace moe {

namespace {

constexpr int BM = 256;    // max rows per tile
constexpr int BK = 64;     // k per step
constexpr int NT = 256;    // threads
constexpr int PF = 2;      // weight prefetch depth (steps)
constexpr int FRAG = 2048; // 16-byte fragments per packed block (32 KiB)
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

struct PackedArgs {
  const int32_t* tiles;
  int ntn;                      // N-tiles per M-tile (max over groups)
  int E, K;
  const uint16_t* a_r;
  const uint16_t* a_s;
  int64_t lda_r, lda_s;
  const int32_t* perm;          // GEMM1: routed A row = perm[j] / K
  int kdim_r, kdim_s;
  const u32x4* b_r;             // packed routed weights
  int nt_r;                     // output tiles per routed expert
  const u32x4* b_s;             // packed shared weights
  int nt_s;
  int ncol_r, ncol_s;
  uint16_t* c_r;
  uint16_t* c_s;
  int64_t ldc_r, ldc_s;
};

__device__ __forceinline__ int swz(int r, int c) { return r * 8 + (c ^ ((r ^ (r >> 3)) & 7)); }

// The work of one tile with NRB 32-row blocks (compile time, so the MFMA
// loop has no branches and the fragment reads of a k slice can all be in
// flight together).
template <bool kGateUp, int NRB>
__device__ __forceinline__ void packed_tile(const PackedArgs& p, u32x4* sA, int g, int row0,
                                            int nrows, int ntile) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lh = lane >> 5;
  const bool sh = (g == p.E);
  const int ncol = sh ? p.ncol_s : p.ncol_r;
  const int n0 = ntile * (kGateUp ? 128 : 256);
  const int kdim = sh ? p.kdim_s : p.kdim_r;
  const int nsteps = kdim / BK;
  const int last = nsteps - 1;
  const uint16_t* A = sh ? p.a_s : p.a_r;
  const int64_t lda = sh ? p.lda_s : p.lda_r;
  const u32x4* bw = (sh ? p.b_s : p.b_r + (int64_t)g * p.nt_r * nsteps * FRAG) +
                    (int64_t)ntile * nsteps * FRAG + wave * 512 + lane;

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
  u32x4 ra[2][NRB];   // two register stages of activation rows
  auto aload = [&](u32x4 (&st)[NRB], int j, int step) {
    st[j] = *reinterpret_cast<const u32x4*>(abase + (int64_t)arow[j] * lda +
                                            min(step, last) * BK);
  };
  auto astore = [&](const u32x4 (&st)[NRB], int j, int buf) {
    sA[buf * BM * 8 + swz((tid >> 3) + 32 * j, ch)] = st[j];
  };
  u32x4 rb[PF][8];    // weight fragments [slot][cb * 4 + kk]
  auto bload = [&](u32x4 (&dst)[8], int step) {
    const u32x4* src = bw + (int64_t)min(step, last) * FRAG;
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[i] = __builtin_nontemporal_load(src + i * 64);
  };

  f32x16 acc[NRB][2];
#pragma unroll
  for (int r = 0; r < NRB; ++r)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[r][c][i] = 0.0f;

  // One step on LDS buffer `buf` with weight slot `b`; the next step's
  // activation rows move from registers `st` to LDS buffer `nbuf` and `st`
  // is refilled with step `ld`, spread over the four k slices.
  auto step_body = [&](bool active, int buf, const u32x4 (&b)[8], u32x4 (&st)[NRB], int nbuf,
                       int ld) {
    const u32x4* as = sA + buf * BM * 8;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (active) {
        const int c = 4 * lh + kk;
        bf16x8 a[NRB];
#pragma unroll
        for (int r = 0; r < NRB; ++r) a[r] = as_bf16x8(as[swz(r * 32 + lr, c)]);
        const bf16x8 b0 = as_bf16x8(b[kk]);
        const bf16x8 b1 = as_bf16x8(b[4 + kk]);
#pragma unroll
        for (int r = 0; r < NRB; ++r) {
          acc[r][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[r], b0, acc[r][0], 0, 0, 0);
          acc[r][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[r], b1, acc[r][1], 0, 0, 0);
        }
      }
#pragma unroll
      for (int j = kk; j < NRB; j += 4) {
        astore(st, j, nbuf);
        aload(st, j, ld);
      }
    }
  };

  // Prologue: weights for steps 0..PF-1, activations of step 0 in LDS, of
  // steps 1 and 2 in the two register stages.
#pragma unroll
  for (int s = 0; s < PF; ++s) bload(rb[s], s);
#pragma unroll
  for (int j = 0; j < NRB; ++j) aload(ra[0], j, 0);
#pragma unroll
  for (int j = 0; j < NRB; ++j) astore(ra[0], j, 0);
#pragma unroll
  for (int j = 0; j < NRB; ++j) aload(ra[1], j, 1);
#pragma unroll
  for (int j = 0; j < NRB; ++j) aload(ra[0], j, 2);
  __syncthreads();

  // Step t: LDS buffer t % 2; ra[(t+1) % 2] holds step t+1; weight slot
  // t % PF.  Unrolled by PF (even) so every index is static.
  for (int s = 0; s < nsteps; s += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int t = s + u;
      step_body(t < nsteps, u & 1, rb[u], ra[(u + 1) & 1], (u + 1) & 1, t + 3);
      bload(rb[u], t + PF);
      __syncthreads();
    }
  }

  // Epilogue: lane holds column lane%32, rows 8*(i/4) + 4*(lane/32) + i%4.
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
        const int col = n0 + wave * 32 + lr;
        if (col < ncol) {
          const float gv = acc[r][0][i], uv = acc[r][1][i];
          crow[col] = (uint16_t)f32_to_bf16_bits(gv / (1.0f + __expf(-gv)) * uv);
        }
      } else {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          const int col = n0 + wave * 64 + cb * 32 + lr;
          if (col < ncol) crow[col] = (uint16_t)f32_to_bf16_bits(acc[r][cb][i]);
        }
      }
    }
  }
}

template <bool kGateUp>
__global__ void __launch_bounds__(NT, 1) grouped_gemm_bf16_packed(PackedArgs p) {
  extern __shared__ u32x4 smem[];
  const int64_t work = (int64_t)p.tiles[0] * p.ntn;
  const int64_t per = (work + kNumXcd - 1) / kNumXcd;
  const int64_t q = blockIdx.x / kNumXcd;
  const int64_t w = (int64_t)(blockIdx.x % kNumXcd) * per + q;
  if (q >= per || w >= work) return;
  int ntile;
  const int32_t* ent = decode_work(p.tiles, w, p.ntn, ntile);
  const int g = ent[0], row0 = ent[1], nrows = ent[2];
  if (ntile >= ((g == p.E) ? p.nt_s : p.nt_r)) return;
  switch ((nrows + 31) >> 5) {
    case 1: packed_tile<kGateUp, 1>(p, smem, g, row0, nrows, ntile); break;
    case 2: packed_tile<kGateUp, 2>(p, smem, g, row0, nrows, ntile); break;
    case 3: packed_tile<kGateUp, 3>(p, smem, g, row0, nrows, ntile); break;
    case 4: packed_tile<kGateUp, 4>(p, smem, g, row0, nrows, ntile); break;
    case 5: packed_tile<kGateUp, 5>(p, smem, g, row0, nrows, ntile); break;
    case 6: packed_tile<kGateUp, 6>(p, smem, g, row0, nrows, ntile); break;
    case 7: packed_tile<kGateUp, 7>(p, smem, g, row0, nrows, ntile); break;
    default: packed_tile<kGateUp, 8>(p, smem, g, row0, nrows, ntile); break;
  }
}

// Few-row variant (every group has at most 32 * NRB rows, NRB <= 2: decode
// batches).  The activation rows are few and L2-resident, so each wave
// loads its own MFMA operands for them straight from global memory: waves
// are independent (no LDS, no barrier), use few registers, and two waves
// share each SIMD, which keeps more weight loads in flight.
template <bool kGateUp, int NRB>
__global__ void __launch_bounds__(NT, 2) grouped_gemm_bf16_packed_few(PackedArgs p) {
  constexpr int D = NRB == 1 ? 3 : 2;   // steps of weights + activations in flight
  const int64_t work = (int64_t)p.tiles[0] * p.ntn;
  const int64_t per = (work + kNumXcd - 1) / kNumXcd;
  const int64_t q = blockIdx.x / kNumXcd;
  const int64_t w = (int64_t)(blockIdx.x % kNumXcd) * per + q;
  if (q >= per || w >= work) return;
  int ntile;
  const int32_t* ent = decode_work(p.tiles, w, p.ntn, ntile);
  const int g = ent[0], row0 = ent[1], nrows = ent[2];
  const bool sh = (g == p.E);
  if (ntile >= (sh ? p.nt_s : p.nt_r)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lh = lane >> 5;
  const int ncol = sh ? p.ncol_s : p.ncol_r;
  const int n0 = ntile * (kGateUp ? 128 : 256);
  const int kdim = sh ? p.kdim_s : p.kdim_r;
  const int nsteps = kdim / BK;
  const int last = nsteps - 1;
  const uint16_t* A = sh ? p.a_s : p.a_r;
  const int64_t lda = sh ? p.lda_s : p.lda_r;
  const u32x4* bw = (sh ? p.b_s : p.b_r + (int64_t)g * p.nt_r * nsteps * FRAG) +
                    (int64_t)ntile * nsteps * FRAG + wave * 512 + lane;
  // This lane's activation rows: tile rows r * 32 + lane % 32 (rows past
  // the end re-read the first row; their outputs are never stored); k from
  // 32 * lane_half, as in the weight fragments.
  const uint16_t* ap[NRB];
#pragma unroll
  for (int r = 0; r < NRB; ++r) {
    const int row = r * 32 + lr;
    const int rr = row < nrows ? row : 0;
    const int a = (!sh && kGateUp) ? p.perm[row0 + rr] / p.K : row0 + rr;
    ap[r] = A + (int64_t)a * lda + lh * 32;
  }
  u32x4 rb[D][8], ra[D][NRB][4];
  auto load = [&](int slot, int step) {
    const int st = min(step, last);
    const u32x4* src = bw + (int64_t)st * FRAG;
#pragma unroll
    for (int i = 0; i < 8; ++i) rb[slot][i] = __builtin_nontemporal_load(src + i * 64);
#pragma unroll
    for (int r = 0; r < NRB; ++r)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        ra[slot][r][kk] = *reinterpret_cast<const u32x4*>(ap[r] + st * BK + kk * 8);
  };
  f32x16 acc[NRB][2];
#pragma unroll
  for (int r = 0; r < NRB; ++r)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[r][c][i] = 0.0f;
#pragma unroll
  for (int s = 0; s < D; ++s) load(s, s);
  for (int s = 0; s < nsteps; s += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      if (s + u < nsteps) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const bf16x8 b0 = as_bf16x8(rb[u][kk]);
          const bf16x8 b1 = as_bf16x8(rb[u][4 + kk]);
#pragma unroll
          for (int r = 0; r < NRB; ++r) {
            const bf16x8 a = as_bf16x8(ra[u][r][kk]);
            acc[r][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b0, acc[r][0], 0, 0, 0);
            acc[r][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b1, acc[r][1], 0, 0, 0);
          }
        }
      }
      load(u, s + u + D);
    }
  }
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
        const int col = n0 + wave * 32 + lr;
        if (col < ncol) {
          const float gv = acc[r][0][i], uv = acc[r][1][i];
          crow[col] = (uint16_t)f32_to_bf16_bits(gv / (1.0f + __expf(-gv)) * uv);
        }
      } else {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          const int col = n0 + wave * 64 + cb * 32 + lr;
          if (col < ncol) crow[col] = (uint16_t)f32_to_bf16_bits(acc[r][cb][i]);
        }
      }
    }
  }
}

hipError_t set_attrs_packed() {
  static hipError_t once = []() {
    hipError_t e = hipFuncSetAttribute((const void*)grouped_gemm_bf16_packed<true>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsP);
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute((const void*)grouped_gemm_bf16_packed<false>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsP);
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
  e = launch_build_tiles(offsets, d.E, d.T, d.Is > 0, BM, tiles, s);
  if (e != hipSuccess) return e;
  const int64_t mt = ffn_max_mtiles(d.N, d.T, d.E, BM);
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
  // Every group has at most T rows (a token picks an expert at most once).
  const int few = d.T <= 32 ? 1 : d.T <= 64 ? 2 : 0;
  if (few == 1)
    MOE_TIMED_LAUNCH(s, "grouped_gemm_bf16_packed_few<true, 1>",
      hipLaunchKernelGGL((grouped_gemm_bf16_packed_few<true, 1>), dim3(grid(mt * a1.ntn)), dim3(NT),
                         0, s, a1));
  else if (few == 2)
    MOE_TIMED_LAUNCH(s, "grouped_gemm_bf16_packed_few<true, 2>",
      hipLaunchKernelGGL((grouped_gemm_bf16_packed_few<true, 2>), dim3(grid(mt * a1.ntn)), dim3(NT),
                         0, s, a1));
  else
    MOE_TIMED_LAUNCH(s, "grouped_gemm_bf16_packed<true>",
      hipLaunchKernelGGL(grouped_gemm_bf16_packed<true>, dim3(grid(mt * a1.ntn)), dim3(NT), kLdsP, s,
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
  if (few == 1)
    MOE_TIMED_LAUNCH(s, "grouped_gemm_bf16_packed_few<false, 1>",
      hipLaunchKernelGGL((grouped_gemm_bf16_packed_few<false, 1>), dim3(grid(mt * a2.ntn)),
                         dim3(NT), 0, s, a2));
  else if (few == 2)
    MOE_TIMED_LAUNCH(s, "grouped_gemm_bf16_packed_few<false, 2>",
      hipLaunchKernelGGL((grouped_gemm_bf16_packed_few<false, 2>), dim3(grid(mt * a2.ntn)),
                         dim3(NT), 0, s, a2));
  else
    MOE_TIMED_LAUNCH(s, "grouped_gemm_bf16_packed<false>",
      hipLaunchKernelGGL(grouped_gemm_bf16_packed<false>, dim3(grid(mt * a2.ntn)), dim3(NT), kLdsP,
                         s, a2));
  return hipGetLastError();
}

}  // namespace moe
