// Grouped expert GEMMs on bf16 MFMA (gfx950), fp32 accumulation.
//
// Every routed expert and the shared expert is a SwiGLU FFN (mqxn.cn/news/19449,
// section 3.1; one shared + fine-grained routed experts of width 2048 on the
// page "从 1024 块 GPU 到 558 万美元：拆解 DeepSeek-V3 的算法-系统协同设计", section 2.2):
//   GEMM1: [g u] = x_rows W13^T, h = silu(g) * u    (rows gathered via perm)
//   GEMM2: y_rows = h_rows W2^T
// The shared expert is group E of the same launch with all T tokens in order.
//
// Workgroup tile: up to 256 rows of one group x 256 weight rows, k in steps
// of 64.  The rows of a tile are the group's actual rows (at most 256): only
// the 32-row MFMA blocks that hold rows are computed, so an expert with 140
// rows costs 5 row blocks and its weight slice is read once.  4 waves; wave w
// owns weight rows [64w, 64w+64) for all rows of the tile (for GEMM1, 32 gate
// rows and the 32 matching up rows, so SiLU(g)*u is formed in registers).
//
// Both operands are staged through LDS (XOR-swizzled by 16-byte chunk, so
// MFMA operand reads are conflict free).  Global loads read whole 128-byte
// lines (8 lanes per row) and go through two register stages, so every load
// has two compute steps to arrive: at step s the LDS holds step s, the
// registers hold steps s+1 and s+2.  The loads are unconditional (rows past
// the tile's end re-read its first row, loads past the last step re-read the
// last step), which keeps the compiler's memory-counter waits partial.
#include "moe_internal.hpp"

#include <algorithm>

namespace moe {

namespace {

constexpr int BM = 256;    // max rows per tile
constexpr int BNB = 256;   // weight rows per tile
constexpr int BK = 64;     // k per step
constexpr int NT = 256;    // threads
#ifndef MOE_WEIGHT_NT
#define MOE_WEIGHT_NT 1
#endif
constexpr size_t kLds = (size_t)2 * (BM + BNB) * 8 * sizeof(u32x4);   // 128 KiB

struct GemmArgs {
  const int32_t* tiles;
  int ntn;                       // N-tiles per M-tile
  int E, K;
  const uint16_t* a_r;           // routed A rows base
  const uint16_t* a_s;           // shared A rows base
  int64_t lda_r, lda_s;
  const int32_t* perm;           // GEMM1: routed A row = perm[j] / K (token)
  int kdim_r, kdim_s;
  const uint16_t* b_r;           // routed weights, expert stride b_es
  int64_t b_es;
  const uint16_t* b_s;           // shared weights
  int ncol_r, ncol_s;            // output columns (GEMM1: I / Is; GEMM2: H)
  uint16_t* c_r;
  uint16_t* c_s;
  int64_t ldc_r, ldc_s;
};

struct Stage {
  u32x4 a[8], b[8];
};

// Physical 16-byte chunk of logical chunk c in LDS row r (rows of 128 bytes).
// Rows r and r+8 differ in the XOR term, so 8 consecutive rows (a 32-bank
// LDS cycle) and 16 consecutive rows (a 64-bank cycle) of one logical chunk
// fall in distinct banks.
__device__ __forceinline__ int swz(int r, int c) { return r * 8 + (c ^ ((r ^ (r >> 3)) & 7)); }

// kStoreGU (with kGateUp): the epilogue stores g and u themselves in fp32,
// row r of a group at c + r * ldc (g in columns [0, ncol), u in
// [ncol, 2 ncol)), for the backward of the FFN.
template <bool kGateUp, bool kStoreGU = false>
__global__ void __launch_bounds__(NT, 1) grouped_gemm_bf16(GemmArgs p) {
  extern __shared__ u32x4 smem[];
  u32x4* sA = smem;                   // [2][BM * 8]
  u32x4* sB = smem + 2 * BM * 8;      // [2][BNB * 8]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lh = lane >> 5;

  // Work item: dealt to the XCDs in chunks over the real work count.
  const int64_t work = (int64_t)p.tiles[0] * p.ntn;
  const int64_t w = xcd_chunked(blockIdx.x, work);
  if (w < 0) return;
  int ntile;
  const int32_t* ent = decode_work(p.tiles, w, p.ntn, ntile);
  const int g = ent[0], row0 = ent[1], nrows = ent[2];
  const bool sh = (g == p.E);
  const int ncol = sh ? p.ncol_s : p.ncol_r;
  const int n0 = ntile * (kGateUp ? BNB / 2 : BNB);
  if (n0 >= ncol) return;
  const int kdim = sh ? p.kdim_s : p.kdim_r;
  const uint16_t* A = sh ? p.a_s : p.a_r;
  const int64_t lda = sh ? p.lda_s : p.lda_r;
  const uint16_t* B = sh ? p.b_s : p.b_r + (int64_t)g * p.b_es;
  const int64_t ldb = kdim;

  // Rows this thread stages: r = tid/8 + 32 j (j < 8), 16-byte chunk tid % 8.
  const int ch = tid & 7;
  const int first = (!sh && kGateUp) ? p.perm[row0] / p.K : row0;
  int arow[8], brow[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = (tid >> 3) + 32 * j;
    int a = first;
    if (r < nrows) a = (!sh && kGateUp) ? p.perm[row0 + r] / p.K : row0 + r;
    arow[j] = a;
    int col, src;
    if (kGateUp) {   // tile row r: wave r/64, gate (r%64 < 32) or up column
      const int wv = r >> 6, jj = r & 63;
      col = n0 + wv * 32 + (jj & 31);
      src = (jj < 32) ? col : ncol + col;
    } else {
      col = n0 + r;
      src = col;
    }
    brow[j] = col < ncol ? src : 0;   // a column past ncol is never stored
  }
  const uint16_t* abase = A + ch * 8;
  const uint16_t* bbase = B + ch * 8;
  const int nsteps = kdim / BK;
  const int last = nsteps - 1;

  // Load / store one staged row pair (A row and weight row j) of a step.
  auto gload1 = [&](Stage& st, int j, int step) {
    const int k0 = min(step, last) * BK;
    st.a[j] = *reinterpret_cast<const u32x4*>(abase + (int64_t)arow[j] * lda + k0);
    const u32x4* pb = reinterpret_cast<const u32x4*>(bbase + (int64_t)brow[j] * ldb + k0);
#if MOE_WEIGHT_NT
    st.b[j] = __builtin_nontemporal_load(pb);
#else
    st.b[j] = *pb;
#endif
  };
  auto sstore1 = [&](const Stage& st, int j, int buf) {
    const int r = (tid >> 3) + 32 * j;
    const int o = buf * BM * 8 + swz(r, ch);
    sA[o] = st.a[j];
    sB[o] = st.b[j];
  };

  f32x16 acc[8][2];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[r][c][i] = 0.0f;
  const int nrb = (nrows + 31) >> 5;

  // One step: MFMAs on LDS buffer `buf`; between its four 16-wide k slices,
  // the next step's rows move from registers `st` to LDS buffer `nbuf`, and
  // `st` is refilled with step `ld` from memory.
  auto step_body = [&](int buf, Stage& st, int nbuf, int ld) {
    const u32x4* as = sA + buf * BM * 8;
    const u32x4* bs = sB + buf * BNB * 8;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int c = 2 * kk + lh;
      const int br0 = wave * 64 + lr, br1 = br0 + 32;
      const bf16x8 b0 = as_bf16x8(bs[swz(br0, c)]);
      const bf16x8 b1 = as_bf16x8(bs[swz(br1, c)]);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        if (r < nrb) {
          const int ar = r * 32 + lr;
          const bf16x8 a = as_bf16x8(as[swz(ar, c)]);
          acc[r][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b0, acc[r][0], 0, 0, 0);
          acc[r][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b1, acc[r][1], 0, 0, 0);
        }
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        sstore1(st, 2 * kk + jj, nbuf);
        gload1(st, 2 * kk + jj, ld);
      }
    }
  };

  // Register stage R[t % 2] holds step t; LDS buffer t % 2 holds step t.
  Stage R0, R1;
#pragma unroll
  for (int j = 0; j < 8; ++j) gload1(R0, j, 0);
#pragma unroll
  for (int j = 0; j < 8; ++j) sstore1(R0, j, 0);
#pragma unroll
  for (int j = 0; j < 8; ++j) gload1(R1, j, 1);
#pragma unroll
  for (int j = 0; j < 8; ++j) gload1(R0, j, 2);
  __syncthreads();
  for (int s = 0; s < nsteps; s += 2) {
    step_body(0, R1, 1, s + 3);     // step s; stage s+1 to LDS; load s+3
    __syncthreads();
    if (s + 1 < nsteps) {
      step_body(1, R0, 0, s + 4);   // step s+1; stage s+2 to LDS; load s+4
      __syncthreads();
    }
  }

  // Epilogue.  32x32 block layout: lane holds column lane%32, rows
  // 8*(i/4) + 4*(lane/32) + i%4.
  uint16_t* C = sh ? p.c_s : p.c_r;
  const int64_t ldc = sh ? p.ldc_s : p.ldc_r;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    if (r >= nrb) break;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = r * 32 + 8 * (i >> 2) + 4 * lh + (i & 3);
      if (row >= nrows) continue;
      uint16_t* crow = C + (int64_t)(row0 + row) * ldc;
      if (kGateUp && kStoreGU) {
        const int col = n0 + wave * 32 + lr;
        if (col < ncol) {
          float* grow = reinterpret_cast<float*>(sh ? p.c_s : p.c_r) + (int64_t)(row0 + row) * ldc;
          grow[col] = acc[r][0][i];
          grow[ncol + col] = acc[r][1][i];
        }
      } else if (kGateUp) {
        const int col = n0 + wave * 32 + lr;
        if (col < ncol) {
          const float gv = acc[r][0][i], uv = acc[r][1][i];
          const float hv = gv / (1.0f + __expf(-gv)) * uv;
          crow[col] = (uint16_t)f32_to_bf16_bits(hv);
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

bool g_attr_set = false;

hipError_t set_attrs() {
  if (g_attr_set) return hipSuccess;
  hipError_t e = hipFuncSetAttribute((const void*)grouped_gemm_bf16<true>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute((const void*)grouped_gemm_bf16<false>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute((const void*)grouped_gemm_bf16<true, true>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
  if (e == hipSuccess) g_attr_set = true;
  return e;
}


}  // namespace

size_t ffn_tiles_bytes(const FfnDims& d) {
  return (size_t)(8 + 8 * ffn_max_mtiles(d.N, d.T, d.E, ffn_list_tile_rows(d.T))) *
         sizeof(int32_t);
}

// h holds routed rows [0, N) with width I, then shared rows [N, N+T) with width Is.
hipError_t launch_ffn_bf16(const FfnDims& d, const uint16_t* x, const int32_t* perm,
                           const int32_t* offsets, const uint16_t* w13, const uint16_t* w2,
                           const uint16_t* ws13, const uint16_t* ws2, uint16_t* h,
                           int32_t* tiles, uint16_t* y, uint16_t* ys, hipStream_t s) {
  hipError_t e = set_attrs();
  if (e != hipSuccess) return e;
  e = ffn_build_tiles(d, offsets, BM, tiles, s);
  if (e != hipSuccess) return e;
  const int64_t mt = ffn_grid_mtiles(d, BM);
  uint16_t* hs = h + d.N * d.I;

  GemmArgs a1{};
  a1.tiles = tiles;
  a1.ntn = (int)((std::max(d.I, d.Is) + BNB / 2 - 1) / (BNB / 2));
  a1.E = d.E;
  a1.K = d.K;
  a1.a_r = x;
  a1.a_s = x;
  a1.lda_r = a1.lda_s = d.H;
  a1.perm = perm;
  a1.kdim_r = a1.kdim_s = d.H;
  a1.b_r = w13;
  a1.b_es = (int64_t)2 * d.I * d.H;
  a1.b_s = ws13;
  a1.ncol_r = d.I;
  a1.ncol_s = d.Is;
  a1.c_r = h;
  a1.c_s = hs;
  a1.ldc_r = d.I;
  a1.ldc_s = d.Is;
  MOE_TIMED_LAUNCH(s, "grouped_gemm_bf16<true>",
    hipLaunchKernelGGL(grouped_gemm_bf16<true>, dim3(xcd_grid(mt * a1.ntn)), dim3(NT), kLds, s, a1));
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  GemmArgs a2{};
  a2.tiles = tiles;
  a2.ntn = (d.H + BNB - 1) / BNB;
  a2.E = d.E;
  a2.K = d.K;
  a2.a_r = h;
  a2.a_s = hs;
  a2.lda_r = d.I;
  a2.lda_s = d.Is;
  a2.perm = nullptr;
  a2.kdim_r = d.I;
  a2.kdim_s = d.Is;
  a2.b_r = w2;
  a2.b_es = (int64_t)d.H * d.I;
  a2.b_s = ws2;
  a2.ncol_r = a2.ncol_s = d.H;
  a2.c_r = y;
  a2.c_s = ys;
  a2.ldc_r = a2.ldc_s = d.H;
  MOE_TIMED_LAUNCH(s, "grouped_gemm_bf16<false>",
    hipLaunchKernelGGL(grouped_gemm_bf16<false>, dim3(xcd_grid(mt * a2.ntn)), dim3(NT), kLds, s, a2));
  return hipGetLastError();
}

hipError_t launch_gate_up_bf16(const FfnDims& d, const uint16_t* x, const int32_t* perm,
                               const int32_t* offsets, const uint16_t* w13, const uint16_t* ws13,
                               int32_t* tiles, float* gu, int64_t ldgu, float* gus,
                               int64_t ldgus, hipStream_t s) {
  hipError_t e = set_attrs();
  if (e != hipSuccess) return e;
  e = ffn_build_tiles(d, offsets, BM, tiles, s);
  if (e != hipSuccess) return e;
  const int64_t mt = ffn_grid_mtiles(d, BM);
  GemmArgs a{};
  a.tiles = tiles;
  a.ntn = (int)((std::max(d.I, d.Is) + BNB / 2 - 1) / (BNB / 2));
  a.E = d.E;
  a.K = d.K;
  a.a_r = a.a_s = x;
  a.lda_r = a.lda_s = d.H;
  a.perm = perm;
  a.kdim_r = a.kdim_s = d.H;
  a.b_r = w13;
  a.b_es = (int64_t)2 * d.I * d.H;
  a.b_s = ws13;
  a.ncol_r = d.I;
  a.ncol_s = d.Is;
  a.c_r = reinterpret_cast<uint16_t*>(gu);
  a.c_s = reinterpret_cast<uint16_t*>(gus);
  a.ldc_r = ldgu;
  a.ldc_s = ldgus;
  MOE_TIMED_LAUNCH(s, "grouped_gemm_bf16<gate_up>",
    hipLaunchKernelGGL((grouped_gemm_bf16<true, true>), dim3(xcd_grid(mt * a.ntn)), dim3(NT), kLds,
                       s, a));
  return hipGetLastError();
}

}  // namespace moe
