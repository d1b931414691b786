// FP8 block-scaled expert FFN (gfx950).
//
// "深入理解 DeepSeek-V3：大规模缩放挑战与对 AI 架构硬件的反思（中文精读）", section 3.2:
// activations are quantised per 1x128 tile and weights per 128x128 block,
// with fp32 accumulation; the page on the algorithm-system co-design
// ("从 1024 块 GPU 到 558 万美元…", section 5.1) describes the block-wise FP8 GEMM:
// fp8 operands whose block scales are applied during accumulation.
//
// Quantiser: per 1x128 tile, a = max |v|, scale = a / 448, inv = 448 / a
// (both computed in double, rounded to fp32; scale 1 / inv 0 for a == 0);
// code = OCP e4m3fn nearest to the fp32 product v * inv, ties to even,
// saturated at +-448.
//
// GEMM: each 128-wide k block is one MFMA pair (32x32x64 e4m3, fp32 result);
// the block's partial sum is scaled by a_scale[row] * b_scale[block] and added
// to the fp32 accumulator (on MI355X the matrix core already accumulates in
// fp32, so the promotion only applies the scales).  GEMM1 forms
// h = silu(g) * u and quantises it per 1x128 tile in the epilogue; GEMM2
// writes bf16.  Tiles, scheduling and LDS layout follow the bf16 kernel.
#include "moe_internal.hpp"
#include "fp8_device.hpp"

#include <algorithm>

namespace moe {

namespace {

// One 128-wide tile per 16 lanes (8 values each); 256 threads = 16 tiles.
// kPow2: power-of-two scales (the matrix cores apply them), else a / 448.
template <bool kPow2>
__global__ void __launch_bounds__(256)
quant_rows_kernel(const uint16_t* __restrict__ x, int64_t rows, int cols,
                  uint8_t* __restrict__ q, float* __restrict__ sc) {
  const int tiles_per_row = cols / 128;
  const int64_t tile = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  const bool ok = tile < rows * tiles_per_row;
  const int64_t r = ok ? tile / tiles_per_row : 0;
  const int c = ok ? (int)(tile % tiles_per_row) * 128 + sub * 8 : 0;
  float v[8];
  float m = 0.0f;
  if (ok) {
    const uint4 p = *reinterpret_cast<const uint4*>(x + r * cols + c);
    const uint32_t u[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf16_bits_to_f32(u[j] & 0xFFFFu);
      v[2 * j + 1] = bf16_bits_to_f32(u[j] >> 16);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if (!ok) return;
  float scale, inv;
  if (kPow2)
    tile_scale_pow2(m, scale, inv);
  else
    tile_scale(m, scale, inv);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) lo |= f32_to_e4m3(v[j] * inv) << (8 * j);
#pragma unroll
  for (int j = 0; j < 4; ++j) hi |= f32_to_e4m3(v[4 + j] * inv) << (8 * j);
  *reinterpret_cast<uint2*>(q + r * cols + c) = make_uint2(lo, hi);
  if (sub == 0) sc[r * tiles_per_row + c / 128] = scale;
}

constexpr int BM = 256, BNB = 256, BK = 128, NT = 256;
constexpr size_t kLds8 = (size_t)2 * (BM + BNB) * 8 * sizeof(uint4) + 2 * BM * sizeof(float);

struct Gemm8Args {
  const int32_t* tiles;
  int ntn, E, K;
  const uint8_t* a_r;
  const uint8_t* a_s;
  const float* as_r;        // A scales, [rows][kdim/128]
  const float* as_s;
  const int32_t* perm;      // GEMM1: routed A row = perm[j] / K
  int kdim_r, kdim_s;
  const uint8_t* b_r;
  int64_t b_es;
  const float* bs_r;        // [E][rows/128][kdim/128]
  int64_t bs_es;
  const uint8_t* b_s;
  const float* bs_s;
  int ncol_r, ncol_s;
  uint8_t* hq_r;            // GEMM1 outputs (e4m3 + [rows][ncol/128] scales)
  uint8_t* hq_s;
  float* hs_r;
  float* hs_s;
  uint16_t* c_r;            // GEMM2 outputs (bf16, ld = ncol)
  uint16_t* c_s;
};


template <bool kGateUp>
__global__ void __launch_bounds__(NT, 1) grouped_gemm_fp8(Gemm8Args p) {
  extern __shared__ uint4 smem[];
  uint4* sA = smem;                            // [2][BM * 8]
  uint4* sB = smem + 2 * BM * 8;               // [2][BNB * 8]
  float* sAs = reinterpret_cast<float*>(smem + 2 * (BM + BNB) * 8);   // [2][BM]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lh = lane >> 5;

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
  const int kb_total = kdim / 128;
  const uint8_t* A = sh ? p.a_s : p.a_r;
  const float* As = sh ? p.as_s : p.as_r;
  const uint8_t* B = sh ? p.b_s : p.b_r + (int64_t)g * p.b_es;
  const float* Bs = sh ? p.bs_s : p.bs_r + (int64_t)g * p.bs_es;

  const int ch = tid & 7;
  int arow[8], brow[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = (tid >> 3) + 32 * j;
    arow[j] = -1;
    if (r < nrows) arow[j] = (!sh && kGateUp) ? p.perm[row0 + r] / p.K : row0 + r;
    int col, src;
    if (kGateUp) {
      const int wv = r >> 6, jj = r & 63;
      col = n0 + wv * 32 + (jj & 31);
      src = (jj < 32) ? col : ncol + col;
    } else {
      col = n0 + r;
      src = col;
    }
    brow[j] = (col < ncol) ? src : -1;
  }
  // Row whose A scale this thread stages.
  int srow = -1;
  if (tid < nrows) srow = (!sh && kGateUp) ? p.perm[row0 + tid] / p.K : row0 + tid;
  // B scale blocks of this wave's two 32-column blocks.
  int bblk0, bblk1;
  if (kGateUp) {
    bblk0 = n0 / 128;
    bblk1 = (ncol + n0) / 128;
  } else {
    bblk0 = bblk1 = (n0 + wave * 64) / 128;
  }

  uint4 ra[8], rb[8];
  float ras = 0.0f;
  auto gload = [&](int step) {
    const int k0 = step * BK + ch * 16;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      ra[j] = make_uint4(0, 0, 0, 0);
      if (arow[j] >= 0) ra[j] = *reinterpret_cast<const uint4*>(A + (int64_t)arow[j] * kdim + k0);
      rb[j] = make_uint4(0, 0, 0, 0);
      if (brow[j] >= 0) rb[j] = *reinterpret_cast<const uint4*>(B + (int64_t)brow[j] * kdim + k0);
    }
    ras = (srow >= 0) ? As[(int64_t)srow * kb_total + step] : 0.0f;
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = (tid >> 3) + 32 * j;
      const int o = r * 8 + (ch ^ (r & 7));
      sA[buf * BM * 8 + o] = ra[j];
      sB[buf * BNB * 8 + o] = rb[j];
    }
    sAs[buf * BM + tid] = ras;
  };

  f32x16 acc[8][2];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[r][c][i] = 0.0f;

  const int nrb = (nrows + 31) >> 5;
  const int nsteps = kb_total;
  gload(0);
  sstore(0);
  if (nsteps > 1) gload(1);
  __syncthreads();

  for (int step = 0; step < nsteps; ++step) {
    const uint4* a_s = sA + (step & 1) * BM * 8;
    const uint4* b_s = sB + (step & 1) * BNB * 8;
    const float* as_s = sAs + (step & 1) * BM;
    const float bsc0 = Bs[(int64_t)bblk0 * kb_total + step];
    const float bsc1 = Bs[(int64_t)bblk1 * kb_total + step];
    const int br0 = wave * 64 + lr, br1 = br0 + 32;
    // B operands of the two 64-wide halves of the 128 block.
    i32x8 b0[2], b1[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int c = 4 * s + 2 * lh;
      b0[s] = as_i32x8(b_s[br0 * 8 + (c ^ (br0 & 7))], b_s[br0 * 8 + ((c + 1) ^ (br0 & 7))]);
      b1[s] = as_i32x8(b_s[br1 * 8 + (c ^ (br1 & 7))], b_s[br1 * 8 + ((c + 1) ^ (br1 & 7))]);
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if (r < nrb) {
        const int ar = r * 32 + lr;
        f32x16 p0, p1;
#pragma unroll
        for (int i = 0; i < 16; ++i) p0[i] = p1[i] = 0.0f;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int c = 4 * s + 2 * lh;
          const i32x8 a = as_i32x8(a_s[ar * 8 + (c ^ (ar & 7))], a_s[ar * 8 + ((c + 1) ^ (ar & 7))]);
          p0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b0[s], p0, 0, 0, 0, 127, 0, 127);
          p1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b1[s], p1, 0, 0, 0, 127, 0, 127);
        }
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const float4 a4 = *reinterpret_cast<const float4*>(as_s + r * 32 + 8 * qd + 4 * lh);
          const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int i = 4 * qd + u;
            acc[r][0][i] = fmaf(p0[i], av[u] * bsc0, acc[r][0][i]);
            acc[r][1][i] = fmaf(p1[i], av[u] * bsc1, acc[r][1][i]);
          }
        }
      }
    }
    if (step + 1 < nsteps) {
      sstore((step + 1) & 1);
      if (step + 2 < nsteps) gload(step + 2);
    }
    __syncthreads();
  }

  if (kGateUp) {
    // h = silu(g) * u, then 1x128 quantisation: the tile's 128 h columns of a
    // row are spread over 4 waves x 32 lanes; row max by lane shuffles, then
    // across waves through LDS (reusing the A-scale buffer).
    float* s_amax = sAs;   // [4 waves][32 rows] of tile maxima per pass (the A-scale buffer)
    uint8_t* HQ = sh ? p.hq_s : p.hq_r;
    float* HS = sh ? p.hs_s : p.hs_r;
    const int col = n0 + wave * 32 + lr;
    const int nblk = ncol / 128;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if (r >= nrb) break;
      float hv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float gv = acc[r][0][i], uv = acc[r][1][i];
        hv[i] = gv / (1.0f + __expf(-gv)) * uv;
        float m = fabsf(hv[i]);
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
        // lanes 0 and 32 hold the maxima of their rows
        if (lr == 0) s_amax[wave * 32 + 8 * (i >> 2) + 4 * lh + (i & 3)] = m;
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int rl = 8 * (i >> 2) + 4 * lh + (i & 3);
        const int row = r * 32 + rl;
        float m = fmaxf(fmaxf(s_amax[rl], s_amax[32 + rl]), fmaxf(s_amax[64 + rl], s_amax[96 + rl]));
        float scale, inv;
        tile_scale(m, scale, inv);
        if (row < nrows) {
          const int64_t hrow = row0 + row;
          HQ[hrow * ncol + col] = (uint8_t)f32_to_e4m3(hv[i] * inv);
          if (wave == 0 && lr == 0) HS[hrow * nblk + n0 / 128] = scale;
        }
      }
      __syncthreads();
    }
  } else {
    uint16_t* C = sh ? p.c_s : p.c_r;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if (r >= nrb) break;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = r * 32 + 8 * (i >> 2) + 4 * lh + (i & 3);
        if (row >= nrows) continue;
        uint16_t* crow = C + (int64_t)(row0 + row) * ncol;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          const int col = n0 + wave * 64 + cb * 32 + lr;
          if (col < ncol) crow[col] = (uint16_t)f32_to_bf16_bits(acc[r][cb][i]);
        }
      }
    }
  }
}

hipError_t set_attrs8() {
  static hipError_t once = []() {
    hipError_t e = hipFuncSetAttribute((const void*)grouped_gemm_fp8<true>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds8);
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute((const void*)grouped_gemm_fp8<false>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds8);
  }();
  return once;
}


}  // namespace

hipError_t launch_quant_rows(const uint16_t* x, int64_t rows, int cols, uint8_t* q, float* sc,
                             bool pow2, hipStream_t s) {
  const int64_t tiles = rows * (cols / 128);
  const dim3 grid((unsigned)((tiles + 15) / 16));
  if (pow2)
    MOE_TIMED_LAUNCH(s, "quant_rows_kernel<pow2>",
      hipLaunchKernelGGL(quant_rows_kernel<true>, grid, dim3(256), 0, s, x, rows, cols, q, sc));
  else
    MOE_TIMED_LAUNCH(s, "quant_rows_kernel",
      hipLaunchKernelGGL(quant_rows_kernel<false>, grid, dim3(256), 0, s, x, rows, cols, q, sc));
  return hipGetLastError();
}

// hq: routed rows [0, N) width I, then shared rows width Is; hs likewise with
// I/128 and Is/128 scales per row.
hipError_t launch_ffn_fp8(const FfnDims& d, const uint8_t* xq, const float* xs,
                          const int32_t* perm, const int32_t* offsets, const uint8_t* w13,
                          const float* w13s, const uint8_t* w2, const float* w2s,
                          const uint8_t* ws13, const float* ws13s, const uint8_t* ws2,
                          const float* ws2s, uint8_t* hq, float* hs, int32_t* tiles,
                          uint16_t* y, uint16_t* ys, hipStream_t s) {
  hipError_t e = set_attrs8();
  if (e != hipSuccess) return e;
  e = ffn_build_tiles(d, offsets, BM, tiles, s);
  if (e != hipSuccess) return e;
  const int64_t mt = ffn_grid_mtiles(d, BM);
  uint8_t* hq_s = hq + d.N * d.I;
  float* hs_s = hs + d.N * (d.I / 128);

  Gemm8Args a1{};
  a1.tiles = tiles;
  a1.ntn = (std::max(d.I, d.Is) + BNB / 2 - 1) / (BNB / 2);
  a1.E = d.E;
  a1.K = d.K;
  a1.a_r = a1.a_s = xq;
  a1.as_r = a1.as_s = xs;
  a1.perm = perm;
  a1.kdim_r = a1.kdim_s = d.H;
  a1.b_r = w13;
  a1.b_es = (int64_t)2 * d.I * d.H;
  a1.bs_r = w13s;
  a1.bs_es = (int64_t)(2 * d.I / 128) * (d.H / 128);
  a1.b_s = ws13;
  a1.bs_s = ws13s;
  a1.ncol_r = d.I;
  a1.ncol_s = d.Is;
  a1.hq_r = hq;
  a1.hq_s = hq_s;
  a1.hs_r = hs;
  a1.hs_s = hs_s;
  MOE_TIMED_LAUNCH(s, "grouped_gemm_fp8<true>",
    hipLaunchKernelGGL(grouped_gemm_fp8<true>, dim3(xcd_grid(mt * a1.ntn)), dim3(NT), kLds8, s, a1));
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  Gemm8Args a2{};
  a2.tiles = tiles;
  a2.ntn = (d.H + BNB - 1) / BNB;
  a2.E = d.E;
  a2.K = d.K;
  a2.a_r = hq;
  a2.a_s = hq_s;
  a2.as_r = hs;
  a2.as_s = hs_s;
  a2.perm = nullptr;
  a2.kdim_r = d.I;
  a2.kdim_s = d.Is;
  a2.b_r = w2;
  a2.b_es = (int64_t)d.H * d.I;
  a2.bs_r = w2s;
  a2.bs_es = (int64_t)(d.H / 128) * (d.I / 128);
  a2.b_s = ws2;
  a2.bs_s = ws2s;
  a2.ncol_r = a2.ncol_s = d.H;
  a2.c_r = y;
  a2.c_s = ys;
  MOE_TIMED_LAUNCH(s, "grouped_gemm_fp8<false>",
    hipLaunchKernelGGL(grouped_gemm_fp8<false>, dim3(xcd_grid(mt * a2.ntn)), dim3(NT), kLds8, s, a2));
  return hipGetLastError();
}

}  // namespace moe
