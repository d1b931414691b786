// One wave slot of one tile of the few-row grouped expert GEMM on bf16
// weights in the packed streaming layout (gfx950), shared by the decode
// batches' GEMM kernels and the one-launch decode layer.
//
// Few-row tiles: every group of a decode batch has at most 32 * NRB rows
// (NRB <= 2).  The activation rows are few and L2-resident, so each wave
// loads its own MFMA operands for them straight from global memory: waves
// are independent (no LDS, no barrier), use few registers, and two waves
// share each SIMD, which keeps more weight loads in flight.  The four wave
// slots of a tile each take a quarter of its packed weight tile.  The
// arithmetic of a slot does not depend on which wave or workgroup runs it,
// so every caller gets the same bits.
#pragma once

#include "moe_internal.hpp"

namespace moe {

constexpr int kPackedBK = 64;      // k per packed step
constexpr int kPackedFrag = 2048;  // 16-byte fragments per packed block (32 KiB)
constexpr int kFewSlots = 4;       // waves (packed wave slots) per tile

// Arguments of the packed grouped GEMMs: routed groups (..._r) and the
// shared expert (group E, ..._s).
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

// Wave slot `wave` of the tile (group g, rows row0 .. row0 + nrows, output
// tile ntile), D steps of weights and activations in flight.  GEMM1
// (kGateUp) writes h = silu(g) * u, GEMM2 the bf16 output rows.
template <bool kGateUp, int NRB, int D>
__device__ __forceinline__ void few_tile(const PackedArgs& p, int g, int row0, int nrows,
                                         int ntile, int wave) {
  const bool sh = (g == p.E);
  const int lane = threadIdx.x & 63;
  const int lr = lane & 31, lh = lane >> 5;
  const int ncol = sh ? p.ncol_s : p.ncol_r;
  const int n0 = ntile * (kGateUp ? 128 : 256);
  const int kdim = sh ? p.kdim_s : p.kdim_r;
  const int nsteps = kdim / kPackedBK;
  const int last = nsteps - 1;
  const uint16_t* A = sh ? p.a_s : p.a_r;
  const int64_t lda = sh ? p.lda_s : p.lda_r;
  const u32x4* bw = (sh ? p.b_s : p.b_r + (int64_t)g * p.nt_r * nsteps * kPackedFrag) +
                    (int64_t)ntile * nsteps * kPackedFrag + wave * 512 + lane;
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
    const u32x4* src = bw + (int64_t)st * kPackedFrag;
#pragma unroll
    for (int i = 0; i < 8; ++i) rb[slot][i] = __builtin_nontemporal_load(src + i * 64);
#pragma unroll
    for (int r = 0; r < NRB; ++r)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        ra[slot][r][kk] = *reinterpret_cast<const u32x4*>(ap[r] + st * kPackedBK + kk * 8);
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


}  // namespace moe
