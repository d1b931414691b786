// Grouped FP8 expert GEMMs with the e4m3 weights in a packed streaming
// layout (gfx950), fp32 accumulation.
//
// Quantisation granularity from "深入理解 DeepSeek-V3：大规模缩放挑战与对 AI 架构硬件的反思
// （中文精读）", section 3.2: activations per 1x128 tile, weights per 128x128
// block, fp32 accumulation.  The layer math (SwiGLU experts, the shared expert
// as group E) is that of the bf16 kernels.
//
// Packed layout: for every (matrix, output tile, 128-k step) one contiguous
// 32 KiB block holding the MFMA operand fragments in consumption order,
//   block = [wave 4][col block 2][k half 2][16-byte half 2][lane 64] x 16 bytes
// lane l of (wave w, col block cb, k half kk, half hf) holds weight row
//   GEMM1: cb = 0 gate row n0 + 32w + l%32, cb = 1 up row I + n0 + 32w + l%32
//   GEMM2: row n0 + 64w + 32cb + l%32
// at k = 128 step + 64 kk + 32 (l / 32) + 16 hf .. +16 (rows past the matrix:
// zeros).  The weight block scales stay in their row-major
// [matrices][rows/128][k/128] array.
//
// Roles: the weights are the MFMA's row operand and the tokens its column
// operand, so every lane of a 32x32 result block holds one token (column) and
// 16 weight rows.  Each 128-k step is one scale block: two 32x32x64 e4m3 MFMAs
// give its partial sum, which is added to the fp32 accumulator times
// (token scale of the lane) x (weight block scale of the wave): one multiply
// and 16 FMAs per block, with no per-row scale vectors.  (On MI355X the
// matrix core accumulates in fp32, so nothing needs promoting; only the
// scales are applied per block.)
//
// Tiles hold up to 128 tokens (4 blocks of 32) so that accumulators,
// partial sums and operands all fit in registers next to the two weight
// register stages.  Weight tiles read by one M-tile stream non-temporally;
// tiles shared by several M-tiles of a group stay in L2 for the others.
#include "moe_internal.hpp"

#include <algorithm>

namespace moe {

namespace {

constexpr int BM = kMinTileRows;   // 128 tokens per tile (NRB <= 4)
constexpr int BK = 128;            // k per step: one scale block
constexpr int NT = 256;
constexpr int FRAG = 2048;         // 16-byte fragments per packed block (32 KiB)
// LDS: token tile double buffer + token scales; the epilogue reuses it.
constexpr size_t kLdsMain = (size_t)2 * BM * 8 * sizeof(u32x4) + 2 * BM * sizeof(float);
// Epilogue LDS rows are padded by 16 bytes (kQRow, kCRow), so that the 32
// token rows a wave writes with one instruction fall in different banks.
constexpr int kQRow = 128 + 16;    // bytes per h-code row
constexpr int kCRow = 256 + 8;     // bf16 values per output row
constexpr size_t kLdsEpi1 = (size_t)4 * BM * sizeof(float) + (size_t)BM * kQRow;  // amax + codes
constexpr size_t kLdsEpi2 = (size_t)BM * kCRow * sizeof(uint16_t);                // bf16 rows
constexpr size_t kLds = std::max(kLdsMain, std::max(kLdsEpi1, kLdsEpi2));        // 66 KiB

// fp32 -> e4m3fn bits: round to nearest even, saturate at 448.
__device__ __forceinline__ uint32_t to_e4m3(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a >= 0x43E00000u) return sign | 0x7Eu;            // |v| >= 448 (or inf/nan)
  if (a >= 0x3C800000u) {                               // |v| >= 2^-6: normal
    const uint32_t mant = a & 0x7FFFFFu;
    uint32_t code = (((a >> 23) - 120u) << 3) | (mant >> 20);
    const uint32_t rem = mant & 0xFFFFFu;
    code += (rem > 0x80000u || (rem == 0x80000u && (code & 1u))) ? 1u : 0u;
    return sign | (code > 0x7Eu ? 0x7Eu : code);
  }
  const float sc = __uint_as_float(a) * 512.0f;         // subnormal: units of 2^-9
  return sign | (uint32_t)__builtin_rintf(sc);
}

// ---------------------------------------------------------------- packing

template <bool kGateUp>
__global__ void __launch_bounds__(256)
pack8_kernel(const uint8_t* __restrict__ src, u32x4* __restrict__ dst, int64_t nfrag, int n,
             int kd, int rows_total, int nt, int steps) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= nfrag) return;
  const int l = (int)(c & 63), hf = (int)((c >> 6) & 1), kk = (int)((c >> 7) & 1),
            cb = (int)((c >> 8) & 1), w = (int)((c >> 9) & 3);
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
  const int k = ks * BK + 64 * kk + 32 * (l >> 5) + 16 * hf;
  u32x4 v = {0, 0, 0, 0};
  if (ok) v = *reinterpret_cast<const u32x4*>(src + (e * rows_total + row) * (int64_t)kd + k);
  dst[c] = v;
}

// ---------------------------------------------------------------- GEMM

struct Packed8Args {
  const int32_t* tiles;
  int ntn;                      // N-tiles per M-tile (max over groups)
  int E, K;
  const uint8_t* a_r;           // token rows (e4m3), row length kdim
  const uint8_t* a_s;
  const float* as_r;            // token scales [rows][kdim / 128]
  const float* as_s;
  const int32_t* perm;          // GEMM1: routed token row = perm[j] / K
  int kdim_r, kdim_s;
  const u32x4* b_r;             // packed routed weights
  const u32x4* b_s;             // packed shared weights
  int nt_r, nt_s;               // output tiles per matrix
  const float* bs_r;            // weight block scales [E][rows / 128][kdim / 128]
  const float* bs_s;
  int ncol_r, ncol_s;           // output columns (I or Is for GEMM1, H for GEMM2)
  uint8_t* hq_r;                // GEMM1 outputs: e4m3 h + [rows][ncol / 128] scales
  uint8_t* hq_s;
  float* hs_r;
  float* hs_s;
  uint16_t* c_r;                // GEMM2 outputs: bf16, row length ncol
  uint16_t* c_s;
};

__device__ __forceinline__ int swz(int r, int c) { return r * 8 + (c ^ ((r ^ (r >> 3)) & 7)); }

__device__ __forceinline__ i32x8 cat8(u32x4 p, u32x4 q) {
  i32x8 r;
  r[0] = (int)p.x; r[1] = (int)p.y; r[2] = (int)p.z; r[3] = (int)p.w;
  r[4] = (int)q.x; r[5] = (int)q.y; r[6] = (int)q.z; r[7] = (int)q.w;
  return r;
}

template <bool kGateUp, int NRB, bool kStream>
__device__ __forceinline__ void fp8_tile(const Packed8Args& p, u32x4* smem, int g, int row0,
                                         int nrows, int ntile) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, lh = lane >> 5;
  const bool sh = (g == p.E);
  const int ncol = sh ? p.ncol_s : p.ncol_r;
  const int n0 = ntile * (kGateUp ? 128 : 256);
  const int kdim = sh ? p.kdim_s : p.kdim_r;
  const int nsteps = kdim / BK;
  const int last = nsteps - 1;
  const uint8_t* A = sh ? p.a_s : p.a_r;
  const float* As = sh ? p.as_s : p.as_r;
  const int nt = sh ? p.nt_s : p.nt_r;
  const u32x4* bw = (sh ? p.b_s : p.b_r + (int64_t)g * nt * nsteps * FRAG) +
                    (int64_t)ntile * nsteps * FRAG + wave * 512 + lane;
  // Weight block scales of this wave's two 32-row blocks.
  const int rows_total = kGateUp ? 2 * ncol : ncol;
  const float* bs = (sh ? p.bs_s : p.bs_r + (int64_t)g * (rows_total / 128) * nsteps);
  const int rb0 = kGateUp ? n0 / 128 : (n0 + 64 * wave) / 128;
  const int rb1 = kGateUp ? (ncol + n0) / 128 : rb0;
  const float* bs0 = bs + (int64_t)rb0 * nsteps;
  const float* bs1 = bs + (int64_t)rb1 * nsteps;

  u32x4* sA = smem;                                            // [2][BM * 8]
  float* sS = reinterpret_cast<float*>(smem + 2 * BM * 8);     // [2][BM]

  // Token rows staged by this thread: r = tid/8 + 32 j (j < NRB), chunk
  // tid % 8; thread tid < BM also stages the scale of row tid.  Rows past
  // the tile's end re-read its first row (their results are not stored).
  const int ch = tid & 7;
  const int first = (!sh && kGateUp) ? p.perm[row0] / p.K : row0;
  const uint8_t* arow[NRB];
#pragma unroll
  for (int j = 0; j < NRB; ++j) {
    const int r = (tid >> 3) + 32 * j;
    int a = first;
    if (r < nrows) a = (!sh && kGateUp) ? p.perm[row0 + r] / p.K : row0 + r;
    arow[j] = A + (int64_t)a * kdim + ch * 16;
  }
  int srow = first;
  if (tid < nrows) srow = (!sh && kGateUp) ? p.perm[row0 + tid] / p.K : row0 + tid;
  const float* sptr = As + (int64_t)srow * nsteps;
  const bool stages_scale = tid < 32 * NRB;

  u32x4 ra[2][NRB];
  float rs[2];
  auto aload = [&](int st, int j, int step) {
    ra[st][j] = *reinterpret_cast<const u32x4*>(arow[j] + min(step, last) * BK);
  };
  auto astore = [&](int st, int j, int buf) {
    sA[buf * BM * 8 + swz((tid >> 3) + 32 * j, ch)] = ra[st][j];
  };
  auto sload = [&](int st, int step) { rs[st] = sptr[min(step, last)]; };
  auto sstore = [&](int st, int buf) {
    if (stages_scale) sS[buf * BM + tid] = rs[st];
  };
  u32x4 rb[2][8];   // weight fragments [slot][(cb * 2 + kk) * 2 + hf]
  auto bload = [&](int slot, int i, int step) {
    const u32x4* src = bw + (int64_t)min(step, last) * FRAG + i * 64;
    rb[slot][i] = kStream ? __builtin_nontemporal_load(src) : *src;
  };

  f32x16 acc[NRB][2];
#pragma unroll
  for (int r = 0; r < NRB; ++r)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[r][c][i] = 0.0f;

  // Step on LDS buffer `buf` with weight slot `u`.  Per token block r: the
  // two MFMA pairs (one per weight block) of block r are issued, then the
  // scaled accumulation of block r - 1, so MFMA latency hides behind VALU
  // work; token-staging operations and, after the last block, the weight
  // refill of this slot are spread between the blocks.
  // Weight block scales of the step, loaded one step ahead (scalar loads
  // waited for in the same step would stall it).
  float sbn0 = bs0[0], sbn1 = bs1[0];
  auto step_body = [&](int buf, int u, int step) {
    const u32x4* as = sA + buf * BM * 8;
    const float* ss = sS + buf * BM;
    const float sb0 = sbn0, sb1 = sbn1;
    sbn0 = bs0[min(step + 1, last)];
    sbn1 = bs1[min(step + 1, last)];
    const int nst = (u + 1) & 1;      // register stage holding step + 1
    f32x16 part[2][2];
    float sc[2][2];
    auto flush = [&](int r) {
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          acc[r][c][i] = fmaf(part[r & 1][c][i], sc[r & 1][c], acc[r][c][i]);
    };
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      const int row = r * 32 + lr;
      const i32x8 t0 = cat8(as[swz(row, 2 * lh)], as[swz(row, 2 * lh + 1)]);
      const i32x8 t1 = cat8(as[swz(row, 4 + 2 * lh)], as[swz(row, 4 + 2 * lh + 1)]);
      const float sa = ss[row];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const i32x8 w0 = cat8(rb[u][c * 4 + 0], rb[u][c * 4 + 1]);
        const i32x8 w1 = cat8(rb[u][c * 4 + 2], rb[u][c * 4 + 3]);
        f32x16 z;
#pragma unroll
        for (int i = 0; i < 16; ++i) z[i] = 0.0f;
        z = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w0, t0, z, 0, 0, 0, 127, 0, 127);
        part[r & 1][c] =
            __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w1, t1, z, 0, 0, 0, 127, 0, 127);
      }
      sc[r & 1][0] = sa * sb0;
      sc[r & 1][1] = sa * sb1;
      if (r > 0) flush(r - 1);
      // token staging: chunk r of step + 1 to LDS, its registers refilled
      // with step + 3 (the other stage already holds step + 2)
      astore(nst, r, buf ^ 1);
      aload(nst, r, step + 3);
      if (r == 0) {
        sstore(nst, buf ^ 1);
        sload(nst, step + 3);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    flush(NRB - 1);
#pragma unroll
    for (int i = 0; i < 8; ++i) bload(u, i, step + 2);
  };

  // Prologue (in loop order: tokens of step j + 1, then weights of step j).
#pragma unroll
  for (int j = 0; j < NRB; ++j) aload(0, j, 0);
  sload(0, 0);
#pragma unroll
  for (int j = 0; j < NRB; ++j) aload(1, j, 1);
  sload(1, 1);
#pragma unroll
  for (int i = 0; i < 8; ++i) bload(0, i, 0);
#pragma unroll
  for (int j = 0; j < NRB; ++j) astore(0, j, 0);
  sstore(0, 0);
#pragma unroll
  for (int j = 0; j < NRB; ++j) aload(0, j, 2);
  sload(0, 2);
#pragma unroll
  for (int i = 0; i < 8; ++i) bload(1, i, 1);
  __syncthreads();

  // Step t: LDS buffer t % 2, weight slot t % 2, token registers of step
  // t + 1 in stage (t + 1) % 2.
  int s = 0;
  for (; s + 2 <= nsteps; s += 2) {
    step_body(0, 0, s);
    __syncthreads();
    step_body(1, 1, s + 1);
    __syncthreads();
  }
  if (s < nsteps) {
    step_body(0, 0, s);
    __syncthreads();
  }

  // Epilogue.  Lane (r, lr) holds token r * 32 + lr; value i of column block
  // c is weight row 8 (i / 4) + 4 lh + i % 4 of that block.
  if (kGateUp) {
    // h = silu(g) * up; each token's 128 h columns of this tile are one
    // quantisation tile (32 per wave): amax over lanes lh = 0, 1 by a
    // shuffle, over the 4 waves through LDS.
    float* sMax = reinterpret_cast<float*>(smem);                   // [4][BM]
    uint8_t* sQ = reinterpret_cast<uint8_t*>(smem) + 4 * BM * 4;   // [BM][kQRow]
    float hv[NRB][16];
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float gv = acc[r][0][i], uv = acc[r][1][i];
        hv[r][i] = gv / (1.0f + __expf(-gv)) * uv;
        m = fmaxf(m, fabsf(hv[r][i]));
      }
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      if (lh == 0) sMax[wave * BM + r * 32 + lr] = m;
    }
    __syncthreads();
    uint8_t* HQ = sh ? p.hq_s : p.hq_r;
    float* HS = sh ? p.hs_s : p.hs_r;
    const int nblk = ncol / 128;
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      const int tok = r * 32 + lr;
      const float m = fmaxf(fmaxf(sMax[tok], sMax[BM + tok]),
                            fmaxf(sMax[2 * BM + tok], sMax[3 * BM + tok]));
      float scale = 1.0f, inv = 0.0f;
      if (m > 0.0f) {
        scale = (float)((double)m / 448.0);
        inv = (float)(448.0 / (double)m);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t word = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) word |= to_e4m3(hv[r][4 * q + b] * inv) << (8 * b);
        // h columns 32 wave + 8 q + 4 lh .. +4 of this tile
        *reinterpret_cast<uint32_t*>(sQ + tok * kQRow + 32 * wave + 8 * q + 4 * lh) = word;
      }
      if (wave == 0 && lh == 0 && tok < nrows) HS[(int64_t)(row0 + tok) * nblk + n0 / 128] = scale;
    }
    __syncthreads();
    // 16-byte coalesced copy: 8 threads per token row of 128 codes.
    for (int c = tid; c < nrows * 8; c += NT) {
      const int tok = c >> 3, part = c & 7;
      *reinterpret_cast<u32x4*>(HQ + (int64_t)(row0 + tok) * ncol + n0 + 16 * part) =
          *reinterpret_cast<const u32x4*>(sQ + tok * kQRow + 16 * part);
    }
  } else {
    __syncthreads();   // the token tile is no longer read
    uint16_t* sC = reinterpret_cast<uint16_t*>(smem);   // [BM][kCRow]
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      const int tok = r * 32 + lr;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = 64 * wave + 32 * c + 8 * q + 4 * lh;
          const uint32_t lo = pack_bf16x2(acc[r][c][4 * q], acc[r][c][4 * q + 1]);
          const uint32_t hi = pack_bf16x2(acc[r][c][4 * q + 2], acc[r][c][4 * q + 3]);
          *reinterpret_cast<uint2*>(sC + tok * kCRow + col) = make_uint2(lo, hi);
        }
    }
    __syncthreads();
    uint16_t* C = sh ? p.c_s : p.c_r;
    const int width = min(256, ncol - n0);   // multiple of 8 (H % 128 == 0)
    const int per_row = width / 8;
    for (int c = tid; c < nrows * 32; c += NT) {
      const int tok = c >> 5, part = c & 31;
      if (part < per_row)
        *reinterpret_cast<u32x4*>(C + (int64_t)(row0 + tok) * ncol + n0 + 8 * part) =
            *reinterpret_cast<const u32x4*>(sC + tok * kCRow + 8 * part);
    }
  }
}

template <bool kGateUp>
__global__ void __launch_bounds__(NT, 1) grouped_gemm_fp8_packed(Packed8Args p) {
  extern __shared__ u32x4 smem[];
  const int64_t work = (int64_t)p.tiles[0] * p.ntn;
  const int64_t w = xcd_chunked(blockIdx.x, work);
  if (w < 0) return;
  int ntile;
  const int32_t* ent = decode_work(p.tiles, w, p.ntn, ntile);
  const int g = ent[0], row0 = ent[1], nrows = ent[2];
  if (ntile >= ((g == p.E) ? p.nt_s : p.nt_r)) return;
  // A weight tile read by one M-tile only streams past the caches; one
  // shared by several M-tiles of a group stays in L2 for the others.
  const bool stream = ent[4] == 1;
  switch (((nrows + 31) >> 5) * 2 + (stream ? 1 : 0)) {
#define MOE_FP8_CASE(n)                                                                    \
    case 2 * n: fp8_tile<kGateUp, n, false>(p, smem, g, row0, nrows, ntile); break;       \
    case 2 * n + 1: fp8_tile<kGateUp, n, true>(p, smem, g, row0, nrows, ntile); break;
    MOE_FP8_CASE(1)
    MOE_FP8_CASE(2)
    MOE_FP8_CASE(3)
    MOE_FP8_CASE(4)
#undef MOE_FP8_CASE
    default:
      break;
  }
}

hipError_t set_attrs_fp8_packed() {
  static hipError_t once = []() {
    hipError_t e = hipFuncSetAttribute((const void*)grouped_gemm_fp8_packed<true>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute((const void*)grouped_gemm_fp8_packed<false>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
  }();
  return once;
}

}  // namespace

// Packed fp8 sizes in bytes.  GEMM1 matrices: n = I or Is output columns in
// tiles of 128, kd = H; GEMM2 matrices: n = H output rows in tiles of 256,
// kd = I or Is.
size_t packed8_bytes(bool gate_up, int64_t experts, int n, int kd) {
  const int64_t nt = gate_up ? (n + 127) / 128 : (n + 255) / 256;
  return (size_t)(experts * nt * (kd / BK) * FRAG) * sizeof(u32x4);
}

hipError_t launch_pack8(bool gate_up, const uint8_t* src, void* dst, int64_t experts, int n,
                        int kd, hipStream_t s) {
  const int nt = gate_up ? (n + 127) / 128 : (n + 255) / 256;
  const int steps = kd / BK;
  const int64_t nfrag = experts * nt * steps * FRAG;
  const unsigned blocks = (unsigned)((nfrag + 255) / 256);
  if (gate_up)
    MOE_TIMED_LAUNCH(s, "pack8_kernel<true>",
      hipLaunchKernelGGL(pack8_kernel<true>, dim3(blocks), dim3(256), 0, s, src, (u32x4*)dst,
                         nfrag, n, kd, 2 * n, nt, steps));
  else
    MOE_TIMED_LAUNCH(s, "pack8_kernel<false>",
      hipLaunchKernelGGL(pack8_kernel<false>, dim3(blocks), dim3(256), 0, s, src, (u32x4*)dst,
                         nfrag, n, kd, n, nt, steps));
  return hipGetLastError();
}

// hq: routed rows [0, N) width I, then shared rows width Is; hs likewise
// with I/128 and Is/128 scales per row.
hipError_t launch_ffn_fp8_packed(const FfnDims& d, const uint8_t* xq, const float* xs,
                                 const int32_t* perm, const int32_t* offsets, const void* w13p,
                                 const float* w13s, const void* w2p, const float* w2s,
                                 const void* ws13p, const float* ws13s, const void* ws2p,
                                 const float* ws2s, uint8_t* hq, float* hs, int32_t* tiles,
                                 uint16_t* y, uint16_t* ys, hipStream_t s) {
  hipError_t e = set_attrs_fp8_packed();
  if (e != hipSuccess) return e;
  // balanced M-tiles: a weight tile's M-tiles stream it at the same pace
  e = ffn_build_tiles(d, offsets, BM, tiles, s, true);
  if (e != hipSuccess) return e;
  const int64_t mt = ffn_grid_mtiles(d, BM);

  Packed8Args a1{};
  a1.tiles = tiles;
  a1.nt_r = (d.I + 127) / 128;
  a1.nt_s = (d.Is + 127) / 128;
  a1.ntn = std::max(a1.nt_r, a1.nt_s);
  a1.E = d.E;
  a1.K = d.K;
  a1.a_r = a1.a_s = xq;
  a1.as_r = a1.as_s = xs;
  a1.perm = perm;
  a1.kdim_r = a1.kdim_s = d.H;
  a1.b_r = (const u32x4*)w13p;
  a1.b_s = (const u32x4*)ws13p;
  a1.bs_r = w13s;
  a1.bs_s = ws13s;
  a1.ncol_r = d.I;
  a1.ncol_s = d.Is;
  a1.hq_r = hq;
  a1.hq_s = hq + d.N * d.I;
  a1.hs_r = hs;
  a1.hs_s = hs + d.N * (d.I / 128);
  MOE_TIMED_LAUNCH(s, "grouped_gemm_fp8_packed<true>",
    hipLaunchKernelGGL(grouped_gemm_fp8_packed<true>, dim3(xcd_grid(mt * a1.ntn)), dim3(NT), kLds, s,
                       a1));
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  Packed8Args a2{};
  a2.tiles = tiles;
  a2.nt_r = a2.nt_s = (d.H + 255) / 256;
  a2.ntn = a2.nt_r;
  a2.E = d.E;
  a2.K = d.K;
  a2.a_r = hq;
  a2.a_s = a1.hq_s;
  a2.as_r = hs;
  a2.as_s = a1.hs_s;
  a2.perm = nullptr;
  a2.kdim_r = d.I;
  a2.kdim_s = d.Is;
  a2.b_r = (const u32x4*)w2p;
  a2.b_s = (const u32x4*)ws2p;
  a2.bs_r = w2s;
  a2.bs_s = ws2s;
  a2.ncol_r = a2.ncol_s = d.H;
  a2.c_r = y;
  a2.c_s = ys;
  MOE_TIMED_LAUNCH(s, "grouped_gemm_fp8_packed<false>",
    hipLaunchKernelGGL(grouped_gemm_fp8_packed<false>, dim3(xcd_grid(mt * a2.ntn)), dim3(NT), kLds, s,
                       a2));
  return hipGetLastError();
}

}  // namespace moe
