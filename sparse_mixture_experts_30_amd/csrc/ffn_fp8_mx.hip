// Grouped FP8 expert GEMMs whose block scales are applied by the matrix
// cores (gfx950), for e4m3 weights and activations with power-of-two scales.
//
// "深入理解 DeepSeek-V3：大规模缩放挑战与对 AI 架构硬件的反思（中文精读）", section 3.2:
// activations per 1x128 tile and weights per 128x128 block; dequantising
// means moving each partial sum out of the matrix unit to multiply it by the
// scales, which is costly, and the page asks for matrix units that take the
// scaling factors themselves.  gfx950's scaled MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4) is such a unit: every lane passes one
// E8M0 exponent for the operand values it holds, and the product is formed
// as (a 2^sa)(b 2^sb) inside the instruction.  With power-of-two block scales
// the whole k loop therefore runs on the matrix cores: the accumulator is the
// MFMA's own, with no per-block vector work at all.
//
// Operand roles and lane layout (measured on gfx950 with a layout probe):
// weights are the row operand A, tokens the column operand B.  Lane l of a
// 32x32x64 MFMA holds row (A) or column (B) l % 32 and 32 e4m3 values of one
// k half; the instruction splits each lane's 32 bytes into two 32-wide scale
// blocks and takes block b's scale of row/column r from lane r + 32 b.  Every
// 64-k MFMA lies inside one 128-k scale block, and both lanes of a row or
// column carry that block's scale, so each lane simply passes the scale of
// its own row (weight block) or token.
//
// The accumulation inside the e4m3 MFMA is not a full fp32 sum: against an
// exact sum the result differs by up to about 2^-13 of the magnitudes added
// (products and the accumulator input), as on the page's Hopper tensor cores
// (13 fraction bits).  Summed over the k loop that stays below the bf16
// rounding of the outputs; the parity tests bound the whole layer.
//
// Tiles: up to 256 tokens (8 blocks of 32) x 256 weight rows (GEMM1: the
// gate and up rows of 128 h columns; GEMM2: 256 output columns), 4 waves,
// wave w on weight rows 64 w .. +64 (two 32-row blocks) for all tokens, so a
// 256-row expert reads each weight tile from HBM once; a larger expert is
// cut into M-tiles of equal height, which stream the shared weight tile at
// the same pace (the second reader hits L2).  Weights stream from the packed
// layout of moe_pack_weight straight into a ring of four half-step register
// slots (1.5 steps of lead); token rows (gathered through perm for GEMM1) go
// through a double-buffered, XOR-swizzled LDS tile with their scales.  The
// 8 x 2 accumulator blocks of a wave (256 fp32 per lane) live in the
// accumulation registers.  GEMM1's epilogue forms h = silu(g) * u and
// quantises it per 1x128 tile with a power-of-two scale; GEMM2 writes bf16
// rows through LDS.
#include "moe_internal.hpp"

#include <algorithm>

namespace moe {

namespace {

constexpr int BM = 256;            // tokens per tile (NRB <= 8 blocks of 32)
constexpr int BK = 128;            // k per step: one scale block
constexpr int NT = 256;
constexpr int FRAG = 2048;         // 16-byte fragments per packed block (32 KiB)
// LDS: token tile double buffer + token scales; the epilogues reuse it
// (GEMM1: tile maxima [4][BM] + codes [BM][128]; GEMM2: bf16 rows of half
// the tokens, [BM/2][256]).
constexpr size_t kLdsMain = (size_t)2 * BM * 8 * sizeof(u32x4) + 2 * BM * sizeof(float);
// Epilogue LDS rows are padded by 16 bytes (kQRow, kCRow), so that the 32
// token rows a wave writes with one instruction fall in different banks.
constexpr int kQRow = 128 + 16;    // bytes per h-code row
constexpr int kCRow = 256 + 8;     // bf16 values per output row
constexpr size_t kLdsEpi1 = (size_t)4 * BM * sizeof(float) + (size_t)BM * kQRow;
constexpr size_t kLdsEpi2 = (size_t)(BM / 2) * kCRow * sizeof(uint16_t);
constexpr size_t kLds = std::max(kLdsMain, std::max(kLdsEpi1, kLdsEpi2));   // 66 KiB

// fp32 -> e4m3fn bits, round to nearest even; |v| <= 448 on this path.
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a >= 0x43E00000u) return sign | 0x7Eu;
  if (a >= 0x3C800000u) {
    const uint32_t mant = a & 0x7FFFFFu;
    uint32_t code = (((a >> 23) - 120u) << 3) | (mant >> 20);
    const uint32_t rem = mant & 0xFFFFFu;
    code += (rem > 0x80000u || (rem == 0x80000u && (code & 1u))) ? 1u : 0u;
    return sign | (code > 0x7Eu ? 0x7Eu : code);
  }
  return sign | (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
}

// E8M0 exponent of a positive power-of-two fp32 scale: its exponent field
// (both formats have bias 127).
__device__ __forceinline__ int e8m0_of(float s) { return (int)(__float_as_uint(s) >> 23) & 0xFF; }

struct MxArgs {
  const int32_t* tiles;
  int ntn;                      // N-tiles per M-tile (max over groups)
  int E, K;
  const uint8_t* a_r;           // token rows (e4m3), row length kdim
  const uint8_t* a_s;
  const float* as_r;            // token scales [rows][kdim / 128], powers of two
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

// LDS slot of 16-byte chunk c of token row r: the chunk index is XORed with
// a key of r % 32 only, so that the 32 rows a wave reads with one
// instruction hit distinct banks, while rows 32 apart (token blocks) keep the
// same key and their addresses differ by a constant (immediate offsets).
__device__ __forceinline__ int swz(int r, int c) {
  const int k = r & 31;
  return r * 8 + (c ^ ((k ^ (k >> 3)) & 7));
}

__device__ __forceinline__ i32x8 cat8(u32x4 p, u32x4 q) {
  i32x8 r;
  r[0] = (int)p.x; r[1] = (int)p.y; r[2] = (int)p.z; r[3] = (int)p.w;
  r[4] = (int)q.x; r[5] = (int)q.y; r[6] = (int)q.z; r[7] = (int)q.w;
  return r;
}

template <bool kGateUp, int NRB, bool kStream>
__device__ __forceinline__ void mx_tile(const MxArgs& p, u32x4* smem, int g, int row0, int nrows,
                                        int ntile) {
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
  // Weight block scales of this wave's two 32-row blocks (GEMM1: the gate
  // and up rows of h columns n0 .. n0 + 127; GEMM2: rows n0 + 64 w ..).
  const int rows_total = kGateUp ? 2 * ncol : ncol;
  const float* bs = (sh ? p.bs_s : p.bs_r + (int64_t)g * (rows_total / 128) * nsteps);
  const int rb0 = kGateUp ? n0 / 128 : (n0 + 64 * wave) / 128;
  const int rb1 = kGateUp ? (ncol + n0) / 128 : rb0;
  const float* bs0 = bs + (int64_t)rb0 * nsteps;
  const float* bs1 = bs + (int64_t)rb1 * nsteps;

  u32x4* sA = smem;                                            // [2][BM * 8]
  float* sS = reinterpret_cast<float*>(smem + 2 * BM * 8);     // [2][BM]

  // Token rows staged by this thread: r = tid / 8 + 32 j (j < NRB), chunk
  // tid % 8; thread tid < 32 NRB also stages the scale of row tid.  Rows past
  // the tile's end re-read its first row (their results are not stored).
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
  const uint8_t* abase = A + ch * 16;
  int srow = first;
  if (tid < nrows) srow = (!sh && kGateUp) ? p.perm[row0 + tid] / p.K : row0 + tid;
  const float* sptr = As + (int64_t)srow * nsteps;
  const bool stages_scale = tid < 32 * NRB;

  // One register stage of token staging: during step t the registers of
  // chunk j (step t + 1) move to the other LDS buffer and are refilled with
  // step t + 2 at once, a full step ahead of their next store.
  u32x4 ra[NRB];
  float rs;
  auto aload = [&](int j, int step) {
    ra[j] = *reinterpret_cast<const u32x4*>(abase + (int64_t)arow[j] * kdim +
                                            min(step, last) * BK);
  };
  auto astore = [&](int j, int buf) {
    sA[buf * BM * 8 + swz((tid >> 3) + 32 * j, ch)] = ra[j];
  };
  auto sload = [&](int step) { rs = sptr[min(step, last)]; };
  auto sstore = [&](int buf) {
    if (stages_scale) sS[buf * BM + tid] = rs;
  };
  // Weight fragments in a ring of kHalf half-step slots: half-step h = 2
  // step + kk (one 64-k half of a step) holds, for each column block c, the
  // two 16-byte fragments of packed index (c * 2 + kk) * 2 + half.  A slot is
  // refilled with half-step h + kHalf right after its last MFMA, so the
  // weight stream has kHalf - 1 half-steps in flight.
  constexpr int kHalf = 4;
  i32x8 wh[kHalf][2];
  auto bload = [&](int slot, int h) {
    const int step = h >> 1, kk = h & 1;
    const u32x4* src = bw + (int64_t)min(step, last) * FRAG;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int i = (c * 2 + kk) * 2;
      const u32x4 lo = kStream ? __builtin_nontemporal_load(src + i * 64) : src[i * 64];
      const u32x4 hi =
          kStream ? __builtin_nontemporal_load(src + (i + 1) * 64) : src[(i + 1) * 64];
      wh[slot][c] = cat8(lo, hi);
    }
  };

  f32x16 acc[NRB][2];
#pragma unroll
  for (int r = 0; r < NRB; ++r)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[r][c][i] = 0.0f;

  // Weight block scales of the step (E8M0), loaded one step ahead.
  float sbn0 = bs0[0], sbn1 = bs1[0];
  // Step on LDS buffer `buf`, its two k halves in weight slots sa and sb.
  // Each k half runs over the token blocks; block r's fragment is read from
  // LDS one block ahead of its two MFMAs (gate/up or two output row blocks),
  // so the LDS latency hides behind the previous block's matrix work.  In the
  // first half each block also moves its token chunk of the next step to
  // the other LDS buffer and refills the registers with the step after.
  auto step_body = [&](int buf, int sa, int sb, int step) {
    const u32x4* as = sA + buf * BM * 8;
    const float* ss = sS + buf * BM;
    const int sw0 = e8m0_of(sbn0), sw1 = e8m0_of(sbn1);
    sbn0 = bs0[min(step + 1, last)];
    sbn1 = bs1[min(step + 1, last)];
    auto tread = [&](int r, int kk) {
      const int row = r * 32 + lr;
      return cat8(as[swz(row, 4 * kk + 2 * lh)], as[swz(row, 4 * kk + 2 * lh + 1)]);
    };
    int st[NRB];
#pragma unroll
    for (int r = 0; r < NRB; ++r) st[r] = e8m0_of(ss[r * 32 + lr]);
    i32x8 tn = tread(0, 0);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int slot = kk ? sb : sa;
#pragma unroll
      for (int r = 0; r < NRB; ++r) {
        const i32x8 t = tn;
        if (r + 1 < NRB) tn = tread(r + 1, kk);
        else if (kk == 0) tn = tread(0, 1);
        acc[r][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wh[slot][0], t, acc[r][0],
                                                                    0, 0, 0, sw0, 0, st[r]);
        acc[r][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wh[slot][1], t, acc[r][1],
                                                                    0, 0, 0, sw1, 0, st[r]);
        if (kk == 0) {
          astore(r, buf ^ 1);
          aload(r, step + 2);
          if (r == 0) {
            sstore(buf ^ 1);
            sload(step + 2);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      bload(slot, 2 * step + kk + kHalf);
    }
  };

  // Prologue: step 0's tokens in LDS buffer 0, step 1's in registers, the
  // first kHalf half-steps of weights in their slots.
#pragma unroll
  for (int j = 0; j < NRB; ++j) aload(j, 0);
  sload(0);
#pragma unroll
  for (int j = 0; j < NRB; ++j) astore(j, 0);
  sstore(0);
#pragma unroll
  for (int j = 0; j < NRB; ++j) aload(j, 1);
  sload(1);
#pragma unroll
  for (int h = 0; h < kHalf; ++h) bload(h, h);
  __syncthreads();

  // Step t: LDS buffer t % 2, weight slots 2t % kHalf and (2t + 1) % kHalf,
  // token registers of step t + 1; unrolled by U steps (LDS buffer and slot
  // pattern both repeat) so every index is static.
  constexpr int U = (kHalf % 2) ? 2 * kHalf : (kHalf / 2 % 2 ? kHalf : kHalf / 2);
  static_assert((2 * U) % kHalf == 0 && U % 2 == 0, "unroll period");
  int s = 0;
  for (; s + U <= nsteps; s += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      step_body(u & 1, (2 * u) % kHalf, (2 * u + 1) % kHalf, s + u);
      __syncthreads();
    }
  }
#pragma unroll
  for (int u = 0; u < U - 1; ++u) {
    if (s + u < nsteps) {   // uniform over the workgroup
      step_body(u & 1, (2 * u) % kHalf, (2 * u + 1) % kHalf, s + u);
      __syncthreads();
    }
  }

  // Epilogue.  Lane (r, lr) holds token r * 32 + lr; value i of column block
  // c is weight row 8 (i / 4) + 4 lh + i % 4 of that block.
  if (kGateUp) {
    // h = silu(g) * u over the tile's 128 h columns of each token (one
    // quantisation tile), one token block at a time: the block's maximum
    // over lane halves by a shuffle and over the 4 waves through LDS, then
    // its codes; only one block's 16 h values are live at a time.
    float* sMax = reinterpret_cast<float*>(smem);                   // [4][BM]
    uint8_t* sQ = reinterpret_cast<uint8_t*>(smem) + 4 * BM * 4;   // [BM][kQRow]
    uint8_t* HQ = sh ? p.hq_s : p.hq_r;
    float* HS = sh ? p.hs_s : p.hs_r;
    const int nblk = ncol / 128;
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      float hv[16];
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float gv = acc[r][0][i], uv = acc[r][1][i];
        hv[i] = gv / (1.0f + __expf(-gv)) * uv;
        m = fmaxf(m, fabsf(hv[i]));
      }
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      const int tok = r * 32 + lr;
      if (lh == 0) sMax[wave * BM + tok] = m;
      __syncthreads();
      m = fmaxf(fmaxf(sMax[tok], sMax[BM + tok]), fmaxf(sMax[2 * BM + tok], sMax[3 * BM + tok]));
      // smallest power of two 2^e >= m / 448 (m / 448 in double is a power
      // of two only when it is computed exactly), e in [-126, 127]
      float scale = 1.0f, inv = 0.0f;
      if (m > 0.0f) {
        const uint64_t b = (uint64_t)__double_as_longlong((double)m / 448.0);
        int e = (int)((b >> 52) & 0x7FF) - 1023;
        if (b & 0xFFFFFFFFFFFFFull) ++e;
        e = min(max(e, -126), 127);
        scale = __uint_as_float((uint32_t)(e + 127) << 23);
        inv = __uint_as_float((uint32_t)(127 - e) << 23);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t word = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) word |= e4m3_rne(hv[4 * q + b] * inv) << (8 * b);
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
    // bf16 rows staged in LDS for 16-byte stores, half the tokens at a time.
    uint16_t* sC = reinterpret_cast<uint16_t*>(smem);   // [BM / 2][kCRow]
    uint16_t* C = sh ? p.c_s : p.c_r;
    const int width = min(256, ncol - n0);   // multiple of 8 (H % 128 == 0)
    const int per_row = width / 8;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (half * 4 >= NRB) break;
      __syncthreads();   // the token tile (or the first half) is no longer read
#pragma unroll
      for (int r = half * 4; r < NRB && r < half * 4 + 4; ++r) {
        const int tok = (r - half * 4) * 32 + lr;
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
      const int base = half * (BM / 2);
      const int rows_here = min(nrows - base, BM / 2);
      for (int c = tid; c < rows_here * 32; c += NT) {
        const int tok = c >> 5, part = c & 31;
        if (part < per_row)
          *reinterpret_cast<u32x4*>(C + (int64_t)(row0 + base + tok) * ncol + n0 + 8 * part) =
              *reinterpret_cast<const u32x4*>(sC + tok * kCRow + 8 * part);
      }
    }
  }
}

template <bool kGateUp>
__global__ void __launch_bounds__(NT, 1) grouped_gemm_fp8_mx(MxArgs p) {
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
#define MOE_MX_CASE(n)                                                                   \
    case 2 * n: mx_tile<kGateUp, n, false>(p, smem, g, row0, nrows, ntile); break;      \
    case 2 * n + 1: mx_tile<kGateUp, n, true>(p, smem, g, row0, nrows, ntile); break;
    MOE_MX_CASE(1)
    MOE_MX_CASE(2)
    MOE_MX_CASE(3)
    MOE_MX_CASE(4)
    MOE_MX_CASE(5)
    MOE_MX_CASE(6)
    MOE_MX_CASE(7)
    MOE_MX_CASE(8)
#undef MOE_MX_CASE
    default:
      break;
  }
}

hipError_t set_attrs_fp8_mx() {
  static hipError_t once = []() {
    hipError_t e = hipFuncSetAttribute((const void*)grouped_gemm_fp8_mx<true>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute((const void*)grouped_gemm_fp8_mx<false>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
  }();
  return once;
}

}  // namespace

// Packed e4m3 weights (moe_pack_weight's fp8 layout) with power-of-two block
// scales.  hq: routed rows [0, N) width I, then the shared expert's rows
// width Is; hs likewise with I/128 and Is/128 scales per row.
hipError_t launch_ffn_fp8_mx(const FfnDims& d, const uint8_t* xq, const float* xs,
                             const int32_t* perm, const int32_t* offsets, const void* w13p,
                             const float* w13s, const void* w2p, const float* w2s,
                             const void* ws13p, const float* ws13s, const void* ws2p,
                             const float* ws2s, uint8_t* hq, float* hs, int32_t* tiles,
                             uint16_t* y, uint16_t* ys, hipStream_t s) {
  hipError_t e = set_attrs_fp8_mx();
  if (e != hipSuccess) return e;
  // balanced M-tiles: an expert of 257..512 rows runs as two tiles of equal
  // height that stream its weight tiles side by side (the second reader hits
  // L2) instead of a full tile and a short one racing ahead
  e = ffn_build_tiles(d, offsets, BM, tiles, s, true);
  if (e != hipSuccess) return e;
  const int64_t mt = ffn_grid_mtiles(d, BM);

  MxArgs a1{};
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
  MOE_TIMED_LAUNCH(s, "grouped_gemm_fp8_mx<true>",
    hipLaunchKernelGGL(grouped_gemm_fp8_mx<true>, dim3(xcd_grid(mt * a1.ntn)), dim3(NT), kLds, s,
                       a1));
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  MxArgs a2{};
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
  MOE_TIMED_LAUNCH(s, "grouped_gemm_fp8_mx<false>",
    hipLaunchKernelGGL(grouped_gemm_fp8_mx<false>, dim3(xcd_grid(mt * a2.ntn)), dim3(NT), kLds, s,
                       a2));
  return hipGetLastError();
}

}  // namespace moe
