// FP8 backward of the grouped SwiGLU expert FFN (training), e4m3 MFMA with
// row-major e4m3 weights and fp32 accumulation (gfx950).
//
// FP8 training ("深入理解 DeepSeek-V3：大规模缩放挑战与对 AI 架构硬件的反思（中文精读）",
// section 3.2): activations in 1x128 tiles, weights in 128x128 blocks, fp32
// accumulation.  The page says no more about the backward; its reading here:
// every operand of a backward GEMM that is an activation or a gradient is
// quantised in tiles of 128 along that GEMM's contraction, the weights keep
// their 128x128 blocks (a block is a block in either direction), and the
// forward quantities are recomputed as the FP8 forward computes them.  With
// [g; u] = W13 x, h = silu(g) u, y = W2 h and the row gradients dy:
//   GU    [g u] = Q(x_rows) W13^T     rows x 2n, k = H    (recompute, fp32 out)
//   DH    dh    = Q(dy) W2            rows x n,  k = H    (epilogue: dg, du, h)
//   DX    dx    = Q([dg du]) W13      rows x H,  k = 2n   (bf16 out)
//   DW2   dW2   = Qc(dy)^T Qc(h)      H x n,     k = the expert's rows
//   DW13  dW13  = Qc([dg du])^T Qc(x) 2n x H,    k = the expert's rows
// Q quantises rows in 1x128 tiles, Qc columns in tiles of 128 of the
// expert's rows (the last tile shorter); the scale rule is the forward's
// (a / 448, or a power of two for MOE_FP8_E4M3_E8M0 weights).
//
// One GEMM kernel serves all five: C[m][n] = sum over 128-k blocks of
// sa[m][kb] sb[n][kb] (A[m][kb] . B[n][kb]), A with k contiguous, B with k
// contiguous (NK) or n contiguous (KN: the weight used along its rows, as W2
// in DH and W13 in DX, transposed 4 x 4 bytes at a time in registers on its
// way into LDS).  The weight gradients contract over an expert's rows, so
// their operands are written once, quantised and transposed, into columns
// [128 f_g, 128 (f_g + t_g)) of [feature][padded rows] arrays, where f_g is
// the first of the expert's t_g row tiles (zero-filled past its rows).
// Tiles are 128 x 128 with 128-k steps (one scale block): 8 waves of 32 x
// 64, two e4m3 MFMAs (32 x 32 x 64, unit E8M0 scales) per 32 x 32 block and
// step into a partial that is scaled and added to the fp32 accumulator.
#include "moe_internal.hpp"
#include "fp8_device.hpp"

#include <algorithm>

namespace moe {

namespace {

constexpr int QB = 128;     // tile rows / columns / k per step
constexpr int QT = 512;     // threads of the GEMM (8 waves)

enum : int { M_GU = 0, M_DH = 1, M_DX = 2, M_WG = 3 };
enum : int { SB_ROW = 0, SB_BLK_NK = 1, SB_BLK_KN = 2 };

// Per segment (0: routed experts, 1: the shared expert).
struct B8Args {
  const int32_t* tiles;     // dgrad: row-tile list (group, first row, rows, ...)
  const int32_t* gfirst;    // wgrad: first row tile of each group, [E + 2]
  int ntn;                  // N tiles per M tile (dgrad) / per group (wgrad: mtn x ntn)
  int mtn;
  int E, K;
  int N[2], Kd[2], M[2];
  const uint8_t* a[2];
  int64_t lda[2];
  const float* as[2];
  int64_t ldas[2];
  const int32_t* perm;      // GU: routed A row = x row perm[r] / K
  const uint8_t* b[2];
  int64_t ldb[2];
  int64_t bstride;          // routed weight per expert (dgrad)
  const float* bs[2];
  int64_t ldbs[2];
  int64_t bsstride;
  void* c[2];
  int64_t ldc[2];
  int64_t cstride;          // routed weight gradient per expert (wgrad)
  const float* gu[2];       // DH epilogue: [g u] rows, [dg du] rows, h rows
  int64_t ldgu[2];
  float* da[2];
  float* h[2];
  int ne[2];
};

// E8M0 exponent of a power-of-two fp32 scale (both have exponent bias 127).
__device__ __forceinline__ int e8m0_bits(float s) { return (int)(__float_as_uint(s) >> 23) & 0xFF; }

// kP2: power-of-two scales, applied by the scaled MFMA itself (each lane
// passes the scale of its own A row / B row or block), so the k loop
// accumulates in the matrix cores with no per-block vector work.
template <int kMode, bool kKN, int kSB, bool kP2>
__global__ void __launch_bounds__(QT) bwd8_gemm(B8Args p) {
  __shared__ uint4 sA[2][QB * 8];
  __shared__ uint4 sB[2][QB * 8];
  __shared__ float sAs[2][QB];
  __shared__ float sBs[2][QB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lh = lane >> 5;
  const int wm = wave & 3, wn = wave >> 2;     // A rows 32 wm .., B rows 64 wn ..
  // per-segment fields by selection (an indexed kernel argument would be
  // copied to scratch memory)
#define SEG(f) (seg ? p.f[1] : p.f[0])

  // ---- the tile: segment, A rows, N columns, k range
  int seg, g, row0, nrows, n0, kb0, nsteps;
  if (kMode != M_WG) {
    const int j = blockIdx.x / p.ntn;
    if (j >= p.tiles[0]) return;
    const int32_t* ent = p.tiles + 8 + 8 * j;
    g = ent[0];
    row0 = ent[1];
    nrows = ent[2];
    seg = g == p.E ? 1 : 0;
    n0 = (blockIdx.x % p.ntn) * QB;
    if (n0 >= SEG(N)) return;
    kb0 = 0;
    nsteps = SEG(Kd) / QB;
  } else {
    g = blockIdx.y;
    seg = g == p.E ? 1 : 0;
    const int mt = blockIdx.x / p.ntn;
    n0 = (blockIdx.x % p.ntn) * QB;
    row0 = mt * QB;
    if (row0 >= SEG(M) || n0 >= SEG(N)) return;
    nrows = QB;
    kb0 = p.gfirst[g];
    nsteps = p.gfirst[g + 1] - kb0;
  }
  const uint8_t* A = SEG(a);
  const float* As = SEG(as);
  const uint8_t* B = SEG(b) + (kMode != M_WG && seg == 0 ? (int64_t)g * p.bstride : 0);
  const float* Bs = SEG(bs) + (kMode != M_WG && seg == 0 ? (int64_t)g * p.bsstride : 0);

  // ---- load assignment: A (and NK B) rows r = tid / 8 + 64 j, 16-byte
  // chunk tid % 8; KN B: k rows 4 (tid % 32) .. + 4, n bytes 8 (tid / 32)
  // .. + 8
  const int ch = tid & 7;
  auto arow_ptr = [&](int r) -> const uint8_t* {
    if (r >= nrows) return nullptr;
    int64_t row = row0 + r;
    if (kMode == M_GU && seg == 0) row = p.perm[row0 + r] / p.K;
    return A + row * SEG(lda) + ch * 16;
  };
  const uint8_t* const aptr[2] = {arow_ptr(tid >> 3), arow_ptr((tid >> 3) + 64)};
  const float* sptr = nullptr;             // A scale row this thread stages
  if (tid < nrows) {
    int64_t row = row0 + tid;
    if (kMode == M_GU && seg == 0) row = p.perm[row0 + tid] / p.K;
    sptr = As + row * SEG(ldas) + kb0;
  }
  const int kq = tid & 31, nq = tid >> 5;

  // staged loads of the next step (named, not arrays: the compiler would
  // keep small arrays reached from these lambdas in scratch memory)
  uint4 ra0, ra1, rb0, rb1;
  uint2 rk0, rk1, rk2, rk3;
  float ras = 0.0f, rbs = 0.0f;
  const int nrow0 = n0 + (tid >> 3), nrow1 = nrow0 + 64;
  auto gload = [&](int step) {
    const int64_t kbyte = (int64_t)(kb0 + step) * QB;
    ra0 = aptr[0] ? *reinterpret_cast<const uint4*>(aptr[0] + kbyte) : make_uint4(0, 0, 0, 0);
    ra1 = aptr[1] ? *reinterpret_cast<const uint4*>(aptr[1] + kbyte) : make_uint4(0, 0, 0, 0);
    if (kKN) {
      const uint8_t* bk = B + (kbyte + 4 * kq) * SEG(ldb) + n0 + 8 * nq;
      const int64_t ldb = SEG(ldb);
      rk0 = *reinterpret_cast<const uint2*>(bk);
      rk1 = *reinterpret_cast<const uint2*>(bk + ldb);
      rk2 = *reinterpret_cast<const uint2*>(bk + 2 * ldb);
      rk3 = *reinterpret_cast<const uint2*>(bk + 3 * ldb);
    } else {
      rb0 = *reinterpret_cast<const uint4*>(B + (int64_t)nrow0 * SEG(ldb) + kbyte + ch * 16);
      rb1 = *reinterpret_cast<const uint4*>(B + (int64_t)nrow1 * SEG(ldb) + kbyte + ch * 16);
    }
    ras = sptr ? sptr[step] : 0.0f;
    if (kSB == SB_ROW && tid >= QB && tid < 2 * QB)
      rbs = Bs[(int64_t)(n0 + tid - QB) * SEG(ldbs) + kb0 + step];
  };
  const int ar0 = tid >> 3, ar1 = ar0 + 64;
  auto sstore = [&](int buf) {
    sA[buf][ar0 * 8 + (ch ^ (ar0 & 7))] = ra0;
    sA[buf][ar1 * 8 + (ch ^ (ar1 & 7))] = ra1;
    if (kKN) {
      // k rows 4kq .. 4kq + 3 of 8 n bytes -> 8 n rows of 4 k bytes
      uint32_t* s32 = reinterpret_cast<uint32_t*>(sB[buf]);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int sh = 8 * (c & 3);
        const uint32_t w0 = c < 4 ? rk0.x : rk0.y, w1 = c < 4 ? rk1.x : rk1.y;
        const uint32_t w2 = c < 4 ? rk2.x : rk2.y, w3 = c < 4 ? rk3.x : rk3.y;
        const uint32_t v = ((w0 >> sh) & 0xFFu) | (((w1 >> sh) & 0xFFu) << 8) |
                           (((w2 >> sh) & 0xFFu) << 16) | (((w3 >> sh) & 0xFFu) << 24);
        const int n = 8 * nq + c;
        s32[n * 32 + 4 * ((kq >> 2) ^ (n & 7)) + (kq & 3)] = v;
      }
    } else {
      sB[buf][ar0 * 8 + (ch ^ (ar0 & 7))] = rb0;
      sB[buf][ar1 * 8 + (ch ^ (ar1 & 7))] = rb1;
    }
    if (tid < QB) sAs[buf][tid] = ras;
    if (kSB == SB_ROW && tid >= QB && tid < 2 * QB) sBs[buf][tid - QB] = rbs;
  };

  f32x16 acc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;

  if (nsteps > 0) {
    gload(0);
    sstore(0);
    if (nsteps > 1) gload(1);
  }
  __syncthreads();
  const int ar = 32 * wm + lr;
  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    float bsc = 1.0f;
    if (kSB == SB_BLK_NK)
      bsc = Bs[(int64_t)(n0 / QB) * (SEG(Kd) / QB) + kb0 + step];
    else if (kSB == SB_BLK_KN)
      bsc = Bs[(int64_t)(kb0 + step) * (SEG(N) / QB) + n0 / QB];
    if (kP2) {
      const int ea = e8m0_bits(sAs[buf][ar]);
      int eb[2];
#pragma unroll
      for (int j = 0; j < 2; ++j)
        eb[j] = e8m0_bits(kSB == SB_ROW ? sBs[buf][64 * wn + 32 * j + lr] : bsc);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int c = 4 * s + 2 * lh;
        const i32x8 af =
            as_i32x8(sA[buf][ar * 8 + (c ^ (ar & 7))], sA[buf][ar * 8 + ((c + 1) ^ (ar & 7))]);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int br = 64 * wn + 32 * j + lr;
          const i32x8 bf = as_i32x8(sB[buf][br * 8 + (c ^ (br & 7))],
                                    sB[buf][br * 8 + ((c + 1) ^ (br & 7))]);
          acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf, acc[j], 0, 0, 0, ea,
                                                                  0, eb[j]);
        }
      }
    } else {
      f32x16 part[2];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) part[j][e] = 0.0f;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int c = 4 * s + 2 * lh;
        const i32x8 af =
            as_i32x8(sA[buf][ar * 8 + (c ^ (ar & 7))], sA[buf][ar * 8 + ((c + 1) ^ (ar & 7))]);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int br = 64 * wn + 32 * j + lr;
          const i32x8 bf = as_i32x8(sB[buf][br * 8 + (c ^ (br & 7))],
                                    sB[buf][br * 8 + ((c + 1) ^ (br & 7))]);
          part[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf, part[j], 0, 0, 0,
                                                                   127, 0, 127);
        }
      }
      // C row 8 (e / 4) + 4 lh + e % 4 of the A block, column lr of the B block
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float sb = kSB == SB_ROW ? sBs[buf][64 * wn + 32 * j + lr] : bsc;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float sa = sAs[buf][32 * wm + 8 * (e >> 2) + 4 * lh + (e & 3)];
          acc[j][e] = fmaf(part[j][e], sa * sb, acc[j][e]);
        }
      }
    }
    if (step + 1 < nsteps) {
      sstore((step + 1) & 1);
      if (step + 2 < nsteps) gload(step + 2);
    }
    __syncthreads();
  }

  // ---- epilogue
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = 32 * wm + 8 * (e >> 2) + 4 * lh + (e & 3);
      const int n = n0 + 64 * wn + 32 * j + lr;
      if (m >= nrows) continue;
      const int64_t row = row0 + m;
      const float v = acc[j][e];
      if (kMode == M_GU) {
        static_cast<float*>(SEG(c))[row * SEG(ldc) + n] = v;
      } else if (kMode == M_DH) {
        // dh -> dg = dh u silu'(g), du = dh silu(g), h = silu(g) u
        const int ne = SEG(ne);
        const float* gu = SEG(gu) + row * SEG(ldgu);
        const float gv = gu[n], uv = gu[ne + n];
        const float sg = 1.0f / (1.0f + __expf(-gv));
        float* da = SEG(da) + row * SEG(ldgu);
        da[n] = v * uv * sg * (1.0f + gv * (1.0f - sg));
        da[ne + n] = v * gv * sg;
        SEG(h)[row * ne + n] = gv * sg * uv;
      } else {
        uint16_t* c = static_cast<uint16_t*>(SEG(c)) +
                      (kMode == M_WG && seg == 0 ? (int64_t)g * p.cstride : 0);
        c[row * SEG(ldc) + n] = (uint16_t)f32_to_bf16_bits(v);
      }
    }
}
#undef SEG

// 1x128 row quantiser of a [rows, cols] bf16 or fp32 matrix (row stride
// ld), as the forward's: one 128-wide tile per 16 lanes.
template <typename TIn, bool kPow2>
__global__ void __launch_bounds__(256)
q8_rows_kernel(const TIn* __restrict__ x, int64_t ld, int64_t rows, int cols,
               uint8_t* __restrict__ q, float* __restrict__ sc) {
  const int tpr = cols / 128;
  const int64_t tile = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  const bool ok = tile < rows * tpr;
  const int64_t r = ok ? tile / tpr : 0;
  const int c = ok ? (int)(tile % tpr) * 128 + sub * 8 : 0;
  float v[8];
  float m = 0.0f;
  if (ok) {
    if (sizeof(TIn) == 2) {
      const uint4 pv = *reinterpret_cast<const uint4*>(x + r * ld + c);
      const uint32_t u[4] = {pv.x, pv.y, pv.z, pv.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = bf16_bits_to_f32(u[j] & 0xFFFFu);
        v[2 * j + 1] = bf16_bits_to_f32(u[j] >> 16);
      }
    } else {
      const float4 a = *reinterpret_cast<const float4*>(x + r * ld + c);
      const float4 b = *reinterpret_cast<const float4*>(x + r * ld + c + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
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
  if (sub == 0) sc[r * tpr + c / 128] = scale;
}

// Column quantiser of the weight-gradient operands: row tile j of the list
// (group g, rows r0 .. r0 + n, n <= 128) x 64 features.  Each feature's
// 128 values (zero past n) get one scale; the codes go to
// out[f][128 j .. 128 j + 128) and the scale to outs[f * ldt + j].  Rows of
// the shared expert (group E) come from the second source.  kX: the source
// is x, read at token perm[r] / K (routed) or r (shared).
struct ColArgs {
  const int32_t* tiles;
  int E, K;
  const void* src[2];
  int64_t ld[2];
  int F[2];
  const int32_t* perm;
  uint8_t* out;
  int64_t ldo;             // bytes per feature row of out
  float* outs;
  int64_t ldt;             // scales per feature row
};

template <typename TIn, bool kX, bool kPow2>
__global__ void __launch_bounds__(256) q8_cols_kernel(ColArgs p) {
  __shared__ float s[QB][65];
  const int j = blockIdx.x;
  if (j >= p.tiles[0]) return;
  const int32_t* ent = p.tiles + 8 + 8 * j;
  const int g = ent[0], r0 = ent[1], n = ent[2];
  const int seg = g == p.E ? 1 : 0;
  const int f0 = blockIdx.y * 64;
  if (f0 >= (seg ? p.F[1] : p.F[0])) return;
  const TIn* src = static_cast<const TIn*>(seg ? p.src[1] : p.src[0]);
  const int64_t ld = seg ? p.ld[1] : p.ld[0];
  const int tid = threadIdx.x;
  // load 128 rows x 64 features: thread -> row tid / 2 .. in passes, 32 features
  for (int e = tid; e < QB * 64; e += 256) {
    const int r = e >> 6, f = e & 63;
    float v = 0.0f;
    if (r < n) {
      int64_t row = r0 + r;
      if (kX && seg == 0) row = p.perm[row] / p.K;
      const TIn raw = src[row * ld + f0 + f];
      if (sizeof(TIn) == 2)
        v = bf16_bits_to_f32((uint32_t)(uint16_t)raw);
      else
        v = (float)raw;
    }
    s[r][f] = v;
  }
  __syncthreads();
  // 4 threads per feature, 32 rows each
  const int f = tid >> 2, part = tid & 3;
  float m = 0.0f;
  for (int r = 32 * part; r < 32 * part + 32; ++r) m = fmaxf(m, fabsf(s[r][f]));
  m = fmaxf(m, __shfl_xor(m, 1, 64));
  m = fmaxf(m, __shfl_xor(m, 2, 64));
  float scale, inv;
  if (kPow2)
    tile_scale_pow2(m, scale, inv);
  else
    tile_scale(m, scale, inv);
  uint32_t w[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    uint32_t v = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) v |= f32_to_e4m3(s[32 * part + 4 * d + b][f] * inv) << (8 * b);
    w[d] = v;
  }
  uint8_t* o = p.out + (int64_t)(f0 + f) * p.ldo + (int64_t)j * QB + 32 * part;
  *reinterpret_cast<uint4*>(o) = make_uint4(w[0], w[1], w[2], w[3]);
  *reinterpret_cast<uint4*>(o + 16) = make_uint4(w[4], w[5], w[6], w[7]);
  if (part == 0) p.outs[(int64_t)(f0 + f) * p.ldt + j] = scale;
}

// First row tile of each group (routed experts, then the shared expert):
// gfirst[g] = sum over groups before g of ceil(rows / 128); gfirst[E + 1]
// is the total.
__global__ void __launch_bounds__(1024)
group_first_kernel(const int32_t* __restrict__ offsets, int E, int64_t T, int has_shared,
                   int32_t* __restrict__ gfirst) {
  __shared__ int32_t s[1024];
  const int g = threadIdx.x;
  int32_t n = 0;
  if (g < E) n = offsets[g + 1] - offsets[g];
  else if (g == E && has_shared) n = (int32_t)T;
  const int32_t mt = (n + QB - 1) / QB;
  s[g] = mt;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t v = g >= off ? s[g - off] : 0;
    __syncthreads();
    s[g] += v;
    __syncthreads();
  }
  if (g <= E) gfirst[g] = s[g] - mt;
  if (g == E) gfirst[E + 1] = s[g];
}

// Workspace plan.
struct Ws8 {
  size_t tiles, gfirst, xq, xs, gu_r, gu_s, dyq_r, dys_r, dyq_s, dys_s, da_r, da_s, h_r, h_s,
      daq_r, das_r, daq_s, das_s, dyT, dyTs, hT, hTs, daT, daTs, xT, xTs, total;
  int64_t maxt, kp;
};

Ws8 plan8(const FfnDims& d) {
  Ws8 w{};
  size_t o = 0;
  auto take = [&](size_t b) {
    size_t at = o;
    o += (b + 255) / 256 * 256;
    return at;
  };
  const int64_t N = d.N, T = d.T, H = d.H, I = d.I, Is = d.Is;
  const bool sh = Is > 0;
  w.maxt = ffn_max_mtiles(N, sh ? T : 0, d.E, QB);
  w.kp = w.maxt * QB;
  const int64_t Imax = std::max(I, Is);
  w.tiles = take((size_t)(w.maxt + 1) * 8 * 4);
  w.gfirst = take((size_t)(d.E + 2) * 4);
  w.xq = take((size_t)T * H);
  w.xs = take((size_t)T * (H / 128) * 4);
  w.gu_r = take((size_t)N * 2 * I * 4);
  w.gu_s = take((size_t)T * 2 * Is * 4);
  w.dyq_r = take((size_t)N * H);
  w.dys_r = take((size_t)N * (H / 128) * 4);
  w.dyq_s = take((size_t)T * H);
  w.dys_s = take((size_t)T * (H / 128) * 4);
  w.da_r = take((size_t)N * 2 * I * 4);
  w.da_s = take((size_t)T * 2 * Is * 4);
  w.h_r = take((size_t)N * I * 4);
  w.h_s = take((size_t)T * Is * 4);
  w.daq_r = take((size_t)N * 2 * I);
  w.das_r = take((size_t)N * (2 * I / 128) * 4);
  w.daq_s = take((size_t)T * 2 * Is);
  w.das_s = take((size_t)T * (2 * Is / 128) * 4);
  w.dyT = take((size_t)H * w.kp);
  w.dyTs = take((size_t)H * w.maxt * 4);
  w.hT = take((size_t)Imax * w.kp);
  w.hTs = take((size_t)Imax * w.maxt * 4);
  w.daT = take((size_t)2 * Imax * w.kp);
  w.daTs = take((size_t)2 * Imax * w.maxt * 4);
  w.xT = take((size_t)H * w.kp);
  w.xTs = take((size_t)H * w.maxt * 4);
  w.total = o;
  return w;
}

template <typename T>
T* at8(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

template <typename TIn>
hipError_t q8_rows(const TIn* x, int64_t ld, int64_t rows, int cols, uint8_t* q, float* sc,
                   bool pow2, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int64_t tiles = rows * (cols / 128);
  const dim3 grid((unsigned)((tiles + 15) / 16));
  if (pow2)
    MOE_TIMED_LAUNCH(s, "q8_rows_kernel",
      hipLaunchKernelGGL((q8_rows_kernel<TIn, true>), grid, dim3(256), 0, s, x, ld, rows, cols,
                         q, sc));
  else
    MOE_TIMED_LAUNCH(s, "q8_rows_kernel",
      hipLaunchKernelGGL((q8_rows_kernel<TIn, false>), grid, dim3(256), 0, s, x, ld, rows, cols,
                         q, sc));
  return hipGetLastError();
}

template <typename TIn, bool kX>
hipError_t q8_cols(const ColArgs& a, int64_t maxt, int fmax, bool pow2, hipStream_t s) {
  const dim3 grid((unsigned)maxt, (unsigned)((fmax + 63) / 64));
  if (pow2)
    MOE_TIMED_LAUNCH(s, "q8_cols_kernel",
      hipLaunchKernelGGL((q8_cols_kernel<TIn, kX, true>), grid, dim3(256), 0, s, a));
  else
    MOE_TIMED_LAUNCH(s, "q8_cols_kernel",
      hipLaunchKernelGGL((q8_cols_kernel<TIn, kX, false>), grid, dim3(256), 0, s, a));
  return hipGetLastError();
}

template <int kMode, bool kKN, int kSB>
hipError_t gemm8(const B8Args& a, dim3 grid, const char* name, bool pow2, hipStream_t s) {
  if (pow2)
    MOE_TIMED_LAUNCH(s, name,
      hipLaunchKernelGGL((bwd8_gemm<kMode, kKN, kSB, true>), grid, dim3(QT), 0, s, a));
  else
    MOE_TIMED_LAUNCH(s, name,
      hipLaunchKernelGGL((bwd8_gemm<kMode, kKN, kSB, false>), grid, dim3(QT), 0, s, a));
  return hipGetLastError();
}

#define B8CALL(x)                        \
  do {                                   \
    hipError_t e_ = (x);                 \
    if (e_ != hipSuccess) return e_;     \
  } while (0)

}  // namespace

size_t ffn_backward_fp8_ws_bytes(const FfnDims& d) { return plan8(d).total; }

hipError_t launch_ffn_backward_fp8(const FfnDims& d, bool pow2, const uint16_t* x,
                                   const int32_t* perm, const int32_t* offsets,
                                   const uint8_t* w13, const float* w13s, const uint8_t* w2,
                                   const float* w2s, const uint8_t* ws13, const float* ws13s,
                                   const uint8_t* ws2, const float* ws2s, const uint16_t* dy,
                                   const uint16_t* dys, uint16_t* dx, uint16_t* dxs,
                                   uint16_t* dw13, uint16_t* dw2, uint16_t* dws13,
                                   uint16_t* dws2, void* ws, hipStream_t s) {
  const Ws8 L = plan8(d);
  const int64_t N = d.N, T = d.T;
  const int H = d.H, I = d.I, Is = d.Is, E = d.E;
  const bool sh = Is > 0;
  int32_t* tiles = at8<int32_t>(ws, L.tiles);
  int32_t* gfirst = at8<int32_t>(ws, L.gfirst);
  B8CALL(launch_build_tiles(offsets, E, T, true, sh, QB, tiles, s, false));
  MOE_TIMED_LAUNCH(s, "group_first_kernel",
    hipLaunchKernelGGL(group_first_kernel, dim3(1), dim3(1024), 0, s, offsets, E, T, sh ? 1 : 0,
                       gfirst));
  B8CALL(hipGetLastError());

  uint8_t* xq = at8<uint8_t>(ws, L.xq);
  float* xsc = at8<float>(ws, L.xs);
  float* gu_r = at8<float>(ws, L.gu_r);
  float* gu_s = at8<float>(ws, L.gu_s);
  float* da_r = at8<float>(ws, L.da_r);
  float* da_s = at8<float>(ws, L.da_s);
  float* h_r = at8<float>(ws, L.h_r);
  float* h_s = at8<float>(ws, L.h_s);
  uint8_t *dyq_r = at8<uint8_t>(ws, L.dyq_r), *dyq_s = at8<uint8_t>(ws, L.dyq_s);
  float *dys_r = at8<float>(ws, L.dys_r), *dys_s = at8<float>(ws, L.dys_s);
  uint8_t *daq_r = at8<uint8_t>(ws, L.daq_r), *daq_s = at8<uint8_t>(ws, L.daq_s);
  float *das_r = at8<float>(ws, L.das_r), *das_s = at8<float>(ws, L.das_s);
  const int64_t maxt = L.maxt;
  const int ntn_d = (std::max(2 * I, std::max(2 * Is, H)) + QB - 1) / QB;

  // x rows, quantised per 1x128 tile (the F2 forward's x)
  B8CALL(q8_rows<uint16_t>(x, H, T, H, xq, xsc, pow2, s));

  // GU: [g u] = Q(x_rows) W13^T
  B8Args a{};
  a.tiles = tiles;
  a.gfirst = gfirst;
  a.E = E;
  a.K = d.K;
  a.perm = perm;
  a.ntn = ntn_d;
  a.N[0] = 2 * I;
  a.N[1] = 2 * Is;
  a.Kd[0] = a.Kd[1] = H;
  a.a[0] = a.a[1] = xq;
  a.lda[0] = a.lda[1] = H;
  a.as[0] = a.as[1] = xsc;
  a.ldas[0] = a.ldas[1] = H / 128;
  a.b[0] = w13;
  a.b[1] = ws13;
  a.ldb[0] = a.ldb[1] = H;
  a.bstride = (int64_t)2 * I * H;
  a.bs[0] = w13s;
  a.bs[1] = ws13s;
  a.bsstride = (int64_t)(2 * I / 128) * (H / 128);
  a.c[0] = gu_r;
  a.c[1] = gu_s;
  a.ldc[0] = 2 * I;
  a.ldc[1] = 2 * Is;
  const dim3 grid_d((unsigned)(maxt * ntn_d));
  B8CALL((gemm8<M_GU, false, SB_BLK_NK>(a, grid_d, "bwd8_gemm<gu>", pow2, s)));

  // dy rows quantised per 1x128 tile along H
  B8CALL(q8_rows<uint16_t>(dy, H, N, H, dyq_r, dys_r, pow2, s));
  if (sh) B8CALL(q8_rows<uint16_t>(dys, H, T, H, dyq_s, dys_s, pow2, s));

  // DH: dh = Q(dy) W2, epilogue dg, du, h
  B8Args b{};
  b.tiles = tiles;
  b.E = E;
  b.K = d.K;
  b.ntn = ntn_d;
  b.N[0] = I;
  b.N[1] = Is;
  b.Kd[0] = b.Kd[1] = H;
  b.a[0] = dyq_r;
  b.a[1] = dyq_s;
  b.lda[0] = b.lda[1] = H;
  b.as[0] = dys_r;
  b.as[1] = dys_s;
  b.ldas[0] = b.ldas[1] = H / 128;
  b.b[0] = w2;
  b.b[1] = ws2;
  b.ldb[0] = I;
  b.ldb[1] = Is;
  b.bstride = (int64_t)H * I;
  b.bs[0] = w2s;
  b.bs[1] = ws2s;
  b.bsstride = (int64_t)(H / 128) * (I / 128);
  b.gu[0] = gu_r;
  b.gu[1] = gu_s;
  b.ldgu[0] = 2 * I;
  b.ldgu[1] = 2 * Is;
  b.da[0] = da_r;
  b.da[1] = da_s;
  b.h[0] = h_r;
  b.h[1] = h_s;
  b.ne[0] = I;
  b.ne[1] = Is;
  B8CALL((gemm8<M_DH, true, SB_BLK_KN>(b, grid_d, "bwd8_gemm<dh>", pow2, s)));

  // [dg du] rows quantised per 1x128 tile along 2n
  B8CALL(q8_rows<float>(da_r, 2 * I, N, 2 * I, daq_r, das_r, pow2, s));
  if (sh) B8CALL(q8_rows<float>(da_s, 2 * Is, T, 2 * Is, daq_s, das_s, pow2, s));

  // DX: dx = Q([dg du]) W13
  if (dx) {
    B8Args c{};
    c.tiles = tiles;
    c.E = E;
    c.K = d.K;
    c.ntn = ntn_d;
    c.N[0] = c.N[1] = H;
    c.Kd[0] = 2 * I;
    c.Kd[1] = 2 * Is;
    c.a[0] = daq_r;
    c.a[1] = daq_s;
    c.lda[0] = 2 * I;
    c.lda[1] = 2 * Is;
    c.as[0] = das_r;
    c.as[1] = das_s;
    c.ldas[0] = 2 * I / 128;
    c.ldas[1] = 2 * Is / 128;
    c.b[0] = w13;
    c.b[1] = ws13;
    c.ldb[0] = c.ldb[1] = H;
    c.bstride = (int64_t)2 * I * H;
    c.bs[0] = w13s;
    c.bs[1] = ws13s;
    c.bsstride = (int64_t)(2 * I / 128) * (H / 128);
    c.c[0] = dx;
    c.c[1] = dxs;
    c.ldc[0] = c.ldc[1] = H;
    B8CALL((gemm8<M_DX, true, SB_BLK_KN>(c, grid_d, "bwd8_gemm<dx>", pow2, s)));
  }

  // the weight-gradient operands, quantised per column in row tiles and
  // transposed
  uint8_t* dyT = at8<uint8_t>(ws, L.dyT);
  uint8_t* hT = at8<uint8_t>(ws, L.hT);
  uint8_t* daT = at8<uint8_t>(ws, L.daT);
  uint8_t* xT = at8<uint8_t>(ws, L.xT);
  float* dyTs = at8<float>(ws, L.dyTs);
  float* hTs = at8<float>(ws, L.hTs);
  float* daTs = at8<float>(ws, L.daTs);
  float* xTs = at8<float>(ws, L.xTs);
  ColArgs q{};
  q.tiles = tiles;
  q.E = E;
  q.K = d.K;
  q.perm = perm;
  q.ldo = L.kp;
  q.ldt = maxt;
  q.src[0] = dy;
  q.src[1] = dys;
  q.ld[0] = q.ld[1] = H;
  q.F[0] = H;
  q.F[1] = sh ? H : 0;
  q.out = dyT;
  q.outs = dyTs;
  B8CALL((q8_cols<uint16_t, false>(q, maxt, H, pow2, s)));
  q.src[0] = h_r;
  q.src[1] = h_s;
  q.ld[0] = I;
  q.ld[1] = Is;
  q.F[0] = I;
  q.F[1] = Is;
  q.out = hT;
  q.outs = hTs;
  B8CALL((q8_cols<float, false>(q, maxt, std::max(I, Is), pow2, s)));
  q.src[0] = da_r;
  q.src[1] = da_s;
  q.ld[0] = 2 * I;
  q.ld[1] = 2 * Is;
  q.F[0] = 2 * I;
  q.F[1] = 2 * Is;
  q.out = daT;
  q.outs = daTs;
  B8CALL((q8_cols<float, false>(q, maxt, 2 * std::max(I, Is), pow2, s)));
  q.src[0] = q.src[1] = x;
  q.ld[0] = q.ld[1] = H;
  q.F[0] = H;
  q.F[1] = sh ? H : 0;
  q.out = xT;
  q.outs = xTs;
  B8CALL((q8_cols<uint16_t, true>(q, maxt, H, pow2, s)));

  // DW2 = Qc(dy)^T Qc(h): M = H, N = n, k = the expert's row tiles
  B8Args w{};
  w.gfirst = gfirst;
  w.E = E;
  w.M[0] = w.M[1] = H;
  w.N[0] = I;
  w.N[1] = Is;
  w.ntn = (std::max(I, Is) + QB - 1) / QB;
  w.a[0] = w.a[1] = dyT;
  w.lda[0] = w.lda[1] = L.kp;
  w.as[0] = w.as[1] = dyTs;
  w.ldas[0] = w.ldas[1] = maxt;
  w.b[0] = w.b[1] = hT;
  w.ldb[0] = w.ldb[1] = L.kp;
  w.bs[0] = w.bs[1] = hTs;
  w.ldbs[0] = w.ldbs[1] = maxt;
  w.c[0] = dw2;
  w.c[1] = dws2;
  w.ldc[0] = I;
  w.ldc[1] = Is;
  w.cstride = (int64_t)H * I;
  const dim3 grid_w2((unsigned)((H / QB) * w.ntn), (unsigned)(E + (sh ? 1 : 0)));
  B8CALL((gemm8<M_WG, false, SB_ROW>(w, grid_w2, "bwd8_gemm<dw2>", pow2, s)));

  // DW13 = Qc([dg du])^T Qc(x): M = 2n, N = H
  B8Args v{};
  v.gfirst = gfirst;
  v.E = E;
  v.M[0] = 2 * I;
  v.M[1] = 2 * Is;
  v.N[0] = v.N[1] = H;
  v.ntn = H / QB;
  v.a[0] = v.a[1] = daT;
  v.lda[0] = v.lda[1] = L.kp;
  v.as[0] = v.as[1] = daTs;
  v.ldas[0] = v.ldas[1] = maxt;
  v.b[0] = v.b[1] = xT;
  v.ldb[0] = v.ldb[1] = L.kp;
  v.bs[0] = v.bs[1] = xTs;
  v.ldbs[0] = v.ldbs[1] = maxt;
  v.c[0] = dw13;
  v.c[1] = dws13;
  v.ldc[0] = v.ldc[1] = H;
  v.cstride = (int64_t)2 * I * H;
  const dim3 grid_w13((unsigned)((2 * std::max(I, Is) / QB) * v.ntn),
                      (unsigned)(E + (sh ? 1 : 0)));
  B8CALL((gemm8<M_WG, false, SB_ROW>(v, grid_w13, "bwd8_gemm<dw13>", pow2, s)));
  return hipSuccess;
}

}  // namespace moe
