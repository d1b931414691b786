// Backward of the grouped SwiGLU expert FFN (training), bf16 MFMA with
// row-major bf16 weights and fp32 accumulation.
//
// The experts are SwiGLU FFNs (mqxn.cn/news/19449, section 3.1): [g; u] =
// W13 x, h = silu(g) u, y = W2 h, 256 routed experts plus one always-active
// shared expert ("从 1024 块 GPU 到 558 万美元：拆解 DeepSeek-V3 的算法-系统协同设计",
// section 2.2).  Given the gradient dy of every expert output row (the
// routed rows in expert-sorted order, then the shared expert's T rows), the
// exact derivatives are
//   dh = dy W2,   dg = dh u silu'(g),   du = dh silu(g),
//   dx_row = [dg du] W13,   dW2 = sum_rows dy^T h,   dW13 = sum_rows [dg du]^T x.
// Five grouped GEMMs compute them, all on one tile routine:
//   GU   [g u] = x_rows W13^T      rows x 2I, k = H    (recompute, fp32 out)
//   DH   dh    = dy W2             rows x I,  k = H    (epilogue: SwiGLU backward)
//   DX   dx    = da W13            rows x H,  k = 2I
//   DW2  dW2   = dy^T h            H x I,     k = the expert's rows
//   DW13 dW13  = da^T x_rows       2I x H,    k = the expert's rows
// The MFMA wants both operands with 8 consecutive k values per lane.  Tiles
// go through LDS in one layout, [row][k] with k contiguous (32 per row, the
// 16-byte chunk c of row r stored at chunk c ^ ((r / 4) % 4), so that 16
// consecutive rows read at one chunk hit 16 different bank groups).  An
// operand whose k runs along memory rows (the weights of DH and DX, both
// operands of the weight gradients) is transposed on its way into LDS: each
// thread loads 8 consecutive elements of one k row and writes them as 8
// 2-byte LDS stores.
#include "moe_internal.hpp"

#include <algorithm>

namespace moe {

namespace {

constexpr int BBM = 128, BBN = 128, BBK = 32, BNT = 256;

enum : int { A_ROWS = 0, A_COLS = 1 };           // A(m,k): row m k-contiguous / k rows m-contiguous
enum : int { B_NK = 0, B_KN = 1 };               // B(k,n): row n k-contiguous / k rows n-contiguous
enum : int { E_GU = 0, E_DH = 1, E_STORE = 2 };  // epilogues

struct BwdArgs {
  // dims [routed, shared]; M of row-tiled GEMMs is the tile's row count
  int M[2], N[2], K[2];
  const uint16_t* a[2];
  int64_t lda[2];
  int64_t astride;          // per routed expert (0: row-space operand)
  const uint16_t* b[2];
  int64_t ldb[2];
  int64_t bstride;
  int a_gather, b_gather;   // routed row j -> token perm[j] / K (x as the operand)
  int b_rows;               // B_KN row index: 1 = the group's row space, 0 = a weight row
  const int32_t* perm;
  int topk;
  void* c[2];
  int64_t ldc[2];
  int64_t cstride;          // per routed expert (weight gradients)
  const float* gu[2];       // E_DH: [g u] rows, fp32
  int64_t ldgu[2];
  uint16_t* da[2];          // E_DH outputs: [dg du] bf16 and h bf16
  int64_t ldda[2];
  uint16_t* h[2];
  int64_t ldh[2];
  const int32_t* tiles;     // row-tiled: tile list and N-tiles per M-tile
  int ntn;
  const int32_t* offsets;   // weight-tiled: rows of each expert
  int E;
  int64_t T;
  int mt, nt;               // weight-tiled: M- and N-tiles per group
};

__device__ __forceinline__ int lds_at(int r, int k) {
  return r * BBK + ((((k >> 3) ^ (r >> 2)) & 3) << 3) + (k & 7);
}

// One 128 x 128 tile of group g (s = 0 routed, 1 shared).  Row-tiled:
// rows row0 + [m0, m0 + Mv) of the row space.  Weight-tiled: rows [m0,
// m0 + 128) of an M x N weight gradient, k over the group's rows row0 + [0, Kv).
template <int AM, int BMD, int EPI, bool WG>
__device__ void bwd_tile(const BwdArgs& p, uint16_t* sA, uint16_t* sB, int g, int s, int64_t row0,
                         int m0, int Mv, int n0, int Nv, int Kv) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lh = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  const uint16_t* A = p.a[s] + (s == 0 ? (int64_t)g * p.astride : 0);
  const uint16_t* B = p.b[s] + (s == 0 ? (int64_t)g * p.bstride : 0);
  const int64_t lda = p.lda[s], ldb = p.ldb[s];

  // row-space row -> the row of the operand (x is read through perm)
  auto xrow = [&](int64_t r, bool gather) -> int64_t {
    return (gather && s == 0) ? (int64_t)(p.perm[r] / p.topk) : r;
  };

  // Per thread and step: two 16-byte chunks of A and two of B.
  u32x4 ra[2], rb[2];
  auto load = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = tid + BNT * j;
      u32x4 v = {0, 0, 0, 0};
      if (AM == A_ROWS) {
        const int m = c >> 2, kc = c & 3;
        if (m < Mv) {
          const int64_t r = xrow(row0 + m0 + m, p.a_gather);
          v = *reinterpret_cast<const u32x4*>(A + r * lda + k0 + kc * 8);
        }
      } else {
        const int k = c >> 4, mc = c & 15;
        if (k0 + k < Kv && m0 + mc * 8 < Mv)
          v = *reinterpret_cast<const u32x4*>(A + (row0 + k0 + k) * lda + m0 + mc * 8);
      }
      ra[j] = v;
      v = (u32x4){0, 0, 0, 0};
      if (BMD == B_NK) {
        const int n = c >> 2, kc = c & 3;
        if (n0 + n < Nv) v = *reinterpret_cast<const u32x4*>(B + (int64_t)(n0 + n) * ldb + k0 + kc * 8);
      } else {
        const int k = c >> 4, nc = c & 15;
        if (k0 + k < Kv && n0 + nc * 8 < Nv) {
          const int64_t r = p.b_rows ? xrow(row0 + k0 + k, p.b_gather) : (int64_t)(k0 + k);
          v = *reinterpret_cast<const u32x4*>(B + r * ldb + n0 + nc * 8);
        }
      }
      rb[j] = v;
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = tid + BNT * j;
      if (AM == A_ROWS) {
        const int m = c >> 2, kc = c & 3;
        *reinterpret_cast<u32x4*>(sA + lds_at(m, kc * 8)) = ra[j];
      } else {
        const int k = c >> 4, mc = c & 15;
        const uint32_t w[4] = {ra[j].x, ra[j].y, ra[j].z, ra[j].w};
#pragma unroll
        for (int i = 0; i < 8; ++i)
          sA[lds_at(mc * 8 + i, k)] = (uint16_t)(w[i >> 1] >> (16 * (i & 1)));
      }
      if (BMD == B_NK) {
        const int n = c >> 2, kc = c & 3;
        *reinterpret_cast<u32x4*>(sB + lds_at(n, kc * 8)) = rb[j];
      } else {
        const int k = c >> 4, nc = c & 15;
        const uint32_t w[4] = {rb[j].x, rb[j].y, rb[j].z, rb[j].w};
#pragma unroll
        for (int i = 0; i < 8; ++i)
          sB[lds_at(nc * 8 + i, k)] = (uint16_t)(w[i >> 1] >> (16 * (i & 1)));
      }
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  const int nsteps = (Kv + BBK - 1) / BBK;
  if (nsteps > 0) {
    load(0);
    store();
    __syncthreads();
  }
  for (int st = 0; st < nsteps; ++st) {
    if (st + 1 < nsteps) load((st + 1) * BBK);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int ar = wm * 64 + i * 32 + lr;
        af[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(sA + lds_at(ar, kk * 16 + lh * 8)));
        const int br = wn * 64 + i * 32 + lr;
        bfr[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(sB + lds_at(br, kk * 16 + lh * 8)));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
    if (st + 1 < nsteps) {
      store();
      __syncthreads();
    }
  }

  // Epilogue: lane holds column lr of each 32 x 32 block, rows
  // 8 (q / 4) + 4 lh + q % 4.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int m = m0 + wm * 64 + i * 32 + 8 * (q >> 2) + 4 * lh + (q & 3);
        const int n = n0 + wn * 64 + j * 32 + lr;
        if (m >= (WG ? Mv : m0 + Mv) || n >= Nv) continue;
        const float v = acc[i][j][q];
        if (WG) {
          uint16_t* C = (uint16_t*)p.c[s] + (s == 0 ? (int64_t)g * p.cstride : 0);
          C[(int64_t)m * p.ldc[s] + n] = (uint16_t)f32_to_bf16_bits(v);
        } else if (EPI == E_GU) {
          float* C = (float*)p.c[s];
          C[(row0 + m) * p.ldc[s] + n] = v;
        } else if (EPI == E_DH) {
          const float* gu = p.gu[s] + (row0 + m) * p.ldgu[s];
          const float gv = gu[n], uv = gu[Nv + n];
          const float sg = 1.0f / (1.0f + __expf(-gv));
          uint16_t* da = p.da[s] + (row0 + m) * p.ldda[s];
          da[n] = (uint16_t)f32_to_bf16_bits(v * uv * sg * (1.0f + gv * (1.0f - sg)));
          da[Nv + n] = (uint16_t)f32_to_bf16_bits(v * gv * sg);
          p.h[s][(row0 + m) * p.ldh[s] + n] = (uint16_t)f32_to_bf16_bits(gv * sg * uv);
        } else {
          uint16_t* C = (uint16_t*)p.c[s];
          C[(row0 + m) * p.ldc[s] + n] = (uint16_t)f32_to_bf16_bits(v);
        }
      }
}

// Row-tiled GEMMs (GU, DH, DX): work item = (M-tile of the tile list, N-tile).
template <int AM, int BMD, int EPI>
__global__ void __launch_bounds__(BNT) bwd_rows_kernel(BwdArgs p) {
  __shared__ uint16_t lds[(BBM + BBN) * BBK];   // 16 KiB: A tile, then B tile
  const int64_t work = (int64_t)p.tiles[0] * p.ntn;
  const int64_t per = (work + kNumXcd - 1) / kNumXcd;
  const int64_t q = blockIdx.x / kNumXcd;
  const int64_t w = (int64_t)(blockIdx.x % kNumXcd) * per + q;
  if (q >= per || w >= work) return;
  int ntile;
  const int32_t* ent = decode_work(p.tiles, w, p.ntn, ntile);
  const int g = ent[0], row0 = ent[1], nrows = ent[2];
  const int s = (g == p.E) ? 1 : 0;
  if (ntile * BBN >= p.N[s]) return;
  bwd_tile<AM, BMD, EPI, false>(p, lds, lds + BBM * BBK, g, s, row0, 0, nrows, ntile * BBN, p.N[s],
                                p.K[s]);
}

// Weight-gradient GEMMs (DW2, DW13): work item = (group, M-tile, N-tile),
// k over the group's rows (an expert without rows gets a zero gradient).
template <int AM, int BMD>
__global__ void __launch_bounds__(BNT) bwd_weights_kernel(BwdArgs p) {
  __shared__ uint16_t lds[(BBM + BBN) * BBK];
  const int64_t per_g = (int64_t)p.mt * p.nt;
  const int64_t groups = p.E + (p.M[1] > 0 ? 1 : 0);
  const int64_t work = groups * per_g;
  const int64_t per = (work + kNumXcd - 1) / kNumXcd;
  const int64_t q = blockIdx.x / kNumXcd;
  const int64_t w = (int64_t)(blockIdx.x % kNumXcd) * per + q;
  if (q >= per || w >= work) return;
  const int g = (int)(w / per_g);
  const int rest = (int)(w % per_g);
  const int mtile = rest / p.nt, ntile = rest % p.nt;
  const int s = (g == p.E) ? 1 : 0;
  if (mtile * BBM >= p.M[s] || ntile * BBN >= p.N[s]) return;
  const int64_t row0 = s ? 0 : p.offsets[g];
  const int rows = s ? (int)p.T : p.offsets[g + 1] - p.offsets[g];
  bwd_tile<AM, BMD, E_STORE, true>(p, lds, lds + BBM * BBK, g, s, row0, mtile * BBM, p.M[s],
                                   ntile * BBN, p.N[s], rows);
}

unsigned grid_for(int64_t work) {
  return (unsigned)(((work + kNumXcd - 1) / kNumXcd) * kNumXcd);
}

}  // namespace

size_t ffn_backward_ws_bytes(const FfnDims& d) {
  const int64_t rows_r = d.N, rows_s = d.Is > 0 ? d.T : 0;
  auto al = [](size_t b) { return (b + 255) / 256 * 256; };
  return al((size_t)(rows_r * 2 * d.I + rows_s * 2 * d.Is) * 4) +      // gu fp32
         al((size_t)(rows_r * 2 * d.I + rows_s * 2 * d.Is) * 2) +      // da bf16
         al((size_t)(rows_r * d.I + rows_s * d.Is) * 2) +              // h bf16
         al(ffn_tiles_bytes(d));
}

hipError_t launch_ffn_backward(const FfnDims& d, const uint16_t* x, const int32_t* perm,
                               const int32_t* offsets, const uint16_t* w13, const uint16_t* w2,
                               const uint16_t* ws13, const uint16_t* ws2, const uint16_t* dy,
                               const uint16_t* dys, uint16_t* dx, uint16_t* dxs, uint16_t* dw13,
                               uint16_t* dw2, uint16_t* dws13, uint16_t* dws2, void* ws,
                               hipStream_t s) {
  const int64_t N = d.N, T = d.T;
  const int H = d.H, I = d.I, Is = d.Is, E = d.E;
  const bool sh = Is > 0;
  auto al = [](size_t b) { return (b + 255) / 256 * 256; };
  char* base = (char*)ws;
  float* gu_r = (float*)base;
  float* gu_s = gu_r + N * 2 * I;
  base += al((size_t)(N * 2 * I + (sh ? T : 0) * 2 * Is) * 4);
  uint16_t* da_r = (uint16_t*)base;
  uint16_t* da_s = da_r + N * 2 * I;
  base += al((size_t)(N * 2 * I + (sh ? T : 0) * 2 * Is) * 2);
  uint16_t* h_r = (uint16_t*)base;
  uint16_t* h_s = h_r + N * I;
  base += al((size_t)(N * I + (sh ? T : 0) * Is) * 2);
  int32_t* tiles = (int32_t*)base;

  hipError_t e = launch_build_tiles(offsets, E, T, true, sh, BBM, tiles, s);
  if (e != hipSuccess) return e;
  const int64_t mt = ffn_max_mtiles(N, T, E, BBM);

  BwdArgs p{};
  p.perm = perm;
  p.topk = d.K;
  p.tiles = tiles;
  p.offsets = offsets;
  p.E = E;
  p.T = T;

  // GU: [g u] = x_rows W13^T (rows x 2I, k = H), fp32.
  {
    BwdArgs q = p;
    q.N[0] = 2 * I; q.N[1] = 2 * Is; q.K[0] = q.K[1] = H;
    q.a[0] = q.a[1] = x; q.lda[0] = q.lda[1] = H; q.a_gather = 1;
    q.b[0] = w13; q.b[1] = ws13; q.ldb[0] = q.ldb[1] = H; q.bstride = (int64_t)2 * I * H;
    q.c[0] = gu_r; q.c[1] = gu_s; q.ldc[0] = 2 * I; q.ldc[1] = 2 * Is;
    q.ntn = (std::max(2 * I, 2 * Is) + BBN - 1) / BBN;
    MOE_TIMED_LAUNCH(s, "bwd_rows_kernel<gu>",
      hipLaunchKernelGGL((bwd_rows_kernel<A_ROWS, B_NK, E_GU>), dim3(grid_for(mt * q.ntn)),
                         dim3(BNT), 0, s, q));
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // DH: dh = dy W2 (rows x I, k = H); epilogue writes [dg du] and h.
  {
    BwdArgs q = p;
    q.N[0] = I; q.N[1] = Is; q.K[0] = q.K[1] = H;
    q.a[0] = dy; q.a[1] = dys; q.lda[0] = q.lda[1] = H;
    q.b[0] = w2; q.b[1] = ws2; q.ldb[0] = I; q.ldb[1] = Is; q.bstride = (int64_t)H * I;
    q.b_rows = 0;
    q.gu[0] = gu_r; q.gu[1] = gu_s; q.ldgu[0] = 2 * I; q.ldgu[1] = 2 * Is;
    q.da[0] = da_r; q.da[1] = da_s; q.ldda[0] = 2 * I; q.ldda[1] = 2 * Is;
    q.h[0] = h_r; q.h[1] = h_s; q.ldh[0] = I; q.ldh[1] = Is;
    q.ntn = (std::max(I, Is) + BBN - 1) / BBN;
    MOE_TIMED_LAUNCH(s, "bwd_rows_kernel<dh>",
      hipLaunchKernelGGL((bwd_rows_kernel<A_ROWS, B_KN, E_DH>), dim3(grid_for(mt * q.ntn)),
                         dim3(BNT), 0, s, q));
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // DX: dx_rows = [dg du] W13 (rows x H, k = 2I).
  if (dx || dxs) {
    BwdArgs q = p;
    q.N[0] = q.N[1] = H; q.K[0] = 2 * I; q.K[1] = 2 * Is;
    q.a[0] = da_r; q.a[1] = da_s; q.lda[0] = 2 * I; q.lda[1] = 2 * Is;
    q.b[0] = w13; q.b[1] = ws13; q.ldb[0] = q.ldb[1] = H; q.bstride = (int64_t)2 * I * H;
    q.b_rows = 0;
    q.c[0] = dx; q.c[1] = dxs; q.ldc[0] = q.ldc[1] = H;
    q.ntn = (H + BBN - 1) / BBN;
    MOE_TIMED_LAUNCH(s, "bwd_rows_kernel<dx>",
      hipLaunchKernelGGL((bwd_rows_kernel<A_ROWS, B_KN, E_STORE>), dim3(grid_for(mt * q.ntn)),
                         dim3(BNT), 0, s, q));
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // DW2: dW2 = dy^T h (H x I, k = the expert's rows).
  {
    BwdArgs q = p;
    q.M[0] = q.M[1] = H; q.N[0] = I; q.N[1] = sh ? Is : 0;
    q.a[0] = dy; q.a[1] = dys; q.lda[0] = q.lda[1] = H; q.astride = 0;
    q.b[0] = h_r; q.b[1] = h_s; q.ldb[0] = I; q.ldb[1] = Is; q.bstride = 0;
    q.b_rows = 1; q.b_gather = 0;
    q.c[0] = dw2; q.c[1] = dws2; q.ldc[0] = I; q.ldc[1] = Is; q.cstride = (int64_t)H * I;
    if (!sh) q.M[1] = 0;
    q.mt = (H + BBM - 1) / BBM;
    q.nt = (std::max(I, Is) + BBN - 1) / BBN;
    const int64_t work = (int64_t)(E + (sh ? 1 : 0)) * q.mt * q.nt;
    MOE_TIMED_LAUNCH(s, "bwd_weights_kernel<dw2>",
      hipLaunchKernelGGL((bwd_weights_kernel<A_COLS, B_KN>), dim3(grid_for(work)), dim3(BNT), 0,
                         s, q));
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // DW13: dW13 = [dg du]^T x_rows (2I x H, k = the expert's rows).
  {
    BwdArgs q = p;
    q.M[0] = 2 * I; q.M[1] = sh ? 2 * Is : 0; q.N[0] = q.N[1] = H;
    q.a[0] = da_r; q.a[1] = da_s; q.lda[0] = 2 * I; q.lda[1] = 2 * Is; q.astride = 0;
    q.b[0] = q.b[1] = x; q.ldb[0] = q.ldb[1] = H; q.bstride = 0;
    q.b_rows = 1; q.b_gather = 1;
    q.c[0] = dw13; q.c[1] = dws13; q.ldc[0] = q.ldc[1] = H; q.cstride = (int64_t)2 * I * H;
    q.mt = (std::max(2 * I, 2 * Is) + BBM - 1) / BBM;
    q.nt = (H + BBN - 1) / BBN;
    const int64_t work = (int64_t)(E + (sh ? 1 : 0)) * q.mt * q.nt;
    MOE_TIMED_LAUNCH(s, "bwd_weights_kernel<dw13>",
      hipLaunchKernelGGL((bwd_weights_kernel<A_COLS, B_KN>), dim3(grid_for(work)), dim3(BNT), 0,
                         s, q));
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace moe
