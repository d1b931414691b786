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
// Five grouped GEMMs compute them:
//   GU   [g u] = x_rows W13^T      rows x 2I, k = H    (recompute, fp32 out)
//   DH   dh    = dy W2             rows x I,  k = H    (epilogue: SwiGLU backward)
//   DX   dx    = da W13            rows x H,  k = 2I
//   DW2  dW2   = dy^T h            H x I,     k = the expert's rows
//   DW13 dW13  = da^T x_rows       2I x H,    k = the expert's rows
// GU is the forward's row-major gate/up GEMM (ffn_bf16.hip) storing g and
// u.  The other four share one tile routine.
//
// The MFMA wants both operands with 8 consecutive k values per lane, so
// tiles go through LDS as [row][k] with k contiguous (64 per row in eight
// XOR-swizzled 16-byte chunks).  In DH
// and DX the weight's k runs along its memory rows: each thread loads 8
// consecutive elements of one k row and writes them as 8 2-byte LDS
// stores.  The weight gradients contract over the expert's rows, which run
// along memory rows in every operand; instead of transposing in LDS, their
// operands are written once in transposed form ([column][row], k
// contiguous): x (gathered through perm) and dy by a transpose kernel, [dg
// du] and h by DH's epilogue.  Each routed expert's rows start at a column
// that is a multiple of 32 (pcol), the gap filled with zeros, so the weight
// gradient GEMMs read whole 16-byte chunks (a last half step of 32 columns
// is zero-filled).  Every row stride of the workspace is an odd multiple of
// 128 bytes.
#include "moe_internal.hpp"
#include "permute_device.hpp"

#include <algorithm>

namespace moe {

namespace {

constexpr int BBM = 128, BBN = 128, BNT = 256;
constexpr int WTM = 256;   // weight-gradient tile rows
constexpr int kPad = 32;   // column alignment of each expert in the transposed operands

enum : int { B_NK = 0, B_KN = 1 };   // B(k,n): row n k-contiguous / k rows n-contiguous
enum : int { E_DH = 1, E_STORE = 2 };

// Epilogue destinations; the tile's row m0 + m and column n0 + n.
struct Epi {
  uint16_t* c;              // E_STORE: C(m, n) at c + m * ldc + n
  int64_t ldc;
  const float* gu;          // E_DH: [g u] rows (fp32), [dg du] rows (bf16), and the
  int64_t ldgu;             // transposed [dg du] and h at column m (zero up to mpad)
  uint16_t* da;
  int64_t ldda;
  uint16_t* daT;
  uint16_t* hT;
  int64_t ldT;
  int mpad;
};

struct BwdArgs {
  // [routed, shared]
  int N[2], K[2];
  const uint16_t* a[2];
  int64_t lda[2];
  const uint16_t* b[2];
  int64_t ldb[2];
  int64_t bstride;          // routed weight per expert (row-tiled B)
  uint16_t* c[2];
  int64_t ldc[2];
  int64_t cstride;          // routed weight gradient per expert
  const float* gu[2];
  int64_t ldgu[2];
  uint16_t* da[2];
  int64_t ldda[2];
  uint16_t* daT[2];
  uint16_t* hT[2];
  int64_t ldT[2];
  const int32_t* tiles;     // row-tiled: tile list and N-tiles per M-tile
  int ntn;
  const int32_t* offsets;
  const int32_t* pcol;      // padded first column of each routed expert, [E + 1]
  int E;
  int64_t T, Tp;
  int M[2];                 // weight-tiled: gradient rows
  int mt, nt;               // weight-tiled: M- and N-tiles per group
};

// Physical 16-byte chunk of logical chunk c in LDS row r, for rows of BK k
// (BK / 8 chunks): 16 consecutive rows read at one logical chunk fall in 16
// distinct bank groups.
template <int BK>
__device__ __forceinline__ int swz(int r, int c) {
  if (BK == 64) return r * 8 + (c ^ ((r ^ (r >> 3)) & 7));
  return r * 4 + (c ^ ((r >> 2) & 3));
}

// One TM x 128 tile: C(m, n) = sum_k A(m, k) B(k, n) for rows [m0, m0 +
// TM) below Mv and columns [n0, n0 + 128) below Nv, k in [0, Kv) (a
// multiple of 32; with BK = 64 a last half step is zero-filled).  A(m, k) =
// A[m * lda + k]; B(k, n) = B[n * ldb + k] (B_NK) or B[k * ldb + n] (B_KN).
// Four waves, 2 x 2, each TM / 2 x 64.  k steps of BK through two LDS
// buffers and two register stages: at step s the LDS holds step s and the
// registers steps s + 1 and s + 2, so every load has two steps of MFMAs to
// arrive.  BK = 64 suits long k (the row GEMMs); the weight gradients, with
// k the few rows of one expert, take BK = 32 and TM = 256: half the LDS per
// step, and 85 rather than 64 flop per byte read from L2.
template <int BK, int TM, int BMD, int EPI>
__device__ __forceinline__ void bwd_tile(u32x4 (*lds)[(TM + BBN) * (BK / 8)],
                                         const uint16_t* __restrict__ A, int64_t lda,
                                         const uint16_t* __restrict__ B, int64_t ldb, int m0,
                                         int Mv, int n0, int Nv, int Kv, const Epi& ep) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lh = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  constexpr int CH = BK / 8;           // 16-byte chunks per LDS row
  constexpr int NS = BK / 16;          // 16-wide k slices per step = B chunks per thread
  constexpr int NA = TM * CH / BNT;    // A chunks per thread
  constexpr int MI = TM / 64;          // 32-row blocks per wave
  const int nsteps = (Kv + BK - 1) / BK;

  // Thread's rows: A (and B_NK) row tid / CH + (256 / CH) j, chunk tid % CH;
  // B_KN (BK = 64): k rows 4 (tid / 16) + j, n chunk tid % 16, a 4 x 8 block
  // that is transposed in registers and stored as eight 8-byte [n][k] runs.
  static_assert(BMD != B_KN || BK == 64, "the k-row operand is staged in 64-k steps");
  struct Stage {
    u32x4 a[NA], b[NS];
  };
  const int ch = tid % CH;
  auto gload_a = [&](Stage& st, int j, int step) {
    if (step >= nsteps) return;   // past the last step: the stage is never used
    const int k0 = step * BK;
    const int m = tid / CH + (BNT / CH) * j;
    st.a[j] = (m0 + m < Mv && k0 + ch * 8 < Kv)
                  ? *reinterpret_cast<const u32x4*>(A + (int64_t)(m0 + m) * lda + k0 + ch * 8)
                  : (u32x4){0, 0, 0, 0};
  };
  auto gload_b = [&](Stage& st, int j, int step) {
    if (step >= nsteps) return;
    const int k0 = step * BK;
    if (BMD == B_NK) {
      const int n = tid / CH + (BNT / CH) * j;
      st.b[j] = (n0 + n < Nv && k0 + ch * 8 < Kv)
                    ? *reinterpret_cast<const u32x4*>(B + (int64_t)(n0 + n) * ldb + k0 + ch * 8)
                    : (u32x4){0, 0, 0, 0};
    } else {
      const int k = 4 * (tid >> 4) + j, nc = tid & 15;
      st.b[j] = (n0 + nc * 8 < Nv && k0 + k < Kv)
                    ? *reinterpret_cast<const u32x4*>(B + (int64_t)(k0 + k) * ldb + n0 + nc * 8)
                    : (u32x4){0, 0, 0, 0};
    }
  };
  auto sstore_a = [&](const Stage& st, int j, int buf) {
    const int m = tid / CH + (BNT / CH) * j;
    lds[buf][swz<BK>(m, ch)] = st.a[j];
  };
  auto sstore_b = [&](const Stage& st, int j, int buf) {
    u32x4* sB = lds[buf] + TM * CH;
    if (BMD == B_NK) {
      const int n = tid / CH + (BNT / CH) * j;
      sB[swz<BK>(n, ch)] = st.b[j];
    } else if (j == NS - 1) {   // all four k rows are in: transpose and store
      const int kq = tid >> 4, nc = tid & 15;
      uint16_t* sb = reinterpret_cast<uint16_t*>(sB);
      const uint32_t w[4][4] = {{st.b[0].x, st.b[0].y, st.b[0].z, st.b[0].w},
                                {st.b[1].x, st.b[1].y, st.b[1].z, st.b[1].w},
                                {st.b[2].x, st.b[2].y, st.b[2].z, st.b[2].w},
                                {st.b[3].x, st.b[3].y, st.b[3].z, st.b[3].w}};
#pragma unroll
      for (int i = 0; i < 8; ++i) {   // column n = 8 nc + i: k rows 4 kq .. 4 kq + 3
        const int sh = 16 * (i & 1);
        const uint32_t e0 = (w[0][i >> 1] >> sh) & 0xFFFFu, e1 = (w[1][i >> 1] >> sh) & 0xFFFFu;
        const uint32_t e2 = (w[2][i >> 1] >> sh) & 0xFFFFu, e3 = (w[3][i >> 1] >> sh) & 0xFFFFu;
        *reinterpret_cast<uint2*>(sb + swz<BK>(nc * 8 + i, kq >> 1) * 8 + (kq & 1) * 4) =
            (uint2){e0 | (e1 << 16), e2 | (e3 << 16)};
      }
    }
  };

  f32x16 acc[MI][2];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  // One step: MFMAs on LDS buffer `buf`; between its 16-wide k slices the
  // next step moves from registers `st` to buffer `nbuf`, and `st` is
  // refilled with step `ld`.
  auto step_body = [&](int buf, Stage& st, int nbuf, int ld) {
    const u32x4* sA = lds[buf];
    const u32x4* sB = lds[buf] + TM * CH;
#pragma unroll
    for (int kk = 0; kk < NS; ++kk) {
      const int c = 2 * kk + lh;
      bf16x8 af[MI], bfr[2];
#pragma unroll
      for (int i = 0; i < MI; ++i) af[i] = as_bf16x8(sA[swz<BK>(wm * (TM / 2) + i * 32 + lr, c)]);
#pragma unroll
      for (int j = 0; j < 2; ++j) bfr[j] = as_bf16x8(sB[swz<BK>(wn * 64 + j * 32 + lr, c)]);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
#pragma unroll
      for (int j = kk; j < NA; j += NS) {
        sstore_a(st, j, nbuf);
        gload_a(st, j, ld);
      }
      if (BMD == B_NK) {
        sstore_b(st, kk, nbuf);
        gload_b(st, kk, ld);
      } else if (kk == NS - 1) {   // the k-row block is stored whole, then reloaded
        sstore_b(st, NS - 1, nbuf);
#pragma unroll
        for (int j = 0; j < NS; ++j) gload_b(st, j, ld);
      }
    }
  };

  if (nsteps > 0) {
    Stage R0, R1;
#pragma unroll
    for (int j = 0; j < NA; ++j) gload_a(R0, j, 0);
#pragma unroll
    for (int j = 0; j < NS; ++j) gload_b(R0, j, 0);
#pragma unroll
    for (int j = 0; j < NA; ++j) sstore_a(R0, j, 0);
#pragma unroll
    for (int j = 0; j < NS; ++j) sstore_b(R0, j, 0);
#pragma unroll
    for (int j = 0; j < NA; ++j) gload_a(R1, j, 1);
#pragma unroll
    for (int j = 0; j < NS; ++j) gload_b(R1, j, 1);
#pragma unroll
    for (int j = 0; j < NA; ++j) gload_a(R0, j, 2);
#pragma unroll
    for (int j = 0; j < NS; ++j) gload_b(R0, j, 2);
    __syncthreads();
    for (int st = 0; st < nsteps; st += 2) {
      step_body(0, R1, 1, st + 3);     // step st; stage st+1 to LDS; load st+3
      __syncthreads();
      if (st + 1 < nsteps) {
        step_body(1, R0, 0, st + 4);   // step st+1; stage st+2 to LDS; load st+4
        __syncthreads();
      }
    }
  }

  // Epilogue: lane holds column lr of each 32 x 32 block, rows
  // 8 (q / 4) + 4 lh + q % 4.
  if (EPI == E_STORE) {
    // Through LDS, 64 rows of each wave's TM / 2 x 64 sub-tile at a time,
    // so that every global store writes 16 contiguous bytes (eight lanes
    // cover one 128-byte row segment).
    constexpr int OLD = 72;   // LDS row stride (elements): 16-byte aligned, 4-bank skew
    uint16_t* so = reinterpret_cast<uint16_t*>(lds[0]) + wave * 64 * OLD;
#pragma unroll
    for (int pass = 0; pass < MI / 2; ++pass) {
      __syncthreads();   // the LDS is free (main loop, or the previous pass, is done)
#pragma unroll
      for (int ii = 0; ii < 2; ++ii)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 16; ++q)
            so[(ii * 32 + 8 * (q >> 2) + 4 * lh + (q & 3)) * OLD + j * 32 + lr] =
                (uint16_t)f32_to_bf16_bits(acc[2 * pass + ii][j][q]);
      __syncthreads();
      const int rb = m0 + wm * (TM / 2) + pass * 64, cb = n0 + wn * 64;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int r = (lane >> 3) + 8 * t, c = (lane & 7) * 8;
        if (rb + r < Mv && cb + c < Nv)
          *reinterpret_cast<u32x4*>(ep.c + (int64_t)(rb + r) * ep.ldc + cb + c) =
              *reinterpret_cast<const u32x4*>(so + r * OLD + c);
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 64 + j * 32 + lr;
      if (n >= Nv) continue;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int mb = m0 + wm * (TM / 2) + i * 32 + 8 * qq + 4 * lh;   // rows mb .. mb + 3
        {
          float dg[4], du[4], hv[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            dg[r] = du[r] = hv[r] = 0.0f;
            const int m = mb + r;
            if (m < Mv) {
              const float v = acc[i][j][4 * qq + r];
              const float* gu = ep.gu + (int64_t)m * ep.ldgu;
              const float gv = gu[n], uv = gu[Nv + n];
              const float sg = 1.0f / (1.0f + __expf(-gv));
              dg[r] = v * uv * sg * (1.0f + gv * (1.0f - sg));
              du[r] = v * gv * sg;
              hv[r] = gv * sg * uv;
              uint16_t* da = ep.da + (int64_t)m * ep.ldda;
              da[n] = (uint16_t)f32_to_bf16_bits(dg[r]);
              da[Nv + n] = (uint16_t)f32_to_bf16_bits(du[r]);
            }
          }
          if (mb < ep.mpad) {   // four consecutive columns of the transposed rows
            const uint2 pg = {pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3])};
            const uint2 pu = {pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3])};
            const uint2 ph = {pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
            *reinterpret_cast<uint2*>(ep.daT + (int64_t)n * ep.ldT + mb) = pg;
            *reinterpret_cast<uint2*>(ep.daT + (int64_t)(Nv + n) * ep.ldT + mb) = pu;
            *reinterpret_cast<uint2*>(ep.hT + (int64_t)n * ep.ldT + mb) = ph;
          }
        }
      }
    }
}

// Row-tiled GEMMs (DH, DX): work item = (M-tile of the tile list, N-tile).
// A is the tile's rows (dy or [dg du]), B the group's weight (k rows).
template <int EPI>
__global__ void __launch_bounds__(BNT) bwd_rows_kernel(BwdArgs p) {
  constexpr int BK = 64;
  __shared__ u32x4 lds[2][(BBM + BBN) * (BK / 8)];   // 64 KiB
  const int64_t work = (int64_t)p.tiles[0] * p.ntn;
  const int64_t w = xcd_chunked(blockIdx.x, work);
  if (w < 0) return;
  int ntile;
  const int32_t* ent = decode_work(p.tiles, w, p.ntn, ntile);
  const int g = ent[0], row0 = ent[1], nrows = ent[2];
  const int s = (g == p.E) ? 1 : 0;
  if (ntile * BBN >= p.N[s]) return;
  const uint16_t* A = p.a[s] + (int64_t)row0 * p.lda[s];
  const uint16_t* B = p.b[s] + (s == 0 ? (int64_t)g * p.bstride : 0);
  Epi ep{};
  if (EPI == E_STORE) {
    ep.c = p.c[s] + (int64_t)row0 * p.ldc[s];
    ep.ldc = p.ldc[s];
  } else {
    // transposed columns: the shared expert's rows are its tokens; a routed
    // expert's rows start at its padded column
    const int64_t col = s ? row0 : p.pcol[g] + (row0 - p.offsets[g]);
    ep.gu = p.gu[s] + (int64_t)row0 * p.ldgu[s];
    ep.ldgu = p.ldgu[s];
    ep.da = p.da[s] + (int64_t)row0 * p.ldda[s];
    ep.ldda = p.ldda[s];
    ep.daT = p.daT[s] + col;
    ep.hT = p.hT[s] + col;
    ep.ldT = p.ldT[s];
    ep.mpad = (nrows + kPad - 1) / kPad * kPad;
  }
  bwd_tile<BK, BBM, B_KN, EPI>(lds, A, p.lda[s], B, p.ldb[s], 0, nrows, ntile * BBN, p.N[s], p.K[s],
                          ep);
}

// Weight-gradient GEMMs (DW2, DW13): work item = (group, 256-row M-tile,
// N-tile); A and B are transposed operands, k over the group's padded
// columns (an expert without rows gets a zero gradient).  The tiles are
// short (k = one expert's rows), so a fixed grid of two workgroups per CU
// loops over them instead of one launch per tile: workgroup i of an XCD
// takes tiles i, i + n, i + 2n, ... of that XCD's contiguous range, so the
// XCD's workgroups work on neighbouring tiles (one expert's operands) at a
// time.
constexpr int kWgradPerCu = 2;

__global__ void __launch_bounds__(BNT, kWgradPerCu) bwd_wgrad_kernel(BwdArgs p) {
  constexpr int BK = 32;
  __shared__ u32x4 lds[2][(WTM + BBN) * (BK / 8)];   // 48 KiB
  const int64_t per_g = (int64_t)p.mt * p.nt;
  const int64_t groups = p.E + (p.M[1] > 0 ? 1 : 0);
  const int64_t work = groups * per_g;
  // Workgroup b takes the items of virtual workgroups b, b + G, b + 2G, ...
  // (G, the grid, a multiple of kXcdGrid), dealt out in XCD chunks: every
  // XCD gets its share of each part of the list, the shared expert's long
  // tiles at its end included.
  for (int64_t vb = blockIdx.x;; vb += gridDim.x) {
    const int64_t w = xcd_chunked(vb, work);
    if (w < 0) break;
    const int g = (int)(w / per_g);
    const int rest = (int)(w % per_g);
    const int mtile = rest / p.nt, ntile = rest % p.nt;
    const int s = (g == p.E) ? 1 : 0;
    if (mtile * WTM >= p.M[s] || ntile * BBN >= p.N[s]) continue;   // uniform
    const int64_t col = s ? 0 : p.pcol[g];
    const int kv = s ? (int)p.Tp : p.pcol[g + 1] - p.pcol[g];
    Epi ep{};
    ep.c = p.c[s] + (s == 0 ? (int64_t)g * p.cstride : 0);
    ep.ldc = p.ldc[s];
    bwd_tile<BK, WTM, B_NK, E_STORE>(lds, p.a[s] + col, p.lda[s], p.b[s] + col, p.ldb[s],
                                     mtile * WTM, p.M[s], ntile * BBN, p.N[s], kv, ep);
    __syncthreads();   // the next tile's prologue rewrites the LDS
  }
}

// pcol[e] = sum over e' < e of the row count of e' rounded up to kPad, for
// e <= E (one workgroup of 1024 threads, E < 1024).
__global__ void __launch_bounds__(1024)
pad_columns_kernel(const int32_t* __restrict__ offsets, int E, int32_t* __restrict__ pcol) {
  __shared__ int32_t wsum[16];
  const int e = threadIdx.x;
  const int32_t c = e < E ? (offsets[e + 1] - offsets[e] + kPad - 1) / kPad * kPad : 0;
  const int32_t incl = block_inclusive_scan<1024>(c, wsum);
  if (e <= E) pcol[e] = incl - c;
}

// dst[h][c0 + jj] = src[row(jj)][h] for a block of 32 columns and 64 h, zero
// where the column has no row.  Routed (pcol != null): column block c0 lies
// in the expert e with pcol[e] <= c0 < pcol[e + 1]; its column j is row
// offsets[e] + j of the sorted order, read from src row perm[...] / topk
// when gathering (topk > 0) or from that row itself.  Shared: column t is
// row t, for t < T.
constexpr int TR_COLS = 32, TR_H = 64, TR_LD = 72;   // LDS row stride (elements)

__global__ void __launch_bounds__(256)
transpose_kernel(const uint16_t* __restrict__ src, int H, const int32_t* __restrict__ perm,
                 int topk, const int32_t* __restrict__ offsets,
                 const int32_t* __restrict__ pcol, int E, int64_t T, uint16_t* __restrict__ dst,
                 int64_t ldd) {
  __shared__ uint16_t tile[TR_COLS * TR_LD];
  const int tid = threadIdx.x;
  const int64_t c0 = (int64_t)blockIdx.x * TR_COLS;
  const int h0 = blockIdx.y * TR_H;
  int64_t first = 0, count = 0;   // sorted rows of this column block
  if (pcol) {
    if (c0 >= pcol[E]) return;     // uniform
    int lo = 0, hi = E - 1;        // largest e with pcol[e] <= c0
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pcol[mid] <= c0) lo = mid; else hi = mid - 1;
    }
    const int64_t j0 = c0 - pcol[lo];
    first = offsets[lo] + j0;
    count = offsets[lo + 1] - offsets[lo] - j0;
  } else {
    first = c0;
    count = T - c0;
  }
  // load: thread -> (column jj, 8 consecutive h)
  {
    const int jj = tid >> 3, hc = tid & 7;
    u32x4 v = {0, 0, 0, 0};
    if (jj < count) {
      const int64_t j = first + jj;
      const int64_t row = (pcol && topk > 0) ? (int64_t)(perm[j] / topk) : j;
      v = *reinterpret_cast<const u32x4*>(src + row * H + h0 + hc * 8);
    }
    *reinterpret_cast<u32x4*>(tile + jj * TR_LD + hc * 8) = v;
  }
  __syncthreads();
  // store: thread -> (h, 8 consecutive columns)
  {
    const int h = tid >> 2, cc = tid & 3;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)tile[(cc * 8 + 2 * i) * TR_LD + h] |
             ((uint32_t)tile[(cc * 8 + 2 * i + 1) * TR_LD + h] << 16);
    *reinterpret_cast<u32x4*>(dst + (int64_t)(h0 + h) * ldd + c0 + cc * 8) =
        (u32x4){w[0], w[1], w[2], w[3]};
  }
}


// Workgroups of the looping weight-gradient kernel: kWgradPerCu per CU of
// the current device rounded down to a multiple of kXcdGrid (at least one).
unsigned wgrad_grid(int64_t work) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  const int64_t slots = std::max<int64_t>((int64_t)cus * kWgradPerCu / kXcdGrid, 1) * kXcdGrid;
  return (unsigned)std::min<int64_t>(slots, xcd_grid(work));
}

// Row stride (elements) of at least n whose size in bytes is an odd
// multiple of 128: successive rows of a tile then fall in different memory
// channels (a power-of-two stride would put them all in a few).
int64_t spread_ld(int64_t n, int elem_bytes) {
  const int64_t q = 128 / elem_bytes;
  int64_t ld = (n + q - 1) / q * q;
  if ((ld / q) % 2 == 0) ld += q;
  return ld;
}

// Workspace segments (bytes, 256-aligned) and row strides (elements).
struct BwdLayout {
  size_t gu, da, daT, hT, xT, dyT, pcol, tiles, total;
  int64_t NP, Tp;            // transposed columns: routed (capacity), shared
  int64_t ldr, lds;          // transposed row strides: routed, shared
  int64_t ldgu_r, ldgu_s;    // [g u] rows (fp32)
  int64_t ldda_r, ldda_s;    // [dg du] rows (bf16)
};

BwdLayout bwd_layout(const FfnDims& d) {
  BwdLayout L{};
  const int64_t rs = d.Is > 0 ? d.T : 0;
  // every expert's padded width is below its rows + kPad
  L.NP = (d.N + kPad - 1) / kPad * kPad + (int64_t)kPad * d.E;
  L.Tp = (rs + kPad - 1) / kPad * kPad;
  L.ldr = spread_ld(L.NP, 2);
  L.lds = spread_ld(L.Tp, 2);
  L.ldgu_r = spread_ld(2 * d.I, 4);
  L.ldgu_s = spread_ld(2 * d.Is, 4);
  L.ldda_r = spread_ld(2 * d.I, 2);
  L.ldda_s = spread_ld(2 * d.Is, 2);
  size_t o = 0;
  auto take = [&](size_t b) {
    const size_t at = o;
    o += (b + 255) / 256 * 256;
    return at;
  };
  L.gu = take((size_t)(d.N * L.ldgu_r + rs * L.ldgu_s) * 4);
  L.da = take((size_t)(d.N * L.ldda_r + rs * L.ldda_s) * 2);
  L.daT = take((size_t)(2 * d.I * L.ldr + 2 * d.Is * L.lds) * 2);
  L.hT = take((size_t)(d.I * L.ldr + d.Is * L.lds) * 2);
  L.xT = take((size_t)d.H * (L.ldr + L.lds) * 2);
  L.dyT = take((size_t)d.H * (L.ldr + L.lds) * 2);
  L.pcol = take((size_t)(d.E + 1) * 4);
  L.tiles = take(ffn_tiles_bytes(d));
  L.total = o;
  return L;
}

}  // namespace

size_t ffn_backward_ws_bytes(const FfnDims& d) { return bwd_layout(d).total; }

hipError_t launch_ffn_backward(const FfnDims& d, const uint16_t* x, const int32_t* perm,
                               const int32_t* offsets, const uint16_t* w13, const uint16_t* w2,
                               const uint16_t* ws13, const uint16_t* ws2, const uint16_t* dy,
                               const uint16_t* dys, uint16_t* dx, uint16_t* dxs, uint16_t* dw13,
                               uint16_t* dw2, uint16_t* dws13, uint16_t* dws2, void* ws,
                               hipStream_t s) {
  const int64_t N = d.N, T = d.T;
  const int H = d.H, I = d.I, Is = d.Is, E = d.E;
  const bool sh = Is > 0;
  const BwdLayout L = bwd_layout(d);
  char* base = (char*)ws;
  float* gu_r = (float*)(base + L.gu);
  float* gu_s = gu_r + N * L.ldgu_r;
  uint16_t* da_r = (uint16_t*)(base + L.da);
  uint16_t* da_s = da_r + N * L.ldda_r;
  uint16_t* daT_r = (uint16_t*)(base + L.daT);
  uint16_t* daT_s = daT_r + 2 * I * L.ldr;
  uint16_t* hT_r = (uint16_t*)(base + L.hT);
  uint16_t* hT_s = hT_r + I * L.ldr;
  uint16_t* xT_r = (uint16_t*)(base + L.xT);
  uint16_t* xT_s = xT_r + H * L.ldr;
  uint16_t* dyT_r = (uint16_t*)(base + L.dyT);
  uint16_t* dyT_s = dyT_r + H * L.ldr;
  int32_t* pcol = (int32_t*)(base + L.pcol);
  int32_t* tiles = (int32_t*)(base + L.tiles);

  // GU: [g u] = x_rows W13^T (rows x 2I, k = H), fp32, with the forward's
  // row-major gate/up GEMM.
  hipError_t e = launch_gate_up_bf16(d, x, perm, offsets, w13, ws13, tiles, gu_r, L.ldgu_r, gu_s,
                                     L.ldgu_s, s);
  if (e != hipSuccess) return e;
  e = launch_build_tiles(offsets, E, T, true, sh, BBM, tiles, s);
  if (e != hipSuccess) return e;
  const int64_t mt = ffn_max_mtiles(N, T, E, BBM);

  // Padded columns, then x (gathered) and dy in transposed form.
  MOE_TIMED_LAUNCH(s, "pad_columns_kernel",
    hipLaunchKernelGGL(pad_columns_kernel, dim3(1), dim3(1024), 0, s, offsets, E, pcol));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  {
    const dim3 gr((unsigned)((L.NP + TR_COLS - 1) / TR_COLS), H / TR_H);
    MOE_TIMED_LAUNCH(s, "transpose_kernel<x>",
      hipLaunchKernelGGL(transpose_kernel, gr, dim3(256), 0, s, x, H, perm, d.K, offsets, pcol, E,
                         T, xT_r, L.ldr));
    MOE_TIMED_LAUNCH(s, "transpose_kernel<dy>",
      hipLaunchKernelGGL(transpose_kernel, gr, dim3(256), 0, s, dy, H, perm, 0, offsets, pcol, E,
                         T, dyT_r, L.ldr));
    if (sh) {
      const dim3 gs((unsigned)(L.Tp / TR_COLS), H / TR_H);
      MOE_TIMED_LAUNCH(s, "transpose_kernel<x>",
        hipLaunchKernelGGL(transpose_kernel, gs, dim3(256), 0, s, x, H, nullptr, 0, nullptr,
                           nullptr, E, T, xT_s, L.lds));
      MOE_TIMED_LAUNCH(s, "transpose_kernel<dy>",
        hipLaunchKernelGGL(transpose_kernel, gs, dim3(256), 0, s, dys, H, nullptr, 0, nullptr,
                           nullptr, E, T, dyT_s, L.lds));
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }

  BwdArgs p{};
  p.tiles = tiles;
  p.offsets = offsets;
  p.pcol = pcol;
  p.E = E;
  p.T = T;
  p.Tp = L.Tp;

  // DH: dh = dy W2 (rows x I, k = H); epilogue writes [dg du] (rows and
  // transposed) and h (transposed).
  {
    BwdArgs q = p;
    q.N[0] = I; q.N[1] = Is; q.K[0] = q.K[1] = H;
    q.a[0] = dy; q.a[1] = dys; q.lda[0] = q.lda[1] = H;
    q.b[0] = w2; q.b[1] = ws2; q.ldb[0] = I; q.ldb[1] = Is; q.bstride = (int64_t)H * I;
    q.gu[0] = gu_r; q.gu[1] = gu_s; q.ldgu[0] = L.ldgu_r; q.ldgu[1] = L.ldgu_s;
    q.da[0] = da_r; q.da[1] = da_s; q.ldda[0] = L.ldda_r; q.ldda[1] = L.ldda_s;
    q.daT[0] = daT_r; q.daT[1] = daT_s; q.hT[0] = hT_r; q.hT[1] = hT_s;
    q.ldT[0] = L.ldr; q.ldT[1] = L.lds;
    q.ntn = (std::max(I, Is) + BBN - 1) / BBN;
    MOE_TIMED_LAUNCH(s, "bwd_rows_kernel<dh>",
      hipLaunchKernelGGL(bwd_rows_kernel<E_DH>, dim3(xcd_grid(mt * q.ntn)), dim3(BNT), 0, s, q));
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // DX: dx_rows = [dg du] W13 (rows x H, k = 2I).
  if (dx || dxs) {
    BwdArgs q = p;
    q.N[0] = q.N[1] = H; q.K[0] = 2 * I; q.K[1] = 2 * Is;
    q.a[0] = da_r; q.a[1] = da_s; q.lda[0] = L.ldda_r; q.lda[1] = L.ldda_s;
    q.b[0] = w13; q.b[1] = ws13; q.ldb[0] = q.ldb[1] = H; q.bstride = (int64_t)2 * I * H;
    q.c[0] = dx; q.c[1] = dxs; q.ldc[0] = q.ldc[1] = H;
    q.ntn = (H + BBN - 1) / BBN;
    MOE_TIMED_LAUNCH(s, "bwd_rows_kernel<dx>",
      hipLaunchKernelGGL(bwd_rows_kernel<E_STORE>, dim3(xcd_grid(mt * q.ntn)), dim3(BNT), 0, s,
                         q));
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // DW2: dW2 = dy^T h (H x I, k = the expert's rows): A = dy^T, B = h^T.
  {
    BwdArgs q = p;
    q.M[0] = H; q.M[1] = sh ? H : 0; q.N[0] = I; q.N[1] = Is;
    q.a[0] = dyT_r; q.a[1] = dyT_s; q.lda[0] = L.ldr; q.lda[1] = L.lds;
    q.b[0] = hT_r; q.b[1] = hT_s; q.ldb[0] = L.ldr; q.ldb[1] = L.lds;
    q.c[0] = dw2; q.c[1] = dws2; q.ldc[0] = I; q.ldc[1] = Is; q.cstride = (int64_t)H * I;
    q.mt = (H + WTM - 1) / WTM;
    q.nt = (std::max(I, Is) + BBN - 1) / BBN;
    const int64_t work = (int64_t)(E + (sh ? 1 : 0)) * q.mt * q.nt;
    MOE_TIMED_LAUNCH(s, "bwd_wgrad_kernel<dw2>",
      hipLaunchKernelGGL(bwd_wgrad_kernel, dim3(wgrad_grid(work)), dim3(BNT), 0, s, q));
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // DW13: dW13 = [dg du]^T x_rows (2I x H, k = the expert's rows): A =
  // [dg du]^T, B = x_rows^T.
  {
    BwdArgs q = p;
    q.M[0] = 2 * I; q.M[1] = sh ? 2 * Is : 0; q.N[0] = q.N[1] = H;
    q.a[0] = daT_r; q.a[1] = daT_s; q.lda[0] = L.ldr; q.lda[1] = L.lds;
    q.b[0] = xT_r; q.b[1] = xT_s; q.ldb[0] = L.ldr; q.ldb[1] = L.lds;
    q.c[0] = dw13; q.c[1] = dws13; q.ldc[0] = q.ldc[1] = H; q.cstride = (int64_t)2 * I * H;
    q.mt = (std::max(2 * I, 2 * Is) + WTM - 1) / WTM;
    q.nt = (H + BBN - 1) / BBN;
    const int64_t work = (int64_t)(E + (sh ? 1 : 0)) * q.mt * q.nt;
    MOE_TIMED_LAUNCH(s, "bwd_wgrad_kernel<dw13>",
      hipLaunchKernelGGL(bwd_wgrad_kernel, dim3(wgrad_grid(work)), dim3(BNT), 0, s, q));
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace moe
