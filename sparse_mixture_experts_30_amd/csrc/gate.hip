// Gate and selection kernels (gfx950).
//
// The gate of the layer (page "从 1024 块 GPU 到 558 万美元：拆解 DeepSeek-V3 的算法-系统协同设计",
// section 2.2, MoEGate): logits = x W^T computed in fp32, sigmoid scores, a
// per-expert bias added only to choose, the per-group sum of the two largest
// choice scores, the topk_group best groups, the top_k best experts inside
// them (0.0 for experts outside), weights from the unbiased scores normalised
// over the chosen experts when top_k > 1, times routed_scaling_factor.
//
// Gate GEMM: x is exact in bf16, the fp32 gate weight w splits exactly into
// three bf16 parts (hi = w truncated to bf16, mid = (w - hi) truncated,
// lo = w - hi - mid, which has at most 8 significant bits).  Each product of a
// bf16 x with a bf16 part is exact in fp32, so three bf16 MFMAs accumulated in
// fp32 give an fp32-accurate x w^T at bf16-MFMA rate.  The split is done once
// per call by a small kernel that also lays the three parts out in MFMA
// fragment order; the GEMM then streams them straight into registers.
#include "moe_internal.hpp"
#include "gate_split.hpp"
#include "select_device.hpp"

#include <float.h>

#include <atomic>

namespace moe {

namespace {

constexpr int GBM = 128;   // tokens per tile
constexpr int GEB = 4;     // 32-expert blocks per tile (one per wave)
constexpr int GBK = 64;    // k per step
constexpr int GTHREADS = 256;
constexpr int GFRAG = 3 * 4 * 64;   // 16-byte fragments per (expert block, step)

// wp block (eb, step) = [part 3][k slice 4][lane 64] x 16 bytes: lane l of
// slice kk holds expert 32 eb + l%32 (zero past E) at k = 64 step +
// 32 (l / 32) + 8 kk .. +8, as bf16 part hi, mid or lo.
__global__ void __launch_bounds__(256)
gate_split_kernel(const float* __restrict__ wg, u32x4* __restrict__ wp, int E, int H,
                  int64_t nslot) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;   // (eb, step, kk, lane)
  if (c >= nslot) return;
  const int nsteps = H / GBK;
  const int lane = (int)(c & 63), kk = (int)((c >> 6) & 3);
  const int64_t rest = c >> 8;
  const int step = (int)(rest % nsteps);
  const int64_t eb = rest / nsteps;
  const int e = (int)(eb * 32 + (lane & 31));
  const int k = step * GBK + 32 * (lane >> 5) + 8 * kk;
  u32x4 p = {0, 0, 0, 0}, q = {0, 0, 0, 0};
  if (e < E) {
    p = *reinterpret_cast<const u32x4*>(wg + (int64_t)e * H + k);
    q = *reinterpret_cast<const u32x4*>(wg + (int64_t)e * H + k + 4);
  }
  u32x4 h, m, l;
  split3(p, q, h, m, l);
  u32x4* dst = wp + (eb * nsteps + step) * GFRAG + kk * 64 + lane;
  dst[0] = h;
  dst[256] = m;
  dst[512] = l;
}

__device__ __forceinline__ int gswz(int r, int c) { return r * 8 + (c ^ ((r ^ (r >> 3)) & 7)); }

// partials[ks][t][e] = sum over the ks-th k range of x[t,h] w[e,h].
// Tile: 128 tokens x 128 experts; wave w owns expert block 4 blockIdx.y + w
// (32 experts) for all 128 tokens (four 32x32 MFMA blocks, each fed by the
// three weight parts).  The token tile is shared through double-buffered,
// XOR-swizzled LDS; the weight parts go straight from the split copy into
// registers, one step ahead.  Two workgroups share a CU.
__global__ void __launch_bounds__(GTHREADS, 2)
gate_logits_bf16_kernel(const uint16_t* __restrict__ x, const u32x4* __restrict__ wp,
                        float* __restrict__ part, int64_t T, int H, int E, int neb,
                        int steps_per_split) {
  __shared__ u32x4 sA[2][GBM * 8];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, lh = lane >> 5;
  const int64_t m0 = (int64_t)blockIdx.x * GBM;
  const int eb = blockIdx.y * GEB + wave;
  const bool active = eb < neb;
  const int ebc = active ? eb : neb - 1;        // idle waves re-read a valid block
  const int ks = blockIdx.z;
  const int nsteps_all = H / GBK;
  const int s0 = ks * steps_per_split;
  const int nsteps = min(nsteps_all, s0 + steps_per_split) - s0;
  const int last = nsteps - 1;
  if (nsteps <= 0) {                            // an empty split contributes zero
    const int e = eb * 32 + lr;
    if (active && e < E)
      for (int r = 0; r < GBM / 2; ++r) {
        const int64_t t = m0 + 2 * r + lh;
        if (t < T) part[((int64_t)ks * T + t) * E + e] = 0.0f;
      }
    return;                                     // uniform over the workgroup
  }

  // Token rows staged by this thread: (tid / 8) + 32 j, chunk tid % 8; rows
  // past T re-read row T - 1 (results dropped).
  const int ch = tid & 7;
  const uint16_t* arow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t t = min(m0 + (tid >> 3) + 32 * j, T - 1);
    arow[j] = x + t * H + s0 * GBK + ch * 8;
  }
  const u32x4* bsrc = wp + ((int64_t)ebc * nsteps_all + s0) * GFRAG + lane;
  u32x4 ra[4], rb[2][12];
  auto aload = [&](int step) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      ra[j] = *reinterpret_cast<const u32x4*>(arow[j] + min(step, last) * GBK);
  };
  auto astore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) sA[buf][gswz((tid >> 3) + 32 * j, ch)] = ra[j];
  };
  auto bload = [&](int slot, int step) {
    const u32x4* src = bsrc + (int64_t)min(step, last) * GFRAG;
#pragma unroll
    for (int i = 0; i < 12; ++i) rb[slot][i] = src[i * 64];   // [part][kk]
  };

  f32x16 acc[4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[r][i] = 0.0f;

  aload(0);
  bload(0, 0);
  astore(0);
  aload(1);
  bload(1, 1);
  __syncthreads();

  auto step_body = [&](int buf, int u, int step) {
    const u32x4* as = sA[buf];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8 a[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) a[r] = as_bf16x8(as[gswz(r * 32 + lr, 4 * lh + kk)]);
      if (active) {
#pragma unroll
        for (int pt = 0; pt < 3; ++pt) {
          const bf16x8 b = as_bf16x8(rb[u][pt * 4 + kk]);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[r], b, acc[r], 0, 0, 0);
        }
      }
    }
    astore(buf ^ 1);
    aload(step + 2);
    bload(u, step + 2);
    __syncthreads();
  };
  int s = 0;
  for (; s + 2 <= nsteps; s += 2) {
    step_body(0, 0, s);
    step_body(1, 1, s + 1);
  }
  if (s < nsteps) step_body(0, 0, s);

  // C layout of a 32x32 MFMA block: lane holds column lane%32 and rows
  // 8*(i/4) + 4*(lane/32) + i%4 for i = 0..15.
  const int e = eb * 32 + lr;
  if (active && e < E) {
    float* base = part + (int64_t)ks * T * E;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t t = m0 + r * 32 + 8 * (i >> 2) + 4 * lh + (i & 3);
        if (t < T) base[t * E + e] = acc[r][i];
      }
  }
}

// fp32 activations: plain fp32 FMA dot products (used for fp32 layers).
// 16x16 output tile per 256-thread block, k in LDS slices of 64.
__global__ void __launch_bounds__(256)
gate_logits_f32_kernel(const float* __restrict__ x, const float* __restrict__ wg,
                       float* __restrict__ out, int64_t T, int H, int E) {
  __shared__ float sx[16][65], sw[16][65];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int64_t t = (int64_t)blockIdx.x * 16 + ty;
  const int e = blockIdx.y * 16 + tx;
  float acc = 0.0f;
  for (int k0 = 0; k0 < H; k0 += 64) {
    for (int j = threadIdx.x; j < 16 * 64; j += 256) {
      int r = j >> 6, c = j & 63;
      int64_t tt = (int64_t)blockIdx.x * 16 + r;
      int ee = blockIdx.y * 16 + r;
      sx[r][c] = (tt < T && k0 + c < H) ? x[tt * H + k0 + c] : 0.0f;
      sw[r][c] = (ee < E && k0 + c < H) ? wg[(int64_t)ee * H + k0 + c] : 0.0f;
    }
    __syncthreads();
#pragma unroll 16
    for (int c = 0; c < 64; ++c) acc = fmaf(sx[ty][c], sw[tx][c], acc);
    __syncthreads();
  }
  if (t < T && e < E) out[t * E + e] = acc;
}

constexpr int SEL_WAVES = 4;
static_assert(SEL_WAVES == SEL_PARTS, "a deep-split token's parts are summed by the waves");

// One wavefront selects for one token; lane l holds experts e = l + 64 v.
// SW = 1: a workgroup holds SEL_WAVES tokens.  SW = SEL_WAVES (deep k
// splits, small batches): a workgroup holds one token, its waves first sum
// contiguous quarters of the splits (four times the loads in flight, over
// four times the CUs), the quarters are added in wave order through LDS
// (a fixed order: the result does not depend on timing), and wave 0 selects.
template <int SW>
__global__ void __launch_bounds__(SEL_WAVES * 64)
select_kernel(const float* __restrict__ part, int ksplit, const float* __restrict__ bias,
              float* __restrict__ logits_out, int32_t* __restrict__ idx_out,
              float* __restrict__ w_out, int64_t T, int E, int G, int TG, int K, float rho) {
  __shared__ float s_c[SEL_WAVES][512];
  __shared__ float s_s[SEL_WAVES][512];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = SW == 1 ? (int64_t)blockIdx.x * SEL_WAVES + wave : (int64_t)blockIdx.x;
  if (t >= T) return;   // uniform over the workgroup when SW > 1
  const int V = (E + 63) / 64;
  const int s_begin = SW == 1 ? 0 : sel_part_begin(ksplit, wave);
  const int s_end = SW == 1 ? ksplit : sel_part_begin(ksplit, wave + 1);
  float lgs[SEL_MAXV];
  sum_splits(part, T * E, t, E, lane, s_begin, s_end, lgs);
  if (SW > 1) {
    // quarters added in wave order; wave 0 goes on alone (no workgroup
    // barrier below this point)
#pragma unroll
    for (int v = 0; v < SEL_MAXV; ++v) {
      const int e = lane + 64 * v;
      if (v < V && e < E) s_c[wave][e] = lgs[v];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int v = 0; v < SEL_MAXV; ++v) {
      const int e = lane + 64 * v;
      if (v < V && e < E) {
        float acc = s_c[0][e];
#pragma unroll
        for (int w = 1; w < SW; ++w) acc += s_c[w][e];
        lgs[v] = acc;
      }
    }
  }

  select_token(lgs, lane, bias, s_c[wave], s_s[wave], E, G, TG, K, rho,
               logits_out ? logits_out + t * E : nullptr, idx_out + t * K, w_out + t * K,
               nullptr);
}

// ---------------------------------------------------------------- gate + selection in one kernel
//
// The gate mode MOE_GATE_FUSED: one workgroup computes the logits of 64
// tokens for every expert over the whole hidden size (eight waves, wave w
// the 32 experts of block w, three bf16 weight parts per k slice as above),
// keeps them in LDS and selects in the same launch, so no partial sums go to
// memory.  The selection is spread over teams of SEL_TEAM threads per token
// (select_team: thread q of a team holds experts [q E/8, (q+1) E/8) in
// registers, the group scores are merged with lane shuffles inside the team
// and exchanged through LDS, and each of the K picks is the team's butterfly
// maximum); its arithmetic is select_token's, so the routing is the same
// function of the fp32 logits.  Holding all experts of its tokens, a
// workgroup can hold only 64 tokens if a 16384-token batch is to fill 256
// compute units, half the split kernel's 128: each weight byte from L2 then
// feeds half as many MFMAs, and the split kernels stay the default.
constexpr int FG_T = 64;                 // tokens per workgroup
constexpr int FG_WAVES = 8;              // wave w: expert block w
constexpr int FG_THREADS = FG_WAVES * 64;
static_assert(FG_THREADS == FG_T * SEL_TEAM, "one selection team per token");
constexpr int FG_DEPTH = 2;              // k steps of weights in flight per wave

__host__ __device__ constexpr int fg_lde(int E) { return E + 4; }   // logit row stride (floats)

size_t fg_lds_bytes(int E) {
  const size_t tiles = (size_t)2 * FG_T * 8 * sizeof(u32x4);
  const size_t sel = (size_t)FG_T * fg_lde(E) * 4 + (size_t)FG_T * SEL_TG * 4;
  return tiles > sel ? tiles : sel;
}

__global__ void __launch_bounds__(FG_THREADS, 1)
gate_select_fused_kernel(const uint16_t* __restrict__ x, const u32x4* __restrict__ wp,
                         const float* __restrict__ bias, float* __restrict__ logits_out,
                         int32_t* __restrict__ idx_out, float* __restrict__ w_out, int64_t T,
                         int H, int E, int G, int TG, int K, float rho) {
  extern __shared__ u32x4 fsm[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, lh = lane >> 5;
  const int64_t t0 = (int64_t)blockIdx.x * FG_T;
  const bool active = wave < E / 32;             // uniform per wave
  const int nsteps = H / GBK, last = nsteps - 1;

  // Activation chunk of this thread: token row tid / 8 (rows past T re-read
  // row T - 1; their results are dropped), 16-byte chunk tid % 8.
  const int ch = tid & 7;
  const uint16_t* arow = x + min(t0 + (tid >> 3), T - 1) * H + ch * 8;
  const u32x4* bsrc = wp + (int64_t)(active ? wave : 0) * nsteps * GFRAG + lane;
  u32x4 ra, rb[FG_DEPTH][12];
  auto aload = [&](int step) {
    ra = *reinterpret_cast<const u32x4*>(arow + min(step, last) * GBK);
  };
  auto astore = [&](int buf) { fsm[buf * FG_T * 8 + gswz(tid >> 3, ch)] = ra; };
  auto bload = [&](u32x4 (&dst)[12], int step) {
    if (!active) return;
    const u32x4* src = bsrc + (int64_t)min(step, last) * GFRAG;
#pragma unroll
    for (int i = 0; i < 12; ++i) dst[i] = src[i * 64];   // [part][kk]
  };

  f32x16 acc[2];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[r][i] = 0.0f;

  // Step t reads LDS buffer t % 2 and weight slot t % FG_DEPTH; the weights
  // of a step are requested FG_DEPTH steps ahead, its activation rows two.
  aload(0);
  astore(0);
  aload(1);
#pragma unroll
  for (int j = 0; j < FG_DEPTH; ++j) bload(rb[j], j);
  __syncthreads();

  auto step_body = [&](int buf, u32x4 (&b)[12], int step) {
    const u32x4* as = fsm + buf * FG_T * 8;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const bf16x8 a0 = as_bf16x8(as[gswz(lr, 4 * lh + kk)]);
      const bf16x8 a1 = as_bf16x8(as[gswz(32 + lr, 4 * lh + kk)]);
      if (active) {
#pragma unroll
        for (int pt = 0; pt < 3; ++pt) {
          const bf16x8 bv = as_bf16x8(b[pt * 4 + kk]);
          acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bv, acc[0], 0, 0, 0);
          acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bv, acc[1], 0, 0, 0);
        }
      }
    }
    astore(buf ^ 1);
    aload(step + 2);
    bload(b, step + FG_DEPTH);
    __syncthreads();
  };
  constexpr int U = (FG_DEPTH % 2) ? 2 * FG_DEPTH : FG_DEPTH;   // every index static
  int s = 0;
  for (; s + U <= nsteps; s += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) step_body(u & 1, rb[u % FG_DEPTH], s + u);
  }
#pragma unroll
  for (int u = 0; u < U - 1; ++u)
    if (s + u < nsteps) step_body(u & 1, rb[u % FG_DEPTH], s + u);

  // Logits of the 64 tokens into LDS (over the activation buffers, which
  // every wave has finished reading at the last barrier).  C layout of a
  // 32x32 block: lane holds column lane%32, rows 8*(i/4) + 4*(lane/32) + i%4.
  const int lde = fg_lde(E);
  float* s_lg = reinterpret_cast<float*>(fsm);
  float* s_g = s_lg + FG_T * lde;
  if (active) {
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        s_lg[(r * 32 + 8 * (i >> 2) + 4 * lh + (i & 3)) * lde + wave * 32 + lr] = acc[r][i];
  }
  __syncthreads();

  // The logits rows out of LDS, consecutive threads on consecutive experts.
  if (logits_out) {
    const int rows = (int)min((int64_t)FG_T, T - t0);
    for (int i = tid; i < rows * E; i += FG_THREADS) {
      const int r = i / E, e = i - r * E;
      logits_out[(t0 + r) * E + e] = s_lg[r * lde + e];
    }
  }

  // Selection: thread q of token tk's team reads its experts' logits.
  const int tk = tid / SEL_TEAM, q = tid % SEL_TEAM;
  const int64_t t = t0 + tk;
  const bool valid = t < T;
  const int64_t tc = valid ? t : T - 1;   // rows past T: nothing is written
  const int EQ = E / SEL_TEAM, e0 = q * EQ;
  float lg[SEL_TQ];
#pragma unroll
  for (int j = 0; j < SEL_TQ; j += 4) {
    if (j < EQ) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(s_lg + tk * lde + e0 + j);
#pragma unroll
      for (int i = 0; i < 4; ++i) lg[j + i] = v[i];
    }
  }
  select_team(lg, q, valid, bias, s_g + tk * SEL_TG, E, G, TG, K, rho, idx_out + tc * K,
              w_out + tc * K);
}

}  // namespace

int gate_ksplit(int64_t T, int H, int E) {
  const int nsteps = H / GBK;
  if (H % GBK || nsteps < 1) return 1;
  const int64_t tiles = ((T + GBM - 1) / GBM) * ((gate_expert_blocks(E) + GEB - 1) / GEB);
  // Splits divide the k steps evenly, at least two steps each, so that
  // every split has work, and keep the grid within ~512 workgroups.  Small
  // batches split k finely so that the weight stream is spread over many
  // CUs: the power-of-two count that reaches ~512 workgroups, or more (up to
  // 64) while the partial sums written and re-read (ks T E fp32) stay below
  // the split weight's 6 E H bytes.
  auto ok = [&](int c) { return nsteps % c == 0 && nsteps / c >= 2 && tiles * c <= 512; };
  int ks = 1;
  while (ks < 32 && ok(ks * 2)) ks *= 2;
  for (int c = ks + 1; c <= 64; ++c)
    if (ok(c) && (int64_t)c * T * 4 <= (int64_t)H * 6) ks = c;
  return ks;
}

int gate_expert_blocks(int E) { return (E + 31) / 32; }

size_t gate_split_bytes(int H, int E) {
  return (size_t)gate_expert_blocks(E) * (H / GBK) * GFRAG * sizeof(u32x4);
}

hipError_t launch_gate_logits(const void* x, bool x_bf16, const float* gate_w, void* wsplit,
                              float* partials, int64_t T, int H, int E, int ksplit,
                              hipStream_t s) {
  if (x_bf16) {
    const int neb = gate_expert_blocks(E);
    const int64_t nslot = (int64_t)neb * (H / GBK) * 256;
    MOE_TIMED_LAUNCH(s, "gate_split_kernel",
      hipLaunchKernelGGL(gate_split_kernel, dim3((unsigned)((nslot + 255) / 256)), dim3(256), 0,
                         s, gate_w, (u32x4*)wsplit, E, H, nslot));
    const int nsteps = H / GBK;
    const int spk = (nsteps + ksplit - 1) / ksplit;
    dim3 grid((unsigned)((T + GBM - 1) / GBM), (neb + GEB - 1) / GEB, ksplit);
    MOE_TIMED_LAUNCH(s, "gate_logits_bf16_kernel",
      hipLaunchKernelGGL(gate_logits_bf16_kernel, grid, dim3(GTHREADS), 0, s,
                         (const uint16_t*)x, (const u32x4*)wsplit, partials, T, H, E, neb, spk));
  } else {
    dim3 grid((unsigned)((T + 15) / 16), (E + 15) / 16);
    MOE_TIMED_LAUNCH(s, "gate_logits_f32_kernel",
      hipLaunchKernelGGL(gate_logits_f32_kernel, grid, dim3(256), 0, s, (const float*)x, gate_w,
                         partials, T, H, E));
  }
  return hipGetLastError();
}

namespace {
std::atomic<int> g_gate_mode{0};   // 0 split kernels, 1 fused whenever the shape allows
}  // namespace

void set_gate_mode(int mode) { g_gate_mode.store(mode); }
int gate_mode() { return g_gate_mode.load(); }

bool gate_fused_shape_ok(int H, int E, int G, int TG, int K) {
  return H % GBK == 0 && H >= GBK && E <= 32 * FG_WAVES && select_team_ok(E, G, TG, K);
}

// The split kernels are the default at every batch size: at T = 16384 on
// an MI355X (one 64-token tile per compute unit) the fused kernel takes
// about 0.28 ms against 0.26 ms for the k-split gate plus the selection,
// because a workgroup that holds all experts of its tokens can hold only 64
// of them, which doubles the weight bytes each MFMA is fed from L2.
bool gate_use_fused(int64_t T, int H, int E, int G, int TG, int K) {
  return g_gate_mode.load() == 1 && T >= 1 && gate_fused_shape_ok(H, E, G, TG, K);
}

hipError_t launch_gate_select_fused(const uint16_t* x, const float* gate_w, void* wsplit,
                                    const float* bias, float* logits_out, int32_t* idx,
                                    float* w, int64_t T, int H, int E, int G, int TG, int K,
                                    float rho, hipStream_t s) {
  static hipError_t attr = hipFuncSetAttribute((const void*)gate_select_fused_kernel,
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)fg_lds_bytes(32 * FG_WAVES));
  if (attr != hipSuccess) return attr;
  const int neb = gate_expert_blocks(E);
  const int64_t nslot = (int64_t)neb * (H / GBK) * 256;
  MOE_TIMED_LAUNCH(s, "gate_split_kernel",
    hipLaunchKernelGGL(gate_split_kernel, dim3((unsigned)((nslot + 255) / 256)), dim3(256), 0, s,
                       gate_w, (u32x4*)wsplit, E, H, nslot));
  MOE_TIMED_LAUNCH(s, "gate_select_fused_kernel",
    hipLaunchKernelGGL(gate_select_fused_kernel, dim3((unsigned)((T + FG_T - 1) / FG_T)),
                       dim3(FG_THREADS), fg_lds_bytes(E), s, (const uint16_t*)x,
                       (const u32x4*)wsplit, bias, logits_out, idx, w, T, H, E, G, TG, K, rho));
  return hipGetLastError();
}

hipError_t launch_select(const float* partials, int ksplit, const float* bias, float* logits_out,
                         int32_t* idx, float* w, int64_t T, int E, int G, int TG, int K,
                         float rho, hipStream_t s) {
  if (ksplit >= SEL_DEEP) {
    MOE_TIMED_LAUNCH(s, "select_kernel",
      hipLaunchKernelGGL(select_kernel<SEL_WAVES>, dim3((unsigned)T), dim3(SEL_WAVES * 64), 0, s,
                         partials, ksplit, bias, logits_out, idx, w, T, E, G, TG, K, rho));
  } else {
    dim3 grid((unsigned)((T + SEL_WAVES - 1) / SEL_WAVES));
    MOE_TIMED_LAUNCH(s, "select_kernel",
      hipLaunchKernelGGL(select_kernel<1>, grid, dim3(SEL_WAVES * 64), 0, s, partials, ksplit,
                         bias, logits_out, idx, w, T, E, G, TG, K, rho));
  }
  return hipGetLastError();
}

}  // namespace moe
