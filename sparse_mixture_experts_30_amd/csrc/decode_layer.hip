// The whole MoE layer of a decode batch (1 <= T <= 32 tokens) in one
// launch (gfx950): gate -> selection -> permutation and tile list -> routed
// and shared expert GEMMs -> combine.
//
// The steps are those of the layer (page "从 1024 块 GPU 到 558 万美元：拆解 DeepSeek-V3
// 的算法-系统协同设计", sections 2.2 and 2.3; the decode batch of about 32 tokens
// and the overlap of the always-active shared expert with the routed ones
// follow "深入理解 DeepSeek-V3：大规模缩放挑战与对 AI 架构硬件的反思（中文精读）", section
// 3.1).  A decode batch is too small to fill the GPU with any one step, and
// its time is the weight stream of the active experts; what a single launch
// adds is that nothing waits for a kernel boundary:
//   - the shared expert's two GEMMs need only x, so they stream their
//     weights from the first moment, under the gate and the routing;
//   - a routed expert's down projection starts as soon as that expert's
//     gate/up projection is complete, while other experts are still in
//     their first GEMM;
//   - a token's combine starts as soon as its experts' outputs are written.
//
// Roles, by workgroup index (512 threads = 8 waves each):
//   [0, wg_sel)           gate items (two per workgroup, four waves each):
//                         32 experts x one k range, as the decode gate
//   [wg_sel, wg_router)   selection, as the selection kernel: eight tokens
//                         per workgroup, or two (four waves per token) when
//                         the gate has 16 k ranges or more
//   wg_router             the stable permutation and the routed tile list
//   [wg_sh1, wg_sh2)      shared expert GEMM1, eight wave slots each
//   [wg_sh2, wg_r1)       shared expert GEMM2
//   [wg_r1, wg_r2)        routed GEMM1 (sized for the most groups the batch
//                         can have; slots past the tile list do nothing)
//   [wg_r2, wg_comb)      routed GEMM2
//   [wg_comb, wg_end)     one token's combine each
//
// Hand-offs.  A workgroup waits only for workgroups with a lower index,
// which the hardware dispatches first, so every wait ends; each wait is also
// bounded (a timeout sets bit 2 of the device error flag and the workgroup
// goes on without the data it waited for).  A workgroup signals completion
// with one 64-bit flag set to this call's key (never reused, so flags left
// by earlier calls or never written read as "not done"; under graph capture
// the key comes from a device counter that a one-thread kernel advances
// ahead of the layer): every wave drains its stores, the workgroup meets at
// a barrier, and one wave fences (release, agent scope: the L2 write-back
// that makes the stores visible to the other XCDs) and sets the flag.  A
// consumer workgroup polls with one wave, which fences (acquire) before the
// workgroup's barrier.  Agent-scope fences are serialised across the GPU
// (about 9 ns each under load, measured), so they are taken once per
// workgroup, not per wave; the polls sleep between reads.  The routing flag,
// which every GEMM workgroup polls, is written in 32 copies 4 KiB apart so
// that the polls spread over the memory channels, and holds key + 1 + the
// length of the routed tile list, so that the GEMM workgroups past the list
// (the grid is sized for the most groups a batch can have) leave without a
// fence.
//
// The arithmetic of every step is the one of the multi-launch decode path
// (same gate items, same split-order sum of the gate's k ranges, same
// selection, permutation, GEMM wave slots and combine), so both give the
// same bits.
#include "moe_internal.hpp"
#include "combine_device.hpp"
#include "decode_device.hpp"
#include "packed_few.hpp"
#include "permute_device.hpp"
#include "select_device.hpp"

#include <algorithm>
#include <atomic>

namespace moe {

namespace {

constexpr int LT = 512;              // threads per workgroup
constexpr int LW = LT / kWave;       // waves per workgroup
constexpr int kSpinMax = 1 << 16;    // polls before a wait gives up (~0.1 s)
constexpr int kRouteCopies = 32;     // copies of the routing flag
constexpr int kRouteStride = 512;    // ... this many flags (4 KiB) apart

// Workgroup counts and flag offsets (in 64-bit flags) of one launch.
struct Plan {
  int ks, kchunk, neb, ngate, sel_tpw, maxg, nt1, nt1s, nt2;
  int s1, s1s, s2;                   // wave slots: routed GEMM1 per group, shared GEMM1, GEMM2
  int wg_sel, wg_router, wg_sh1, wg_sh2, wg_r1, wg_r2, wg_comb, wg_end;
  int64_t f_epoch, f_gate, f_sel, f_route, f_sh1, f_sh2, f_r1, f_r2, f_gtile, f_total;
};

Plan make_plan(int64_t T, int H, int E, int K, int I, int Is) {
  Plan p{};
  p.ks = decode_ksplit(H, E);
  p.kchunk = ((H + p.ks - 1) / p.ks + 7) / 8 * 8;
  p.neb = (E + 31) / 32;
  p.ngate = p.neb * p.ks;
  p.sel_tpw = p.ks >= SEL_DEEP ? LW / SEL_PARTS : LW;
  p.maxg = (int)std::min<int64_t>(E, T * K);
  p.nt1 = (I + 127) / 128;
  p.nt1s = (Is + 127) / 128;
  p.nt2 = (H + 255) / 256;
  p.s1 = p.nt1 * kFewSlots;
  p.s1s = Is > 0 ? p.nt1s * kFewSlots : 0;
  p.s2 = p.nt2 * kFewSlots;
  auto wgs = [](int64_t slots) { return (int)((slots + LW - 1) / LW); };
  p.wg_sel = (p.ngate + 1) / 2;
  p.wg_router = p.wg_sel + (int)((T + p.sel_tpw - 1) / p.sel_tpw);
  p.wg_sh1 = p.wg_router + 1;
  p.wg_sh2 = p.wg_sh1 + wgs(p.s1s);
  p.wg_r1 = p.wg_sh2 + (Is > 0 ? wgs(p.s2) : 0);
  p.wg_r2 = p.wg_r1 + wgs((int64_t)p.maxg * p.s1);
  p.wg_comb = p.wg_r2 + wgs((int64_t)p.maxg * p.s2);
  p.wg_end = p.wg_comb + (int)T;
  // [epoch][gate WGs][selection WGs][route copies][shared GEMM1 / GEMM2 WGs]
  // [routed GEMM1 / GEMM2 WGs][tile index of each expert: E int32]
  int64_t o = 0;
  p.f_epoch = o++;
  p.f_gate = o;
  o += p.wg_sel;
  p.f_sel = o;
  o += p.wg_router - p.wg_sel;
  o = (o + kRouteStride - 1) / kRouteStride * kRouteStride;
  p.f_route = o;
  o += (int64_t)kRouteCopies * kRouteStride;
  p.f_sh1 = o;
  o += p.wg_sh2 - p.wg_sh1;
  p.f_sh2 = o;
  o += p.wg_r1 - p.wg_sh2;
  p.f_r1 = o;
  o += p.wg_r2 - p.wg_r1;
  p.f_r2 = o;
  o += p.wg_comb - p.wg_r2;
  p.f_gtile = o;
  o += (E + 1) / 2;
  p.f_total = o;
  return p;
}

struct LayerArgs {
  Plan p;
  int T, H, E, G, TG, K, I, Is;
  float rho;
  const uint16_t* x;
  const float* gate_w;
  const float* bias;
  float* part;                       // [ks][T][E]
  float* logits;                     // nullable
  int32_t* idx;
  float* w;
  int32_t *counts, *offsets, *perm, *pos, *err, *tiles;
  PackedArgs g1, g2;                 // GEMM1 / GEMM2 (tiles: the routed list)
  uint16_t* out;
  uint64_t* flags;
  uint64_t key;                      // this call's key, unless epoch is set
  const uint64_t* epoch;             // under graph capture: key from this counter
};

struct GateLds {
  float red[2][3][16][kWave];
};
struct SelectLds {
  float s_c[LW][512];
  float s_s[LW][512];
};
struct RouteLds {
  PermuteLds<LT> perm;
  int32_t count;                     // entries of the tile list
};
struct CombineLds {
  int32_t sp[64];
  float sw[64];
};
union LayerLds {
  GateLds gate;
  SelectLds sel;
  RouteLds route;
  CombineLds comb;
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// The calling wave waits until f[0 .. n) all hold key, then fences
// (acquire, agent scope).  Bounded: returns false on timeout.
__device__ __forceinline__ bool wave_wait(const uint64_t* f, int n, uint64_t key) {
  const int lane = lane_id();
  for (int it = 0; it < kSpinMax; ++it) {
    bool ok = true;
    for (int i = lane; i < n; i += kWave)
      ok = ok && __hip_atomic_load(f + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == key;
    if (__ballot(!ok) == 0) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      return true;
    }
    __builtin_amdgcn_s_sleep(8);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return false;
}

// The workgroup waits for f[0 .. n): wave 0 polls and fences, the others
// meet it at the barrier.  Every thread calls it; all get the result.
__device__ __forceinline__ bool wg_wait(const uint64_t* f, int n, uint64_t key) {
  bool ok = true;
  if (threadIdx.x < kWave) ok = wave_wait(f, n, key);
  return __syncthreads_and(ok);
}

// Every wave's stores drained, a barrier, then wave 0 writes the L2 back
// (release, agent scope) and sets the flag.  Every thread calls it.
__device__ __forceinline__ void wg_publish(uint64_t* f, uint64_t key) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x < kWave) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    if (lane_id() == 0) __hip_atomic_store(f, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The routing flag holds key + 1 + the number of routed tile list entries,
// so a workgroup learns how many entries there are without a fence and one
// with nothing to do leaves at once.  The calling wave polls its copy of the
// flag; with `fence` it then fences (acquire) to read what the router
// wrote.  Returns the count, or -1 on timeout.
__device__ __forceinline__ int route_wait(const LayerArgs& a, uint64_t key, bool fence) {
  const uint64_t* f = a.flags + a.p.f_route + (int64_t)(blockIdx.x % kRouteCopies) * kRouteStride;
  for (int it = 0; it < kSpinMax; ++it) {
    const uint64_t d =
        __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - key - 1;
    if (d <= (uint64_t)PMAXE) {
      if (fence) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      return (int)d;
    }
    __builtin_amdgcn_s_sleep(8);
  }
  return -1;
}

// The workgroup's route_wait: wave 0 polls, and fences when
// first_slot < slots_per_entry x the count (a GEMM1 workgroup with work; a
// combine passes -1 and 0); the count is broadcast through LDS.  Every
// thread calls it.
__device__ __forceinline__ int wg_route_wait(const LayerArgs& a, uint64_t key,
                                             int first_slot, int slots_per_entry,
                                             int32_t& bcast) {
  if (threadIdx.x < kWave) {
    int n = route_wait(a, key, false);
    if (n >= 0 && first_slot < n * slots_per_entry) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (lane_id() == 0) bcast = n;
  }
  __syncthreads();
  return bcast;
}

// Bit 2 of the device error flag after a timed-out wait.  The router
// rewrites the flag (its bit 1) once per call, so a wave that is not
// ordered after the router first waits for it (bounded too).
__device__ __forceinline__ void report_timeout(const LayerArgs& a, uint64_t key,
                                               bool after_route) {
  if (!after_route) route_wait(a, key, false);
  if (lane_id() == 0) atomicOr(a.err, 2);
}

__device__ __forceinline__ void gate_role(const LayerArgs& a, uint64_t key, int b,
                                          GateLds& L) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int item = 2 * b + (wave >> 2);
  const bool valid = item < a.p.ngate;
  const int eb = item % a.p.neb, ks = item / a.p.neb;
  gate_mfma_item(a.x, a.gate_w, a.part, a.T, a.H, a.E, a.p.kchunk, eb, ks, wave & 3, valid,
                 L.red[wave >> 2]);
  wg_publish(a.flags + a.p.f_gate + b, key);
}

// Selection of sel_tpw tokens (the batch selection kernel's arithmetic).
// Up to SEL_DEEP k ranges: one wave per token sums every range in order.
// Deeper: four waves per token sum contiguous parts of the ranges, the parts
// are added in wave order through LDS, and the first of them selects.
__device__ __forceinline__ void select_role(const LayerArgs& a, uint64_t key, int b,
                                            SelectLds& L) {
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool deep = a.p.ks >= SEL_DEEP;
  const int t = b * a.p.sel_tpw + (deep ? wave / SEL_PARTS : wave);
  const int q = deep ? wave % SEL_PARTS : 0;
  const int E = a.E;
  const bool ok = wg_wait(a.flags + a.p.f_gate, a.p.wg_sel, key);
  float lgs[SEL_MAXV];
  if (t < a.T)
    sum_splits(a.part, (int64_t)a.T * E, t, E, lane, deep ? sel_part_begin(a.p.ks, q) : 0,
               deep ? sel_part_begin(a.p.ks, q + 1) : a.p.ks, lgs);
  if (deep) {
    const int V = (E + 63) / 64;
    if (t < a.T) {
#pragma unroll
      for (int v = 0; v < SEL_MAXV; ++v) {
        const int e = lane + 64 * v;
        if (v < V && e < E) L.s_c[wave][e] = lgs[v];
      }
    }
    __syncthreads();
    if (q == 0 && t < a.T) {
#pragma unroll
      for (int v = 0; v < SEL_MAXV; ++v) {
        const int e = lane + 64 * v;
        if (v < V && e < E) {
          float acc = L.s_c[wave][e];
#pragma unroll
          for (int w = 1; w < SEL_PARTS; ++w) acc += L.s_c[wave + w][e];
          lgs[v] = acc;
        }
      }
    }
  }
  if (q == 0 && t < a.T)
    select_token(lgs, lane, a.bias, L.s_c[wave], L.s_s[wave], E, a.G, a.TG, a.K, a.rho,
                 a.logits ? a.logits + (int64_t)t * E : nullptr, a.idx + (int64_t)t * a.K,
                 a.w + (int64_t)t * a.K, nullptr);
  wg_publish(a.flags + a.p.f_sel + b, key);
  if (!ok && threadIdx.x < kWave) report_timeout(a, key, false);
}

// The stable permutation of the batch's choices, the routed tile list and
// each expert's place in it.
__device__ __forceinline__ void router_role(const LayerArgs& a, uint64_t key, RouteLds& L) {
  const int tid = threadIdx.x;
  const int E = a.E;
  const bool sel_ok = wg_wait(a.flags + a.p.f_sel, a.p.wg_router - a.p.wg_sel, key);
  block_permute<LT>(L.perm, a.idx, a.T * a.K, E, a.counts, a.offsets, a.perm, a.pos, a.err);
  // the thread that rewrote the flag adds the timeout bit
  if (tid == 0 && !sel_ok) atomicOr(a.err, 2);
  // Routed tile list (format of build_tiles_kernel): one tile per
  // non-empty group (no group has more than T <= 32 rows).
  const int g = tid;
  int32_t n = 0, r0 = 0;
  if (g < E) {
    n = L.perm.h[g];
    r0 = L.perm.s[g] - n;
  }
  const int32_t mt = n > 0 ? 1 : 0;
  const int32_t end = block_inclusive_scan<LT>(mt, L.perm.wsum);
  if (mt) {
    int32_t* ent = a.tiles + 8 + 8 * (int64_t)(end - 1);
    ent[0] = g;
    ent[1] = r0;
    ent[2] = n;
    ent[3] = end - 1;
    ent[4] = 1;
  }
  if (g < E) reinterpret_cast<int32_t*>(a.flags + a.p.f_gtile)[g] = mt ? end - 1 : -1;
  if (g == LT - 1) {
    a.tiles[0] = end;
    L.count = end;
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid < kWave) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    if (tid < kRouteCopies)
      __hip_atomic_store(a.flags + a.p.f_route + (int64_t)tid * kRouteStride,
                         key + 1 + (uint64_t)L.count,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Shared expert GEMM1 / GEMM2, workgroup b of the role: wave slots 8 b ..
__device__ __forceinline__ void shared_gemm1(const LayerArgs& a, uint64_t key, int b) {
  const int i = b * LW + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (i < a.p.s1s) few_tile<true, 1, 3>(a.g1, a.E, 0, a.T, i / kFewSlots, i % kFewSlots);
  wg_publish(a.flags + a.p.f_sh1 + b, key);
}

__device__ __forceinline__ void shared_gemm2(const LayerArgs& a, uint64_t key, int b) {
  const int i = b * LW + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool ok = wg_wait(a.flags + a.p.f_sh1, a.p.wg_sh2 - a.p.wg_sh1, key);
  if (i < a.p.s2) few_tile<false, 1, 3>(a.g2, a.E, 0, a.T, i / kFewSlots, i % kFewSlots);
  wg_publish(a.flags + a.p.f_sh2 + b, key);
  if (!ok && threadIdx.x < kWave) report_timeout(a, key, false);
}

// Routed GEMM1 / GEMM2 over the tile list, workgroup b of the role: wave
// slot i = 8 b + wave is slot i % S of the list's entry i / S.  A workgroup
// whose slots all lie past the list leaves without a flag: no consumer
// waits for it.
__device__ __forceinline__ void routed_gemm1(const LayerArgs& a, uint64_t key, int b,
                                             int32_t& bcast) {
  const int i = b * LW + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ntl = wg_route_wait(a, key, b * LW, a.p.s1, bcast);
  if (ntl < 0) {   // without the tile list there is nothing this workgroup may read
    if (threadIdx.x < kWave) report_timeout(a, key, true);
    return;
  }
  if (b * LW >= ntl * a.p.s1) return;
  const int j = i / a.p.s1;
  if (j < ntl) {
    const int32_t* ent = a.tiles + 8 + 8 * j;
    const int r = i - j * a.p.s1;
    few_tile<true, 1, 3>(a.g1, ent[0], ent[1], ent[2], r / kFewSlots, r % kFewSlots);
  }
  wg_publish(a.flags + a.p.f_r1 + b, key);
}

__device__ __forceinline__ void routed_gemm2(const LayerArgs& a, uint64_t key, int b,
                                             int32_t& bcast) {
  const int i = b * LW + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // no fence here: the wait for the GEMM1 flags below acquires what the
  // router wrote too (the GEMM1 workgroups acquired it before they
  // released their own stores)
  const int ntl = wg_route_wait(a, key, 0, 0, bcast);
  if (ntl < 0) {
    if (threadIdx.x < kWave) report_timeout(a, key, true);
    return;
  }
  if (b * LW >= ntl * a.p.s2) return;
  // the list entries of this workgroup's slots, and the GEMM1 workgroups
  // that wrote their h rows
  const int jlo = (b * LW) / a.p.s2;
  const int jhi = min((b * LW + LW - 1) / a.p.s2, ntl - 1);
  const int w0 = jlo * a.p.s1 / LW, w1 = ((jhi + 1) * a.p.s1 - 1) / LW;
  const bool ok = wg_wait(a.flags + a.p.f_r1 + w0, w1 - w0 + 1, key);
  const int j = i / a.p.s2;
  if (j < ntl) {
    const int32_t* ent = a.tiles + 8 + 8 * j;
    const int r = i - j * a.p.s2;
    few_tile<false, 1, 3>(a.g2, ent[0], ent[1], ent[2], r / kFewSlots, r % kFewSlots);
  }
  wg_publish(a.flags + a.p.f_r2 + b, key);
  if (!ok && threadIdx.x < kWave) report_timeout(a, key, true);
}

__device__ __forceinline__ void combine_role(const LayerArgs& a, uint64_t key, int t,
                                             CombineLds& L, int32_t& bcast) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // without the routing there is nothing to combine
  const int ntl = wg_route_wait(a, key, -1, 0, bcast);
  if (ntl < 0) {
    if (threadIdx.x < kWave) report_timeout(a, key, true);
    return;
  }
  // wave w waits for the GEMM2 workgroups of the token's slots k = w, w + 8,
  // ...; the last wave also for the shared expert's
  const int32_t* gtile = reinterpret_cast<const int32_t*>(a.flags + a.p.f_gtile);
  bool ok = true;
  for (int k = wave; k < a.K; k += LW) {
    const int g = a.idx[(int64_t)t * a.K + k];
    const int j = (g >= 0 && g < a.E) ? gtile[g] : -1;
    if (j >= 0 && j < ntl) {
      const int w0 = j * a.p.s2 / LW, w1 = ((j + 1) * a.p.s2 - 1) / LW;
      ok = wave_wait(a.flags + a.p.f_r2 + w0, w1 - w0 + 1, key) && ok;
    }
  }
  if (a.Is > 0 && wave == LW - 1)
    ok = wave_wait(a.flags + a.p.f_sh2, a.p.wg_r1 - a.p.wg_sh2, key) && ok;
  if (!ok) report_timeout(a, key, true);
  __syncthreads();
  combine_row_bf16<LT>(a.g2.c_r, a.Is > 0 ? a.g2.c_s : nullptr, a.pos, a.w, a.out, t, a.H,
                       a.K, (int64_t)a.T * a.K, L.sp, L.sw);
}

// Key of a call that reads it from the device (graph replays): a bijective
// mix (the splitmix64 finaliser) of the epoch counter, so successive epochs
// give distinct keys.
__device__ __forceinline__ uint64_t epoch_key(uint64_t e) {
  uint64_t z = e + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return z ? z : 1;
}

__global__ void __launch_bounds__(LT) decode_layer_kernel(LayerArgs a) {
  __shared__ LayerLds lds;
  __shared__ int32_t bcast;
  const int b = blockIdx.x;
  const uint64_t key = a.epoch ? epoch_key(*a.epoch) : a.key;
  const Plan& p = a.p;
  if (b < p.wg_sel) {
    gate_role(a, key, b, lds.gate);
  } else if (b < p.wg_router) {
    select_role(a, key, b - p.wg_sel, lds.sel);
  } else if (b == p.wg_router) {
    router_role(a, key, lds.route);
  } else if (b < p.wg_sh2) {
    shared_gemm1(a, key, b - p.wg_sh1);
  } else if (b < p.wg_r1) {
    shared_gemm2(a, key, b - p.wg_sh2);
  } else if (b < p.wg_r2) {
    routed_gemm1(a, key, b - p.wg_r1, bcast);
  } else if (b < p.wg_comb) {
    routed_gemm2(a, key, b - p.wg_r2, bcast);
  } else {
    combine_role(a, key, b - p.wg_comb, lds.comb, bcast);
  }
}

// Advances the epoch counter of a captured call (the kernel boundary orders
// it before the layer kernel that reads it).
__global__ void decode_epoch_kernel(uint64_t* e) {
  if (threadIdx.x == 0) *e = *e + 1;
}

// Keys of successive calls: a per-process random start, then a counter;
// never zero.
uint64_t next_key() {
  static std::atomic<uint64_t> counter{0};
  static const uint64_t base = [] {
    uint64_t v = (uint64_t)(uintptr_t)&counter;
    v ^= (uint64_t)__builtin_readcyclecounter() * 0x9E3779B97F4A7C15ull;
    return v;
  }();
  const uint64_t k = base + 0x9E3779B97F4A7C15ull * (counter.fetch_add(1) + 1);
  return k ? k : 1;
}

}  // namespace

bool decode_layer_ok(int64_t T, int H, int E, int K, int I, int Is) {
  static_assert(PMAXE <= LT, "one thread per expert in the tile list");
  return decode_route_ok(T, H, E, K) && H % kPackedBK == 0 && I % kPackedBK == 0 &&
         Is % kPackedBK == 0;
}

size_t decode_layer_flags_bytes(int H, int E, int K, int I, int Is) {
  // the plan of the largest batch has the most workgroups
  return (size_t)make_plan(kDecodeMaxT, H, E, K, I, Is).f_total * sizeof(uint64_t);
}

hipError_t launch_decode_layer(const uint16_t* x, const float* gate_w, const float* bias,
                               const void* w13p, const void* w2p, const void* ws13p,
                               const void* ws2p, int64_t T, int H, int E, int G, int TG, int K,
                               int I, int Is, float rho, float* partials, float* logits,
                               int32_t* idx, float* w, int32_t* counts, int32_t* offsets,
                               int32_t* perm, int32_t* pos, int32_t* err, int32_t* tiles,
                               uint16_t* h, uint16_t* y, uint16_t* ys, uint16_t* out,
                               void* flags, hipStream_t s) {
  if (T < 1 || T > kDecodeMaxT) return hipErrorInvalidValue;
  LayerArgs a{};
  a.p = make_plan(T, H, E, K, I, Is);
  if (a.p.kchunk > DG_MAXK) return hipErrorInvalidValue;
  a.T = (int)T;
  a.H = H;
  a.E = E;
  a.G = G;
  a.TG = TG;
  a.K = K;
  a.I = I;
  a.Is = Is;
  a.rho = rho;
  a.x = x;
  a.gate_w = gate_w;
  a.bias = bias;
  a.part = partials;
  a.logits = logits;
  a.idx = idx;
  a.w = w;
  a.counts = counts;
  a.offsets = offsets;
  a.perm = perm;
  a.pos = pos;
  a.err = err;
  a.tiles = tiles;
  const int64_t N = T * K;
  PackedArgs& g1 = a.g1;
  g1.tiles = tiles;
  g1.ntn = std::max(a.p.nt1, a.p.nt1s);
  g1.E = E;
  g1.K = K;
  g1.a_r = g1.a_s = x;
  g1.lda_r = g1.lda_s = H;
  g1.perm = perm;
  g1.kdim_r = g1.kdim_s = H;
  g1.b_r = (const u32x4*)w13p;
  g1.nt_r = a.p.nt1;
  g1.b_s = (const u32x4*)ws13p;
  g1.nt_s = a.p.nt1s;
  g1.ncol_r = I;
  g1.ncol_s = Is;
  g1.c_r = h;
  g1.c_s = h + N * I;
  g1.ldc_r = I;
  g1.ldc_s = Is;
  PackedArgs& g2 = a.g2;
  g2.tiles = tiles;
  g2.ntn = a.p.nt2;
  g2.E = E;
  g2.K = K;
  g2.a_r = h;
  g2.a_s = h + N * I;
  g2.lda_r = I;
  g2.lda_s = Is;
  g2.perm = nullptr;
  g2.kdim_r = I;
  g2.kdim_s = Is;
  g2.b_r = (const u32x4*)w2p;
  g2.nt_r = a.p.nt2;
  g2.b_s = (const u32x4*)ws2p;
  g2.nt_s = a.p.nt2;
  g2.ncol_r = g2.ncol_s = H;
  g2.c_r = y;
  g2.c_s = ys;
  g2.ldc_r = g2.ldc_s = H;
  a.out = out;
  a.flags = (uint64_t*)flags;
  // A key passed as an argument would be replayed unchanged by a captured
  // graph, and a replay would then take the flags of the one before for its
  // own: under capture the key comes from a device counter that a one-thread
  // kernel advances before each replay of the layer.
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(s, &cap);
  if (e != hipSuccess) return e;
  a.key = next_key();
  a.epoch = nullptr;
  if (cap != hipStreamCaptureStatusNone) {
    uint64_t* epoch = a.flags + a.p.f_epoch;
    a.epoch = epoch;
    MOE_TIMED_LAUNCH(s, "decode_epoch_kernel",
      hipLaunchKernelGGL(decode_epoch_kernel, dim3(1), dim3(64), 0, s, epoch));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  MOE_TIMED_LAUNCH(s, "decode_layer_kernel",
    hipLaunchKernelGGL(decode_layer_kernel, dim3((unsigned)a.p.wg_end), dim3(LT), 0, s, a));
  return hipGetLastError();
}

}  // namespace moe
