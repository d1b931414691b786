// Internal declarations shared by the HIP sources of libmoe (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------- vector types
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kNumXcd = 8;  // MI355X: 8 XCDs, workgroups dispatched round-robin

// ---------------------------------------------------------------- scalar helpers
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  return __builtin_bit_cast(bf16x8, v);
}
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

// 16-byte streaming load (non-temporal: data read once, not kept in cache).
__device__ __forceinline__ u32x4 load_stream16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Map a linear workgroup id onto a work index so that each XCD receives one
// contiguous range of the work list (consecutive ids go to different XCDs).
// `nb` is the grid size (a multiple of kNumXcd).
__device__ __forceinline__ int xcd_contiguous(int b, int nb) {
  int per = nb / kNumXcd;
  return (b % kNumXcd) * per + b / kNumXcd;
}

// Work item of workgroup b when chunks of kXcdChunk consecutive items go to
// the XCDs in turn (chunk c to XCD c % kNumXcd).  Each XCD then gets an even
// share of every part of a grouped GEMM's work list (the shared expert's
// heavy tiles at its end included), while the neighbouring items of a chunk
// (M-tiles that share a weight tile, N-tiles that share a group's rows) stay
// on one XCD and its L2.  The grid is a multiple of kXcdGrid (xcd_grid);
// returns -1 for the surplus workgroups past `work`.
constexpr int kXcdChunk = 16;
constexpr int64_t kXcdGrid = (int64_t)kNumXcd * kXcdChunk;
__device__ __forceinline__ int64_t xcd_chunked(int64_t b, int64_t work) {
  const int64_t q = b / kNumXcd;
  const int64_t w = ((q / kXcdChunk) * kNumXcd + b % kNumXcd) * kXcdChunk + q % kXcdChunk;
  return w < work ? w : -1;
}
inline unsigned xcd_grid(int64_t max_work) {
  return (unsigned)(((max_work + kXcdGrid - 1) / kXcdGrid) * kXcdGrid);
}

// ---------------------------------------------------------------- kernel timer
// Brackets one kernel launch with HIP events on its stream while the timer
// (moe_kernel_timer_enable) is on; `name` must be a string literal.
class KernelTimerScope {
 public:
  KernelTimerScope(hipStream_t s, const char* name);
  ~KernelTimerScope();
  KernelTimerScope(const KernelTimerScope&) = delete;
  KernelTimerScope& operator=(const KernelTimerScope&) = delete;

 private:
  hipStream_t s_;
  const char* name_;
  void* begin_ = nullptr;
};

#define MOE_TIMED_LAUNCH(stream, name, ...)             \
  do {                                                  \
    ::moe::KernelTimerScope moe_timer_scope_((stream), (name)); \
    __VA_ARGS__;                                        \
  } while (0)

// ---------------------------------------------------------------- host launchers

// Gate: the fp32 weight is split into three bf16 parts in `wsplit`
// (gate_split_bytes) and multiplied on bf16 MFMA; partials [ksplit, T, E].
hipError_t launch_gate_logits(const void* x, bool x_bf16, const float* gate_w, void* wsplit,
                              float* partials, int64_t T, int H, int E, int ksplit,
                              hipStream_t s);
int gate_expert_blocks(int E);
size_t gate_split_bytes(int H, int E);
int gate_ksplit(int64_t T, int H, int E);
hipError_t launch_select(const float* partials, int ksplit, const float* bias, float* logits_out,
                         int32_t* idx, float* w, int64_t T, int E, int G, int TG, int K,
                         float rho, hipStream_t s);
// Gate and selection in one launch (bf16 tokens): no partial sums in memory.
// gate_use_fused: the gate mode asks for it (set_gate_mode: 0 split, 1
// fused) and the shape allows it.
bool gate_fused_shape_ok(int H, int E, int G, int TG, int K);
bool gate_use_fused(int64_t T, int H, int E, int G, int TG, int K);
void set_gate_mode(int mode);
int gate_mode();
hipError_t launch_gate_select_fused(const uint16_t* x, const float* gate_w, void* wsplit,
                                    const float* bias, float* logits_out, int32_t* idx,
                                    float* w, int64_t T, int H, int E, int G, int TG, int K,
                                    float rho, hipStream_t s);

// Decode routing (decode.hip): gate, selection, permutation and the tile
// list of the expert GEMMs in three launches, for 1 <= T <= kDecodeMaxT.
constexpr int kDecodeMaxT = 32;
bool decode_route_ok(int64_t T, int H, int E, int K);
int decode_ksplit(int H, int E);   // partial sums [ksplit, T, E] in `partials`
hipError_t launch_decode_route(const void* x, bool x_bf16, const float* gate_w,
                               const float* bias, float* partials, float* logits_out,
                               int32_t* idx, float* w, int64_t T, int H, int E, int G, int TG,
                               int K, float rho, int32_t* counts, int32_t* offsets,
                               int32_t* perm, int32_t* pos, int32_t* err, int32_t* tiles,
                               bool has_routed, bool has_shared, hipStream_t s);

// The whole decode layer in one launch (decode_layer.hip): bf16 tokens and
// packed bf16 weights, 1 <= T <= kDecodeMaxT; flags: a workspace region of
// decode_layer_flags_bytes (no initial contents needed).
bool decode_layer_ok(int64_t T, int H, int E, int K, int I, int Is);
size_t decode_layer_flags_bytes(int H, int E, int K, int I, int Is);
hipError_t launch_decode_layer(const uint16_t* x, const float* gate_w, const float* bias,
                               const void* w13p, const void* w2p, const void* ws13p,
                               const void* ws2p, int64_t T, int H, int E, int G, int TG, int K,
                               int I, int Is, float rho, float* partials, float* logits,
                               int32_t* idx, float* w, int32_t* counts, int32_t* offsets,
                               int32_t* perm, int32_t* pos, int32_t* err, int32_t* tiles,
                               uint16_t* h, uint16_t* y, uint16_t* ys, uint16_t* out,
                               void* flags, hipStream_t s);

int permute_nblk(int64_t N);
hipError_t launch_permute(const int32_t* idx, int64_t N, int E, int32_t* hist, int32_t* counts,
                          int32_t* offsets, int32_t* perm, int32_t* pos, int32_t* err,
                          hipStream_t s);

// Expert FFN tile schedule (see ffn_sched.hip for the entry format).  The
// smallest M-tile height any GEMM uses sizes the list in the workspace.
constexpr int kMinTileRows = 128;
// Tile height of the few-row kernels of batches of at most 64 tokens.
inline int ffn_list_tile_rows(int64_t T) { return T <= 32 ? 32 : T <= 64 ? 64 : kMinTileRows; }
// Groups of an expert-FFN launch: the routed experts, the shared expert.
constexpr int kGroupRouted = 1, kGroupShared = 2, kGroupsAll = 3;
int64_t ffn_max_mtiles(int64_t N, int64_t T, int E, int BM);
// balanced: a group's M-tiles get equal row counts (+-1) instead of full
// tiles and a remainder.
hipError_t launch_build_tiles(const int32_t* offsets, int E, int64_t T, bool has_routed,
                              bool has_shared, int BM, int32_t* tiles, hipStream_t s,
                              bool balanced = false);

// Work item w (0 <= w < tiles[0] * ntn) of a grouped GEMM with ntn N-tiles:
// returns the M-tile entry and the N-tile.  Inside a group the N-tile index
// is the slow one, so workgroups that run together on one XCD share one
// weight slice across the group's M-tiles.
__device__ __forceinline__ const int32_t* decode_work(const int32_t* tiles, int64_t w, int ntn,
                                                      int& ntile) {
  const int64_t i0 = w / ntn;
  const int32_t* e0 = tiles + 8 + 8 * i0;
  const int32_t L = e0[3], mt = e0[4];
  const int64_t local = w - (int64_t)L * ntn;
  ntile = (int)(local / mt);
  return tiles + 8 + 8 * (int64_t)(L + local % mt);
}

// Expert FFN plans: the GEMMs.
struct FfnDims {
  int64_t T;       // tokens
  int64_t N;       // routed rows T*K
  int H, I, Is, E, K;
  int groups = kGroupsAll;   // which groups the launch computes
  bool tiles_ready = false;  // the tile list is already built (decode routing)
};
size_t ffn_tiles_bytes(const FfnDims& d);
// M-tiles a launch over d's groups can have (sizes its grid).
int64_t ffn_grid_mtiles(const FfnDims& d, int BM);
// The tile list of d's groups with M-tiles of BM rows, unless d says it is
// ready and no group can exceed one tile (T <= BM).
hipError_t ffn_build_tiles(const FfnDims& d, const int32_t* offsets, int BM, int32_t* tiles,
                           hipStream_t s, bool balanced = false);
hipError_t launch_ffn_bf16(const FfnDims& d, const uint16_t* x, const int32_t* perm,
                           const int32_t* offsets, const uint16_t* w13, const uint16_t* w2,
                           const uint16_t* ws13, const uint16_t* ws2, uint16_t* h,
                           int32_t* tiles, uint16_t* y, uint16_t* ys, hipStream_t s);
// [g u] = x_rows W13^T in fp32 (routed rows in expert order, row stride
// ldgu; the shared expert's T rows at gus, stride ldgus), with the
// row-major GEMM1 of ffn_bf16.hip.
hipError_t launch_gate_up_bf16(const FfnDims& d, const uint16_t* x, const int32_t* perm,
                               const int32_t* offsets, const uint16_t* w13, const uint16_t* ws13,
                               int32_t* tiles, float* gu, int64_t ldgu, float* gus,
                               int64_t ldgus, hipStream_t s);
// Packed weight layout (ffn_bf16_packed.hip).
size_t packed_bytes(bool gate_up, int64_t experts, int n, int kd);
hipError_t launch_pack(bool gate_up, const uint16_t* src, void* dst, int64_t experts, int n,
                       int kd, hipStream_t s);
hipError_t launch_ffn_bf16_packed(const FfnDims& d, const uint16_t* x, const int32_t* perm,
                                  const int32_t* offsets, const void* w13p, const void* w2p,
                                  const void* ws13p, const void* ws2p, uint16_t* h,
                                  int32_t* tiles, uint16_t* y, uint16_t* ys, hipStream_t s);
hipError_t launch_ffn_f32(const FfnDims& d, const float* x, const int32_t* perm,
                          const int32_t* offsets, const float* w13, const float* w2,
                          const float* ws13, const float* ws2, float* h, float* y, float* ys,
                          hipStream_t s);
// Packed fp8 weight layout (ffn_fp8_packed.hip).
size_t packed8_bytes(bool gate_up, int64_t experts, int n, int kd);
hipError_t launch_pack8(bool gate_up, const uint8_t* src, void* dst, int64_t experts, int n,
                        int kd, hipStream_t s);
hipError_t launch_ffn_fp8_packed(const FfnDims& d, const uint8_t* xq, const float* xs,
                                 const int32_t* perm, const int32_t* offsets, const void* w13p,
                                 const float* w13s, const void* w2p, const float* w2s,
                                 const void* ws13p, const float* ws13s, const void* ws2p,
                                 const float* ws2s, uint8_t* hq, float* hs, int32_t* tiles,
                                 uint16_t* y, uint16_t* ys, hipStream_t s);
// 1x128 e4m3 quantisation of bf16 rows; pow2: power-of-two scales.
hipError_t launch_quant_rows(const uint16_t* x, int64_t rows, int cols, uint8_t* q, float* sc,
                             bool pow2, hipStream_t s);
// e4m3 weights (packed) and activations with power-of-two block scales,
// applied by the matrix cores (ffn_fp8_mx.hip).
hipError_t launch_ffn_fp8_mx(const FfnDims& d, const uint8_t* xq, const float* xs,
                             const int32_t* perm, const int32_t* offsets, const void* w13p,
                             const float* w13s, const void* w2p, const float* w2s,
                             const void* ws13p, const float* ws13s, const void* ws2p,
                             const float* ws2s, uint8_t* hq, float* hs, int32_t* tiles,
                             uint16_t* y, uint16_t* ys, hipStream_t s);
hipError_t launch_ffn_fp8(const FfnDims& d, const uint8_t* xq, const float* xs,
                          const int32_t* perm, const int32_t* offsets, const uint8_t* w13,
                          const float* w13s, const uint8_t* w2, const float* w2s,
                          const uint8_t* ws13, const float* ws13s, const uint8_t* ws2,
                          const float* ws2s, uint8_t* hq, float* hs, int32_t* tiles,
                          uint16_t* y, uint16_t* ys, hipStream_t s);

hipError_t launch_combine(const void* y, const void* ys, const int32_t* pos, const float* w,
                          void* out, int64_t T, int H, int K, bool bf16, hipStream_t s);

// Backward of the grouped SwiGLU expert FFN (ffn_backward.hip): row-major
// bf16 weights; dy/dys are the gradients of the expert output rows (routed
// rows in expert-sorted order, then the shared expert's T rows).
size_t ffn_backward_ws_bytes(const FfnDims& d);
hipError_t launch_ffn_backward(const FfnDims& d, const uint16_t* x, const int32_t* perm,
                               const int32_t* offsets, const uint16_t* w13, const uint16_t* w2,
                               const uint16_t* ws13, const uint16_t* ws2, const uint16_t* dy,
                               const uint16_t* dys, uint16_t* dx, uint16_t* dxs, uint16_t* dw13,
                               uint16_t* dw2, uint16_t* dws13, uint16_t* dws2, void* ws,
                               hipStream_t s);

// FP8 backward of the expert FFNs (ffn_backward_fp8.hip): row-major e4m3
// weights with fp32 128x128 block scales; pow2 selects power-of-two
// activation and gradient scales.  Outputs as launch_ffn_backward's.
size_t ffn_backward_fp8_ws_bytes(const FfnDims& d);
hipError_t launch_ffn_backward_fp8(const FfnDims& d, bool pow2, const uint16_t* x,
                                   const int32_t* perm, const int32_t* offsets,
                                   const uint8_t* w13, const float* w13s, const uint8_t* w2,
                                   const float* w2s, const uint8_t* ws13, const float* ws13s,
                                   const uint8_t* ws2, const float* ws2s, const uint16_t* dy,
                                   const uint16_t* dys, uint16_t* dx, uint16_t* dxs,
                                   uint16_t* dw13, uint16_t* dw2, uint16_t* dws13,
                                   uint16_t* dws2, void* ws, hipStream_t s);


// Selection-bias update from per-expert counts (one workgroup, E <= 512).
hipError_t launch_bias_update(const int32_t* counts, float* bias, int E, float gamma,
                              hipStream_t s);

}  // namespace moe
