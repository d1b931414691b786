// C ABI of libmoe: argument validation, workspace layout and launch order.
// Every check happens on the host before anything is enqueued.
#include "moe.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "moe_internal.hpp"
#include "backward.hpp"

namespace {

thread_local char g_msg[512] = "";

moe_status fail(moe_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return s;
}

moe_status hip_fail(hipError_t e, const char* where) {
  return fail(MOE_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
inline size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// e4m3 weights, with block scales a / 448 or powers of two.
bool is_fp8(moe_dtype w) { return w == MOE_FP8_E4M3 || w == MOE_FP8_E4M3_E8M0; }

// Shape checks shared by every entry point.
moe_status check_cfg(const moe_config* c) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "cfg is NULL");
  const int H = c->hidden_size, E = c->n_routed_experts, G = c->n_group, TG = c->topk_group,
            K = c->num_experts_per_tok, I = c->moe_intermediate_size,
            Is = c->shared_intermediate_size;
  if (H <= 0 || E <= 0 || G <= 0 || I <= 0 || Is < 0)
    return fail(MOE_ERR_INVALID_ARG, "sizes must be positive (H=%d E=%d G=%d I=%d Is=%d)", H, E, G,
                I, Is);
  if (E % G != 0 || E / G < 2)
    return fail(MOE_ERR_INVALID_ARG, "n_routed_experts %% n_group must be 0 with >= 2 experts per "
                "group (E=%d G=%d)", E, G);
  if (TG < 1 || TG > G)
    return fail(MOE_ERR_INVALID_ARG, "topk_group must be in [1, n_group] (TG=%d G=%d)", TG, G);
  if (K < 1 || K > E)
    return fail(MOE_ERR_INVALID_ARG, "num_experts_per_tok must be in [1, E] (K=%d E=%d)", K, E);
  if (!(isfinite(c->routed_scaling_factor) && c->routed_scaling_factor > 0.0f))
    return fail(MOE_ERR_INVALID_ARG, "routed_scaling_factor must be finite and > 0");
  const moe_dtype a = c->act_dtype, w = c->weight_dtype;
  if (a != MOE_F32 && a != MOE_BF16)
    return fail(MOE_ERR_INVALID_ARG, "act_dtype must be MOE_F32 or MOE_BF16");
  if (w != MOE_F32 && w != MOE_BF16 && !is_fp8(w))
    return fail(MOE_ERR_INVALID_ARG, "unknown weight_dtype");
  // Valid for the method, not handled by these kernels:
  if (E > 512) return fail(MOE_ERR_UNSUPPORTED, "n_routed_experts > 512");
  if (G > 64) return fail(MOE_ERR_UNSUPPORTED, "n_group > 64");
  if (K > 64) return fail(MOE_ERR_UNSUPPORTED, "num_experts_per_tok > 64");
  if ((a == MOE_F32) != (w == MOE_F32))
    return fail(MOE_ERR_UNSUPPORTED, "fp32 activations need fp32 weights and vice versa");
  const int mult = is_fp8(w) ? 128 : 64;
  if (H % mult || I % mult || Is % mult)
    return fail(MOE_ERR_UNSUPPORTED, "hidden and FFN sizes must be multiples of %d", mult);
  return MOE_OK;
}

moe_status check_T(int64_t T, const moe_config* c) {
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T < 0");
  if (T * (int64_t)c->num_experts_per_tok > 0x7fffffffLL || T > 0x7fffffffLL)
    return fail(MOE_ERR_UNSUPPORTED, "T * top_k exceeds int32 indexing");
  return MOE_OK;
}

size_t act_bytes(const moe_config* c) { return c->act_dtype == MOE_BF16 ? 2 : 4; }

// Workspace segments (byte offsets, 256-aligned).
struct Layout {
  size_t err, part, gsplit, idx, w, counts, offsets, perm, pos, hist, tiles, tiles2, h, hs, xq,
      xs, y, ys, flags, total;
  int ksplit;
  bool decode;   // decode routing (gate, selection, permutation, tile list in three launches)
};

Layout layout(const moe_config* c, int64_t T) {
  Layout L{};
  const int64_t H = c->hidden_size, E = c->n_routed_experts, K = c->num_experts_per_tok,
                I = c->moe_intermediate_size, Is = c->shared_intermediate_size;
  const int64_t N = T * K;
  const bool fp8 = is_fp8(c->weight_dtype);
  L.ksplit = c->act_dtype == MOE_BF16 ? moe::gate_ksplit(T, (int)H, (int)E) : 1;
  L.decode = moe::decode_route_ok(T, (int)H, (int)E, (int)K);
  const int64_t nparts = std::max<int64_t>(L.ksplit, L.decode ? moe::decode_ksplit((int)H, (int)E) : 1);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o += up(bytes);
    return at;
  };
  L.err = take(sizeof(int32_t));
  L.part = take((size_t)nparts * T * E * 4);
  L.gsplit = c->act_dtype == MOE_BF16 ? take(moe::gate_split_bytes((int)H, (int)E)) : o;
  L.idx = take((size_t)N * 4);
  L.w = take((size_t)N * 4);
  L.counts = take((size_t)E * 4);
  L.offsets = take((size_t)(E + 1) * 4);
  L.perm = take((size_t)N * 4);
  L.pos = take((size_t)N * 4);
  L.hist = take((size_t)moe::permute_nblk(N) * (E + 1) * 4);
  moe::FfnDims d{T, N, (int)H, (int)I, (int)Is, (int)E, (int)K};
  L.tiles = take(moe::ffn_tiles_bytes(d));
  L.tiles2 = take(moe::ffn_tiles_bytes(d));   // the shared expert's list on a second stream
  const size_t hel = (size_t)(N * I + T * Is);
  if (fp8) {
    L.h = take(hel);
    L.hs = take(hel / 128 * 4);
    L.xq = take((size_t)T * H);
    L.xs = take((size_t)T * H / 128 * 4);
  } else {
    L.h = take(hel * act_bytes(c));
    L.hs = L.xq = L.xs = o;
  }
  L.y = take((size_t)N * H * act_bytes(c));
  L.ys = take((size_t)T * H * act_bytes(c));
  // completion flags of the one-launch decode layer (bf16)
  L.flags = (L.decode && c->act_dtype == MOE_BF16 && c->weight_dtype == MOE_BF16)
                ? take(moe::decode_layer_flags_bytes((int)H, (int)E, (int)K, (int)I, (int)Is))
                : o;
  L.total = o;
  return L;
}

template <typename P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

moe_status check_ws(void* ws, size_t ws_bytes, const Layout& L) {
  if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) % kAlign)
    return fail(MOE_ERR_WORKSPACE, "workspace must be %zu-byte aligned", kAlign);
  if (ws_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, L.total);
  return MOE_OK;
}

#define CHECK(expr)                  \
  do {                               \
    moe_status _s = (expr);          \
    if (_s != MOE_OK) return _s;     \
  } while (0)
#define NONNULL(p)                                                     \
  do {                                                                 \
    if (!(p)) return fail(MOE_ERR_INVALID_ARG, "%s is NULL", #p);      \
  } while (0)
#define HIPCALL(expr, where)                              \
  do {                                                    \
    hipError_t _e = (expr);                               \
    if (_e != hipSuccess) return hip_fail(_e, where);     \
  } while (0)

// ---- the pieces, after validation -------------------------------------------

moe_status run_gate(const moe_config* c, int64_t T, const void* x, const float* gate_w,
                    const float* bias, float* logits, int32_t* idx, float* w, void* ws,
                    const Layout& L, hipStream_t s) {
  float* part = at<float>(ws, L.part);
  const bool bf16 = c->act_dtype == MOE_BF16;
  if (bf16 && moe::gate_use_fused(T, c->hidden_size, c->n_routed_experts, c->n_group,
                                  c->topk_group, c->num_experts_per_tok)) {
    HIPCALL(moe::launch_gate_select_fused((const uint16_t*)x, gate_w, at<void>(ws, L.gsplit), bias,
                                          logits, idx, w, T, c->hidden_size,
                                          c->n_routed_experts, c->n_group, c->topk_group,
                                          c->num_experts_per_tok, c->routed_scaling_factor, s),
            "gate and selection");
    return MOE_OK;
  }
  HIPCALL(moe::launch_gate_logits(x, bf16, gate_w, at<void>(ws, L.gsplit), part, T,
                                  c->hidden_size, c->n_routed_experts, L.ksplit, s),
          "gate logits");
  HIPCALL(moe::launch_select(part, L.ksplit, bias, logits, idx, w, T, c->n_routed_experts,
                             c->n_group, c->topk_group, c->num_experts_per_tok,
                             c->routed_scaling_factor, s),
          "select");
  return MOE_OK;
}

moe_status run_permute(const moe_config* c, int64_t T, const int32_t* idx, int32_t* counts,
                       int32_t* offsets, int32_t* perm, int32_t* pos, void* ws, const Layout& L,
                       hipStream_t s) {
  HIPCALL(moe::launch_permute(idx, T * c->num_experts_per_tok, c->n_routed_experts,
                              at<int32_t>(ws, L.hist), counts, offsets, perm, pos,
                              at<int32_t>(ws, L.err), s),
          "permute");
  return MOE_OK;
}

// groups: which groups to compute (moe::kGroupRouted / kGroupShared);
// tiles: the tile list to use (built here unless tiles_ready); quantize: fp8
// weights only, quantise x first (else xq / xs already hold it).
moe_status run_ffn(const moe_config* c, int64_t T, const void* x, const int32_t* perm,
                   const int32_t* offsets, const moe_weights* wt, void* y, void* ys, void* ws,
                   const Layout& L, hipStream_t s, int groups = moe::kGroupsAll,
                   int32_t* tiles = nullptr, bool tiles_ready = false, bool quantize = true) {
  moe::FfnDims d{T, T * c->num_experts_per_tok, c->hidden_size, c->moe_intermediate_size,
                 c->shared_intermediate_size, c->n_routed_experts, c->num_experts_per_tok};
  d.groups = groups;
  d.tiles_ready = tiles_ready;
  if (!tiles) tiles = at<int32_t>(ws, L.tiles);
  switch (c->weight_dtype) {
    case MOE_F32:
      HIPCALL(moe::launch_ffn_f32(d, (const float*)x, perm, offsets, (const float*)wt->w13,
                                  (const float*)wt->w2, (const float*)wt->ws13,
                                  (const float*)wt->ws2, at<float>(ws, L.h), (float*)y,
                                  (float*)ys, s),
              "ffn f32");
      break;
    case MOE_BF16:
      if (wt->packed) {
        HIPCALL(moe::launch_ffn_bf16_packed(d, (const uint16_t*)x, perm, offsets, wt->w13, wt->w2,
                                            wt->ws13, wt->ws2, at<uint16_t>(ws, L.h),
                                            tiles, (uint16_t*)y,
                                            (uint16_t*)ys, s),
                "ffn bf16 packed");
      } else {
        HIPCALL(moe::launch_ffn_bf16(d, (const uint16_t*)x, perm, offsets,
                                     (const uint16_t*)wt->w13, (const uint16_t*)wt->w2,
                                     (const uint16_t*)wt->ws13, (const uint16_t*)wt->ws2,
                                     at<uint16_t>(ws, L.h), tiles,
                                     (uint16_t*)y, (uint16_t*)ys, s),
                "ffn bf16");
      }
      break;
    case MOE_FP8_E4M3_E8M0: {
      uint8_t* xq = at<uint8_t>(ws, L.xq);
      float* xs = at<float>(ws, L.xs);
      if (quantize)
        HIPCALL(moe::launch_quant_rows((const uint16_t*)x, T, c->hidden_size, xq, xs, true, s),
                "quantise x");
      HIPCALL(moe::launch_ffn_fp8_mx(d, xq, xs, perm, offsets, wt->w13, wt->w13_scale, wt->w2,
                                     wt->w2_scale, wt->ws13, wt->ws13_scale, wt->ws2,
                                     wt->ws2_scale, at<uint8_t>(ws, L.h), at<float>(ws, L.hs),
                                     tiles, (uint16_t*)y, (uint16_t*)ys, s),
              "ffn fp8 (power-of-two scales)");
      break;
    }
    case MOE_FP8_E4M3: {
      uint8_t* xq = at<uint8_t>(ws, L.xq);
      float* xs = at<float>(ws, L.xs);
      if (quantize)
        HIPCALL(moe::launch_quant_rows((const uint16_t*)x, T, c->hidden_size, xq, xs, false, s),
                "quantise x");
      if (wt->packed) {
        HIPCALL(moe::launch_ffn_fp8_packed(d, xq, xs, perm, offsets, wt->w13, wt->w13_scale,
                                           wt->w2, wt->w2_scale, wt->ws13, wt->ws13_scale, wt->ws2,
                                           wt->ws2_scale, at<uint8_t>(ws, L.h), at<float>(ws, L.hs),
                                           tiles, (uint16_t*)y, (uint16_t*)ys,
                                           s),
                "ffn fp8 packed");
        break;
      }
      HIPCALL(moe::launch_ffn_fp8(d, xq, xs, perm, offsets, (const uint8_t*)wt->w13, wt->w13_scale,
                                  (const uint8_t*)wt->w2, wt->w2_scale, (const uint8_t*)wt->ws13,
                                  wt->ws13_scale, (const uint8_t*)wt->ws2, wt->ws2_scale,
                                  at<uint8_t>(ws, L.h), at<float>(ws, L.hs),
                                  tiles, (uint16_t*)y, (uint16_t*)ys, s),
              "ffn fp8");
      break;
    }
  }
  return MOE_OK;
}

moe_status check_weights(const moe_config* c, const moe_weights* w, bool need_gate) {
  NONNULL(w);
  if (w->packed != 0 && w->packed != 1)
    return fail(MOE_ERR_INVALID_ARG, "moe_weights.packed must be 0 or 1");
  if (w->packed && c->weight_dtype == MOE_F32)
    return fail(MOE_ERR_UNSUPPORTED, "the packed weight layout is for bf16 and fp8 weights");
  if (need_gate) {
    NONNULL(w->gate_w);
    NONNULL(w->bias);
  }
  NONNULL(w->w13);
  NONNULL(w->w2);
  const bool fp8 = is_fp8(c->weight_dtype);
  if (c->weight_dtype == MOE_FP8_E4M3_E8M0 && !w->packed)
    return fail(MOE_ERR_UNSUPPORTED, "e4m3 weights with power-of-two scales must be packed "
                "(moe_pack_weight)");
  if (fp8) {
    NONNULL(w->w13_scale);
    NONNULL(w->w2_scale);
  }
  if (c->shared_intermediate_size > 0) {
    NONNULL(w->ws13);
    NONNULL(w->ws2);
    if (fp8) {
      NONNULL(w->ws13_scale);
      NONNULL(w->ws2_scale);
    }
  }
  return MOE_OK;
}


// Events that order a call's work across its two streams, one pair per
// device and host thread (created on first use, reused by every later call:
// a wait takes the event's most recent record at the time it is enqueued).
struct ForkJoin {
  hipEvent_t fork = nullptr, join = nullptr;
};

hipError_t fork_join_events(ForkJoin** out) {
  constexpr int kMaxDevices = 64;
  thread_local ForkJoin ev[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  ForkJoin& f = ev[dev];
  if (!f.fork && (e = hipEventCreateWithFlags(&f.fork, hipEventDisableTiming)) != hipSuccess)
    return e;
  if (!f.join && (e = hipEventCreateWithFlags(&f.join, hipEventDisableTiming)) != hipSuccess)
    return e;
  *out = &f;
  return hipSuccess;
}

// The layer on stream s.  With s2 (not null), the shared expert's GEMMs run
// on s2, forked from s at the start and joined back before the combine.
moe_status forward_impl(const moe_config* cfg, int64_t T, const void* x, const moe_weights* w,
                        void* out, float* logits, int32_t* topk_idx, float* topk_w,
                        int32_t* counts, int32_t* perm, void* ws, size_t ws_bytes,
                        hipStream_t s, hipStream_t s2, bool one_launch = false) {
  CHECK(check_cfg(cfg));
  CHECK(check_T(T, cfg));
  if (T == 0) return MOE_OK;
  NONNULL(x);
  NONNULL(out);
  CHECK(check_weights(cfg, w, true));
  const Layout L = layout(cfg, T);
  CHECK(check_ws(ws, ws_bytes, L));
  if (one_launch &&
      !(L.decode && cfg->act_dtype == MOE_BF16 && cfg->weight_dtype == MOE_BF16 && w->packed &&
        moe::decode_layer_ok(T, cfg->hidden_size, cfg->n_routed_experts,
                             cfg->num_experts_per_tok, cfg->moe_intermediate_size,
                             cfg->shared_intermediate_size)))
    return fail(MOE_ERR_UNSUPPORTED,
                "the one-launch decode layer takes 1 <= T <= %d bf16 tokens and packed bf16 "
                "weights", moe::kDecodeMaxT);
  int32_t* idx = topk_idx ? topk_idx : at<int32_t>(ws, L.idx);
  float* wt = topk_w ? topk_w : at<float>(ws, L.w);
  int32_t* cnt = counts ? counts : at<int32_t>(ws, L.counts);
  int32_t* pm = perm ? perm : at<int32_t>(ws, L.perm);
  int32_t* offs = at<int32_t>(ws, L.offsets);
  int32_t* pos = at<int32_t>(ws, L.pos);
  int32_t* tiles = at<int32_t>(ws, L.tiles);
  void* y = at<void>(ws, L.y);
  const bool sh = cfg->shared_intermediate_size > 0;
  void* ys = sh ? at<void>(ws, L.ys) : nullptr;
  const bool fp8 = is_fp8(cfg->weight_dtype);
  // The fp32 expert kernels compute every group in one launch.
  const bool split = s2 && sh && cfg->weight_dtype != MOE_F32;

  ForkJoin* ev = nullptr;
  if (split) {
    HIPCALL(fork_join_events(&ev), "fork/join events");
    if (fp8)   // x is quantised once, before the fork, for both streams
      HIPCALL(moe::launch_quant_rows((const uint16_t*)x, T, cfg->hidden_size, at<uint8_t>(ws, L.xq),
                                     at<float>(ws, L.xs),
                                     cfg->weight_dtype == MOE_FP8_E4M3_E8M0, s),
              "quantise x");
    HIPCALL(hipEventRecord(ev->fork, s), "fork");
    HIPCALL(hipStreamWaitEvent(s2, ev->fork, 0), "fork");
    CHECK(run_ffn(cfg, T, x, pm, offs, w, y, ys, ws, L, s2, moe::kGroupShared,
                  at<int32_t>(ws, L.tiles2), false, false));
    HIPCALL(hipEventRecord(ev->join, s2), "join");
  }
  const int groups = split ? moe::kGroupRouted : moe::kGroupsAll;
  if (one_launch) {
    HIPCALL(moe::launch_decode_layer(
                (const uint16_t*)x, w->gate_w, w->bias, w->w13, w->w2, w->ws13, w->ws2, T,
                cfg->hidden_size, cfg->n_routed_experts, cfg->n_group, cfg->topk_group,
                cfg->num_experts_per_tok, cfg->moe_intermediate_size,
                cfg->shared_intermediate_size, cfg->routed_scaling_factor,
                at<float>(ws, L.part), logits, idx, wt, cnt, offs, pm, pos,
                at<int32_t>(ws, L.err), tiles, at<uint16_t>(ws, L.h), (uint16_t*)y,
                (uint16_t*)ys, (uint16_t*)out, at<void>(ws, L.flags), s),
            "decode layer");
    return MOE_OK;
  }
  if (L.decode) {
    HIPCALL(moe::launch_decode_route(x, cfg->act_dtype == MOE_BF16, w->gate_w, w->bias,
                                     at<float>(ws, L.part), logits, idx, wt, T, cfg->hidden_size,
                                     cfg->n_routed_experts, cfg->n_group, cfg->topk_group,
                                     cfg->num_experts_per_tok, cfg->routed_scaling_factor, cnt,
                                     offs, pm, pos, at<int32_t>(ws, L.err), tiles, true,
                                     (groups & moe::kGroupShared) && sh, s),
            "decode routing");
  } else {
    CHECK(run_gate(cfg, T, x, w->gate_w, w->bias, logits, idx, wt, ws, L, s));
    CHECK(run_permute(cfg, T, idx, cnt, offs, pm, pos, ws, L, s));
  }
  CHECK(run_ffn(cfg, T, x, pm, offs, w, y, ys, ws, L, s, groups, tiles, L.decode, !split));
  if (split) HIPCALL(hipStreamWaitEvent(s, ev->join, 0), "join");
  HIPCALL(moe::launch_combine(y, ys, pos, wt, out, T, cfg->hidden_size, cfg->num_experts_per_tok,
                              cfg->act_dtype == MOE_BF16, s),
          "combine");
  return MOE_OK;
}

// ---- the no-allocation forward ----------------------------------------------
// Workspace of moe_forward_noalloc: one static device array, of which every GPU
// that runs the library holds its own copy until the process ends.  In host
// code `scratch` names a host-side stand-in, not device memory: its device
// address comes from hipGetSymbolAddress, looked up once per device with
// that device current, and only that address is ever handed to kernels.
constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_address(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

size_t moe_workspace_bytes(const moe_config* cfg, int64_t T) {
  if (check_cfg(cfg) != MOE_OK || T < 0 || check_T(T, cfg) != MOE_OK) return 0;
  return layout(cfg, T).total;
}

moe_status moe_set_gate_mode(int mode) {
  if (mode != MOE_GATE_SPLIT && mode != MOE_GATE_FUSED)
    return fail(MOE_ERR_INVALID_ARG, "gate mode %d is neither 0 (split) nor 1 (fused)", mode);
  moe::set_gate_mode(mode);
  return MOE_OK;
}

moe_status moe_gate(const moe_config* cfg, int64_t T, const void* x, const float* gate_w,
                    const float* bias, float* logits, int32_t* topk_idx, float* topk_w, void* ws,
                    size_t ws_bytes, void* stream) {
  CHECK(check_cfg(cfg));
  CHECK(check_T(T, cfg));
  if (T == 0) return MOE_OK;
  NONNULL(x);
  NONNULL(gate_w);
  NONNULL(bias);
  NONNULL(topk_idx);
  NONNULL(topk_w);
  const Layout L = layout(cfg, T);
  CHECK(check_ws(ws, ws_bytes, L));
  return run_gate(cfg, T, x, gate_w, bias, logits, topk_idx, topk_w, ws, L, (hipStream_t)stream);
}

moe_status moe_permute(const moe_config* cfg, int64_t T, const int32_t* topk_idx, int32_t* counts,
                       int32_t* offsets, int32_t* perm, int32_t* pos, void* ws, size_t ws_bytes,
                       void* stream) {
  CHECK(check_cfg(cfg));
  CHECK(check_T(T, cfg));
  if (T == 0) return MOE_OK;
  NONNULL(topk_idx);
  NONNULL(counts);
  NONNULL(offsets);
  NONNULL(perm);
  NONNULL(pos);
  const Layout L = layout(cfg, T);
  CHECK(check_ws(ws, ws_bytes, L));
  return run_permute(cfg, T, topk_idx, counts, offsets, perm, pos, ws, L, (hipStream_t)stream);
}

moe_status moe_expert_ffn(const moe_config* cfg, int64_t T, const void* x, const int32_t* perm,
                          const int32_t* offsets, const moe_weights* w, void* y, void* y_shared,
                          void* ws, size_t ws_bytes, void* stream) {
  CHECK(check_cfg(cfg));
  CHECK(check_T(T, cfg));
  if (T == 0) return MOE_OK;
  NONNULL(x);
  NONNULL(perm);
  NONNULL(offsets);
  NONNULL(y);
  CHECK(check_weights(cfg, w, false));
  if (cfg->shared_intermediate_size > 0) NONNULL(y_shared);
  const Layout L = layout(cfg, T);
  CHECK(check_ws(ws, ws_bytes, L));
  return run_ffn(cfg, T, x, perm, offsets, w, y,
                 cfg->shared_intermediate_size > 0 ? y_shared : nullptr, ws, L,
                 (hipStream_t)stream);
}

moe_status moe_combine(const moe_config* cfg, int64_t T, const void* y, const void* y_shared,
                       const int32_t* pos, const float* topk_w, void* out, void* stream) {
  CHECK(check_cfg(cfg));
  CHECK(check_T(T, cfg));
  if (T == 0) return MOE_OK;
  NONNULL(y);
  NONNULL(pos);
  NONNULL(topk_w);
  NONNULL(out);
  if (cfg->shared_intermediate_size > 0) NONNULL(y_shared);
  if (cfg->hidden_size % 8)
    return fail(MOE_ERR_UNSUPPORTED, "hidden_size must be a multiple of 8");
  HIPCALL(moe::launch_combine(y, cfg->shared_intermediate_size > 0 ? y_shared : nullptr, pos,
                              topk_w, out, T, cfg->hidden_size, cfg->num_experts_per_tok,
                              cfg->act_dtype == MOE_BF16, (hipStream_t)stream),
          "combine");
  return MOE_OK;
}

moe_status moe_forward(const moe_config* cfg, int64_t T, const void* x, const moe_weights* w,
                       void* out, float* logits, int32_t* topk_idx, float* topk_w,
                       int32_t* counts, int32_t* perm, void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(cfg, T, x, w, out, logits, topk_idx, topk_w, counts, perm, ws, ws_bytes,
                      (hipStream_t)stream, nullptr);
}

moe_status moe_forward_noalloc(const moe_config* cfg, int64_t T, const void* x,
                               const moe_weights* w, void* out, float* logits, int32_t* topk_idx,
                               float* topk_w, int32_t* counts, int32_t* perm, void* stream) {
  CHECK(check_cfg(cfg));
  CHECK(check_T(T, cfg));
  if (T == 0) return MOE_OK;
  const size_t need = layout(cfg, T).total;
  if (need > kScratchBytes)
    return fail(MOE_ERR_UNSUPPORTED,
                "moe_forward_noalloc: %lld tokens need %zu bytes of workspace, the static "
                "scratch holds %zu (use moe_forward with a caller workspace)",
                (long long)T, need, kScratchBytes);
  void* ws = nullptr;
  HIPCALL(scratch_address(&ws), "static scratch address");
  return forward_impl(cfg, T, x, w, out, logits, topk_idx, topk_w, counts, perm, ws,
                      kScratchBytes, (hipStream_t)stream, nullptr);
}

moe_status moe_forward_decode_fused(const moe_config* cfg, int64_t T, const void* x,
                                    const moe_weights* w, void* out, float* logits,
                                    int32_t* topk_idx, float* topk_w, int32_t* counts,
                                    int32_t* perm, void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(cfg, T, x, w, out, logits, topk_idx, topk_w, counts, perm, ws, ws_bytes,
                      (hipStream_t)stream, nullptr, true);
}

moe_status moe_forward_overlap(const moe_config* cfg, int64_t T, const void* x,
                               const moe_weights* w, void* out, float* logits, int32_t* topk_idx,
                               float* topk_w, int32_t* counts, int32_t* perm, void* ws,
                               size_t ws_bytes, void* stream, void* shared_stream) {
  if (!shared_stream || shared_stream == stream)
    return fail(MOE_ERR_INVALID_ARG, "shared_stream must be a stream other than stream");
  return forward_impl(cfg, T, x, w, out, logits, topk_idx, topk_w, counts, perm, ws, ws_bytes,
                      (hipStream_t)stream, (hipStream_t)shared_stream);
}

size_t moe_expert_ffn_backward_workspace_bytes(const moe_config* cfg, int64_t T) {
  if (check_cfg(cfg) != MOE_OK || check_T(T, cfg) != MOE_OK) return 0;
  if (cfg->act_dtype != MOE_BF16 || cfg->weight_dtype == MOE_F32) return 0;
  moe::FfnDims d{T, T * cfg->num_experts_per_tok, cfg->hidden_size, cfg->moe_intermediate_size,
                 cfg->shared_intermediate_size, cfg->n_routed_experts,
                 cfg->num_experts_per_tok};
  return is_fp8(cfg->weight_dtype) ? moe::ffn_backward_fp8_ws_bytes(d)
                                   : moe::ffn_backward_ws_bytes(d);
}

moe_status moe_expert_ffn_backward(const moe_config* cfg, int64_t T, const void* x,
                                   const int32_t* perm, const int32_t* offsets,
                                   const moe_weights* w, const void* dy, const void* dy_shared,
                                   void* dx, void* dx_shared, void* dw13, void* dw2,
                                   void* dws13, void* dws2, void* ws, size_t ws_bytes,
                                   void* stream) {
  CHECK(check_cfg(cfg));
  CHECK(check_T(T, cfg));
  const bool fp8 = is_fp8(cfg->weight_dtype);
  if (cfg->act_dtype != MOE_BF16 || cfg->weight_dtype == MOE_F32)
    return fail(MOE_ERR_UNSUPPORTED,
                "the expert backward takes bf16 activations with bf16 or e4m3 weights");
  if (T == 0) return MOE_OK;
  NONNULL(w);
  if (w->packed)
    return fail(MOE_ERR_UNSUPPORTED, "the expert backward reads row-major weights (packed = 0)");
  NONNULL(x);
  NONNULL(perm);
  NONNULL(offsets);
  NONNULL(w->w13);
  NONNULL(w->w2);
  NONNULL(dy);
  NONNULL(dw13);
  NONNULL(dw2);
  const bool sh = cfg->shared_intermediate_size > 0;
  if (sh) {
    NONNULL(w->ws13);
    NONNULL(w->ws2);
    NONNULL(dy_shared);
    NONNULL(dws13);
    NONNULL(dws2);
  }
  if (fp8) {
    NONNULL(w->w13_scale);
    NONNULL(w->w2_scale);
    if (sh) {
      NONNULL(w->ws13_scale);
      NONNULL(w->ws2_scale);
    }
  }
  moe::FfnDims d{T, T * cfg->num_experts_per_tok, cfg->hidden_size, cfg->moe_intermediate_size,
                 cfg->shared_intermediate_size, cfg->n_routed_experts,
                 cfg->num_experts_per_tok};
  const size_t need = fp8 ? moe::ffn_backward_fp8_ws_bytes(d) : moe::ffn_backward_ws_bytes(d);
  if (!ws || ws_bytes < need || ((uintptr_t)ws & 255))
    return fail(MOE_ERR_WORKSPACE, "workspace must be 256-byte aligned and >= %zu bytes", need);
  if (fp8) {
    HIPCALL(moe::launch_ffn_backward_fp8(
                d, cfg->weight_dtype == MOE_FP8_E4M3_E8M0, (const uint16_t*)x, perm, offsets,
                (const uint8_t*)w->w13, w->w13_scale, (const uint8_t*)w->w2, w->w2_scale,
                (const uint8_t*)(sh ? w->ws13 : nullptr), sh ? w->ws13_scale : nullptr,
                (const uint8_t*)(sh ? w->ws2 : nullptr), sh ? w->ws2_scale : nullptr,
                (const uint16_t*)dy, (const uint16_t*)(sh ? dy_shared : nullptr), (uint16_t*)dx,
                (uint16_t*)(sh ? dx_shared : nullptr), (uint16_t*)dw13, (uint16_t*)dw2,
                (uint16_t*)(sh ? dws13 : nullptr), (uint16_t*)(sh ? dws2 : nullptr), ws,
                (hipStream_t)stream),
            "expert backward (e4m3)");
    return MOE_OK;
  }
  HIPCALL(moe::launch_ffn_backward(d, (const uint16_t*)x, perm, offsets,
                                   (const uint16_t*)w->w13, (const uint16_t*)w->w2,
                                   (const uint16_t*)(sh ? w->ws13 : nullptr),
                                   (const uint16_t*)(sh ? w->ws2 : nullptr), (const uint16_t*)dy,
                                   (const uint16_t*)(sh ? dy_shared : nullptr), (uint16_t*)dx,
                                   (uint16_t*)(sh ? dx_shared : nullptr), (uint16_t*)dw13,
                                   (uint16_t*)dw2, (uint16_t*)(sh ? dws13 : nullptr),
                                   (uint16_t*)(sh ? dws2 : nullptr), ws, (hipStream_t)stream),
          "expert backward");
  return MOE_OK;
}

size_t moe_backward_workspace_bytes(const moe_config* cfg, int64_t T) {
  if (check_cfg(cfg) != MOE_OK || check_T(T, cfg) != MOE_OK) return 0;
  if (cfg->weight_dtype == MOE_F32 || cfg->act_dtype != MOE_BF16) return 0;
  moe::FfnDims d{T, T * cfg->num_experts_per_tok, cfg->hidden_size, cfg->moe_intermediate_size,
                 cfg->shared_intermediate_size, cfg->n_routed_experts,
                 cfg->num_experts_per_tok};
  return moe::layer_backward_ws_bytes(d, is_fp8(cfg->weight_dtype));
}

moe_status moe_backward(const moe_config* cfg, int64_t T, const void* x, const moe_weights* w,
                        const float* logits, const int32_t* topk_idx, const float* topk_w,
                        const int32_t* perm, const int32_t* offsets, const int32_t* pos,
                        const void* y, const void* dout, void* dx, float* dgate_w, void* dw13,
                        void* dw2, void* dws13, void* dws2, void* ws, size_t ws_bytes,
                        void* stream) {
  CHECK(check_cfg(cfg));
  CHECK(check_T(T, cfg));
  const bool fp8 = is_fp8(cfg->weight_dtype);
  if (cfg->act_dtype != MOE_BF16 || cfg->weight_dtype == MOE_F32)
    return fail(MOE_ERR_UNSUPPORTED,
                "the layer backward takes bf16 activations with bf16 or e4m3 weights");
  if (T == 0) return MOE_OK;
  NONNULL(w);
  if (w->packed)
    return fail(MOE_ERR_UNSUPPORTED, "the layer backward reads row-major weights (packed = 0)");
  NONNULL(x);
  NONNULL(w->gate_w);
  NONNULL(w->w13);
  NONNULL(w->w2);
  NONNULL(logits);
  NONNULL(topk_idx);
  NONNULL(topk_w);
  NONNULL(perm);
  NONNULL(offsets);
  NONNULL(pos);
  NONNULL(y);
  NONNULL(dout);
  NONNULL(dx);
  NONNULL(dgate_w);
  NONNULL(dw13);
  NONNULL(dw2);
  const bool sh = cfg->shared_intermediate_size > 0;
  if (sh) {
    NONNULL(w->ws13);
    NONNULL(w->ws2);
    NONNULL(dws13);
    NONNULL(dws2);
  }
  if (fp8) {
    NONNULL(w->w13_scale);
    NONNULL(w->w2_scale);
    if (sh) {
      NONNULL(w->ws13_scale);
      NONNULL(w->ws2_scale);
    }
  }
  moe::FfnDims d{T, T * cfg->num_experts_per_tok, cfg->hidden_size, cfg->moe_intermediate_size,
                 cfg->shared_intermediate_size, cfg->n_routed_experts,
                 cfg->num_experts_per_tok};
  const size_t need = moe::layer_backward_ws_bytes(d, fp8);
  if (!ws || ws_bytes < need || ((uintptr_t)ws & 255))
    return fail(MOE_ERR_WORKSPACE, "workspace must be 256-byte aligned and >= %zu bytes", need);
  moe::ExpertWeights ew{w->w13, w->w2, sh ? w->ws13 : nullptr, sh ? w->ws2 : nullptr};
  if (fp8) {
    ew.w13s = w->w13_scale;
    ew.w2s = w->w2_scale;
    ew.ws13s = sh ? w->ws13_scale : nullptr;
    ew.ws2s = sh ? w->ws2_scale : nullptr;
    ew.fp8 = true;
    ew.pow2 = cfg->weight_dtype == MOE_FP8_E4M3_E8M0;
  }
  HIPCALL(moe::launch_layer_backward(
              d, (const uint16_t*)x, w->gate_w, logits, topk_idx, topk_w, perm, offsets, pos,
              (const uint16_t*)y, (const uint16_t*)dout, ew, cfg->routed_scaling_factor,
              (uint16_t*)dx, dgate_w, (uint16_t*)dw13, (uint16_t*)dw2,
              (uint16_t*)(sh ? dws13 : nullptr), (uint16_t*)(sh ? dws2 : nullptr), ws,
              (hipStream_t)stream),
          "layer backward");
  return MOE_OK;
}

moe_status moe_bias_update(const moe_config* cfg, const int32_t* counts, float gamma,
                           float* bias, void* stream) {
  CHECK(check_cfg(cfg));
  if (!(gamma >= 0.0f) || isinf(gamma))
    return fail(MOE_ERR_INVALID_ARG, "gamma must be finite and >= 0");
  NONNULL(counts);
  NONNULL(bias);
  HIPCALL(moe::launch_bias_update(counts, bias, cfg->n_routed_experts, gamma,
                                  (hipStream_t)stream),
          "bias update");
  return MOE_OK;
}

moe_status moe_quantize_act(const moe_config* cfg, int64_t rows, const void* x, uint8_t* xq,
                            float* xs, void* stream) {
  CHECK(check_cfg(cfg));
  if (rows < 0) return fail(MOE_ERR_INVALID_ARG, "rows < 0");
  if (rows == 0) return MOE_OK;
  if (cfg->act_dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "the fp8 quantiser takes bf16 activations");
  if (cfg->hidden_size % 128) return fail(MOE_ERR_UNSUPPORTED, "hidden_size %% 128 != 0");
  NONNULL(x);
  NONNULL(xq);
  NONNULL(xs);
  HIPCALL(moe::launch_quant_rows((const uint16_t*)x, rows, cfg->hidden_size, xq, xs,
                                 cfg->weight_dtype == MOE_FP8_E4M3_E8M0,
                                 (hipStream_t)stream),
          "quantise");
  return MOE_OK;
}

size_t moe_packed_bytes(const moe_config* cfg, moe_weight_id which) {
  if (check_cfg(cfg) != MOE_OK || cfg->weight_dtype == MOE_F32) return 0;
  const int H = cfg->hidden_size, I = cfg->moe_intermediate_size,
            Is = cfg->shared_intermediate_size, E = cfg->n_routed_experts;
  auto bytes = is_fp8(cfg->weight_dtype) ? moe::packed8_bytes : moe::packed_bytes;
  switch (which) {
    case MOE_W13: return bytes(true, E, I, H);
    case MOE_W2: return bytes(false, E, H, I);
    case MOE_WS13: return Is ? bytes(true, 1, Is, H) : 0;
    case MOE_WS2: return Is ? bytes(false, 1, H, Is) : 0;
  }
  return 0;
}

moe_status moe_pack_weight(const moe_config* cfg, moe_weight_id which, const void* src,
                           void* dst, void* stream) {
  CHECK(check_cfg(cfg));
  if (cfg->weight_dtype == MOE_F32)
    return fail(MOE_ERR_UNSUPPORTED, "the packed weight layout is for bf16 and fp8 weights");
  if (which < MOE_W13 || which > MOE_WS2) return fail(MOE_ERR_INVALID_ARG, "unknown weight id");
  const int H = cfg->hidden_size, I = cfg->moe_intermediate_size,
            Is = cfg->shared_intermediate_size, E = cfg->n_routed_experts;
  if ((which == MOE_WS13 || which == MOE_WS2) && Is == 0)
    return fail(MOE_ERR_INVALID_ARG, "no shared expert (shared_intermediate_size == 0)");
  NONNULL(src);
  NONNULL(dst);
  const bool gate_up = which == MOE_W13 || which == MOE_WS13;
  const int64_t experts = (which == MOE_W13 || which == MOE_W2) ? E : 1;
  const int inter = (which == MOE_W13 || which == MOE_W2) ? I : Is;
  const int n = gate_up ? inter : H, kd = gate_up ? H : inter;
  if (is_fp8(cfg->weight_dtype))
    HIPCALL(moe::launch_pack8(gate_up, (const uint8_t*)src, dst, experts, n, kd,
                              (hipStream_t)stream),
            "pack weight");
  else
    HIPCALL(moe::launch_pack(gate_up, (const uint16_t*)src, dst, experts, n, kd,
                             (hipStream_t)stream),
            "pack weight");
  return MOE_OK;
}

moe_status moe_get_device_error(void* ws, size_t ws_bytes, void* stream) {
  if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
  if (ws_bytes < sizeof(int32_t)) return fail(MOE_ERR_WORKSPACE, "workspace too small");
  int32_t flag = 0;
  hipStream_t s = (hipStream_t)stream;
  HIPCALL(hipMemcpyAsync(&flag, ws, sizeof(flag), hipMemcpyDeviceToHost, s), "read error flag");
  HIPCALL(hipStreamSynchronize(s), "synchronise");
  if (flag & 2)
    return fail(MOE_ERR_DEVICE_CHECK,
                "a completion wait of the one-launch decode layer timed out: outputs unreliable");
  if (flag) return fail(MOE_ERR_DEVICE_CHECK, "an expert index was outside [0, E)");
  return MOE_OK;
}

const char* moe_strerror(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_DEVICE_CHECK: return "device check failed (expert index out of range)";
  }
  return "unknown status";
}

const char* moe_last_error(void) { return g_msg; }

}  // extern "C"
