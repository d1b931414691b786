// Backward of the whole layer (training), bf16 activations with bf16 or e4m3
// expert weights, with the routing held at the forward's choice: the gradient reaches the gate only through the chosen
// experts' weights, and the selection-only bias gets none.
//
// The forward (page "从 1024 块 GPU 到 558 万美元：拆解 DeepSeek-V3 的算法-系统协同设计",
// section 2.2, MoEGate; the combine of section 2.3) is
//   logits = x Wg^T,  s = sigmoid(logits) of the chosen experts,
//   w_k = rho s_k / (sum_j s_j + 1e-20) (top_k > 1) or rho s_k,
//   out_t = shared(x_t) + sum_k w_tk y_tk,   y_tk = FFN_idx[t,k](x_t).
// Given dout, with D = sum_j s_j + 1e-20:
//   dy_tk = w_tk dout_t,   dw_tk = <dout_t, y_tk>,
//   ds_k = rho (dw_k / D - sum_j dw_j s_j / D^2)  (or rho dw_k for top-1),
//   dlogit_tk = ds_k s_k (1 - s_k),
//   dWg[e] = sum over the rows routed to e of dlogit x_t,
//   dx_t = sum_k dlogit_tk Wg[idx_tk] + shared'(x_t)^T dout_t + sum_k FFN'^T dy_tk.
// The expert FFNs' part is the expert backward (ffn_backward.hip); the
// kernels here do the combine and routing-weight backward, the gate's
// weight gradient, and the assembly of dx.
#include "moe_internal.hpp"
#include "backward.hpp"

namespace moe {

namespace {

constexpr int LB_THREADS = 256;

__device__ __forceinline__ void unpack8(const u32x4 v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ u32x4 pack8(const float (&f)[8]) {
  return (u32x4){pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                 pack_bf16x2(f[6], f[7])};
}

// Sum of v over the workgroup in a fixed order (wave shuffles, then the
// waves in order); every thread gets the result.
__device__ __forceinline__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float s = 0.0f;
#pragma unroll
  for (int w = 0; w < LB_THREADS / 64; ++w) s += red[w];
  __syncthreads();
  return s;
}

// One workgroup per token t: the routed rows' output gradients dy (bf16, in
// the sorted row order), dw_tk, and the logit gradients of the chosen experts.
__global__ void __launch_bounds__(LB_THREADS)
combine_route_bwd_kernel(const uint16_t* __restrict__ dout, const uint16_t* __restrict__ y,
                         const int32_t* __restrict__ pos, const float* __restrict__ topk_w,
                         const float* __restrict__ logits, const int32_t* __restrict__ idx, int H,
                         int K, int E, float rho, uint16_t* __restrict__ dyr,
                         float* __restrict__ dlogit) {
  __shared__ float red[LB_THREADS / 64];
  __shared__ float s_dw[64], s_s[64];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  const int nc = H / 8;
  const uint16_t* drow = dout + t * H;
  for (int k = 0; k < K; ++k) {
    const int64_t j = pos[t * K + k];
    const float wk = topk_w[t * K + k];
    const uint16_t* yrow = y + j * H;
    uint16_t* grow = dyr + j * H;
    float part = 0.0f;
    for (int c = tid; c < nc; c += LB_THREADS) {
      float d[8], yv[8], g[8];
      unpack8(*reinterpret_cast<const u32x4*>(drow + c * 8), d);
      unpack8(*reinterpret_cast<const u32x4*>(yrow + c * 8), yv);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        part = fmaf(d[i], yv[i], part);
        g[i] = wk * d[i];
      }
      *reinterpret_cast<u32x4*>(grow + c * 8) = pack8(g);
    }
    const float dw = block_sum(part, red);
    if (tid == 0) s_dw[k] = dw;
  }
  __syncthreads();
  // the scores as the forward's selection forms them (sigmoid in double,
  // rounded to fp32), summed in slot order
  if (tid < K) {
    const float lg = logits[t * E + idx[t * K + tid]];
    s_s[tid] = (float)(1.0 / (1.0 + exp(-(double)lg)));
  }
  __syncthreads();
  if (tid < K) {
    float D = 0.0f, sdw = 0.0f;
    for (int k = 0; k < K; ++k) {
      D += s_s[k];
      sdw += s_dw[k] * s_s[k];
    }
    D += 1e-20f;
    const float sk = s_s[tid];
    const float ds = K > 1 ? rho * (s_dw[tid] / D - sdw / (D * D)) : rho * s_dw[tid];
    dlogit[t * K + tid] = ds * sk * (1.0f - sk);
  }
}

// dWg[e][h] = sum over the rows j of expert e (sorted order) of
// dlogit[perm[j]] x[perm[j] / K][h], fp32, rows added in order; an expert
// without rows gets zeros.  Workgroup (e, 256 columns).
__global__ void __launch_bounds__(LB_THREADS)
gate_dw_kernel(const uint16_t* __restrict__ x, const int32_t* __restrict__ perm,
               const int32_t* __restrict__ offsets, const float* __restrict__ dlogit, int H,
               int K, float* __restrict__ dgw) {
  const int e = blockIdx.x;
  const int h = blockIdx.y * LB_THREADS + threadIdx.x;
  if (h >= H) return;   // no barrier here
  const int r0 = offsets[e], r1 = offsets[e + 1];
  float acc = 0.0f;
  constexpr int B = 8;   // rows whose loads are issued together
  for (int j0 = r0; j0 < r1; j0 += B) {
    float xv[B], g[B];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      xv[u] = 0.0f;
      g[u] = 0.0f;
      if (j0 + u < r1) {
        const int f = perm[j0 + u];
        g[u] = dlogit[f];
        xv[u] = bf16_bits_to_f32(x[(int64_t)(f / K) * H + h]);
      }
    }
#pragma unroll
    for (int u = 0; u < B; ++u)
      if (j0 + u < r1) acc = fmaf(g[u], xv[u], acc);
  }
  dgw[(int64_t)e * H + h] = acc;
}

// dx_t = (shared expert's dx_t) + sum_k (dx of row pos[t, k] + dlogit_tk
// Wg[idx_tk]), fp32 in that order, rounded once to bf16.
__global__ void __launch_bounds__(LB_THREADS)
dx_assemble_kernel(const uint16_t* __restrict__ dxr, const uint16_t* __restrict__ dxs,
                   const int32_t* __restrict__ pos, const int32_t* __restrict__ idx,
                   const float* __restrict__ dlogit, const float* __restrict__ gw, int H, int K,
                   uint16_t* __restrict__ dx) {
  const int64_t t = blockIdx.x;
  for (int c = threadIdx.x; c < H / 8; c += LB_THREADS) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (dxs) unpack8(*reinterpret_cast<const u32x4*>(dxs + t * H + c * 8), acc);
    for (int k = 0; k < K; ++k) {
      float r[8];
      unpack8(*reinterpret_cast<const u32x4*>(dxr + (int64_t)pos[t * K + k] * H + c * 8), r);
      const float g = dlogit[t * K + k];
      const float* wr = gw + (int64_t)idx[t * K + k] * H + c * 8;
      const u32x4 w0 = *reinterpret_cast<const u32x4*>(wr);
      const u32x4 w1 = *reinterpret_cast<const u32x4*>(wr + 4);
      const float wv[8] = {__uint_as_float(w0.x), __uint_as_float(w0.y), __uint_as_float(w0.z),
                           __uint_as_float(w0.w), __uint_as_float(w1.x), __uint_as_float(w1.y),
                           __uint_as_float(w1.z), __uint_as_float(w1.w)};
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(g, wv[i], acc[i] + r[i]);
    }
    *reinterpret_cast<u32x4*>(dx + t * H + c * 8) = pack8(acc);
  }
}

size_t al256(size_t b) { return (b + 255) / 256 * 256; }

}  // namespace

size_t layer_backward_ws_bytes(const FfnDims& d, bool fp8) {
  const size_t rows = (size_t)d.N * d.H * 2;
  return al256(rows) + al256(rows) + al256((size_t)d.T * d.H * 2) + al256((size_t)d.N * 4) +
         (fp8 ? ffn_backward_fp8_ws_bytes(d) : ffn_backward_ws_bytes(d));
}

hipError_t launch_layer_backward(const FfnDims& d, const uint16_t* x, const float* gate_w,
                                 const float* logits, const int32_t* idx, const float* topk_w,
                                 const int32_t* perm, const int32_t* offsets, const int32_t* pos,
                                 const uint16_t* y, const uint16_t* dout, const ExpertWeights& wt,
                                 float rho, uint16_t* dx, float* dgate_w, uint16_t* dw13,
                                 uint16_t* dw2, uint16_t* dws13, uint16_t* dws2, void* ws,
                                 hipStream_t s) {
  const bool sh = d.Is > 0;
  char* base = (char*)ws;
  uint16_t* dyr = (uint16_t*)base;
  base += al256((size_t)d.N * d.H * 2);
  uint16_t* dxr = (uint16_t*)base;
  base += al256((size_t)d.N * d.H * 2);
  uint16_t* dxs = (uint16_t*)base;
  base += al256((size_t)d.T * d.H * 2);
  float* dlogit = (float*)base;
  base += al256((size_t)d.N * 4);
  void* wsf = base;

  MOE_TIMED_LAUNCH(s, "combine_route_bwd_kernel",
    hipLaunchKernelGGL(combine_route_bwd_kernel, dim3((unsigned)d.T), dim3(LB_THREADS), 0, s,
                       dout, y, pos, topk_w, logits, idx, d.H, d.K, d.E, rho, dyr, dlogit));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // The shared expert's output gradient is dout itself.  e4m3 weights take
  // the FP8 expert backward (operands quantised per 128 along each GEMM's
  // contraction), bf16 weights the bf16 one.
  if (wt.fp8)
    e = launch_ffn_backward_fp8(d, wt.pow2, x, perm, offsets, (const uint8_t*)wt.w13, wt.w13s,
                                (const uint8_t*)wt.w2, wt.w2s, (const uint8_t*)wt.ws13, wt.ws13s,
                                (const uint8_t*)wt.ws2, wt.ws2s, dyr, sh ? dout : nullptr, dxr,
                                sh ? dxs : nullptr, dw13, dw2, dws13, dws2, wsf, s);
  else
    e = launch_ffn_backward(d, x, perm, offsets, (const uint16_t*)wt.w13,
                            (const uint16_t*)wt.w2, (const uint16_t*)wt.ws13,
                            (const uint16_t*)wt.ws2, dyr, sh ? dout : nullptr, dxr,
                            sh ? dxs : nullptr, dw13, dw2, dws13, dws2, wsf, s);
  if (e != hipSuccess) return e;
  MOE_TIMED_LAUNCH(s, "gate_dw_kernel",
    hipLaunchKernelGGL(gate_dw_kernel, dim3(d.E, (d.H + LB_THREADS - 1) / LB_THREADS),
                       dim3(LB_THREADS), 0, s, x, perm, offsets, dlogit, d.H, d.K, dgate_w));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  MOE_TIMED_LAUNCH(s, "dx_assemble_kernel",
    hipLaunchKernelGGL(dx_assemble_kernel, dim3((unsigned)d.T), dim3(LB_THREADS), 0, s, dxr,
                       sh ? dxs : nullptr, pos, idx, dlogit, gate_w, d.H, d.K, dx));
  return hipGetLastError();
}

}  // namespace moe
