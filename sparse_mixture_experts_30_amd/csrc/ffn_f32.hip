// Expert FFNs in fp32 arithmetic for fp32 layers (activations and weights
// fp32).  One thread per output element with plain fp32 FMA dot products: a
// correctness path for small fp32 layers, not a tuned kernel.
//
// SwiGLU expert (mqxn.cn/news/19449, section 3.1): h = silu(x Wg^T) * (x Wu^T),
// y = h W2^T; routed rows gathered through the expert-sorted order, the
// shared expert on all tokens ("从 1024 块 GPU 到 558 万美元：拆解 DeepSeek-V3 的算法-系统协同设计",
// section 2.2).
#include "moe_internal.hpp"

namespace moe {

namespace {

// Expert of sorted row j: the e with offsets[e] <= j < offsets[e+1].
__device__ int expert_of_row(const int32_t* offsets, int E, int64_t j) {
  int lo = 0, hi = E;  // offsets[lo] <= j < offsets[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (offsets[mid] <= j) lo = mid; else hi = mid;
  }
  return lo;
}

// h rows [0, N): routed (width I); rows [N, N+T): shared (width Is).
__global__ void ffn1_f32_kernel(const float* __restrict__ x, const int32_t* __restrict__ perm,
                                const int32_t* __restrict__ offsets,
                                const float* __restrict__ w13, const float* __restrict__ ws13,
                                float* __restrict__ h, int64_t T, int64_t N, int H, int I,
                                int Is, int E, int K) {
  const int64_t j = blockIdx.x;  // row
  const int n = blockIdx.y * blockDim.x + threadIdx.x;
  const float *xr, *wg, *wu;
  float* out;
  if (j < N) {
    if (n >= I) return;
    const int e = expert_of_row(offsets, E, j);
    xr = x + (int64_t)(perm[j] / K) * H;
    wg = w13 + ((int64_t)e * 2 * I + n) * H;
    wu = w13 + ((int64_t)e * 2 * I + I + n) * H;
    out = h + j * I + n;
  } else {
    if (n >= Is) return;
    const int64_t t = j - N;
    xr = x + t * H;
    wg = ws13 + (int64_t)n * H;
    wu = ws13 + (int64_t)(Is + n) * H;
    out = h + N * I + t * Is + n;
  }
  float g = 0.0f, u = 0.0f;
  for (int k = 0; k < H; ++k) {
    g = fmaf(xr[k], wg[k], g);
    u = fmaf(xr[k], wu[k], u);
  }
  *out = g / (1.0f + expf(-g)) * u;
}

__global__ void ffn2_f32_kernel(const float* __restrict__ h, const int32_t* __restrict__ offsets,
                                const float* __restrict__ w2, const float* __restrict__ ws2,
                                float* __restrict__ y, float* __restrict__ ys, int64_t T,
                                int64_t N, int H, int I, int Is, int E) {
  const int64_t j = blockIdx.x;
  const int m = blockIdx.y * blockDim.x + threadIdx.x;
  if (m >= H) return;
  const float *hr, *wr;
  float* out;
  int n;
  if (j < N) {
    const int e = expert_of_row(offsets, E, j);
    hr = h + j * I;
    wr = w2 + ((int64_t)e * H + m) * I;
    out = y + j * H + m;
    n = I;
  } else {
    const int64_t t = j - N;
    hr = h + N * I + t * Is;
    wr = ws2 + (int64_t)m * Is;
    out = ys + t * H + m;
    n = Is;
  }
  float acc = 0.0f;
  for (int k = 0; k < n; ++k) acc = fmaf(hr[k], wr[k], acc);
  *out = acc;
}

}  // namespace

hipError_t launch_ffn_f32(const FfnDims& d, const float* x, const int32_t* perm,
                          const int32_t* offsets, const float* w13, const float* w2,
                          const float* ws13, const float* ws2, float* h, float* y, float* ys,
                          hipStream_t s) {
  const int64_t rows = d.N + (d.Is > 0 ? d.T : 0);
  if (rows > 0x7fffffff) return hipErrorInvalidValue;
  const int imax = d.I > d.Is ? d.I : d.Is;
  MOE_TIMED_LAUNCH(s, "ffn1_f32_kernel",
    hipLaunchKernelGGL(ffn1_f32_kernel, dim3((unsigned)rows, (imax + 127) / 128), dim3(128), 0, s,
                       x, perm, offsets, w13, ws13, h, d.T, d.N, d.H, d.I, d.Is, d.E, d.K));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  MOE_TIMED_LAUNCH(s, "ffn2_f32_kernel",
    hipLaunchKernelGGL(ffn2_f32_kernel, dim3((unsigned)rows, (d.H + 127) / 128), dim3(128), 0, s,
                       h, offsets, w2, ws2, y, ys, d.T, d.N, d.H, d.I, d.Is, d.E));
  return hipGetLastError();
}

}  // namespace moe
