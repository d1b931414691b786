// Backward of the whole layer (layer_backward.hip), on top of the expert
// backward declared in moe_internal.hpp.
#pragma once

#include "moe_internal.hpp"

namespace moe {

// Row-major expert weights of the backward: bf16, or e4m3 with fp32
// 128x128 block scales (pow2: power-of-two activation and gradient scales).
struct ExpertWeights {
  const void *w13, *w2, *ws13, *ws2;
  const float *w13s = nullptr, *w2s = nullptr, *ws13s = nullptr, *ws2s = nullptr;
  bool fp8 = false, pow2 = false;
};

size_t layer_backward_ws_bytes(const FfnDims& d, bool fp8);
hipError_t launch_layer_backward(const FfnDims& d, const uint16_t* x, const float* gate_w,
                                 const float* logits, const int32_t* idx, const float* topk_w,
                                 const int32_t* perm, const int32_t* offsets, const int32_t* pos,
                                 const uint16_t* y, const uint16_t* dout, const ExpertWeights& wt,
                                 float rho, uint16_t* dx, float* dgate_w, uint16_t* dw13,
                                 uint16_t* dw2, uint16_t* dws13, uint16_t* dws2, void* ws,
                                 hipStream_t s);

}  // namespace moe
