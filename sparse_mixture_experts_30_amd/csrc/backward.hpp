// Backward of the whole layer (layer_backward.hip), on top of the expert
// backward declared in moe_internal.hpp.
#pragma once

#include "moe_internal.hpp"

namespace moe {

size_t layer_backward_ws_bytes(const FfnDims& d);
hipError_t launch_layer_backward(const FfnDims& d, const uint16_t* x, const float* gate_w,
                                 const float* logits, const int32_t* idx, const float* topk_w,
                                 const int32_t* perm, const int32_t* offsets, const int32_t* pos,
                                 const uint16_t* y, const uint16_t* dout, const uint16_t* w13,
                                 const uint16_t* w2, const uint16_t* ws13, const uint16_t* ws2,
                                 float rho, uint16_t* dx, float* dgate_w, uint16_t* dw13,
                                 uint16_t* dw2, uint16_t* dws13, uint16_t* dws2, void* ws,
                                 hipStream_t s);

}  // namespace moe
