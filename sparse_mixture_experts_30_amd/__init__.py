"""MI355X-native DeepSeek-V3-style MoE layer forward: sigmoid gate with a
selection-only bias, group-limited top-k routing, stable token permutation by
expert, SwiGLU grouped expert GEMMs (bf16 MFMA, e4m3 block-scaled variant),
an always-active shared expert, the weighted combine, the load-balancing
update of the selection bias, and the backward of the layer (gate, combine,
expert FFNs).  Decode batches take a three-launch routing schedule, and the
shared expert can run on a second stream beside the routed ones.  All compute is in the HIP kernels of
libmoe.so; this package only marshals arguments."""
from ._lib import (EXPORTS, MOE_BF16, MOE_ERR_DEVICE_CHECK, MOE_ERR_HIP, MOE_ERR_INVALID_ARG,
                   MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_F32, MOE_FP8_E4M3, MOE_FP8_E4M3_E8M0, MOE_OK,
                   MOE_W13, MOE_W2, MOE_WS13, MOE_WS2, moe_pack_weight, moe_packed_bytes,
                   MoeConfig, MoeError, MoeWeights, SO_PATH, config, lib, moe_bias_update,
                   moe_backward, moe_backward_workspace_bytes, moe_combine, moe_expert_ffn,
                   moe_expert_ffn_backward,
                   moe_expert_ffn_backward_workspace_bytes, moe_forward, moe_forward_noalloc,
                   moe_forward_overlap, moe_forward_decode_fused, MOE_NOALLOC_SCRATCH_BYTES,
                   moe_gate, moe_get_device_error,
                   moe_kernel_timer_enable, moe_kernel_timer_read, moe_last_error,
                   moe_permute, moe_quantize_act, moe_strerror, moe_workspace_bytes, weights,
                   moe_set_gate_mode, MOE_GATE_SPLIT, MOE_GATE_FUSED)

__all__ = [n for n in dir() if not n.startswith("_")]
