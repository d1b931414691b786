"""ctypes binding of libmoe (include/moe.h).  Argument marshalling only: every
step of the layer runs in the HIP kernels of libmoe.so.  Tensors are passed
as device pointers (torch tensors on the GPU, or raw integer addresses)."""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
SO_PATH = os.path.join(HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP, \
    MOE_ERR_DEVICE_CHECK = range(6)
MOE_F32, MOE_BF16, MOE_FP8_E4M3, MOE_FP8_E4M3_E8M0 = 0, 1, 2, 3

# Every function declared in include/moe.h.
EXPORTS = ("moe_workspace_bytes", "moe_gate", "moe_permute", "moe_expert_ffn", "moe_combine",
           "moe_forward", "moe_forward_overlap", "moe_forward_noalloc", "moe_forward_decode_fused",
           "moe_quantize_act", "moe_packed_bytes", "moe_pack_weight",
           "moe_get_device_error", "moe_strerror", "moe_last_error", "moe_kernel_timer_enable",
           "moe_kernel_timer_read", "moe_bias_update", "moe_expert_ffn_backward",
           "moe_expert_ffn_backward_workspace_bytes", "moe_backward",
           "moe_backward_workspace_bytes", "moe_set_gate_mode")
MOE_W13, MOE_W2, MOE_WS13, MOE_WS2 = 0, 1, 2, 3


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[{status}] {msg}")
        self.status = status


class MoeConfig(ctypes.Structure):
    _fields_ = [("hidden_size", ctypes.c_int32), ("n_routed_experts", ctypes.c_int32),
                ("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32),
                ("num_experts_per_tok", ctypes.c_int32), ("moe_intermediate_size", ctypes.c_int32),
                ("shared_intermediate_size", ctypes.c_int32),
                ("routed_scaling_factor", ctypes.c_float),
                ("act_dtype", ctypes.c_int), ("weight_dtype", ctypes.c_int)]


class MoeWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("gate_w", "bias", "w13", "w13_scale", "w2",
                                               "w2_scale", "ws13", "ws13_scale", "ws2",
                                               "ws2_scale")] + [("packed", ctypes.c_int32)]


_lib = None


def lib():
    """Load libmoe.so; raise if it was not built (there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(SO_PATH):
            raise RuntimeError(f"{SO_PATH} is missing: build it with "
                               f"'python -m sparse_mixture_experts_30_amd.build'")
        L = ctypes.CDLL(SO_PATH)
        vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
        cfgp = ctypes.POINTER(MoeConfig)
        wp = ctypes.POINTER(MoeWeights)
        sig = {
            "moe_workspace_bytes": (sz, [cfgp, i64]),
            "moe_gate": (ctypes.c_int, [cfgp, i64, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
            "moe_permute": (ctypes.c_int, [cfgp, i64, vp, vp, vp, vp, vp, vp, sz, vp]),
            "moe_expert_ffn": (ctypes.c_int, [cfgp, i64, vp, vp, vp, wp, vp, vp, vp, sz, vp]),
            "moe_combine": (ctypes.c_int, [cfgp, i64, vp, vp, vp, vp, vp, vp]),
            "moe_forward": (ctypes.c_int, [cfgp, i64, vp, wp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
            "moe_forward_overlap": (ctypes.c_int, [cfgp, i64, vp, wp, vp, vp, vp, vp, vp, vp, vp, sz,
                                                   vp, vp]),
            "moe_forward_noalloc": (ctypes.c_int, [cfgp, i64, vp, wp, vp, vp, vp, vp, vp, vp, vp]),
            "moe_forward_decode_fused": (ctypes.c_int, [cfgp, i64, vp, wp, vp, vp, vp, vp, vp, vp,
                                                        vp, sz, vp]),
            "moe_quantize_act": (ctypes.c_int, [cfgp, i64, vp, vp, vp, vp]),
            "moe_bias_update": (ctypes.c_int, [cfgp, vp, ctypes.c_float, vp, vp]),
            "moe_expert_ffn_backward_workspace_bytes": (sz, [cfgp, i64]),
            "moe_expert_ffn_backward": (ctypes.c_int, [cfgp, i64, vp, vp, vp, wp, vp, vp, vp, vp, vp,
                                                       vp, vp, vp, vp, sz, vp]),
            "moe_backward_workspace_bytes": (sz, [cfgp, i64]),
            "moe_backward": (ctypes.c_int, [cfgp, i64, vp, wp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                            vp, vp, vp, vp, vp, vp, sz, vp]),
            "moe_packed_bytes": (sz, [cfgp, ctypes.c_int]),
            "moe_pack_weight": (ctypes.c_int, [cfgp, ctypes.c_int, vp, vp, vp]),
            "moe_get_device_error": (ctypes.c_int, [vp, sz, vp]),
            "moe_strerror": (ctypes.c_char_p, [ctypes.c_int]),
            "moe_last_error": (ctypes.c_char_p, []),
            "moe_kernel_timer_enable": (ctypes.c_int, [ctypes.c_int, ctypes.c_char_p]),
            "moe_set_gate_mode": (ctypes.c_int, [ctypes.c_int]),
            "moe_kernel_timer_read": (ctypes.c_int, [ctypes.c_int,
                                                     ctypes.POINTER(ctypes.c_char_p),
                                                     ctypes.POINTER(ctypes.c_double),
                                                     ctypes.POINTER(ctypes.c_int64)]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _ptr(t) -> Optional[int]:
    """Device address of a torch tensor (or an int address, or None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int):
    if status != MOE_OK:
        raise MoeError(status, lib().moe_last_error().decode())


def config(H, E, G, TG, K, I, Is, rho, act="bf16", wdtype="bf16") -> MoeConfig:
    dt = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8_E4M3, "fp8e8m0": MOE_FP8_E4M3_E8M0}
    return MoeConfig(H, E, G, TG, K, I, Is, float(rho), dt[act], dt[wdtype])


def weights(gate_w=None, bias=None, w13=None, w13_scale=None, w2=None, w2_scale=None, ws13=None,
            ws13_scale=None, ws2=None, ws2_scale=None, packed=False) -> MoeWeights:
    return MoeWeights(*[_ptr(t) for t in (gate_w, bias, w13, w13_scale, w2, w2_scale, ws13,
                                          ws13_scale, ws2, ws2_scale)], int(bool(packed)))


def moe_workspace_bytes(cfg: MoeConfig, T: int) -> int:
    return lib().moe_workspace_bytes(ctypes.byref(cfg), T)


def moe_gate(cfg, T, x, gate_w, bias, logits, topk_idx, topk_w, ws, stream=None):
    _check(lib().moe_gate(ctypes.byref(cfg), T, _ptr(x), _ptr(gate_w), _ptr(bias), _ptr(logits),
                          _ptr(topk_idx), _ptr(topk_w), _ptr(ws), _nbytes(ws) if ws is not None
                          else 0, _stream(stream)))


def moe_permute(cfg, T, topk_idx, counts, offsets, perm, pos, ws, stream=None):
    _check(lib().moe_permute(ctypes.byref(cfg), T, _ptr(topk_idx), _ptr(counts), _ptr(offsets),
                             _ptr(perm), _ptr(pos), _ptr(ws),
                             _nbytes(ws) if ws is not None else 0, _stream(stream)))


def moe_expert_ffn(cfg, T, x, perm, offsets, w: MoeWeights, y, y_shared, ws, stream=None):
    _check(lib().moe_expert_ffn(ctypes.byref(cfg), T, _ptr(x), _ptr(perm), _ptr(offsets),
                                ctypes.byref(w), _ptr(y), _ptr(y_shared), _ptr(ws),
                                _nbytes(ws) if ws is not None else 0, _stream(stream)))


def moe_combine(cfg, T, y, y_shared, pos, topk_w, out, stream=None):
    _check(lib().moe_combine(ctypes.byref(cfg), T, _ptr(y), _ptr(y_shared), _ptr(pos),
                             _ptr(topk_w), _ptr(out), _stream(stream)))


def moe_forward(cfg, T, x, w: MoeWeights, out, ws, logits=None, topk_idx=None, topk_w=None,
                counts=None, perm=None, stream=None):
    _check(lib().moe_forward(ctypes.byref(cfg), T, _ptr(x), ctypes.byref(w), _ptr(out),
                             _ptr(logits), _ptr(topk_idx), _ptr(topk_w), _ptr(counts), _ptr(perm),
                             _ptr(ws), _nbytes(ws) if ws is not None else 0, _stream(stream)))


def moe_forward_decode_fused(cfg, T, x, w: MoeWeights, out, ws, logits=None, topk_idx=None,
                             topk_w=None, counts=None, perm=None, stream=None):
    """moe_forward of a decode batch (T <= 32, bf16, packed) as one launch."""
    _check(lib().moe_forward_decode_fused(ctypes.byref(cfg), T, _ptr(x), ctypes.byref(w),
                                          _ptr(out), _ptr(logits), _ptr(topk_idx),
                                          _ptr(topk_w), _ptr(counts), _ptr(perm), _ptr(ws),
                                          _nbytes(ws) if ws is not None else 0,
                                          _stream(stream)))


# Bytes of the static workspace of moe_forward_noalloc (include/moe.h).
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20


def moe_forward_noalloc(cfg, T, x, w: MoeWeights, out, logits=None, topk_idx=None, topk_w=None,
                        counts=None, perm=None, stream=None):
    """moe_forward on the library's static per-GPU workspace (no allocation)."""
    _check(lib().moe_forward_noalloc(ctypes.byref(cfg), T, _ptr(x), ctypes.byref(w), _ptr(out),
                                     _ptr(logits), _ptr(topk_idx), _ptr(topk_w), _ptr(counts),
                                     _ptr(perm), _stream(stream)))


def moe_forward_overlap(cfg, T, x, w: MoeWeights, out, ws, shared_stream, logits=None,
                        topk_idx=None, topk_w=None, counts=None, perm=None, stream=None):
    """moe_forward with the shared expert on shared_stream (a torch stream or
    a raw hipStream_t), joined back into stream before the combine."""
    _check(lib().moe_forward_overlap(ctypes.byref(cfg), T, _ptr(x), ctypes.byref(w), _ptr(out),
                                     _ptr(logits), _ptr(topk_idx), _ptr(topk_w), _ptr(counts),
                                     _ptr(perm), _ptr(ws), _nbytes(ws) if ws is not None else 0,
                                     _stream(stream), _stream(shared_stream)))


def moe_backward_workspace_bytes(cfg, T) -> int:
    return lib().moe_backward_workspace_bytes(ctypes.byref(cfg), T)


def moe_backward(cfg, T, x, w: MoeWeights, logits, topk_idx, topk_w, perm, offsets, pos, y, dout,
                 dx, dgate_w, dw13, dw2, dws13, dws2, ws, stream=None):
    _check(lib().moe_backward(ctypes.byref(cfg), T, _ptr(x), ctypes.byref(w), _ptr(logits),
                              _ptr(topk_idx), _ptr(topk_w), _ptr(perm), _ptr(offsets), _ptr(pos),
                              _ptr(y), _ptr(dout), _ptr(dx), _ptr(dgate_w), _ptr(dw13),
                              _ptr(dw2), _ptr(dws13), _ptr(dws2), _ptr(ws),
                              _nbytes(ws) if ws is not None else 0, _stream(stream)))


def moe_quantize_act(cfg, rows, x, xq, xs, stream=None):
    _check(lib().moe_quantize_act(ctypes.byref(cfg), rows, _ptr(x), _ptr(xq), _ptr(xs),
                                  _stream(stream)))


def moe_expert_ffn_backward_workspace_bytes(cfg: MoeConfig, T: int) -> int:
    return lib().moe_expert_ffn_backward_workspace_bytes(ctypes.byref(cfg), T)


def moe_expert_ffn_backward(cfg, T, x, perm, offsets, w: MoeWeights, dy, dy_shared, dx, dx_shared,
                            dw13, dw2, dws13, dws2, ws, stream=None):
    _check(lib().moe_expert_ffn_backward(ctypes.byref(cfg), T, _ptr(x), _ptr(perm), _ptr(offsets),
                                         ctypes.byref(w), _ptr(dy), _ptr(dy_shared), _ptr(dx),
                                         _ptr(dx_shared), _ptr(dw13), _ptr(dw2), _ptr(dws13),
                                         _ptr(dws2), _ptr(ws), _nbytes(ws) if ws is not None else 0,
                                         _stream(stream)))


def moe_bias_update(cfg, counts, gamma, bias, stream=None):
    _check(lib().moe_bias_update(ctypes.byref(cfg), _ptr(counts), float(gamma), _ptr(bias),
                                 _stream(stream)))


def moe_packed_bytes(cfg: MoeConfig, which: int) -> int:
    return lib().moe_packed_bytes(ctypes.byref(cfg), which)


def moe_pack_weight(cfg, which, src, dst, stream=None):
    _check(lib().moe_pack_weight(ctypes.byref(cfg), which, _ptr(src), _ptr(dst), _stream(stream)))


def moe_get_device_error(ws, stream=None) -> int:
    """Returns the status (MOE_OK or MOE_ERR_DEVICE_CHECK) instead of raising."""
    return lib().moe_get_device_error(_ptr(ws), _nbytes(ws), _stream(stream))


def moe_kernel_timer_enable(on: bool, only: Optional[str] = None) -> None:
    _check(lib().moe_kernel_timer_enable(1 if on else 0, only.encode() if only else None))


MOE_GATE_SPLIT, MOE_GATE_FUSED = 0, 1


def moe_set_gate_mode(mode: int) -> None:
    _check(lib().moe_set_gate_mode(int(mode)))


def moe_kernel_timer_read() -> dict:
    """{kernel name: (summed ms, launches)} since the last read."""
    L = lib()
    cap = 64
    names = (ctypes.c_char_p * cap)()
    ms = (ctypes.c_double * cap)()
    cnt = (ctypes.c_int64 * cap)()
    n = L.moe_kernel_timer_read(cap, names, ms, cnt)
    return {names[i].decode(): (ms[i], int(cnt[i])) for i in range(min(n, cap))}


def moe_strerror(status: int) -> str:
    return lib().moe_strerror(status).decode()


def moe_last_error() -> str:
    return lib().moe_last_error().decode()
