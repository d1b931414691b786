"""Seeded synthetic inputs for the MoE layer forward (shared by the oracle side
and the HIP side; holds none of the layer's arithmetic).

The workload shapes follow the DeepSeek-V3 pages: hidden size 7168 ("7K",
Insights into DeepSeek-V3 digest, section 3.1), 256 routed experts in 8 groups
with each token limited to 4 groups (same digest, section 3.3), 8 routed + 1
shared expert per token (section 3.1), expert FFN width 2048 (the algorithm-
system co-design explainer, section 2.2), ~32 tokens per decode batch
(section 3.1) and sequence length 4096 (digest, Table 2).
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")

# Tensor ids of the generator streams.
T_X, T_WG, T_BIAS, T_W13, T_W2, T_WS13, T_WS2, T_XCAL, T_TEST = 0, 1, 2, 3, 4, 5, 6, 7, 8


def build(force: bool = True) -> str:
    """Compile libsynth.so with gcc (OpenMP; no fp contraction)."""
    if force or not os.path.exists(_SO):
        src = os.path.join(_HERE, "synth.c")
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC",
                               "-shared", src, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        vp, i64, u64, u32, d = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                ctypes.c_uint32, ctypes.c_double)
        L.synth_normal_f32.argtypes = [vp, i64, u64, u32, u32, d]
        L.synth_normal_bf16.argtypes = [vp, i64, u64, u32, u32, d]
        L.synth_uniform_f32.argtypes = [vp, i64, u64, u32, u32, d, d]
        L.synth_words.argtypes = [vp, i64, u64, u32, u32]
        L.synth_normal_e4m3_blocks.argtypes = [vp, vp, i64, i64, u64, u32, u32, d, ctypes.c_int]
        for f in (L.synth_normal_f32, L.synth_normal_bf16, L.synth_uniform_f32,
                  L.synth_words, L.synth_normal_e4m3_blocks):
            f.restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def normal_f32(n: int, seed: int, tensor: int, sub: int, std: float, out=None) -> np.ndarray:
    out = np.empty(n, np.float32) if out is None else out
    lib().synth_normal_f32(_ptr(out), n, seed, tensor, sub, std)
    return out


def normal_bf16(n: int, seed: int, tensor: int, sub: int, std: float, out=None) -> np.ndarray:
    """bf16 bit patterns (uint16)."""
    out = np.empty(n, np.uint16) if out is None else out
    lib().synth_normal_bf16(_ptr(out), n, seed, tensor, sub, std)
    return out


def uniform_f32(n: int, seed: int, tensor: int, sub: int, lo: float, hi: float) -> np.ndarray:
    out = np.empty(n, np.float32)
    lib().synth_uniform_f32(_ptr(out), n, seed, tensor, sub, lo, hi)
    return out


def words(n: int, seed: int, tensor: int, sub: int) -> np.ndarray:
    out = np.empty(n, np.uint64)
    lib().synth_words(_ptr(out), n, seed, tensor, sub)
    return out


def normal_e4m3_blocks(rows: int, cols: int, seed: int, tensor: int, sub: int, std: float,
                       q=None, s=None, pow2: bool = False):
    """e4m3 codes [rows, cols] (uint8) and fp32 scales [rows/128, cols/128]
    (scale a/448 of the block's max |v|, or with pow2 the smallest power of
    two not below it)."""
    assert rows % 128 == 0 and cols % 128 == 0
    q = np.empty((rows, cols), np.uint8) if q is None else q
    s = np.empty((rows // 128, cols // 128), np.float32) if s is None else s
    lib().synth_normal_e4m3_blocks(_ptr(q), _ptr(s), rows, cols, seed, tensor, sub, std,
                                   1 if pow2 else 0)
    return q, s


def bf16_to_f32(u16: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (u16.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    """One workload: layer shape, dtypes and input distributions."""
    name: str
    T: int
    H: int
    E: int
    G: int
    TG: int
    K: int
    I: int
    Is: int
    rho: float
    act: str          # "f32" | "bf16"      (x and the layer output)
    wdtype: str       # "f32" | "bf16" | "fp8" | "fp8e8m0"   (expert + shared weights;
                      #  fp8e8m0: e4m3 with power-of-two block scales)
    bias_lo: float
    bias_hi: float
    seed: int = 0
    bias_file: Optional[str] = None   # stored calibrated bias (Zipf loads)

    def with_T(self, T: int) -> "MoEConfig":
        return dataclasses.replace(self, T=T)

    def replace(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)

    @property
    def routed_flop_per_token(self) -> float:
        return 6.0 * self.H * self.I * self.K

    @property
    def flop_per_token(self) -> float:
        return 6.0 * self.H * (self.I * self.K + self.Is) + 2.0 * self.H * self.E


_GOLDEN = os.path.join(os.path.dirname(_HERE), "tests", "golden")

# Tiny correctness layer, all fp32.
C1 = MoEConfig("tiny-fp32-T64-H128-E16", T=64, H=128, E=16, G=4, TG=2, K=2, I=64, Is=64,
               rho=1.0, act="f32", wdtype="f32", bias_lo=-0.1, bias_hi=0.1)
# Gate + permute at the V3 shape.
C2 = MoEConfig("v3-gate-permute-T16384", T=16384, H=7168, E=256, G=8, TG=4, K=8, I=2048,
               Is=2048, rho=2.5, act="bf16", wdtype="bf16", bias_lo=-0.05, bias_hi=0.05)
# Full layer at the V3 shape, bf16.
C3 = MoEConfig("v3-layer-bf16-T4096", T=4096, H=7168, E=256, G=8, TG=4, K=8, I=2048,
               Is=2048, rho=2.5, act="bf16", wdtype="bf16", bias_lo=-0.05, bias_hi=0.05)
# Expert GEMM at a size where it is MFMA-bound (512 rows per expert).
C3X = C3.replace(name="v3-layer-bf16-T16384", T=16384)
# Decode-shaped, Zipf(1.2)-skewed loads (bias calibrated offline, stored).
C4A = C3.replace(name="v3-decode-zipf-K8-T32", T=32,
                 bias_file=os.path.join(_GOLDEN, "zipf_bias_k8.txt"))
C4B = C4A.replace(name="v3-decode-zipf-K8-T256", T=256)
C4C = C3.replace(name="v3-decode-zipf-K1-T32", T=32, K=1,
                 bias_file=os.path.join(_GOLDEN, "zipf_bias_k1.txt"))
C4D = C4C.replace(name="v3-decode-zipf-K1-T256", T=256)
# FP8 block-scaled layer.
C5 = C3.replace(name="v3-layer-fp8-T8192", T=8192, wdtype="fp8")
# The same with power-of-two block scales, which the matrix cores apply.
C5P = C5.replace(name="v3-layer-fp8e8m0-T8192", wdtype="fp8e8m0")

CONFIGS = {c.name: c for c in (C1, C2, C3, C3X, C4A, C4B, C4C, C4D, C5, C5P)}


def load_bias_file(path: str) -> np.ndarray:
    """Bias stored as hex float32 bit patterns, one per line (# comments)."""
    vals = []
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                vals.append(int(line, 16))
    return np.array(vals, dtype=np.uint32).view(np.float32)


def gen_x(cfg: MoEConfig, T: Optional[int] = None, tensor: int = T_X):
    """Token hidden states [T, H]: N(0, 1); fp32 or bf16 bits (uint16)."""
    T = cfg.T if T is None else T
    n = T * cfg.H
    if cfg.act == "f32":
        return normal_f32(n, cfg.seed, tensor, 0, 1.0).reshape(T, cfg.H)
    return normal_bf16(n, cfg.seed, tensor, 0, 1.0).reshape(T, cfg.H)


def gen_gate(cfg: MoEConfig):
    """Gate weight [E, H] fp32 ~ N(0, 1/H) and selection bias [E] fp32."""
    wg = normal_f32(cfg.E * cfg.H, cfg.seed, T_WG, 0, 1.0 / np.sqrt(cfg.H)).reshape(cfg.E, cfg.H)
    if cfg.bias_file is not None:
        b = load_bias_file(cfg.bias_file)
        assert b.shape == (cfg.E,), (b.shape, cfg.E)
    else:
        b = uniform_f32(cfg.E, cfg.seed, T_BIAS, 0, cfg.bias_lo, cfg.bias_hi)
    return wg, b


def _expert_matrix(cfg: MoEConfig, tensor: int, sub: int, rows: int, cols: int, std: float,
                   out=None, out_s=None):
    if cfg.wdtype == "f32":
        r = normal_f32(rows * cols, cfg.seed, tensor, sub, std,
                       out=None if out is None else out.reshape(-1))
        return r.reshape(rows, cols), None
    if cfg.wdtype == "bf16":
        r = normal_bf16(rows * cols, cfg.seed, tensor, sub, std,
                        out=None if out is None else out.reshape(-1))
        return r.reshape(rows, cols), None
    q, s = normal_e4m3_blocks(rows, cols, cfg.seed, tensor, sub, std, q=out, s=out_s,
                              pow2=cfg.wdtype == "fp8e8m0")
    return q, s


def _wdt(cfg):
    return {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8, "fp8e8m0": np.uint8}[cfg.wdtype]


def gen_expert_weights(cfg: MoEConfig):
    """Routed expert weights: w13 [E, 2I, H] (rows 0..I-1 gate, I..2I-1 up),
    w2 [E, H, I]; N(0, 1/fan_in).  fp8: plus scales [E, 2I/128, H/128] and
    [E, H/128, I/128]."""
    E, H, I = cfg.E, cfg.H, cfg.I
    w13 = np.empty((E, 2 * I, H), _wdt(cfg))
    w2 = np.empty((E, H, I), _wdt(cfg))
    s13 = s2 = None
    if cfg.wdtype in ("fp8", "fp8e8m0"):
        s13 = np.empty((E, 2 * I // 128, H // 128), np.float32)
        s2 = np.empty((E, H // 128, I // 128), np.float32)
    for e in range(E):
        _expert_matrix(cfg, T_W13, e, 2 * I, H, 1.0 / np.sqrt(H), out=w13[e],
                       out_s=None if s13 is None else s13[e])
        _expert_matrix(cfg, T_W2, e, H, I, 1.0 / np.sqrt(I), out=w2[e],
                       out_s=None if s2 is None else s2[e])
    return w13, s13, w2, s2


def gen_shared_weights(cfg: MoEConfig):
    """Shared expert: ws13 [2Is, H], ws2 [H, Is] (+ scales for fp8)."""
    if cfg.Is == 0:
        return None, None, None, None
    ws13, ss13 = _expert_matrix(cfg, T_WS13, 0, 2 * cfg.Is, cfg.H, 1.0 / np.sqrt(cfg.H))
    ws2, ss2 = _expert_matrix(cfg, T_WS2, 0, cfg.H, cfg.Is, 1.0 / np.sqrt(cfg.Is))
    return ws13, ss13, ws2, ss2


def gen_inputs(cfg: MoEConfig, T: Optional[int] = None, ffn: bool = True) -> dict:
    """All host inputs of one workload as numpy arrays."""
    d = {"cfg": cfg}
    d["x"] = gen_x(cfg, T)
    d["gate_w"], d["bias"] = gen_gate(cfg)
    if ffn:
        d["w13"], d["w13_s"], d["w2"], d["w2_s"] = gen_expert_weights(cfg)
        d["ws13"], d["ws13_s"], d["ws2"], d["ws2_s"] = gen_shared_weights(cfg)
    return d
