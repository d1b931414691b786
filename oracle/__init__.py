"""Python access to the fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the CPU
baseline leg of the benchmark, never by the product path.  It shares no code
with the HIP library; both only read the same generator-made input arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")

F32, BF16, E4M3 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc: OpenMP, no fp contraction, no fast-math."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                               os.path.join(_HERE, "oracle.c"), "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


class Cfg(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("E", ctypes.c_int32), ("G", ctypes.c_int32),
                ("TG", ctypes.c_int32), ("K", ctypes.c_int32), ("I", ctypes.c_int32),
                ("Is", ctypes.c_int32), ("rho", ctypes.c_double)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        L.oracle_threads.restype = ctypes.c_int
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_decode.restype = ctypes.c_double
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_quant_rows.argtypes = [i64, i32, vp, vp, vp]
        L.oracle_quant_rows.restype = None
        L.oracle_quant_rows_pow2.argtypes = [i64, i32, vp, vp, vp]
        L.oracle_quant_rows_pow2.restype = None
        L.oracle_logits.argtypes = [i64, i32, i32, vp, i32, vp, vp]
        L.oracle_logits.restype = None
        L.oracle_route_f64.argtypes = [ctypes.POINTER(Cfg), i64, vp, vp, vp, vp, vp]
        L.oracle_route_f64.restype = ctypes.c_int
        L.oracle_route_f32.argtypes = [ctypes.POINTER(Cfg), i64, vp, vp, vp, vp]
        L.oracle_route_f32.restype = ctypes.c_int
        L.oracle_permute.argtypes = [i64, i32, i32, vp, vp, vp, vp, vp]
        L.oracle_permute.restype = ctypes.c_int
        L.oracle_layer.argtypes = [ctypes.POINTER(Cfg), i64, vp, vp, i32, vp, vp,
                                   vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp]
        L.oracle_layer.restype = ctypes.c_int
        L.oracle_ffn.argtypes = [ctypes.POINTER(Cfg), i64, vp, vp, vp, i32, vp, vp, vp, vp,
                                 vp, vp, vp, vp, i32, i32, vp]
        L.oracle_ffn.restype = ctypes.c_int
        L.oracle_combine.argtypes = [i64, i32, i32, vp, vp, vp, vp, vp]
        L.oracle_combine.restype = None
        L.oracle_ffn_backward.argtypes = [ctypes.POINTER(Cfg), i32, i64, vp, vp, i32, vp, vp, vp,
                                          vp, vp, i32, vp, vp, vp]
        L.oracle_ffn_backward.restype = ctypes.c_int
        L.oracle_ffn_backward_fp8.argtypes = [ctypes.POINTER(Cfg), i32, i64, vp, vp, i32, vp,
                                              vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp]
        L.oracle_ffn_backward_fp8.restype = ctypes.c_int
        L.oracle_ffn_backward_entries.argtypes = [ctypes.POINTER(Cfg), i32, i64, vp, vp, i32, vp,
                                                  vp, vp, vp, vp, i32, i64, vp, vp, vp, vp]
        L.oracle_ffn_backward_entries.restype = ctypes.c_int
        L.oracle_bias_update.argtypes = [i32, vp, ctypes.c_float, vp, vp]
        L.oracle_bias_update.restype = ctypes.c_int
        _lib = L
    return _lib


def _c(a, dtype=None):
    a = np.ascontiguousarray(a if dtype is None else np.asarray(a, dtype=dtype))
    return a


def _p(a):
    return None if a is None else a.ctypes.data


def cfg_of(c) -> Cfg:
    """Oracle shape record from a synth.MoEConfig (or any object with the fields)."""
    return Cfg(c.H, c.E, c.G, c.TG, c.K, c.I, c.Is, float(c.rho))


def dtype_code(arr: np.ndarray, declared: str) -> int:
    return _WD[declared]


def threads() -> int:
    return lib().oracle_threads()


def e4m3_decode(code: int) -> float:
    return lib().oracle_e4m3_decode(code)


def e4m3_encode(v: float) -> int:
    return lib().oracle_e4m3_encode(v)


# Weight dtypes of the configs: "fp8" is e4m3 with block scales a / 448
# (R7), "fp8e8m0" e4m3 with power-of-two block scales (R14); both decode as
# code * scale.
_WD = {"f32": F32, "bf16": BF16, "fp8": E4M3, "fp8e8m0": E4M3}
# Activation quantisation mode of the fp8 data path per weight dtype.
_QUANT_MODE = {"fp8": 1, "fp8e8m0": 2}


def _quant_mode(cfg, quant_act) -> int:
    if not quant_act:
        return 0
    if cfg.wdtype not in _QUANT_MODE:
        raise ValueError(f"activation quantisation needs fp8 weights, not {cfg.wdtype}")
    return _QUANT_MODE[cfg.wdtype]


def quant_rows(v: np.ndarray, pow2: bool = False):
    """1x128 e4m3 quantisation of a float32 [rows, cols] array -> (codes u8,
    scales f32); pow2 selects power-of-two scales (R14) instead of a / 448."""
    v = _c(v, np.float32)
    rows, cols = v.shape
    assert cols % 128 == 0
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, cols // 128), np.float32)
    f = lib().oracle_quant_rows_pow2 if pow2 else lib().oracle_quant_rows
    f(rows, cols, _p(v), _p(q), _p(s))
    return q, s


def logits(x: np.ndarray, x_kind: str, gate_w: np.ndarray) -> np.ndarray:
    """x [T,H] (float32, or bf16 bits as uint16) times gate_w [E,H]^T in fp64."""
    x = _c(x)
    gate_w = _c(gate_w, np.float32)
    T, H = x.shape
    E = gate_w.shape[0]
    out = np.empty((T, E), np.float64)
    lib().oracle_logits(T, H, E, _p(x), F32 if x_kind == "f32" else BF16, _p(gate_w), _p(out))
    return out


def route_f64(cfg, lg: np.ndarray, bias: np.ndarray):
    """fp64 router -> (idx int32 [T,K], w float64 [T,K], margin float64 [T])."""
    lg = _c(lg, np.float64)
    bias = _c(bias, np.float32)
    T = lg.shape[0]
    idx = np.empty((T, cfg.K), np.int32)
    w = np.empty((T, cfg.K), np.float64)
    m = np.empty(T, np.float64)
    rc = lib().oracle_route_f64(ctypes.byref(cfg_of(cfg)), T, _p(lg), _p(bias), _p(idx), _p(w), _p(m))
    if rc:
        raise ValueError(f"oracle_route_f64 rejected the configuration (rc={rc})")
    return idx, w, m


def route_f32(cfg, lg32: np.ndarray, bias: np.ndarray):
    """Router under the fp32 selection contract -> (idx int32 [T,K], w float64 [T,K])."""
    lg32 = _c(lg32, np.float32)
    bias = _c(bias, np.float32)
    T = lg32.shape[0]
    idx = np.empty((T, cfg.K), np.int32)
    w = np.empty((T, cfg.K), np.float64)
    rc = lib().oracle_route_f32(ctypes.byref(cfg_of(cfg)), T, _p(lg32), _p(bias), _p(idx), _p(w))
    if rc:
        raise ValueError(f"oracle_route_f32 rejected the configuration (rc={rc})")
    return idx, w


def permute(idx: np.ndarray, E: int):
    """-> (counts [E], offsets [E+1], perm [T*K], pos [T*K]), all int32."""
    idx = _c(idx, np.int32)
    T, K = idx.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(T * K, np.int32)
    pos = np.empty(T * K, np.int32)
    rc = lib().oracle_permute(T, K, E, _p(idx), _p(counts), _p(offsets), _p(perm), _p(pos))
    if rc:
        raise ValueError("oracle_permute: expert index out of range")
    return counts, offsets, perm, pos


def layer(cfg, inp: dict, idx: np.ndarray, w: np.ndarray, tokens=None, quant_act=False):
    """Layer output (fp64) for the listed tokens (default: all) -> [n_tok, H]."""
    x = _c(inp["x"])
    T = x.shape[0]
    tokens = np.arange(T, dtype=np.int64) if tokens is None else _c(tokens, np.int64)
    idx = _c(idx, np.int32)
    w = _c(w, np.float64)
    wd = _WD[cfg.wdtype]
    xd = F32 if cfg.act == "f32" else BF16
    g = lambda k: None if inp.get(k) is None else _c(inp[k])
    arrs = [g(k) for k in ("w13", "w13_s", "w2", "w2_s", "ws13", "ws13_s", "ws2", "ws2_s")]
    out = np.empty((len(tokens), cfg.H), np.float64)
    rc = lib().oracle_layer(ctypes.byref(cfg_of(cfg)), len(tokens), _p(tokens), _p(x), xd,
                            _p(idx), _p(w), *[_p(a) for a in arrs], wd,
                            _quant_mode(cfg, quant_act), _p(out))
    if rc:
        raise ValueError("oracle_layer failed (bad expert index or allocation)")
    return out


def ffn(cfg, inp: dict, tokens, experts, quant_act=False):
    """FFN_{experts[n]}(x_{tokens[n]}) in fp64 -> [n, H]; expert -1 = shared."""
    x = _c(inp["x"])
    tokens = _c(tokens, np.int64)
    experts = _c(experts, np.int32)
    wd = _WD[cfg.wdtype]
    xd = F32 if cfg.act == "f32" else BF16
    g = lambda k: None if inp.get(k) is None else _c(inp[k])
    arrs = [g(k) for k in ("w13", "w13_s", "w2", "w2_s", "ws13", "ws13_s", "ws2", "ws2_s")]
    out = np.empty((len(tokens), cfg.H), np.float64)
    rc = lib().oracle_ffn(ctypes.byref(cfg_of(cfg)), len(tokens), _p(tokens), _p(experts), _p(x),
                          xd, *[_p(a) for a in arrs], wd, _quant_mode(cfg, quant_act), _p(out))
    if rc:
        raise ValueError("oracle_ffn failed (bad expert index or allocation)")
    return out


def combine(y: np.ndarray, ys, pos: np.ndarray, w: np.ndarray, K: int) -> np.ndarray:
    """out[t] = ys[t] + sum_k w[t,k] y[pos[t*K+k]] in fp64 (y, ys as float64 arrays)."""
    y = _c(y, np.float64)
    ys = None if ys is None else _c(ys, np.float64)
    pos = _c(pos, np.int32)
    w = _c(w, np.float64)
    T = w.shape[0]
    H = y.shape[1]
    out = np.empty((T, H), np.float64)
    lib().oracle_combine(T, K, H, _p(y), _p(ys), _p(pos), _p(w), _p(out))
    return out


def forward(cfg, inp: dict, tokens=None, quant_act=False):
    """Whole layer on the listed tokens with the oracle's own fp64 routing.
    Returns dict(logits, idx, w, margin, out)."""
    x = inp["x"] if tokens is None else inp["x"][np.asarray(tokens)]
    lg = logits(x, cfg.act, inp["gate_w"])
    idx, w, m = route_f64(cfg, lg, inp["bias"])
    sub = dict(inp)
    sub["x"] = x
    out = layer(cfg, sub, idx, w, quant_act=quant_act)
    return {"logits": lg, "idx": idx, "w": w, "margin": m, "out": out}


def bias_update(counts: np.ndarray, gamma: float, bias: np.ndarray) -> np.ndarray:
    """One load-balancing step of the fp32 selection bias -> new bias [E] float32.

    Each expert's bias moves by gamma toward the mean load sum(counts)/E (up
    when below it, down when above, unchanged at it), rounded once to fp32;
    gamma is taken as an fp32 value.
    """
    counts = _c(counts, np.int32)
    bias = _c(bias, np.float32)
    E = counts.shape[0]
    assert bias.shape == (E,)
    out = np.empty(E, np.float32)
    rc = lib().oracle_bias_update(E, _p(counts), float(np.float32(gamma)), _p(bias), _p(out))
    if rc:
        raise ValueError("oracle_bias_update rejected its arguments")
    return out


def ffn_backward(cfg, inp: dict, expert: int, tokens, dy, want=("dx", "dw13", "dw2"),
                 quant_act=False):
    """Exact (fp64) backward of one SwiGLU expert (-1: shared) over rows with
    inputs x[tokens[r]] and output gradients dy [n, H] -> dict of dx [n, H],
    dw13 [2 n_e, H], dw2 [H, n_e] (the weight gradients summed over the rows).
    e4m3 weights: the backward of the dequantised weights, or with quant_act
    the FP8 backward (R15: x, dy, [dg du], h quantised in tiles of 128 along
    each GEMM's contraction; the rows are the expert's, in sorted order)."""
    x = _c(inp["x"])
    tokens = _c(tokens, np.int64)
    dy = _c(dy, np.float64)
    n = len(tokens)
    H = cfg.H
    ne = cfg.Is if expert < 0 else cfg.I
    if cfg.wdtype in _QUANT_MODE:
        xd = F32 if cfg.act == "f32" else BF16
        g = lambda k: None if inp.get(k) is None else _c(inp[k])
        arrs = [g(k) for k in ("w13", "w13_s", "w2", "w2_s", "ws13", "ws13_s", "ws2", "ws2_s")]
        out = {"dx": np.empty((n, H)) if "dx" in want else None,
               "dw13": np.empty((2 * ne, H)) if "dw13" in want else None,
               "dw2": np.empty((H, ne)) if "dw2" in want else None}
        rc = lib().oracle_ffn_backward_fp8(ctypes.byref(cfg_of(cfg)), int(expert), n,
                                           _p(tokens), _p(x), xd, _p(dy),
                                           *[_p(a) for a in arrs], _quant_mode(cfg, quant_act),
                                           _p(out["dx"]), _p(out["dw13"]), _p(out["dw2"]))
        if rc:
            raise ValueError("oracle_ffn_backward_fp8 rejected its arguments")
        return {k: v for k, v in out.items() if v is not None}
    if quant_act:
        raise ValueError("the quantised backward needs e4m3 weights")
    wd = {"f32": F32, "bf16": BF16}[cfg.wdtype]
    xd = F32 if cfg.act == "f32" else BF16
    g = lambda k: None if inp.get(k) is None else _c(inp[k])
    out = {"dx": np.empty((n, H)) if "dx" in want else None,
           "dw13": np.empty((2 * ne, H)) if "dw13" in want else None,
           "dw2": np.empty((H, ne)) if "dw2" in want else None}
    rc = lib().oracle_ffn_backward(ctypes.byref(cfg_of(cfg)), int(expert), n, _p(tokens), _p(x),
                                   xd, _p(dy), _p(g("w13")), _p(g("w2")), _p(g("ws13")),
                                   _p(g("ws2")), wd, _p(out["dx"]), _p(out["dw13"]),
                                   _p(out["dw2"]))
    if rc:
        raise ValueError("oracle_ffn_backward rejected its arguments")
    return {k: v for k, v in out.items() if v is not None}


def ffn_backward_entries(cfg, inp: dict, expert: int, tokens, dy, which, rows, cols):
    """Selected entries of the expert's weight gradients (fp64), one by one:
    which[q] = 0 -> dW13[rows[q], cols[q]], 1 -> dW2[rows[q], cols[q]]."""
    x = _c(inp["x"])
    tokens = _c(tokens, np.int64)
    dy = _c(dy, np.float64)
    which, rows, cols = (_c(a, np.int32) for a in (which, rows, cols))
    wd = {"f32": F32, "bf16": BF16}[cfg.wdtype]
    xd = F32 if cfg.act == "f32" else BF16
    g = lambda k: None if inp.get(k) is None else _c(inp[k])
    out = np.empty(len(which), np.float64)
    rc = lib().oracle_ffn_backward_entries(ctypes.byref(cfg_of(cfg)), int(expert), len(tokens),
                                           _p(tokens), _p(x), xd, _p(dy), _p(g("w13")),
                                           _p(g("w2")), _p(g("ws13")), _p(g("ws2")), wd,
                                           len(which), _p(which), _p(rows), _p(cols), _p(out))
    if rc:
        raise ValueError("oracle_ffn_backward_entries rejected its arguments")
    return out


def routing_weights(cfg, lg: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Routing weights of the chosen experts from the logits, fp64 ("从 1024 块
    GPU 到 558 万美元：拆解 DeepSeek-V3 的算法-系统协同设计", section 2.2, MoEGate): the
    unbiased sigmoid scores s of the chosen experts, divided by their sum (plus
    1e-20) when top_k > 1, times routed_scaling_factor -> [T, K]."""
    lg = np.asarray(lg, np.float64)
    idx = np.asarray(idx)
    s = 1.0 / (1.0 + np.exp(-np.take_along_axis(lg, idx.astype(np.int64), axis=1)))
    if cfg.K > 1:
        s = s / (s.sum(axis=1, keepdims=True) + 1e-20)
    return s * cfg.rho


def round_bf16(v: np.ndarray) -> np.ndarray:
    """Values rounded to fp32, then to bf16 (nearest, ties to even), as fp64."""
    u = np.ascontiguousarray(v, np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def layer_backward(cfg, inp: dict, idx: np.ndarray, dout: np.ndarray, tokens=None,
                   want=("dx", "dgate_w", "dw"), quant_act=False) -> dict:
    """Exact fp64 gradients of L = sum_t <dout_t, out_t> for the layer with
    its routing held at idx (the top-k choice is piecewise constant in the
    inputs: the gradient reaches the gate only through the chosen experts'
    weights).  out_t = shared(x_t) + sum_k w_tk FFN_idx[t,k](x_t) with w from
    routing_weights; the bias only selects and gets no gradient.
    Returns dx [T, H], dgate_w [E, H], and with "dw" wanted dw13 [E, 2I, H],
    dw2 [E, H, I] and, with a shared expert, dws13 [2Is, H], dws2 [H, Is].
    With tokens (indices into x, idx and dout), L sums over those tokens only:
    dx holds their rows, and dgate_w[e] is exact for an expert e all of whose
    tokens are listed.
    e4m3 weights with quant_act: the FP8 layer -- the expert outputs y of the
    activation-quantised forward (F2) enter the routing-weight gradient, and
    each expert's backward is the FP8 backward (R15) of its rows, in sorted
    order, with dy = w dout ("深入理解 DeepSeek-V3…", section 3.2); the
    combine, routing-weight and gate terms are the formulas above.  The
    routed rows' dy reach the expert backward as bf16 values (its operands'
    interface type), so their e4m3 codes are decided from bf16-rounded dy."""
    if tokens is not None:
        tokens = np.asarray(tokens, np.int64)
        inp = dict(inp, x=np.asarray(inp["x"])[tokens])
        idx, dout = np.asarray(idx)[tokens], np.asarray(dout)[tokens]
    T, H, E, K, I = inp["x"].shape[0], cfg.H, cfg.E, cfg.K, cfg.I
    x = np.asarray(inp["x"])
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64) if x.dtype == np.uint16 \
        else x.astype(np.float64)
    gw = np.asarray(inp["gate_w"], np.float64)
    dout = np.asarray(dout, np.float64)
    idx = np.asarray(idx, np.int64)
    lg = logits(x, cfg.act, inp["gate_w"])
    s = 1.0 / (1.0 + np.exp(-np.take_along_axis(lg, idx, axis=1)))          # [T, K]
    w = routing_weights(cfg, lg, idx)
    tok = np.repeat(np.arange(T), K)
    y = ffn(cfg, inp, tok, idx.ravel().astype(np.int32),
            quant_act=quant_act).reshape(T, K, H)                            # expert outputs
    dw = np.einsum("th,tkh->tk", dout, y)
    if K > 1:   # w_k = rho s_k / D, D = sum_j s_j + 1e-20
        D = s.sum(axis=1, keepdims=True) + 1e-20
        ds = cfg.rho * (dw / D - (dw * s).sum(axis=1, keepdims=True) / D ** 2)
    else:
        ds = cfg.rho * dw
    dlg = ds * s * (1.0 - s)                                                 # d logit of the chosen
    wdw = "dw" in want
    parts = ("dx", "dw13", "dw2") if wdw else ("dx",)
    out = {"dgate_w": np.zeros((E, H))}
    if wdw:
        out["dw13"], out["dw2"] = np.zeros((E, 2 * I, H)), np.zeros((E, H, I))
    np.add.at(out["dgate_w"], idx.ravel(), dlg.ravel()[:, None] * xf[tok])
    dx = np.einsum("tk,tkh->th", dlg, gw[idx])
    if "dx" not in want and not wdw:
        return out
    for e in np.unique(idx):
        rows = np.flatnonzero(idx.ravel() == e)
        dy = w.ravel()[rows, None] * dout[tok[rows]]
        b = ffn_backward(cfg, inp, int(e), tok[rows], round_bf16(dy) if quant_act else dy,
                         want=parts, quant_act=quant_act)
        if wdw:
            out["dw13"][e], out["dw2"][e] = b["dw13"], b["dw2"]
        np.add.at(dx, tok[rows], b["dx"])
    if cfg.Is:
        b = ffn_backward(cfg, inp, -1, np.arange(T), dout, want=parts, quant_act=quant_act)
        if wdw:
            out["dws13"], out["dws2"] = b["dw13"], b["dw2"]
        dx += b["dx"]
    out["dx"] = dx
    return out
