"""Helpers for the GPU parity tests: run the C-ABI entry points on device
tensors and compare with the oracle on the same generator-made inputs."""
import sys

import numpy as np
import torch

import oracle
import synth
import sparse_mixture_experts_30_amd as moe
from synth import device as sd

DEV = "cuda"


def log(msg):
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# fp8 layer against the oracle that also quantises x and h per 1x128 tile
# (the kernels' own data path): the remaining error is accumulation order in
# fp32 and the bf16 rounding of y and out, a few 1e-3; a mis-scaled tile
# (a wrong activation or weight scale) moves a token by far more.
FP8_QUANT_TOL = 1e-2


def worst_row_rel(a, b):
    """Largest per-row relative L2 error of a against b ([n, H])."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float((np.linalg.norm(a - b, axis=1) /
                  np.maximum(np.linalg.norm(b, axis=1), 1e-300)).max())


def host(t) -> np.ndarray:
    """Device tensor -> numpy (bf16 widened exactly to float32)."""
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


def sync():
    torch.cuda.synchronize()


def run_gate(cfg, dev, T, ws=None):
    E, K = cfg.E, cfg.K
    lg = torch.empty((T, E), dtype=torch.float32, device=DEV)
    idx = torch.empty((T, K), dtype=torch.int32, device=DEV)
    w = torch.empty((T, K), dtype=torch.float32, device=DEV)
    ws = sd.workspace(cfg, T) if ws is None else ws
    moe.moe_gate(sd.moe_config(cfg), T, dev["x"], dev["gate_w"], dev["bias"], lg, idx, w, ws)
    sync()
    return host(lg), host(idx), host(w)


def run_permute(cfg, idx_np, ws=None):
    T = idx_np.shape[0]
    N = T * cfg.K
    idx = torch.from_numpy(np.ascontiguousarray(idx_np, np.int32)).to(DEV)
    counts = torch.empty(cfg.E, dtype=torch.int32, device=DEV)
    offsets = torch.empty(cfg.E + 1, dtype=torch.int32, device=DEV)
    perm = torch.empty(max(N, 1), dtype=torch.int32, device=DEV)
    pos = torch.empty(max(N, 1), dtype=torch.int32, device=DEV)
    ws = sd.workspace(cfg, T) if ws is None else ws
    moe.moe_permute(sd.moe_config(cfg), T, idx, counts, offsets, perm, pos, ws)
    status = moe.moe_get_device_error(ws)
    return host(counts), host(offsets), host(perm)[:N], host(pos)[:N], status


def check_routing(cfg, x_host, gate_w, bias, lg_gpu, idx_gpu, w_gpu, label=""):
    """Logits within 1e-5 relative L2 of the fp64 oracle; indices bit-exact
    when the oracle re-selects from the GPU's fp32 logits; weights within
    1e-6 * rho; the oracle's own fp64 routing differs only at near-ties."""
    lg_ref = oracle.logits(x_host, cfg.act, gate_w)
    r = rel_l2(lg_gpu, lg_ref)
    idx_c, w_c = oracle.route_f32(cfg, lg_gpu, bias)
    exact = np.array_equal(idx_c, idx_gpu)
    werr = float(np.abs(w_gpu - w_c).max())
    idx_o, _, margin = oracle.route_f64(cfg, lg_ref, bias)
    # The chosen set is what the layer uses; slot order between two chosen
    # experts with near-equal scores may differ between fp32 and fp64.
    differ = np.any(np.sort(idx_o, 1) != np.sort(idx_gpu, 1), axis=1)
    order_only = int(np.sum(np.any(idx_o != idx_gpu, axis=1) & ~differ))
    log(f"[routing {label}] logits relL2={r:.3e} idx exact={exact} w maxerr={werr:.3e} "
        f"independent set differs={int(differ.sum())}/{len(differ)} (slot order only: "
        f"{order_only}) max margin of differing={float(margin[differ].max()) if differ.any() else 0:.2e}")
    assert r <= 1e-5, r
    assert exact, np.argwhere(idx_c != idx_gpu)[:5]
    assert werr <= 1e-6 * cfg.rho, werr
    assert np.all(margin[differ] < 1e-5)
    assert differ.mean() <= 0.01
    return lg_ref


def layer_reference(cfg, inp, idx_gpu_tok, tokens, quant_act=False):
    """Oracle layer output on `tokens` with the oracle's own fp64 routing.
    Tokens whose routing sits within 1e-5 of a tie may legitimately be routed
    differently by fp32 arithmetic: for those, the GPU's (equally valid)
    choice is used with fp64 weights.  Returns (out [n, H], n_alternative)."""
    x_sub = inp["x"][tokens]
    lg = oracle.logits(x_sub, cfg.act, inp["gate_w"])
    idx_o, w_o, margin = oracle.route_f64(cfg, lg, inp["bias"])
    differ = np.any(np.sort(idx_o, 1) != np.sort(idx_gpu_tok, 1), axis=1)
    assert np.all(margin[differ] < 1e-5), margin[differ]
    idx_ref = np.where(differ[:, None], idx_gpu_tok, idx_o).astype(np.int32)
    s = 1.0 / (1.0 + np.exp(-lg))
    sel = np.take_along_axis(s, idx_ref.astype(np.int64), 1)
    w_alt = sel / (sel.sum(1, keepdims=True) + 1e-20) if cfg.K > 1 else sel
    w_ref = np.where(differ[:, None], w_alt * cfg.rho, w_o)
    sub = dict(inp)
    sub["x"] = x_sub
    out = oracle.layer(cfg, sub, idx_ref, w_ref, quant_act=quant_act)
    return out, int(differ.sum())


def run_forward(cfg, dev, T, ws=None, with_routing=True):
    out = torch.empty((T, cfg.H), dtype=torch.bfloat16 if cfg.act == "bf16" else torch.float32,
                      device=DEV)
    ws = sd.workspace(cfg, T) if ws is None else ws
    lg = idx = w = counts = perm = None
    if with_routing:
        lg = torch.empty((T, cfg.E), dtype=torch.float32, device=DEV)
        idx = torch.empty((T, cfg.K), dtype=torch.int32, device=DEV)
        w = torch.empty((T, cfg.K), dtype=torch.float32, device=DEV)
        counts = torch.empty(cfg.E, dtype=torch.int32, device=DEV)
        perm = torch.empty(T * cfg.K, dtype=torch.int32, device=DEV)
    W = sd.weights_struct(dev)
    moe.moe_forward(sd.moe_config(cfg), T, dev["x"], W, out, ws, logits=lg, topk_idx=idx,
                    topk_w=w, counts=counts, perm=perm)
    sync()
    # no expert index out of range, no completion wait given up
    assert moe.moe_get_device_error(ws) == moe.MOE_OK, moe.moe_last_error()
    r = {"out": host(out)}
    if with_routing:
        r.update(logits=host(lg), idx=host(idx), w=host(w), counts=host(counts), perm=host(perm))
    return r


def random_routing(T, K, E, seed, skew=False):
    """Seeded routing indices with K distinct experts per token; skew puts
    expert 0 first on every token."""
    keys = synth.words(T * E, seed, synth.T_TEST, 31).reshape(T, E)
    idx = np.argsort(keys, axis=1, kind="stable")[:, :K].astype(np.int32)
    if skew:
        for t in range(T):
            row = [0] + [e for e in idx[t] if e != 0][:K - 1]
            idx[t] = row
    return idx
