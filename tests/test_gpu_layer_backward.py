"""GPU parity of the layer backward (moe_backward) against the fp64 oracle:
dx, the gate weight's gradient and every expert weight gradient, with the
routing the GPU's own forward chose (moe_gate, moe_permute, moe_expert_ffn);
experts without rows must get exact zeros."""
import numpy as np
import pytest
import torch

import oracle
import synth
import sparse_mixture_experts_30_amd as moe
from synth import device as sd

from gpu_util import DEV, FP8_QUANT_TOL, host, log, rel_l2, sync

pytestmark = pytest.mark.gpu

TOL = 2e-2   # bf16 inputs and outputs, bf16 dy rows, [dg du] and h; fp32 accumulation

CASES = [
    synth.C3.replace(name="lbwd-T300-H1024-E64-K8", T=300, H=1024, E=64, G=8, TG=4, K=8, I=256,
                     Is=256, rho=2.5),
    # top-1 (no normalisation), no shared expert, most experts without rows
    synth.C3.replace(name="lbwd-T40-H512-E128-K1-noshared", T=40, H=512, E=128, G=8, TG=2, K=1,
                     I=128, Is=0, rho=2.5),
    # one group, top-6; I and Is not multiples of the 128-wide tile
    synth.C3.replace(name="lbwd-T150-H512-E32-G1-K6-I192-Is320", T=150, H=512, E=32, G=1, TG=1,
                     K=6, I=192, Is=320, rho=1.7),
]


# e4m3 expert weights (fp32 or power-of-two block scales): the FP8 expert
# backward inside.  Against the oracle's FP8 layer backward (the forward's
# expert outputs of the activation-quantised forward, each expert's FP8
# backward): the GPU's dy rows are rounded to bf16 before they are quantised,
# and y is the GPU forward's; against the exact backward of the dequantised
# weights, the e4m3 rounding of every GEMM's operands.
FP8_CASES = [
    synth.C5.replace(name="lbwd8-T300-H1024-E16-K4", T=300, H=1024, E=16, G=4, TG=2, K=4, I=256,
                     Is=256, rho=2.5),
    synth.C5.replace(name="lbwd8p2-T300-H1024-E16-K4", T=300, H=1024, E=16, G=4, TG=2, K=4,
                     I=256, Is=256, rho=2.5, wdtype="fp8e8m0"),
    synth.C5.replace(name="lbwd8-T60-H256-E64-K1-noshared", T=60, H=256, E=64, G=8, TG=2, K=1,
                     I=128, Is=0, rho=1.0),
]


@pytest.mark.parametrize("cfg", CASES + FP8_CASES, ids=lambda c: c.name)
def test_layer_backward(cfg):
    log(f"layer backward {cfg.name}")
    fp8 = cfg.wdtype in ("fp8", "fp8e8m0")
    inp = synth.gen_inputs(cfg)
    dev = sd.to_device(inp)            # row-major weights (the backward's layout)
    T, H, E, K, I, Is = cfg.T, cfg.H, cfg.E, cfg.K, cfg.I, cfg.Is
    N = T * K
    C = sd.moe_config(cfg)
    W = sd.weights_struct(dev)
    ws = sd.workspace(cfg, T)
    f32, i32 = dict(dtype=torch.float32, device=DEV), dict(dtype=torch.int32, device=DEV)
    bf = dict(dtype=torch.bfloat16, device=DEV)
    lg, idx, w = torch.empty((T, E), **f32), torch.empty((T, K), **i32), torch.empty((T, K), **f32)
    counts, offsets = torch.empty(E, **i32), torch.empty(E + 1, **i32)
    perm, pos = torch.empty(N, **i32), torch.empty(N, **i32)
    y, ys = torch.empty((N, H), **bf), torch.empty((T, H), **bf)
    moe.moe_gate(C, T, dev["x"], dev["gate_w"], dev["bias"], lg, idx, w, ws)
    moe.moe_permute(C, T, idx, counts, offsets, perm, pos, ws)
    # the forward's expert outputs (e4m3: from the packed layout, which takes
    # both scale forms)
    devp = sd.packed_copy(dev) if fp8 else None   # kept alive until the end
    Wf = sd.weights_struct(devp) if fp8 else W
    moe.moe_expert_ffn(C, T, dev["x"], perm, offsets, Wf, y, ys if Is else None, ws)
    rng = np.random.default_rng(31)
    dout_b = torch.from_numpy(rng.standard_normal((T, H), dtype=np.float32)).to(torch.bfloat16)
    dout = dout_b.to(DEV)
    dx = torch.full((T, H), float("nan"), **bf)
    dgw = torch.full((E, H), float("nan"), **f32)
    dw13 = torch.full((E, 2 * I, H), float("nan"), **bf)
    dw2 = torch.full((E, H, I), float("nan"), **bf)
    dws13 = torch.empty((2 * Is, H), **bf) if Is else None
    dws2 = torch.empty((H, Is), **bf) if Is else None
    wsb = torch.empty(moe.moe_backward_workspace_bytes(C, T), dtype=torch.uint8, device=DEV)
    moe.moe_backward(C, T, dev["x"], W, lg, idx, w, perm, offsets, pos, y, dout, dx, dgw, dw13,
                     dw2, dws13, dws2, wsb)
    sync()

    dout64 = dout_b.float().numpy().astype(np.float64)
    ref = oracle.layer_backward(cfg, inp, host(idx), dout64, quant_act=fp8)
    cnt = host(counts)
    g13, g2, ggw = host(dw13), host(dw2), host(dgw)
    errs = {"dx": rel_l2(host(dx), ref["dx"]), "dgate_w": rel_l2(ggw, ref["dgate_w"])}
    for e in range(E):
        if cnt[e] == 0:
            assert np.all(g13[e] == 0) and np.all(g2[e] == 0) and np.all(ggw[e] == 0), e
    busy = cnt > 0
    errs["dw13"] = rel_l2(g13[busy], ref["dw13"][busy])
    errs["dw2"] = rel_l2(g2[busy], ref["dw2"][busy])
    if Is:
        errs["dws13"] = rel_l2(host(dws13), ref["dws13"])
        errs["dws2"] = rel_l2(host(dws2), ref["dws2"])
    log("  " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()) +
        f"; experts with rows {int(busy.sum())}/{E}")
    for k, v in errs.items():
        assert v <= (FP8_QUANT_TOL if fp8 else TOL), (k, v)
    if fp8:
        ex = oracle.layer_backward(cfg, inp, host(idx), dout64)
        got = {"dx": host(dx), "dgate_w": ggw, "dw13": g13[busy], "dw2": g2[busy]}
        exact = {"dx": ex["dx"], "dgate_w": ex["dgate_w"], "dw13": ex["dw13"][busy],
                 "dw2": ex["dw2"][busy]}
        if Is:
            got.update(dws13=host(dws13), dws2=host(dws2))
            exact.update(dws13=ex["dws13"], dws2=ex["dws2"])
        e2 = {k: rel_l2(got[k], exact[k]) for k in got}
        log("  vs the exact backward of the dequantised weights: " +
            ", ".join(f"{k} {v:.2e}" for k, v in e2.items()))
        for k, v in e2.items():
            assert v <= 1e-1, (k, v)
