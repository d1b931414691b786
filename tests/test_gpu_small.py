"""GPU parity of every C-ABI entry point against the fp64 oracle at sizes the
oracle finishes in seconds (several tiles, ragged tails, edge cases)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import sparse_mixture_experts_30_amd as moe
from synth import device as sd

from gpu_util import (DEV, FP8_QUANT_TOL, check_routing, host, layer_reference, log,
                      random_routing, rel_l2, run_forward, run_gate, run_permute, sync,
                      worst_row_rel)

pytestmark = pytest.mark.gpu

C1 = synth.C1
# bf16, several tiles, ragged T, ~37 rows per expert
SMALL_BF16 = synth.C3.replace(name="bf16-T300-H1024-E64", T=300, H=1024, E=64, G=8, TG=4, K=8,
                              I=256, Is=256, rho=2.5)
# I not a multiple of the 128-wide h tile; shared width != routed width
RAGGED_BF16 = synth.C3.replace(name="bf16-T1000-H512-E32-I192-Is320", T=1000, H=512, E=32, G=4,
                               TG=2, K=4, I=192, Is=320, rho=1.7, bias_lo=-0.1, bias_hi=0.1)
# 512 rows per expert: several M-tiles per group
TALL_BF16 = synth.C3.replace(name="bf16-T2048-E8-K2", T=2048, H=256, E=8, G=2, TG=1, K=2, I=128,
                             Is=128, rho=1.0)
# top-1, no shared expert, 7 tokens
K1_NOSHARED = synth.C3.replace(name="bf16-T7-K1-noshared", T=7, H=512, E=16, G=4, TG=2, K=1,
                               I=128, Is=0, rho=2.5)
SMALL_FP8 = synth.C5.replace(name="fp8-T200-H1024-E32", T=200, H=1024, E=32, G=4, TG=2, K=4,
                             I=256, Is=384, rho=2.5)
TINY_T1 = SMALL_BF16.replace(name="bf16-T1", T=1)
# fp8 with 256 rows per expert: two 128-row M-tiles share each weight tile
TALL_FP8 = synth.C5.replace(name="fp8-T1024-H512-E8-K2", T=1024, H=512, E=8, G=2, TG=1, K=2,
                            I=256, Is=256, rho=1.0)
# 32 < T <= 64: decode path with two 32-row blocks per group
DECODE48 = synth.C3.replace(name="bf16-T48-H512-E16", T=48, H=512, E=16, G=4, TG=2, K=4, I=256,
                            Is=128, rho=2.5)

# >= 256 rows per expert (wide 128 x 512 tiles) with ragged widths: 3 h-tiles
# of 128 (the second wide tile half empty), a shared width of 2 tiles, and a
# hidden size of 3 row tiles of 256 for the down projection
WIDE_RAGGED = synth.C3.replace(name="bf16-T1100-H768-E4-K1-I384-Is256", T=1100, H=768, E=4,
                               G=2, TG=1, K=1, I=384, Is=256, rho=1.3)

# e4m3 with power-of-two block scales (the matrix cores apply them; packed
# weights only): ragged groups of 256-row tiles, and groups of two 256-row
# tiles with 3 h-tiles (I = 384), an odd number of 128-k steps (H = 640) and
# a shared width of one tile
SMALL_FP8P2 = SMALL_FP8.replace(name="fp8e8m0-T200-H1024-E32", wdtype="fp8e8m0")
TALL_FP8P2 = synth.C5.replace(name="fp8e8m0-T2100-H640-E8-K2-I384", T=2100, H=640, E=8, G=2,
                              TG=1, K=2, I=384, Is=128, rho=1.0, wdtype="fp8e8m0")

LAYER_CASES = [C1, SMALL_BF16, RAGGED_BF16, TALL_BF16, K1_NOSHARED, TINY_T1, DECODE48, SMALL_FP8,
               TALL_FP8, WIDE_RAGGED, SMALL_FP8P2, TALL_FP8P2]
# layouts each weight dtype takes: row-major (not for power-of-two fp8) and packed
ROWMAJOR_OK = ("f32", "bf16", "fp8")


def _tol(cfg):
    return {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2, "fp8e8m0": 6e-2}[cfg.wdtype]


_inputs = {}


def inputs(cfg):
    if cfg.name not in _inputs:
        inp = synth.gen_inputs(cfg)
        _inputs[cfg.name] = (inp, sd.to_device(inp))
    return _inputs[cfg.name]


# 12 k steps of 64 split 6 ways (a split count that is not a power of two)
GATE_SPLIT6 = synth.C3.replace(name="bf16-T32-H768-E64-split6", T=32, H=768, E=64, G=8, TG=4,
                               K=8, I=128, Is=128, rho=2.5)


# 36 k steps split 18 ways: the split sums are shared by a token's four waves
# (uneven quarters of 4 and 5 splits)
GATE_SPLIT18 = synth.C3.replace(name="bf16-T8-H2304-E64-split18", T=8, H=2304, E=64, G=8, TG=4,
                                K=8, I=128, Is=128, rho=2.5)


@pytest.mark.parametrize("cfg", [C1, SMALL_BF16, RAGGED_BF16, K1_NOSHARED, TINY_T1, GATE_SPLIT6,
                                 GATE_SPLIT18],
                         ids=lambda c: c.name)
def test_gate(cfg):
    log(f"gate {cfg.name}")
    inp, dev = inputs(cfg)
    lg, idx, w = run_gate(cfg, dev, cfg.T)
    check_routing(cfg, inp["x"], inp["gate_w"], inp["bias"], lg, idx, w, cfg.name)


def test_gate_negative_choice_scores_pick_masked_experts():
    """Selection-only bias so negative that kept groups hold fewer than K
    positive choices: masked experts (choice 0.0) must win, as printed."""
    cfg = SMALL_BF16.replace(name="neg-bias", T=64, bias_lo=-1.5, bias_hi=-0.9)
    inp, dev = inputs(cfg)
    lg, idx, w = run_gate(cfg, dev, cfg.T)
    check_routing(cfg, inp["x"], inp["gate_w"], inp["bias"], lg, idx, w, cfg.name)
    # the case is exercised: chosen experts outside the kept groups
    Eg = cfg.E // cfg.G
    c = 1 / (1 + np.exp(-lg.astype(np.float64))) + inp["bias"].astype(np.float64)
    g = np.sort(c.reshape(cfg.T, cfg.G, Eg), axis=2)[:, :, -2:].sum(2)
    kept = np.argsort(-g, axis=1, kind="stable")[:, :cfg.TG]
    outside = [not set((idx[t] // Eg).tolist()) <= set(kept[t].tolist()) for t in range(cfg.T)]
    assert np.mean(outside) > 0.5


@pytest.mark.parametrize("T,K,E,skew", [(1, 1, 16, False), (300, 8, 64, False), (1000, 4, 32, True),
                                        (5000, 8, 256, False), (2100, 1, 8, True),
                                        (513, 8, 512, False)])
def test_permute(T, K, E, skew):
    log(f"permute T={T} K={K} E={E} skew={skew}")
    cfg = SMALL_BF16.replace(T=T, K=K, E=E, G=1 if E < 16 else 8, TG=1)
    idx = random_routing(T, K, E, seed=T + K, skew=skew)
    counts, offsets, perm, pos, status = run_permute(cfg, idx)
    rc, ro, rp, rq = oracle.permute(idx, E)
    assert status == moe.MOE_OK
    np.testing.assert_array_equal(counts, rc)
    np.testing.assert_array_equal(offsets, ro)
    np.testing.assert_array_equal(perm, rp)
    np.testing.assert_array_equal(pos, rq)


def test_permute_flags_out_of_range_index():
    cfg = SMALL_BF16.replace(T=50)
    idx = random_routing(50, cfg.K, cfg.E, seed=3)
    idx[17, 2] = cfg.E
    *_, status = run_permute(cfg, idx)
    assert status == moe.MOE_ERR_DEVICE_CHECK
    idx[17, 2] = 0 if 0 not in idx[17] else 63
    *_, status = run_permute(cfg, idx)
    assert status == moe.MOE_OK


FFN_CASES = [(C1, False), (SMALL_BF16, False), (RAGGED_BF16, False), (TALL_BF16, False),
             (K1_NOSHARED, False), (SMALL_FP8, False), (SMALL_BF16, True), (RAGGED_BF16, True),
             (TALL_BF16, True), (K1_NOSHARED, True), (DECODE48, True), (DECODE48, False),
             (SMALL_FP8, True), (TALL_FP8, True), (TALL_FP8, False), (WIDE_RAGGED, True),
             (SMALL_FP8P2, True), (TALL_FP8P2, True)]


def _case_id(c):
    return c[0].name + ("-packed" if c[1] else "")


@pytest.mark.parametrize("case", FFN_CASES, ids=_case_id)
def test_expert_ffn(case):
    """y (expert-sorted rows) and y_shared against the oracle's per-row FFN,
    on an oracle-made routing and permutation."""
    cfg, packed = case
    log(f"ffn {cfg.name} packed={packed}")
    inp, dev = inputs(cfg)
    if packed:
        dev = sd.packed_copy(dev)
    T, K, H = cfg.T, cfg.K, cfg.H
    lg = oracle.logits(inp["x"], cfg.act, inp["gate_w"])
    idx, _, _ = oracle.route_f64(cfg, lg, inp["bias"])
    counts, offsets, perm, pos = oracle.permute(idx, cfg.E)
    dt = torch.bfloat16 if cfg.act == "bf16" else torch.float32
    y = torch.empty((T * K, H), dtype=dt, device=DEV)
    ys = torch.empty((T, H), dtype=dt, device=DEV) if cfg.Is else None
    ws = sd.workspace(cfg, T)
    moe.moe_expert_ffn(sd.moe_config(cfg), T, dev["x"], torch.from_numpy(perm).to(DEV),
                       torch.from_numpy(offsets).to(DEV), sd.weights_struct(dev), y, ys, ws)
    sync()
    experts = np.repeat(np.arange(cfg.E), counts).astype(np.int32)
    ref = oracle.ffn(cfg, inp, perm // K, experts)
    r = rel_l2(host(y), ref)
    rows = np.linalg.norm(host(y) - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
    log(f"  y relL2={r:.3e} worst row={rows.max():.3e}")
    assert r <= _tol(cfg) and rows.max() <= 3 * _tol(cfg)
    if cfg.Is:
        refs = oracle.ffn(cfg, inp, np.arange(T), -np.ones(T, np.int32))
        rs = rel_l2(host(ys), refs)
        log(f"  y_shared relL2={rs:.3e}")
        assert rs <= _tol(cfg)
    if cfg.wdtype in ("fp8", "fp8e8m0"):
        # Against the oracle that quantises x and h per 1x128 tile as the
        # kernels do: what is left is accumulation order and the bf16 output,
        # so a mis-scaled tile or a wrong block-scale index shows here.
        ref2 = oracle.ffn(cfg, inp, perm // K, experts, quant_act=True)
        r2 = rel_l2(host(y), ref2)
        rows2 = (np.linalg.norm(host(y) - ref2, axis=1) /
                 np.maximum(np.linalg.norm(ref2, axis=1), 1e-30))
        log(f"  y vs activation-quantised oracle relL2={r2:.3e} worst row={rows2.max():.3e}")
        assert r2 <= FP8_QUANT_TOL and rows2.max() <= 3 * FP8_QUANT_TOL
        if cfg.Is:
            refs2 = oracle.ffn(cfg, inp, np.arange(T), -np.ones(T, np.int32), quant_act=True)
            rs2 = rel_l2(host(ys), refs2)
            log(f"  y_shared vs activation-quantised oracle relL2={rs2:.3e}")
            assert rs2 <= FP8_QUANT_TOL


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_combine(act):
    T, K, H = 333, 8, 1024
    cfg = SMALL_BF16.replace(T=T, K=K, H=H, act=act, wdtype=act)
    y32 = synth.normal_f32(T * K * H, 5, synth.T_TEST, 40, 1.0).reshape(T * K, H)
    ys32 = synth.normal_f32(T * H, 5, synth.T_TEST, 41, 1.0).reshape(T, H)
    if act == "bf16":
        y_bits = synth.normal_bf16(T * K * H, 5, synth.T_TEST, 40, 1.0).reshape(T * K, H)
        ys_bits = synth.normal_bf16(T * H, 5, synth.T_TEST, 41, 1.0).reshape(T, H)
        y_h, ys_h = synth.bf16_to_f32(y_bits), synth.bf16_to_f32(ys_bits)
        y_d, ys_d = sd.tensor(y_bits), sd.tensor(ys_bits)
    else:
        y_h, ys_h, y_d, ys_d = y32, ys32, sd.tensor(y32), sd.tensor(ys32)
    w = synth.uniform_f32(T * K, 5, synth.T_TEST, 42, 0.0, 0.5).reshape(T, K)
    idx = random_routing(T, K, cfg.E, seed=9)
    _, _, _, pos = oracle.permute(idx, cfg.E)
    out = torch.empty((T, H), dtype=y_d.dtype, device=DEV)
    for shared in (True, False):
        moe.moe_combine(sd.moe_config(cfg.replace(Is=cfg.Is if shared else 0)), T, y_d,
                        ys_d if shared else None, torch.from_numpy(pos).to(DEV),
                        sd.tensor(w), out)
        sync()
        ref = oracle.combine(y_h, ys_h if shared else None, pos, w, K)
        r = rel_l2(host(out), ref)
        log(f"combine {act} shared={shared} relL2={r:.3e}")
        assert r <= (4e-3 if act == "bf16" else 1e-6)


FORWARD_CASES = [(c, False) for c in LAYER_CASES if c.wdtype in ROWMAJOR_OK] + \
    [(c, True) for c in LAYER_CASES if c.wdtype != "f32"]


@pytest.mark.parametrize("case", FORWARD_CASES, ids=_case_id)
def test_forward(case):
    cfg, packed = case
    log(f"forward {cfg.name} packed={packed}")
    inp, dev = inputs(cfg)
    if packed:
        dev = sd.packed_copy(dev)
    r = run_forward(cfg, dev, cfg.T)
    check_routing(cfg, inp["x"], inp["gate_w"], inp["bias"], r["logits"], r["idx"], r["w"],
                  cfg.name)
    # counts and permutation: the oracle's, from the oracle's re-selection on
    # the GPU logits (bit-exact by the check above)
    idx_c, _ = oracle.route_f32(cfg, r["logits"], inp["bias"])
    rc, _, rp, _ = oracle.permute(idx_c, cfg.E)
    np.testing.assert_array_equal(r["counts"], rc)
    np.testing.assert_array_equal(r["perm"], rp)
    ref, nalt = layer_reference(cfg, inp, r["idx"], np.arange(cfg.T))
    rel = rel_l2(r["out"], ref)
    worst = worst_row_rel(r["out"], ref)
    log(f"  out relL2={rel:.3e} worst token={worst:.3e} (tol {_tol(cfg)}), "
        f"near-tie tokens={nalt}")
    assert rel <= _tol(cfg) and worst <= 3 * _tol(cfg)
    if cfg.wdtype in ("fp8", "fp8e8m0"):
        ref2, _ = layer_reference(cfg, inp, r["idx"], np.arange(cfg.T), quant_act=True)
        r2, w2 = rel_l2(r["out"], ref2), worst_row_rel(r["out"], ref2)
        log(f"  out vs activation-quantised oracle relL2={r2:.3e} worst token={w2:.3e}")
        assert r2 <= FP8_QUANT_TOL and w2 <= 3 * FP8_QUANT_TOL


@pytest.mark.parametrize("cfg", [SMALL_FP8, SMALL_FP8P2], ids=lambda c: c.wdtype)
def test_quantize_act_bit_exact(cfg):
    inp, dev = inputs(cfg)
    T, H = cfg.T, cfg.H
    xq = torch.empty((T, H), dtype=torch.uint8, device=DEV)
    xs = torch.empty((T, H // 128), dtype=torch.float32, device=DEV)
    moe.moe_quantize_act(sd.moe_config(cfg), T, dev["x"], xq, xs)
    sync()
    q_ref, s_ref = oracle.quant_rows(synth.bf16_to_f32(inp["x"]), pow2=cfg.wdtype == "fp8e8m0")
    np.testing.assert_array_equal(host(xs), s_ref)
    np.testing.assert_array_equal(host(xq), q_ref)


def test_quantize_act_pow2_edge_values():
    """Power-of-two scales at their boundaries: rows whose tile maximum is
    448 * 2^k exactly (scale 2^k), one bf16 step above (2^(k+1)), an
    all-zero tile (scale 1, zero codes), and tiny and huge magnitudes."""
    cfg = SMALL_FP8P2.replace(T=6, H=256)
    x = np.zeros((6, 256), np.float32)
    rng = np.random.default_rng(3)
    x[:, :] = rng.standard_normal((6, 256)).astype(np.float32) * 0.5
    x[3, :128] *= 2.0 ** -100
    x[4, 128:] *= 2.0 ** 100
    x = ((x.view(np.uint32) >> 16) << 16).view(np.float32)   # truncated to bf16 values
    x[0, 7] = 448.0 * 2.0 ** -3                 # exactly 448 * 2^-3
    x[1, 9] = 448.0 * 2.0 ** -3 + 0.5           # one bf16 step above it (56 -> 56.5)
    x[2, 128:] = 0.0
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)   # exact: the values are bf16
    assert np.array_equal(synth.bf16_to_f32(xb), x)
    xq = torch.empty((6, 256), dtype=torch.uint8, device=DEV)
    xs = torch.empty((6, 2), dtype=torch.float32, device=DEV)
    moe.moe_quantize_act(sd.moe_config(cfg), 6, sd.tensor(xb), xq, xs)
    sync()
    q_ref, s_ref = oracle.quant_rows(x, pow2=True)
    assert s_ref[0, 0] == 2.0 ** -3 and s_ref[1, 0] == 2.0 ** -2 and s_ref[2, 1] == 1.0
    np.testing.assert_array_equal(host(xs), s_ref)
    np.testing.assert_array_equal(host(xq), q_ref)


# Edge cases of the routing shape, through the whole layer (packed bf16):
#   the largest expert count (512: eight experts per lane in the select),
#   one group (group-limited routing reduces to plain top-k),
#   every group kept (TG = G), the smallest group (2 experts), and top-k
#   equal to every expert of the kept groups.
EDGE_CASES = [
    synth.C3.replace(name="bf16-T96-H256-E512-G16-TG4-K8", T=96, H=256, E=512, G=16, TG=4, K=8,
                     I=128, Is=128, rho=2.5),
    synth.C3.replace(name="bf16-T80-H256-E32-G1-K6", T=80, H=256, E=32, G=1, TG=1, K=6, I=128,
                     Is=128, rho=1.5),
    synth.C3.replace(name="bf16-T80-H256-E32-G4-TG4-K5", T=80, H=256, E=32, G=4, TG=4, K=5,
                     I=128, Is=128, rho=1.5),
    synth.C3.replace(name="bf16-T80-H256-E16-G8-TG3-K2", T=80, H=256, E=16, G=8, TG=3, K=2,
                     I=128, Is=0, rho=1.5),
    synth.C3.replace(name="bf16-T80-H256-E16-G8-TG3-K6-all", T=80, H=256, E=16, G=8, TG=3, K=6,
                     I=128, Is=128, rho=1.5),
    # fewer routed rows than experts (the GEMM grids are sized for at most
    # min(E, T * K) non-empty groups): two-block decode tiles, and 256-row tiles
    synth.C3.replace(name="bf16-T40-H256-E256-K1", T=40, H=256, E=256, G=8, TG=4, K=1, I=128,
                     Is=128, rho=2.5),
    synth.C3.replace(name="bf16-T100-H256-E512-G16-TG4-K2", T=100, H=256, E=512, G=16, TG=4,
                     K=2, I=128, Is=128, rho=2.5),
]


@pytest.mark.parametrize("cfg", EDGE_CASES, ids=lambda c: c.name)
def test_forward_routing_edge_cases(cfg):
    log(f"edge {cfg.name}")
    inp, dev = inputs(cfg)
    dev = sd.packed_copy(dev)
    r = run_forward(cfg, dev, cfg.T)
    check_routing(cfg, inp["x"], inp["gate_w"], inp["bias"], r["logits"], r["idx"], r["w"],
                  cfg.name)
    idx_c, _ = oracle.route_f32(cfg, r["logits"], inp["bias"])
    rc, _, rp, _ = oracle.permute(idx_c, cfg.E)
    np.testing.assert_array_equal(r["counts"], rc)
    np.testing.assert_array_equal(r["perm"], rp)
    if cfg.K == cfg.TG * (cfg.E // cfg.G):
        # every expert of the kept groups is chosen, on tokens where all of
        # them have a positive choice score (a masked expert scores 0.0 and
        # may beat a negative one)
        Eg = cfg.E // cfg.G
        c = 1 / (1 + np.exp(-r["logits"].astype(np.float64))) + inp["bias"].astype(np.float64)
        checked = 0
        for t in range(cfg.T):
            groups = sorted(set((r["idx"][t] // Eg).tolist()))
            kept = [g * Eg + j for g in groups for j in range(Eg)]
            if len(groups) == cfg.TG and np.all(c[t, kept] > 0):
                assert sorted(r["idx"][t].tolist()) == kept
                checked += 1
        assert checked >= 0.9 * cfg.T
    ref, nalt = layer_reference(cfg, inp, r["idx"], np.arange(cfg.T))
    rel = rel_l2(r["out"], ref)
    log(f"  out relL2={rel:.3e}, near-tie tokens={nalt}")
    assert rel <= _tol(cfg)


def test_forward_graph_replay():
    """moe_forward captured into a HIP graph (torch.cuda.CUDAGraph) replays
    bit-identically to eager execution, several times, with eager forwards
    and synchronisations between the replays (the path issues no memset or
    host synchronisation, so it can be captured)."""
    cfg = SMALL_BF16
    inp, dev = inputs(cfg)
    dev = sd.packed_copy(dev)
    T = cfg.T
    C = sd.moe_config(cfg)
    W = sd.weights_struct(dev)
    ws = sd.workspace(cfg, T)
    out = torch.empty((T, cfg.H), dtype=torch.bfloat16, device=DEV)
    idx = torch.empty((T, cfg.K), dtype=torch.int32, device=DEV)
    sync()

    def fwd():
        moe.moe_forward(C, T, dev["x"], W, out, ws, topk_idx=idx,
                        stream=torch.cuda.current_stream())

    fwd()
    sync()
    ref, ref_idx = out.clone(), idx.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd()
    sync()
    for rep in range(4):
        out.fill_(0)
        idx.fill_(-1)
        sync()
        g.replay()
        sync()
        assert torch.equal(out, ref), f"replay {rep}"
        assert torch.equal(idx, ref_idx), f"replay {rep}"
        fwd()          # eager work between replays
        sync()
        assert torch.equal(out, ref)


def test_forward_deterministic():
    cfg = RAGGED_BF16
    inp, dev = inputs(cfg)
    a = run_forward(cfg, dev, cfg.T)
    b = run_forward(cfg, dev, cfg.T)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_forward_zero_tokens_is_noop():
    cfg = SMALL_BF16
    inp, dev = inputs(cfg)
    out = torch.zeros((1, cfg.H), dtype=torch.bfloat16, device=DEV)
    moe.moe_forward(sd.moe_config(cfg), 0, dev["x"], sd.weights_struct(dev), out, None)
    sync()
    assert torch.count_nonzero(out).item() == 0


def test_kernel_timer_names_every_launch():
    cfg = SMALL_BF16
    inp, dev = inputs(cfg)
    dev = sd.packed_copy(dev)
    moe.moe_kernel_timer_read()
    moe.moe_kernel_timer_enable(True)
    for _ in range(3):
        run_forward(cfg, dev, cfg.T)
    moe.moe_kernel_timer_enable(False)
    kt = moe.moe_kernel_timer_read()
    log(f"  {kt}")
    gemm1 = [k for k in kt if k.startswith("grouped_gemm") and "<true" in k]
    gemm2 = [k for k in kt if k.startswith("grouped_gemm") and "<false" in k]
    assert len(gemm1) == 1 and len(gemm2) == 1, list(kt)
    for name in ("gate_logits_bf16_kernel", "select_kernel", "hist_kernel", "scan_kernel",
                 "scatter_kernel", "build_tiles_kernel", gemm1[0], gemm2[0],
                 "combine_bf16_kernel"):
        assert name in kt, name
        ms, n = kt[name]
        # one launch per forward (the tile list may be built once per GEMM)
        assert n % 3 == 0 and 3 <= n <= (6 if name == "build_tiles_kernel" else 3), (name, n)
        assert ms > 0, (name, ms)
    # restricted to one kernel
    moe.moe_kernel_timer_enable(True, "combine_bf16_kernel")
    run_forward(cfg, dev, cfg.T)
    moe.moe_kernel_timer_enable(False)
    kt = moe.moe_kernel_timer_read()
    assert list(kt) == ["combine_bf16_kernel"] and kt["combine_bf16_kernel"][1] == 1


def test_pack_layout():
    """moe_pack_weight against the layout stated in include/moe.h, written
    out here with numpy: per (expert, tile, 64-k step) a block of
    [wave 4][col block 2][k slice 4][lane 64][8 values]."""
    cfg = RAGGED_BF16          # I = 192: a partial GEMM1 tile (zero padding)
    inp, dev = inputs(cfg)
    C = sd.moe_config(cfg)
    E, H, I = cfg.E, cfg.H, cfg.I
    w13 = synth.bf16_to_f32(inp["w13"]).view(np.uint32) >> 16
    w2 = synth.bf16_to_f32(inp["w2"]).view(np.uint32) >> 16
    for key, which, src, gate_up, n, kd in (("w13", moe.MOE_W13, w13, True, I, H),
                                            ("w2", moe.MOE_W2, w2, False, H, I)):
        buf = torch.empty(moe.moe_packed_bytes(C, which), dtype=torch.uint8, device=DEV)
        moe.moe_pack_weight(C, which, dev[key], buf)
        got = host(buf).view(np.uint16).reshape(-1, 8)
        nt = -(-n // (128 if gate_up else 256))
        steps = kd // 64
        c = np.arange(got.shape[0])
        l, kk, cb, w = c & 63, (c >> 6) & 3, (c >> 8) & 1, (c >> 9) & 3
        rest = c >> 11
        ks, tile, e = rest % steps, (rest // steps) % nt, rest // (steps * nt)
        if gate_up:
            col = tile * 128 + 32 * w + (l & 31)
            ok = col < n
            row = np.where(cb == 1, n + col, col)
        else:
            row = tile * 256 + 64 * w + 32 * cb + (l & 31)
            ok = row < n
        k0 = ks * 64 + 32 * (l >> 5) + 8 * kk
        ref = np.zeros_like(got)
        idx = np.nonzero(ok)[0]
        for j in range(8):
            ref[idx, j] = src[e[idx], row[idx], k0[idx] + j]
        np.testing.assert_array_equal(got, ref)


def test_pack_layout_fp8():
    """moe_pack_weight for e4m3 weights against the layout stated in
    include/moe.h, written out with numpy: per (expert, tile, 128-k step) a
    block of [wave 4][col block 2][k half 2][16-byte half 2][lane 64][16 codes]."""
    cfg = SMALL_FP8            # Is = 384: three GEMM1 tiles for the shared expert
    inp, dev = inputs(cfg)
    C = sd.moe_config(cfg)
    E, H, I, Is = cfg.E, cfg.H, cfg.I, cfg.Is
    for key, which, experts, gate_up, n, kd in (("w13", moe.MOE_W13, E, True, I, H),
                                                ("w2", moe.MOE_W2, E, False, H, I),
                                                ("ws13", moe.MOE_WS13, 1, True, Is, H),
                                                ("ws2", moe.MOE_WS2, 1, False, H, Is)):
        src = inp[key].reshape(experts, -1, kd)
        buf = torch.empty(moe.moe_packed_bytes(C, which), dtype=torch.uint8, device=DEV)
        moe.moe_pack_weight(C, which, dev[key], buf)
        got = host(buf).reshape(-1, 16)
        nt = -(-n // (128 if gate_up else 256))
        steps = kd // 128
        assert got.shape[0] == experts * nt * steps * 2048
        c = np.arange(got.shape[0])
        l, hf, kk, cb, w = c & 63, (c >> 6) & 1, (c >> 7) & 1, (c >> 8) & 1, (c >> 9) & 3
        rest = c >> 11
        ks, tile, e = rest % steps, (rest // steps) % nt, rest // (steps * nt)
        if gate_up:
            col = tile * 128 + 32 * w + (l & 31)
            ok = col < n
            row = np.where(cb == 1, n + col, col)
        else:
            row = tile * 256 + 64 * w + 32 * cb + (l & 31)
            ok = row < n
        k0 = ks * 128 + 64 * kk + 32 * (l >> 5) + 16 * hf
        ref = np.zeros_like(got)
        idx = np.nonzero(ok)[0]
        for j in range(16):
            ref[idx, j] = src[e[idx], row[idx], k0[idx] + j]
        np.testing.assert_array_equal(got, ref, err_msg=key)


# A token row of NaN (a NaN in x): every choice score of that token is NaN.
# Selection treats a NaN choice as -inf, so the token still gets K distinct
# valid expert ids; with every group kept (TG = G) no masked 0.0 scores exist
# to fall back on.  Decode (T <= 32) and batch schedules.
NAN_CASES = [synth.C3.replace(name="bf16-T20-H256-E16-G4-TG4-K4-nan", T=20, H=256, E=16, G=4,
                              TG=4, K=4, I=128, Is=128, rho=2.5),
             synth.C3.replace(name="bf16-T100-H256-E32-G4-TG4-K8-nan", T=100, H=256, E=32, G=4,
                              TG=4, K=8, I=128, Is=128, rho=2.5),
             synth.C3.replace(name="bf16-T100-H256-E32-G4-TG2-K8-nan", T=100, H=256, E=32, G=4,
                              TG=2, K=8, I=128, Is=128, rho=2.5)]


@pytest.mark.parametrize("cfg", NAN_CASES, ids=lambda c: c.name)
def test_forward_nan_token_routes_to_valid_experts(cfg):
    log(f"nan token {cfg.name}")
    inp, _ = inputs(cfg)
    inp = dict(inp)
    bad = cfg.T // 3
    x = inp["x"].copy()
    x[bad, 5] = 0x7FC0                      # bf16 quiet NaN
    inp["x"] = x
    dev = sd.packed_copy(sd.to_device(inp))
    ws = sd.workspace(cfg, cfg.T)
    r = run_forward(cfg, dev, cfg.T, ws=ws)
    assert moe.moe_get_device_error(ws) == moe.MOE_OK
    idx = r["idx"]
    assert idx.min() >= 0 and idx.max() < cfg.E
    assert all(len(set(row.tolist())) == cfg.K for row in idx)
    assert np.all(np.isnan(r["logits"][bad]))
    good = np.array([t for t in range(cfg.T) if t != bad])
    # the other tokens route as the oracle's contract re-selection says
    idx_c, _ = oracle.route_f32(cfg, r["logits"][good], inp["bias"])
    np.testing.assert_array_equal(idx[good], idx_c)
    assert np.all(np.isfinite(r["out"][good]))
    rc, _, rp, _ = oracle.permute(idx, cfg.E)
    np.testing.assert_array_equal(r["counts"], rc)
    np.testing.assert_array_equal(r["perm"], rp)
    ref, _ = layer_reference(cfg, inp, idx[good], good)
    rel = rel_l2(r["out"][good], ref)
    log(f"  nan token {bad}: ids {idx[bad].tolist()}; other tokens relL2={rel:.3e}")
    assert rel <= 2e-2


def test_combine_skips_positions_out_of_range():
    """A caller-made pos outside [0, T*K) adds nothing to its token."""
    T, K, H = 40, 4, 512
    cfg = SMALL_BF16.replace(T=T, K=K, H=H)
    y_bits = synth.normal_bf16(T * K * H, 6, synth.T_TEST, 43, 1.0).reshape(T * K, H)
    w = synth.uniform_f32(T * K, 6, synth.T_TEST, 44, 0.1, 0.5).reshape(T, K)
    idx = random_routing(T, K, cfg.E, seed=11)
    _, _, _, pos = oracle.permute(idx, cfg.E)
    pos = pos.copy()
    pos[3 * K + 1] = T * K            # one past the end
    pos[7 * K + 2] = -5
    pos[9 * K + 0] = 2 ** 31 - 1
    keep = np.ones(T * K, bool)
    keep[[3 * K + 1, 7 * K + 2, 9 * K]] = False
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    moe.moe_combine(sd.moe_config(cfg.replace(Is=0)), T, sd.tensor(y_bits), None,
                    torch.from_numpy(pos).to(DEV), sd.tensor(w), out)
    sync()
    y = synth.bf16_to_f32(y_bits).astype(np.float64)
    ref = np.zeros((T, H))
    for f in np.flatnonzero(keep):
        ref[f // K] += w.ravel()[f] * y[pos[f]]
    r = rel_l2(host(out), ref)
    log(f"combine with out-of-range positions relL2={r:.3e}")
    assert r <= 4e-3


@pytest.mark.parametrize("T", [20, 50])
def test_expert_ffn_repeated_expert_ids(T):
    """moe_permute and moe_expert_ffn take any ids in [0, E), also a token
    that names one expert in several slots: a group then holds more rows
    than there are tokens (here every token sends all K slots to expert 3,
    K * T rows), past the few-row kernels' tile height."""
    cfg = DECODE48.replace(name=f"bf16-T{T}-repeated", T=T)
    inp, dev = inputs(cfg)
    dev = sd.packed_copy(dev)
    K, H = cfg.K, cfg.H
    idx = random_routing(T, K, cfg.E, seed=13)
    idx[:, :] = 3
    idx[1, 2] = 0
    counts, offsets, perm, pos, status = run_permute(cfg, idx)
    assert status == moe.MOE_OK and counts[3] == T * K - 1
    rc, ro, rp, _ = oracle.permute(idx, cfg.E)
    np.testing.assert_array_equal(perm, rp)
    y = torch.empty((T * K, H), dtype=torch.bfloat16, device=DEV)
    ys = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    ws = sd.workspace(cfg, T)
    moe.moe_expert_ffn(sd.moe_config(cfg), T, dev["x"], torch.from_numpy(perm).to(DEV),
                       torch.from_numpy(offsets).to(DEV), sd.weights_struct(dev), y, ys, ws)
    sync()
    experts = np.repeat(np.arange(cfg.E), counts).astype(np.int32)
    ref = oracle.ffn(cfg, inp, perm // K, experts)
    worst = worst_row_rel(host(y), ref)
    log(f"  repeated ids T={T}: y relL2={rel_l2(host(y), ref):.3e} worst row={worst:.3e}")
    assert worst <= 3 * 2e-2
