"""Pins of the fp64 oracle to things other than itself: hand-worked cases,
brute-force enumeration, closed forms, special cases that reduce to library
routines, and invariants of the method.  CPU only."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


class Shape:
    def __init__(self, **kw):
        self.__dict__.update(kw)


def _logit(tok):
    return {"0": 0.0, "ln3": math.log(3.0), "-ln3": -math.log(3.0)}[tok]


# ---------------------------------------------------------------- hand cases

def _hand_cases():
    with open(os.path.join(GOLD, "routing_hand_cases.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _hand_cases(), ids=lambda c: c["name"])
def test_routing_hand_cases(case):
    cfg = Shape(H=1, E=case["E"], G=case["G"], TG=case["TG"], K=case["K"], I=0, Is=0,
                rho=case["rho"])
    lg = np.array([[_logit(t) for t in case["logits"]]], np.float64)
    bias = np.array(case["bias"], np.float32)
    idx, w, _ = oracle.route_f64(cfg, lg, bias)
    assert idx[0].tolist() == case["idx"]
    np.testing.assert_allclose(w[0], case["w"], rtol=1e-12, atol=0)
    # The fp32 contract router takes the same decisions on these exact inputs.
    idx32, w32 = oracle.route_f32(cfg, lg.astype(np.float32), bias)
    assert idx32[0].tolist() == case["idx"]
    np.testing.assert_allclose(w32[0], case["w"], rtol=1e-6, atol=0)


def test_ffn_closed_form_h1():
    with open(os.path.join(GOLD, "ffn_closed_form.json")) as f:
        c = json.load(f)
    cfg = synth.MoEConfig("h1", T=1, H=1, E=2, G=1, TG=1, K=1, I=1, Is=1, rho=c["rho"],
                          act="f32", wdtype="f32", bias_lo=0, bias_hi=0)
    inp = {"x": np.array([c["x"]], np.float32),
           "gate_w": np.array(c["gate_w"], np.float32),
           "bias": np.array(c["bias"], np.float32),
           "w13": np.array(c["w13"], np.float32), "w13_s": None,
           "w2": np.array(c["w2"], np.float32), "w2_s": None,
           "ws13": np.array(c["ws13"], np.float32), "ws13_s": None,
           "ws2": np.array(c["ws2"], np.float32), "ws2_s": None}
    r = oracle.forward(cfg, inp)
    assert r["idx"].tolist() == [[1]]
    np.testing.assert_allclose(r["w"], [[1.0]], rtol=1e-15)
    np.testing.assert_allclose(r["out"][0], c["out"], rtol=1e-14)


# ---------------------------------------------------------------- logits

@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_logits_match_numpy_matmul(kind):
    T, H, E = 37, 256, 24
    if kind == "f32":
        x = synth.normal_f32(T * H, 3, synth.T_TEST, 0, 1.0).reshape(T, H)
        xf = x.astype(np.float64)
    else:
        x = synth.normal_bf16(T * H, 3, synth.T_TEST, 0, 1.0).reshape(T, H)
        xf = synth.bf16_to_f32(x).astype(np.float64)
    wg = synth.normal_f32(E * H, 3, synth.T_TEST, 1, 1 / 16).reshape(E, H)
    lg = oracle.logits(x, kind, wg)
    ref = xf @ wg.astype(np.float64).T
    np.testing.assert_allclose(lg, ref, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- routing: brute force

def _brute_route(cfg, lg, bias, f32):
    """Exhaustive reference: best group set = the TG-subset with the largest
    sum of group scores, group score = best pair sum inside the group; best
    expert set = the K-subset with the largest sum of masked scores."""
    E, G, TG, K = cfg.E, cfg.G, cfg.TG, cfg.K
    Eg = E // G
    s64 = 1.0 / (1.0 + np.exp(-lg.astype(np.float64)))
    if f32:
        s = s64.astype(np.float32)
        c = (s + bias.astype(np.float32)).astype(np.float32)
    else:
        s, c = s64, s64 + bias.astype(np.float64)
    out = []
    for t in range(lg.shape[0]):
        g = []
        for j in range(G):
            best = None
            for a, b in itertools.combinations(range(j * Eg, (j + 1) * Eg), 2):
                v = c[t, a] + c[t, b]
                best = v if best is None or v > best else best
            g.append(float(best))
        gset = max(itertools.combinations(range(G), TG), key=lambda S: sum(g[j] for j in S))
        cm = np.array([float(c[t, e]) if (e // Eg) in gset else 0.0 for e in range(E)])
        eset = max(itertools.combinations(range(E), K), key=lambda S: sum(cm[e] for e in S))
        out.append((set(eset), cm))
    return out, s64


@pytest.mark.parametrize("G,TG,K", [(4, 2, 2), (2, 1, 1), (2, 1, 3), (4, 1, 2), (4, 3, 3),
                                    (4, 4, 2), (1, 1, 2), (8, 3, 2)])
@pytest.mark.parametrize("f32", [False, True])
def test_route_bruteforce_tiny(G, TG, K, f32):
    E, T = 16, 24
    cfg = Shape(H=1, E=E, G=G, TG=TG, K=K, I=0, Is=0, rho=1.0)
    lg = synth.normal_f32(T * E, 11 + G + 7 * K, synth.T_TEST, TG, 1.0).reshape(T, E).astype(np.float64)
    bias = synth.uniform_f32(E, 5 + G, synth.T_TEST, 100 + K, -0.1, 0.1)
    if f32:
        idx, w = oracle.route_f32(cfg, lg.astype(np.float32), bias)
        ref, s64 = _brute_route(cfg, lg.astype(np.float32), bias, True)
        s64 = 1.0 / (1.0 + np.exp(-lg.astype(np.float32).astype(np.float64)))
    else:
        idx, w, margin = oracle.route_f64(cfg, lg, bias)
        ref, s64 = _brute_route(cfg, lg, bias, False)
    for t in range(T):
        eset, cm = ref[t]
        assert set(idx[t].tolist()) == eset, (t, idx[t], eset)
        # slot order: descending masked score, then lower index
        vals = [(-cm[e], e) for e in idx[t]]
        assert vals == sorted(vals)
        sw = s64[t, idx[t]]
        expect = sw / (sw.sum() + 1e-20) if K > 1 else sw
        np.testing.assert_allclose(w[t], expect * cfg.rho, rtol=1e-12)


def test_route_special_case_single_group_is_plain_topk():
    """G = 1 (or TG = G): the group limit is inert, idx = top-K of s + b;
    with b = 0 as well, top-K of the logits (sigmoid is increasing)."""
    T, E, K = 200, 64, 6
    lg = synth.normal_f32(T * E, 1, synth.T_TEST, 2, 1.0).reshape(T, E).astype(np.float64)
    bias = synth.uniform_f32(E, 1, synth.T_TEST, 3, -0.05, 0.05)
    s = 1 / (1 + np.exp(-lg))
    for G, TG in [(1, 1), (8, 8)]:
        cfg = Shape(H=1, E=E, G=G, TG=TG, K=K, I=0, Is=0, rho=2.5)
        idx, _, _ = oracle.route_f64(cfg, lg, bias)
        ref = np.argsort(-(s + bias.astype(np.float64)), axis=1, kind="stable")[:, :K]
        np.testing.assert_array_equal(idx, ref)
        idx0, w0, _ = oracle.route_f64(cfg, lg, np.zeros(E, np.float32))
        np.testing.assert_array_equal(idx0, np.argsort(-lg, axis=1, kind="stable")[:, :K])


def test_route_k1_weight_is_scaled_sigmoid():
    T, E = 64, 32
    cfg = Shape(H=1, E=E, G=4, TG=2, K=1, I=0, Is=0, rho=2.5)
    lg = synth.normal_f32(T * E, 2, synth.T_TEST, 4, 1.5).reshape(T, E).astype(np.float64)
    bias = synth.uniform_f32(E, 2, synth.T_TEST, 5, -0.05, 0.05)
    idx, w, _ = oracle.route_f64(cfg, lg, bias)
    sel = np.take_along_axis(lg, idx.astype(np.int64), axis=1)
    np.testing.assert_allclose(w, 2.5 / (1 + np.exp(-sel)), rtol=1e-15)


# ---------------------------------------------------------------- routing: invariants at the V3 shape

@pytest.fixture(scope="module")
def v3_route():
    cfg = synth.C2
    T = 384
    x = synth.gen_x(cfg, T)
    wg, b = synth.gen_gate(cfg)
    lg = oracle.logits(x, "bf16", wg)
    idx, w, m = oracle.route_f64(cfg, lg, b)
    return cfg, lg, b, idx, w, m


def test_invariants_v3(v3_route):
    cfg, lg, b, idx, w, m = v3_route
    Eg = cfg.E // cfg.G
    s = 1 / (1 + np.exp(-lg))
    c = s + b.astype(np.float64)
    for t in range(lg.shape[0]):
        assert len(set(idx[t].tolist())) == cfg.K               # no duplicates
        groups = set((idx[t] // Eg).tolist())
        assert len(groups) <= cfg.TG                            # at most TG groups
        g = np.sort(c[t].reshape(cfg.G, Eg), axis=1)[:, -2:].sum(1)
        kept = set(np.argsort(-g, kind="stable")[:cfg.TG].tolist())
        assert groups <= kept                                   # inside the kept groups
    np.testing.assert_allclose(w.sum(1), cfg.rho, rtol=1e-12)   # sum w = rho (K > 1)
    sel = np.take_along_axis(s, idx.astype(np.int64), 1)
    np.testing.assert_allclose(w / w[:, :1], sel / sel[:, :1], rtol=1e-12)  # w_i/w_j = s_i/s_j
    assert np.all(m > 0)


def test_bias_changes_selection_only(v3_route):
    cfg, lg, b, idx, w, _ = v3_route
    # A constant shift of the bias keeps every choice (all kept scores stay
    # positive here), so the weights must be bit-identical.
    idx2, w2, _ = oracle.route_f64(cfg, lg, (b + np.float32(0.25)).astype(np.float32))
    np.testing.assert_array_equal(idx2, idx)
    assert np.array_equal(w2, w)
    # A bias that changes the choice gives weights from the unbiased scores.
    b3 = b.copy()
    b3[idx[0, 0]] -= 3.0
    idx3, w3, _ = oracle.route_f64(cfg, lg, b3)
    assert idx[0, 0] not in idx3[0]
    s = 1 / (1 + np.exp(-lg[0, idx3[0]]))
    np.testing.assert_allclose(w3[0], cfg.rho * s / (s.sum() + 1e-20), rtol=1e-12)


def test_contract_router_agrees_with_f64_router_away_from_ties(v3_route):
    cfg, lg, b, idx, w, m = v3_route
    idx32, w32 = oracle.route_f32(cfg, lg.astype(np.float32), b)
    differ = np.any(idx32 != idx, axis=1)
    # fp32 rounding of logits/scores moves choice scores by ~1e-7; a
    # different decision is only possible inside that margin.
    assert np.all(m[differ] < 1e-5)
    assert differ.mean() < 0.01
    np.testing.assert_allclose(w32[~differ], w[~differ], rtol=2e-6)


# ---------------------------------------------------------------- permutation

@pytest.mark.parametrize("T,K,E", [(1, 1, 4), (7, 2, 16), (513, 8, 256), (300, 1, 64)])
def test_permute_is_stable_argsort(T, K, E):
    r = synth.words(T * K, 9, synth.T_TEST, T)
    # skewed ids: half the picks on expert 3 (distinct experts per token are
    # not needed for the permutation itself)
    idx = np.where(r % 2 == 0, 3 % E, (r >> 8) % E).astype(np.int32).reshape(T, K)
    counts, offsets, perm, pos = oracle.permute(idx, E)
    np.testing.assert_array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    assert offsets[0] == 0 and offsets[-1] == T * K
    np.testing.assert_array_equal(np.diff(offsets), counts)
    np.testing.assert_array_equal(perm, np.argsort(idx.ravel(), kind="stable"))
    np.testing.assert_array_equal(pos[perm], np.arange(T * K))
    np.testing.assert_array_equal(np.sort(perm), np.arange(T * K))


def test_permute_rejects_bad_index():
    with pytest.raises(ValueError):
        oracle.permute(np.array([[0, 5]], np.int32), 4)


# ---------------------------------------------------------------- FFN + combine

def _np_ffn(x, w13, w2):
    """Dense numpy SwiGLU: x [n,H], w13 [2I,H], w2 [H,I]."""
    a = x @ w13.T
    I = w2.shape[1]
    g, u = a[:, :I], a[:, I:]
    return (g / (1 + np.exp(-g)) * u) @ w2.T


def _as64(a, kind):
    if a is None:
        return None
    return synth.bf16_to_f32(a).astype(np.float64) if kind == "bf16" else a.astype(np.float64)


@pytest.mark.parametrize("wdtype", ["f32", "bf16"])
def test_dense_masked_equivalence(wdtype):
    """out = shared(x) + sum over ALL experts of m[t,e] FFN_e(x), m = w at the
    chosen experts and 0 elsewhere (numpy, no permutation) must equal the
    oracle's routed sum."""
    cfg = synth.C1.replace(T=40, H=128, E=8, G=4, TG=2, K=3, I=64, Is=96, rho=1.7,
                           act="f32" if wdtype == "f32" else "bf16", wdtype=wdtype)
    inp = synth.gen_inputs(cfg)
    r = oracle.forward(cfg, inp)
    x = _as64(inp["x"], cfg.act)
    mask = np.zeros((cfg.T, cfg.E))
    np.put_along_axis(mask, r["idx"].astype(np.int64), r["w"], axis=1)
    ref = _np_ffn(x, _as64(inp["ws13"], wdtype), _as64(inp["ws2"], wdtype))
    for e in range(cfg.E):
        ref += mask[:, e:e + 1] * _np_ffn(x, _as64(inp["w13"][e], wdtype), _as64(inp["w2"][e], wdtype))
    np.testing.assert_allclose(r["out"], ref, rtol=1e-11, atol=1e-12)


def test_single_expert_reduces_to_dense_swiglu():
    """Two identical experts, one group, top-1: out = rho sigmoid(l*) FFN(x) + shared(x)."""
    cfg = synth.C1.replace(T=16, E=2, G=1, TG=1, K=1, rho=2.5)
    inp = synth.gen_inputs(cfg)
    inp["w13"][1] = inp["w13"][0]
    inp["w2"][1] = inp["w2"][0]
    r = oracle.forward(cfg, inp)
    x = inp["x"].astype(np.float64)
    sel = np.take_along_axis(r["logits"], r["idx"].astype(np.int64), 1)
    ref = (2.5 / (1 + np.exp(-sel))) * _np_ffn(x, inp["w13"][0].astype(np.float64),
                                              inp["w2"][0].astype(np.float64))
    ref += _np_ffn(x, inp["ws13"].astype(np.float64), inp["ws2"].astype(np.float64))
    np.testing.assert_allclose(r["out"], ref, rtol=1e-11, atol=1e-12)


def test_zero_expert_weights_leave_shared_only():
    cfg = synth.C1
    inp = synth.gen_inputs(cfg)
    inp["w13"][:] = 0
    r = oracle.forward(cfg, inp)
    ref = _np_ffn(inp["x"].astype(np.float64), inp["ws13"].astype(np.float64),
                  inp["ws2"].astype(np.float64))
    np.testing.assert_allclose(r["out"], ref, rtol=1e-12, atol=1e-13)


def test_no_shared_expert():
    cfg = synth.C1.replace(Is=0)
    inp = synth.gen_inputs(cfg)
    r = oracle.forward(cfg, inp)
    x = inp["x"].astype(np.float64)
    ref = np.zeros((cfg.T, cfg.H))
    for t in range(cfg.T):
        for k in range(cfg.K):
            e = r["idx"][t, k]
            ref[t] += r["w"][t, k] * _np_ffn(x[t:t + 1], inp["w13"][e].astype(np.float64),
                                             inp["w2"][e].astype(np.float64))[0]
    np.testing.assert_allclose(r["out"], ref, rtol=1e-11, atol=1e-12)


def test_token_subset_equals_full_rows():
    cfg = synth.C1
    inp = synth.gen_inputs(cfg)
    r = oracle.forward(cfg, inp)
    toks = np.array([5, 0, 63, 17])
    out = oracle.layer(cfg, inp, r["idx"], r["w"], tokens=toks)
    assert np.array_equal(out, r["out"][toks])


# ---------------------------------------------------------------- e4m3 and the 1x128 quantiser

def test_e4m3_decode_matches_torch_for_all_codes():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = np.array([oracle.e4m3_decode(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan) and nan.sum() == 2   # 0x7F, 0xFF
    np.testing.assert_array_equal(mine[~nan], ref[~nan])
    assert mine[0x7E] == 448.0 and mine[0x01] == 2.0 ** -9 and mine[0x08] == 2.0 ** -6


def test_e4m3_encode_roundtrip_and_torch_rounding():
    for c in range(256):
        v = oracle.e4m3_decode(c)
        if not np.isnan(v):
            got = oracle.e4m3_encode(np.float32(v))
            assert oracle.e4m3_decode(got) == v
    # Midpoints between neighbouring codes (ties) and random values: the
    # round-to-nearest-even encoder agrees with torch's float8 cast.
    vals = [oracle.e4m3_decode(c) for c in range(0x7E)]
    mids = [(a + b) / 2 for a, b in zip(vals[:-1], vals[1:])]
    rnd = synth.normal_f32(20000, 4, synth.T_TEST, 9, 60.0)
    tiny = synth.normal_f32(2000, 4, synth.T_TEST, 10, 0.01)
    allv = np.concatenate([np.array(mids), -np.array(mids), rnd, tiny]).astype(np.float32)
    allv = np.clip(allv, -448, 448)
    ref = torch.from_numpy(allv).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mine = np.array([oracle.e4m3_encode(v) for v in allv], np.uint8)
    np.testing.assert_array_equal(mine, ref)
    assert oracle.e4m3_encode(np.float32(1e6)) == 0x7E            # saturation
    assert oracle.e4m3_encode(np.float32(-1e6)) == 0xFE


def test_quant_rows_definition():
    x = synth.normal_f32(5 * 384, 6, synth.T_TEST, 11, 3.0).reshape(5, 384)
    x[2, 128:256] = 0.0                                             # an all-zero tile
    q, s = oracle.quant_rows(x)
    assert s[2, 1] == 1.0 and np.all(q[2, 128:256] == 0)
    for r in range(5):
        for t in range(3):
            tile = x[r, t * 128:(t + 1) * 128]
            a = float(np.abs(tile).max())
            if a == 0:
                continue
            assert s[r, t] == np.float32(a / 448.0)
            inv = np.float32(448.0 / a)
            prod = np.clip((tile * inv).astype(np.float32), -448, 448)
            ref = torch.from_numpy(prod).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            np.testing.assert_array_equal(q[r, t * 128:(t + 1) * 128], ref)
            assert np.abs(prod).max() >= 447.0                       # the max maps to ~448
    # dequantised error within half an e4m3 step (relative 2^-4) of each value
    deq = np.vectorize(oracle.e4m3_decode)(q) * np.repeat(s, 128, axis=1)
    err = np.abs(deq - x)
    assert np.all(err <= np.abs(x) * 2 ** -4 + np.repeat(s, 128, axis=1) * 2 ** -9 + 1e-30)


def test_generator_e4m3_weights_decode_close_to_draws():
    """The generator's block-scaled weights dequantise to the normal draws
    they were made from within an e4m3 rounding step."""
    q, s = synth.normal_e4m3_blocks(256, 384, 0, synth.T_TEST, 12, 0.05)
    v = synth.normal_f32(256 * 384, 0, synth.T_TEST, 12, 0.05).reshape(256, 384)
    deq = np.vectorize(oracle.e4m3_decode)(q) * np.kron(s, np.ones((128, 128), np.float32))
    np.testing.assert_allclose(deq, v, rtol=2 ** -4, atol=float(s.max()) * 2 ** -9)
    # and the oracle's encoder gives the same codes on the same scaled values
    for bi in range(2):
        for bj in range(3):
            blk = v[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]
            inv = np.float32(448.0 / float(np.abs(blk).max()))
            mine = np.array([oracle.e4m3_encode(t) for t in (blk * inv).astype(np.float32).ravel()])
            np.testing.assert_array_equal(mine.reshape(128, 128),
                                          q[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128])


def test_fp8_layer_uses_dequantised_weights():
    """F1 mode: the layer on e4m3 weights equals the layer on their
    dequantised fp32 values."""
    cfg8 = synth.C1.replace(T=12, H=256, E=4, G=2, TG=1, K=2, I=128, Is=128, act="bf16",
                            wdtype="fp8")
    inp = synth.gen_inputs(cfg8)
    r8 = oracle.forward(cfg8, inp)
    deq = lambda q, s: (np.vectorize(oracle.e4m3_decode)(q) *
                        np.kron(s, np.ones((128, 128)))).astype(np.float32)
    inp32 = dict(inp)
    inp32["w13"] = np.stack([deq(inp["w13"][e], inp["w13_s"][e]) for e in range(cfg8.E)])
    inp32["w2"] = np.stack([deq(inp["w2"][e], inp["w2_s"][e]) for e in range(cfg8.E)])
    inp32["ws13"] = deq(inp["ws13"], inp["ws13_s"])
    inp32["ws2"] = deq(inp["ws2"], inp["ws2_s"])
    for k in ("w13_s", "w2_s", "ws13_s", "ws2_s"):
        inp32[k] = None
    cfg32 = cfg8.replace(wdtype="f32")
    r32 = oracle.forward(cfg32, inp32)
    np.testing.assert_array_equal(r8["idx"], r32["idx"])
    # e4m3 code x fp32 scale needs up to 28 significant bits, so the fp32
    # copy above is rounded (relative 2^-24 per weight); a wrong block-scale
    # index would be off by far more.
    np.testing.assert_allclose(r8["out"], r32["out"], rtol=1e-5, atol=1e-6)
    # F2 (activations quantised too) stays close to F1
    r2 = oracle.forward(cfg8, inp, quant_act=True)
    rel = np.linalg.norm(r2["out"] - r8["out"]) / np.linalg.norm(r8["out"])
    assert 1e-4 < rel < 0.1


def _pow2_ceil(r):
    """Smallest power of two >= r > 0, with numpy's frexp (r = m 2^e, m in
    [0.5, 1): r itself when m == 0.5, else 2^e)."""
    m, e = np.frexp(r)
    return np.ldexp(1.0, np.where(m == 0.5, e - 1, e))


def _qdq_1x128_torch(v, pow2=False):
    """1x128 quantise-dequantise of the rows of v, written independently of
    the oracle with torch's float8_e4m3fn cast ("深入理解 DeepSeek-V3…", section
    3.2: one scale per 1x128 activation tile): a = max |v| of the fp32 tile,
    scale = a/448 and inverse = 448/a each rounded once to fp32 (scale 1 for
    an all-zero tile), code = e4m3 of the fp32 product (clamped to +-448
    first, since torch maps magnitudes past 464 to NaN), value = code *
    scale.  pow2: the scale is the smallest power of two >= a/448 and the
    inverse its reciprocal (both exact)."""
    v = np.asarray(v, np.float64).astype(np.float32)
    n = v.shape[-1]
    t = v.reshape(-1, n // 128, 128)
    a = np.abs(t).max(axis=-1, keepdims=True).astype(np.float64)
    nz = a > 0
    if pow2:
        p2 = _pow2_ceil(np.where(nz, a, 448.0) / 448.0)
        scale = np.where(nz, p2, 1.0).astype(np.float32)
        inv = np.where(nz, 1.0 / p2, 0.0).astype(np.float32)
    else:
        scale = np.where(nz, (a / 448.0).astype(np.float32), np.float32(1.0))
        inv = np.where(nz, (448.0 / np.where(nz, a, 1.0)).astype(np.float32), np.float32(0.0))
    prod = (t * inv.astype(np.float32)).astype(np.float32)
    codes = torch.from_numpy(np.clip(prod, -448.0, 448.0)).to(torch.float8_e4m3fn)
    return (codes.to(torch.float64).numpy() * scale.astype(np.float64)).reshape(v.shape)


def _fp8_layer_numpy(cfg, inp, idx, w, quant_x, quant_h):
    """The layer on dequantised e4m3 weights with numpy fp64 matmuls, each
    GEMM input optionally passed through the 1x128 quantiser first (with
    power-of-two scales for the fp8e8m0 weights' data path)."""
    pow2 = cfg.wdtype == "fp8e8m0"
    deq = lambda q, s: (torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy()
                        * np.kron(s.astype(np.float64), np.ones((128, 128))))
    x = synth.bf16_to_f32(inp["x"]).astype(np.float64)
    xq = _qdq_1x128_torch(x, pow2) if quant_x else x

    def ffn(w13, w2, xr):
        a = w13 @ xr
        n = w13.shape[0] // 2
        h = a[:n] / (1.0 + np.exp(-a[:n])) * a[n:]
        if quant_h:
            h = _qdq_1x128_torch(h[None, :], pow2)[0]
        return w2 @ h

    ws13, ws2 = deq(inp["ws13"], inp["ws13_s"]), deq(inp["ws2"], inp["ws2_s"])
    w13 = [deq(inp["w13"][e], inp["w13_s"][e]) for e in range(cfg.E)]
    w2 = [deq(inp["w2"][e], inp["w2_s"][e]) for e in range(cfg.E)]
    out = np.empty((x.shape[0], cfg.H))
    for t in range(x.shape[0]):
        out[t] = ffn(ws13, ws2, xq[t])
        for k in range(cfg.K):
            out[t] += w[t, k] * ffn(w13[idx[t, k]], w2[idx[t, k]], xq[t])
    return out


@pytest.mark.parametrize("wdtype", ["fp8", "fp8e8m0"])
def test_fp8_activation_quantised_mode_matches_numpy_expression(wdtype):
    """F2 (the oracle with the activations quantised as the fp8 data path
    does): x quantised per 1x128 tile before W13, h = silu(g) * u quantised
    per 1x128 tile after the SwiGLU and before W2 ("深入理解 DeepSeek-V3…",
    section 3.2: every GEMM's activation input in 1x128 tiles).  Pinned to a
    numpy/torch re-expression at 1e-10; the readings that differ from it --
    h left unquantised, x left unquantised, neither (F1), or the quantiser
    applied to the W2 output instead of its input -- each sit orders of
    magnitude further away, so an oracle making any of those slips fails."""
    cfg = synth.C5.replace(name="f2-pin", T=10, H=256, E=4, G=2, TG=1, K=2, I=256, Is=128,
                           rho=2.5, wdtype=wdtype)
    pow2 = wdtype == "fp8e8m0"
    inp = synth.gen_inputs(cfg)
    lg = oracle.logits(inp["x"], cfg.act, inp["gate_w"])
    idx, w, _ = oracle.route_f64(cfg, lg, inp["bias"])
    got = oracle.layer(cfg, inp, idx, w, quant_act=True)
    ref = _fp8_layer_numpy(cfg, inp, idx, w, quant_x=True, quant_h=True)
    rel = lambda a, b: np.linalg.norm(a - b) / np.linalg.norm(b)
    assert rel(got, ref) < 1e-10
    # F1 (no activation quantisation) is the same numpy expression unquantised
    f1 = oracle.layer(cfg, inp, idx, w, quant_act=False)
    assert rel(f1, _fp8_layer_numpy(cfg, inp, idx, w, quant_x=False, quant_h=False)) < 1e-10
    # each wrong reading is far from F2
    for qx, qh in ((True, False), (False, True), (False, False)):
        assert rel(_fp8_layer_numpy(cfg, inp, idx, w, quant_x=qx, quant_h=qh), ref) > 1e-4

    def ffn_quant_after_w2(w13, w2, xr):   # the quantiser on the output instead
        a = w13 @ xr
        n = w13.shape[0] // 2
        h = a[:n] / (1.0 + np.exp(-a[:n])) * a[n:]
        return _qdq_1x128_torch((w2 @ h)[None, :], pow2)[0]

    deq = lambda q, s: (torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy()
                        * np.kron(s.astype(np.float64), np.ones((128, 128))))
    xq = _qdq_1x128_torch(synth.bf16_to_f32(inp["x"]).astype(np.float64), pow2)
    slip = np.stack([ffn_quant_after_w2(deq(inp["ws13"], inp["ws13_s"]),
                                        deq(inp["ws2"], inp["ws2_s"]), xq[t]) +
                     sum(w[t, k] * ffn_quant_after_w2(deq(inp["w13"][idx[t, k]],
                                                          inp["w13_s"][idx[t, k]]),
                                                      deq(inp["w2"][idx[t, k]],
                                                          inp["w2_s"][idx[t, k]]), xq[t])
                         for k in range(cfg.K)) for t in range(cfg.T)])
    assert rel(slip, ref) > 1e-4
    # the expert rows (moe_expert_ffn's y) follow the same expression
    e = int(idx[0, 0])
    y = oracle.ffn(cfg, inp, np.array([0]), np.array([e], np.int32), quant_act=True)[0]
    a = deq(inp["w13"][e], inp["w13_s"][e]) @ xq[0]
    h = a[:cfg.I] / (1.0 + np.exp(-a[:cfg.I])) * a[cfg.I:]
    y_ref = deq(inp["w2"][e], inp["w2_s"][e]) @ _qdq_1x128_torch(h[None, :], pow2)[0]
    assert np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref) < 1e-10
    # the two scale rules give different F2 layers (the mode is honoured)
    other = cfg.replace(wdtype="fp8" if pow2 else "fp8e8m0")
    assert rel(oracle.layer(other, inp, idx, w, quant_act=True), got) > 1e-4


def _qdq_cols_torch(v, pow2=False):
    """Column tiles of 128 rows (the last one shorter) through the same
    independent quantiser: rows padded with zeros to a multiple of 128 (no
    change to a tile's maximum or codes), each column cut along the rows."""
    n, f = v.shape
    pad = (-n) % 128
    vp = np.concatenate([v, np.zeros((pad, f))]) if pad else v
    return _qdq_1x128_torch(np.ascontiguousarray(vp.T), pow2).T[:n]


def _fp8_backward_numpy(cfg, inp, e, tokens, dy, quant, dgrad_tiles="rows", wgrad_tiles="cols",
                        quant_h=True):
    """The FP8 backward of one expert written out with numpy fp64 matmuls on
    the dequantised e4m3 weights: x, dy and [dg du] quantised per 1x128 tile
    along the contraction of the dgrad GEMMs (H, H and 2n), and for the
    weight gradients dy, h, [dg du] and x per column in tiles of 128 of the
    expert's rows ("深入理解 DeepSeek-V3…", section 3.2: activations and
    gradients in tiles of 128 along the contraction, weights in 128x128
    blocks).  dgrad_tiles / wgrad_tiles = the other axis and quant_h = False
    give the slips the pin must tell apart."""
    pow2 = cfg.wdtype == "fp8e8m0"
    deq = lambda q, s: (torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy()
                        * np.kron(s.astype(np.float64), np.ones((128, 128))))
    if e < 0:
        w13, w2 = deq(inp["ws13"], inp["ws13_s"]), deq(inp["ws2"], inp["ws2_s"])
    else:
        w13, w2 = deq(inp["w13"][e], inp["w13_s"][e]), deq(inp["w2"][e], inp["w2_s"][e])
    n = w13.shape[0] // 2
    ident = lambda v: v
    qr = (lambda v: _qdq_1x128_torch(v, pow2)) if quant else ident
    qc = (lambda v: _qdq_cols_torch(v, pow2)) if quant else ident
    qd = qr if dgrad_tiles == "rows" else qc
    qw = qc if wgrad_tiles == "cols" else qr
    x = synth.bf16_to_f32(inp["x"]).astype(np.float64)[tokens]
    a = qr(x) @ w13.T
    g, u = a[:, :n], a[:, n:]
    sg = 1.0 / (1.0 + np.exp(-g))
    h = g * sg * u
    dh = qd(dy) @ w2
    da = np.concatenate([dh * u * sg * (1.0 + g * (1.0 - sg)), dh * g * sg], axis=1)
    return {"dx": qd(da) @ w13, "dw2": qw(dy).T @ (qw(h) if quant_h else h),
            "dw13": qw(da).T @ qw(x)}


@pytest.mark.parametrize("wdtype", ["fp8", "fp8e8m0"])
def test_fp8_backward_matches_numpy_expression(wdtype):
    """The oracle's FP8 backward (reading R15) against the numpy expression
    above, for a routed expert and the shared expert, over 200 rows (one full
    column tile and a short one), at 1e-10.  The readings it must not take --
    the operands left unquantised, dgrad tiles cut along the rows instead of
    the contraction, weight-gradient tiles cut along the features, h left
    unquantised -- each sit orders of magnitude further away.  Unquantised,
    the oracle is the exact backward of the dequantised weights."""
    cfg = synth.C5.replace(name="b8-pin", T=200, H=256, E=2, G=1, TG=1, K=1, I=128, Is=256,
                           rho=1.0, wdtype=wdtype)
    inp = synth.gen_inputs(cfg)
    # magnitudes that vary by powers of two along rows and along columns, so
    # that tiles cut along either axis get different scales (with
    # power-of-two scales, tiles of similar magnitude would share them)
    spread = np.ldexp(1.0, (np.arange(cfg.T)[:, None] % 3) + (np.arange(cfg.H)[None, :] % 5))
    x = synth.bf16_to_f32(inp["x"]).astype(np.float64) * spread
    inp["x"] = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)   # exact
    rng = np.random.default_rng(5)
    # worst row: the rows of small magnitude are where the tile axis shows
    rel = lambda a, b: (np.linalg.norm(a - b, axis=1) / np.linalg.norm(b, axis=1)).max()
    for e in (1, -1):
        tokens = rng.permutation(cfg.T)
        dy = synth.bf16_to_f32(synth.normal_bf16(200 * cfg.H, 4, synth.T_TEST, 2 + e, 0.05))
        dy = dy.reshape(200, cfg.H).astype(np.float64) * np.ldexp(
            1.0, 3 * (np.arange(200)[:, None] % 6) - 3 * (np.arange(cfg.H)[None, :] % 6))
        got = oracle.ffn_backward(cfg, inp, e, tokens, dy, quant_act=True)
        ref = _fp8_backward_numpy(cfg, inp, e, tokens, dy, quant=True)
        exact = _fp8_backward_numpy(cfg, inp, e, tokens, dy, quant=False)
        for k in ("dx", "dw13", "dw2"):
            assert got[k].shape == ref[k].shape, k
            assert rel(got[k], ref[k]) < 1e-10, (e, k, rel(got[k], ref[k]))
            assert rel(exact[k], ref[k]) > 1e-4, k
        unq = oracle.ffn_backward(cfg, inp, e, tokens, dy, quant_act=False)
        for k in ("dx", "dw13", "dw2"):
            assert rel(unq[k], exact[k]) < 1e-10, k
        slip = _fp8_backward_numpy(cfg, inp, e, tokens, dy, quant=True, dgrad_tiles="cols")
        assert rel(slip["dx"], ref["dx"]) > 1e-4
        slip = _fp8_backward_numpy(cfg, inp, e, tokens, dy, quant=True, wgrad_tiles="rows")
        assert rel(slip["dw2"], ref["dw2"]) > 1e-4
        slip = _fp8_backward_numpy(cfg, inp, e, tokens, dy, quant=True, quant_h=False)
        assert rel(slip["dw2"], ref["dw2"]) > 1e-4


def test_fp8_backward_pow2_unquantised_equals_fp32_backward():
    """With power-of-two block scales every dequantised weight is exact in
    fp32, so the oracle's unquantised FP8 backward must equal its exact fp32
    backward run on those fp32 weights (two independent weight paths: block
    scales in the e4m3 reader, none in the fp32 one)."""
    cfg = synth.C5.replace(name="b8-f32", T=40, H=256, E=2, G=1, TG=1, K=1, I=128, Is=128,
                           rho=1.0, wdtype="fp8e8m0")
    inp = synth.gen_inputs(cfg)
    deq = lambda q, s: (torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy()
                        * np.kron(s.astype(np.float64), np.ones((128, 128))))
    f32 = dict(inp)
    for k in ("w13", "w2"):
        f32[k] = np.stack([deq(inp[k][e], inp[k + "_s"][e]) for e in range(cfg.E)]
                          ).astype(np.float32)
        f32["ws" + k[1:]] = deq(inp["ws" + k[1:]], inp["ws" + k[1:] + "_s"]).astype(np.float32)
    for k in ("w13", "w2"):
        assert np.array_equal(f32[k].astype(np.float64),
                              np.stack([deq(inp[k][e], inp[k + "_s"][e]) for e in range(cfg.E)]))
    cfg32 = cfg.replace(wdtype="f32")
    rng = np.random.default_rng(9)
    tokens = rng.permutation(cfg.T)
    dy = synth.bf16_to_f32(synth.normal_bf16(cfg.T * cfg.H, 5, synth.T_TEST, 0, 1.0)).reshape(
        cfg.T, cfg.H).astype(np.float64)
    for e in (0, -1):
        a = oracle.ffn_backward(cfg, inp, e, tokens, dy, quant_act=False)
        b = oracle.ffn_backward(cfg32, f32, e, tokens, dy)
        for k in ("dx", "dw13", "dw2"):
            np.testing.assert_allclose(a[k], b[k], rtol=1e-12, atol=1e-12 * np.abs(b[k]).max())


def test_quant_rows_pow2_definition():
    """Power-of-two 1x128 scales: every scale is a power of two, the
    smallest one with scale >= max|v| / 448 (so max|code| lies in (224, 448]),
    codes are torch's e4m3 of v / scale (exact division), all-zero tiles get
    scale 1 and zero codes; at max|v| = 448 * 2^k exactly the scale is 2^k,
    one float ulp above it is 2^(k+1)."""
    rng = np.random.default_rng(5)
    v = (rng.standard_normal((6, 512)) * np.exp(rng.uniform(-12, 4, (6, 1)))).astype(np.float32)
    v[2, 128:256] = 0.0
    v[3, 0:128] *= 0.0
    v[3, 0] = 448.0 * 2.0 ** -5                       # max exactly 448 * 2^-5
    v[4, 256:384] = np.float32(0.5) * v[4, 256:384] / np.abs(v[4, 256:384]).max()
    v[4, 300] = np.nextafter(np.float32(448.0 * 2.0 ** -9), np.float32(1.0))  # one ulp above
    q, s = oracle.quant_rows(v, pow2=True)
    m, e = np.frexp(s.astype(np.float64))
    assert np.all(m == 0.5), "scales are powers of two"
    t = v.reshape(6, 4, 128).astype(np.float64)
    a = np.abs(t).max(axis=-1)
    nz = a > 0
    assert np.all(s[~nz] == 1.0) and np.all(q.reshape(6, 4, 128)[~nz] == 0)
    assert np.all(s[nz] >= a[nz] / 448.0) and np.all(s[nz] / 2 < a[nz] / 448.0)
    assert s[3, 0] == 2.0 ** -5 and s[4, 2] == 2.0 ** -8
    ref = torch.from_numpy((t / s[..., None].astype(np.float64)).astype(np.float32))
    ref = ref.to(torch.float8_e4m3fn).view(torch.uint8).numpy().reshape(6, 512)
    np.testing.assert_array_equal(q, ref)
    codes = np.vectorize(oracle.e4m3_decode)(q).reshape(6, 4, 128)
    peak = np.abs(codes).max(axis=-1)
    assert np.all(peak[nz] > 224.0 - 1e-9) and np.all(peak[nz] <= 448.0)


def test_generator_pow2_e4m3_weights():
    """fp8e8m0 weights: block scales are powers of two (the smallest not
    below the block's max |w| / 448) and dequantise to the normal draws
    within an e4m3 rounding step."""
    q, s = synth.normal_e4m3_blocks(256, 384, 0, synth.T_TEST, 12, 0.05, pow2=True)
    v = synth.normal_f32(256 * 384, 0, synth.T_TEST, 12, 0.05).reshape(256, 384)
    m, _ = np.frexp(s.astype(np.float64))
    assert np.all(m == 0.5)
    a = np.abs(v.reshape(2, 128, 3, 128)).max(axis=(1, 3)).astype(np.float64)
    assert np.all(s >= a / 448.0) and np.all(s / 2 < a / 448.0)
    deq = (torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy() *
           np.kron(s, np.ones((128, 128))))
    np.testing.assert_allclose(deq, v, rtol=2 ** -4, atol=float(s.max()) * 2 ** -9)


# ---------------------------------------------------------------- per-row FFN and the combine step

def test_ffn_rows_match_numpy_and_compose_to_layer():
    cfg = synth.C1.replace(T=30, H=128, E=8, G=4, TG=2, K=3, I=64, Is=96, rho=1.3)
    inp = synth.gen_inputs(cfg)
    r = oracle.forward(cfg, inp)
    counts, offsets, perm, pos = oracle.permute(r["idx"], cfg.E)
    experts = np.repeat(np.arange(cfg.E), counts)
    y = oracle.ffn(cfg, inp, perm // cfg.K, experts)              # sorted-order rows
    ys = oracle.ffn(cfg, inp, np.arange(cfg.T), -np.ones(cfg.T, np.int32))
    x = inp["x"].astype(np.float64)
    for j in (0, 7, len(perm) - 1):
        e, t = experts[j], perm[j] // cfg.K
        ref = _np_ffn(x[t:t + 1], inp["w13"][e].astype(np.float64), inp["w2"][e].astype(np.float64))
        np.testing.assert_allclose(y[j], ref[0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ys, _np_ffn(x, inp["ws13"].astype(np.float64),
                                           inp["ws2"].astype(np.float64)), rtol=1e-12, atol=1e-13)
    # combine of the sorted rows = the layer computed token by token
    out = oracle.combine(y, ys, pos, r["w"], cfg.K)
    np.testing.assert_allclose(out, r["out"], rtol=1e-12, atol=1e-13)


def test_combine_formula_on_random_rows():
    T, K, H = 9, 3, 16
    y = synth.normal_f32(T * K * H, 7, synth.T_TEST, 20, 1.0).reshape(T * K, H).astype(np.float64)
    ys = synth.normal_f32(T * H, 7, synth.T_TEST, 21, 1.0).reshape(T, H).astype(np.float64)
    w = synth.uniform_f32(T * K, 7, synth.T_TEST, 22, 0, 2).reshape(T, K).astype(np.float64)
    pos = np.argsort(synth.words(T * K, 7, synth.T_TEST, 23), kind="stable").astype(np.int32)
    out = oracle.combine(y, ys, pos, w, K)
    ref = ys + np.einsum("tk,tkh->th", w, y[pos.reshape(T, K)])
    np.testing.assert_allclose(out, ref, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(oracle.combine(y, None, pos, w, K), ref - ys, rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------- bias update

def _bias_cases():
    with open(os.path.join(GOLD, "bias_update_hand_cases.json")) as f:
        return json.load(f)["cases"]


def _f32(vals):
    return np.array([float(v) for v in vals], np.float32)


@pytest.mark.parametrize("case", _bias_cases(), ids=lambda c: c["name"])
def test_bias_update_hand_cases(case):
    out = oracle.bias_update(np.array(case["counts"]), case["gamma"], _f32(case["bias"]))
    if "expected_bits" in case:
        want = np.array(case["expected_bits"], np.uint32)
    else:
        want = _f32(case["expected"]).view(np.uint32)
    assert out.view(np.uint32).tolist() == want.tolist()


def test_bias_update_rejects_bad_arguments():
    b = np.zeros(3, np.float32)
    for gamma in (-0.1, float("nan"), float("inf")):
        with pytest.raises(ValueError):
            oracle.bias_update(np.array([1, 2, 3]), gamma, b)
    with pytest.raises(ValueError):
        oracle.bias_update(np.array([1, -2, 3]), 0.1, b)


def test_bias_update_moves_depend_on_counts_only():
    # With dyadic biases and step every sum is exact, so adding a constant to
    # every bias adds it to every result: the moves are the same.
    rng = np.random.default_rng(5)
    counts = rng.integers(0, 40, 64)
    b = (rng.integers(-1024, 1024, 64) / 1024.0).astype(np.float32)
    gamma = 2.0 ** -8
    d0 = oracle.bias_update(counts, gamma, b).astype(np.float64) - b
    d1 = oracle.bias_update(counts, gamma, b + np.float32(0.5)).astype(np.float64) - (b + 0.5)
    assert np.array_equal(d0, d1)
    mean = counts.sum() / 64
    assert np.array_equal(np.sign(d0), np.sign(mean - counts) * (gamma > 0))


def test_bias_update_is_permutation_equivariant():
    rng = np.random.default_rng(6)
    counts = rng.integers(0, 9, 33)
    b = rng.standard_normal(33).astype(np.float32)
    p = rng.permutation(33)
    out = oracle.bias_update(counts, 0.01, b)
    outp = oracle.bias_update(counts[p], 0.01, b[p])
    assert np.array_equal(out[p].view(np.uint32), outp.view(np.uint32))


def test_bias_update_balances_a_skewed_router():
    # Closed loop on a small group-limited router: route, count, update.  A
    # bias that favours three experts is driven back toward the mean load;
    # a sign slip in the update would make the imbalance grow instead.
    cfg = Shape(H=1, E=16, G=4, TG=2, K=2, I=0, Is=0, rho=1.0)
    rng = np.random.default_rng(7)
    lg = rng.standard_normal((512, 16))
    bias = np.zeros(16, np.float32)
    bias[:3] = 0.5

    def imbalance(b):
        idx, _, _ = oracle.route_f64(cfg, lg, b)
        counts, _, _, _ = oracle.permute(idx, 16)
        return counts, counts.max() / counts.mean()

    _, start = imbalance(bias)
    history = []
    for _ in range(400):
        counts, r = imbalance(bias)
        history.append(r)
        bias = oracle.bias_update(counts, 0.005, bias)
    assert start > 2.0
    assert np.mean(history[-50:]) < 1.25


# ---------------------------------------------------------------- expert FFN backward

FD_CFG = synth.C1.replace(name="fd-T6-H16-E4-I8", T=6, H=16, E=4, G=2, TG=1, K=1, I=8, Is=8,
                          rho=1.0)


@pytest.fixture(scope="module")
def fd_inputs():
    return synth.gen_inputs(FD_CFG)


def _loss(cfg, inp, expert, tokens, dy):
    """L = sum_r <dy_r, FFN(x_{tokens[r]})> in fp64."""
    y = oracle.ffn(cfg, inp, tokens, np.full(len(tokens), expert, np.int32))
    return float((y * dy).sum())


@pytest.mark.parametrize("expert", [2, -1])
def test_ffn_backward_matches_finite_differences(fd_inputs, expert):
    # Central differences of L with exact fp32 perturbations (2^-12 added to
    # values near 0.3 is exact), error O(eps^2): every entry of dW13, dW2 and
    # of the input gradient (a token used by two rows gets both rows' dx).
    cfg, inp = FD_CFG, fd_inputs
    tokens = np.array([0, 3, 5, 3], np.int64)
    rng = np.random.default_rng(11)
    dy = rng.standard_normal((len(tokens), cfg.H))
    b = oracle.ffn_backward(cfg, inp, expert, tokens, dy)
    eps = np.float32(2.0 ** -12)
    k13, k2 = ("ws13", "ws2") if expert < 0 else ("w13", "w2")

    def fd(key, index):
        plus, minus = dict(inp), dict(inp)
        a = inp[key].copy(); a[index] += eps; plus[key] = a
        a = inp[key].copy(); a[index] -= eps; minus[key] = a
        return (_loss(cfg, plus, expert, tokens, dy) - _loss(cfg, minus, expert, tokens, dy)) / (
            2 * float(eps))

    e = expert
    w13_shape = b["dw13"].shape
    fd13 = np.array([[fd(k13, (i, j) if e < 0 else (e, i, j)) for j in range(w13_shape[1])]
                     for i in range(w13_shape[0])])
    np.testing.assert_allclose(b["dw13"], fd13, rtol=1e-5, atol=1e-8)
    fd2 = np.array([[fd(k2, (i, j) if e < 0 else (e, i, j)) for j in range(b["dw2"].shape[1])]
                    for i in range(b["dw2"].shape[0])])
    np.testing.assert_allclose(b["dw2"], fd2, rtol=1e-5, atol=1e-8)
    for t in np.unique(tokens):
        fdx = np.array([fd("x", (t, j)) for j in range(cfg.H)])
        np.testing.assert_allclose(b["dx"][tokens == t].sum(0), fdx, rtol=1e-5, atol=1e-8)


def test_ffn_backward_linear_in_dy_and_additive_over_rows(fd_inputs):
    cfg, inp = FD_CFG, fd_inputs
    rng = np.random.default_rng(12)
    t1, t2 = np.array([1, 2], np.int64), np.array([4, 0, 5], np.int64)
    d1, d2 = rng.standard_normal((2, cfg.H)), rng.standard_normal((3, cfg.H))
    b1 = oracle.ffn_backward(cfg, inp, 1, t1, d1)
    b2 = oracle.ffn_backward(cfg, inp, 1, t2, d2)
    both = oracle.ffn_backward(cfg, inp, 1, np.concatenate([t1, t2]), np.concatenate([d1, d2]))
    np.testing.assert_allclose(both["dw13"], b1["dw13"] + b2["dw13"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(both["dw2"], b1["dw2"] + b2["dw2"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(both["dx"], np.concatenate([b1["dx"], b2["dx"]]), rtol=1e-12)
    scaled = oracle.ffn_backward(cfg, inp, 1, t1, -3.0 * d1)
    for k in ("dx", "dw13", "dw2"):
        np.testing.assert_allclose(scaled[k], -3.0 * b1[k], rtol=1e-12, atol=1e-14)


def test_ffn_backward_zero_up_rows_give_zero_grads_but_gate_rows(fd_inputs):
    # With the up rows of W13 zero, u = 0: h = 0 so dW2 = 0, the gate rows get
    # no gradient (dg = dh u silu' = 0) and only the up rows get one.
    cfg, inp = FD_CFG, dict(fd_inputs)
    w13 = inp["w13"].copy()
    w13[:, cfg.I:, :] = 0.0
    inp["w13"] = w13
    dy = np.random.default_rng(13).standard_normal((3, cfg.H))
    b = oracle.ffn_backward(cfg, inp, 0, np.array([0, 1, 2]), dy)
    assert np.all(b["dw2"] == 0.0)
    assert np.all(b["dw13"][:cfg.I] == 0.0)
    assert np.any(b["dw13"][cfg.I:] != 0.0)


@pytest.mark.parametrize("expert", [1, -1])
def test_ffn_backward_entries_equal_full_gradients(fd_inputs, expert):
    cfg, inp = FD_CFG, fd_inputs
    tokens = np.array([2, 0, 5, 5, 1], np.int64)
    dy = np.random.default_rng(14).standard_normal((len(tokens), cfg.H))
    full = oracle.ffn_backward(cfg, inp, expert, tokens, dy)
    ne = cfg.Is if expert < 0 else cfg.I
    which = np.array([0] * (2 * ne * cfg.H) + [1] * (cfg.H * ne))
    r13, c13 = np.divmod(np.arange(2 * ne * cfg.H), cfg.H)
    r2, c2 = np.divmod(np.arange(cfg.H * ne), ne)
    got = oracle.ffn_backward_entries(cfg, inp, expert, tokens, dy, which,
                                      np.concatenate([r13, r2]), np.concatenate([c13, c2]))
    np.testing.assert_allclose(got[:2 * ne * cfg.H], full["dw13"].ravel(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(got[2 * ne * cfg.H:], full["dw2"].ravel(), rtol=1e-12, atol=1e-14)


# Layer backward with the routing held fixed (a top-k choice is piecewise
# constant): central differences of L = sum_t <dout_t, out_t>, where out comes
# from the oracle's forward with the routing weights recomputed from the
# perturbed logits.  Every perturbation must leave the routing unchanged.
LB_CFGS = [synth.C1.replace(name="lbwd-T6-H16-E4-K2", T=6, H=16, E=4, G=2, TG=1, K=2, I=8, Is=8,
                            rho=2.5),
           synth.C1.replace(name="lbwd-T5-H16-E4-K1-noshared", T=5, H=16, E=4, G=2, TG=2, K=1,
                            I=8, Is=0, rho=1.7)]


def _layer_loss(cfg, inp, idx, dout):
    lg = oracle.logits(inp["x"], cfg.act, inp["gate_w"])
    idx2, _, _ = oracle.route_f64(cfg, lg, inp["bias"])
    assert np.array_equal(idx2, idx), "perturbation changed the routing"
    out = oracle.layer(cfg, inp, idx, oracle.routing_weights(cfg, lg, idx))
    return float((out * dout).sum())


@pytest.mark.parametrize("cfg", LB_CFGS, ids=lambda c: c.name)
def test_layer_backward_matches_finite_differences(cfg):
    inp = synth.gen_inputs(cfg)
    lg = oracle.logits(inp["x"], cfg.act, inp["gate_w"])
    idx, w, margin = oracle.route_f64(cfg, lg, inp["bias"])
    assert margin.min() > 1e-3
    # the weights the backward differentiates are the router's own
    np.testing.assert_array_equal(oracle.routing_weights(cfg, lg, idx), w)
    dout = np.random.default_rng(21).standard_normal((cfg.T, cfg.H))
    b = oracle.layer_backward(cfg, inp, idx, dout)
    eps = np.float32(2.0 ** -12)

    def fd(key, index):
        plus, minus = dict(inp), dict(inp)
        a = inp[key].copy(); a[index] += eps; plus[key] = a
        a = inp[key].copy(); a[index] -= eps; minus[key] = a
        return (_layer_loss(cfg, plus, idx, dout) - _layer_loss(cfg, minus, idx, dout)) / (
            2 * float(eps))

    keys = [("x", "dx"), ("gate_w", "dgate_w"), ("w13", "dw13"), ("w2", "dw2")]
    if cfg.Is:
        keys += [("ws13", "dws13"), ("ws2", "dws2")]
    for key, gkey in keys:
        num = np.array([fd(key, ix) for ix in np.ndindex(*inp[key].shape)]).reshape(inp[key].shape)
        # central differences carry an O(eps^2) curvature term: 1e-5 of the
        # gradient's scale covers it, and a dropped term or wrong sign is O(1)
        np.testing.assert_allclose(b[gkey], num, rtol=1e-5, atol=1e-5 * np.abs(num).max(),
                                   err_msg=gkey)


def test_layer_backward_gate_gradient_zero_when_weights_cannot_move():
    # top-1 with rho: w = rho * s, so the gate gets dlogit = rho <dout, y> s (1 - s);
    # with dout orthogonal to every chosen expert's output the gate gradient
    # vanishes while the experts' gradients do not.
    cfg = LB_CFGS[1]
    inp = synth.gen_inputs(cfg)
    lg = oracle.logits(inp["x"], cfg.act, inp["gate_w"])
    idx, _, _ = oracle.route_f64(cfg, lg, inp["bias"])
    y = oracle.ffn(cfg, inp, np.arange(cfg.T), idx[:, 0])
    dout = np.random.default_rng(22).standard_normal((cfg.T, cfg.H))
    dout -= (np.einsum("th,th->t", dout, y) / np.einsum("th,th->t", y, y))[:, None] * y
    b = oracle.layer_backward(cfg, inp, idx, dout)
    np.testing.assert_allclose(b["dgate_w"], 0.0, atol=1e-12)
    assert np.abs(b["dw2"]).max() > 1e-3


def test_layer_backward_token_subsets_agree_with_the_whole():
    # dx rows depend on their own token only; an expert's gate gradient on
    # the tokens routed to it only
    cfg = LB_CFGS[0]
    inp = synth.gen_inputs(cfg)
    lg = oracle.logits(inp["x"], cfg.act, inp["gate_w"])
    idx, _, _ = oracle.route_f64(cfg, lg, inp["bias"])
    dout = np.random.default_rng(23).standard_normal((cfg.T, cfg.H))
    full = oracle.layer_backward(cfg, inp, idx, dout)
    sub = oracle.layer_backward(cfg, inp, idx, dout, tokens=[4, 1], want=("dx",))
    np.testing.assert_allclose(sub["dx"], full["dx"][[4, 1]], rtol=1e-12, atol=1e-14)
    e = int(idx[0, 0])
    toks = np.flatnonzero((idx == e).any(axis=1))
    sub = oracle.layer_backward(cfg, inp, idx, dout, tokens=toks, want=("dgate_w",))
    np.testing.assert_allclose(sub["dgate_w"][e], full["dgate_w"][e], rtol=1e-12, atol=1e-14)


# FP8 layer backward (e4m3 expert weights, quant_act): the gate's gradient is
# that of the activation-quantised forward (F2) with the routing held -- the
# F2 expert outputs do not depend on the gate weight, so central differences
# of L = sum_t <dout_t, out_F2_t> in gate_w pin the combine and routing-weight
# terms; the experts' terms are the FP8 expert backward, pinned above, and
# differ from the exact backward of the dequantised weights by the e4m3
# rounding of their operands.
LB8_CFG = synth.C5.replace(name="lbwd8-T6-H128-E4-K2", T=6, H=128, E=4, G=2, TG=1, K=2, I=128,
                           Is=128, rho=2.5)


def test_fp8_layer_backward_gate_gradient_matches_f2_differences():
    cfg = LB8_CFG
    inp = synth.gen_inputs(cfg)
    lg = oracle.logits(inp["x"], cfg.act, inp["gate_w"])
    idx, _, margin = oracle.route_f64(cfg, lg, inp["bias"])
    assert margin.min() > 1e-4
    dout = np.random.default_rng(24).standard_normal((cfg.T, cfg.H))
    b = oracle.layer_backward(cfg, inp, idx, dout, want=("dgate_w",), quant_act=True)
    eps = 2.0 ** -12

    def loss(gw):
        lg2 = oracle.logits(inp["x"], cfg.act, gw)
        idx2, _, _ = oracle.route_f64(cfg, lg2, inp["bias"])
        assert np.array_equal(idx2, idx), "perturbation changed the routing"
        out = oracle.layer(cfg, inp, idx, oracle.routing_weights(cfg, lg2, idx), quant_act=True)
        return float((out * dout).sum())

    gw = inp["gate_w"].astype(np.float64)
    num = np.zeros_like(gw)
    for e in np.unique(idx):
        for h in range(cfg.H):
            p, m = gw.copy(), gw.copy()
            p[e, h] += eps
            m[e, h] -= eps
            num[e, h] = (loss(p) - loss(m)) / (2 * eps)
    np.testing.assert_allclose(b["dgate_w"], num, rtol=1e-5, atol=1e-5 * np.abs(num).max())
    # the unquantised mode gives a different (dequantised-forward) gate gradient
    b1 = oracle.layer_backward(cfg, inp, idx, dout, want=("dgate_w",))
    d = np.linalg.norm(b1["dgate_w"] - b["dgate_w"]) / np.linalg.norm(b["dgate_w"])
    assert 1e-4 < d < 0.2, d


def test_fp8_layer_backward_experts_are_the_fp8_expert_backward():
    # quant_act moves every expert term by about the e4m3 rounding of its
    # operands; without it the layer backward of e4m3 weights is the exact
    # backward of the dequantised weights (central differences in x)
    cfg = LB8_CFG
    inp = synth.gen_inputs(cfg)
    lg = oracle.logits(inp["x"], cfg.act, inp["gate_w"])
    idx, _, _ = oracle.route_f64(cfg, lg, inp["bias"])
    dout = np.random.default_rng(25).standard_normal((cfg.T, cfg.H))
    bq = oracle.layer_backward(cfg, inp, idx, dout, quant_act=True)
    be = oracle.layer_backward(cfg, inp, idx, dout)
    for k in ("dx", "dw13", "dw2", "dws13", "dws2"):
        busy = np.unique(idx) if k in ("dw13", "dw2") else slice(None)
        d = np.linalg.norm(bq[k][busy] - be[k][busy]) / np.linalg.norm(be[k][busy])
        assert 1e-3 < d < 0.15, (k, d)
    # the exact mode's dx: central differences of the dequantised-weight
    # forward in x would need bf16 x perturbations; the routing weights and
    # experts are differentiated in fp64 through the float x the oracle reads
    xf = (inp["x"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    w = oracle.routing_weights(cfg, lg, idx)
    t, h = 3, 17
    eps = 2.0 ** -10

    def loss(xv):
        x2 = dict(inp, x=xv.astype(np.float32))
        cf = cfg.replace(act="f32")
        lg2 = oracle.logits(x2["x"], "f32", inp["gate_w"])
        out = oracle.layer(cf, x2, idx, oracle.routing_weights(cf, lg2, idx))
        return float((out * dout).sum())

    p, m = xf.copy(), xf.copy()
    p[t, h] += eps
    m[t, h] -= eps
    num = (loss(p) - loss(m)) / (2 * eps)
    assert abs(be["dx"][t, h] - num) <= 1e-5 * max(1.0, abs(num)), (be["dx"][t, h], num)
    assert np.array_equal(w, oracle.routing_weights(cfg, lg, idx))


def test_round_bf16_is_torch_bf16_cast():
    # the bf16 rounding of the FP8 layer backward's dy rows: fp32 first, then
    # nearest-even to bf16, as torch's cast does it (ties, subnormals, signs)
    import torch
    rng = np.random.default_rng(26)
    v = rng.standard_normal(200000) * np.exp(rng.uniform(-90, 90, 200000))
    v[:4] = [0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8]   # exact ties
    got = oracle.round_bf16(v)
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).float().double().numpy()
    np.testing.assert_array_equal(got, ref)
    assert got[2] == 1.0 and got[3] == 1.0 + 2.0 ** -6
