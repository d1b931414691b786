"""Writes zipf_bias_k8.txt and zipf_bias_k1.txt: selection biases under which
the expert loads of the V3-shape gate follow Zipf(1.2).

The co-design explainer ('从 1024 块 GPU 到 558 万美元：拆解 DeepSeek-V3 的算法-系统协同设计',
section 2.2) says the per-expert bias is a buffer adjusted from the observed
load, outside the gradient, and that it only affects the choice.  No update
rule is printed, so this script uses a plain one offline to make a skewed,
reproducible routing for the decode workloads:

  target   : Zipf(1.2) over a seeded random ranking of the experts, scaled to
             T_cal * top_k picks and water-filled under the cap load <= T_cal
             (an expert is picked at most once per token);
  update   : b_e += eta * (log target_e - log max(load_e, 1/2)), loads from
             the oracle's fp64 router on a seeded calibration batch of
             T_cal = 16384 tokens (generator stream x_cal);
  finally  : shift b by a constant so that min b >= 0, which keeps every
             choice score positive and so leaves all selections unchanged.

Only the oracle and the generator are called.  Run from the repository root:
    python tests/golden/make_zipf_bias.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth   # noqa: E402

T_CAL = 16384
ZIPF_S = 1.2
ITERS = 400


def waterfill(p, total, cap):
    """Scale p to sum to total with every entry <= cap (excess spread
    proportionally over the uncapped entries)."""
    t = np.zeros_like(p)
    free = np.ones(len(p), bool)
    remaining = total
    while True:
        t[free] = p[free] / p[free].sum() * remaining
        over = free & (t > cap)
        if not over.any():
            return t
        t[over] = cap
        free &= ~over
        remaining = total - t[~free].sum()


def calibrate(K, lg, E, rank_perm):
    cfg = synth.C3.replace(K=K)
    r = np.arange(1, E + 1, dtype=np.float64)
    p = np.empty(E)
    p[rank_perm] = r ** -ZIPF_S
    target = waterfill(p / p.sum(), T_CAL * K, float(T_CAL))
    b = np.zeros(E, np.float32)
    best = None
    for it in range(ITERS):
        idx, _, _ = oracle.route_f64(cfg, lg, b)
        load = np.bincount(idx.ravel(), minlength=E).astype(np.float64)
        q = load / load.sum()
        tq = target / target.sum()
        kl = float(np.sum(np.where(tq > 0, tq * np.log(tq / np.maximum(q, 1e-12)), 0.0)))
        if best is None or kl < best[0]:
            best = (kl, b.copy(), load.copy())
        eta = 0.05 if it < 200 else 0.02
        b = (b + eta * (np.log(target) - np.log(np.maximum(load, 0.5)))).astype(np.float32)
    kl, b, load = best
    b = (b - b.min()).astype(np.float32)
    idx2, _, _ = oracle.route_f64(cfg, lg, b)
    load2 = np.bincount(idx2.ravel(), minlength=E)
    assert np.array_equal(load2, load), "shift changed the routing"
    return b, load, target, kl


def main():
    cfg = synth.C3
    wg, _ = synth.gen_gate(cfg.replace(bias_file=None))
    xcal = synth.gen_x(cfg, T_CAL, tensor=synth.T_XCAL)
    lg = oracle.logits(xcal, "bf16", wg)
    rank_perm = np.argsort(synth.words(cfg.E, cfg.seed, synth.T_TEST, 777), kind="stable")
    for K, name in ((8, "zipf_bias_k8.txt"), (1, "zipf_bias_k1.txt")):
        b, load, target, kl = calibrate(K, lg, cfg.E, rank_perm)
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), name)
        order = np.argsort(-target, kind="stable")
        with open(path, "w") as f:
            f.write(f"# Selection bias (float32 bit patterns, one per expert) for the V3-shape gate\n"
                    f"# (seed 0), top_k={K}, calibrated so expert loads follow Zipf({ZIPF_S}).\n"
                    f"# Written by tests/golden/make_zipf_bias.py (oracle router on {T_CAL} tokens).\n"
                    f"# KL(target || achieved) = {kl:.4f}; active experts = {(load > 0).sum()}\n"
                    f"# top-8 target loads: {np.round(target[order[:8]]).astype(int).tolist()}\n"
                    f"# top-8 achieved   : {load[order[:8]].astype(int).tolist()}\n")
            for v in b.view(np.uint32):
                f.write(f"{v:08x}\n")
        print(name, "KL", round(kl, 4), "max load", int(load.max()), "active", int((load > 0).sum()))


if __name__ == "__main__":
    main()
