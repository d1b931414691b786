"""Benchmark: one MoE layer forward (gate, permute, expert FFNs, combine) per
step on one MI355X, V3 shape (H=7168, 256 routed experts in 8 groups, top-4
groups, top-8, expert and shared FFN width 2048, routed scaling 2.5), bf16,
T=4096 tokens of synthetic seeded input resident in HBM.  bf16 expert weights
are packed once into the streaming layout (moe_pack_weight) before timing,
as a model load would.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--cpu-sample S]
    python bench.py --copy-calibration     (a 1 GiB device copy, for counters)

Prints one JSON line.  A step is timed by HIP events on the launch stream,
with a 1 GiB scratch write before each step (outside its events) so that no
cache holds its inputs; ms_per_step is the median over the K steps, and the
back-to-back figure is reported beside it.  The per-kernel times (HIP events
on the stream each kernel runs on) give the roofline of the dominant kernel.
The CPU baseline is the fp64 oracle on a bounded sample of tokens.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0       # dense fp8 MFMA


def log(msg):
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


KERNEL_SOURCES = {
    # kernel name (as the library's timer and rocprofv3 name it) -> sources it is built from
    "grouped_gemm_bf16_packed": ("ffn_bf16_packed.hip", "packed_few.hpp", "moe_internal.hpp"),
    "grouped_gemm_bf16_packed_x2": ("ffn_bf16_packed.hip", "packed_few.hpp", "moe_internal.hpp"),
    "grouped_gemm_bf16_packed_few": ("ffn_bf16_packed.hip", "packed_few.hpp", "moe_internal.hpp"),
    "grouped_gemm_bf16_packed_wide": ("ffn_bf16_packed.hip", "packed_few.hpp",
                                      "moe_internal.hpp"),
    "decode_layer_kernel": ("decode_layer.hip", "combine_device.hpp", "decode_device.hpp",
                            "gate_split.hpp", "packed_few.hpp", "permute_device.hpp",
                            "select_device.hpp", "moe_internal.hpp"),
    "grouped_gemm_fp8_packed": ("ffn_fp8_packed.hip", "moe_internal.hpp"),
    "grouped_gemm_fp8_mx": ("ffn_fp8_mx.hip", "moe_internal.hpp"),
    "grouped_gemm_bf16": ("ffn_bf16.hip", "moe_internal.hpp"),
    "grouped_gemm_fp8": ("ffn_fp8.hip", "moe_internal.hpp"),
    "gate_logits_bf16_kernel": ("gate.hip", "gate_split.hpp", "moe_internal.hpp"),
    "gate_select_fused_kernel": ("gate.hip", "gate_split.hpp", "moe_internal.hpp"),
}


def kernel_source_digest(kernel):
    """sha256 over the sources a kernel is compiled from (None if unknown)."""
    import hashlib
    base = kernel.split("<")[0]
    files = KERNEL_SOURCES.get(base)
    if not files:
        return None
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(HERE, "sparse_mixture_experts_30_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _traffic(workload, kernel):
    """HBM bytes per launch of `kernel` on `workload`, from the committed
    counter record (FETCH_SIZE + WRITE_SIZE, calibrated), or None when there is
    no record or the kernel source changed since it was taken."""
    path = os.path.join(HERE, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except OSError:
        return None
    entry = rec.get(f"{workload}:{kernel}")
    if not entry or entry.get("kernel_source_sha256") != kernel_source_digest(kernel):
        return None
    return entry.get("hbm_bytes_per_launch")


def kernel_work(kernel, cfg, active):
    """Algorithmic (bytes, flop) of one launch of `kernel` on cfg, counting the
    active experts' weights once, each activation row once and each result
    once; None for kernels without a model here."""
    T, H, E, K, I, Is = cfg.T, cfg.H, cfg.E, cfg.K, cfg.I, cfg.Is
    N = T * K
    fp8 = cfg.wdtype in ("fp8", "fp8e8m0")
    wb = 1 if fp8 else {"bf16": 2, "f32": 4}[cfg.wdtype]
    ab = 2 if cfg.act == "bf16" else 4
    hb = 1 if fp8 else ab       # h is kept in e4m3 on the fp8 path
    scale = (lambda r, c: (r // 128) * (c // 128) * 4) if fp8 else (lambda r, c: 0)
    hsc = ((N * I + T * Is) // 128) * 4 if fp8 else 0
    base = kernel.split("<")[0]
    gate_up = "<true" in kernel
    if base.startswith("grouped_gemm"):
        if gate_up:
            w = active * (2 * I * H * wb + scale(2 * I, H)) + (2 * Is * H * wb + scale(2 * Is, H))
            a_in = T * H * (1 if fp8 else ab) + (T * (H // 128) * 4 if fp8 else 0)
            out = (N * I + T * Is) * hb + hsc
            flop = 2.0 * (N * 2 * I + T * 2 * Is) * H
        else:
            w = active * (H * I * wb + scale(H, I)) + (H * Is * wb + scale(H, Is))
            a_in = (N * I + T * Is) * hb + hsc
            out = (N + T) * H * ab
            flop = 2.0 * (N * I + T * Is) * H
        return w + a_in + out, flop
    if base == "gate_logits_bf16_kernel":
        return T * H * ab + E * H * 4 + T * E * 4, 2.0 * T * E * H
    if base == "gate_select_fused_kernel":
        # x and the gate weight (fp32) in; the logits, ids and weights out
        return T * H * ab + E * H * 4 + E * 4 + T * E * 4 + T * K * 8, 2.0 * T * E * H
    if base == "decode_layer_kernel":
        # the whole layer in one launch: the layer's own algorithmic work
        # (x and the output once, the gate weight and bias, the active
        # experts' and the shared expert's weights once)
        w = (active * 3 * H * I + 3 * H * Is) * wb
        return (w + E * H * 4 + E * 4 + 2 * T * H * ab,
                T * (6.0 * H * (I * K + Is) + 2.0 * H * E))
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="v3-layer-bf16-T4096")
    ap.add_argument("--cpu-sample", type=int, default=None,
                    help="tokens of the workload run through the fp64 oracle (0 = skip; default "
                         "384, 96 for the e4m3 layers, whose oracle also quantises: about 15 s "
                         "of host time either way)")
    ap.add_argument("--profile-only", action="store_true",
                    help="for rocprofv3: warmup + steps and the per-kernel breakdown only (no "
                         "oracle, no second entry point, no backward), print the JSON line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="copy 1 GiB device-to-device 5 times (HBM counter calibration)")
    ap.add_argument("--overlap", action="store_true",
                    help="time moe_forward_overlap (shared expert on a second stream) as the step")
    ap.add_argument("--fused", action="store_true",
                    help="time moe_forward_decode_fused (the decode layer in one launch) as the "
                         "step")
    ap.add_argument("--gate-fused", action="store_true",
                    help="gate + permute workload: run the gate and the selection as one kernel "
                         "(MOE_GATE_FUSED) in the timed step")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the expert-FFN backward measurement of the bf16 layer workloads")
    ap.add_argument("--row-major", action="store_true",
                    help="use the row-major weight layout instead of the packed one")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        a.fill_(1)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 1 << 30, "copies": 5}))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import sparse_mixture_experts_30_amd as moe
    from synth import device as sd

    cfg = synth.CONFIGS[args.workload]
    T, H, E, K, I, Is = cfg.T, cfg.H, cfg.E, cfg.K, cfg.I, cfg.Is
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # The gate + permute workload times those two entry points only; every
    # other workload times the whole layer.
    gate_only = cfg.name == synth.C2.name
    t0 = time.time()
    log(f"[bench] {cfg.name}: generating inputs")
    if gate_only:
        inp = {"cfg": cfg, "x": synth.gen_x(cfg)}
        inp["gate_w"], inp["bias"] = synth.gen_gate(cfg)
    else:
        inp = synth.gen_inputs(cfg)
    log(f"[bench] generated in {time.time() - t0:.1f}s; uploading")
    d = sd.to_device(inp)
    # The expert-FFN backward (training) reads row-major weights (bf16, or
    # e4m3 for the FP8 backward): kept for the layer workloads of at least
    # 1024 tokens.
    with_bwd = (not args.no_backward and not args.profile_only and not gate_only and
                cfg.wdtype in ("bf16", "fp8", "fp8e8m0") and cfg.act == "bf16" and T >= 1024)
    drow = d if with_bwd else None
    if cfg.wdtype != "f32" and not args.row_major and not gate_only:
        d = sd.packed_copy(d)   # the row-major device copies are released here unless kept
    W = None if gate_only else sd.weights_struct(d)
    C = sd.moe_config(cfg)
    ws = sd.workspace(cfg, T)
    act_dt = torch.bfloat16 if cfg.act == "bf16" else torch.float32
    out = torch.empty((T, H), dtype=act_dt, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] inputs resident in HBM ({time.time() - t0:.1f}s)")
    stream = torch.cuda.current_stream()

    lg = torch.empty((T, E), dtype=torch.float32, device=dev)
    idx = torch.empty((T, K), dtype=torch.int32, device=dev)
    wt = torch.empty((T, K), dtype=torch.float32, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offs = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(T * K, dtype=torch.int32, device=dev)
    pos = torch.empty(T * K, dtype=torch.int32, device=dev)

    # The layer step: moe_forward on one stream, or (--overlap)
    # moe_forward_overlap, the shared expert's GEMMs on a second stream, or
    # (--fused) moe_forward_decode_fused, a decode batch in one launch.
    shared_stream = torch.cuda.Stream()
    fused_ok = (not gate_only and T <= 32 and cfg.act == "bf16" and cfg.wdtype == "bf16" and
                not args.row_major)
    entries = [] if gate_only else (["moe_forward", "moe_forward_overlap"] +
                                    (["moe_forward_decode_fused"] if fused_ok else []))
    if args.fused and not fused_ok:
        sys.exit("--fused: the one-launch decode layer takes T <= 32, bf16, packed weights")
    if gate_only:
        entry = ("moe_gate (MOE_GATE_FUSED) + moe_permute" if args.gate_fused
                 else "moe_gate + moe_permute")
    else:
        entry = ("moe_forward_decode_fused" if args.fused else
                 "moe_forward_overlap" if args.overlap else "moe_forward")

    def forward(name):
        if name == "moe_forward_overlap":
            moe.moe_forward_overlap(C, T, d["x"], W, out, ws, shared_stream, stream=stream)
        elif name == "moe_forward_decode_fused":
            moe.moe_forward_decode_fused(C, T, d["x"], W, out, ws, stream=stream)
        else:
            moe.moe_forward(C, T, d["x"], W, out, ws, stream=stream)

    if args.gate_fused:
        if not gate_only:
            sys.exit("--gate-fused: for the gate + permute workload")
        moe.moe_set_gate_mode(moe.MOE_GATE_FUSED)

    def step():
        if gate_only:
            moe.moe_gate(C, T, d["x"], d["gate_w"], d["bias"], lg, idx, wt, ws, stream=stream)
            moe.moe_permute(C, T, idx, counts, offs, perm, pos, ws, stream=stream)
        else:
            forward(entry)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Per-kernel breakdown (every launch bracketed by HIP events on its
    # stream), to find the dominant kernel; not part of the timed region.
    moe.moe_kernel_timer_read()
    moe.moe_kernel_timer_enable(True)
    nbreak = max(3, min(args.steps, 10))
    for _ in range(nbreak):
        step()
    torch.cuda.synchronize()
    moe.moe_kernel_timer_enable(False)
    kt = moe.moe_kernel_timer_read()
    kernels_ms = {k: v[0] / v[1] for k, v in kt.items()}
    dominant = max(kt, key=lambda k: kt[k][0])

    # Timed region: K steps between a synchronisation on both sides, each
    # step bracketed by its own events on the launch stream, and a 1 GiB
    # scratch write before every step (outside its events) so that neither
    # the L2s nor the 256 MB Infinity Cache hold x, the gate weight or a
    # previous step's weights; the step time is the median.  Only the
    # dominant kernel is bracketed by the library's per-kernel events here.
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    moe.moe_kernel_timer_enable(True, dominant)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i, (e0, e1) in enumerate(evs):
        flush.fill_(i & 0xFF)
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    moe.moe_kernel_timer_enable(False)
    dom_ms, dom_launches = moe.moe_kernel_timer_read()[dominant]
    dom_ms /= dom_launches
    step_ms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    ms = float(np.median(step_ms))
    # The same steps back to back (no scratch writes): the warm figure.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    warm_ms = ev0.elapsed_time(ev1) / args.steps
    del flush
    log(f"[bench] {ms:.3f} ms/step (median, caches flushed; {warm_ms:.3f} back to back); "
        f"dominant kernel {dominant}: {dom_ms:.3f} ms/launch")

    # The other forward entry points, not in a profiled run (their launches
    # would mix into the traced kernels' figures).  Three rounds that
    # alternate every entry point, K steps each, each step after the 1 GiB
    # scratch write, so that all see the same clocks and cold caches; the
    # medians of the per-step times are reported.
    other = []
    if not gate_only and not args.profile_only:
        times = {e: [] for e in entries}
        flush_o = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        for e in entries:
            for _ in range(2):
                forward(e)
        for r in range(3):
            for e in entries:
                for i in range(args.steps):
                    flush_o.fill_((r + i) & 0xFF)
                    ev0.record(stream)
                    forward(e)
                    ev1.record(stream)
                    torch.cuda.synchronize()
                    times[e].append(ev0.elapsed_time(ev1))
        del flush_o
        med = {e: statistics.median(v) for e, v in times.items()}
        for e in entries:
            if e == entry:
                continue
            other.append({"entry_point": e, "ms": round(med[e], 4),
                          "tokens_per_s": round(T / (med[e] * 1e-3), 1),
                          "step_entry_point_ms_same_rounds": round(med[entry], 4)})
            log(f"[bench] {e}: {med[e]:.3f} ms/step (step entry point {entry} "
                f"{med[entry]:.3f} ms in the same rounds)")
    if gate_only and not args.profile_only and not args.gate_fused:
        # The gate and selection in one kernel (MOE_GATE_FUSED) against the
        # default split kernels: alternating rounds, cold caches, medians.
        times = {moe.MOE_GATE_SPLIT: [], moe.MOE_GATE_FUSED: []}
        flush_o = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        try:
            for r in range(3):
                for mode in times:
                    moe.moe_set_gate_mode(mode)
                    step()
                    for i in range(args.steps):
                        flush_o.fill_((r + i) & 0xFF)
                        ev0.record(stream)
                        step()
                        ev1.record(stream)
                        torch.cuda.synchronize()
                        times[mode].append(ev0.elapsed_time(ev1))
        finally:
            moe.moe_set_gate_mode(moe.MOE_GATE_SPLIT)
        del flush_o
        ms_s = statistics.median(times[moe.MOE_GATE_SPLIT])
        ms_f = statistics.median(times[moe.MOE_GATE_FUSED])
        other.append({"entry_point": "moe_gate (MOE_GATE_FUSED) + moe_permute", "ms": round(ms_f, 4),
                      "tokens_per_s": round(T / (ms_f * 1e-3), 1),
                      "step_entry_point_ms_same_rounds": round(ms_s, 4)})
        log(f"[bench] fused gate: {ms_f:.3f} ms/step (split gate {ms_s:.3f} ms in the same "
            f"rounds)")

    # Per-phase timing with the separate entry points (same kernels, same
    # stream), HIP events between phases.
    y = torch.empty((T * K, H), dtype=act_dt, device=dev) if not gate_only else None
    ys = torch.empty((T, H), dtype=act_dt, device=dev) if Is and not gate_only else None
    phases = ["gate", "permute"] + ([] if gate_only else ["expert_ffn", "combine"])
    acc = {p: 0.0 for p in phases}
    nrep = max(3, min(args.steps, 10))
    for rep in range(nrep + 1):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)]
        evs[0].record(stream)
        moe.moe_gate(C, T, d["x"], d["gate_w"], d["bias"], lg, idx, wt, ws, stream=stream)
        evs[1].record(stream)
        moe.moe_permute(C, T, idx, counts, offs, perm, pos, ws, stream=stream)
        evs[2].record(stream)
        if not gate_only:
            moe.moe_expert_ffn(C, T, d["x"], perm, offs, W, y, ys, ws, stream=stream)
            evs[3].record(stream)
            moe.moe_combine(C, T, y, ys, pos, wt, out, stream=stream)
            evs[4].record(stream)
        torch.cuda.synchronize()
        if rep:  # first repetition is a warmup
            for i, p in enumerate(phases):
                acc[p] += evs[i].elapsed_time(evs[i + 1]) / nrep
    cnt = counts.cpu().numpy()
    active = int((cnt > 0).sum())

    # Load-balancing update of the selection bias from this batch's counts:
    # the training-step follow-up to the forward, not part of the layer step.
    # One launch reads E counts and reads and writes E biases (12 E bytes),
    # a single workgroup: launch latency bound.  Timed on a copy of the bias.
    bias_copy = d["bias"].clone()
    nbu = 200
    moe.moe_bias_update(C, counts, 1e-3, bias_copy, stream=stream)
    torch.cuda.synchronize()
    moe.moe_kernel_timer_read()
    moe.moe_kernel_timer_enable(True, "bias_update_kernel")
    eb0, eb1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    eb0.record(stream)
    for _ in range(nbu):
        moe.moe_bias_update(C, counts, 1e-3, bias_copy, stream=stream)
    eb1.record(stream)
    torch.cuda.synchronize()
    moe.moe_kernel_timer_enable(False)
    bu_ms, bu_launches = moe.moe_kernel_timer_read()["bias_update_kernel"]
    bias_update = {"kernel_us": round(bu_ms / bu_launches * 1e3, 2),
                   "calls_per_s": round(nbu / (eb0.elapsed_time(eb1) * 1e-3), 1),
                   "bytes_per_launch": 12 * E, "bound": "launch latency (one workgroup)"}

    # Backward (training), reported beside the layer step, on this batch's
    # routing: the expert FFNs alone (output gradients of the routed rows and
    # of the shared expert -> input and weight gradients), and the whole
    # layer (the gradient of the layer output -> dx, the gate weight's and
    # every expert weight's gradients).
    backward = layer_backward = None
    if drow is not None:
        gen = torch.Generator(device=dev).manual_seed(23)
        dyb = torch.randn((T * K, H), generator=gen, device=dev).to(torch.bfloat16)
        dysb = torch.randn((T, H), generator=gen, device=dev).to(torch.bfloat16) if Is else None
        bf = dict(dtype=torch.bfloat16, device=dev)
        dxb = torch.empty((T * K, H), **bf)
        dxsb = torch.empty((T, H), **bf) if Is else None
        dw13 = torch.empty((E, 2 * I, H), **bf)
        dw2 = torch.empty((E, H, I), **bf)
        dws13 = torch.empty((2 * Is, H), **bf) if Is else None
        dws2 = torch.empty((H, Is), **bf) if Is else None
        Wrow = sd.weights_struct(drow)

        def timed(fn):
            """(ms per call over 5 calls, per-kernel ms of one call)."""
            fn()
            torch.cuda.synchronize()
            moe.moe_kernel_timer_read()
            moe.moe_kernel_timer_enable(True)
            fn()
            torch.cuda.synchronize()
            moe.moe_kernel_timer_enable(False)
            kms = {k: round(v[0] / v[1], 4) for k, v in moe.moe_kernel_timer_read().items()}
            eb0.record(stream)
            for _ in range(5):
                fn()
            eb1.record(stream)
            torch.cuda.synchronize()
            return eb0.elapsed_time(eb1) / 5, kms

        bwd_fp8 = cfg.wdtype in ("fp8", "fp8e8m0")
        bpeak = FP8_PEAK_TFLOPS if bwd_fp8 else BF16_PEAK_TFLOPS

        def figures(bms, flop, nbytes, kms):
            return {"ms": round(bms, 3), "tflops": round(flop / (bms * 1e-3) / 1e12, 1),
                    "mfma_frac": round(flop / (bms * 1e-3) / 1e12 / bpeak, 4),
                    "hbm_gbs": round(nbytes / (bms * 1e-3) / 1e9, 1),
                    "hbm_frac": round(nbytes / (bms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "algorithmic_flop": flop, "algorithmic_bytes": nbytes, "kernels_ms": kms}

        rows_i = T * K * I + T * Is
        bflop = 16.0 * rows_i * H     # recompute 4, dh 2, dx 4, dW2 2, dW13 4 (x rows*I*H)
        # weights read once (bf16 or e4m3) and their bf16 gradients written
        # once, x, dy, dx once
        wrb = 1 if bwd_fp8 else 2
        bbytes = (wrb + 2) * (active * 3 * H * I + 3 * H * Is) + 3 * (T * K + T) * H * 2
        wsb = torch.empty(moe.moe_expert_ffn_backward_workspace_bytes(C, T), dtype=torch.uint8,
                          device=dev)
        bms, bk = timed(lambda: moe.moe_expert_ffn_backward(
            C, T, drow["x"], perm, offs, Wrow, dyb, dysb, dxb, dxsb, dw13, dw2, dws13, dws2, wsb,
            stream=stream))
        backward = figures(bms, bflop, bbytes, bk)
        backward["dtype"] = "e4m3 operands, fp32 accumulation" if bwd_fp8 else "bf16"
        del wsb

    if drow is not None:
        # the layer: y (the routed expert outputs) from the phase timing above
        dout = torch.randn((T, H), generator=gen, device=dev).to(torch.bfloat16)
        dxl = torch.empty((T, H), **bf)
        dgw = torch.empty((E, H), dtype=torch.float32, device=dev)
        wsl = torch.empty(moe.moe_backward_workspace_bytes(C, T), dtype=torch.uint8, device=dev)
        lms, lk = timed(lambda: moe.moe_backward(
            C, T, drow["x"], Wrow, lg, idx, wt, perm, offs, pos, y, dout, dxl, dgw, dw13, dw2,
            dws13, dws2, wsl, stream=stream))
        # + the combine's dot products, the gate's weight gradient and dx: 6 T K H;
        # + y and dout read, the gate weight read and its gradient written
        layer_backward = figures(lms, bflop + 6.0 * T * K * H,
                                 bbytes + (T * K + T) * H * 2 + 2 * E * H * 4, lk)
        layer_backward["dtype"] = backward["dtype"]
        del dyb, dysb, dxb, dxsb, dw13, dw2, dws13, dws2, wsl, dout, dxl, dgw

    # Algorithmic work (routed rows only; active experts' weights only).
    fp8 = cfg.wdtype in ("fp8", "fp8e8m0")
    wbytes = 1 if fp8 else (2 if cfg.wdtype == "bf16" else 4)
    abytes = 2 if cfg.act == "bf16" else 4
    expert_w = 3 * H * I * wbytes
    shared_w = 3 * H * Is * wbytes
    mfma_peak = FP8_PEAK_TFLOPS if fp8 else BF16_PEAK_TFLOPS
    tok_s = T / (ms * 1e-3)
    if gate_only:
        # x and the gate weight in; routing (idx, w), counts, perm and pos out
        flop = 2.0 * T * H * E
        layer_bytes = T * H * abytes + E * H * 4 + E * 4 + T * K * 8 + E * 8 + T * K * 8
        ffn = None
    else:
        flop = T * (6.0 * H * (I * K + Is) + 2.0 * H * E)
        layer_bytes = active * expert_w + shared_w + E * H * 4 + E * 4 + 2 * T * H * abytes
        ffn_flop = T * 6.0 * H * (I * K + Is)
        ffn_bytes = active * expert_w + shared_w + T * H * abytes + (T * K + T) * H * abytes
        ffn_ms = acc["expert_ffn"]
        ffn_gbs = ffn_bytes / (ffn_ms * 1e-3) / 1e9
        ffn_tflops = ffn_flop / (ffn_ms * 1e-3) / 1e12
        ffn = {"ms": round(ffn_ms, 4), "hbm_gbs": round(ffn_gbs, 1), "tflops": round(ffn_tflops, 1),
               "hbm_frac": round(ffn_gbs / HBM_PEAK_GBS, 4),
               "mfma_frac": round(ffn_tflops / mfma_peak, 4)}

    work = kernel_work(dominant, cfg, active)
    if work is None:
        roof = {"kernel": dominant, "bound": None, "achieved": None, "peak": None, "unit": None,
                "frac": None, "traffic": None, "avg_launch_ms": round(dom_ms, 4)}
    else:
        kbytes, kflop = work
        ridge = mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9)
        if kflop / kbytes > ridge:
            ach, peak, unit, bound = kflop / (dom_ms * 1e-3) / 1e12, mfma_peak, "TFLOP/s", "mfma"
        else:
            ach, peak, unit, bound = kbytes / (dom_ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s", "hbm"
        roof = {"kernel": dominant, "bound": bound, "achieved": round(ach, 1), "peak": peak,
                "unit": unit, "frac": round(ach / peak, 4),
                "traffic": _traffic(cfg.name, dominant),
                "avg_launch_ms": round(dom_ms, 4), "launches_timed": dom_launches,
                "algorithmic_bytes_per_launch": kbytes, "algorithmic_flop_per_launch": kflop,
                "hbm_gbs": round(kbytes / (dom_ms * 1e-3) / 1e9, 1),
                "mfma_tflops": round(kflop / (dom_ms * 1e-3) / 1e12, 1)}

    result = {
        "metric": "MoE layer tokens/s + % bf16 MFMA peak (prefill), % HBM peak (decode)",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "timing": {"step": "median of per-step HIP events, 1 GiB scratch written before each",
                   "min_ms": round(step_ms[0], 4), "max_ms": round(step_ms[-1], 4),
                   "warm_ms_per_step": round(warm_ms, 4)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "fp8-e4m3", "fp8e8m0": "fp8-e4m3 (power-of-two scales)",
                  "f32": "f32"}[cfg.wdtype],
        "data": "synthetic: seeded N(0,1) tokens, N(0,1/fan_in) weights, gate N(0,1/H), bias "
                + (f"from {os.path.basename(cfg.bias_file)} (Zipf(1.2) expert loads)"
                   if cfg.bias_file
                   else f"U({cfg.bias_lo},{cfg.bias_hi})"),
        "config": {"workload": cfg.name, "T": T, "hidden": H, "n_routed_experts": E,
                   "n_group": cfg.G, "topk_group": cfg.TG, "top_k": K, "moe_inter": I,
                   "shared_inter": Is, "routed_scaling_factor": cfg.rho,
                   "act_dtype": cfg.act, "weight_dtype": cfg.wdtype},
        "layer": {"tflops": round(flop / (ms * 1e-3) / 1e12, 2),
                  "mfma_frac": round(flop / (ms * 1e-3) / 1e12 / mfma_peak, 4),
                  "hbm_gbs": round(layer_bytes / (ms * 1e-3) / 1e9, 1),
                  "hbm_frac": round(layer_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                  "algorithmic_bytes": layer_bytes, "algorithmic_flop": flop,
                  "active_experts": active},
        "phases_ms": {p: round(v, 4) for p, v in acc.items()},
        "kernels_ms": {k: round(v, 4) for k, v in sorted(kernels_ms.items())},
        "expert_ffn": ffn,
        "entry_point": entry,
        "other_entry_points": other,
        "bias_update": bias_update,
        "expert_backward": backward,
        "layer_backward": layer_backward,
        "roofline": roof,
    }

    if args.cpu_sample is None:
        args.cpu_sample = 96 if cfg.wdtype in ("fp8", "fp8e8m0") else 384
    if args.cpu_sample > 0 and not args.profile_only:
        import oracle
        S = min(args.cpu_sample * (64 if gate_only else 1), T)
        toks = np.arange(S)
        log(f"[bench] cpu baseline: oracle on {S} tokens")
        t1 = time.perf_counter()
        if gate_only:
            lg_ref = oracle.logits(inp["x"][:S], "bf16", inp["gate_w"])
            idx_ref, _, _ = oracle.route_f64(cfg, lg_ref, inp["bias"])
            oracle.permute(idx_ref, E)
            what = "fp64 gate logits, group-limited routing and the stable permutation"
        else:
            oracle.forward(cfg, inp, tokens=toks)
            what = "fp64 gate logits, routing and the layer output"
        dt = time.perf_counter() - t1
        cpu_model = None
        try:
            with open("/proc/cpuinfo") as f:
                for line in f:
                    if line.startswith("model name"):
                        cpu_model = line.split(":", 1)[1].strip()
                        break
        except OSError:
            pass
        result["cpu_baseline"] = {"value": round(S / dt, 3), "unit": "tokens/s",
                                  "cores": oracle.threads(), "cpu_model": cpu_model,
                                  "kind": "oracle",
                                  "sample": f"first {S} of the {T} tokens of {cfg.name}: {what} "
                                            f"({dt:.1f} s)"}
    print(json.dumps(result))


if __name__ == "__main__":
    main()
