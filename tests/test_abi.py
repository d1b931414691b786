"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects invalid arguments on the host before any HIP
call."""
import ctypes
import os
import re

import pytest

import sparse_mixture_experts_30_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x1000  # never dereferenced: every call below fails validation first


def _header_functions():
    with open(os.path.join(ROOT, "include", "moe.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function():
    names = _header_functions()
    assert names == sorted(moe.EXPORTS)
    L = moe.lib()
    for n in names:
        assert getattr(L, n) is not None


def _cfg(**kw):
    base = dict(H=7168, E=256, G=8, TG=4, K=8, I=2048, Is=2048, rho=2.5, act="bf16", wdtype="bf16")
    base.update(kw)
    return moe.config(base["H"], base["E"], base["G"], base["TG"], base["K"], base["I"],
                      base["Is"], base["rho"], base["act"], base["wdtype"])


def _gate(cfg, T=4, ws_bytes=1 << 40, x=FAKE, gw=FAKE, b=FAKE, idx=FAKE, w=FAKE, ws=FAKE * 256):
    return moe.lib().moe_gate(ctypes.byref(cfg), T, x, gw, b, None, idx, w, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(E=250, G=8), moe.MOE_ERR_INVALID_ARG),          # E % G != 0
    (dict(E=8, G=8), moe.MOE_ERR_INVALID_ARG),            # one expert per group
    (dict(TG=9), moe.MOE_ERR_INVALID_ARG),                # topk_group > n_group
    (dict(TG=0), moe.MOE_ERR_INVALID_ARG),
    (dict(K=0), moe.MOE_ERR_INVALID_ARG),
    (dict(K=257), moe.MOE_ERR_INVALID_ARG),               # K > E
    (dict(rho=0.0), moe.MOE_ERR_INVALID_ARG),
    (dict(rho=float("inf")), moe.MOE_ERR_INVALID_ARG),
    (dict(rho=float("nan")), moe.MOE_ERR_INVALID_ARG),
    (dict(H=-1), moe.MOE_ERR_INVALID_ARG),
    (dict(E=1024, G=8), moe.MOE_ERR_UNSUPPORTED),         # E > 512
    (dict(E=256, G=128), moe.MOE_ERR_UNSUPPORTED),        # G > 64
    (dict(K=65), moe.MOE_ERR_UNSUPPORTED),
    (dict(H=7000), moe.MOE_ERR_UNSUPPORTED),              # H % 64
    (dict(wdtype="fp8", I=2048 + 64), moe.MOE_ERR_UNSUPPORTED),  # fp8 needs % 128
    (dict(wdtype="fp8e8m0", H=7168 - 64), moe.MOE_ERR_UNSUPPORTED),
    (dict(act="f32", wdtype="bf16"), moe.MOE_ERR_UNSUPPORTED),
])
def test_config_validation(kw, status):
    cfg = _cfg(**kw)
    assert _gate(cfg) == status
    assert moe.moe_workspace_bytes(cfg, 16) == 0
    assert moe.moe_last_error() != ""


def test_argument_validation():
    cfg = _cfg()
    assert _gate(cfg, T=-1) == moe.MOE_ERR_INVALID_ARG
    assert _gate(cfg, x=None) == moe.MOE_ERR_INVALID_ARG
    assert _gate(cfg, gw=None) == moe.MOE_ERR_INVALID_ARG
    assert _gate(cfg, idx=None) == moe.MOE_ERR_INVALID_ARG
    assert _gate(cfg, ws=None) == moe.MOE_ERR_WORKSPACE
    assert _gate(cfg, ws_bytes=100) == moe.MOE_ERR_WORKSPACE
    assert _gate(cfg, ws=FAKE * 256 + 4) == moe.MOE_ERR_WORKSPACE       # misaligned
    assert "workspace" in moe.moe_last_error()
    # T == 0 is a no-op that succeeds without touching any pointer
    assert _gate(cfg, T=0, x=None, ws=None) == moe.MOE_OK
    L = moe.lib()
    assert L.moe_permute(ctypes.byref(cfg), 4, None, FAKE, FAKE, FAKE, FAKE, FAKE * 256, 1 << 40,
                         None) == moe.MOE_ERR_INVALID_ARG
    w = moe.weights(gate_w=FAKE, bias=FAKE, w13=FAKE, w2=FAKE)           # no shared weights
    assert L.moe_expert_ffn(ctypes.byref(cfg), 4, FAKE, FAKE, FAKE, ctypes.byref(w), FAKE, FAKE,
                            FAKE * 256, 1 << 40, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_forward(ctypes.byref(cfg), 4, FAKE, ctypes.byref(w), FAKE, None, None, None,
                         None, None, FAKE * 256, 1 << 40, None) == moe.MOE_ERR_INVALID_ARG
    # the overlapped forward needs a second stream distinct from the first
    wf = moe.weights(gate_w=FAKE, bias=FAKE, w13=FAKE, w2=FAKE, ws13=FAKE, ws2=FAKE)
    for s1, s2 in ((None, None), (FAKE, FAKE)):
        assert L.moe_forward_overlap(ctypes.byref(cfg), 4, FAKE, ctypes.byref(wf), FAKE, None,
                                     None, None, None, None, FAKE * 256, 1 << 40, s1,
                                     s2) == moe.MOE_ERR_INVALID_ARG
    assert "shared_stream" in moe.moe_last_error()
    assert L.moe_forward_overlap(ctypes.byref(cfg), 4, FAKE, ctypes.byref(w), FAKE, None, None,
                                 None, None, None, FAKE * 256, 1 << 40, None,
                                 FAKE) == moe.MOE_ERR_INVALID_ARG   # shared weights missing
    assert L.moe_combine(ctypes.byref(cfg), 4, FAKE, None, FAKE, FAKE, FAKE, None) == \
        moe.MOE_ERR_INVALID_ARG                                          # y_shared NULL, Is > 0
    # the one-launch decode layer: 1 <= T <= 32, bf16 tokens, packed bf16
    # weights; anything else is refused on the host
    wp = moe.weights(gate_w=FAKE, bias=FAKE, w13=FAKE, w2=FAKE, ws13=FAKE, ws2=FAKE)
    wp.packed = 1
    wp8 = moe.weights(gate_w=FAKE, bias=FAKE, w13=FAKE, w13_scale=FAKE, w2=FAKE, w2_scale=FAKE,
                      ws13=FAKE, ws13_scale=FAKE, ws2=FAKE, ws2_scale=FAKE)
    wp8.packed = 1
    for c, ww, T in ((cfg, wf, 4), (cfg, wp, 33), (_cfg(wdtype="fp8"), wp8, 4)):
        assert L.moe_forward_decode_fused(ctypes.byref(c), T, FAKE, ctypes.byref(ww), FAKE, None,
                                          None, None, None, None, FAKE * 256, 1 << 40,
                                          None) == moe.MOE_ERR_UNSUPPORTED, (T, ww.packed)
        assert "one-launch" in moe.moe_last_error()
    assert L.moe_forward_decode_fused(ctypes.byref(cfg), 0, None, ctypes.byref(wp), None, None,
                                      None, None, None, None, None, 0, None) == moe.MOE_OK
    cfg8 = _cfg(wdtype="fp8")
    w8 = moe.weights(gate_w=FAKE, bias=FAKE, w13=FAKE, w2=FAKE, ws13=FAKE, ws2=FAKE)
    assert L.moe_forward(ctypes.byref(cfg8), 4, FAKE, ctypes.byref(w8), FAKE, None, None, None,
                         None, None, FAKE * 256, 1 << 40, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_quantize_act(ctypes.byref(_cfg(act="f32", wdtype="f32")), 4, FAKE, FAKE, FAKE,
                              None) == moe.MOE_ERR_UNSUPPORTED
    # e4m3 with power-of-two scales: packed weights only
    cfg8p = _cfg(wdtype="fp8e8m0")
    w8s = moe.weights(gate_w=FAKE, bias=FAKE, w13=FAKE, w13_scale=FAKE, w2=FAKE, w2_scale=FAKE,
                      ws13=FAKE, ws13_scale=FAKE, ws2=FAKE, ws2_scale=FAKE)
    assert L.moe_forward(ctypes.byref(cfg8p), 4, FAKE, ctypes.byref(w8s), FAKE, None, None, None,
                         None, None, FAKE * 256, 1 << 40, None) == moe.MOE_ERR_UNSUPPORTED
    assert "packed" in moe.moe_last_error()
    assert moe.moe_packed_bytes(cfg8p, moe.MOE_W13) == moe.moe_packed_bytes(cfg8, moe.MOE_W13) > 0
    assert L.moe_get_device_error(None, 0, None) == moe.MOE_ERR_WORKSPACE
    # bias update: the step must be finite and >= 0; both arrays are required
    for gamma in (-1e-3, float("nan"), float("inf")):
        assert L.moe_bias_update(ctypes.byref(cfg), FAKE, gamma, FAKE,
                                 None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_bias_update(ctypes.byref(cfg), None, 1e-3, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_bias_update(ctypes.byref(cfg), FAKE, 1e-3, None, None) == moe.MOE_ERR_INVALID_ARG
    bad = _cfg()
    bad.n_group = 3
    assert L.moe_bias_update(ctypes.byref(bad), FAKE, 1e-3, FAKE, None) != moe.MOE_OK
    # expert backward: row-major bf16 or e4m3 weights; required arrays; workspace
    def bwd(c, w, dy=FAKE, ws=FAKE * 256, ws_bytes=1 << 40):
        return L.moe_expert_ffn_backward(ctypes.byref(c), 4, FAKE, FAKE, FAKE, ctypes.byref(w), dy,
                                         FAKE, None, None, FAKE, FAKE, FAKE, FAKE, ws, ws_bytes,
                                         None)
    wrow = moe.weights(w13=FAKE, w2=FAKE, ws13=FAKE, ws2=FAKE)
    assert bwd(cfg, moe.weights(w13=FAKE, w2=FAKE, ws13=FAKE, ws2=FAKE, packed=1)) == \
        moe.MOE_ERR_UNSUPPORTED
    assert bwd(_cfg(act="f32", wdtype="f32"), wrow) == moe.MOE_ERR_UNSUPPORTED
    # e4m3 weights: the FP8 backward, which needs the block scales
    assert bwd(_cfg(wdtype="fp8"), wrow) == moe.MOE_ERR_INVALID_ARG
    w8 = moe.weights(w13=FAKE, w13_scale=FAKE, w2=FAKE, w2_scale=FAKE, ws13=FAKE,
                     ws13_scale=FAKE, ws2=FAKE, ws2_scale=FAKE)
    assert bwd(_cfg(wdtype="fp8"), w8, ws_bytes=100) == moe.MOE_ERR_WORKSPACE
    w8.packed = 1
    assert bwd(_cfg(wdtype="fp8e8m0"), w8) == moe.MOE_ERR_UNSUPPORTED
    assert bwd(cfg, wrow, dy=None) == moe.MOE_ERR_INVALID_ARG
    assert bwd(cfg, wrow, ws_bytes=100) == moe.MOE_ERR_WORKSPACE
    assert bwd(cfg, wrow, ws=FAKE * 256 + 4) == moe.MOE_ERR_WORKSPACE
    assert moe.moe_expert_ffn_backward_workspace_bytes(_cfg(act="f32", wdtype="f32"), 16) == 0
    for wd in ("fp8", "fp8e8m0"):
        assert moe.moe_expert_ffn_backward_workspace_bytes(_cfg(wdtype=wd), 16) > 0
    # layer backward: the same dtype and layout rules; every forward array is required
    def lbwd(c, w, logits=FAKE, dgw=FAKE, ws=FAKE * 256, ws_bytes=1 << 40):
        return L.moe_backward(ctypes.byref(c), 4, FAKE, ctypes.byref(w), logits, FAKE, FAKE, FAKE,
                              FAKE, FAKE, FAKE, FAKE, FAKE, dgw, FAKE, FAKE, FAKE, FAKE, ws,
                              ws_bytes, None)
    wg = moe.weights(gate_w=FAKE, w13=FAKE, w2=FAKE, ws13=FAKE, ws2=FAKE)
    # e4m3 weights: the FP8 expert backward inside, which needs the block scales
    assert lbwd(_cfg(wdtype="fp8"), wg) == moe.MOE_ERR_INVALID_ARG
    wg8 = moe.weights(gate_w=FAKE, w13=FAKE, w13_scale=FAKE, w2=FAKE, w2_scale=FAKE, ws13=FAKE,
                      ws13_scale=FAKE, ws2=FAKE, ws2_scale=FAKE)
    assert lbwd(_cfg(wdtype="fp8e8m0"), wg8, ws_bytes=100) == moe.MOE_ERR_WORKSPACE
    wg8.packed = 1
    assert lbwd(_cfg(wdtype="fp8"), wg8) == moe.MOE_ERR_UNSUPPORTED
    assert lbwd(_cfg(act="f32", wdtype="f32"), wg) == moe.MOE_ERR_UNSUPPORTED
    assert lbwd(cfg, moe.weights(gate_w=FAKE, w13=FAKE, w2=FAKE, ws13=FAKE, ws2=FAKE,
                                 packed=1)) == moe.MOE_ERR_UNSUPPORTED
    assert lbwd(cfg, wrow) == moe.MOE_ERR_INVALID_ARG                    # no gate weight
    assert lbwd(cfg, wg, logits=None) == moe.MOE_ERR_INVALID_ARG
    assert lbwd(cfg, wg, dgw=None) == moe.MOE_ERR_INVALID_ARG
    assert lbwd(cfg, wg, ws_bytes=100) == moe.MOE_ERR_WORKSPACE
    assert moe.moe_backward_workspace_bytes(_cfg(act="f32", wdtype="f32"), 16) == 0
    for wd in ("fp8", "fp8e8m0"):
        assert moe.moe_backward_workspace_bytes(_cfg(wdtype=wd), 16) > \
            moe.moe_expert_ffn_backward_workspace_bytes(_cfg(wdtype=wd), 16)
    assert moe.moe_backward_workspace_bytes(cfg, 16) > moe.moe_expert_ffn_backward_workspace_bytes(
        cfg, 16)
    assert moe.moe_expert_ffn_backward_workspace_bytes(cfg, 16) > 0


def test_workspace_bytes_grows_with_tokens():
    cfg = _cfg()
    a, b = moe.moe_workspace_bytes(cfg, 32), moe.moe_workspace_bytes(cfg, 4096)
    assert 0 < a < b
    assert b % 256 == 0
    # y [T*K, H] bf16 alone is part of it
    assert b > 4096 * 8 * 7168 * 2


def test_strerror():
    for s in range(6):
        assert moe.moe_strerror(s)
    assert moe.moe_strerror(99) == "unknown status"


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    import sparse_mixture_experts_30_amd._lib as L
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "SO_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="missing"):
        L.lib()


def test_kernel_timer_without_launches():
    # enabling, disabling and reading touch no device when nothing was launched
    moe.moe_kernel_timer_enable(True, "grouped_gemm_bf16_packed<true>")
    moe.moe_kernel_timer_enable(False)
    assert moe.moe_kernel_timer_read() == {}


def test_noalloc_forward_limit_and_constant():
    """moe_forward_noalloc: the static workspace size in the header and the
    binding agree, batches whose workspace exceeds it are refused on the
    host (nothing enqueued, no HIP call), and T = 0 is a no-op."""
    with open(os.path.join(ROOT, "include", "moe.h")) as f:
        m = re.search(r"#define MOE_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", f.read())
    assert m and int(m.group(1)) << int(m.group(2)) == moe.MOE_NOALLOC_SCRATCH_BYTES
    cfg = _cfg()
    W = moe.MoeWeights()
    for T, fits in ((256, True), (288, True), (289, False), (4096, False)):
        assert (moe.moe_workspace_bytes(cfg, T) <= moe.MOE_NOALLOC_SCRATCH_BYTES) == fits, T
    st = moe.lib().moe_forward_noalloc(ctypes.byref(cfg), 4096, FAKE, ctypes.byref(W), FAKE,
                                       None, None, None, None, None, None)
    assert st == moe.MOE_ERR_UNSUPPORTED
    assert "static" in moe.moe_last_error()
    st = moe.lib().moe_forward_noalloc(ctypes.byref(cfg), 0, FAKE, ctypes.byref(W), FAKE,
                                       None, None, None, None, None, None)
    assert st == moe.MOE_OK
    st = moe.lib().moe_forward_noalloc(ctypes.byref(_cfg(K=0)), 4, FAKE, ctypes.byref(W), FAKE,
                                       None, None, None, None, None, None)
    assert st == moe.MOE_ERR_INVALID_ARG


def test_gate_mode_values():
    """moe_set_gate_mode takes 0 (split) and 1 (fused) and rejects anything
    else on the host."""
    L = moe.lib()
    for bad in (-1, 2, 100):
        assert L.moe_set_gate_mode(bad) == moe.MOE_ERR_INVALID_ARG
    for mode in (moe.MOE_GATE_FUSED, moe.MOE_GATE_SPLIT):
        assert L.moe_set_gate_mode(mode) == moe.MOE_OK
